// Parallax decode for gfx950: new queries (one or a few per sequence) against a bf16 key/value cache.
//
// The decode path of the pages' hardware section (gist.science technical summary
// of "Parallax: Parameterized Local Linear Attention for Language Modeling",
// "Hardware-aware algorithm": a dedicated decode kernel in which the softmax and
// covariance branches share one KV stream).  The probe u = P^T (q - kbar) needs
// the whole sequence's kbar, so the cache is streamed twice:
//   pass 1   split-KV partials of the online softmax: m, l, o = sum p v, kbar = sum p k;
//   combine  m, l, o, kbar over splits -> lse, o, kbar, u = P^T (q - kbar), alpha = u.kbar;
//   pass 2   split-KV partials of c = sum_j p_j (u.k_j - alpha) (v_j - o) with p_j = exp(s_j - lse);
//   finish   out = o + sum over splits of c.
// The work is bandwidth-bound (a few flops per cache byte), so the inner loops
// are fp32 VALU on LDS-staged bf16 tiles: the cache is read straight from HBM in
// 16-byte chunks, with no fp16 staging copy.  One workgroup (256 threads) owns
// one (batch, kv head, key split) and all query heads of that kv head.
// The cache is either one contiguous [B][L][Hkv][d] array per tensor or a pool of
// pages [num_pages][page_size][Hkv][d] with a per-sequence block table (the PAGED
// instantiations): key j of sequence b lives in page block_table[b][j / page_size].
// Several new tokens per sequence (T > 1, the last T entries of the sequence, token t seeing keys
// [0, L_b - T + 1 + t)) share a workgroup as extra rows: the template's row count is
// (query heads per kv head) x (tokens in the chunk) <= 8, and longer runs of tokens go in chunks.
#include <math.h>

#include "fast_common.h"
#include "plx_internal.h"

namespace plx {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTile = 64;          // keys per LDS tile
constexpr int kRowH = kD + 8;      // padded LDS row (bf16 elements)
constexpr int kMaxG = 8;          // rows (query head, new token) per workgroup of the fp32 kernels
constexpr int kMaxRowsM = 16;     // rows per workgroup of the matrix-core kernels

struct DecParams {
  const u16 *q, *kc, *vc, *P;
  const int32_t* seqlens;
  const int32_t* block_table;    // paged cache: [B][max_pages] page indices
  int max_pages, page_shift, num_pages;
  void* out;                     // fp32, or bf16 when out_bf16
  float* cor;                    // per query |out - o| / |out| [B][Hq] (nullable)
  int out_bf16;
  // workspace
  float *pm, *pl, *po, *pk;      // pass 1 partials: [B][Hq][ns] (m, l) and [B][Hq][ns][128] (o, kbar)
  float *so, *su, *salpha, *slse;  // combined: o, u [B][Hq][128], alpha, lse [B][Hq]
  float* pc;                     // pass 2 partials [B][Hq][ns][128]
  int B, L, Hq, Hkv, G, window, ns, chunk;
  int D;                         // head dim of the caller's rows (128, or 64 zero-padded to 128 internally)
  int T, t0;                     // new tokens per sequence; first token of this launch's chunk
  int Tc;                        // tokens in the chunk
  float scale;
};

// Keys [lo, hi) that new token t of sequence b sees.
__device__ __forceinline__ void row_range(const DecParams& p, int b, int t, int& lo, int& hi) {
  int Lb = p.L;
  if (p.seqlens) Lb = min(max(p.seqlens[b], 0), p.L);
  hi = max(0, Lb - (p.T - 1 - t));
  lo = p.window > 0 ? max(0, hi - p.window) : 0;
}

// Keys any token of the chunk sees.
__device__ __forceinline__ void seq_range(const DecParams& p, int b, int& lo, int& hi) {
  int l2, h2;
  row_range(p, b, p.t0, lo, h2);
  row_range(p, b, p.t0 + p.Tc - 1, l2, hi);
}

// Index (sequence, token, query head) of row r of a workgroup of kv head g: the rows are the G query
// heads of the group for each token of the chunk.
__device__ __forceinline__ int64_t row_bh(const DecParams& p, int b, int g, int r) {
  const int t = p.t0 + r / p.G;
  return (static_cast<int64_t>(b) * p.T + t) * p.Hq + g * p.G + r % p.G;
}

struct __align__(16) DecTiles {
  union {
    struct {
      u16 k[1][kTile * kRowH];
      u16 v[1][kTile * kRowH];
    };
    float red[4][kMaxG][kD * 2];   // after the key loop: the 4 key parts of each accumulator
  };
  float q[kMaxG][kD];
  float u[kMaxG][kD];
  float s[kMaxG][kTile];
  float w[kMaxG][kTile];
  float corr[kMaxG];
};

// One K and V tile in LDS (about 47 KB with the rest, so three workgroups fit a CU; measured, three
// stream the cache faster than two with double-buffered tiles, and than four).  The next tile (64
// keys x 16 chunks of 16 bytes each, 4 + 4 chunks per thread) is fetched into registers at the start
// of an iteration and stored into LDS after the current tile's work and a barrier, so that the loads
// are in flight while it runs (the loops' barriers are lds_barrier(), which does not wait for them).  Keys at
// or beyond `hi` read the last valid key (their weight is 0).
// (eight named registers rather than an array: an array live across the loop stays in scratch memory)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
struct TileRegs {
  u32x4 k0, k1, k2, k3, v0, v1, v2, v3;
};

// Cache row (token slot) of key `key` of sequence b.  A paged cache looks the page up in the block
// table; entries outside [0, num_pages) are clamped into the pool, so a bad table gives wrong values
// for that sequence but never an access outside the caller's arrays.
template <bool PAGED>
__device__ __forceinline__ int64_t cache_row(const DecParams& p, int b, int key) {
  if constexpr (PAGED) {
    int pg = p.block_table[static_cast<int64_t>(b) * p.max_pages + (key >> p.page_shift)];
    pg = min(max(pg, 0), p.num_pages - 1);
    return (static_cast<int64_t>(pg) << p.page_shift) + (key & ((1 << p.page_shift) - 1));
  } else {
    return static_cast<int64_t>(b) * p.L + key;
  }
}

// Chunk c (8 elements) of a cache row; chunks past a D < 128 head read as zeros.
__device__ __forceinline__ u32x4 fetch16(const u16* base, const DecParams& p, int64_t row, int g, int c) {
  if (c * 8 >= p.D) return u32x4{0u, 0u, 0u, 0u};
  return *reinterpret_cast<const u32x4*>(base + (row * p.Hkv + g) * p.D + c * 8);
}

template <bool PAGED>
__device__ __forceinline__ TileRegs tile_fetch(const DecParams& p, int b, int g, int key0, int hi, int tid) {
  const int r = tid >> 4, c = tid & 15;   // chunk j of the thread: row r + 16 j, chunk c
  const int64_t ra = cache_row<PAGED>(p, b, min(key0 + r, hi - 1));
  const int64_t rb = cache_row<PAGED>(p, b, min(key0 + r + 16, hi - 1));
  const int64_t rc = cache_row<PAGED>(p, b, min(key0 + r + 32, hi - 1));
  const int64_t rd = cache_row<PAGED>(p, b, min(key0 + r + 48, hi - 1));
  TileRegs R;
  R.k0 = fetch16(p.kc, p, ra, g, c);
  R.k1 = fetch16(p.kc, p, rb, g, c);
  R.k2 = fetch16(p.kc, p, rc, g, c);
  R.k3 = fetch16(p.kc, p, rd, g, c);
  R.v0 = fetch16(p.vc, p, ra, g, c);
  R.v1 = fetch16(p.vc, p, rb, g, c);
  R.v2 = fetch16(p.vc, p, rc, g, c);
  R.v3 = fetch16(p.vc, p, rd, g, c);
  return R;
}

__device__ __forceinline__ void tile_store(const TileRegs& R, DecTiles& T, int buf, int tid) {
  const int r = tid >> 4, c = tid & 15;
  u16* k = &T.k[buf][r * kRowH + c * 8];
  u16* v = &T.v[buf][r * kRowH + c * 8];
  *reinterpret_cast<u32x4*>(k) = R.k0;
  *reinterpret_cast<u32x4*>(k + 16 * kRowH) = R.k1;
  *reinterpret_cast<u32x4*>(k + 32 * kRowH) = R.k2;
  *reinterpret_cast<u32x4*>(k + 48 * kRowH) = R.k3;
  *reinterpret_cast<u32x4*>(v) = R.v0;
  *reinterpret_cast<u32x4*>(v + 16 * kRowH) = R.v1;
  *reinterpret_cast<u32x4*>(v + 32 * kRowH) = R.v2;
  *reinterpret_cast<u32x4*>(v + 48 * kRowH) = R.v3;
}

// Dot products of the tile's keys with the G vectors in `vecs` (q or u): dots[h][j].
// 256 threads; thread t takes dot (t / tpd) and a 128/tpd slice of d.
template <int G>
__device__ __forceinline__ void tile_dots(const DecTiles& T, int buf, const float (*vecs)[kD], float (*dots)[kTile],
                                          int tid) {
  constexpr int ndots = G * kTile;
  if constexpr (ndots > 256) {               // 8 rows: two whole dots per thread
#pragma unroll
    for (int rep = 0; rep < ndots / 256; ++rep) {
      const int dot = tid + 256 * rep;
      const int h = dot / kTile, j = dot % kTile;
      const u16* kr = &T.k[buf][j * kRowH];
      float acc = 0.f;
#pragma unroll 4
      for (int c = 0; c < kD; c += 8) {
        const uint4 w = *reinterpret_cast<const uint4*>(kr + c);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = fmaf(__uint_as_float(ws[e] << 16), vecs[h][c + 2 * e], acc);
          acc = fmaf(__uint_as_float(ws[e] & 0xffff0000u), vecs[h][c + 2 * e + 1], acc);
        }
      }
      dots[h][j] = acc;
    }
    return;
  }
  constexpr int tpd = ndots > 256 ? 1 : 256 / ndots;   // threads per dot: 4, 2 or 1
  constexpr int len = kD / tpd;
  const int dot = tid / tpd, part = tid % tpd;
  const int h = dot / kTile, j = dot % kTile;
  const u16* kr = &T.k[buf][j * kRowH + part * len];
  const float* vr = &vecs[h][part * len];
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < len; c += 8) {
    const uint4 w = *reinterpret_cast<const uint4*>(kr + c);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(__uint_as_float(ws[e] << 16), vr[c + 2 * e], acc);
      acc = fmaf(__uint_as_float(ws[e] & 0xffff0000u), vr[c + 2 * e + 1], acc);
    }
  }
  if constexpr (tpd >= 2) acc += __shfl_xor(acc, 1, 64);
  if constexpr (tpd >= 4) acc += __shfl_xor(acc, 2, 64);
  if (part == 0) dots[h][j] = acc;
}

// ---------------------------------- pass 1 ----------------------------------
template <int G, bool PAGED>
__global__ __launch_bounds__(256) void k_dec_pass1(DecParams p) {
  __shared__ DecTiles T;
  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  int lo, hi;
  seq_range(p, b, lo, hi);
  const int k0 = max(lo, sp * p.chunk), k1 = min(hi, (sp + 1) * p.chunk);
  const float c2 = p.scale * kLog2e;
  for (int e = tid; e < G * kD; e += 256) {
    const int h = e / kD, d = e % kD;
    T.q[h][d] = d < p.D ? bf16_to_f32(p.q[row_bh(p, b, g, h) * p.D + d]) * c2 : 0.f;  // scores in log2 units
  }
  // keys of this split that each of the wave's rows sees (the softmax of row h is done by wave h % 4)
  constexpr int RW = G > 4 ? 2 : 1;   // rows per wave
  int rlo[RW], rhi[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int r = (tid >> 6) + 4 * i;
    rlo[i] = k0;
    rhi[i] = k1;
    if (r < G) {
      int a, c;
      row_range(p, b, p.t0 + r / p.G, a, c);
      rlo[i] = max(k0, a);
      rhi[i] = min(k1, c);
    }
  }
  // accumulator ownership: thread t -> dims 2*(t%64), +1 ; keys j = part (mod 4)
  const int dp = tid & 63, part = tid >> 6;
  float o[G][2], kb[G][2];
  float m[RW], l[RW];  // per row, kept by the softmax wave and broadcast through LDS
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) o[h][0] = o[h][1] = kb[h][0] = kb[h][1] = 0.f;
  const int nt = k1 > k0 ? (k1 - k0 + kTile - 1) / kTile : 0;
  TileRegs R{};
  if (nt > 0) {
    R = tile_fetch<PAGED>(p, b, g, k0, k1, tid);
    tile_store(R, T, 0, tid);
  }
  __syncthreads();
  for (int it = 0; it < nt; ++it) {
    const int buf = 0, key0 = k0 + it * kTile;
    R = tile_fetch<PAGED>(p, b, g, key0 + kTile, k1, tid);   // (past the last tile: rereads the last key)
    tile_dots<G>(T, buf, T.q, T.s, tid);
    lds_barrier();
    const int w = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int r = w + 4 * i;
      if (r < G) {  // online softmax of row r over this tile
        const float sv = key0 + lane >= rlo[i] && key0 + lane < rhi[i] ? T.s[r][lane] : -INFINITY;
        float tm = sv;
#pragma unroll
        for (int o2 = 32; o2 > 0; o2 >>= 1) tm = fmaxf(tm, __shfl_xor(tm, o2, 64));
        const float mn = fmaxf(m[i], tm);
        const float corr = m[i] == -INFINITY ? 0.f : exp2f(m[i] - mn);
        const float pv = sv == -INFINITY ? 0.f : exp2f(sv - mn);
        float ts = pv;
#pragma unroll
        for (int o2 = 32; o2 > 0; o2 >>= 1) ts += __shfl_xor(ts, o2, 64);
        l[i] = l[i] * corr + ts;
        m[i] = mn;
        T.w[r][lane] = pv;
        if (lane == 0) T.corr[r] = corr;
      }
    }
    lds_barrier();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float cr = T.corr[h];
      o[h][0] *= cr;
      o[h][1] *= cr;
      kb[h][0] *= cr;
      kb[h][1] *= cr;
    }
#pragma unroll 4
    for (int j = part; j < kTile; j += 4) {
      const uint32_t kw = *reinterpret_cast<const uint32_t*>(&T.k[buf][j * kRowH + 2 * dp]);
      const uint32_t vw = *reinterpret_cast<const uint32_t*>(&T.v[buf][j * kRowH + 2 * dp]);
      const float k0f = __uint_as_float(kw << 16), k1f = __uint_as_float(kw & 0xffff0000u);
      const float v0f = __uint_as_float(vw << 16), v1f = __uint_as_float(vw & 0xffff0000u);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pw = T.w[h][j];
        o[h][0] = fmaf(pw, v0f, o[h][0]);
        o[h][1] = fmaf(pw, v1f, o[h][1]);
        kb[h][0] = fmaf(pw, k0f, kb[h][0]);
        kb[h][1] = fmaf(pw, k1f, kb[h][1]);
      }
    }
    lds_barrier();
    tile_store(R, T, 0, tid);
    lds_barrier();
  }
  // reduce the 4 key parts and write the partials
#pragma unroll
  for (int h = 0; h < G; ++h) {
    T.red[part][h][2 * dp] = o[h][0];
    T.red[part][h][2 * dp + 1] = o[h][1];
    T.red[part][h][kD + 2 * dp] = kb[h][0];
    T.red[part][h][kD + 2 * dp + 1] = kb[h][1];
  }
  __syncthreads();
  for (int e = tid; e < G * 2 * kD; e += 256) {
    const int h = e / (2 * kD), r = e % (2 * kD);
    const float s = T.red[0][h][r] + T.red[1][h][r] + T.red[2][h][r] + T.red[3][h][r];
    const int64_t base = (row_bh(p, b, g, h) * p.ns + sp) * kD;
    if (r < kD) p.po[base + r] = s;
    else p.pk[base + r - kD] = s;
  }
  const int w = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int r = w + 4 * i;
    if (r < G && lane == 0) {
      const int64_t si = row_bh(p, b, g, r) * p.ns + sp;
      p.pm[si] = m[i];
      p.pl[si] = l[i];
    }
  }
}

// ------------------------------- combine 1 -----------------------------------
// one block (128 threads) per (batch, query head): lse, o, kbar, u = P^T (q - kbar), alpha
__global__ __launch_bounds__(128) void k_dec_combine1(DecParams p) {
  __shared__ float xs[kD];
  __shared__ float red[2];
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int64_t bh = static_cast<int64_t>(b) * p.Hq + h;
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < p.ns; ++s) M = fmaxf(M, p.pm[bh * p.ns + s]);
  float L = 0.f, o = 0.f, kb = 0.f;
#pragma unroll 8
  for (int s = 0; s < p.ns; ++s) {
    const float ms = p.pm[bh * p.ns + s];
    if (ms == -INFINITY) continue;
    const float f = exp2f(ms - M);
    L += p.pl[bh * p.ns + s] * f;
    o += p.po[(bh * p.ns + s) * kD + d] * f;
    kb += p.pk[(bh * p.ns + s) * kD + d] * f;
  }
  const bool has = L > 0.f;
  o = has ? o / L : 0.f;
  kb = has ? kb / L : 0.f;
  const float qd = d < p.D ? bf16_to_f32(p.q[bh * p.D + d]) : 0.f;
  xs[d] = qd - kb;
  __syncthreads();
  float u = 0.f;
  const u16* Ph = p.P + static_cast<int64_t>(h) * p.D * p.D;
  if (d < p.D)
    for (int bb = 0; bb < p.D; ++bb) u = fmaf(bf16_to_f32(Ph[bb * p.D + d]), xs[bb], u);  // u[d] = sum_b P[b][d] x[b]
  float al = u * kb;
#pragma unroll
  for (int o2 = 32; o2 > 0; o2 >>= 1) al += __shfl_xor(al, o2, 64);
  if ((d & 63) == 0) red[d >> 6] = al;
  __syncthreads();
  al = red[0] + red[1];
  p.so[bh * kD + d] = o;
  p.su[bh * kD + d] = u;
  if (d == 0) {
    p.salpha[bh] = al;
    p.slse[bh] = has ? M + log2f(L) : -INFINITY;   // log2 units of the scaled scores
  }
}

// ---------------------------------- pass 2 ----------------------------------
template <int G, bool PAGED>
__global__ __launch_bounds__(256) void k_dec_pass2(DecParams p) {
  __shared__ DecTiles T;
  __shared__ float st[kMaxG][2];  // lse (log2 units), alpha
  __shared__ int rng[kMaxG][2];   // keys of this split each row sees
  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  int lo, hi;
  seq_range(p, b, lo, hi);
  const int k0 = max(lo, sp * p.chunk), k1 = min(hi, (sp + 1) * p.chunk);
  const float c2 = p.scale * kLog2e;
  for (int e = tid; e < G * kD; e += 256) {
    const int h = e / kD, d = e % kD;
    const int64_t bh = row_bh(p, b, g, h);
    T.q[h][d] = d < p.D ? bf16_to_f32(p.q[bh * p.D + d]) * c2 : 0.f;
    T.u[h][d] = p.su[bh * kD + d];
  }
  if (tid < G) {
    const int64_t bh = row_bh(p, b, g, tid);
    st[tid][0] = p.slse[bh];
    st[tid][1] = p.salpha[bh];
    int a, c;
    row_range(p, b, p.t0 + tid / p.G, a, c);
    rng[tid][0] = max(k0, a);
    rng[tid][1] = min(k1, c);
  }
  const int dp = tid & 63, part = tid >> 6;
  float cv[G][2], ws[G];
#pragma unroll
  for (int h = 0; h < G; ++h) cv[h][0] = cv[h][1] = ws[h] = 0.f;
  const int nt = k1 > k0 ? (k1 - k0 + kTile - 1) / kTile : 0;
  TileRegs R{};
  if (nt > 0) {
    R = tile_fetch<PAGED>(p, b, g, k0, k1, tid);
    tile_store(R, T, 0, tid);
  }
  __syncthreads();
  for (int it = 0; it < nt; ++it) {
    const int buf = 0, key0 = k0 + it * kTile;
    R = tile_fetch<PAGED>(p, b, g, key0 + kTile, k1, tid);   // (past the last tile: rereads the last key)
    tile_dots<G>(T, buf, T.q, T.s, tid);
    tile_dots<G>(T, buf, T.u, T.w, tid);
    lds_barrier();
    // weights w_j = p_j (u.k_j - alpha), p_j = exp2(s_j - lse)
    for (int e = tid; e < G * kTile; e += 256) {
      const int h = e / kTile, j = e % kTile;
      const float lse = st[h][0];
      const int key = key0 + j;
      const float pw = (key >= rng[h][0] && key < rng[h][1] && lse > -INFINITY) ? exp2f(T.s[h][j] - lse) : 0.f;
      T.w[h][j] = pw * (T.w[h][j] - st[h][1]);
    }
    lds_barrier();
#pragma unroll 4
    for (int j = part; j < kTile; j += 4) {
      const uint32_t vw = *reinterpret_cast<const uint32_t*>(&T.v[buf][j * kRowH + 2 * dp]);
      const float v0f = __uint_as_float(vw << 16), v1f = __uint_as_float(vw & 0xffff0000u);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float wj = T.w[h][j];
        cv[h][0] = fmaf(wj, v0f, cv[h][0]);
        cv[h][1] = fmaf(wj, v1f, cv[h][1]);
        ws[h] += wj;
      }
    }
    lds_barrier();
    tile_store(R, T, 0, tid);
    lds_barrier();
  }
  // partial c = sum w v - (sum w) o
#pragma unroll
  for (int h = 0; h < G; ++h) {
    T.red[part][h][2 * dp] = cv[h][0];
    T.red[part][h][2 * dp + 1] = cv[h][1];
    if (dp == 0) T.red[part][h][kD] = ws[h];
  }
  __syncthreads();
  for (int e = tid; e < G * kD; e += 256) {
    const int h = e / kD, d = e % kD;
    const int64_t bh = row_bh(p, b, g, h);
    const float s = T.red[0][h][d] + T.red[1][h][d] + T.red[2][h][d] + T.red[3][h][d];
    const float wsum = T.red[0][h][kD] + T.red[1][h][kD] + T.red[2][h][kD] + T.red[3][h][kD];
    p.pc[(bh * p.ns + sp) * kD + d] = s - wsum * p.so[bh * kD + d];
  }
}

// out = o + sum over splits of c
__global__ __launch_bounds__(128) void k_dec_finish(DecParams p) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int64_t bh = static_cast<int64_t>(b) * p.Hq + h;
  float c = 0.f;
#pragma unroll 8
  for (int s = 0; s < p.ns; ++s) c += p.pc[(bh * p.ns + s) * kD + d];
  const float r = p.so[bh * kD + d] + c;
  if (d < p.D) {
    if (p.out_bf16) static_cast<u16*>(p.out)[bh * p.D + d] = static_cast<u16>(f32_to_bf16(r));
    else static_cast<float*>(p.out)[bh * p.D + d] = r;
  }
  if (p.cor) {
    __shared__ float part[2][2];
    float cc = c * c, oo = r * r;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      cc += __shfl_xor(cc, o, 64);
      oo += __shfl_xor(oo, o, 64);
    }
    if ((d & 63) == 0) {
      part[d >> 6][0] = cc;
      part[d >> 6][1] = oo;
    }
    __syncthreads();
    if (d == 0) {
      const float C = part[0][0] + part[1][0], O = part[0][1] + part[1][1];
      p.cor[bh] = O > 0.f ? sqrtf(C / O) : 0.f;
    }
  }
}

// ------------------ pass 1 and pass 2 on the matrix cores (3 to 16 rows) ------------------
// With 3 to 16 rows (query heads x new tokens) per workgroup the fp32 dot products and sums above take
// more VALU time than a tile takes to arrive.  These variants form the scores (and pass 2's u.k), o, kbar
// and the correction's sum W v with v_mfma_f32_16x16x32_bf16, rows padded to 16:
//   scores  S^T (16 keys x 16 rows) = K (16 keys x 32 dims) . Q^T (32 dims x 16 rows), 4 dim steps;
//   sums    o^T (16 dims x 16 rows) += V^T (16 dims x 32 keys) . P~^T (32 keys x 16 rows), 2 key steps.
// Lane l always holds row n = l % 16 of its results, so the running maximum, its rescale and the row
// sums stay per lane.  Wave w scores keys 16 w .. 16 w + 15 of each 64-key tile and forms the sums for
// dims 32 w .. 32 w + 31 over the whole tile.  The cache's bf16 values and q are used as they are; u, the
// weights p~ (pass 1) and W = p (u.k - alpha) (pass 2) are bf16 pairs hi + lo (hi rounded, lo the rounded
// remainder: about 16 bits), each product taking two MFMAs, and l and sum W are summed from the same
// pairs, so o = sum p~ v / l and c = sum W (v - o) hold for the weights used.  (Single bf16 weights give
// 2.6e-2 of max error / rms on a sequence of three keys, whose rows are several times the tensor's rms.)
typedef __bf16 dbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 dbf16x4 __attribute__((ext_vector_type(4)));
typedef float df32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowM = 144;   // tile row stride in bf16 elements (288 bytes: the score row reads and the
                             // transpose loads of a 16-lane group hit distinct banks)
constexpr int kPRow = 72;    // weight-tile row stride (144 bytes: the 16 rows' reads hit distinct banks)
constexpr float kMomTau = 8.f;

struct __align__(16) MDecTiles {
  u16 k[kTile * kRowM];
  u16 v[kTile * kRowM];
  u16 pw[2][16 * kPRow];     // bf16 weights per (hi / lo, row, key)
  float smax[4][16];         // per (score wave, row): the wave's 16-key maximum (pass 1)
  float rsum[4][16];         // per (score wave, row): l (pass 1) or sum W (pass 2), after the loop
};

__device__ __forceinline__ void mtile_store(const TileRegs& R, MDecTiles& T, int tid) {
  const int r = tid >> 4, c = tid & 15;
  u16* k = &T.k[r * kRowM + c * 8];
  u16* v = &T.v[r * kRowM + c * 8];
  *reinterpret_cast<u32x4*>(k) = R.k0;
  *reinterpret_cast<u32x4*>(k + 16 * kRowM) = R.k1;
  *reinterpret_cast<u32x4*>(k + 32 * kRowM) = R.k2;
  *reinterpret_cast<u32x4*>(k + 48 * kRowM) = R.k3;
  *reinterpret_cast<u32x4*>(v) = R.v0;
  *reinterpret_cast<u32x4*>(v + 16 * kRowM) = R.v1;
  *reinterpret_cast<u32x4*>(v + 32 * kRowM) = R.v2;
  *reinterpret_cast<u32x4*>(v + 48 * kRowM) = R.v3;
}

// A operand V^T or K^T (16 dims x 32 keys) for dims 16 db + [0, 16) and keys 32 ks + [0, 32): lane l gets
// dim 16 db + l % 16 and keys 32 ks + 8 (l / 16) + [0, 8), by two transpose loads (ds_read_b64_tr_b16:
// lane i of a 16-lane group receives element i % 4 of the 8 bytes that lane 4 j + i / 4 addresses, as its
// element j), source lane 4 j + a pointing at dims 16 db + 4 a + [0, 4) of key 32 ks + 8 (l / 16) + j
// (+ 4 for the second load).
__device__ __forceinline__ dbf16x8 mcols(const u16* tile, int l, int ks, int db) {
  const int G = l >> 4, j = (l >> 2) & 3, a = l & 3;
  const u16* src = tile + (32 * ks + 8 * G + j) * kRowM + 16 * db + 4 * a;
  const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)src);
  const v4i16 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(src + 4 * kRowM));
  const dbf16x4 xb = __builtin_bit_cast(dbf16x4, x), yb = __builtin_bit_cast(dbf16x4, y);
  return __builtin_shufflevector(xb, yb, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A operand K (16 keys x 32 dims) of key block kb, dim step st: lane l gets key 16 kb + l % 16 and dims
// 32 st + 8 (l / 16) + [0, 8) (one 16-byte row read).
__device__ __forceinline__ dbf16x8 mrows(const u16* tile, int l, int kb, int st) {
  return __builtin_bit_cast(dbf16x8, *reinterpret_cast<const uint4*>(tile + (16 * kb + (l & 15)) * kRowM + 32 * st +
                                                                     8 * (l >> 4)));
}

// B operand of the scores: row n = l % 16 of x (q or u rows of the workgroup, bf16), dims 32 st + 8 (l / 16)
// + [0, 8); rows >= R and dims >= D read as zeros.  src(n) returns the row's element pointer (bf16).
__device__ __forceinline__ dbf16x8 mvec_bf16(const u16* row, int l, int st, int D) {
  const int d0 = 32 * st + 8 * (l >> 4);
  if (!row || d0 >= D) return dbf16x8{};
  return __builtin_bit_cast(dbf16x8, *reinterpret_cast<const uint4*>(row + d0));
}

// Stores a lane's 4 weights (row n, keys k4 .. k4 + 3) as bf16 pairs hi + lo into the weight tiles and
// returns their sum as the pairs represent them.
__device__ __forceinline__ float mweights_store(MDecTiles& T, int n, int k4, const float (&x)[4]) {
  uint32_t hw[2], lw[2];
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < 4; r += 2) {
    const uint32_t h0 = f32_to_bf16(x[r]), h1 = f32_to_bf16(x[r + 1]);
    const float r0 = x[r] - __uint_as_float(h0 << 16), r1 = x[r + 1] - __uint_as_float(h1 << 16);
    const uint32_t l0 = f32_to_bf16(r0), l1 = f32_to_bf16(r1);
    hw[r / 2] = h0 | (h1 << 16);
    lw[r / 2] = l0 | (l1 << 16);
    sum += (__uint_as_float(h0 << 16) + __uint_as_float(l0 << 16)) + (__uint_as_float(h1 << 16) + __uint_as_float(l1 << 16));
  }
  *reinterpret_cast<uint2*>(&T.pw[0][n * kPRow + k4]) = uint2{hw[0], hw[1]};
  *reinterpret_cast<uint2*>(&T.pw[1][n * kPRow + k4]) = uint2{lw[0], lw[1]};
  return sum;
}

// B operand (32 keys x 16 rows) of the sums: row n = l % 16 of the weight tile `half` (0 hi, 1 lo),
// keys k0 .. k0 + 7 (16 bytes).
__device__ __forceinline__ dbf16x8 mweights(const MDecTiles& T, int half, int n, int k0) {
  return __builtin_bit_cast(dbf16x8, *reinterpret_cast<const uint4*>(&T.pw[half][n * kPRow + k0]));
}

template <bool PAGED>
__global__ __launch_bounds__(256) void k_dec_mpass1(DecParams p) {
  __shared__ MDecTiles T;
  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, n = l & 15, G4 = l >> 4;
  int lo, hi;
  seq_range(p, b, lo, hi);
  const int k0 = max(lo, sp * p.chunk), k1 = min(hi, (sp + 1) * p.chunk);
  const float c2 = p.scale * kLog2e;
  // the lane's row: its q operand and the keys of this split it sees
  const bool rowok = n < p.G * p.Tc;   // the workgroup's rows: G query heads x Tc tokens, at most 16
  int rlo = k0, rhi = k0;
  const u16* qrow = nullptr;
  if (rowok) {
    int a, c;
    row_range(p, b, p.t0 + n / p.G, a, c);
    rlo = max(k0, a);
    rhi = min(k1, c);
    qrow = p.q + row_bh(p, b, g, n) * p.D;
  }
  dbf16x8 qB[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) qB[st] = mvec_bf16(qrow, l, st, p.D);
  df32x4 accO[2], accK[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) accO[i] = accK[i] = df32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, lpart = 0.f;
  const int nt = k1 > k0 ? (k1 - k0 + kTile - 1) / kTile : 0;
  TileRegs Rg{};
  if (nt > 0) {
    Rg = tile_fetch<PAGED>(p, b, g, k0, k1, tid);
    mtile_store(Rg, T, tid);
  }
  __syncthreads();
  for (int it = 0; it < nt; ++it) {
    const int key0 = k0 + it * kTile;
    Rg = tile_fetch<PAGED>(p, b, g, key0 + kTile, k1, tid);   // (past the last tile: rereads the last key)
    // scores of keys 16 w + 4 (l / 16) + [0, 4) for row n
    df32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mrows(T.k, l, w, st), qB[st], sacc, 0, 0, 0);
    float sv[4], mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + 16 * w + 4 * G4 + r;
      sv[r] = key >= rlo && key < rhi ? sacc[r] * c2 : -INFINITY;
      mx = fmaxf(mx, sv[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (l < 16) T.smax[w][l] = mx;
    lds_barrier();
    // lazy running maximum of the row (moves only when the tile exceeds it by kMomTau, log2 units)
    const float tm = fmaxf(fmaxf(T.smax[0][n], T.smax[1][n]), fmaxf(T.smax[2][n], T.smax[3][n]));
    if (tm > m_run + kMomTau) {
      const float f = m_run == -INFINITY ? 0.f : exp2f(m_run - tm);
      m_run = tm;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        accO[i] *= f;
        accK[i] *= f;
      }
      lpart *= f;
    }
    float e[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) e[r] = sv[r] == -INFINITY ? 0.f : exp2f(sv[r] - m_run);
    lpart += mweights_store(T, n, 16 * w + 4 * G4, e);
    lds_barrier();
    // o^T and kbar^T for dims 32 w + [0, 32)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const dbf16x8 ph = mweights(T, 0, n, 32 * ks + 8 * G4), pl = mweights(T, 1, n, 32 * ks + 8 * G4);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const dbf16x8 av = mcols(T.v, l, ks, 2 * w + i), ak = mcols(T.k, l, ks, 2 * w + i);
        accO[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, ph, accO[i], 0, 0, 0);
        accK[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, ph, accK[i], 0, 0, 0);
        accO[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pl, accO[i], 0, 0, 0);
        accK[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, pl, accK[i], 0, 0, 0);
      }
    }
    lds_barrier();
    mtile_store(Rg, T, tid);
    lds_barrier();
  }
  // l of each row: the lanes of a row in a wave, then the four waves
  lpart += __shfl_xor(lpart, 16, 64);
  lpart += __shfl_xor(lpart, 32, 64);
  if (l < 16) T.rsum[w][l] = lpart;
  __syncthreads();
  if (rowok) {
    const int64_t bh = row_bh(p, b, g, n);
    const int64_t base = (bh * p.ns + sp) * kD;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 16 * (2 * w + i) + 4 * G4 + r;   // accumulator row = dim, column = row n
        p.po[base + d] = accO[i][r];
        p.pk[base + d] = accK[i][r];
      }
    if (w == 0 && G4 == 0) {
      p.pm[bh * p.ns + sp] = m_run;
      p.pl[bh * p.ns + sp] = T.rsum[0][n] + T.rsum[1][n] + T.rsum[2][n] + T.rsum[3][n];
    }
  }
}

template <bool PAGED>
__global__ __launch_bounds__(256) void k_dec_mpass2(DecParams p) {
  __shared__ MDecTiles T;
  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, n = l & 15, G4 = l >> 4;
  int lo, hi;
  seq_range(p, b, lo, hi);
  const int k0 = max(lo, sp * p.chunk), k1 = min(hi, (sp + 1) * p.chunk);
  const float c2 = p.scale * kLog2e;
  const bool rowok = n < p.G * p.Tc;   // the workgroup's rows: G query heads x Tc tokens, at most 16
  int rlo = k0, rhi = k0;
  const u16* qrow = nullptr;
  float lse = -INFINITY, alpha = 0.f;
  int64_t bh = 0;
  if (rowok) {
    int a, c;
    row_range(p, b, p.t0 + n / p.G, a, c);
    rlo = max(k0, a);
    rhi = min(k1, c);
    bh = row_bh(p, b, g, n);
    qrow = p.q + bh * p.D;
    lse = p.slse[bh];
    alpha = p.salpha[bh];
  }
  if (lse == -INFINITY) rhi = rlo;   // a row with no visible key contributes nothing
  dbf16x8 qB[4], uB[4], uL[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    qB[st] = mvec_bf16(qrow, l, st, p.D);
    dbf16x8 ub{}, ul{};
    if (rowok) {
      const float* ur = p.su + bh * kD + 32 * st + 8 * G4;   // (zero past D)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 h = static_cast<__bf16>(ur[e]);
        ub[e] = h;
        ul[e] = static_cast<__bf16>(ur[e] - static_cast<float>(h));
      }
    }
    uB[st] = ub;
    uL[st] = ul;
  }
  df32x4 accC[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) accC[i] = df32x4{0.f, 0.f, 0.f, 0.f};
  float wpart = 0.f;
  const int nt = k1 > k0 ? (k1 - k0 + kTile - 1) / kTile : 0;
  TileRegs Rg{};
  if (nt > 0) {
    Rg = tile_fetch<PAGED>(p, b, g, k0, k1, tid);
    mtile_store(Rg, T, tid);
  }
  __syncthreads();
  for (int it = 0; it < nt; ++it) {
    const int key0 = k0 + it * kTile;
    Rg = tile_fetch<PAGED>(p, b, g, key0 + kTile, k1, tid);
    df32x4 sacc = {0.f, 0.f, 0.f, 0.f}, racc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const dbf16x8 kr = mrows(T.k, l, w, st);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr, qB[st], sacc, 0, 0, 0);
      racc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr, uB[st], racc, 0, 0, 0);
      racc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr, uL[st], racc, 0, 0, 0);
    }
    // W = p (u.k - alpha), p = exp2(s - lse), as bf16 pairs; sum W from the same pairs
    float wv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + 16 * w + 4 * G4 + r;
      wv[r] = key >= rlo && key < rhi ? exp2f(sacc[r] * c2 - lse) * (racc[r] - alpha) : 0.f;
    }
    wpart += mweights_store(T, n, 16 * w + 4 * G4, wv);
    lds_barrier();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const dbf16x8 wh = mweights(T, 0, n, 32 * ks + 8 * G4), wl = mweights(T, 1, n, 32 * ks + 8 * G4);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const dbf16x8 av = mcols(T.v, l, ks, 2 * w + i);
        accC[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, wh, accC[i], 0, 0, 0);
        accC[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, wl, accC[i], 0, 0, 0);
      }
    }
    lds_barrier();
    mtile_store(Rg, T, tid);
    lds_barrier();
  }
  wpart += __shfl_xor(wpart, 16, 64);
  wpart += __shfl_xor(wpart, 32, 64);
  if (l < 16) T.rsum[w][l] = wpart;
  __syncthreads();
  if (rowok) {
    const float wsum = T.rsum[0][n] + T.rsum[1][n] + T.rsum[2][n] + T.rsum[3][n];
    const int64_t base = (bh * p.ns + sp) * kD;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 16 * (2 * w + i) + 4 * G4 + r;
        p.pc[base + d] = accC[i][r] - wsum * p.so[bh * kD + d];   // partial c = sum W v - (sum W) o
      }
  }
}

struct DecWs {
  float *pm, *pl, *po, *pk, *so, *su, *salpha, *slse, *pc;
  int ns, chunk;
  size_t bytes;
};

DecWs dec_layout(const Geom& g, void* ws) {
  DecWs w{};
  const int slices = g.B * g.Hkv;
  const int ntiles = (g.Tk + kTile - 1) / kTile;
  // about 2048 workgroups per pass; fewer (1024) for a handful of (sequence, kv head) slices, where the
  // per-split combine costs more than the extra parallelism gains (measured at 1 and 8 sequences)
  const int target = slices < 32 ? 1024 : 2048;
  int ns = slices > 0 ? (target + slices - 1) / slices : 1;
  ns = ns < 1 ? 1 : (ns > ntiles ? ntiles : ns);
  if (ns < 1) ns = 1;
  w.ns = ns;
  w.chunk = (ntiles + ns - 1) / ns * kTile;
  char* base = static_cast<char*>(ws);
  size_t off = 0;
  const size_t bh = static_cast<size_t>(g.B) * g.Tq * g.Hq;   // one row per (sequence, new token, query head)
  w.pm = reinterpret_cast<float*>(base + ws_take(off, bh * ns * 4));
  w.pl = reinterpret_cast<float*>(base + ws_take(off, bh * ns * 4));
  w.po = reinterpret_cast<float*>(base + ws_take(off, bh * ns * kD * 4));
  w.pk = reinterpret_cast<float*>(base + ws_take(off, bh * ns * kD * 4));
  w.pc = reinterpret_cast<float*>(base + ws_take(off, bh * ns * kD * 4));
  w.so = reinterpret_cast<float*>(base + ws_take(off, bh * kD * 4));
  w.su = reinterpret_cast<float*>(base + ws_take(off, bh * kD * 4));
  w.salpha = reinterpret_cast<float*>(base + ws_take(off, bh * 4));
  w.slse = reinterpret_cast<float*>(base + ws_take(off, bh * 4));
  w.bytes = off;
  return w;
}

}  // namespace

bool fast_decode_supported(const Geom& g) {
  const int G = g.Hq / g.Hkv;
  return g.bf16 && (g.d == kD || g.d == 64) && !g.p_per_query && (G == 1 || G == 2 || G == 4 || G == 8);
}

size_t fast_decode_workspace(const Geom& g) { return dec_layout(g, nullptr).bytes; }

namespace {

// One pass kernel over every chunk of new tokens.  A chunk holds up to 16 / G tokens, so a workgroup has
// G x (tokens in the chunk) <= 16 rows; 3 to 16 rows run on the matrix-core kernels (rows padded to 16),
// 1 or 2 rows on the fp32 kernels.
template <bool PASS2, bool PAGED>
void launch_pass(DecParams p, const dim3& grid, hipStream_t stream) {
  const int per = kMaxRowsM / p.G;   // tokens per chunk at most (G is 1, 2, 4 or 8)
  for (int t0 = 0; t0 < p.T; t0 += p.Tc) {
    p.t0 = t0;
    p.Tc = min(per, p.T - t0);
    const int rows = p.G * p.Tc;
    if (!PASS2) {
      if (rows == 1) hipLaunchKernelGGL((k_dec_pass1<1, PAGED>), grid, dim3(256), 0, stream, p);
      else if (rows == 2) hipLaunchKernelGGL((k_dec_pass1<2, PAGED>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((k_dec_mpass1<PAGED>), grid, dim3(256), 0, stream, p);
    } else {
      if (rows == 1) hipLaunchKernelGGL((k_dec_pass2<1, PAGED>), grid, dim3(256), 0, stream, p);
      else if (rows == 2) hipLaunchKernelGGL((k_dec_pass2<2, PAGED>), grid, dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((k_dec_mpass2<PAGED>), grid, dim3(256), 0, stream, p);
    }
  }
}

template <bool PAGED>
void launch_all(const DecParams& p, const dim3& grid, int Hq, int BT, hipStream_t stream) {
  mark_begin(PLX_KERNEL_DECODE_PASS1, stream);
  launch_pass<false, PAGED>(p, grid, stream);
  mark_end(PLX_KERNEL_DECODE_PASS1, stream);
  hipLaunchKernelGGL(k_dec_combine1, dim3(Hq, BT), dim3(128), 0, stream, p);
  mark_begin(PLX_KERNEL_DECODE_PASS2, stream);
  launch_pass<true, PAGED>(p, grid, stream);
  mark_end(PLX_KERNEL_DECODE_PASS2, stream);
  hipLaunchKernelGGL(k_dec_finish, dim3(Hq, BT), dim3(128), 0, stream, p);
}

}  // namespace

hipError_t launch_fast_decode(const Geom& g, const void* q, const void* kc, const void* vc, const int32_t* seqlens,
                              const void* P, void* out, float* cor, void* ws, hipStream_t stream,
                              const PagedCache* paged) {
  if (decode_path() == PLX_DECODE_AUTO && moment_decode_supported(g, paged))
    return launch_moment_decode(g, q, kc, vc, seqlens, P, out, cor, stream, paged);
  const DecWs w = dec_layout(g, ws);
  DecParams p{};
  p.q = static_cast<const u16*>(q);
  p.kc = static_cast<const u16*>(kc);
  p.vc = static_cast<const u16*>(vc);
  p.P = static_cast<const u16*>(P);
  p.seqlens = seqlens;
  p.out = out;
  p.out_bf16 = g.out_bf16;
  p.cor = cor;
  p.pm = w.pm;
  p.pl = w.pl;
  p.po = w.po;
  p.pk = w.pk;
  p.so = w.so;
  p.su = w.su;
  p.salpha = w.salpha;
  p.slse = w.slse;
  p.pc = w.pc;
  p.B = g.B;
  p.L = g.Tk;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.G = g.Hq / g.Hkv;
  p.window = g.window;
  p.D = g.d;
  p.T = g.Tq;
  p.t0 = 0;
  p.Tc = g.Tq;
  p.ns = w.ns;
  p.chunk = w.chunk;
  p.scale = g.scale;
  const dim3 grid(w.ns, g.Hkv, g.B);
  if (paged) {
    p.block_table = paged->block_table;
    p.max_pages = paged->max_pages;
    p.num_pages = paged->num_pages;
    int shift = 0;
    while ((1 << shift) < paged->page_size) ++shift;
    p.page_shift = shift;
    launch_all<true>(p, grid, g.Hq, g.B * g.Tq, stream);
  } else {
    launch_all<false>(p, grid, g.Hq, g.B * g.Tq, stream);
  }
  return hipGetLastError();
}

}  // namespace plx
