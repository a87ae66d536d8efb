// Single-read Parallax decode for gfx950: one new query per sequence against a bf16 key/value cache,
// the cache read once.
//
// The pages' decode kernel lets both branches share one KV stream (gist.science technical summary of
// "Parallax: Parameterized Local Linear Attention for Language Modeling", "Hardware-aware algorithm").
// The probe u = P^T (q - kbar) needs the whole sequence's kbar, so instead of a second pass over the
// cache this kernel accumulates the softmax-weighted moment of the keys and values with them:
//   M = sum_j v_j y_j^T  with  y_j = bf16(p~_j k_j)   (d x d per query head),
//   kbar~ = sum_j y_j,   o~ = sum_j w_j v_j,   l = sum_j w_j,   w_j = bf16(p~_j),
// and after the last key  o = o~ / l,  kbar = kbar~ / l,  u = P^T (q - kbar),  alpha = u . kbar  and
//   out = o + M u / l - alpha o.
// Since sum_j w_j (v_j - o) = 0 exactly for these o and l, M u / l - alpha o = sum_j (u . y_j / l)(v_j - o):
// the correction of the definition, o + sum_j p_j (u . (k_j - kbar))(v_j - o), with y_j / l in place of
// p_j k_j.  kbar is summed from the same rounded products as M (not from exact weights times keys) so that
// this identity holds for the values actually accumulated: otherwise M u / l and alpha o, each of size
// |u . k| |v|, would cancel with a residue of bf16's rounding of p~ k times that size (about 8e-2 of the
// output's rms once scores spread over tens of units).
// M costs 2 d^2 flop per key and head, far more than the two-pass form, so it runs on the matrix cores:
// per 16 keys, M_h += V^T Y_h on v_mfma_f32_32x32x16_bf16 with the cache's bf16 rows as they are; o~ takes
// the rounded weights as a matrix of (query head) columns on the same instruction; kbar~ and l are fp32
// sums of the rounded values.
//
// One 512-thread workgroup (8 waves) owns one (sequence, key/value head) and its one or two query heads,
// so no partial results leave the workgroup and no workspace is used.  Wave w owns the key dims
// 32 (w % 4) + [0, 32) of M and the value dims of tiles 2 (w / 4), 2 (w / 4) + 1.  Key tiles of 64 rows
// arrive by direct-to-LDS DMA, four buffers deep; rows are stored 256 bytes each with the 16-byte chunks of
// row r permuted (slot = chunk ^ f(r)) so that the transpose loads (ds_read_b64_tr_b16) that form the
// k-major operands, and the row loads of the scores, hit distinct banks.  Waves 0-3 compute the next tile's
// scores (16 keys each, v_mfma_f32_16x16x32_bf16) while all waves run the current tile's products; the
// running maximum is lazy (it moves only when a tile exceeds it by 8 in log2 units).
#include <math.h>

#include "fast_common.h"
#include "plx_internal.h"

namespace plx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMT = 64;        // keys per tile
constexpr int kMBuf = 4;       // tile buffers
constexpr float kMLog2e = 1.4426950408889634f;
constexpr float kMTau = 8.f;

struct MomParams {
  const u16 *q, *kc, *vc, *P;
  const int32_t* seqlens;
  const int32_t* __restrict__ block_table;   // paged cache: [B][max_pages] (pages of >= 64 keys)
  int max_pages, page_shift, num_pages;
  void* out;       // fp32, or bf16 when out_bf16
  float* cor;      // per query head |out - o| / |out| (nullable)
  int out_bf16;
  int B, L, Hq, Hkv, window;
  float scale;
};

struct __align__(16) MomShared {
  union {
    struct {
      u16 k[kMBuf][kMT * kD];
      u16 v[kMBuf][kMT * kD];
    } t;
    float M[2][kD][kD + 1];    // epilogue: the moment of each query head, rows padded against bank conflicts
  };
  uint4 qb[4][64];             // score operands (bf16 q) per (step, lane)
  f32x4 sc[4][64];             // scaled scores of the next tile per (score wave, lane), between the two phases
  float pt[2][2][kMT];         // p~ of a tile per (buffer, head, key), fp32
  u16 pw[2][5][kMT];           // the same as bf16 pairs per (buffer, row, key): rows h = hi, HW + h = lo, 2 HW = 0
  float smax[2][4][2];         // per (buffer, score wave, head): the tile maximum (log2 units)
  float lsum[4][2];
  float vec[3][2][kD];         // epilogue: o, kbar, u per head
  float opart[2][2][kD];       // epilogue: o~ and kbar~ per (key half, head)
  float kpart[2][2][kD];
  float red[3][2][2];   // per (quantity, head, wave of the head)
};

// Chunk permutation of row r within a tile (an involution on 0..15): slot = chunk ^ f(r).
__device__ __forceinline__ int mswz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

__device__ __forceinline__ float bfv(__bf16 x) { return static_cast<float>(x); }

// Cache row of key `key` of sequence b (paged: page table lookup, the page index clamped into the pool).
template <bool PAGED>
__device__ __forceinline__ int64_t mrow(const MomParams& p, int b, int key) {
  if constexpr (PAGED) {
    // a scalar load (the entry is the same for the whole wave): it is waited for on the scalar counter,
    // not on the vector-memory counter that also counts the tile copies in flight
    const __attribute__((address_space(4))) int32_t* bt =
        (const __attribute__((address_space(4))) int32_t*)p.block_table;
    int pg = bt[static_cast<int64_t>(b) * p.max_pages + (key >> p.page_shift)];
    pg = min(max(pg, 0), p.num_pages - 1);
    return (static_cast<int64_t>(pg) << p.page_shift) + (key & ((1 << p.page_shift) - 1));
  } else {
    return static_cast<int64_t>(b) * p.L + key;
  }
}

// DMA of key tile `tile` (keys key0 .. key0 + 63, those at or past hi read the last valid key) into buffer
// buf: 16 instructions of 1 KB for K and 16 for V, four per wave.  Instruction i covers rows 4 i .. 4 i + 3;
// lane l fills slot l % 16 of row 4 i + l / 16, i.e. fetches chunk (l % 16) ^ f(row) of that row.  The rows
// of a tile are consecutive cache rows (a page holds whole tiles), so each copy is the tile's first row
// (a wave-uniform address) plus a per-lane offset: lrow[jj] = the lane's row, lchunk[jj] = its chunk's bytes.
template <bool PAGED>
__device__ __forceinline__ void mom_dma(const MomParams& p, MomShared& S, int buf, int b, int g, int key0, int hi,
                                        int w, const int (&lrow)[2], const uint32_t (&lchunk)[2]) {
  const int64_t row0 = PAGED ? mrow<true>(p, b, key0) : static_cast<int64_t>(b) * p.L + key0;
  const int64_t e0 = (row0 * p.Hkv + g) * kD;
  const int rmax = hi - 1 - key0;
  const uint32_t rs = static_cast<uint32_t>(p.Hkv) * kD * 2;   // bytes from one cache row to the next
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int i = 2 * w + jj;
    const uint32_t voff = static_cast<uint32_t>(min(lrow[jj], rmax)) * rs + lchunk[jj];
    lds_dma16_sbase(p.kc + e0, voff, &S.t.k[buf][i * 512]);
    lds_dma16_sbase(p.vc + e0, voff, &S.t.v[buf][i * 512]);
  }
}

__device__ __forceinline__ void vm_wait4() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); }

// k-major operand (32 dims of tile dt, 16 keys of k-step ks) of a 32x32x16 MFMA from a row tile in LDS:
// two transpose loads, keys 16 ks + 8 (l / 32) + [0, 4) and + [4, 8).
__device__ __forceinline__ bf16x8 mom_cols(const u16* tile, const int (&loff)[2], int lj, int ks, int dt) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const int extra = ks * 2048 + ((dt ^ lj) << 5);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + loff[0] + extra));
  const s16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(tile + loff[1] + extra));
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 ah = __builtin_bit_cast(bf16x4, a), ch = __builtin_bit_cast(bf16x4, c);
  return __builtin_shufflevector(ah, ch, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int HW, bool PAGED>
__global__ __launch_bounds__(512) void k_dec_moment(MomParams p) {
  __shared__ MomShared S;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63;
  const int G = p.Hq / p.Hkv;
  const int nslice = G / HW;   // workgroups per kv head (1: this kernel runs with HW == G)
  const int b = blockIdx.x / (p.Hkv * nslice), g = (blockIdx.x / nslice) % p.Hkv;
  const int h0 = g * G + (blockIdx.x % nslice) * HW;   // first query head of the workgroup
  int hi = p.L;
  if (p.seqlens) hi = min(max(p.seqlens[b], 0), p.L);
  const int lo = p.window > 0 ? max(0, hi - p.window) : 0;
  const int t0 = lo / kMT;
  const int nt = hi > lo ? (hi - 1) / kMT - t0 + 1 : 0;
  const float c2 = p.scale * kMLog2e;

  // score operands (waves 0-3), the same for each of them: B[k = d][n = head] of a 16x16x32 product,
  // d = 32 st + 8 (l / 16) + [0, 8), kept in LDS (16 bytes per lane and step) rather than in registers
  if (w == 0) {
    const int n = l & 15;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      uint4 raw = {0u, 0u, 0u, 0u};
      if (n < HW)
        raw = *reinterpret_cast<const uint4*>(p.q + (static_cast<int64_t>(b) * p.Hq + h0 + n) * kD + 32 * st +
                                              8 * (l >> 4));
      S.qb[st][l] = raw;
    }
  }
  // transpose-load lane offsets (see mom_cols): lane (G = l / 16, j, a) reads 4 dims of key 8 (G / 2) + j
  const int lG = l >> 4, lj = (l >> 2) & 3, la = l & 3;
  int loff[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int x = 2 * (lG & 1) + (la >> 1), y = 2 * (lG >> 1) + hh;
    loff[hh] = (8 * (lG >> 1) + lj + 4 * hh) * kD + ((x ^ y) << 3) + ((la & 1) << 2);
  }
  // score row loads (waves 0-3): key 16 w + m, chunk 4 st + l / 16
  const int sm = l & 15;
  const int soff = (16 * (w & 3) + sm) * kD;

  const int ks_strip = w & 3, kh = w >> 2;   // K dims 32 ks_strip + [0, 32); keys 32 kh + [0, 32) of each tile
  f32x16 accM[4][HW];                        // M of value tile vt (rows) x the K strip (columns), this key half
  // o~ of value tile ks_strip in columns h (hi weights of head h) and HW + h (lo), kbar~ of K strip ks_strip
  // in columns 4 + h and 4 + HW + h (two products into one accumulator, each filling only its own columns)
  f32x16 accX = f32x16{};
#pragma unroll
  for (int vt = 0; vt < 4; ++vt)
#pragma unroll
    for (int h = 0; h < HW; ++h) accM[vt][h] = f32x16{};
  float m_run[2] = {-INFINITY, -INFINITY};
  float lpart = 0.f;   // waves 0-3, lanes l % 16 < HW: weights of head l % 16

  // scores of tile `tile` (waves 0-3) -> their keys' values in registers and the wave's maxima in LDS
  auto scores = [&](int tile, int buf) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const u16* kt = S.t.k[buf];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int slot = 4 * (st ^ (sm & 3)) + ((l >> 4) ^ (sm >> 2));
      const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kt + soff + slot * 8));
      const bf16x8 qv = __builtin_bit_cast(bf16x8, S.qb[st][l]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qv, acc, 0, 0, 0);
    }
    const int key0 = (t0 + tile) * kMT + 16 * (w & 3) + 4 * (l >> 4);
    float mx = -INFINITY;
    f32x4 sc;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + r;
      sc[r] = key >= lo && key < hi ? acc[r] * c2 : -INFINITY;
      mx = fmaxf(mx, sc[r]);
    }
    S.sc[w & 3][l] = sc;   // (in LDS across the products, not in registers)
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (l < HW) S.smax[tile & 1][w & 3][l] = mx;
  };
  // after the barrier: the tile's maximum per head, the lazy running maximum, the accumulators' rescale,
  // and (waves 0-3) the tile's weights into LDS
  auto weights = [&](int tile) {
    float f[2] = {1.f, 1.f};
    bool any = false;
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      // (the same value in every lane: kept in scalar registers)
      const float tm = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(
          fmaxf(fmaxf(S.smax[tile & 1][0][h], S.smax[tile & 1][1][h]),
                fmaxf(S.smax[tile & 1][2][h], S.smax[tile & 1][3][h])))));
      if (tm > m_run[h] + kMTau) {
        f[h] = m_run[h] == -INFINITY ? 0.f : exp2f(m_run[h] - tm);
        m_run[h] = tm;
        any = true;
      }
    }
    if (any) {   // (uniform: every wave reads the same maxima)
#pragma unroll
      for (int vt = 0; vt < 4; ++vt)
#pragma unroll
        for (int h = 0; h < HW; ++h) accM[vt][h] *= f[h];
      const int n = l & 31;   // accX column n (< 8): head n % HW
      accX *= (HW == 2 && (n & 1)) ? f[HW - 1] : f[0];
      const int n16 = l & 15;
      lpart *= (HW == 2 && n16 == 1) ? f[HW - 1] : f[0];
    }
    if (w < 4) {
      const int n = l & 15;
      if (n < HW) {
        const float mr = n == 0 ? m_run[0] : m_run[HW - 1];
        const float mb = mr == -INFINITY ? 0.f : mr;
        const f32x4 sc = S.sc[w][l];
        float e[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = sc[r] == -INFINITY ? 0.f : exp2f(sc[r] - mb);
          lpart += e[r];
        }
        const int k4 = 16 * w + 4 * (l >> 4);
        *reinterpret_cast<float4*>(&S.pt[tile & 1][n][k4]) = float4{e[0], e[1], e[2], e[3]};
        // the weights as bf16 pairs hi + lo: rows n and HW + n of the o~ operand
        uint32_t hw[2], lw[2];
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const uint32_t h0 = f32_to_bf16(e[r]), h1 = f32_to_bf16(e[r + 1]);
          hw[r / 2] = h0 | (h1 << 16);
          lw[r / 2] = f32_to_bf16(e[r] - __uint_as_float(h0 << 16)) |
                      (f32_to_bf16(e[r + 1] - __uint_as_float(h1 << 16)) << 16);
        }
        *reinterpret_cast<uint2*>(&S.pw[tile & 1][n][k4]) = uint2{hw[0], hw[1]};
        *reinterpret_cast<uint2*>(&S.pw[tile & 1][HW + n][k4]) = uint2{lw[0], lw[1]};
      }
    }
  };

  // weight rows of the two o~ / kbar~ operands (columns 0 .. 2 HW - 1 and 4 .. 4 + 2 HW - 1; zero row 2 HW)
  const int pw_row = min(l & 31, 2 * HW);
  const int pw_row2 = (l & 31) >= 4 && (l & 31) < 4 + 2 * HW ? (l & 31) - 4 : 2 * HW;
  // the lane's rows and chunk offsets in the tile copies
  int lrow[2];
  uint32_t lchunk[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    lrow[jj] = 4 * (2 * w + jj) + (l >> 4);
    lchunk[jj] = 16u * static_cast<uint32_t>((l & 15) ^ mswz(lrow[jj]));
  }
  for (int i = tid; i < 2 * (5 - 2 * HW) * kMT; i += 512)   // the zero rows of both buffers
    S.pw[i / ((5 - 2 * HW) * kMT)][2 * HW + (i / kMT) % (5 - 2 * HW)][i % kMT] = 0;

  // ---- prologue: tiles 0, 1, 2 in flight, scores and weights of tile 0 ----
  vm_wait_all();   // q and seqlens have arrived (no load of ours is in flight across the loop's waits)
#pragma unroll
  for (int tt = 0; tt < 3; ++tt)
    if (tt < nt) mom_dma<PAGED>(p, S, tt, b, g, (t0 + tt) * kMT, hi, w, lrow, lchunk);
  if (nt > 0) {
    if (nt > 2) {
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");   // tile 0 (tiles 1 and 2 may stay in flight)
    } else {
      lds_dma_wait();
    }
    lds_barrier();
    if (w < 4) scores(0, 0);
    lds_barrier();
    weights(0);
  }

  for (int t = 0; t < nt; ++t) {
    const int buf = t % kMBuf, nbuf = (t + 1) % kMBuf;
    // tile t + 1 has arrived (tile t + 2 may still be in flight); every wave is done with tile t - 1
    if (t + 2 < nt) vm_wait4();
    else lds_dma_wait();
    lds_barrier();
    if (t + 3 < nt) mom_dma<PAGED>(p, S, (t + 3) % kMBuf, b, g, (t0 + t + 3) * kMT, hi, w, lrow, lchunk);
    if (w < 4 && t + 1 < nt) scores(t + 1, nbuf);
    // products of tile t: this wave's key half, two steps of 16 keys (ks = 2 kh, 2 kh + 1), each step once
    // per head.  The bf16 pair y = p~ k of the next (step, head) is formed while the matrix cores run the
    // current one's 8 products (the scheduling groups below interleave them).
    const u16* kt = S.t.k[buf];
    const u16* vt16 = S.t.v[buf];
    const float* pt = &S.pt[t & 1][0][0];
    constexpr int NS = 2 * HW;
    // y of (step i / HW, head i % HW) for the lane's 8 keys 16 ks + 8 (l / 32) + [0, 8) and K dim
    // 32 ks_strip + l % 32 as a bf16 pair: hi = y truncated to bf16 (the top 16 bits), lo = the exact
    // remainder (below 2^-7 |y|) rounded to bf16, so hi + lo is y to about 2^-16 relative.  `ak` returns the
    // step's K operand (the A operand of kbar~).
    auto ystep = [&](int i, bf16x8& yh, bf16x8& yl, bf16x8& ak) {
      const int ks = 2 * kh + i / HW, h = i % HW;
      ak = mom_cols(kt, loff, lj, ks, ks_strip);
      const u32x4 kw = __builtin_bit_cast(u32x4, ak);
      const int kk = 16 * ks + 8 * (l >> 5);
      const float4 p0 = *reinterpret_cast<const float4*>(pt + h * kMT + kk);
      const float4 p1 = *reinterpret_cast<const float4*>(pt + h * kMT + kk + 4);
      const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      u32x4 hw, lw;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float y0 = pv[2 * e2] * __uint_as_float(kw[e2] << 16);
        const float y1 = pv[2 * e2 + 1] * __uint_as_float(kw[e2] & 0xffff0000u);
        const uint32_t b0 = __float_as_uint(y0), b1 = __float_as_uint(y1);
        hw[e2] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);   // the high halves of y0 (low) and y1 (high)
        const f32x2 r = {y0 - __uint_as_float(b0 & 0xffff0000u), y1 - __uint_as_float(b1 & 0xffff0000u)};
        lw[e2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
      }
      yh = __builtin_bit_cast(bf16x8, hw);
      yl = __builtin_bit_cast(bf16x8, lw);
    };
    bf16x8 yh, yl, akc;
    ystep(0, yh, yl, akc);
    bf16x8 av[4], avs, bo, bo2;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int ks = 2 * kh + i / HW, h = i % HW;
      if (h == 0) {
#pragma unroll
        for (int vt = 0; vt < 4; ++vt) av[vt] = mom_cols(vt16, loff, lj, ks, vt);
        avs = mom_cols(vt16, loff, lj, ks, ks_strip);
        // B operands of o~ and kbar~: the weight rows (hi, lo per head, zeros) of the lane's column
        const int kk = 16 * ks + 8 * (l >> 5);
        bo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&S.pw[t & 1][pw_row][kk]));
        bo2 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(&S.pw[t & 1][pw_row2][kk]));
      }
      __builtin_amdgcn_sched_barrier(0);
      // (hi products first, so that two products into one accumulator are not back to back)
#pragma unroll
      for (int vt = 0; vt < 4; ++vt)
        accM[vt][h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[vt], yh, accM[vt][h], 0, 0, 0);
      if (h == 0) accX = __builtin_amdgcn_mfma_f32_32x32x16_bf16(avs, bo, accX, 0, 0, 0);
#pragma unroll
      for (int vt = 0; vt < 4; ++vt)
        accM[vt][h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[vt], yl, accM[vt][h], 0, 0, 0);
      if (h == 0) accX = __builtin_amdgcn_mfma_f32_32x32x16_bf16(akc, bo2, accX, 0, 0, 0);
      if (i + 1 < NS) {
        bf16x8 yh2, yl2, ak2;
        ystep(i + 1, yh2, yl2, ak2);
        // the next step's LDS reads first, then each product followed by a share of the VALU work
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        yh = yh2;
        yl = yl2;
        akc = ak2;
      }
    }
    lds_barrier();   // the next tile's maxima are in LDS
    if (t + 1 < nt) weights(t + 1);
  }

  // ---- epilogue ----
  // the two key halves of each partial: o~ and kbar~ through LDS, M added in place
  {
    float lp = lpart;
    lp += __shfl_xor(lp, 16, 64);
    lp += __shfl_xor(lp, 32, 64);
    if (w < 4 && l < HW) S.lsum[w][l] = lp;
    // o~ of value tile ks_strip: accumulator row 8 (r / 4) + 4 (l / 32) + r % 4 of column l % 32; the hi
    // and lo columns of a head are HW lanes apart
    const int n = l & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float other = __shfl(accX[r], l + HW, 64);
      if (n < HW) S.opart[kh][n][32 * ks_strip + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3)] = accX[r] + other;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {   // kbar~ of K strip ks_strip: columns 4 + h and 4 + HW + h
      const float other = __shfl(accX[r], l + HW, 64);
      if (n >= 4 && n < 4 + HW) S.kpart[kh][n - 4][32 * ks_strip + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3)] = accX[r] + other;
    }
  }
  // the moment: the second key half writes its partial (the tile buffers are free: every copy has completed
  // and every wave has passed the loop's last barrier after its last read)
  auto mrow_of = [&](int vt, int r) { return 32 * vt + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3); };
  if (kh == 1) {
#pragma unroll
    for (int vt = 0; vt < 4; ++vt)
#pragma unroll
      for (int h = 0; h < HW; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) S.M[h][mrow_of(vt, r)][32 * ks_strip + (l & 31)] = accM[vt][h][r];
  }
  __syncthreads();
  float Lh[2];
#pragma unroll
  for (int h = 0; h < HW; ++h) Lh[h] = S.lsum[0][h] + S.lsum[1][h] + S.lsum[2][h] + S.lsum[3][h];
  if (kh == 0) {
#pragma unroll
    for (int vt = 0; vt < 4; ++vt)
#pragma unroll
      for (int h = 0; h < HW; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) S.M[h][mrow_of(vt, r)][32 * ks_strip + (l & 31)] += accM[vt][h][r];
  }
  // o and kbar: thread (h, a) of the first HW * 128
  const int eh = tid >> 7, ea = tid & 127;
  if (eh < HW) {
    const float ln = eh == 0 ? Lh[0] : Lh[HW - 1];
    const float inv = ln > 0.f ? 1.f / ln : 0.f;
    S.vec[0][eh][ea] = (S.opart[0][eh][ea] + S.opart[1][eh][ea]) * inv;
    S.vec[1][eh][ea] = (S.kpart[0][eh][ea] + S.kpart[1][eh][ea]) * inv;
  }
  __syncthreads();
  // u = P^T (q - kbar) and alpha = u . kbar
  float uval = 0.f, aval = 0.f;
  if (eh < HW) {
    const int hq = h0 + eh;
    const u16* qrow = p.q + (static_cast<int64_t>(b) * p.Hq + hq) * kD;
    const u16* Ph = p.P + static_cast<int64_t>(hq) * kD * kD;
#pragma unroll 8
    for (int bb = 0; bb < kD; ++bb)
      uval = fmaf(bf16_to_f32(Ph[bb * kD + ea]), bf16_to_f32(qrow[bb]) - S.vec[1][eh][bb], uval);   // u[a] = sum_b P[b][a] x[b]
    aval = uval * S.vec[1][eh][ea];
#pragma unroll
    for (int o2 = 32; o2 > 0; o2 >>= 1) aval += __shfl_xor(aval, o2, 64);
    if (l == 0) S.red[0][eh][(tid >> 6) & 1] = aval;
    S.vec[2][eh][ea] = uval;
  }
  __syncthreads();
  if (eh < HW) {
    const float alpha = S.red[0][eh][0] + S.red[0][eh][1];
    const float ln = eh == 0 ? Lh[0] : Lh[HW - 1];
    const float inv = ln > 0.f ? 1.f / ln : 0.f;
    float mu = 0.f;
#pragma unroll 8
    for (int bb = 0; bb < kD; ++bb) mu = fmaf(S.M[eh][ea][bb], S.vec[2][eh][bb], mu);
    const float o = S.vec[0][eh][ea];
    const float cval = mu * inv - alpha * o;
    const float r = o + cval;
    const int64_t oi = (static_cast<int64_t>(b) * p.Hq + h0 + eh) * kD + ea;
    if (p.out_bf16) static_cast<u16*>(p.out)[oi] = static_cast<u16>(f32_to_bf16(r));
    else static_cast<float*>(p.out)[oi] = r;
    if (p.cor) {
      float cc = cval * cval, oo = r * r;
#pragma unroll
      for (int o2 = 32; o2 > 0; o2 >>= 1) {
        cc += __shfl_xor(cc, o2, 64);
        oo += __shfl_xor(oo, o2, 64);
      }
      if (l == 0) {
        S.red[1][eh][(tid >> 6) & 1] = cc;
        S.red[2][eh][(tid >> 6) & 1] = oo;
      }
    }
  }
  if (p.cor) {
    __syncthreads();
    if (eh < HW && ea == 0) {
      const float C = S.red[1][eh][0] + S.red[1][eh][1], O = S.red[2][eh][0] + S.red[2][eh][1];
      p.cor[static_cast<int64_t>(b) * p.Hq + h0 + eh] = O > 0.f ? sqrtf(C / O) : 0.f;
    }
  }
}

}  // namespace

// One workgroup per (sequence, kv head) and one workgroup per CU: below two workgroups per CU the split-KV
// passes, which spread each sequence over many workgroups, are faster (measured: 128 pairs 1.11 ms against
// 0.82 ms two-pass; 256 and 512 pairs 5-12% faster than two-pass).
constexpr int64_t kMomentMinSlices = 256;

bool moment_decode_supported(const Geom& g, const PagedCache* paged) {
  const int G = g.Hq / g.Hkv;
  return g.bf16 && g.d == kD && !g.p_per_query && g.Tq == 1 && (G == 1 || G == 2) &&
         (!paged || paged->page_size >= kMT) && static_cast<int64_t>(g.B) * g.Hkv >= kMomentMinSlices;
}

hipError_t launch_moment_decode(const Geom& g, const void* q, const void* kc, const void* vc, const int32_t* seqlens,
                                const void* P, void* out, float* cor, hipStream_t stream, const PagedCache* paged) {
  MomParams p{};
  p.q = static_cast<const u16*>(q);
  p.kc = static_cast<const u16*>(kc);
  p.vc = static_cast<const u16*>(vc);
  p.P = static_cast<const u16*>(P);
  p.seqlens = seqlens;
  p.out = out;
  p.cor = cor;
  p.out_bf16 = g.out_bf16;
  p.B = g.B;
  p.L = g.Tk;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.window = g.window;
  p.scale = g.scale;
  const int G = g.Hq / g.Hkv;
  const dim3 grid(g.B * g.Hkv), block(512);
  mark_begin(PLX_KERNEL_DECODE_MOMENT, stream);
  if (paged) {
    p.block_table = paged->block_table;
    p.max_pages = paged->max_pages;
    p.num_pages = paged->num_pages;
    int shift = 0;
    while ((1 << shift) < paged->page_size) ++shift;
    p.page_shift = shift;
    if (G == 2) hipLaunchKernelGGL((k_dec_moment<2, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((k_dec_moment<1, true>), grid, block, 0, stream, p);
  } else {
    if (G == 2) hipLaunchKernelGGL((k_dec_moment<2, false>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((k_dec_moment<1, false>), grid, block, 0, stream, p);
  }
  mark_end(PLX_KERNEL_DECODE_MOMENT, stream);
  return hipGetLastError();
}

}  // namespace plx
