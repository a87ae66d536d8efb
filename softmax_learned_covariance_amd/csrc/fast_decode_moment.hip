// Single-read Parallax decode for gfx950: one new query per sequence against a bf16 key/value cache,
// the cache read once.
//
// The pages' decode kernel lets both branches share one KV stream (gist.science technical summary of
// "Parallax: Parameterized Local Linear Attention for Language Modeling", "Hardware-aware algorithm").
// The probe u = P^T (q - kbar) needs the whole sequence's kbar, so instead of a second pass over the
// cache this kernel accumulates the softmax-weighted moment of the keys and values with them:
//   M = sum_j v_j y_j^T,  kbar~ = sum_j y_j  with  y_j = fp16(p~_j k_j)   (d x d per query head),
//   o~ = sum_j p~_j v_j,  l = sum_j p~_j,
// and after the last key  o = o~ / l,  kbar = kbar~ / l,  u = P^T (q - kbar),  alpha = u . kbar  and
//   out = o + M u / l - alpha o  =  o + sum_j (u . y_j / l)(v_j - o).
// kbar is summed from the same rounded products as M, so that M u / l - alpha o is exactly that sum for
// the values accumulated: each of the two terms is of size |u . k| |v| and they cancel, and a kbar from
// unrounded products would leave the rounding of p~ k times that size.  The correction of the definition,
// sum_j p_j (u . (k_j - kbar))(v_j - o), differs from it only through the rounding of y (fp16: 2^-11
// relative per element).  Where the two terms exceed the output by more than 2^11 (a key far larger than the
// rest dominates), fp32 alone would lose the difference; such a head's correction is then formed directly
// from a second read of its keys.
//
// M costs 2 d^2 flop per key and head, far more than the two-pass form, so it runs on the matrix cores:
// per 16 keys and head, M += V^T Y on v_mfma_f32_32x32x16_f16, plus one product for kbar~ (a ones row
// against Y) and, per 16 keys, one for o~ (the weights as fp16 hi + lo rows against V).  The cache is
// bf16: each value tile is converted in LDS to fp16 times 2^ev, and y is formed as fp16(p~ 2^ek k), with
// power-of-two scales set from each tile's largest magnitudes so that |v| 2^ev < 2^14 and |k| 2^ek < 2^7
// (p~ <= 2^8, so y < 2^15).  The scales only decrease along the sequence: a tile that needs a smaller one
// rescales the accumulators by the exact power of two.  Values down to 2^-27 of the largest seen so far
// keep fp16's full precision, and the output scales exactly with V (and with K at unchanged scores).
//
// One 512-thread workgroup (8 waves) owns one (sequence, key/value head) and its one or two query heads,
// so no partial results leave the workgroup and no workspace is used.  Wave w owns the key dims
// 32 (w % 4) + [0, 32) of M, and keys 32 (w / 4) + [0, 32) of every tile for all 128 value dims.  Key
// tiles of 64 rows arrive by direct-to-LDS DMA, four buffers deep; rows are stored 256 bytes each with the
// 16-byte chunks of row r permuted (slot = chunk ^ f(r)) so that the transpose loads (ds_read_b64_tr_b16)
// that form the k-major operands, and the row loads of the scores, hit distinct banks.  In the phase that
// runs the current tile's products, waves 0-3 first compute the next tile's scores (16 keys each,
// v_mfma_f32_16x16x32_bf16) and its largest |k|, waves 4-7 its largest |v|; after a barrier every wave
// sets the next tile's scales, waves 0-3 its weights (one key and head per lane), and all waves convert
// their share of its values.  The running maximum is lazy (it moves only when a tile exceeds it by 8 in
// log2 units).
#include <math.h>

#include <type_traits>

#include "fast_common.h"
#include "plx_internal.h"

namespace plx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2v __attribute__((ext_vector_type(2)));

constexpr int kMT = 64;        // keys per tile
constexpr int kMBuf = 4;       // tile buffers
constexpr float kMLog2e = 1.4426950408889634f;
constexpr float kMTau = 8.f;
// scale exponents before the first tile that sets them: the largest either rule can ask for (a bf16
// magnitude of at least 2^-126; for k capped so that p~ 2^ek stays finite)
constexpr int kEk0 = 110, kEv0 = 139;

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
      u16 k[kMBuf][kMT * kD];   // bf16 as copied
      u16 v[kMBuf][kMT * kD];   // bf16 as copied, then fp16 times 2^ev (converted in place)
    } t;
    float M[2][kD][kD + 1];    // epilogue: the moment of each query head, rows padded against bank conflicts
    struct {
      float wj[512];        // p_j u.(k_j - kbar) of a batch of 512 keys
      float cacc[4][kD];    // the correction's partial sums per quarter of a batch
    } fb;                   // epilogue, after M: the direct correction of a head (see there)
  };
  uint4 qb[4][64];             // score operands (bf16 q) per (step, lane)
  f32x4 sc[4][64];             // scaled scores of the next tile per (score wave, lane), between the two phases
  float pt[2][2][kMT];         // p~ 2^ek of a tile per (buffer, head, key)
  u16 pw[2][5][kMT];           // p~ as fp16 pairs per (buffer, row, key): rows h = hi, HW + h = lo, 2 HW = 0
  float smax[2][2][16];        // per (buffer, head, 4 score wave + lane row): the largest of 4 keys (log2 units)
  uint32_t amax[2][8];         // per (buffer, wave): largest |k| (waves 0-3, low half) or |v| (4-7, high half)
  float lsum[4][2];
  float vec[3][2][kD];         // epilogue: o, kbar, u per head
  float opart[2][2][kD];       // epilogue: o~ and kbar~ per (key half, head)
  float kpart[2][2][kD];
  float red[5][2][2];   // per (quantity, head, wave of the head)
  float qf[2][kD];      // epilogue: q per head, fp32
};

// Chunk permutation of row r within a tile (an involution on 0..15): slot = chunk ^ f(r).
__device__ __forceinline__ int mswz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

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

// k-major operand (32 dims, 16 keys) of a 32x32x16 MFMA from a row tile in LDS: two transpose loads at the
// lane's offsets o[0], o[1] from `base` (keys 8 (l / 32) + [0, 4) and + [4, 8) of the 16).
__device__ __forceinline__ u32x4 mom_cols(const u16* base, const int (&o)[2]) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + o[0]));
  const s16x4 c = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + o[1]));
  return __builtin_bit_cast(u32x4, __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A wave-uniform float as the scalar register it is.
__device__ __forceinline__ float uniform_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Largest of each 16-bit half (unsigned), and its wave-wide reduction (every lane gets the result).
__device__ __forceinline__ uint32_t pkmax(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2v, a),
                                                                 __builtin_bit_cast(u16x2v, b)));
}
// Wave-wide reduction through DPP moves (no LDS round trips): swaps within quads, the half-row and row
// mirrors leave every lane of a row of 16 with the row's result; broadcasts of lane 15 of rows 0 and 2 into
// rows 1 and 3, then of lane 31 into rows 2 and 3, leave lane 63 with the wave's.
__device__ __forceinline__ uint32_t pkmax_wave63(uint32_t x) {
  auto step = [&](uint32_t v, auto ctrl, auto rows) {
    const int m = __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), decltype(ctrl)::value,
                                              decltype(rows)::value, 0xf, false);
    return pkmax(v, static_cast<uint32_t>(m));
  };
  x = step(x, std::integral_constant<int, 0xB1>{}, std::integral_constant<int, 0xf>{});    // quad_perm 1,0,3,2
  x = step(x, std::integral_constant<int, 0x4E>{}, std::integral_constant<int, 0xf>{});    // quad_perm 2,3,0,1
  x = step(x, std::integral_constant<int, 0x141>{}, std::integral_constant<int, 0xf>{});   // row_half_mirror
  x = step(x, std::integral_constant<int, 0x140>{}, std::integral_constant<int, 0xf>{});   // row_mirror
  x = step(x, std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xa>{});   // row_bcast:15
  x = step(x, std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xc>{});   // row_bcast:31
  return x;
}

// The two bf16 halves of x as floats times 2^e, rounded to an fp16 pair.
__device__ __forceinline__ uint32_t bf16pair_to_f16(uint32_t x, int e) {
  const f32x2 f = {__builtin_amdgcn_ldexpf(__uint_as_float(x << 16), e),
                   __builtin_amdgcn_ldexpf(__uint_as_float(x & 0xffff0000u), e)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
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
  const int ks_strip = w & 3, kh = w >> 2;   // K dims 32 ks_strip + [0, 32); keys 32 kh + [0, 32) of each tile
  // transpose-load lane offsets: lane (G = l / 16, j, a) reads 4 dims of key 8 (G / 2) + j (+ 4 for the
  // second load) of dim tile dt; ov[dt] for the value tiles, os for the wave's K (and V) strip
  int ov[4][2], os[2];
  {
    const int lG = l >> 4, lj = (l >> 2) & 3, la = l & 3;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int x = 2 * (lG & 1) + (la >> 1), y = 2 * (lG >> 1) + hh;
      const int base = (8 * (lG >> 1) + lj + 4 * hh) * kD + ((x ^ y) << 3) + ((la & 1) << 2);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) ov[dt][hh] = base + ((dt ^ lj) << 5);
      os[hh] = base + ((ks_strip ^ lj) << 5);
    }
  }
  // score row loads (waves 0-3): key 16 w + m, chunk 4 st + l / 16
  const int sm = l & 15;
  const int soff = (16 * (w & 3) + sm) * kD;

  f32x16 accM[4][HW];   // M of value tile vt (rows) x the K strip (columns), this key half, times 2^(ek + ev)
  // rows h and HW + h: o~ of head h from the hi and lo weights (times 2^ev), over the V strip's dims
  // (columns); row 4 + h: kbar~ of head h (times 2^ek) over the K strip's dims.  Rows 8 and up stay zero.
  f32x16 accX = f32x16{};
#pragma unroll
  for (int vt = 0; vt < 4; ++vt)
#pragma unroll
    for (int h = 0; h < HW; ++h) accM[vt][h] = f32x16{};
  // A operand that sums Y over keys into row 4 + h: ones in that row
  f16x8 ones[HW];
#pragma unroll
  for (int h = 0; h < HW; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[h][e] = (l & 31) == 4 + h ? static_cast<_Float16>(1.f) : static_cast<_Float16>(0.f);
  float m_run[2] = {-INFINITY, -INFINITY};
  float lpart = 0.f;   // waves 0-3, lanes l < 16 HW: weights of head l / 16 (keys l % 16 of the wave's 16)
  int ek = kEk0, ev = kEv0;   // the current scales' exponents (wave-uniform)

  // scores of tile `tile` (waves 0-3) -> their keys' values and each lane's maximum (4 keys) in LDS
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
    if ((l & 15) < HW) S.smax[tile & 1][l & 15][4 * (w & 3) + (l >> 4)] = mx;
  };
  // largest |k| (waves 0-3) or |v| (waves 4-7) of the tile in buffer buf as bf16 bits, 64 bytes per thread;
  // kept in the low (k) or high (v) half of the wave's entry
  auto absmax = [&](int tile, int buf) {
    const int j = tid & 255;
    const uint4* src = reinterpret_cast<const uint4*>(w < 4 ? S.t.k[buf] : S.t.v[buf]);
    uint32_t m = 0u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint4 a = src[j + 256 * r];
      m = pkmax(pkmax(m, a.x & 0x7fff7fffu), pkmax(a.y & 0x7fff7fffu, pkmax(a.z & 0x7fff7fffu, a.w & 0x7fff7fffu)));
    }
    m = pkmax_wave63(m);
    const uint32_t m1 = max(m & 0xffffu, m >> 16);
    if (l == 63) S.amax[tile & 1][w] = w < 4 ? m1 : m1 << 16;
  };
  // after the barrier that publishes a tile's maxima (the same values in every wave, kept in scalar
  // registers): its scales, the lazy running maximum, and the factors f (per head) that the accumulators
  // take before the tile's products; `any` when one of them moved
  float f[2] = {1.f, 1.f};
  int rk = 0, rv = 0;
  bool any = false;
  auto decide = [&](int tile) {
    {
      const uint4 a = *reinterpret_cast<const uint4*>(&S.amax[tile & 1][0]);
      const uint4 c = *reinterpret_cast<const uint4*>(&S.amax[tile & 1][4]);
      const uint32_t x = __builtin_amdgcn_readfirstlane(
          pkmax(pkmax(pkmax(a.x, a.y), pkmax(a.z, a.w)), pkmax(pkmax(c.x, c.y), pkmax(c.z, c.w))));
      const int kb = static_cast<int>(x & 0xffffu), vb = static_cast<int>(x >> 16);
      // largest magnitude below 2^(E + 1) (E = biased exponent - 127; subnormals as E = -126)
      const int nk = kb ? min(ek, 133 - max(kb >> 7, 1)) : ek;   // |k| 2^ek < 2^7
      const int nv = vb ? min(ev, 140 - max(vb >> 7, 1)) : ev;   // |v| 2^ev < 2^14
      rk = nk - ek;
      rv = nv - ev;
      ek = nk;
      ev = nv;
    }
    f[0] = f[1] = 1.f;
    any = (rk | rv) != 0;
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      const float4* sm = reinterpret_cast<const float4*>(S.smax[tile & 1][h]);
      const float4 a0 = sm[0], a1 = sm[1], a2 = sm[2], a3 = sm[3];
      const float m4 = fmaxf(fmaxf(fmaxf(a0.x, a0.y), fmaxf(a0.z, a0.w)), fmaxf(fmaxf(a1.x, a1.y), fmaxf(a1.z, a1.w)));
      const float n4 = fmaxf(fmaxf(fmaxf(a2.x, a2.y), fmaxf(a2.z, a2.w)), fmaxf(fmaxf(a3.x, a3.y), fmaxf(a3.z, a3.w)));
      const float tm = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(fmaxf(m4, n4))));
      if (tm > m_run[h] + kMTau) {
        f[h] = m_run[h] == -INFINITY ? 0.f : exp2f(m_run[h] - tm);
        m_run[h] = tm;
        any = true;
      }
    }
  };
  // (waves 0-3) the tile's weights into LDS and the running sums l: lane l < 16 HW takes key 16 w + l % 16
  // of head l / 16 (its scaled score is element key % 4 of lane 16 (key / 4) + head of the scores)
  auto weights = [&](int tile) {
    const int kq = l & 15, n = (l >> 4) & 1;
    // (the per-lane choice between two uniform values, each read first as a scalar: a select between two
    // elements of a register array would become an indexed access, which the compiler moves to LDS)
    const float fl = n ? uniform_f(f[HW - 1]) : uniform_f(f[0]);
    lpart *= fl;
    if (l < 16 * HW) {
      const float mr = n ? uniform_f(m_run[HW - 1]) : uniform_f(m_run[0]);
      const float mb = mr == -INFINITY ? 0.f : mr;
      const float sc = reinterpret_cast<const float*>(&S.sc[w][16 * (kq >> 2) + n])[kq & 3];
      const float e = sc == -INFINITY ? 0.f : exp2f(sc - mb);
      lpart += e;
      const int key = 16 * w + kq;
      S.pt[tile & 1][n][key] = __builtin_amdgcn_ldexpf(e, ek);
      // the weight as an fp16 pair hi + lo: rows n and HW + n of the o~ operand
      const _Float16 hv = static_cast<_Float16>(e);
      const _Float16 lv = static_cast<_Float16>(e - static_cast<float>(hv));
      S.pw[tile & 1][n][key] = __builtin_bit_cast(u16, hv);
      S.pw[tile & 1][HW + n][key] = __builtin_bit_cast(u16, lv);
    }
  };
  // the accumulators into the next tile's scales (after the current tile's products)
  auto rescale = [&]() {
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      const float fm = __builtin_amdgcn_ldexpf(f[h], rk + rv);
#pragma unroll
      for (int vt = 0; vt < 4; ++vt) accM[vt][h] *= fm;
    }
    // rows 0-3 (lanes < 32): o~ of head r % HW; rows 4-7 (lanes >= 32): kbar~ of head r
#pragma unroll
    for (int r = 0; r < 4; ++r) accX[r] *= __builtin_amdgcn_ldexpf(f[r % HW], l < 32 ? rv : rk);
  };
  // the thread's 32 bytes of the value tile in buffer buf: bf16 -> fp16 times 2^ev, in place
  auto convert_v = [&](int buf) {
    uint4* vp = reinterpret_cast<uint4*>(S.t.v[buf]);
    const uint4 a = vp[tid], c = vp[tid + 512];
    vp[tid] = uint4{bf16pair_to_f16(a.x, ev), bf16pair_to_f16(a.y, ev), bf16pair_to_f16(a.z, ev),
                    bf16pair_to_f16(a.w, ev)};
    vp[tid + 512] = uint4{bf16pair_to_f16(c.x, ev), bf16pair_to_f16(c.y, ev), bf16pair_to_f16(c.z, ev),
                          bf16pair_to_f16(c.w, ev)};
  };

  // weight rows of the o~ operand (rows 0 .. 2 HW - 1; zero row 2 HW for the rest)
  const int pw_row = min(l & 31, 2 * HW);
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

  // ---- prologue: tiles 0, 1, 2 in flight; scores, scales, weights and values of tile 0 ----
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
    absmax(0, 0);
    lds_barrier();
    decide(0);
    if (w < 4) weights(0);
    convert_v(0);
  }

  for (int t = 0; t < nt; ++t) {
    const int buf = t % kMBuf, nbuf = (t + 1) % kMBuf;
    const bool next = t + 1 < nt;
    // tile t + 1 has arrived (tile t + 2 may still be in flight); tile t's values are converted; every wave
    // is done with tile t - 1
    if (t + 2 < nt) vm_wait4();
    else lds_dma_wait();
    lds_barrier();
    if (t + 3 < nt) mom_dma<PAGED>(p, S, (t + 3) % kMBuf, b, g, (t0 + t + 3) * kMT, hi, w, lrow, lchunk);
    // The next tile's scores (waves 0-3) and largest magnitudes, then the products of tile t:
    // this wave's key half, two steps of 16 keys, each step once per head.  The y of the next (step, head)
    // is formed while the matrix cores run the current one's products (the scheduling groups below
    // interleave them).
    const u16* kb16 = S.t.k[buf] + kh * (32 * kD);
    const u16* vb16 = S.t.v[buf] + kh * (32 * kD);
    const float* pt = &S.pt[t & 1][0][0];
    constexpr int NS = 2 * HW;
    // the K strip of step s: key 32 kh + 16 s + 8 (l / 32) + e, dim 32 ks_strip + l % 32, as floats
    auto kload = [&](int s, float (&kf)[8]) {
      const u32x4 kw = mom_cols(kb16 + s * (16 * kD), os);
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        kf[2 * e2] = __uint_as_float(kw[e2] << 16);
        kf[2 * e2 + 1] = __uint_as_float(kw[e2] & 0xffff0000u);
      }
    };
    // y = fp16(p~ 2^ek k) of (step s, head h)
    auto yform = [&](int s, int h, const float (&kf)[8]) {
      const int kk = 32 * kh + 16 * s + 8 * (l >> 5);
      const float4 p0 = *reinterpret_cast<const float4*>(pt + h * kMT + kk);
      const float4 p1 = *reinterpret_cast<const float4*>(pt + h * kMT + kk + 4);
      const f32x2 y01 = {p0.x * kf[0], p0.y * kf[1]}, y23 = {p0.z * kf[2], p0.w * kf[3]};
      const f32x2 y45 = {p1.x * kf[4], p1.y * kf[5]}, y67 = {p1.z * kf[6], p1.w * kf[7]};
      const f16x2 a = __builtin_convertvector(y01, f16x2), c = __builtin_convertvector(y23, f16x2);
      const f16x2 d = __builtin_convertvector(y45, f16x2), e = __builtin_convertvector(y67, f16x2);
      const f16x4 ac = __builtin_shufflevector(a, c, 0, 1, 2, 3), de = __builtin_shufflevector(d, e, 0, 1, 2, 3);
      return __builtin_shufflevector(ac, de, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    if (next) {
      if (w < 4) scores(t + 1, nbuf);
      absmax(t + 1, nbuf);
    }
    float kf[8];
    kload(0, kf);
    f16x8 y = yform(0, 0, kf);
    f16x8 av[4], avs, wo;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int s = i / HW, h = i % HW;
      if (h == 0) {
#pragma unroll
        for (int vt = 0; vt < 4; ++vt) av[vt] = __builtin_bit_cast(f16x8, mom_cols(vb16 + s * (16 * kD), ov[vt]));
        avs = __builtin_bit_cast(f16x8, mom_cols(vb16 + s * (16 * kD), os));
        // A operand of o~: the weight rows (hi, lo per head, zeros) of the lane's row
        wo = __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(
                                           &S.pw[t & 1][pw_row][32 * kh + 16 * s + 8 * (l >> 5)]));
      }
      __builtin_amdgcn_sched_barrier(0);
      if (h == 0) accX = mfma(wo, avs, accX);
#pragma unroll
      for (int vt = 0; vt < 4; ++vt) accM[vt][h] = mfma(av[vt], y, accM[vt][h]);
      accX = mfma(ones[h], y, accX);
      if (i + 1 < NS) {
        const int s2 = (i + 1) / HW, h2 = (i + 1) % HW;
        if (h2 == 0) kload(s2, kf);
        const f16x8 y2 = yform(s2, h2, kf);
        // the next step's LDS reads first, then each product followed by a share of the VALU work
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int j = 0; j < 6; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        y = y2;
      }
    }
    lds_barrier();   // the next tile's maxima are in LDS; every wave is done with tile t's values
    if (next) {
      decide(t + 1);
      if (any) rescale();   // (uniform)
      if (w < 4) weights(t + 1);
      convert_v(nbuf);
    }
  }
  // every wave is done with the tile buffers, which the epilogue reuses
  lds_barrier();

  // ---- epilogue ----
  // the two key halves of each partial: o~ and kbar~ through LDS, M added in place
  {
    float lp = lpart;
#pragma unroll
    for (int o2 = 1; o2 < 16; o2 <<= 1) lp += __shfl_xor(lp, o2, 64);
    if (w < 4 && (l & 15) == 0 && l < 16 * HW) S.lsum[w][l >> 4] = lp;
    // accX row 4 (l / 32) + r of column l % 32 (r < 4): o~ of head h = rows h (hi) and HW + h (lo) in lanes
    // < 32, kbar~ of head h = row 4 + h in lanes >= 32
    const int col = 32 * ks_strip + (l & 31);
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      if (l < 32) S.opart[kh][h][col] = accX[h] + accX[HW + h];
      else S.kpart[kh][h][col] = accX[h];
    }
  }
  // the moment: the second key half writes its partial (the tile buffers are free: every copy has completed
  // and every wave has passed the barrier after the loop)
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
    S.vec[0][eh][ea] = __builtin_amdgcn_ldexpf(S.opart[0][eh][ea] + S.opart[1][eh][ea], -ev) * inv;
    S.vec[1][eh][ea] = __builtin_amdgcn_ldexpf(S.kpart[0][eh][ea] + S.kpart[1][eh][ea], -ek) * inv;
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
    S.qf[eh][ea] = bf16_to_f32(qrow[ea]);
#pragma unroll
    for (int o2 = 32; o2 > 0; o2 >>= 1) aval += __shfl_xor(aval, o2, 64);
    if (l == 0) S.red[0][eh][(tid >> 6) & 1] = aval;
    S.vec[2][eh][ea] = uval;
  }
  __syncthreads();
  // The moment form: c = M u / l - alpha o.  Its two terms are each about |u . k| |v| and cancel; when they
  // exceed the output by more than 2^11 (a key far larger than the rest dominates the softmax, so kbar is
  // close to it), fp32's rounding of their difference would show, and the head's correction is formed
  // directly instead, c = sum_j p_j (u . (k_j - kbar)) (v_j - o), from a second read of its keys.
  float cval = 0.f, oval = 0.f;
  if (eh < HW) {
    const float alpha = S.red[0][eh][0] + S.red[0][eh][1];
    const float ln = eh == 0 ? Lh[0] : Lh[HW - 1];
    const float inv = ln > 0.f ? 1.f / ln : 0.f;
    float mu = 0.f;
#pragma unroll 8
    for (int bb = 0; bb < kD; ++bb) mu = fmaf(S.M[eh][ea][bb], S.vec[2][eh][bb], mu);
    oval = S.vec[0][eh][ea];
    const float mterm = __builtin_amdgcn_ldexpf(mu, -(ek + ev)) * inv;
    cval = mterm - alpha * oval;
    float cm = fabsf(mterm) + fabsf(alpha * oval), om = fabsf(oval + cval);
#pragma unroll
    for (int o2 = 32; o2 > 0; o2 >>= 1) {
      cm = fmaxf(cm, __shfl_xor(cm, o2, 64));
      om = fmaxf(om, __shfl_xor(om, o2, 64));
    }
    if (l == 0) {
      S.red[3][eh][(tid >> 6) & 1] = cm;
      S.red[4][eh][(tid >> 6) & 1] = om;
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < HW; ++h) {
    const float cm = fmaxf(S.red[3][h][0], S.red[3][h][1]), om = fmaxf(S.red[4][h][0], S.red[4][h][1]);
    if (!(cm > om * 2048.f)) continue;   // (uniform)
    const float mh = uniform_f(h == 0 ? m_run[0] : m_run[HW - 1]), lh = h == 0 ? Lh[0] : Lh[HW - 1];
    const float inv = lh > 0.f ? 1.f / lh : 0.f;
    const int a = tid & 127, part = tid >> 7;
    float acc = 0.f;
    for (int j0 = lo; j0 < hi; j0 += 512) {
      // the weight of key j0 + tid: its score and u . (k - kbar) in fp32 from the cache row
      const int j = j0 + tid;
      float wv = 0.f;
      if (j < hi) {
        const int64_t row = PAGED ? mrow<true>(p, b, j) : static_cast<int64_t>(b) * p.L + j;
        const u16* kr = p.kc + (row * p.Hkv + g) * kD;
        float sc = 0.f, t = 0.f;
        for (int d0 = 0; d0 < kD; d0 += 8) {
          const u32x4 kw = __builtin_bit_cast(u32x4, *reinterpret_cast<const uint4*>(kr + d0));
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float kv = __uint_as_float(e & 1 ? kw[e >> 1] & 0xffff0000u : kw[e >> 1] << 16);
            sc = fmaf(S.qf[h][d0 + e], kv, sc);
            t = fmaf(S.vec[2][h][d0 + e], kv - S.vec[1][h][d0 + e], t);
          }
        }
        wv = exp2f(sc * c2 - mh) * inv * t;
      }
      S.fb.wj[tid] = wv;
      __syncthreads();
      // this thread's value dim a over its quarter of the batch
      const int jq = j0 + 128 * part;
      const int nq = min(128, hi - jq);   // (the same in both waves of the quarter)
      const float oa = S.vec[0][h][a];
      for (int jj = 0; jj < nq; ++jj) {
        const int64_t row = PAGED ? mrow<true>(p, b, jq + jj) : static_cast<int64_t>(b) * p.L + jq + jj;
        const float vv = bf16_to_f32(p.vc[(row * p.Hkv + g) * kD + a]);
        acc = fmaf(S.fb.wj[128 * part + jj], vv - oa, acc);
      }
      __syncthreads();
    }
    S.fb.cacc[part][a] = acc;
    __syncthreads();
    if (eh == h) cval = S.fb.cacc[0][ea] + S.fb.cacc[1][ea] + S.fb.cacc[2][ea] + S.fb.cacc[3][ea];
  }
  if (eh < HW) {
    const float r = oval + cval;
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
