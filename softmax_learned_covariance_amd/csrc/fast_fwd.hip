// Fused two-pass Parallax forward for gfx950 (head_dim DH = 128 or 64; bf16 inputs, fp16 MFMA), and the
// one-pass probe-form forward.
//
// What it computes (gist.science technical summary of "Parallax: Parameterized
// Local Linear Attention for Language Modeling", "Core mechanism": softmax
// output plus the key/value covariance applied to the probe; "Hardware-aware
// algorithm": a FlashAttention-style streaming algorithm in which both branches
// share one stream of K/V tiles):
//   pass 1  online softmax over key tiles, accumulating o and kbar together
//           (K is streamed as extra value columns next to V);
//   probe   u = P^T (q - kbar) with MFMA, alpha = u . kbar;
//   pass 2  the same key tiles again: S = Q K^T and R = U K^T share the K operand
//           (the pages' joint QK / RK product), p = exp(S - lse),
//           W = p (R - alpha), c += W V, rs += rowsum(W);
//   out     o + c - rs * o        (= o + sum_j p_j (u.(k_j - kbar)) (v_j - o)).
//
// Work split.  One 512-thread workgroup (8 waves, 2 per SIMD) owns one
// (batch, key/value head) and a block of query rows for every query head of the
// group, so the group's heads share each K/V tile in LDS.  Each wave owns 32
// query rows of one head; products over d take DH / 16 k-steps and the per-row
// vectors over d (o, kbar, u, c) DH / 32 accumulator tiles; in the accumulator tiles lane l (l % 32 = query,
// l / 32 = half) holds 16 key or feature rows, so row statistics are lane-local
// plus one half-wave swap.  S^T = K Q^T puts keys in registers: P~^T is then
// directly the B operand of o^T = V^T P~^T and kbar^T = K^T P~^T (fp16 staging
// layouts in fast_common.h).  Lazy rescaling: the running maximum only moves
// when a tile's maximum exceeds it by 8 (log2 units), so the accumulators are
// rarely rescaled; p~ = exp2(s - m + 7) <= 2^15 then still fits fp16.
// Key tiles (chunk-major, see fast_common.h) are double-buffered in LDS and
// copied by direct-to-LDS DMA while the previous tile is being computed.
// Blocks are mapped so that all blocks of one (batch, kv head) run on the same
// XCD (their K/V stay in that XCD's L2), longest (most keys) first.
#include <math.h>

#include "fast_common.h"
#include "plx_internal.h"

#ifndef PLX_FWD_POLY_MASK
#define PLX_FWD_POLY_MASK 0
#endif
namespace plx {
// Which of each lane's groups of 8 exponentials in the forward's main kernel go through exp2_fma instead
// of the transcendental unit (bit j: element j of the group).
constexpr unsigned kFwdPolyMask = PLX_FWD_POLY_MASK;

namespace {

constexpr int kWaves = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.f;
// p~ = exp2(s - m + kLift): with the lazy rescale s - m <= kTau, so p~ <= 2^(kTau + kLift) = 2^15 stays
// inside fp16, and weights down to 2^-(14 + kLift) of the row's largest keep fp16's full precision (a
// sharply peaked row has many keys far below its largest weight; their sum still matters for kbar).
constexpr float kLift = 7.f;

struct FwdParams {
  const u16* q;
  const u16* rho;   // probe form only: the caller's probe, like q
  const _Float16 *k16, *k16t, *v16t, *p16t;
  const uint32_t* maxbits;
  const float* knorm;   // [B][Hkv][Tk_pad] running maximum of the key norms (see Staging)
  void* out;        // fp32, or bf16 when out_bf16
  float *lse, *kbar, *osa;
  float* rk;
  float* cor;       // per row |out - o| / |out|, [B][Hq][Tq] (nullable)
  int out_bf16;        // probe form only: rho . kbar per row, [B][Hq][Tq] (nullable)
  int B, Tq, Tk, Tk_pad, Hq, Hkv, G, causal, window;
  int D;            // head dim of the caller's rows (the kernel's DH)
  float scale;
  int row_begin, row_end, rows_per_block, n_rb;  // rows [row_begin, row_end)
};

template <int DH>
struct __align__(16) Tiles {
  _Float16 k[2][kKeyTile * DH];    // key rows tile    [DH/8 chunks][64 keys][8]
  _Float16 kt[2][DH * kKeyTile];   // key columns tile [8 chunks][DH d][8]
  _Float16 vt[2][DH * kKeyTile];
};

template <int DH>
__device__ __forceinline__ f16x8 lds_k(const Tiles<DH>& T, int buf, int r, int c) {
  return *reinterpret_cast<const f16x8*>(&T.k[buf][c * (kKeyTile * 8) + r * 8]);
}
template <int DH>
__device__ __forceinline__ f16x8 lds_kt(const Tiles<DH>& T, int buf, int d, int c) {
  return *reinterpret_cast<const f16x8*>(&T.kt[buf][c * (DH * 8) + d * 8]);
}
template <int DH>
__device__ __forceinline__ f16x8 lds_vt(const Tiles<DH>& T, int buf, int d, int c) {
  return *reinterpret_cast<const f16x8*>(&T.vt[buf][c * (DH * 8) + d * 8]);
}

// Asynchronous global -> LDS copy of one key tile (each array is one contiguous block of DH / 8 KB:
// DH / 8 wave instructions of 1024 bytes, DH / 64 per wave).
template <int DH>
__device__ __forceinline__ void tile_dma(const FwdParams& p, Tiles<DH>& T, int buf, int b, int g, int kt,
                                         bool with_kt, int w, int l) {
  const int64_t tb = kv_tile(b, g, kt, p.Hkv, p.Tk_pad / kKeyTile, DH);
#pragma unroll
  for (int j = 0; j < DH / 64; ++j) {
    const int i = (DH / 64) * w + j;
    const int64_t src = tb + i * 512 + l * 8;
    lds_dma16(p.k16 + src, &T.k[buf][i * 512]);
    if (with_kt) lds_dma16(p.k16t + src, &T.kt[buf][i * 512]);
    lds_dma16(p.v16t + src, &T.vt[buf][i * 512]);
  }
}

// Loads 4 consecutive bf16 values as floats.
__device__ __forceinline__ void load4_bf16(const u16* src, float* dst) {
  const uint2 w = *reinterpret_cast<const uint2*>(src);
  dst[0] = __uint_as_float(w.x << 16);
  dst[1] = __uint_as_float(w.x & 0xffff0000u);
  dst[2] = __uint_as_float(w.y << 16);
  dst[3] = __uint_as_float(w.y & 0xffff0000u);
}

// B operand of a product over d for one query row of NS * 16 elements: d in the permuted-16 order, scaled
// by s.
template <int NS>
__device__ __forceinline__ void load_q_operand(const u16* qrow, bool ok, int hh, float s, f16x8 (&qB)[NS]) {
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    float a[4] = {0.f, 0.f, 0.f, 0.f}, c[4] = {0.f, 0.f, 0.f, 0.f};
    if (ok) {
      load4_bf16(qrow + 16 * st + 4 * hh, a);
      load4_bf16(qrow + 16 * st + 8 + 4 * hh, c);
    }
    qB[st] = pack8(a[0] * s, a[1] * s, a[2] * s, a[3] * s, c[0] * s, c[1] * s, c[2] * s, c[3] * s);
  }
}

// SPLIT: every operand the kernel computes (p~, q - kbar, u, W) is carried as an
// fp16 hi + lo pair (two MFMAs, ~22 significant bits); used for the first query
// rows, whose few visible keys make the output large relative to its rms.
template <bool SPLIT, int DH>
__global__ __launch_bounds__(512) void k_fwd_fast(FwdParams p) {
  constexpr int NS = DH / 16, NT = DH / 32;   // k-steps and accumulator tiles over d
  __shared__ Tiles<DH> T;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, ql = l & 31, hh = l >> 5;

  // block -> (batch, kv head, row block)
  int pair, rb;
  {
    const int npairs = p.B * p.Hkv, id = blockIdx.x;
    if ((npairs & 7) == 0) {
      const int ppx = npairs >> 3, slot = id >> 3;
      rb = p.n_rb - 1 - slot / ppx;
      pair = (id & 7) + 8 * (slot % ppx);
    } else {
      rb = p.n_rb - 1 - id / npairs;
      pair = id % npairs;
    }
  }
  const int b = pair / p.Hkv, g = pair % p.Hkv;
  const int wph = kWaves / p.G;
  const int h = g * p.G + w / wph;
  const int r0 = p.row_begin + rb * p.rows_per_block;
  const int i0 = r0 + (w % wph) * 32;
  const int row = i0 + ql;
  const bool row_ok = row < p.row_end;
  const int off = p.Tk - p.Tq;

  const float sQ = range_scale(__uint_as_float(p.maxbits[0]));
  const float sK = range_scale(__uint_as_float(p.maxbits[1]));
  const float sV = range_scale(__uint_as_float(p.maxbits[2]));
  const float sP = range_scale(__uint_as_float(p.maxbits[3]));
  const float cS = p.scale * kLog2e / (sQ * sK);

  const int64_t qoff = ((static_cast<int64_t>(b) * p.Tq + (row_ok ? row : 0)) * p.Hq + h) * DH;
  const u16* qrow = p.q + qoff;

  // key ranges: block, wave (first / last row), lane (its row)
  const int rlast = min(r0 + p.rows_per_block, p.row_end) - 1;
  const int kend = p.causal ? min(p.Tk, rlast + off + 1) : p.Tk;
  const int kbeg = p.window > 0 ? max(0, r0 + off - p.window + 1) : 0;
  const int t_beg = kbeg / kKeyTile;
  const int t_end = kend > kbeg ? (kend + kKeyTile - 1) / kKeyTile : t_beg;
  const int wlast = min(i0 + 31, p.row_end - 1);
  const bool wave_rows = i0 < p.row_end;
  const int w_kend = wave_rows ? (p.causal ? min(p.Tk, wlast + off + 1) : p.Tk) : 0;
  const int w_kbeg = p.window > 0 ? max(0, i0 + off - p.window + 1) : 0;
  const int w_full_end = p.causal ? min(p.Tk, i0 + off + 1) : p.Tk;                       // every row sees keys < this
  const int w_full_beg = p.window > 0 ? max(0, wlast + off - p.window + 1) : 0;           // ... and >= this
  const int r_kend = row_ok ? (p.causal ? min(p.Tk, row + off + 1) : p.Tk) : 0;
  const int r_kbeg = p.window > 0 ? max(0, row + off - p.window + 1) : 0;

  f16x8 qB[NS];
  load_q_operand(qrow, row_ok, hh, sQ, qB);

  // ---------------- pass 1 ----------------
  f32x16 accO[NT], accK[NT];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
    accO[mt] = f32x16{};
    accK[mt] = f32x16{};
  }
  float m_used = -INFINITY, lpart = 0.f;
  if (t_beg < t_end) tile_dma(p, T, 0, b, g, t_beg, true, w, l);
  lds_dma_wait();
  __syncthreads();
  for (int kt = t_beg; kt < t_end; ++kt) {
    const int buf = (kt - t_beg) & 1;
    if (kt + 1 < t_end) tile_dma(p, T, buf ^ 1, b, g, kt + 1, true, w, l);
    const int key0 = kt * kKeyTile;
    if (key0 < w_kend && key0 + kKeyTile > w_kbeg) {
      f32x16 S[2] = {f32x16{}, f32x16{}};
      {
        // the key-row operands of chunk s + 2 are read while the MFMAs of chunk s run (the
        // scheduling barriers keep the compiler from moving the reads next to their MFMAs)
        f16x8 a[3][2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          a[s][0] = lds_k(T, buf, ql, 2 * s + hh);
          a[s][1] = lds_k(T, buf, 32 + ql, 2 * s + hh);
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if (s + 2 < NS) {
            a[(s + 2) % 3][0] = lds_k(T, buf, ql, 2 * (s + 2) + hh);
            a[(s + 2) % 3][1] = lds_k(T, buf, 32 + ql, 2 * (s + 2) + hh);
          }
          __builtin_amdgcn_sched_barrier(0);
          S[0] = mfma(a[s % 3][0], qB[s], S[0]);
          S[1] = mfma(a[s % 3][1], qB[s], S[1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const bool full = key0 + kKeyTile <= w_full_end && key0 >= w_full_beg;
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= r_kend || key < r_kbeg) S[kb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
      mx = xor32_max(mx);
      const float mt_ = mx * cS;
      const bool need = mt_ > m_used + kTau;
      if (__ballot(need) != 0) {
        const float f = need ? exp2f(m_used - mt_) : 1.f;
        m_used = need ? mt_ : m_used;
        lpart *= f;
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
          accO[mt] *= f;
          accK[mt] *= f;
        }
      }
      const float mb = m_used == -INFINITY ? 0.f : m_used - kLift;
      f16x8 pB[4], pL[SPLIT ? 4 : 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kb = i >> 1, t8 = (i & 1) * 8;
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = fmaf(S[kb][t8 + j], cS, -mb);
          e[j] = (!SPLIT && ((kFwdPolyMask >> j) & 1)) ? exp2_fma(x) : __builtin_amdgcn_exp2f(x);
        }
        if constexpr (SPLIT) pin8(e);
        pB[i] = pack8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
        lpart = sum8(pB[i], lpart);
        if constexpr (SPLIT) {
          pL[i] = pack_lo(e, pB[i]);
          lpart = sum8(pL[i], lpart);
        }
      }
      {
        // step n = (mt, i): the V^T and K^T column operands of step n + 2 are read while step n runs
        f16x8 c[3][2];
        auto load_c = [&](int n, f16x8(&dst)[2]) {
          const int mt = n >> 2, i = n & 3;
          dst[0] = lds_vt(T, buf, 32 * mt + ql, 2 * i + hh);
          dst[1] = lds_kt(T, buf, 32 * mt + ql, 2 * i + hh);
        };
        load_c(0, c[0]);
        load_c(1, c[1]);
#pragma unroll
        for (int n = 0; n < 4 * NT; ++n) {
          const int mt = n >> 2, i = n & 3;
          if (n + 2 < 4 * NT) load_c(n + 2, c[(n + 2) % 3]);
          __builtin_amdgcn_sched_barrier(0);
          accO[mt] = mfma(c[n % 3][0], pB[i], accO[mt]);
          accK[mt] = mfma(c[n % 3][1], pB[i], accK[mt]);
          if constexpr (SPLIT) {
            accO[mt] = mfma(c[n % 3][0], pL[i], accO[mt]);
            accK[mt] = mfma(c[n % 3][1], pL[i], accK[mt]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    lds_dma_wait();
    __syncthreads();
  }

  // ---------------- epilogue 1: o, kbar, lse ----------------
  const float L = xor32_sum(lpart);
  const bool has = L > 0.f;
  const float invL = has ? 1.f / L : 0.f;
  const float lse2 = has ? m_used - kLift + __log2f(L) : -INFINITY;   // (L carries the 2^kLift of p~)
  float* obuf = p.osa;
  // row vectors move to and from memory through the tile buffers (free between the passes and after the
  // second), a wave-private block each
  auto rows_io = [&]() {
    WaveRows r;
    r.lds = reinterpret_cast<float*>(&T) + w * 32 * kWR;
    r.rstride = static_cast<int64_t>(p.Hq) * DH;
    r.base = ((static_cast<int64_t>(b) * p.Tq + min(i0, p.Tq - 1)) * p.Hq + h) * DH;
    r.nrows = max(0, min(32, p.row_end - i0));
    r.l = l;
    r.ql = ql;
    r.hh = hh;
    return r;
  };
  if (row_ok && p.lse && hh == 0) p.lse[(static_cast<int64_t>(b) * p.Hq + h) * p.Tq + row] = lse2 * kLn2;
  if (row_ok) {
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * mt + 8 * j + 4 * hh;
        const float fo = invL / sV, fk = invL / sK;
        const float4 ov = {accO[mt][4 * j] * fo, accO[mt][4 * j + 1] * fo, accO[mt][4 * j + 2] * fo,
                           accO[mt][4 * j + 3] * fo};
        *reinterpret_cast<float4*>(obuf + qoff + d) = ov;
        if (p.kbar) {
          const float4 kv = {accK[mt][4 * j] * fk, accK[mt][4 * j + 1] * fk, accK[mt][4 * j + 2] * fk,
                             accK[mt][4 * j + 3] * fk};
          *reinterpret_cast<float4*>(p.kbar + qoff + d) = kv;
        }
      }
  }

  // ---------------- probe u = P^T (q - kbar) ----------------
  // kbar (unscaled) and x = q - kbar in the accumulator layout: lane (row, hh), d = 32 mt + 8 (r/4) + 4 hh + r%4
  float kbv[NT][16];
  f16x8 xB[NS], xL[SPLIT ? NS : 1];
  float alpha_s = 0.f, sU = 1.f;
  float u2sum = 0.f, k2sum = 0.f;   // |U-hat|^2 (scaled units) and |kbar sK|^2 of the row, for pass 2's W scale
  {
    float xv[NT][16];
    float xmax = 0.f;
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float qv[4] = {0.f, 0.f, 0.f, 0.f};
        if (row_ok) load4_bf16(qrow + 32 * mt + 8 * j + 4 * hh, qv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * j + e;
          kbv[mt][r] = accK[mt][r] * (invL / sK);
          xv[mt][r] = qv[e] - kbv[mt][r];
          k2sum = fmaf(accK[mt][r] * invL, accK[mt][r] * invL, k2sum);   // (kbar sK)^2
          xmax = fmaxf(xmax, fabsf(xv[mt][r]));
        }
      }
    xmax = xor32_max(xmax);
    const float sX = range_scale(xmax);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int mt = s >> 1, t8 = (s & 1) * 8;
      float e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = xv[mt][t8 + j] * sX;   // (sX is a power of two: x sX is exact)
      xB[s] = pack8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      if constexpr (SPLIT) xL[s] = pack_lo(e, xB[s]);   // (single-operand rows form theirs below, one at a time)
    }
    // U^T = P16t X^T.  x always enters as a hi + lo pair: for a sharply peaked row the correction is
    // one dot product u.(k_1 - k_2) of nearly orthogonal vectors, which amplifies the rounding of u's
    // inputs; the 32 extra MFMAs per wave are taken once per row block, not per key tile.
    f32x16 accU[NT];
    const _Float16* prow = p.p16t + (static_cast<int64_t>(h) * DH + ql) * DH + hh * 8;
#pragma unroll
    for (int am = 0; am < NT; ++am) accU[am] = f32x16{};
    if constexpr (SPLIT) {
#pragma unroll
      for (int am = 0; am < NT; ++am)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const f16x8 a = *reinterpret_cast<const f16x8*>(prow + 32 * am * DH + 16 * s);
          accU[am] = mfma(a, xB[s], accU[am]);
          accU[am] = mfma(a, xL[s], accU[am]);
        }
    } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      f16x8 lo;
      {
        const int mt = s >> 1, t8 = (s & 1) * 8;
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = xv[mt][t8 + j] * sX;
        lo = pack_lo(e, xB[s]);
      }
#pragma unroll
      for (int am = 0; am < NT; ++am) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(prow + 32 * am * DH + 16 * s);
        accU[am] = mfma(a, xB[s], accU[am]);
        accU[am] = mfma(a, lo, accU[am]);
      }
    }
    }
    const float fu = 1.f / (sX * sP);
    float umax = 0.f;
#pragma unroll
    for (int am = 0; am < NT; ++am)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        accU[am][r] *= fu;
        umax = fmaxf(umax, fabsf(accU[am][r]));
      }
    umax = xor32_max(umax);
    sU = range_scale(umax);
    // U-hat operand (reusing xB's registers) and alpha = U-hat . kbar in the scaled units of pass 2
    float alpha = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int am = s >> 1, t8 = (s & 1) * 8;
      float e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = accU[am][t8 + j] * sU;
      if constexpr (SPLIT) pin8(e);
      xB[s] = pack8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      if constexpr (SPLIT) xL[s] = pack_lo(e, xB[s]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float uh = static_cast<float>(xB[s][j]);
        if constexpr (SPLIT) uh += static_cast<float>(xL[s][j]);
        alpha += uh * (kbv[am][t8 + j] * sK);
        u2sum = fmaf(uh, uh, u2sum);
      }
    }
    alpha_s = xor32_sum(alpha);
    u2sum = xor32_sum(u2sum);
    k2sum = xor32_sum(k2sum);
  }
  const f16x8* uB = xB;
  const f16x8* uL = xL;

  // ---------------- pass 2 ----------------
  load_q_operand(qrow, row_ok, hh, sQ, qB);
  f32x16 accC[NT];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) accC[mt] = f32x16{};
  float rpart = 0.f;
  // W = p (R - alpha) is packed to fp16 as p 2^-wexp (R - alpha), wexp an integer folded into the exp2
  // argument.  Its range depends on the row: |R_j - alpha| = |U-hat.(k_j - kbar)| <= |U-hat| (|k_j| + |kbar|)
  // and p <= 1, so the row's bound uses the largest key norm among the keys it sees (a running maximum
  // along the sequence, from staging) instead of K's largest entry: one key row far larger than the
  // rest then changes the scale only of the rows that see it, and the other rows' W stay clear of
  // fp16's subnormals.
  float mb2 = 0.f;
  if (has) {
    const float kmax = r_kend > r_kbeg ? p.knorm[(static_cast<int64_t>(b) * p.Hkv + g) * p.Tk_pad + r_kend - 1] * sK : 0.f;
    mb2 = lse2 + static_cast<float>(-range_exp(sqrtf(u2sum) * (kmax + sqrtf(k2sum))));
  }
  __syncthreads();   // (every wave is done with its row block in the tile buffers)
  if (t_beg < t_end) tile_dma(p, T, 0, b, g, t_beg, false, w, l);
  lds_dma_wait();
  __syncthreads();
  for (int kt = t_beg; kt < t_end; ++kt) {
    const int buf = (kt - t_beg) & 1;
    if (kt + 1 < t_end) tile_dma(p, T, buf ^ 1, b, g, kt + 1, false, w, l);
    const int key0 = kt * kKeyTile;
    if (key0 < w_kend && key0 + kKeyTile > w_kbeg) {
      const bool full = key0 + kKeyTile <= w_full_end && key0 >= w_full_beg;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 S = {}, R = {};
        {
          f16x8 a[3];   // key-row operands two chunks ahead
          a[0] = lds_k(T, buf, 32 * kb + ql, hh);
          a[1] = lds_k(T, buf, 32 * kb + ql, 2 + hh);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            if (s + 2 < NS) a[(s + 2) % 3] = lds_k(T, buf, 32 * kb + ql, 2 * (s + 2) + hh);
            __builtin_amdgcn_sched_barrier(0);
            S = mfma(a[s % 3], qB[s], S);
            R = mfma(a[s % 3], uB[s], R);
            if constexpr (SPLIT) R = mfma(a[s % 3], uL[s], R);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (!full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= r_kend || key < r_kbeg) S[r] = -INFINITY;
          }
        }
        f16x8 wB[2], wL[SPLIT ? 2 : 1];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int r = 8 * t + j;
            const float x = fmaf(S[r], cS, -mb2);
            e[j] = ((!SPLIT && ((kFwdPolyMask >> j) & 1)) ? exp2_fma(x) : __builtin_amdgcn_exp2f(x)) * (R[r] - alpha_s);
          }
          if constexpr (SPLIT) pin8(e);
          wB[t] = pack8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
          rpart = sum8(wB[t], rpart);
          if constexpr (SPLIT) {
            wL[t] = pack_lo(e, wB[t]);
            rpart = sum8(wL[t], rpart);
          }
        }
        {
          // step n = (mt, t): V^T column operands two steps ahead
          f16x8 c[3];
          c[0] = lds_vt(T, buf, ql, 4 * kb + hh);
          c[1] = lds_vt(T, buf, ql, 4 * kb + 2 + hh);
#pragma unroll
          for (int n = 0; n < 2 * NT; ++n) {
            const int mt = n >> 1, t = n & 1;
            if (n + 2 < 2 * NT) c[(n + 2) % 3] = lds_vt(T, buf, 32 * ((n + 2) >> 1) + ql, 4 * kb + 2 * ((n + 2) & 1) + hh);
            __builtin_amdgcn_sched_barrier(0);
            accC[mt] = mfma(c[n % 3], wB[t], accC[mt]);
            if constexpr (SPLIT) accC[mt] = mfma(c[n % 3], wL[t], accC[mt]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    lds_dma_wait();
    __syncthreads();
  }

  // ---------------- epilogue 2: out = o + c - rs o ----------------
  const float RS = xor32_sum(rpart);
  float cc = 0.f, oo = 0.f;   // |out - o|^2 and |out|^2 of the lane's half-row
  {
    // W was carried as p 2^-wexp (R - alpha), wexp = mb2 - lse2 (an integer; the fp32 sum keeps it to
    // well within 1/2)
    const float fw = has ? __builtin_ldexpf(1.f, static_cast<int>(rintf(mb2 - lse2))) : 0.f;
    const float fc = fw / (sU * sK * sV);
    const float frs = RS * (fw / (sU * sK));
    const WaveRows wr = rows_io();
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      float ov[16], rv[16];
      wr.load<true>(obuf, mt, ov);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        rv[r] = ov[r] + accC[mt][r] * fc - frs * ov[r];
        cc = fmaf(rv[r] - ov[r], rv[r] - ov[r], cc);
        oo = fmaf(rv[r], rv[r], oo);
      }
      if (p.out_bf16) wr.store<true>(p.out, mt, rv);
      else wr.store(p.out, mt, rv);
    }
  }
  if (p.cor) {
    cc = xor32_sum(cc);
    oo = xor32_sum(oo);
    if (row_ok && hh == 0)
      p.cor[(static_cast<int64_t>(b) * p.Hq + h) * p.Tq + row] = oo > 0.f ? sqrtf(cc / oo) : 0.f;
  }
}

// ------------------------------------------------------------------------------------------
// Probe form, one pass (gist.science summary, "Core mechanism": out_i = o^SA_i - Sigma_KV^(i) rho_i
// with the probe rho_i = W_R x_i supplied by the caller; "Hardware-aware algorithm": one KV stream
// for both branches, the QK and RK products sharing the K operand).  With the probe known up front
//   out = o - (sum_j p_j r_j v_j - a o),   r_j = rho . k_j,   a = sum_j p_j r_j (= rho . kbar),
// so o, c = sum p r v, l and sum p r accumulate together in one online-softmax pass.  Per 32-key
// half of a tile: S = K Q^T and R = K rho^T share the K operand; o += V^T p~ and c += V^T (p~ R)
// share the V^T operand, so every operand read from LDS feeds two MFMAs.  rho is an input (bf16, exact in fp16 after its power-of-two scale), so its
// operand lives in LDS, one 8 KB block per wave; q stays in registers.
// W = p~ R is carried as p~ R 2^-wexp, with wexp set per row from |W| <= 2^15 |rho| |k_j| and the
// largest key norm among the keys the row sees (as in the projector form's pass 2): one key row far
// larger than the rest (which sets K's fp16 scale) then does not push the other rows' W into fp16's
// subnormal range.
// ------------------------------------------------------------------------------------------

template <int DH>
struct __align__(16) ProbeTiles {
  _Float16 k[2][kKeyTile * DH];    // key rows tile    [DH/8 chunks][64 keys][8]
  _Float16 vt[2][DH * kKeyTile];   // value columns    [8 chunks][DH d][8]
  f16x8 rho[kWaves][DH / 16][64];  // per wave: the rho operand of each lane, DH / 16 k-steps
};

template <int DH>
__device__ __forceinline__ void probe_tile_dma(const FwdParams& p, ProbeTiles<DH>& T, int buf, int b, int g, int kt,
                                               int w, int l) {
  const int64_t tb = kv_tile(b, g, kt, p.Hkv, p.Tk_pad / kKeyTile, DH);
#pragma unroll
  for (int j = 0; j < DH / 64; ++j) {
    const int i = (DH / 64) * w + j;
    const int64_t src = tb + i * 512 + l * 8;
    lds_dma16(p.k16 + src, &T.k[buf][i * 512]);
    lds_dma16(p.v16t + src, &T.vt[buf][i * 512]);
  }
}

template <int DH>
__device__ __forceinline__ f16x8 lds_k_probe(const ProbeTiles<DH>& T, int buf, int r, int c) {
  return *reinterpret_cast<const f16x8*>(&T.k[buf][c * (kKeyTile * 8) + r * 8]);
}
template <int DH>
__device__ __forceinline__ f16x8 lds_vt_probe(const ProbeTiles<DH>& T, int buf, int d, int c) {
  return *reinterpret_cast<const f16x8*>(&T.vt[buf][c * (DH * 8) + d * 8]);
}

template <bool SPLIT, int DH>
__global__ __launch_bounds__(512) void k_fwd_probe(FwdParams p) {
  constexpr int NS = DH / 16, NT = DH / 32;   // k-steps and accumulator tiles over d
  __shared__ ProbeTiles<DH> T;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, ql = l & 31, hh = l >> 5;

  int pair, rb;
  {
    const int npairs = p.B * p.Hkv, id = blockIdx.x;
    if ((npairs & 7) == 0) {
      const int ppx = npairs >> 3, slot = id >> 3;
      rb = p.n_rb - 1 - slot / ppx;
      pair = (id & 7) + 8 * (slot % ppx);
    } else {
      rb = p.n_rb - 1 - id / npairs;
      pair = id % npairs;
    }
  }
  const int b = pair / p.Hkv, g = pair % p.Hkv;
  const int wph = kWaves / p.G;
  const int h = g * p.G + w / wph;
  const int r0 = p.row_begin + rb * p.rows_per_block;
  const int i0 = r0 + (w % wph) * 32;
  const int row = i0 + ql;
  const bool row_ok = row < p.row_end;
  const int off = p.Tk - p.Tq;

  const float sQ = range_scale(__uint_as_float(p.maxbits[kMaxQ]));
  const float sK = range_scale(__uint_as_float(p.maxbits[kMaxK]));
  const float sV = range_scale(__uint_as_float(p.maxbits[kMaxV]));
  const float sR = range_scale(__uint_as_float(p.maxbits[kMaxRho]));
  const float cS = p.scale * kLog2e / (sQ * sK);

  const int64_t qoff = ((static_cast<int64_t>(b) * p.Tq + (row_ok ? row : 0)) * p.Hq + h) * DH;

  const int rlast = min(r0 + p.rows_per_block, p.row_end) - 1;
  const int kend = p.causal ? min(p.Tk, rlast + off + 1) : p.Tk;
  const int kbeg = p.window > 0 ? max(0, r0 + off - p.window + 1) : 0;
  const int t_beg = kbeg / kKeyTile;
  const int t_end = kend > kbeg ? (kend + kKeyTile - 1) / kKeyTile : t_beg;
  const int wlast = min(i0 + 31, p.row_end - 1);
  const bool wave_rows = i0 < p.row_end;
  const int w_kend = wave_rows ? (p.causal ? min(p.Tk, wlast + off + 1) : p.Tk) : 0;
  const int w_kbeg = p.window > 0 ? max(0, i0 + off - p.window + 1) : 0;
  const int w_full_end = p.causal ? min(p.Tk, i0 + off + 1) : p.Tk;
  const int w_full_beg = p.window > 0 ? max(0, wlast + off - p.window + 1) : 0;
  const int r_kend = row_ok ? (p.causal ? min(p.Tk, row + off + 1) : p.Tk) : 0;
  const int r_kbeg = p.window > 0 ? max(0, row + off - p.window + 1) : 0;

  f16x8 qB[NS];
  load_q_operand(p.q + qoff, row_ok, hh, sQ, qB);
  float wfac;   // 2^-wexp
  int wexp;
  {
    // the lane's rho operand into the wave's LDS block (read back by the same lane only)
    f16x8 rB[NS];
    load_q_operand(p.rho + qoff, row_ok, hh, sR, rB);
    float r2 = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      T.rho[w][s][l] = rB[s];
#pragma unroll
      for (int j = 0; j < 8; ++j) r2 = fmaf(static_cast<float>(rB[s][j]), static_cast<float>(rB[s][j]), r2);
    }
    // |W| = p~ |rho.k_j| <= 2^15 |rho| |k_j| (p~ <= 2^15), with the largest key norm among the keys the
    // row sees (running maximum along the sequence): the row's scale
    r2 = xor32_sum(r2);
    const float kmax = r_kend > r_kbeg ? p.knorm[(static_cast<int64_t>(b) * p.Hkv + g) * p.Tk_pad + r_kend - 1] * sK : 0.f;
    wexp = -range_exp(32768.f * sqrtf(r2) * kmax);
    wfac = __builtin_ldexpf(1.f, -wexp);
  }

  f32x16 accO[NT], accC[NT];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
    accO[mt] = f32x16{};
    accC[mt] = f32x16{};
  }
  float m_used = -INFINITY, lpart = 0.f, rpart = 0.f;
  if (t_beg < t_end) probe_tile_dma(p, T, 0, b, g, t_beg, w, l);
  lds_dma_wait();
  __syncthreads();
  for (int kt = t_beg; kt < t_end; ++kt) {
    const int buf = (kt - t_beg) & 1;
    if (kt + 1 < t_end) probe_tile_dma(p, T, buf ^ 1, b, g, kt + 1, w, l);
    const int key0 = kt * kKeyTile;
    if (key0 < w_kend && key0 + kKeyTile > w_kbeg) {
      const bool full = key0 + kKeyTile <= w_full_end && key0 >= w_full_beg;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 S = {}, R = {};
        {
          // key-row and rho operands of chunk s + 1 are read while the MFMAs of chunk s run
          f16x8 a[2], r[2];
          a[0] = lds_k_probe(T, buf, 32 * kb + ql, hh);
          r[0] = T.rho[w][0][l];
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            if (s + 1 < NS) {
              a[(s + 1) & 1] = lds_k_probe(T, buf, 32 * kb + ql, 2 * (s + 1) + hh);
              r[(s + 1) & 1] = T.rho[w][s + 1][l];
            }
            __builtin_amdgcn_sched_barrier(0);
            S = mfma(a[s & 1], qB[s], S);
            R = mfma(a[s & 1], r[s & 1], R);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (!full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= r_kend || key < r_kbeg) S[r] = -INFINITY;
          }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[r]);
        mx = xor32_max(mx);
        const float mt_ = mx * cS;
        const bool need = mt_ > m_used + kTau;
        if (__ballot(need) != 0) {
          const float f = need ? exp2f(m_used - mt_) : 1.f;
          m_used = need ? mt_ : m_used;
          lpart *= f;
          rpart *= f;
#pragma unroll
          for (int mt = 0; mt < NT; ++mt) {
            accO[mt] *= f;
            accC[mt] *= f;
          }
        }
        const float mb = m_used == -INFINITY ? 0.f : m_used - kLift;
        f16x8 pB[2], wB[2], pL[SPLIT ? 2 : 1], wL[SPLIT ? 2 : 1];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float e[8], x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            e[j] = __builtin_amdgcn_exp2f(fmaf(S[8 * t + j], cS, -mb));
            x[j] = e[j] * R[8 * t + j] * wfac;
          }
          if constexpr (SPLIT) {
            pin8(e);
            pin8(x);
          }
          pB[t] = pack8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
          wB[t] = pack8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
          lpart = sum8(pB[t], lpart);
          rpart = sum8(wB[t], rpart);
          if constexpr (SPLIT) {
            pL[t] = pack_lo(e, pB[t]);
            wL[t] = pack_lo(x, wB[t]);
            lpart = sum8(pL[t], lpart);
            rpart = sum8(wL[t], rpart);
          }
        }
        {
          // step n = (mt, t): V^T column operands two steps ahead, each feeding o and c
          f16x8 c[3];
          c[0] = lds_vt_probe(T, buf, ql, 4 * kb + hh);
          c[1] = lds_vt_probe(T, buf, ql, 4 * kb + 2 + hh);
#pragma unroll
          for (int n = 0; n < 2 * NT; ++n) {
            const int mt = n >> 1, t = n & 1;
            if (n + 2 < 2 * NT) c[(n + 2) % 3] = lds_vt_probe(T, buf, 32 * ((n + 2) >> 1) + ql, 4 * kb + 2 * ((n + 2) & 1) + hh);
            __builtin_amdgcn_sched_barrier(0);
            accO[mt] = mfma(c[n % 3], pB[t], accO[mt]);
            accC[mt] = mfma(c[n % 3], wB[t], accC[mt]);
            if constexpr (SPLIT) {
              accO[mt] = mfma(c[n % 3], pL[t], accO[mt]);
              accC[mt] = mfma(c[n % 3], wL[t], accC[mt]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    lds_dma_wait();
    __syncthreads();
  }

  // out = o - (c - a o), o = accO / (l sV), c = accC 2^wexp / (l sR sK sV), a = rpart 2^wexp / (l sR sK)
  const float L = xor32_sum(lpart);
  const float RS = xor32_sum(rpart);
  const bool has = L > 0.f;
  const float invL = has ? 1.f / L : 0.f;
  float cc = 0.f, oo = 0.f;   // |out - o|^2 and |out|^2 of the lane's half-row
  if (row_ok) {
    const float fo = invL / sV;
    const float fw = __builtin_ldexpf(1.f, wexp);
    const float fc = fo / sK * (fw / sR);
    const float a = RS * invL / sK * (fw / sR);   // rho . kbar
    if (hh == 0) {
      const int64_t soff = (static_cast<int64_t>(b) * p.Hq + h) * p.Tq + row;
      if (p.lse) p.lse[soff] = has ? (m_used - kLift + __log2f(L)) * kLn2 : -INFINITY;
      if (p.rk) p.rk[soff] = a;
    }
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * mt + 8 * j + 4 * hh;
        float r4[4], o4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o4[e] = accO[mt][4 * j + e] * fo;
          r4[e] = o4[e] - accC[mt][4 * j + e] * fc + a * o4[e];
          cc = fmaf(r4[e] - o4[e], r4[e] - o4[e], cc);
          oo = fmaf(r4[e], r4[e], oo);
        }
        store_out4(p.out, qoff + d, p.out_bf16, r4[0], r4[1], r4[2], r4[3]);
        if (p.osa) *reinterpret_cast<float4*>(p.osa + qoff + d) = float4{o4[0], o4[1], o4[2], o4[3]};
      }
  }
  if (p.cor) {
    cc = xor32_sum(cc);
    oo = xor32_sum(oo);
    if (row_ok && hh == 0)
      p.cor[(static_cast<int64_t>(b) * p.Hq + h) * p.Tq + row] = oo > 0.f ? sqrtf(cc / oo) : 0.f;
  }
}

}  // namespace

bool fast_fwd_supported(const Geom& g) {
  const int G = g.Hq / g.Hkv;
  return g.bf16 && (g.d == kD || g.d == 64) && !g.p_per_query && (G == 1 || G == 2 || G == 4 || G == 8);
}

// Head dim of the staged operands: a head of 64 is staged and computed at 64 (no padding).
static int fwd_dh(const Geom& g) { return g.d == 64 ? 64 : kD; }

size_t fast_fwd_workspace(const Geom& g) {
  const Staging s = staging_layout(nullptr, g.B, g.Tk, g.Hkv, g.Hq, false, fwd_dh(g));
  return s.bytes + align_up(static_cast<size_t>(g.B) * g.Tq * g.Hq * g.d * sizeof(float), 256);
}

hipError_t launch_fast_fwd(const Geom& g, const void* q, const void* k, const void* v,
                           const void* P, void* out, float* lse, float* kbar, float* osa, float* cor,
                           int split_rows, void* ws, hipStream_t stream) {
  const Staging s = staging_layout(ws, g.B, g.Tk, g.Hkv, g.Hq, false, fwd_dh(g));
  float* o_ws = reinterpret_cast<float*>(static_cast<char*>(ws) + s.bytes);
  int split = (split_rows < kMinSplitRows ? kMinSplitRows : split_rows) + rows_without_keys(g);
  if (split > g.Tq) split = g.Tq;
  hipError_t e = launch_staging(s, q, static_cast<int64_t>(g.B) * g.Tq * g.Hq * g.d, k, v, P, g.B, g.Tk,
                                g.Hkv, g.Hq, stream, nullptr, 0, 0, g.d);
  if (e != hipSuccess) return e;
  FwdParams base{};
  {
    FwdParams& p = base;
    p.q = static_cast<const u16*>(q);
    p.k16 = s.k16;
    p.k16t = s.k16t;
    p.v16t = s.v16t;
    p.p16t = s.p16t;
    p.maxbits = s.maxbits;
    p.knorm = s.knorm;
    p.out = out;
    p.out_bf16 = g.out_bf16;
    p.cor = cor;
    p.lse = lse;
    p.kbar = kbar;
    p.osa = osa ? osa : o_ws;
    p.B = g.B;
    p.Tq = g.Tq;
    p.Tk = g.Tk;
    p.Tk_pad = s.Tk_pad;
    p.Hq = g.Hq;
    p.Hkv = g.Hkv;
    p.G = g.Hq / g.Hkv;
    p.causal = g.causal;
    p.window = g.window;
    p.D = g.d;
    p.scale = g.scale;
    p.rows_per_block = 32 * kWaves / p.G;
  }
  // rows [0, split) (the same kernel with hi + lo operands) run on the side lane beside the rest
  const SideLane side = split > 0 && split < g.Tq ? side_fork(stream) : SideLane{stream, stream};
  if (split > 0) {
    FwdParams p = base;
    p.row_begin = 0;
    p.n_rb = (split + p.rows_per_block - 1) / p.rows_per_block;
    p.row_end = split;
    if (s.dh == 64) hipLaunchKernelGGL((k_fwd_fast<true, 64>), dim3(g.B * g.Hkv * p.n_rb), dim3(512), 0, side.stream, p);
    else hipLaunchKernelGGL((k_fwd_fast<true, kD>), dim3(g.B * g.Hkv * p.n_rb), dim3(512), 0, side.stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (split < g.Tq) {
    FwdParams p = base;
    p.row_begin = split;
    p.row_end = g.Tq;
    p.n_rb = (g.Tq - split + p.rows_per_block - 1) / p.rows_per_block;
    const int blocks = g.B * g.Hkv * p.n_rb;
    mark_begin(PLX_KERNEL_FWD, stream);
    if (s.dh == 64) hipLaunchKernelGGL((k_fwd_fast<false, 64>), dim3(blocks), dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((k_fwd_fast<false, kD>), dim3(blocks), dim3(512), 0, stream, p);
    mark_end(PLX_KERNEL_FWD, stream);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  e = side_join(side);
  return e;
}

bool fast_probe_supported(const Geom& g) { return fast_fwd_supported(g); }

size_t fast_probe_workspace(const Geom& g) {
  return staging_layout(nullptr, g.B, g.Tk, g.Hkv, g.Hq, false, fwd_dh(g)).bytes;
}

hipError_t launch_fast_probe(const Geom& g, const void* q, const void* k, const void* v, const void* rho,
                             void* out, float* lse, float* osa, float* rk, float* cor, int split_rows, void* ws,
                             hipStream_t stream) {
  const Staging s = staging_layout(ws, g.B, g.Tk, g.Hkv, g.Hq, false, fwd_dh(g));
  int split = (split_rows < kMinSplitRows ? kMinSplitRows : split_rows) + rows_without_keys(g);
  if (split > g.Tq) split = g.Tq;
  const int64_t q_elems = static_cast<int64_t>(g.B) * g.Tq * g.Hq * g.d;
  // K/V into their fp16 tile layouts; max |q|, |k|, |v|, |rho| for the operand scales (no projector)
  hipError_t e = launch_staging(s, q, q_elems, k, v, nullptr, g.B, g.Tk, g.Hkv, g.Hq, stream, rho, q_elems, kMaxRho,
                                g.d);
  if (e != hipSuccess) return e;
  FwdParams base{};
  {
    FwdParams& p = base;
    p.q = static_cast<const u16*>(q);
    p.rho = static_cast<const u16*>(rho);
    p.k16 = s.k16;
    p.v16t = s.v16t;
    p.maxbits = s.maxbits;
    p.knorm = s.knorm;
    p.out = out;
    p.out_bf16 = g.out_bf16;
    p.cor = cor;
    p.lse = lse;
    p.osa = osa;
    p.rk = rk;
    p.B = g.B;
    p.Tq = g.Tq;
    p.Tk = g.Tk;
    p.Tk_pad = s.Tk_pad;
    p.Hq = g.Hq;
    p.Hkv = g.Hkv;
    p.G = g.Hq / g.Hkv;
    p.causal = g.causal;
    p.window = g.window;
    p.D = g.d;
    p.scale = g.scale;
    p.rows_per_block = 32 * kWaves / p.G;
  }
  const SideLane side = split > 0 && split < g.Tq ? side_fork(stream) : SideLane{stream, stream};
  if (split > 0) {
    FwdParams p = base;
    p.row_begin = 0;
    p.n_rb = (split + p.rows_per_block - 1) / p.rows_per_block;
    p.row_end = split;
    if (s.dh == 64) hipLaunchKernelGGL((k_fwd_probe<true, 64>), dim3(g.B * g.Hkv * p.n_rb), dim3(512), 0, side.stream, p);
    else hipLaunchKernelGGL((k_fwd_probe<true, kD>), dim3(g.B * g.Hkv * p.n_rb), dim3(512), 0, side.stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (split < g.Tq) {
    FwdParams p = base;
    p.row_begin = split;
    p.row_end = g.Tq;
    p.n_rb = (g.Tq - split + p.rows_per_block - 1) / p.rows_per_block;
    mark_begin(PLX_KERNEL_FWD_PROBE, stream);
    if (s.dh == 64) hipLaunchKernelGGL((k_fwd_probe<false, 64>), dim3(g.B * g.Hkv * p.n_rb), dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((k_fwd_probe<false, kD>), dim3(g.B * g.Hkv * p.n_rb), dim3(512), 0, stream, p);
    mark_end(PLX_KERNEL_FWD_PROBE, stream);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return side_join(side);
}

}  // namespace plx
