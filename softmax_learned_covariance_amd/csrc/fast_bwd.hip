// Parallax backward for gfx950 (head_dim DH = 128 or 64; bf16 inputs, fp16 MFMA), for the projector form and
// the probe form.  Products over d take DH / 16 k-steps and vectors over d DH / 32 accumulator tiles.
//
// The pages give no backward; these kernels evaluate the chain rule of the
// forward definition (output = softmax output plus the key/value covariance
// applied to the probe u = P^T (q - kbar), gist.science technical summary of
// "Parallax: Parameterized Local Linear Attention for Language Modeling",
// "Core mechanism").  With g = dout, alpha = u.kbar, t_ij = u_i.k_j,
// G_ij = g_i.v_j, p_ij the softmax weights:
//   du_i    = sum_j p_ij G_ij k_j - (g_i.o_i) kbar_i
//   dkbar_i = -(g_i.o_i) u_i - P du_i          dq_i = P du_i + scale sum_j ds_ij k_j
//   Delta_i = g_i.out_i + dkbar_i.kbar_i       dP   = sum_i (q_i - kbar_i) du_i^T
//   ds_ij   = p_ij (G_ij (t_ij + 1 - alpha_i) + dkbar_i.k_j - Delta_i)
//   dv_j    = sum_i p_ij (t_ij + 1 - alpha_i) g_i
//   dk_j    = sum_i p_ij G_ij u_i + p_ij dkbar_i + scale ds_ij q_i
//
// Kernels (one stream, in order), for query rows >= split_rows:
//   staging   fp16 copies of K, V, P and of q, dout in the MFMA operand layouts;
//   du        query-major, one pass over the key tiles (S, G and (p G) K on MFMA); its
//             epilogue forms u, alpha, P du (the first part of dq), dkbar, Delta and the
//             per-tile row statistics -- every quantity of a row stays in its lane;
//   staging 2 fp16 copies of u and dkbar (per-tensor scales from the du pass);
//   keys      key-major: a block owns 128 keys and streams query tiles; four waves
//             recompute S, T, E, G and the weights, four waves accumulate
//             dv = (p tt)^T g and dk = (p G)^T u + p^T dkbar + scale ds^T q on MFMA and
//             store each 32 x 32 tile of ds;
//   dq        query-major: dq += scale ds K from the stored ds tiles;
//   dP        sum over rows of (q - kbar) du^T, then a fixed-order reduction (on a helper stream,
//             beside the key-major kernel).
// Rows below split_rows run two-pass row and key kernels with hi + lo fp16 operand pairs
// (the row kernel then also forms dq itself), on the helper stream beside the main kernels.
// Everything is deterministic (no atomics on results).
#include <math.h>

#include "fast_common.h"
#include "plx_internal.h"

namespace plx {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------------------------------
// shared helpers
// ------------------------------------------------------------------------------------------

__device__ __forceinline__ float mx(const uint32_t* maxbits, int slot) { return __uint_as_float(maxbits[slot]); }

// Per-row statistics the key-major kernels bound their products with (see RowParams::rowmax).  After
// the row pass, a suffix maximum along the rows turns entry i into the maximum over rows >= i, and the
// rows that see key j are rows >= j - (Tk - Tq) (causal), so one load per statistic bounds a key.
enum RowStat { kStatG = 0, kStatU = 1, kStatE = 2, kStat1mA = 3, kStatDelta = 4, kRowStats = 5 };

__device__ __forceinline__ void rowmax_put(float* rowmax, int b, int g, int Hkv, int Tq_pad, int row, int slot, float v) {
  atomicMax(reinterpret_cast<uint32_t*>(rowmax) + ((static_cast<int64_t>(b) * Hkv + g) * kRowStats + slot) * Tq_pad + row,
            __float_as_uint(v));
}

// Sum of squares of the values of N fp16 operands (the lane's half of a row of 16 N elements).
template <int N>
__device__ __forceinline__ float sumsq(const f16x8 (&x)[N]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) s = fmaf(static_cast<float>(x[i][j]), static_cast<float>(x[i][j]), s);
  return s;
}

__device__ __forceinline__ void load4_bf16(const u16* src, float* dst) {
  const uint2 w = *reinterpret_cast<const uint2*>(src);
  dst[0] = __uint_as_float(w.x << 16);
  dst[1] = __uint_as_float(w.x & 0xffff0000u);
  dst[2] = __uint_as_float(w.y << 16);
  dst[3] = __uint_as_float(w.y & 0xffff0000u);
}

template <int NS>
__device__ __forceinline__ void load_row_operand(const u16* row, bool ok, int hh, float s, f16x8 (&B)[NS], int D) {
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    float a[4] = {0.f, 0.f, 0.f, 0.f}, c[4] = {0.f, 0.f, 0.f, 0.f};
    if (ok && 16 * st < D) {   // a row of D < 128 elements reads as zero-padded
      load4_bf16(row + 16 * st + 4 * hh, a);
      load4_bf16(row + 16 * st + 8 + 4 * hh, c);
    }
    B[st] = pack8(a[0] * s, a[1] * s, a[2] * s, a[3] * s, c[0] * s, c[1] * s, c[2] * s, c[3] * s);
  }
}

// 8 fp32 accumulator values (registers 8t..8t+7 of a tile, times s) as an fp16 operand, and its lo part.
__device__ __forceinline__ void to_operand(const float* v, float s, f16x8& hi, f16x8* lo) {
  float e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = v[j] * s;
  if (lo) pin8(e);
  hi = pack8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
  if (lo) *lo = pack_lo(e, hi);
}

// Same for registers 8t..8t+7 of an accumulator tile.
__device__ __forceinline__ void tile_operand(const f32x16& v, int t, float s, f16x8& hi, f16x8* lo) {
  float e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = v[8 * t + j];
  to_operand(e, s, hi, lo);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// ------------------------------------------------------------------------------------------
// query-major row kernel
// ------------------------------------------------------------------------------------------

struct RowParams {
  const u16 *q, *dout;
  const float *out, *lse, *kbar, *osa;
  const _Float16 *k16, *k16t, *v16, *p16t, *p16;
  uint32_t* maxbits;
  float *dq, *u32, *dkb32, *x32, *du32, *st_alpha, *st_delta;
  float* rstat;        // per 32-row tile: lse (log2 units), 1 - alpha, Delta of each row, [B][Hq][Tq_pad / 32][3][32]
  const float *knorm, *vnorm;   // [B][Hkv][Tk_pad] running maxima of the key and value norms (staging)
  float* rowmax;       // [B][Hkv][kRowStats][Tq_pad]: per row, the largest |g|, |u|, |dkbar|, |1 - alpha|, |Delta|
                       // over the group's query heads (atomicMax of non-negative float bits)
  // probe form (u = -rho supplied per row, no projector): rho, rho . kbar from the forward, drho out
  const u16* rho;
  const float* rk;
  float* drho;
  int D;               // head dim of the caller's rows (the kernels' DH)
  int B, Tq, Tk, Tk_pad, Tq_pad, Hq, Hkv, G, causal, window;
  float scale;
  int row_begin, row_end, rows_per_block, n_rb;
};

template <int DH>
struct __align__(16) RowTiles {
  _Float16 k[2][kKeyTile * DH];
  _Float16 v[2][kKeyTile * DH];
  _Float16 kt[2][DH * kKeyTile];
};

__device__ __forceinline__ f16x8 lds_rows(const _Float16* t, int r, int c) {
  return *reinterpret_cast<const f16x8*>(&t[c * (kKeyTile * 8) + r * 8]);
}
template <int DH>
__device__ __forceinline__ f16x8 lds_cols(const _Float16* t, int d, int c) {
  return *reinterpret_cast<const f16x8*>(&t[c * (DH * 8) + d * 8]);
}

// Asynchronous global -> LDS copy of one key tile: K rows, V rows and K^T, each one contiguous block of
// DH / 8 KB (DH / 8 wave instructions of 1024 bytes, DH / 32 per wave of four).
template <int DH>
__device__ __forceinline__ void row_tile_dma(const RowParams& p, RowTiles<DH>& T, int buf, int b, int g, int kt,
                                             int w, int l) {
  const int64_t tb = kv_tile(b, g, kt, p.Hkv, p.Tk_pad / kKeyTile, DH);
#pragma unroll
  for (int j = 0; j < DH / 32; ++j) {
    const int i = (DH / 32) * w + j;
    const int64_t src = tb + i * 512 + l * 8;
    lds_dma16(p.k16 + src, &T.k[buf][i * 512]);
    lds_dma16(p.v16 + src, &T.v[buf][i * 512]);
    lds_dma16(p.k16t + src, &T.kt[buf][i * 512]);
  }
}

// g.o, g.out and |g|_1 of the lane's query row (its two half-lanes combined).
template <int NT>
__device__ __forceinline__ void row_dots(const RowParams& p, int64_t qoff, bool row_ok, int hh, float& go,
                                         float& gout, float& gabs) {
  go = 0.f;
  gout = 0.f;
  gabs = 0.f;
#pragma unroll
  for (int mt = 0; mt < NT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * mt + 8 * j + 4 * hh;
      float gv[4] = {0.f, 0.f, 0.f, 0.f};
      float4 ov = {0.f, 0.f, 0.f, 0.f}, outv = {0.f, 0.f, 0.f, 0.f};
      if (row_ok) {
        if (d < p.D) load4_bf16(p.dout + qoff + d, gv);
        if (d < p.D) ov = *reinterpret_cast<const float4*>(p.osa + qoff + d);
        if (d < p.D) outv = *reinterpret_cast<const float4*>(p.out + qoff + d);
      }
      go += gv[0] * ov.x + gv[1] * ov.y + gv[2] * ov.z + gv[3] * ov.w;
      gout += gv[0] * outv.x + gv[1] * outv.y + gv[2] * outv.z + gv[3] * outv.w;
      gabs += fabsf(gv[0]) + fabsf(gv[1]) + fabsf(gv[2]) + fabsf(gv[3]);
    }
  go = xor32_sum(go);
  gout = xor32_sum(gout);
  gabs = xor32_sum(gabs);
}

// g.o and g.out of a wave's 32 query rows i0 .. i0 + 31 (head h, batch b), read a row per half-wave (each
// half reads one row's DH values contiguously, so the loads are whole cache lines), summed over the half
// and handed to the lanes that own the row (lanes r and r + 32 of the accumulator layout).
template <int DH>
__device__ __forceinline__ void row_dots_wave(const RowParams& p, int b, int h, int i0, int l, float& go, float& gout) {
  constexpr int PER = DH / 32;   // values of a row per lane
  const int half = l >> 5, c = l & 31;
  go = 0.f;
  gout = 0.f;
#pragma unroll 4
  for (int rp = 0; rp < 16; ++rp) {
    const int row = i0 + 2 * rp + half;
    float a = 0.f, o = 0.f;
    if (row < p.row_end) {
      const int64_t off = ((static_cast<int64_t>(b) * p.Tq + row) * p.Hq + h) * DH + PER * c;
      if constexpr (PER == 4) {
        float gv[4];
        load4_bf16(p.dout + off, gv);
        const float4 ov = *reinterpret_cast<const float4*>(p.osa + off);
        const float4 uv = *reinterpret_cast<const float4*>(p.out + off);
        a = gv[0] * ov.x + gv[1] * ov.y + gv[2] * ov.z + gv[3] * ov.w;
        o = gv[0] * uv.x + gv[1] * uv.y + gv[2] * uv.z + gv[3] * uv.w;
      } else {
        const uint32_t gw = *reinterpret_cast<const uint32_t*>(p.dout + off);
        const float g0 = __uint_as_float(gw << 16), g1 = __uint_as_float(gw & 0xffff0000u);
        const float2 ov = *reinterpret_cast<const float2*>(p.osa + off);
        const float2 uv = *reinterpret_cast<const float2*>(p.out + off);
        a = g0 * ov.x + g1 * ov.y;
        o = g0 * uv.x + g1 * uv.y;
      }
    }
#pragma unroll
    for (int sh = 16; sh > 0; sh >>= 1) {
      a += __shfl_xor(a, sh, 64);
      o += __shfl_xor(o, sh, 64);
    }
    // row i0 + 2 rp is summed in lanes 0-31, row i0 + 2 rp + 1 in lanes 32-63
    const float a0 = __shfl(a, 0, 64), a1 = __shfl(a, 32, 64), o0 = __shfl(o, 0, 64), o1 = __shfl(o, 32, 64);
    if (c == 2 * rp) {
      go = a0;
      gout = o0;
    }
    if (c == 2 * rp + 1) {
      go = a1;
      gout = o1;
    }
  }
}

// Probe form: the per-row vectors the key-major pass needs, from the supplied probe.  u = -rho,
// dkbar = -(g.o) u = (g.o) rho, drho = -du, and dq starts at 0 (no projector term).  Writes u, dkbar,
// drho and the zero dq of the lane's half-row; `du` holds du in the accumulator layout.
template <int NT>
__device__ __forceinline__ void probe_row_vectors(const RowParams& p, int64_t qoff, int64_t woff, bool row_ok, int hh,
                                                  float go,
                                                  const f32x16 (&du)[NT], f32x16 (&u)[NT], f32x16 (&dkb)[NT]) {
#pragma unroll
  for (int mt = 0; mt < NT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * mt + 8 * j + 4 * hh;
      float rv[4] = {0.f, 0.f, 0.f, 0.f};
      if (row_ok) if (d < p.D) load4_bf16(p.rho + qoff + d, rv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u[mt][4 * j + e] = -rv[e];
        dkb[mt][4 * j + e] = go * rv[e];
      }
      if (row_ok) {
        const int r = 4 * j;
        if (d < p.D) *reinterpret_cast<float4*>(p.drho + qoff + d) = float4{-du[mt][r], -du[mt][r + 1], -du[mt][r + 2], -du[mt][r + 3]};
        if (d < p.D) *reinterpret_cast<float4*>(p.dq + qoff + d) = float4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<float4*>(p.u32 + woff + d) = float4{u[mt][r], u[mt][r + 1], u[mt][r + 2], u[mt][r + 3]};
        *reinterpret_cast<float4*>(p.dkb32 + woff + d) = float4{dkb[mt][r], dkb[mt][r + 1], dkb[mt][r + 2], dkb[mt][r + 3]};
      }
    }
}

template <bool SPLIT, bool DQ_PASS, bool PROBE, int DH>
__global__ __launch_bounds__(256) void k_bwd_rows_fast(RowParams p) {
  constexpr int NS = DH / 16, NT = DH / 32;   // k-steps and accumulator tiles over d
  __shared__ RowTiles<DH> T;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, ql = l & 31, hh = l >> 5;
  // four waves: with 8 query heads per kv head, two blocks share a group, four heads each
  const int hsplit = p.G > 4 ? p.G / 4 : 1;
  const int npairs = p.B * p.Hkv * hsplit;
  int pair, rb;
  {
    const int id = blockIdx.x;
    if ((npairs & 7) == 0) {
      const int ppx = npairs >> 3, slot = id >> 3;
      rb = p.n_rb - 1 - slot / ppx;
      pair = (id & 7) + 8 * (slot % ppx);
    } else {
      rb = p.n_rb - 1 - id / npairs;
      pair = id % npairs;
    }
  }
  const int b = pair / (p.Hkv * hsplit), g = pair % (p.Hkv * hsplit) / hsplit, hpart = pair % hsplit;
  const int wph = p.G > 4 ? 1 : 4 / p.G;
  const int h = g * p.G + 4 * hpart + w / wph;
  const int r0 = p.row_begin + rb * p.rows_per_block;
  const int i0 = r0 + (w % wph) * 32;
  const int row = i0 + ql;
  const bool row_ok = row < p.row_end;
  const int off = p.Tk - p.Tq;
  const uint32_t* MB = p.maxbits;
  const float sQ = range_scale(mx(MB, kMaxQ)), sK = range_scale(mx(MB, kMaxK));
  const float sV = range_scale(mx(MB, kMaxV)), sP = range_scale(mx(MB, kMaxP));
  const float sG = range_scale(mx(MB, kMaxDO));
  const float maxK = mx(MB, kMaxK);
  const float cS = p.scale * kLog2e / (sQ * sK);

  const int64_t qoff = ((static_cast<int64_t>(b) * p.Tq + (row_ok ? row : 0)) * p.Hq + h) * p.D;   // caller rows
  const int64_t woff = ((static_cast<int64_t>(b) * p.Tq + (row_ok ? row : 0)) * p.Hq + h) * DH;    // workspace rows
  const int64_t soff = (static_cast<int64_t>(b) * p.Hq + h) * p.Tq + (row_ok ? row : 0);
  float lse2 = row_ok ? p.lse[soff] * kLog2e : 0.f;
  if (!(lse2 > -INFINITY && lse2 < INFINITY)) lse2 = 0.f;  // a row without keys: every S is masked

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

  f16x8 qB[NS], gB[NS];
  load_row_operand(p.q + qoff, row_ok, hh, sQ, qB, p.D);
  load_row_operand(p.dout + qoff, row_ok, hh, sG, gB, p.D);
  // |G_j| = |g.v_j| <= |g| |v_j| with the largest value norm among the keys the row sees (a running
  // maximum along the sequence), so the scale of p G follows the row instead of the tensors' largest
  // entries (probe form: |G - g.o| <= 2 |g| max |v_j|)
  const float gnorm = sqrtf(xor32_sum(sumsq(gB))) / sG;
  const int64_t nbase = (static_cast<int64_t>(b) * p.Hkv + g) * p.Tk_pad;
  const float pmV = r_kend > r_kbeg ? p.vnorm[nbase + r_kend - 1] : 0.f;
  const float sPG = range_scale(PROBE ? 2.f * gnorm * pmV : gnorm * pmV);

  // probe form: du = sum_j p_j (G_j - g.o) k_j directly (kbar is not an input), so g.o comes first
  float go_pre = 0.f;
  if constexpr (PROBE) {
#pragma unroll
    for (int d = 4 * hh; d < DH; d += 8) {
      float gv[4] = {0.f, 0.f, 0.f, 0.f};
      float4 ov = {0.f, 0.f, 0.f, 0.f};
      if (row_ok) {
        if (d < p.D) load4_bf16(p.dout + qoff + d, gv);
        if (d < p.D) ov = *reinterpret_cast<const float4*>(p.osa + qoff + d);
      }
      go_pre += gv[0] * ov.x + gv[1] * ov.y + gv[2] * ov.z + gv[3] * ov.w;
    }
    go_pre = xor32_sum(go_pre);
  }
  const float goS = go_pre * sG * sV;   // g.o in the units of the G tile

  // ---------------- pass 1: du ----------------
  f32x16 accDU[NT];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) accDU[mt] = f32x16{};
  const float fPG = sPG / (sG * sV);
  if (t_beg < t_end) row_tile_dma(p, T, 0, b, g, t_beg, w, l);
  lds_dma_wait();
  __syncthreads();
  for (int kt = t_beg; kt < t_end; ++kt) {
    const int buf = (kt - t_beg) & 1;
    if (kt + 1 < t_end) row_tile_dma(p, T, buf ^ 1, b, g, kt + 1, w, l);
    const int key0 = kt * kKeyTile;
    if (key0 < w_kend && key0 + kKeyTile > w_kbeg) {
      const bool full = key0 + kKeyTile <= w_full_end && key0 >= w_full_beg;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 S = {}, Gt = {};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          S = mfma(lds_rows(T.k[buf], 32 * kb + ql, 2 * s + hh), qB[s], S);
          Gt = mfma(lds_rows(T.v[buf], 32 * kb + ql, 2 * s + hh), gB[s], Gt);
        }
        float pg[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          float sv = S[r];
          if (!full && (key >= r_kend || key < r_kbeg)) sv = -INFINITY;
          pg[r] = __builtin_amdgcn_exp2f(fmaf(sv, cS, -lse2)) * (PROBE ? Gt[r] - goS : Gt[r]) * fPG;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f16x8 hi, lo;
          to_operand(pg + 8 * t, 1.f, hi, SPLIT ? &lo : nullptr);
#pragma unroll
          for (int mt = 0; mt < NT; ++mt) {
            const f16x8 a = lds_cols<DH>(T.kt[buf], 32 * mt + ql, 4 * kb + 2 * t + hh);
            accDU[mt] = mfma(a, hi, accDU[mt]);
            if constexpr (SPLIT) accDU[mt] = mfma(a, lo, accDU[mt]);
          }
        }
      }
    }
    lds_dma_wait();
    __syncthreads();
  }

  // ---------------- epilogue: u, alpha, P du, dkbar, Delta ----------------
  // row vectors in the accumulator layout: element (mt, r) is d = 32 mt + 8 (r/4) + 4 hh + r%4
  float go, gout, gabs;
  row_dots<NT>(p, qoff, row_ok, hh, go, gout, gabs);
  if constexpr (PROBE) go = go_pre;   // the value du was formed with
  f32x16 accU[NT], accPD[NT];
  float alpha = 0.f, dkk = 0.f, umax = 0.f, emax = 0.f, u1 = 0.f, e1 = 0.f, u2 = 0.f, e2 = 0.f;
  if constexpr (PROBE) {
    const float fdu = 1.f / (sPG * sK);
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) accDU[mt] *= fdu;
    probe_row_vectors<NT>(p, qoff, woff, row_ok, hh, go, accDU, accU, accPD);
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        umax = fmaxf(umax, fabsf(accU[mt][r]));
        emax = fmaxf(emax, fabsf(accPD[mt][r]));
        u2 = fmaf(accU[mt][r], accU[mt][r], u2);
        e2 = fmaf(accPD[mt][r], accPD[mt][r], e2);
        u1 += fabsf(accU[mt][r]);
        e1 += fabsf(accPD[mt][r]);
      }
    umax = xor32_max(umax);
    emax = xor32_max(emax);
    u2 = xor32_sum(u2);
    e2 = xor32_sum(e2);
    u1 = xor32_sum(u1);
    e1 = xor32_sum(e1);
    const float rk = row_ok ? p.rk[soff] : 0.f;   // rho . kbar
    alpha = -rk;                                  // u . kbar
    dkk = go * rk;                                // dkbar . kbar
  } else {
    // kbar, x = q - kbar (written out for dP), du = sum p G k - (g.o) kbar (in place, written out)
    float kbv[NT][16], xv[NT][16];
    float xmax = 0.f, dumax = 0.f;
    {
      const float fdu = 1.f / (sPG * sK);
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * mt + 8 * j + 4 * hh;
          float qv[4] = {0.f, 0.f, 0.f, 0.f};
          float4 kv = {0.f, 0.f, 0.f, 0.f};
          if (row_ok) {
            if (d < p.D) load4_bf16(p.q + qoff + d, qv);
            if (d < p.D) kv = *reinterpret_cast<const float4*>(p.kbar + qoff + d);
          }
          const float k4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * j + e;
            kbv[mt][r] = k4[e];
            xv[mt][r] = qv[e] - k4[e];
            accDU[mt][r] = accDU[mt][r] * fdu - go * k4[e];
            xmax = fmaxf(xmax, fabsf(xv[mt][r]));
            dumax = fmaxf(dumax, fabsf(accDU[mt][r]));
          }
          if (row_ok) {
            *reinterpret_cast<float4*>(p.x32 + woff + d) =
                float4{xv[mt][4 * j], xv[mt][4 * j + 1], xv[mt][4 * j + 2], xv[mt][4 * j + 3]};
            *reinterpret_cast<float4*>(p.du32 + woff + d) =
                float4{accDU[mt][4 * j], accDU[mt][4 * j + 1], accDU[mt][4 * j + 2], accDU[mt][4 * j + 3]};
          }
        }
    }
    xmax = xor32_max(xmax);
    dumax = xor32_max(dumax);
    const float sX = range_scale(xmax), sDU = range_scale(dumax);
    // U^T = P16t X^T, then (P du)^T = P16 du^T
    {
      f16x8 xB[NS], xL[SPLIT ? NS : 1];
#pragma unroll
      for (int s = 0; s < NS; ++s) to_operand(&xv[s >> 1][(s & 1) * 8], sX, xB[s], SPLIT ? &xL[SPLIT ? s : 0] : nullptr);
      const _Float16* prt = p.p16t + (static_cast<int64_t>(h) * DH + ql) * DH + hh * 8;
#pragma unroll
      for (int am = 0; am < NT; ++am) {
        accU[am] = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const f16x8 at = *reinterpret_cast<const f16x8*>(prt + 32 * am * DH + 16 * s);
          accU[am] = mfma(at, xB[s], accU[am]);
          if constexpr (SPLIT) accU[am] = mfma(at, xL[SPLIT ? s : 0], accU[am]);
        }
      }
    }
    {
      f16x8 dB[NS], dL[SPLIT ? NS : 1];
#pragma unroll
      for (int s = 0; s < NS; ++s)
        tile_operand(accDU[s >> 1], s & 1, sDU, dB[s], SPLIT ? &dL[SPLIT ? s : 0] : nullptr);
      const _Float16* pr = p.p16 + (static_cast<int64_t>(h) * DH + ql) * DH + hh * 8;
#pragma unroll
      for (int am = 0; am < NT; ++am) {
        accPD[am] = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const f16x8 a = *reinterpret_cast<const f16x8*>(pr + 32 * am * DH + 16 * s);
          accPD[am] = mfma(a, dB[s], accPD[am]);
          if constexpr (SPLIT) accPD[am] = mfma(a, dL[SPLIT ? s : 0], accPD[am]);
        }
      }
    }
    // u (in accU), dq0 = P du (written to dq now, completed after pass 2), dkbar (in accPD), alpha, Delta
    {
      const float fu = 1.f / (sX * sP), fpd = 1.f / (sP * sDU);
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * mt + 8 * j + 4 * hh;
          float pd4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * j + e;
            const float u = accU[mt][r] * fu;
            const float pd = accPD[mt][r] * fpd;
            const float dk = -go * u - pd;
            pd4[e] = pd;
            accU[mt][r] = u;
            accPD[mt][r] = dk;
            alpha += u * kbv[mt][r];
            dkk += dk * kbv[mt][r];
            umax = fmaxf(umax, fabsf(u));
            emax = fmaxf(emax, fabsf(dk));
            u2 = fmaf(u, u, u2);
            e2 = fmaf(dk, dk, e2);
            u1 += fabsf(u);
            e1 += fabsf(dk);
          }
          if (row_ok) {
            if (d < p.D) *reinterpret_cast<float4*>(p.dq + qoff + d) = float4{pd4[0], pd4[1], pd4[2], pd4[3]};
            *reinterpret_cast<float4*>(p.u32 + woff + d) =
                float4{accU[mt][4 * j], accU[mt][4 * j + 1], accU[mt][4 * j + 2], accU[mt][4 * j + 3]};
            *reinterpret_cast<float4*>(p.dkb32 + woff + d) =
                float4{accPD[mt][4 * j], accPD[mt][4 * j + 1], accPD[mt][4 * j + 2], accPD[mt][4 * j + 3]};
          }
        }
    }
    alpha = xor32_sum(alpha);
    dkk = xor32_sum(dkk);
    umax = xor32_max(umax);
    emax = xor32_max(emax);
    u2 = xor32_sum(u2);
    e2 = xor32_sum(e2);
    u1 = xor32_sum(u1);
    e1 = xor32_sum(e1);
  }
  const float delta = gout + dkk;
  if (row_ok && hh == 0) {
    p.st_alpha[soff] = alpha;
    p.st_delta[soff] = delta;
    float* rs = p.rstat + ((static_cast<int64_t>(b) * p.Hq + h) * (p.Tq_pad / 32) + row / 32) * 96 + row % 32;
    rs[0] = lse2;
    rs[32] = 1.f - alpha;
    rs[64] = delta;
    const float st5[kRowStats] = {gnorm, sqrtf(u2), sqrtf(e2), fabsf(1.f - alpha), fabsf(delta)};
#pragma unroll
    for (int k = 0; k < kRowStats; ++k) rowmax_put(p.rowmax, b, g, p.Hkv, p.Tq_pad, row, k, st5[k]);
  }
  {
    // per-tensor maxima for the key-major pass (rows outside the range contribute 0)
    const float wu = wave_max(row_ok ? umax : 0.f), we = wave_max(row_ok ? emax : 0.f);
    const float wd = wave_max(row_ok ? fabsf(delta) : 0.f), wa = wave_max(row_ok ? fabsf(alpha) : 0.f);
    if (l == 0) {
      atomicMax(&p.maxbits[kMaxU], __float_as_uint(wu));
      atomicMax(&p.maxbits[kMaxDKB], __float_as_uint(we));
      atomicMax(&p.maxbits[kMaxDelta], __float_as_uint(wd));
      atomicMax(&p.maxbits[kMaxAlpha], __float_as_uint(wa));
    }
  }

  if constexpr (!DQ_PASS) return;   // dq is completed by k_bwd_dq from the stored ds

  // ---------------- pass 2: dq ----------------
  const float sU = range_scale(umax), sE = range_scale(emax);
  f16x8 uB[NS], uL[SPLIT ? NS : 1], eB[NS], eL[SPLIT ? NS : 1];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    tile_operand(accU[s >> 1], s & 1, sU, uB[s], SPLIT ? &uL[SPLIT ? s : 0] : nullptr);
    tile_operand(accPD[s >> 1], s & 1, sE, eB[s], SPLIT ? &eL[SPLIT ? s : 0] : nullptr);
  }
  // |ds| <= |G| |tt| + |E| + |Delta| with |G| <= |g| max|v_j|, |tt| <= |u| max|k_j| + |1 - alpha|,
  // |E| <= |dkbar| max|k_j|: Euclidean norms, and the largest key and value norms among the row's keys
  const float pmK = r_kend > r_kbeg ? p.knorm[nbase + r_kend - 1] : 0.f;
  const float bound_ds = gnorm * pmV * (sqrtf(u2) * pmK + fabsf(1.f - alpha)) + sqrtf(e2) * pmK + fabsf(delta);
  const float sDS = range_scale(bound_ds);
  const float fT = 1.f / (sU * sK), fE = 1.f / (sE * sK), fG = 1.f / (sG * sV);
  const float one_m_alpha = 1.f - alpha;
  f32x16 accDQ[NT];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) accDQ[mt] = f32x16{};
  if (t_beg < t_end) row_tile_dma(p, T, 0, b, g, t_beg, w, l);
  lds_dma_wait();
  __syncthreads();
  for (int kt = t_beg; kt < t_end; ++kt) {
    const int buf = (kt - t_beg) & 1;
    if (kt + 1 < t_end) row_tile_dma(p, T, buf ^ 1, b, g, kt + 1, w, l);
    const int key0 = kt * kKeyTile;
    if (key0 < w_kend && key0 + kKeyTile > w_kbeg) {
      const bool full = key0 + kKeyTile <= w_full_end && key0 >= w_full_beg;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 S = {}, Tt = {}, E = {}, Gt = {};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const f16x8 a = lds_rows(T.k[buf], 32 * kb + ql, 2 * s + hh);
          S = mfma(a, qB[s], S);
          Tt = mfma(a, uB[s], Tt);
          E = mfma(a, eB[s], E);
          if constexpr (SPLIT) {
            Tt = mfma(a, uL[s], Tt);
            E = mfma(a, eL[s], E);
          }
          Gt = mfma(lds_rows(T.v[buf], 32 * kb + ql, 2 * s + hh), gB[s], Gt);
        }
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          float sv = S[r];
          if (!full && (key >= r_kend || key < r_kbeg)) sv = -INFINITY;
          const float pr = __builtin_amdgcn_exp2f(fmaf(sv, cS, -lse2));
          const float tt = fmaf(Tt[r], fT, one_m_alpha);
          const float dp = fmaf(Gt[r] * fG, tt, E[r] * fE);
          ds[r] = pr * (dp - delta) * sDS;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f16x8 hi, lo;
          to_operand(ds + 8 * t, 1.f, hi, SPLIT ? &lo : nullptr);
#pragma unroll
          for (int mt = 0; mt < NT; ++mt) {
            const f16x8 a = lds_cols<DH>(T.kt[buf], 32 * mt + ql, 4 * kb + 2 * t + hh);
            accDQ[mt] = mfma(a, hi, accDQ[mt]);
            if constexpr (SPLIT) accDQ[mt] = mfma(a, lo, accDQ[mt]);
          }
        }
      }
    }
    lds_dma_wait();
    __syncthreads();
  }
  if (row_ok) {
    const float fq = p.scale / (sDS * sK);
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * mt + 8 * j + 4 * hh;
        if (d >= p.D) continue;   // padding dims of a D < 128 head
        const int r = 4 * j;
        const float4 q0 = *reinterpret_cast<const float4*>(p.dq + qoff + d);  // P du from the epilogue
        *reinterpret_cast<float4*>(p.dq + qoff + d) =
            float4{q0.x + accDQ[mt][r] * fq, q0.y + accDQ[mt][r + 1] * fq, q0.z + accDQ[mt][r + 2] * fq,
                   q0.w + accDQ[mt][r + 3] * fq};
      }
  }
}

// ------------------------------------------------------------------------------------------
// query-major kernel for rows >= split: du and the per-row epilogue, 8 waves (2 per SIMD)
// ------------------------------------------------------------------------------------------
// The first pass and the epilogue of k_bwd_rows_fast for 32 rows per wave and 8 waves per block
// (dq is completed from the stored ds by k_bwd_dq).  The epilogue re-reads q and kbar where it needs
// them instead of holding them in registers, so that a wave fits in the 256 registers that two waves
// per SIMD leave it.

template <int DH>
__device__ __forceinline__ void row_tile_dma8(const RowParams& p, RowTiles<DH>& T, int buf, int b, int g, int kt,
                                              int w, int l) {
  const int64_t tb = kv_tile(b, g, kt, p.Hkv, p.Tk_pad / kKeyTile, DH);
#pragma unroll
  for (int j = 0; j < DH / 64; ++j) {
    const int i = (DH / 64) * w + j;
    const int64_t src = tb + i * 512 + l * 8;
    lds_dma16(p.k16 + src, &T.k[buf][i * 512]);
    lds_dma16(p.v16 + src, &T.v[buf][i * 512]);
    lds_dma16(p.k16t + src, &T.kt[buf][i * 512]);
  }
}

template <bool PROBE, int DH>
__global__ __launch_bounds__(512) void k_bwd_du(RowParams p) {
  constexpr int NS = DH / 16, NT = DH / 32;   // k-steps and accumulator tiles over d
  __shared__ RowTiles<DH> T;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, ql = l & 31, hh = l >> 5;
  const int npairs = p.B * p.Hkv;
  int pair, rb;
  {
    const int id = blockIdx.x;
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
  const int wph = 8 / p.G;
  const int h = g * p.G + w / wph;
  const int r0 = p.row_begin + rb * p.rows_per_block;
  const int i0 = r0 + (w % wph) * 32;
  const int row = i0 + ql;
  const bool row_ok = row < p.row_end;
  const int off = p.Tk - p.Tq;
  const uint32_t* MB = p.maxbits;
  const float sQ = range_scale(mx(MB, kMaxQ)), sK = range_scale(mx(MB, kMaxK));
  const float sV = range_scale(mx(MB, kMaxV)), sP = range_scale(mx(MB, kMaxP));
  const float sG = range_scale(mx(MB, kMaxDO));
  const float cS = p.scale * kLog2e / (sQ * sK);

  const int64_t qoff = ((static_cast<int64_t>(b) * p.Tq + (row_ok ? row : 0)) * p.Hq + h) * p.D;   // caller rows
  const int64_t woff = ((static_cast<int64_t>(b) * p.Tq + (row_ok ? row : 0)) * p.Hq + h) * DH;    // workspace rows
  const int64_t soff = (static_cast<int64_t>(b) * p.Hq + h) * p.Tq + (row_ok ? row : 0);
  float lse2 = row_ok ? p.lse[soff] * kLog2e : 0.f;
  if (!(lse2 > -INFINITY && lse2 < INFINITY)) lse2 = 0.f;  // a row without keys: every S is masked

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

  f16x8 qB[NS], gB[NS];
  load_row_operand(p.q + qoff, row_ok, hh, sQ, qB, p.D);
  load_row_operand(p.dout + qoff, row_ok, hh, sG, gB, p.D);
  // |G_j| = |g.v_j| <= |g| |v_j| with the largest value norm among the keys the row sees (a running
  // maximum along the sequence), so the scale of p G follows the row instead of the tensors' largest
  // entries (probe form: |G - g.o| <= 2 |g| max |v_j|)
  const float gnorm = sqrtf(xor32_sum(sumsq(gB))) / sG;
  const int64_t nbase = (static_cast<int64_t>(b) * p.Hkv + g) * p.Tk_pad;
  const float pmV = r_kend > r_kbeg ? p.vnorm[nbase + r_kend - 1] : 0.f;
  const float sPG = range_scale(PROBE ? 2.f * gnorm * pmV : gnorm * pmV);

  // g.o and g.out of the row, read while the first tile is being copied (the probe form forms du =
  // sum_j p_j (G_j - g.o) k_j directly, kbar not being an input, so it needs g.o first)
  if (t_beg < t_end) row_tile_dma8(p, T, 0, b, g, t_beg, w, l);
  float go, gout;
  row_dots_wave<DH>(p, b, h, i0, l, go, gout);
  const float goS = PROBE ? go * sG * sV : 0.f;   // g.o in the units of the G tile

  // ---------------- du = sum_j p_j G_j k_j (scaled) ----------------
  f32x16 accDU[NT];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) accDU[mt] = f32x16{};
  const float fPG = sPG / (sG * sV);
  lds_dma_wait();
  __syncthreads();
  for (int kt = t_beg; kt < t_end; ++kt) {
    const int buf = (kt - t_beg) & 1;
    if (kt + 1 < t_end) row_tile_dma8(p, T, buf ^ 1, b, g, kt + 1, w, l);
    const int key0 = kt * kKeyTile;
    if (key0 < w_kend && key0 + kKeyTile > w_kbeg) {
      const bool full = key0 + kKeyTile <= w_full_end && key0 >= w_full_beg;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 S = {}, Gt = {};
        // K and V row operands of chunk s + 2 are read while the MFMAs of chunk s run; the
        // scheduling barriers keep the compiler from moving the reads next to their MFMAs
        f16x8 a[3][2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          a[s][0] = lds_rows(T.k[buf], 32 * kb + ql, 2 * s + hh);
          a[s][1] = lds_rows(T.v[buf], 32 * kb + ql, 2 * s + hh);
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if (s + 2 < NS) {
            a[(s + 2) % 3][0] = lds_rows(T.k[buf], 32 * kb + ql, 2 * (s + 2) + hh);
            a[(s + 2) % 3][1] = lds_rows(T.v[buf], 32 * kb + ql, 2 * (s + 2) + hh);
          }
          __builtin_amdgcn_sched_barrier(0);
          S = mfma(a[s % 3][0], qB[s], S);
          Gt = mfma(a[s % 3][1], gB[s], Gt);
          __builtin_amdgcn_sched_barrier(0);
        }
        // the K^T operands of the first du products, read while the weights are formed
        f16x8 kc[NT];
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) kc[mt] = lds_cols<DH>(T.kt[buf], 32 * mt + ql, 4 * kb + hh);
        if (!full) {   // tiles on the causal / window edge only
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= r_kend || key < r_kbeg) S[r] = -INFINITY;
          }
        }
        float pg[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) pg[r] = __builtin_amdgcn_exp2f(fmaf(S[r], cS, -lse2)) * (PROBE ? Gt[r] - goS : Gt[r]) * fPG;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f16x8 hi;
          to_operand(pg + 8 * t, 1.f, hi, nullptr);
#pragma unroll
          for (int mt = 0; mt < NT; ++mt) {
            accDU[mt] = mfma(kc[mt], hi, accDU[mt]);
            if (t == 0) kc[mt] = lds_cols<DH>(T.kt[buf], 32 * mt + ql, 4 * kb + 2 + hh);
          }
        }
      }
    }
    lds_dma_wait();
    __syncthreads();
  }

  // ---------------- epilogue ----------------
  // row vectors in the accumulator layout: element (mt, r) is d = 32 mt + 8 (r/4) + 4 hh + r%4; they move
  // to and from memory through the tile buffers, which are free now (every wave has passed the loop)
  WaveRows wr;
  wr.lds = reinterpret_cast<float*>(&T) + w * 32 * kWR;
  wr.rstride = static_cast<int64_t>(p.Hq) * DH;
  wr.base = ((static_cast<int64_t>(b) * p.Tq + min(i0, p.Tq - 1)) * p.Hq + h) * DH;
  wr.nrows = max(0, min(32, p.row_end - i0));
  wr.l = l;
  wr.ql = ql;
  wr.hh = hh;
  float alpha = 0.f, dkk = 0.f, umax = 0.f, emax = 0.f, u2 = 0.f, e2 = 0.f;
  if constexpr (PROBE) {
    // u = -rho, dkbar = (g.o) rho, drho = -du, dq starts at 0 (no projector term)
    const float fdu = 1.f / (sPG * sK);
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      float rv[16], v[16];
      wr.load<false>(p.rho, mt, rv);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        umax = fmaxf(umax, fabsf(rv[r]));
        emax = fmaxf(emax, fabsf(go * rv[r]));
        u2 = fmaf(rv[r], rv[r], u2);
        e2 = fmaf(go * rv[r], go * rv[r], e2);
        v[r] = -accDU[mt][r] * fdu;
      }
      wr.store(p.drho, mt, v);
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = 0.f;
      wr.store(p.dq, mt, v);
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = -rv[r];
      wr.store(p.u32, mt, v);
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = go * rv[r];
      wr.store(p.dkb32, mt, v);
    }
    umax = xor32_max(umax);
    emax = xor32_max(emax);
    u2 = xor32_sum(u2);
    e2 = xor32_sum(e2);
    const float rk = row_ok ? p.rk[soff] : 0.f;   // rho . kbar
    alpha = -rk;                                  // u . kbar
    dkk = go * rk;                                // dkbar . kbar
  } else {
    // du = sum p G k - (g.o) kbar (in place) and x = q - kbar, both written out for dP
    float xmax = 0.f, dumax = 0.f;
    {
      const float fdu = 1.f / (sPG * sK);
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        float kv[16], qv[16], xv[16], dv[16];
        wr.load<true>(p.kbar, mt, kv);
        wr.load<false>(p.q, mt, qv);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          xv[r] = qv[r] - kv[r];
          accDU[mt][r] = accDU[mt][r] * fdu - go * kv[r];
          dv[r] = accDU[mt][r];
          xmax = fmaxf(xmax, fabsf(xv[r]));
          dumax = fmaxf(dumax, fabsf(accDU[mt][r]));
        }
        wr.store(p.x32, mt, xv);
        wr.store(p.du32, mt, dv);
      }
    }
    xmax = xor32_max(xmax);
    dumax = xor32_max(dumax);
    const float sX = range_scale(xmax), sDU = range_scale(dumax);
    // (P du)^T = P16 du^T
    f32x16 accU[NT], accPD[NT];
    {
      f16x8 dB[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) tile_operand(accDU[s >> 1], s & 1, sDU, dB[s], nullptr);
      const _Float16* pr = p.p16 + (static_cast<int64_t>(h) * DH + ql) * DH + hh * 8;
#pragma unroll
      for (int am = 0; am < NT; ++am) {
        accPD[am] = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s) accPD[am] = mfma(*reinterpret_cast<const f16x8*>(pr + 32 * am * DH + 16 * s), dB[s], accPD[am]);
      }
    }
    // U^T = P16t X^T, with x = q - kbar re-read: operands 2 mt and 2 mt + 1 are registers 0-7 and 8-15 of tile mt
    {
      f16x8 xB[NS];
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        float kv[16], qv[16];
        wr.load<true>(p.kbar, mt, kv);
        wr.load<false>(p.q, mt, qv);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float x8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x8[e] = qv[8 * t + e] - kv[8 * t + e];
          to_operand(x8, sX, xB[2 * mt + t], nullptr);
        }
      }
      const _Float16* prt = p.p16t + (static_cast<int64_t>(h) * DH + ql) * DH + hh * 8;
#pragma unroll
      for (int am = 0; am < NT; ++am) {
        accU[am] = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s) accU[am] = mfma(*reinterpret_cast<const f16x8*>(prt + 32 * am * DH + 16 * s), xB[s], accU[am]);
      }
    }
    // u, dq0 = P du (completed by k_bwd_dq), dkbar = -(g.o) u - P du, alpha = u.kbar, Delta = g.out + dkbar.kbar
    {
      const float fu = 1.f / (sX * sP), fpd = 1.f / (sP * sDU);
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        float kv[16], uv[16], pv[16], ev[16];
        wr.load<true>(p.kbar, mt, kv);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          uv[r] = accU[mt][r] * fu;
          pv[r] = accPD[mt][r] * fpd;
          ev[r] = -go * uv[r] - pv[r];
          alpha += uv[r] * kv[r];
          dkk += ev[r] * kv[r];
          umax = fmaxf(umax, fabsf(uv[r]));
          emax = fmaxf(emax, fabsf(ev[r]));
          u2 = fmaf(uv[r], uv[r], u2);
          e2 = fmaf(ev[r], ev[r], e2);
        }
        wr.store(p.dq, mt, pv);
        wr.store(p.u32, mt, uv);
        wr.store(p.dkb32, mt, ev);
      }
    }
    alpha = xor32_sum(alpha);
    dkk = xor32_sum(dkk);
    umax = xor32_max(umax);
    emax = xor32_max(emax);
    u2 = xor32_sum(u2);
    e2 = xor32_sum(e2);
  }
  const float delta = gout + dkk;
  if (row_ok && hh == 0) {
    p.st_alpha[soff] = alpha;
    p.st_delta[soff] = delta;
    float* rs = p.rstat + ((static_cast<int64_t>(b) * p.Hq + h) * (p.Tq_pad / 32) + row / 32) * 96 + row % 32;
    rs[0] = lse2;
    rs[32] = 1.f - alpha;
    rs[64] = delta;
    const float st5[kRowStats] = {gnorm, sqrtf(u2), sqrtf(e2), fabsf(1.f - alpha), fabsf(delta)};
#pragma unroll
    for (int k = 0; k < kRowStats; ++k) rowmax_put(p.rowmax, b, g, p.Hkv, p.Tq_pad, row, k, st5[k]);
  }
  {
    // per-tensor maxima for the key-major pass (rows outside the range contribute 0), combined over
    // the block first: the atomics all go to the same few words, where they serialise
    __shared__ float red[4][8];
    const float wu = wave_max(row_ok ? umax : 0.f), we = wave_max(row_ok ? emax : 0.f);
    const float wd = wave_max(row_ok ? fabsf(delta) : 0.f), wa = wave_max(row_ok ? fabsf(alpha) : 0.f);
    if (l == 0) {
      red[0][w] = wu;
      red[1][w] = we;
      red[2][w] = wd;
      red[3][w] = wa;
    }
    __syncthreads();
    if (tid < 4) {
      float m = 0.f;
#pragma unroll
      for (int v = 0; v < 8; ++v) m = fmaxf(m, red[tid][v]);
      const int slot = tid == 0 ? kMaxU : tid == 1 ? kMaxDKB : tid == 2 ? kMaxDelta : kMaxAlpha;
      atomicMax(&p.maxbits[slot], __float_as_uint(m));
    }
  }
}

// ------------------------------------------------------------------------------------------
// key-major kernel: dk, dv
// ------------------------------------------------------------------------------------------

struct KeyParams {
  const _Float16 *k16, *v16;
  const _Float16 *q16, *do16, *u16, *e16, *u16lo, *e16lo;   // query-row tiles (and lo halves of u, e)
  const float *lse, *alpha, *delta;
  const uint32_t* maxbits;
  float *dk, *dv;
  _Float16* ds;        // k_bwd_keys_pipe: ds tiles for the dq kernel
  float* dsscale;      // [B][Hkv][Tk_pad / 32]: the scale C of each 32-key group's stored ds tiles
  const float* rowmax; // suffix maxima of the row statistics (see RowParams::rowmax)
  const float* rstat;  // row statistics per 32-row tile (see RowParams)
  int64_t qstride;     // elements between the consecutive query-row copies q16, do16, u16, e16
  int B, Tq, Tk, Tk_pad, Tq_pad, lo_pad, Hq, Hkv, G, causal, window;
  int D;               // head dim of dk, dv rows
  int out_keys;        // k_bwd_keys_fast: keys per batch entry in dk, dv (Tk, or the split rows' buffer)
  float scale;
  int row_lo, row_hi, accumulate, n_kb, key_hi;
};

// Scales of one key's products in the key-major kernels.  dk accumulates (p G) u + p dkbar + scale ds q
// on one accumulator, so the three fp16 operands share a scale C: p G C / sU, p C / sE and
// scale ds C / sQ against the staged u, dkbar and q (scales sU, sE, sQ); dv uses p tt cV.  The bounds
// are Euclidean: |G_ij| <= |g_i| |v_j|, |tt_ij| <= |u_i| |k_j| + |1 - alpha_i|, |E_ij| <= |dkbar_i| |k_j|,
// |ds_ij| <= |G| |tt| + |E| + |Delta_i| (p <= 1), with the key's own norms and, for each row statistic,
// its largest value over the rows that see the key (the suffix maxima of RowParams::rowmax).  So one
// row or key far larger than the rest changes only the scales of the keys it meets.
struct KeyLaneScales {
  float C, cV;
  bool seen;   // some row can see the key
};

__device__ __forceinline__ KeyLaneScales key_lane_scales(const KeyParams& p, int b, int g, int key, bool key_ok,
                                                         float kn, float vn, float sU, float sE, float sQ) {
  const int off = p.Tk - p.Tq;
  const int i_min = p.causal ? max(0, key - off) : 0;
  KeyLaneScales r;
  r.seen = key_ok && i_min < p.Tq;
  float st[kRowStats] = {0.f, 0.f, 0.f, 0.f, 0.f};
  if (r.seen) {
    const float* rm = p.rowmax + (static_cast<int64_t>(b) * p.Hkv + g) * kRowStats * p.Tq_pad + i_min;
#pragma unroll
    for (int k = 0; k < kRowStats; ++k) st[k] = rm[k * p.Tq_pad];
  }
  const float gmax = vn * st[kStatG];
  const float tmax = kn * st[kStatU] + st[kStat1mA];
  const float emax = kn * st[kStatE];
  const float dsmax = gmax * tmax + emax + st[kStatDelta];
  r.cV = range_scale(tmax);
  float C = range_scale(gmax) * sU;
  C = fminf(C, 16384.f * sE);
  r.C = fminf(C, range_scale(p.scale * dsmax) * sQ);
  return r;
}

// One query tile in LDS: query-row tiles [DH/8 chunks][32 rows][8] (chunk-major, as staged); the
// column-layout operands are read from them with transpose loads (tr_cols).
template <bool SPLIT, int DH>
struct __align__(16) KeyTiles {
  static constexpr int NR = SPLIT ? 6 : 4;   // q, dO, u, e (+ u lo, e lo)
  static constexpr int NB = SPLIT ? 1 : 2;
  _Float16 r[NB][NR][32 * DH];
  float stat[NB][3][32];                     // lse2, alpha, delta of the tile's rows
};

__device__ __forceinline__ f16x8 kt_rows(const _Float16* t, int r, int c) {
  return *reinterpret_cast<const f16x8*>(&t[c * (kQTile * 8) + r * 8]);
}
// The same from a tile stored with the per-chunk row swizzle (row_slot_swz).
__device__ __forceinline__ f16x8 kt_rows_swz(const _Float16* t, int r, int c) {
  return *reinterpret_cast<const f16x8*>(&t[c * (kQTile * 8) + row_slot_swz(r, c) * 8]);
}

// Asynchronous copy of one query tile: per array, the query-row tile is one contiguous block of DH / 16 KB
// (DH / 16 wave instructions of 1024 bytes, DH / 64 per wave of four).
template <bool SPLIT, int DH>
__device__ __forceinline__ void key_tile_dma(const KeyParams& p, KeyTiles<SPLIT, DH>& T, int buf, int b, int h,
                                             int q0, int w, int l) {
  constexpr int NR = KeyTiles<SPLIT, DH>::NR;
  const _Float16* srcr[6] = {p.q16, p.do16, p.u16, p.e16, p.u16lo, p.e16lo};
#pragma unroll
  for (int a = 0; a < NR; ++a) {
    const int pad = a < 4 ? p.Tq_pad : p.lo_pad;
    const int64_t tb = q_tile(b, h, q0 / kQTile, p.Hq, pad / kQTile, DH);
#pragma unroll
    for (int j = 0; j < DH / 64; ++j) {
      const int i = (DH / 64) * w + j;
      lds_dma16(srcr[a] + tb + i * 512 + l * 8, &T.r[buf][a][i * 512]);
    }
  }
}

// Row statistics of one query tile (lse in log2 units, alpha, Delta): thread tid < 96 fetches one value.
__device__ __forceinline__ float key_stat_load(const KeyParams& p, int b, int h, int q0, int tid) {
  const int which = tid >> 5, r = tid & 31, row = q0 + r;
  float val = 0.f;
  if (tid < 96 && row < p.Tq) {
    const int64_t so = (static_cast<int64_t>(b) * p.Hq + h) * p.Tq + row;
    if (which == 0) {
      val = p.lse[so] * kLog2e;
      if (!(val > -INFINITY && val < INFINITY)) val = 0.f;
    } else {
      val = which == 1 ? p.alpha[so] : p.delta[so];
    }
  }
  return val;
}

template <bool SPLIT, int DH>
__global__ __launch_bounds__(256) void k_bwd_keys_fast(KeyParams p) {
  constexpr int NS = DH / 16, NT = DH / 32;   // k-steps and accumulator tiles over d
  __shared__ KeyTiles<SPLIT, DH> T;
  constexpr int NB = KeyTiles<SPLIT, DH>::NB;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, ql = l & 31, hh = l >> 5;
  const int tro = tr_lane_offset(l);
  const int npairs = p.B * p.Hkv;
  int pair, kbk;
  {
    const int id = blockIdx.x;
    if ((npairs & 7) == 0) {
      const int ppx = npairs >> 3, slot = id >> 3;
      kbk = slot / ppx;  // causal: the first key blocks see the most rows
      pair = (id & 7) + 8 * (slot % ppx);
    } else {
      kbk = id / npairs;
      pair = id % npairs;
    }
  }
  const int b = pair / p.Hkv, g = pair % p.Hkv;
  const int off = p.Tk - p.Tq;
  const int jb = kbk * 128;            // block's first key
  const int jw = jb + 32 * w;          // wave's first key
  const int key = jw + ql;
  const bool key_ok = key < p.Tk;
  const uint32_t* MB = p.maxbits;
  const float sQ = range_scale(mx(MB, kMaxQ)), sK = range_scale(mx(MB, kMaxK));
  const float sV = range_scale(mx(MB, kMaxV)), sG = range_scale(mx(MB, kMaxDO));
  const float maxU = mx(MB, kMaxU), maxE = mx(MB, kMaxDKB), maxK = mx(MB, kMaxK);
  const float sU = range_scale(maxU), sE = range_scale(maxE);
  const float cS = p.scale * kLog2e / (sQ * sK);
  const float fT = 1.f / (sU * sK), fE = 1.f / (sE * sK), fG = 1.f / (sG * sV);

  // this wave's key rows as B operands (d permuted, as staged)
  f16x8 kB[NS], vB[NS];
  {
    const int kr = key_ok ? key : 0;
    const int64_t roff = kv_tile(b, g, kr / kKeyTile, p.Hkv, p.Tk_pad / kKeyTile, DH) + (kr % kKeyTile) * 8 +
                         hh * (kKeyTile * 8);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kB[s] = *reinterpret_cast<const f16x8*>(p.k16 + roff + s * (2 * kKeyTile * 8));
      vB[s] = *reinterpret_cast<const f16x8*>(p.v16 + roff + s * (2 * kKeyTile * 8));
    }
  }
  const KeyLaneScales ls = key_lane_scales(p, b, g, key, key_ok, sqrtf(xor32_sum(sumsq(kB))) / sK,
                                           sqrtf(xor32_sum(sumsq(vB))) / sV, sU, sE, sQ);
  const float C = ls.C, cV = ls.cV;
  const float c1 = C / sU, c2 = C / sE, c3 = p.scale * C / sQ;
  f32x16 accK[NT], accV[NT];
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
    accK[mt] = f32x16{};
    accV[mt] = f32x16{};
  }
  // query rows that see some key of the block: [i_lo, i_hi)
  const int jmax_b = min(jb + 128, p.key_hi) - 1;
  int i_lo = p.causal ? max(p.row_lo, jb - off) : p.row_lo;
  int i_hi = p.window > 0 ? min(p.row_hi, jmax_b - off + p.window) : p.row_hi;
  const int n_qt = i_hi > i_lo ? (i_hi - 1) / 32 - i_lo / 32 + 1 : 0;
  const int qt0 = i_lo / 32;
  const int total = n_qt * p.G;
  const int jw_last = min(jw + 31, p.Tk - 1);
  const int row_lo_c = p.row_lo, row_hi_c = min(p.row_hi, p.Tq);
  const bool nocausal = !p.causal, nowindow = p.window <= 0;
  if (total > 0) {
    key_tile_dma<SPLIT, DH>(p, T, 0, b, g * p.G, qt0 * 32, w, l);
    const float sv = key_stat_load(p, b, g * p.G, qt0 * 32, tid);
    if (tid < 96) T.stat[0][tid >> 5][tid & 31] = sv;
  }
  lds_dma_wait();
  __syncthreads();
  for (int it = 0; it < total; ++it) {
    const int buf = NB == 2 ? (it & 1) : 0;
    const int qt = qt0 + it % n_qt;
    const int q0 = qt * 32;
    // double-buffered: start the next tile's copy now
    float next_stat = 0.f;
    const bool pre = NB == 2 && it + 1 < total;
    if (pre) {
      const int nit = it + 1, nh = g * p.G + nit / n_qt, nq0 = (qt0 + nit % n_qt) * 32;
      key_tile_dma<SPLIT, DH>(p, T, buf ^ 1, b, nh, nq0, w, l);
      next_stat = key_stat_load(p, b, nh, nq0, tid);
    }
    // wave-uniform skip: no visible pair between these 32 rows and this wave's keys
    const bool any = jw < p.Tk && (!p.causal || jw <= q0 + 31 + off) &&
                     (p.window <= 0 || jw_last > q0 + off - p.window) && q0 + 31 >= p.row_lo && q0 < p.row_hi;
    if (any) {
      const bool full = jw + 32 <= p.Tk && (!p.causal || jw + 31 <= q0 + off) &&
                        (p.window <= 0 || jw > q0 + 31 + off - p.window) && q0 >= p.row_lo &&
                        q0 + 32 <= min(p.row_hi, p.Tq);
      f32x16 S = {}, Tt = {}, E = {}, Gt = {};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        S = mfma(kt_rows(T.r[buf][0], ql, 2 * s + hh), kB[s], S);
        Gt = mfma(kt_rows(T.r[buf][1], ql, 2 * s + hh), vB[s], Gt);
        Tt = mfma(kt_rows(T.r[buf][2], ql, 2 * s + hh), kB[s], Tt);
        E = mfma(kt_rows(T.r[buf][3], ql, 2 * s + hh), kB[s], E);
        if constexpr (SPLIT) {
          Tt = mfma(kt_rows(T.r[buf][4], ql, 2 * s + hh), kB[s], Tt);
          E = mfma(kt_rows(T.r[buf][5], ql, 2 * s + hh), kB[s], E);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        // queries 16t..16t+15 of the tile: registers 8t..8t+7 (rows 8j + 4hh + e, j = 2t, 2t+1)
        float wv[8], wk[8], wp[8], wd[8];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int j = 2 * t + jj;
          const int rr = 8 * j + 4 * hh;
          const float4 L2 = *reinterpret_cast<const float4*>(&T.stat[buf][0][rr]);
          const float4 AL = *reinterpret_cast<const float4*>(&T.stat[buf][1][rr]);
          const float4 DL = *reinterpret_cast<const float4*>(&T.stat[buf][2][rr]);
          const float l2[4] = {L2.x, L2.y, L2.z, L2.w}, al[4] = {AL.x, AL.y, AL.z, AL.w};
          const float dl[4] = {DL.x, DL.y, DL.z, DL.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * j + e, o = 4 * jj + e, i = q0 + rr + e;
            float sv = S[r];
            if (!full) {
              // branch-free visibility test (bitwise, no short-circuit)
              const bool vis = key_ok & (i >= row_lo_c) & (i < row_hi_c) & ((key <= i + off) | nocausal) &
                               ((key > i + off - p.window) | nowindow);
              sv = vis ? sv : -INFINITY;
            }
            const float pr = __builtin_amdgcn_exp2f(fmaf(sv, cS, -l2[e]));
            const float tt = fmaf(Tt[r], fT, 1.f - al[e]);
            const float gt = Gt[r] * fG;
            const float dp = fmaf(gt, tt, E[r] * fE);
            wv[o] = pr * tt * cV;
            wk[o] = pr * gt * c1;
            wp[o] = pr * c2;
            wd[o] = pr * (dp - dl[e]) * c3;
          }
        }
        f16x8 vh, vl, kh, kl, ph, pl, dh, dlo;
        to_operand(wv, 1.f, vh, SPLIT ? &vl : nullptr);
        to_operand(wk, 1.f, kh, SPLIT ? &kl : nullptr);
        to_operand(wp, 1.f, ph, SPLIT ? &pl : nullptr);
        to_operand(wd, 1.f, dh, SPLIT ? &dlo : nullptr);
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
          const f16x8 ag = tr_cols(T.r[buf][1], tro, mt, t), aq = tr_cols(T.r[buf][0], tro, mt, t);
          const f16x8 au = tr_cols(T.r[buf][2], tro, mt, t), ae = tr_cols(T.r[buf][3], tro, mt, t);
          accV[mt] = mfma(ag, vh, accV[mt]);
          accK[mt] = mfma(au, kh, accK[mt]);
          accK[mt] = mfma(ae, ph, accK[mt]);
          accK[mt] = mfma(aq, dh, accK[mt]);
          if constexpr (SPLIT) {
            const f16x8 aul = tr_cols(T.r[buf][4], tro, mt, t), ael = tr_cols(T.r[buf][5], tro, mt, t);
            accV[mt] = mfma(ag, vl, accV[mt]);
            accK[mt] = mfma(au, kl, accK[mt]);
            accK[mt] = mfma(aul, kh, accK[mt]);
            accK[mt] = mfma(ae, pl, accK[mt]);
            accK[mt] = mfma(ael, ph, accK[mt]);
            accK[mt] = mfma(aq, dlo, accK[mt]);
          }
        }
      }
    }
    if (pre && tid < 96) T.stat[buf ^ 1][tid >> 5][tid & 31] = next_stat;
    if (NB == 1 && it + 1 < total) {
      // single buffer: wait until every wave is done with the tile, then copy the next one
      __syncthreads();
      const int nit = it + 1, nh = g * p.G + nit / n_qt, nq0 = (qt0 + nit % n_qt) * 32;
      key_tile_dma<SPLIT, DH>(p, T, 0, b, nh, nq0, w, l);
      const float sv = key_stat_load(p, b, nh, nq0, tid);
      if (tid < 96) T.stat[0][tid >> 5][tid & 31] = sv;
    }
    lds_dma_wait();
    __syncthreads();
  }
  if (key_ok) {
    const float fk = 1.f / C, fv = 1.f / (sG * cV);
    float* dkr = p.dk + ((static_cast<int64_t>(b) * p.out_keys + key) * p.Hkv + g) * p.D;
    float* dvr = p.dv + ((static_cast<int64_t>(b) * p.out_keys + key) * p.Hkv + g) * p.D;
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * mt + 8 * j + 4 * hh, r = 4 * j;
        float4 kv = {accK[mt][r] * fk, accK[mt][r + 1] * fk, accK[mt][r + 2] * fk, accK[mt][r + 3] * fk};
        float4 vv = {accV[mt][r] * fv, accV[mt][r + 1] * fv, accV[mt][r + 2] * fv, accV[mt][r + 3] * fv};
        if (p.accumulate) {
          const float4 k0 = *reinterpret_cast<const float4*>(dkr + d);
          const float4 v0 = *reinterpret_cast<const float4*>(dvr + d);
          kv = float4{kv.x + k0.x, kv.y + k0.y, kv.z + k0.z, kv.w + k0.w};
          vv = float4{vv.x + v0.x, vv.y + v0.y, vv.z + v0.z, vv.w + v0.w};
        }
        *reinterpret_cast<float4*>(dkr + d) = kv;
        *reinterpret_cast<float4*>(dvr + d) = vv;
      }
  }
}

// ------------------------------------------------------------------------------------------
// key-major kernel with role-split, pipelined waves (rows >= split) and the dq kernel
// ------------------------------------------------------------------------------------------
//
// 8 waves (2 per SIMD) own 128 keys: wave w has keys jb + 32 (w & 3) + [0, 32).  Waves 0-3 ("V")
// compute S, T, E and G of their keys against a query tile and every weight of the tile (p tt, p G,
// p, ds); they hand the four fp16 operands to waves 4-7 ("K") through LDS.  The K waves accumulate
// dv = (p tt)^T g and dk = (p G)^T u + p^T dkbar + scale ds^T q and store the ds tile for the dq
// kernel, one query tile behind the V waves.  A tile has two phases: the V waves' MFMAs while the K
// waves take the previous tile's operands from the exchange, then (after a barrier) the V waves'
// vector work beside the K waves' MFMAs.  The two roles issue about as many MFMAs each, and every
// SIMD holds one wave of each role, so one wave's vector work runs beside the other's matrix work.  A query tile is kept in LDS in row layout only
// ([16 chunks][32 rows][8], 32 KB for q, dO, u, e); the column-layout operands of the products over
// queries are read from it with the gfx950 transpose load ds_read_b64_tr_b16 (two per operand).  Three
// tile buffers (tile i - 1 for the K waves, tile i, and the copy of tile i + 1 in flight) and the
// exchange fit in LDS.
//
// The K waves store the tile of ds (as the fp16 operand C scale ds / sQ) in query-major order for
// the dq kernel.  The transpose costs two MFMAs: the ds operand (keys on lanes) times a permutation
// matrix gives an accumulator with queries on lanes.

// s_getreg operand for the SIMD_ID field (bits 5:4) of the HW_ID hardware register.
constexpr int kHwIdSimd = (1 << 11) | (4 << 6) | 4;

// Tensor scales shared by the key-major kernel and the dq kernel (the products' scales are per key,
// key_lane_scales).
struct KeyScales {
  float sQ, sK, sV, sG, sU, sE, cS, fT, fE, fG;
};

__device__ __forceinline__ KeyScales key_scales(const uint32_t* MB, float scale) {
  KeyScales k;
  k.sQ = range_scale(mx(MB, kMaxQ));
  k.sK = range_scale(mx(MB, kMaxK));
  k.sV = range_scale(mx(MB, kMaxV));
  k.sG = range_scale(mx(MB, kMaxDO));
  k.sU = range_scale(mx(MB, kMaxU));
  k.sE = range_scale(mx(MB, kMaxDKB));
  k.cS = scale * kLog2e / (k.sQ * k.sK);
  k.fT = 1.f / (k.sU * k.sK);
  k.fE = 1.f / (k.sE * k.sK);
  k.fG = 1.f / (k.sG * k.sV);
  return k;
}

// Whether keys [jw, jw + 32) and query rows [q0, q0 + 32) hold a visible pair with a row in [row_lo, row_hi).
__device__ __forceinline__ bool tile_pair_any(int jw, int q0, int Tk, int off, int causal, int window, int row_lo,
                                              int row_hi) {
  const int jw_last = min(jw + 31, Tk - 1);
  return jw < Tk && (!causal || jw <= q0 + 31 + off) && (window <= 0 || jw_last > q0 + off - window) &&
         q0 + 31 >= row_lo && q0 < row_hi;
}

template <int DH>
struct __align__(16) KeyTiles3 {
  _Float16 r[3][4][32 * DH];   // q, dO, u, e query-row tiles, three buffers
  f16x8 x[4][4][2][64];        // exchange: per key group p G c1, p c2, ds c3, p tt cV
  float stat[3][3][32];        // lse (log2 units), 1 - alpha, Delta of the tile's rows
  float ksc[4][2][32];         // per key group: its C (entry 0) and each key's cV (set by the V waves)
};
static_assert(sizeof(KeyTiles3<kD>) <= 160 * 1024, "LDS");

// One query tile into LDS buffer `buf`: 4 arrays of DH / 16 KB (consecutive in the workspace), half an
// array per wave (DH / 32 instructions), and the tile's 96 row statistics (wave 0, lanes 0-23).
// The rows of each chunk land swizzled (row_slot_swz): lane l of an instruction fills row slot l % 32
// of chunk 2 i + l / 32 and so fetches the row that belongs there.
template <int DH>
__device__ __forceinline__ void key_tile_dma3(const KeyParams& p, KeyTiles3<DH>& T, int buf, int b, int h, int q0,
                                              int w, int l) {
  const int64_t tb = q_tile(b, h, q0 / kQTile, p.Hq, p.Tq_pad / kQTile, DH);
  const int a = w >> 1;
  const _Float16* src = p.q16 + a * p.qstride + tb;   // q, dO, u, e rows
#pragma unroll
  for (int j = 0; j < DH / 32; ++j) {
    const int i = (DH / 32) * (w & 1) + j, ch = 2 * i + (l >> 5);
    lds_dma16(src + ch * 256 + row_slot_swz(l & 31, ch) * 8, &T.r[buf][a][i * 512]);
  }
  if (w == 0 && l < 24) {
    const float* st = p.rstat + ((static_cast<int64_t>(b) * p.Hq + h) * (p.Tq_pad / 32) + q0 / 32) * 96;
    lds_dma16(st + 4 * l, &T.stat[buf][0][0]);
  }
}

template <int DH>
__global__ __launch_bounds__(512) void k_bwd_keys_pipe(KeyParams p) {
  constexpr int NS = DH / 16, NT = DH / 32;   // k-steps and accumulator tiles over d
  __shared__ KeyTiles3<DH> T;
  __shared__ int wave_simd[8];
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, ql = l & 31, hh = l >> 5;
  // Roles follow the SIMDs: the two waves a SIMD holds become the V and the K wave of one key group,
  // so that every SIMD runs one wave's vector work beside the other's MFMAs.  (The dispatcher need
  // not place waves w and w + 4 together; at 2 waves per SIMD each SIMD holds exactly two.)
  const int simd = __builtin_amdgcn_s_getreg(kHwIdSimd);
  if (l == 0) wave_simd[w] = simd;
  __syncthreads();
  int below = 0, counts = 0;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int sv = __builtin_amdgcn_readfirstlane(wave_simd[v]);
    below += (sv == simd) & (v < w);
    counts += 1 << (8 * (sv & 3));
  }
  const bool paired = counts == 0x02020202;
  const bool is_v = paired ? below == 0 : w < 4;
  const int grp = paired ? simd : (w & 3);
  const int npairs = p.B * p.Hkv;
  int pair, kbk;
  {
    const int id = blockIdx.x;
    if ((npairs & 7) == 0) {
      const int ppx = npairs >> 3, slot = id >> 3;
      kbk = slot / ppx;  // causal: the first key blocks see the most rows
      pair = (id & 7) + 8 * (slot % ppx);
    } else {
      kbk = id / npairs;
      pair = id % npairs;
    }
  }
  const int b = pair / p.Hkv, g = pair % p.Hkv;
  const int off = p.Tk - p.Tq;
  const int jb = kbk * 128;
  const int jw = jb + 32 * grp;
  const int key = jw + ql;
  const bool key_ok = key < p.Tk;
  const KeyScales ks = key_scales(p.maxbits, p.scale);

  // query rows that see some key of the block: [i_lo, i_hi), visited for each head of the group
  const int jmax_b = min(jb + 128, p.key_hi) - 1;
  const int i_lo = p.causal ? max(p.row_lo, jb - off) : p.row_lo;
  const int i_hi = p.window > 0 ? min(p.row_hi, jmax_b - off + p.window) : p.row_hi;
  const int n_qt = i_hi > i_lo ? (i_hi - 1) / 32 - i_lo / 32 + 1 : 0;
  const int qt0 = i_lo / 32;
  const int total = n_qt * p.G;
  const int row_lo_c = p.row_lo, row_hi_c = min(p.row_hi, p.Tq);
  const bool nocausal = !p.causal, nowindow = p.window <= 0;
  // Query tiles are visited from the last one down, the heads of the group interleaved: the blocks
  // of one (batch, kv head) running together then read the same tile at about the same time, so it
  // comes from L2 instead of once per block from memory.
  const int gsh = p.G == 8 ? 3 : p.G == 4 ? 2 : p.G == 2 ? 1 : 0;   // the fast path has G in {1, 2, 4, 8}
  auto tile_head = [&](int it) { return g * p.G + (it & (p.G - 1)); };
  auto tile_row = [&](int it) { return (qt0 + n_qt - 1 - (it >> gsh)) * 32; };
  auto tile_any = [&](int it) {
    return tile_pair_any(jw, tile_row(it), p.Tk, off, p.causal, p.window, p.row_lo, p.row_hi);
  };
  if (total > 0) key_tile_dma3(p, T, 0, b, tile_head(0), tile_row(0), w, l);
  lds_dma_wait();
  __syncthreads();

  const int kr = key_ok ? key : 0;
  const int64_t roff = kv_tile(b, g, kr / kKeyTile, p.Hkv, p.Tk_pad / kKeyTile, DH) + (kr % kKeyTile) * 8 +
                       hh * (kKeyTile * 8);
  const int2 tro = tr_lane_offsets_swz(l);

  if (is_v) {
    // ---------------- V waves: S, T, E, G and the weights of tile it ----------------
    f16x8 kB[NS], vB[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kB[s] = *reinterpret_cast<const f16x8*>(p.k16 + roff + s * (2 * kKeyTile * 8));
      vB[s] = *reinterpret_cast<const f16x8*>(p.v16 + roff + s * (2 * kKeyTile * 8));
    }
    // The dk products of the group's 32 keys share one scale, the smallest C among its keys that some
    // row sees (the stored ds tiles then hold one scale per group); dv takes each key's own cV.
    const KeyLaneScales kls = key_lane_scales(p, b, g, key, key_ok, sqrtf(xor32_sum(sumsq(kB))) / ks.sK,
                                              sqrtf(xor32_sum(sumsq(vB))) / ks.sV, ks.sU, ks.sE, ks.sQ);
    float cgrp = kls.seen ? kls.C : INFINITY;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cgrp = fminf(cgrp, __shfl_xor(cgrp, o, 64));
    if (cgrp == INFINITY) cgrp = 1.f;   // no row sees any key of the group: nothing is accumulated
    cgrp = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(cgrp)));   // (the builtin takes an int)
    const float c1 = cgrp / ks.sU, c2 = cgrp / ks.sE, c3 = p.scale * cgrp / ks.sQ, cV = kls.cV;
    if (hh == 0) T.ksc[grp][1][ql] = cV;
    if (l == 0) T.ksc[grp][0][0] = cgrp;
    if (l == 0 && jw < p.Tk_pad) p.dsscale[(static_cast<int64_t>(b) * p.Hkv + g) * (p.Tk_pad / 32) + jw / 32] = cgrp;
    vm_wait_all();
    for (int it = 0; it <= total; ++it) {
      const int buf = it % 3;
      if (it + 1 < total) key_tile_dma3(p, T, (it + 1) % 3, b, tile_head(it + 1), tile_row(it + 1), w, l);
      const bool any = it < total && tile_any(it);
      f32x16 S = {}, Tt = {}, E = {}, Gt = {};
      float4 st[3][4];   // row statistics of the tile: lse, 1 - alpha, Delta of rows 8 j + 4 hh + [0, 4)
      if (any) {
        // The row operands (q, dO, u, e) of chunk s + 2 are read while the MFMAs of chunk s run; the
        // scheduling barriers keep the compiler from moving the reads next to their MFMAs.
        f16x8 a[3][4];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int o = 0; o < 4; ++o) a[s][o] = kt_rows_swz(T.r[buf][o], ql, 2 * s + hh);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if (s + 2 < NS) {
#pragma unroll
            for (int o = 0; o < 4; ++o) a[(s + 2) % 3][o] = kt_rows_swz(T.r[buf][o], ql, 2 * (s + 2) + hh);
          }
          if (s == NS - 2) {   // the statistics are read while the last MFMAs run
#pragma unroll
            for (int k = 0; k < 3; ++k)
#pragma unroll
              for (int j = 0; j < 4; ++j) st[k][j] = *reinterpret_cast<const float4*>(&T.stat[buf][k][8 * j + 4 * hh]);
          }
          __builtin_amdgcn_sched_barrier(0);
          S = mfma(a[s % 3][0], kB[s], S);
          Gt = mfma(a[s % 3][1], vB[s], Gt);
          Tt = mfma(a[s % 3][2], kB[s], Tt);
          E = mfma(a[s % 3][3], kB[s], E);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // the K waves have taken the previous tile's operands from the exchange
      lds_barrier();
      if (any) {
        const int q0 = tile_row(it);
        const bool full = jw + 32 <= p.Tk && (!p.causal || jw + 31 <= q0 + off) &&
                          (p.window <= 0 || jw > q0 + 31 + off - p.window) && q0 >= p.row_lo &&
                          q0 + 32 <= row_hi_c;
        if (!full) {   // tiles on the causal / window / row-range edge only
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool vis = key_ok & (i >= row_lo_c) & (i < row_hi_c) & ((key <= i + off) | nocausal) &
                             ((key > i + off - p.window) | nowindow);
            if (!vis) S[r] = -INFINITY;
          }
        }
        // Stage by stage over the 16 rows of the lane, so that neighbouring instructions are
        // independent: p, tt = 1 - alpha + T, g = G, b = g tt + dkbar.k - Delta.
        float pr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) pr[r] = fmaf(S[r], ks.cS, -st[0][r >> 2][r & 3]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(pr[r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          Tt[r] = fmaf(Tt[r], ks.fT, st[1][r >> 2][r & 3]);
          Gt[r] = Gt[r] * ks.fG;
          E[r] = fmaf(E[r], ks.fE, -st[2][r >> 2][r & 3]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) E[r] = fmaf(Gt[r], Tt[r], E[r]);
        __builtin_amdgcn_sched_barrier(0);
        // operands p G c1, p c2, p b c3 (= ds c3) and p tt cV
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float w[8];
          f16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = pr[8 * t + e] * Gt[8 * t + e];
          to_operand(w, c1, o, nullptr);
          T.x[grp][0][t][l] = o;
          to_operand(&pr[8 * t], c2, o, nullptr);
          T.x[grp][1][t][l] = o;
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = pr[8 * t + e] * E[8 * t + e];
          to_operand(w, c3, o, nullptr);
          T.x[grp][2][t][l] = o;
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = pr[8 * t + e] * Tt[8 * t + e];
          to_operand(w, cV, o, nullptr);
          T.x[grp][3][t][l] = o;
        }
      }
      lds_dma_wait();
      __syncthreads();
    }
  } else {
    // ---------------- K waves: dv and dk products and the ds tile of tile it - 1 ----------------
    // permutation operands: B[k][n] = 1 iff n = 16 t + perm16(k), k = 8 hh + e
    f16x8 pi[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pi[t][e] = static_cast<_Float16>(ql == 16 * t + perm16(8 * hh + e) ? 1.f : 0.f);
    f32x16 accK[NT], accV[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) accK[mt] = accV[mt] = f32x16{};
    // A ds tile is stored one iteration after it is formed, at the start of the next one: the wait that
    // ends an iteration (for the next tile's copy) then finds the stores long done instead of waiting for them.
    f16x8 ds_hold[2];
    int64_t ds_at = -1;   // element offset of the held tile in ds (-1: none)
    auto store_ds = [&]() {
      if (ds_at >= 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t) *reinterpret_cast<f16x8*>(p.ds + ds_at + t * 512) = ds_hold[t];
        ds_at = -1;
      }
    };
    for (int it = 0; it <= total; ++it) {
      const int pbuf = (it + 2) % 3;
      store_ds();
      if (it + 1 < total) key_tile_dma3(p, T, (it + 1) % 3, b, tile_head(it + 1), tile_row(it + 1), w, l);
      const bool has = it >= 1 && tile_any(it - 1);
      // operands of tile it - 1, taken before the V waves overwrite the exchange with tile it
      f16x8 xk[2], xp[2], xd[2], xv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        xk[t] = T.x[grp][0][t][l];
        xp[t] = T.x[grp][1][t][l];
        xd[t] = T.x[grp][2][t][l];
        xv[t] = T.x[grp][3][t][l];
      }
      lds_barrier();
      if (has) {
        f32x16 DT = {};
        // step n = (t, mt) = (n / NT, n % NT) multiplies the column operands (u, e, q, dO) of d tile mt
        // and query half t; the operands of step n + 2 are read while step n runs
        f16x8 c[3][4];
        auto load_cols = [&](int n, f16x8(&dst)[4]) {
          const int t = n / NT, mt = n % NT;
          dst[0] = tr_cols_swz(T.r[pbuf][2], tro, mt, t);
          dst[1] = tr_cols_swz(T.r[pbuf][3], tro, mt, t);
          dst[2] = tr_cols_swz(T.r[pbuf][0], tro, mt, t);
          dst[3] = tr_cols_swz(T.r[pbuf][1], tro, mt, t);
        };
        load_cols(0, c[0]);
        load_cols(1, c[1]);
#pragma unroll
        for (int n = 0; n < 2 * NT; ++n) {
          const int t = n / NT, mt = n % NT;
          if (n + 2 < 2 * NT) load_cols(n + 2, c[(n + 2) % 3]);
          __builtin_amdgcn_sched_barrier(0);
          accK[mt] = mfma(c[n % 3][0], xk[t], accK[mt]);
          accV[mt] = mfma(c[n % 3][3], xv[t], accV[mt]);
          accK[mt] = mfma(c[n % 3][1], xp[t], accK[mt]);
          accK[mt] = mfma(c[n % 3][2], xd[t], accK[mt]);
          if (mt == NT - 1) DT = mfma(xd[t], pi[t], DT);
          __builtin_amdgcn_sched_barrier(0);
        }
        // DT: lane = query row of the tile, register r = key 8 (r / 4) + 4 hh + r % 4 of the wave's 32
        const int64_t tile = ((static_cast<int64_t>(b) * p.Hq + tile_head(it - 1)) * (p.Tq_pad / 32) +
                              tile_row(it - 1) / 32) * (p.Tk_pad / 32) + jw / 32;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) ds_hold[t][e] = static_cast<_Float16>(DT[8 * t + e]);
        ds_at = tile * 1024 + l * 8;
      }
      lds_dma_wait();
      __syncthreads();
    }
    store_ds();
    if (key_ok) {
      const float fv = 1.f / (ks.sG * T.ksc[grp][1][ql]);
      float* dvr = p.dv + ((static_cast<int64_t>(b) * p.Tk + key) * p.Hkv + g) * p.D;
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * mt + 8 * j + 4 * hh, r = 4 * j;
          float4 vv = {accV[mt][r] * fv, accV[mt][r + 1] * fv, accV[mt][r + 2] * fv, accV[mt][r + 3] * fv};
          if (p.accumulate) {
            const float4 v0 = *reinterpret_cast<const float4*>(dvr + d);
            vv = float4{vv.x + v0.x, vv.y + v0.y, vv.z + v0.z, vv.w + v0.w};
          }
          *reinterpret_cast<float4*>(dvr + d) = vv;
        }
      const float fk = 1.f / T.ksc[grp][0][0];
      float* dkr = p.dk + ((static_cast<int64_t>(b) * p.Tk + key) * p.Hkv + g) * p.D;
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * mt + 8 * j + 4 * hh, r = 4 * j;
          float4 kv = {accK[mt][r] * fk, accK[mt][r + 1] * fk, accK[mt][r + 2] * fk, accK[mt][r + 3] * fk};
          if (p.accumulate) {
            const float4 k0 = *reinterpret_cast<const float4*>(dkr + d);
            kv = float4{kv.x + k0.x, kv.y + k0.y, kv.z + k0.z, kv.w + k0.w};
          }
          *reinterpret_cast<float4*>(dkr + d) = kv;
        }
    }
  }
}

// dq for rows >= split: dq = P du (already in dq) + scale sum_j ds_ij k_j, with ds from the
// key-major kernel.  One 512-thread block (8 waves) owns a (batch, kv head) and 256 / G rows of each
// query head of the group, like the forward; each wave owns a 32-row tile.  The K^T tiles are shared
// by the block through LDS (double-buffered, copied by DMA); each wave streams its stored ds tiles
// (A operand ordering, keys permuted within 16) from memory one key tile ahead.
struct DqParams {
  const _Float16 *ds, *k16t;
  const float* dsscale;   // per 32-key group: the scale C of its stored ds tiles
  const uint32_t* maxbits;
  float* dq;
  int B, Tq, Tk, Tk_pad, Tq_pad, Hq, Hkv, G, causal, window, row_lo, row_hi, row_begin, rows_per_block, n_rb;
  int D;               // head dim of dq rows
  float scale;
};

template <int DH>
struct __align__(16) DqTiles {
  _Float16 kt[2][kKeyTile * DH];
};

template <int DH>
__global__ __launch_bounds__(512) void k_bwd_dq(DqParams p) {
  constexpr int NT = DH / 32;   // accumulator tiles over d
  __shared__ DqTiles<DH> T;
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
  const int wph = 8 / p.G;
  const int h = g * p.G + w / wph;
  const int r0 = p.row_begin + rb * p.rows_per_block;
  const int q0 = r0 + (w % wph) * 32;
  const bool wave_ok = q0 < p.row_hi;
  const int off = p.Tk - p.Tq;
  const KeyScales ks = key_scales(p.maxbits, p.scale);
  // keys the block's rows can see: tiles [t_beg, t_end)
  const int rlast = min(r0 + p.rows_per_block, p.row_hi) - 1;
  const int kend = p.causal ? min(p.Tk, rlast + off + 1) : p.Tk;
  const int kbeg = p.window > 0 ? max(0, r0 + off - p.window + 1) : 0;
  const int t_beg = kbeg / kKeyTile;
  const int t_end = kend > kbeg ? (kend + kKeyTile - 1) / kKeyTile : t_beg;
  const int64_t tile0 = ((static_cast<int64_t>(b) * p.Hq + h) * (p.Tq_pad / 32) + q0 / 32) * (p.Tk_pad / 32);
  // a 32-key block holds a stored ds tile iff the key-major kernel saw a visible pair there
  auto vis = [&](int kb32) {
    return wave_ok && tile_pair_any(32 * kb32, q0, p.Tk, off, p.causal, p.window, p.row_lo, p.row_hi);
  };
  // Loads are unconditional (from an in-bounds tile; blocks without a stored tile are skipped at the
  // MFMAs), so that no value joins a branch and the compiler does not wait for a prefetch early.
  const int64_t tile_rd = wave_ok ? tile0 : 0;
  auto load_ds = [&](int kt, f16x8 (&d)[4]) {
#pragma unroll
    for (int kbh = 0; kbh < 2; ++kbh) {
      const _Float16* src = p.ds + (tile_rd + 2 * kt + kbh) * 1024 + l * 8;
      d[2 * kbh] = *reinterpret_cast<const f16x8*>(src);
      d[2 * kbh + 1] = *reinterpret_cast<const f16x8*>(src + 512);
    }
  };
  auto dma_k = [&](int kt, int buf) {
    const int64_t tb = kv_tile(b, g, kt, p.Hkv, p.Tk_pad / kKeyTile, DH);
#pragma unroll
    for (int j = 0; j < DH / 64; ++j) {
      const int i = (DH / 64) * w + j;
      lds_dma16(p.k16t + tb + i * 512 + l * 8, &T.kt[buf][i * 512]);
    }
  };
  // Each 32-key group stored its ds tiles at its own scale C (dsscale).  The wave's rows take the
  // smallest C among the groups they see, and every other group's operand is brought to it by an exact
  // power of two <= 1 before its products.
  const float* gsc = p.dsscale + (static_cast<int64_t>(b) * p.Hkv + g) * (p.Tk_pad / 32);
  float cdq = INFINITY;
  for (int kb32 = 2 * t_beg + l; kb32 < 2 * t_end; kb32 += 64)
    if (vis(kb32)) cdq = fminf(cdq, gsc[kb32]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cdq = fminf(cdq, __shfl_xor(cdq, o, 64));
  if (cdq == INFINITY) cdq = 1.f;   // no stored tile
  float fcur[2] = {1.f, 1.f}, fnxt[2] = {1.f, 1.f};
  auto load_f = [&](int kt, float (&f)[2]) {
#pragma unroll
    for (int kbh = 0; kbh < 2; ++kbh) f[kbh] = cdq / gsc[2 * kt + kbh];
  };
  f32x16 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x16{};
  f16x8 dcur[4], dnxt[4];
  if (t_beg < t_end) {
    dma_k(t_beg, 0);
    load_ds(t_beg, dcur);
    load_f(t_beg, fcur);
  }
  lds_dma_wait();
  __syncthreads();
  for (int kt = t_beg; kt < t_end; ++kt) {
    const int buf = (kt - t_beg) & 1;
    if (kt + 1 < t_end) {
      dma_k(kt + 1, buf ^ 1);
      load_ds(kt + 1, dnxt);
      load_f(kt + 1, fnxt);
    }
#pragma unroll
    for (int kbh = 0; kbh < 2; ++kbh) {
      if (vis(2 * kt + kbh)) {
        const _Float16 f = static_cast<_Float16>(fcur[kbh]);
        const f16x8 d0 = dcur[2 * kbh] * f, d1 = dcur[2 * kbh + 1] * f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[nt] = mfma(lds_cols<DH>(T.kt[buf], 32 * nt + ql, 4 * kbh + hh), d0, acc[nt]);
          acc[nt] = mfma(lds_cols<DH>(T.kt[buf], 32 * nt + ql, 4 * kbh + 2 + hh), d1, acc[nt]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) dcur[i] = dnxt[i];
    fcur[0] = fnxt[0];
    fcur[1] = fnxt[1];
    lds_dma_wait();
    __syncthreads();
  }
  const int row = q0 + ql;
  if (row >= p.row_lo && row < p.row_hi && row < p.Tq) {
    const float fq = ks.sQ / (cdq * ks.sK);
    float* dqr = p.dq + ((static_cast<int64_t>(b) * p.Tq + row) * p.Hq + h) * p.D;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 32 * nt + 8 * j + 4 * hh, r = 4 * j;
        const float4 q = *reinterpret_cast<const float4*>(dqr + d);
        *reinterpret_cast<float4*>(dqr + d) = float4{q.x + acc[nt][r] * fq, q.y + acc[nt][r + 1] * fq,
                                                     q.z + acc[nt][r + 2] * fq, q.w + acc[nt][r + 3] * fq};
      }
  }
}

// Zeroes n floats (n a multiple of 4; 16-byte aligned).
__global__ __launch_bounds__(256) void k_zero4(float* x, int64_t n4) {
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n4; i += 256LL * gridDim.x)
    reinterpret_cast<float4*>(x)[i] = float4{0.f, 0.f, 0.f, 0.f};
}

// Zeroes two arrays in one launch (n4 float4 each; 16-byte aligned).
__global__ __launch_bounds__(256) void k_zero4x2(float* x, int64_t n4, float* y, int64_t m4) {
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n4 + m4; i += 256LL * gridDim.x) {
    float4* dst = i < n4 ? reinterpret_cast<float4*>(x) + i : reinterpret_cast<float4*>(y) + (i - n4);
    *dst = float4{0.f, 0.f, 0.f, 0.f};
  }
}

// dk[b, key] += dklo[b, key] and the same for dv, for the first nkeys keys of every batch entry (n4: float4
// per key; the buffers hold lo_keys and Tk keys per batch entry; 16-byte aligned).
__global__ __launch_bounds__(256) void k_add_lo(float* dk, float* dv, const float* dklo, const float* dvlo, int B,
                                                int64_t nkeys, int64_t lo_keys, int64_t Tk, int64_t n4) {
  const int64_t per_b = nkeys * n4;
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < 2 * B * per_b; i += 256LL * gridDim.x) {
    const int64_t t = i / (B * per_b), r = i % (B * per_b), b = r / per_b, k = r % per_b;
    float4* dst = reinterpret_cast<float4*>(t == 0 ? dk : dv) + b * Tk * n4 + k;
    const float4 a = reinterpret_cast<const float4*>(t == 0 ? dklo : dvlo)[b * lo_keys * n4 + k];
    const float4 c = *dst;
    *dst = float4{c.x + a.x, c.y + a.y, c.z + a.z, c.w + a.w};
  }
}

// ------------------------------------------------------------------------------------------
// dP = sum over batch and rows of x du^T: partial sums per row chunk, then a fixed-order sum
// ------------------------------------------------------------------------------------------

constexpr int kPChunk = 256;  // rows per partial

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// x = hi + lo, hi = bf16(x), lo = bf16(x - hi): about 16 significant bits; with fp32 accumulation
// hi.hi + hi.lo + lo.hi is a product good to about 2^-16 relative.
__device__ __forceinline__ void split_bf16(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 t = static_cast<__bf16>(x[e]);
    hi[e] = t;
    lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(t));
  }
}

// block (head, chunk): 4 waves; wave w owns rows 32 w .. 32 w + 31 of the 128 x 128 result as four
// 32 x 32 tiles, each summed over 16 input rows per step by three bf16 MFMAs (hi.hi, hi.lo, lo.hi;
// v_mfma_f32_32x32x16_bf16, fp32 accumulation).  Lane (ql, hh) takes rows 8 hh .. 8 hh + 7 of a
// step: x at column 32 w + ql, du at columns 4 ql .. 4 ql + 3 (one float4 a row), so that tile bt
// holds the result columns 4 j + bt (j = 0..31) and a lane stores four tiles' values as one float4.
__global__ __launch_bounds__(256) void k_dp_partial(const float* x32, const float* du32, float* part, int R, int Hq) {
  // the heads of one row chunk are consecutive blocks, so they read the same rows at about the same time
  const int h = blockIdx.x % Hq, c = blockIdx.x / Hq;
  const int w = wave_id(), l = threadIdx.x & 63, ql = l & 31, hh = l >> 5;
  f32x16 acc[4];
#pragma unroll
  for (int bt = 0; bt < 4; ++bt) acc[bt] = f32x16{};
  const int r_beg = c * kPChunk, r_end = min(R, r_beg + kPChunk);
  const int64_t rs = static_cast<int64_t>(Hq) * kD;
  const float* xp = x32 + h * kD + 32 * w + ql;
  const float* dp = du32 + h * kD + 4 * ql;
  // The loads of step i + 1 are in flight while step i is converted and multiplied.  Whole 32-row
  // pairs of steps need no bounds checks; in a last partial pair, rows past the chunk read row
  // r_beg and count as zero.
  float xa[2][8];
  float4 db[2][8];
  auto load_step = [&](int r0, int sb, bool check) {
    const float* xr = xp + static_cast<int64_t>(r0 + 8 * hh) * rs;
    const float* dr = dp + static_cast<int64_t>(r0 + 8 * hh) * rs;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (!check) {
        xa[sb][e] = xr[e * rs];
        db[sb][e] = *reinterpret_cast<const float4*>(dr + e * rs);
      } else {
        const int r = r0 + 8 * hh + e;
        const bool ok = r < r_end;
        const int64_t o = static_cast<int64_t>(ok ? r : r_beg) * rs;
        const float xv = xp[o];
        const float4 dv = *reinterpret_cast<const float4*>(dp + o);
        xa[sb][e] = ok ? xv : 0.f;
        db[sb][e] = ok ? dv : float4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto mul_step = [&](int sb) {
    bf16x8 xh, xl;
    split_bf16(xa[sb], xh, xl);
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = bt == 0 ? db[sb][e].x : bt == 1 ? db[sb][e].y : bt == 2 ? db[sb][e].z : db[sb][e].w;
      bf16x8 dh, dl;
      split_bf16(v, dh, dl);
      acc[bt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, dh, acc[bt], 0, 0, 0);
      acc[bt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, dl, acc[bt], 0, 0, 0);
      acc[bt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl, dh, acc[bt], 0, 0, 0);
    }
  };
  const int r_full = r_beg + (r_end - r_beg) / 32 * 32;
  if (r_beg < r_full) load_step(r_beg, 0, false);
  for (int r0 = r_beg; r0 < r_full; r0 += 32) {
    load_step(r0 + 16, 1, false);
    __builtin_amdgcn_sched_barrier(0);   // keep the loads ahead of the work on the other buffer
    mul_step(0);
    __builtin_amdgcn_sched_barrier(0);
    load_step(r0 + 32 < r_full ? r0 + 32 : r0, 0, false);   // (the last pair re-reads rows in range)
    __builtin_amdgcn_sched_barrier(0);
    mul_step(1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (r_full < r_end) {
    load_step(r_full, 0, true);
    load_step(r_full + 16, 1, true);
    mul_step(0);
    mul_step(1);
  }
  // register r of tile bt: result row 32 w + 8 (r / 4) + 4 hh + r % 4, column 4 ql + bt
  float* dst = part + (static_cast<int64_t>(c) * Hq + h) * kD * kD + 4 * ql;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    *reinterpret_cast<float4*>(dst + (32 * w + 8 * (r >> 2) + 4 * hh + (r & 3)) * kD) =
        float4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
}

// The same partial sums for head dim 64: wave w owns the 32 x 32 tile of result rows 32 (w % 2) and columns
// 32 (w / 2); lane (ql, hh) takes rows 8 hh .. 8 hh + 7 of a 16-row step, x at the tile's column ql of x and
// du at its column ql of du.
__global__ __launch_bounds__(256) void k_dp_partial64(const float* x32, const float* du32, float* part, int R,
                                                      int Hq) {
  constexpr int DH = 64;
  const int h = blockIdx.x % Hq, c = blockIdx.x / Hq;
  const int w = wave_id(), l = threadIdx.x & 63, ql = l & 31, hh = l >> 5;
  const int ra = 32 * (w & 1), cb = 32 * (w >> 1);
  f32x16 acc = f32x16{};
  const int r_beg = c * kPChunk, r_end = min(R, r_beg + kPChunk);
  const int64_t rs = static_cast<int64_t>(Hq) * DH;
  const float* xp = x32 + h * DH + ra + ql;
  const float* dp = du32 + h * DH + cb + ql;
  for (int r0 = r_beg; r0 < r_end; r0 += 16) {
    float xa[8], da[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = r0 + 8 * hh + e;
      const bool ok = r < r_end;
      const int64_t o = static_cast<int64_t>(ok ? r : r_beg) * rs;
      const float xv = xp[o], dv = dp[o];
      xa[e] = ok ? xv : 0.f;
      da[e] = ok ? dv : 0.f;
    }
    bf16x8 xh, xl, dh, dl;
    split_bf16(xa, xh, xl);
    split_bf16(da, dh, dl);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, dh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, dl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl, dh, acc, 0, 0, 0);
  }
  // register r: result row ra + 8 (r / 4) + 4 hh + r % 4, column cb + ql
  float* dst = part + (static_cast<int64_t>(c) * Hq + h) * DH * DH + cb + ql;
#pragma unroll
  for (int r = 0; r < 16; ++r) dst[(ra + 8 * (r >> 2) + 4 * hh + (r & 3)) * DH] = acc[r];
}

// dP[h] = the sum of the partials in chunk order; the partials are dh x dh per head (a D < dh projector takes
// their D x D corner).
__global__ __launch_bounds__(256) void k_dp_reduce(const float* part, float* dP, int nchunks, int Hq, int D, int dh) {
  const int64_t n = static_cast<int64_t>(Hq) * dh * dh;
  for (int64_t e = blockIdx.x * 256LL + threadIdx.x; e < n; e += 256LL * gridDim.x) {
    // in chunk order; eight loads are issued before their adds
    float s = 0.f;
    int c = 0;
    for (; c + 8 <= nchunks; c += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(c + u) * n + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; c < nchunks; ++c) s += part[c * n + e];
    const int64_t hh = e / (dh * dh);
    const int a = static_cast<int>((e / dh) % dh), c2 = static_cast<int>(e % dh);
    if (a < D && c2 < D) dP[(hh * D + a) * D + c2] = s;
  }
}

// ------------------------------------------------------------------------------------------
// workspace layout
// ------------------------------------------------------------------------------------------

struct BwdWs {
  Staging st;
  _Float16 *q16, *do16, *u16, *e16, *u16lo, *e16lo;
  float *u32, *dkb32, *x32, *du32, *alpha, *delta, *part;
  _Float16* ds;   // [B][Hq][Tq_pad / 32][Tk_pad / 32] tiles of 32 x 32 fp16
  float* rstat;   // [B][Hq][Tq_pad / 32][3][32]
  size_t rstat_n;
  float* rowmax;  // [B][Hkv][kRowStats][Tq_pad]
  size_t rowmax_n;
  float* dsscale; // [B][Hkv][Tk_pad / 32]
  float *dklo, *dvlo;  // [B][lo_keys][Hkv][D]: the split rows' dk, dv, added to the others' at the end
  int Tq_pad, lo_rows, lo_pad, nchunks, lo_keys;
  size_t bytes;
};

BwdWs bwd_layout(const Geom& g, int split, void* ws) {
  BwdWs w{};
  const int dh = g.d == 64 ? 64 : kD;   // a head of 64 is staged and computed at 64
  w.st = staging_layout(ws, g.B, g.Tk, g.Hkv, g.Hq, true, dh);
  size_t off = w.st.bytes;
  char* base = static_cast<char*>(ws);
  w.Tq_pad = (g.Tq + 31) / 32 * 32;
  w.lo_rows = split;
  w.lo_pad = (split + 31) / 32 * 32;
  const size_t qh = static_cast<size_t>(g.B) * g.Hq * w.Tq_pad * dh * sizeof(_Float16);
  const size_t lh = static_cast<size_t>(g.B) * g.Hq * w.lo_pad * dh * sizeof(_Float16);
  const size_t rf = static_cast<size_t>(g.B) * g.Tq * g.Hq * dh * sizeof(float);
  const size_t sf = static_cast<size_t>(g.B) * g.Hq * g.Tq * sizeof(float);
  _Float16** h16[4] = {&w.q16, &w.do16, &w.u16, &w.e16};
  for (auto pp : h16) *pp = reinterpret_cast<_Float16*>(base + ws_take(off, qh));   // equal, consecutive blocks
  _Float16** l16[2] = {&w.u16lo, &w.e16lo};
  for (auto pp : l16) *pp = reinterpret_cast<_Float16*>(base + ws_take(off, lh));
  float** f32[4] = {&w.u32, &w.dkb32, &w.x32, &w.du32};
  for (auto pp : f32) *pp = reinterpret_cast<float*>(base + ws_take(off, rf));
  w.alpha = reinterpret_cast<float*>(base + ws_take(off, sf));
  w.delta = reinterpret_cast<float*>(base + ws_take(off, sf));
  const int64_t R = static_cast<int64_t>(g.B) * g.Tq;
  w.nchunks = static_cast<int>((R + kPChunk - 1) / kPChunk);
  w.part = reinterpret_cast<float*>(base + ws_take(off, static_cast<size_t>(w.nchunks) * g.Hq * dh * dh * 4));
  const size_t ds_bytes = static_cast<size_t>(g.B) * g.Hq * (w.Tq_pad / 32) * (w.st.Tk_pad / 32) * 1024 * 2;
  w.ds = reinterpret_cast<_Float16*>(base + ws_take(off, ds_bytes));
  w.rstat_n = static_cast<size_t>(g.B) * g.Hq * w.Tq_pad * 3;
  w.rstat = reinterpret_cast<float*>(base + ws_take(off, w.rstat_n * sizeof(float)));
  w.rowmax_n = static_cast<size_t>(g.B) * g.Hkv * kRowStats * w.Tq_pad;
  w.rowmax = reinterpret_cast<float*>(base + ws_take(off, w.rowmax_n * sizeof(float)));
  w.dsscale = reinterpret_cast<float*>(base + ws_take(off, static_cast<size_t>(g.B) * g.Hkv * (w.st.Tk_pad / 32) * sizeof(float)));
  // the keys that rows < split can see, rounded up to the split key kernel's 128-key blocks
  const int khi = g.causal && split + g.Tk - g.Tq < g.Tk ? split + g.Tk - g.Tq : g.Tk;
  const int khi_blocks = (khi + 127) / 128 * 128;
  w.lo_keys = khi > 0 ? (khi_blocks < g.Tk ? khi_blocks : g.Tk) : 0;
  const size_t lob = static_cast<size_t>(g.B) * w.lo_keys * g.Hkv * g.d * sizeof(float);
  w.dklo = reinterpret_cast<float*>(base + ws_take(off, lob));
  w.dvlo = reinterpret_cast<float*>(base + ws_take(off, lob));
  w.bytes = off;
  return w;
}

int bwd_split(const Geom& g) {
  const int s = 256 + rows_without_keys(g);
  return s < g.Tq ? s : g.Tq;
}

}  // namespace

bool fast_bwd_supported(const Geom& g) {
  const int G = g.Hq / g.Hkv;
  return g.bf16 && (g.d == kD || g.d == 64) && !g.p_per_query && (G == 1 || G == 2 || G == 4 || G == 8) && g.B > 0 &&
         g.Tq > 0 &&
         g.Tk > 0;
}

size_t fast_bwd_workspace(const Geom& g) { return bwd_layout(g, bwd_split(g), nullptr).bytes; }

bool fast_probe_bwd_supported(const Geom& g) { return fast_bwd_supported(g); }

size_t fast_probe_bwd_workspace(const Geom& g) { return fast_bwd_workspace(g); }

hipError_t launch_zero_f32(float* x, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero4, dim3(256), dim3(256), 0, stream, x, n / 4);
  return hipGetLastError();
}

namespace {

struct BwdArgs {
  const void *q, *k, *v, *P, *dout, *rho;   // rho != nullptr: the probe form (P unused)
  const float *out, *lse, *kbar, *osa, *rk;
  float *dq, *dk, *dv, *dP, *drho;
};

hipError_t bwd_impl(const Geom& g, const BwdArgs& a, int split_rows, void* ws, hipStream_t stream) {
  const bool probe = a.rho != nullptr;
  const void *q = a.q, *k = a.k, *v = a.v, *P = a.P, *dout = a.dout;
  const float *out = a.out, *lse = a.lse, *kbar = a.kbar, *osa = a.osa;
  float *dq = a.dq, *dk = a.dk, *dv = a.dv, *dP = a.dP;
  // The workspace is sized for the default split; a larger request is clamped to it.
  int split = split_rows < 0 ? bwd_split(g) : split_rows + rows_without_keys(g);
  if (split < kMinSplitRows + rows_without_keys(g)) split = kMinSplitRows + rows_without_keys(g);
  if (split > bwd_split(g)) split = bwd_split(g);
  const BwdWs w = bwd_layout(g, bwd_split(g), ws);
  const int G = g.Hq / g.Hkv;
  const bool d64 = w.st.dh == 64;   // the kernels instantiated for head dim 64
  const int64_t q_elems = static_cast<int64_t>(g.B) * g.Tq * g.Hq * g.d;
  hipError_t e = launch_staging(w.st, q, q_elems, k, v, P, g.B, g.Tk, g.Hkv, g.Hq, stream, dout, q_elems, kMaxDO, g.d);
  if (e != hipSuccess) return e;

  // row statistics of padded rows stay 0 (the key-major kernel reads whole 32-row tiles); the per-row
  // maxima start at 0 for the row kernels' atomicMax
  hipLaunchKernelGGL(k_zero4x2, dim3(256), dim3(256), 0, stream, w.rstat, static_cast<int64_t>(w.rstat_n / 4),
                     w.rowmax, static_cast<int64_t>(w.rowmax_n / 4));
  RowParams rp{};
  rp.q = static_cast<const u16*>(q);
  rp.dout = static_cast<const u16*>(dout);
  rp.out = out;
  rp.lse = lse;
  rp.kbar = kbar;
  rp.osa = osa;
  rp.k16 = w.st.k16;
  rp.k16t = w.st.k16t;
  rp.v16 = w.st.v16;
  rp.p16t = w.st.p16t;
  rp.p16 = w.st.p16;
  rp.maxbits = w.st.maxbits;
  rp.dq = dq;
  rp.u32 = w.u32;
  rp.dkb32 = w.dkb32;
  rp.x32 = w.x32;
  rp.du32 = w.du32;
  rp.st_alpha = w.alpha;
  rp.st_delta = w.delta;
  rp.rstat = w.rstat;
  rp.knorm = w.st.knorm;
  rp.vnorm = w.st.vnorm;
  rp.rowmax = w.rowmax;
  rp.D = g.d;
  rp.rho = static_cast<const u16*>(a.rho);
  rp.rk = a.rk;
  rp.drho = a.drho;
  rp.Tq_pad = w.Tq_pad;
  rp.B = g.B;
  rp.Tq = g.Tq;
  rp.Tk = g.Tk;
  rp.Tk_pad = w.st.Tk_pad;
  rp.Hq = g.Hq;
  rp.Hkv = g.Hkv;
  rp.G = G;
  rp.causal = g.causal;
  rp.window = g.window;
  rp.scale = g.scale;
  rp.rows_per_block = G > 4 ? 32 : 32 * 4 / G;   // split-row kernel: four waves of 32 rows
  const int hsplit = G > 4 ? G / 4 : 1;           // ... and two blocks per group when G = 8
  // The kernels for rows < split (few blocks, bound by latency) run on a side lane beside the main
  // ones: the row kernel beside the du kernel, the key kernel beside the key-major one.  The fp16 query
  // tiles of q and dout are first read by the key-major kernel, so their staging also runs on the
  // side lane beside du.
  const bool use_side = split > 0 && split < g.Tq;
  SideLane side = use_side ? side_fork(stream) : SideLane{stream, stream};
  e = launch_stage_rows(q, false, w.st.maxbits, kMaxQ, w.q16, nullptr, g.B, g.Tq, w.Tq_pad, g.Hq, 0, 0, side.stream,
                        g.d, w.st.dh);
  if (e != hipSuccess) return e;
  e = launch_stage_rows(dout, false, w.st.maxbits, kMaxDO, w.do16, nullptr, g.B, g.Tq, w.Tq_pad, g.Hq, 0, 0,
                        side.stream, g.d, w.st.dh);
  if (e != hipSuccess) return e;
  if (split > 0) {
    RowParams r = rp;
    r.row_begin = 0;
    r.row_end = split;
    r.n_rb = (split + r.rows_per_block - 1) / r.rows_per_block;
    const dim3 grid(g.B * g.Hkv * hsplit * r.n_rb);
    if (probe) {
      if (d64) hipLaunchKernelGGL((k_bwd_rows_fast<true, true, true, 64>), grid, dim3(256), 0, side.stream, r);
      else hipLaunchKernelGGL((k_bwd_rows_fast<true, true, true, kD>), grid, dim3(256), 0, side.stream, r);
    } else {
      if (d64) hipLaunchKernelGGL((k_bwd_rows_fast<true, true, false, 64>), grid, dim3(256), 0, side.stream, r);
      else hipLaunchKernelGGL((k_bwd_rows_fast<true, true, false, kD>), grid, dim3(256), 0, side.stream, r);
    }
  }
  if (split < g.Tq) {
    RowParams r = rp;
    r.row_begin = split;
    r.row_end = g.Tq;
    r.n_rb = (g.Tq - split + r.rows_per_block - 1) / r.rows_per_block;
    r.rows_per_block = 32 * 8 / G;
    r.n_rb = (g.Tq - split + r.rows_per_block - 1) / r.rows_per_block;
    mark_begin(PLX_KERNEL_BWD_ROWS, stream);
    const dim3 grid(g.B * g.Hkv * r.n_rb);
    if (probe) {
      if (d64) hipLaunchKernelGGL((k_bwd_du<true, 64>), grid, dim3(512), 0, stream, r);
      else hipLaunchKernelGGL((k_bwd_du<true, kD>), grid, dim3(512), 0, stream, r);
    } else {
      if (d64) hipLaunchKernelGGL((k_bwd_du<false, 64>), grid, dim3(512), 0, stream, r);
      else hipLaunchKernelGGL((k_bwd_du<false, kD>), grid, dim3(512), 0, stream, r);
    }
    mark_end(PLX_KERNEL_BWD_ROWS, stream);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = side_join(side);
  if (e != hipSuccess) return e;
  // dP = sum over rows of x du^T (x, du from the row kernels, complete now) on the side lane, beside the
  // key-major kernel
  const SideLane dpl = probe ? SideLane{stream, stream} : side_fork(stream);
  if (!probe) {
    const int R = g.B * g.Tq;
    if (d64)
      hipLaunchKernelGGL(k_dp_partial64, dim3(g.Hq * w.nchunks), dim3(256), 0, dpl.stream, w.x32, w.du32, w.part, R,
                         g.Hq);
    else
      hipLaunchKernelGGL(k_dp_partial, dim3(g.Hq * w.nchunks), dim3(256), 0, dpl.stream, w.x32, w.du32, w.part, R,
                         g.Hq);
    const int nred = (g.Hq * w.st.dh * w.st.dh + 255) / 256;
    hipLaunchKernelGGL(k_dp_reduce, dim3(nred), dim3(256), 0, dpl.stream, w.part, dP, w.nchunks, g.Hq, g.d, w.st.dh);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // per (batch, kv head, statistic): the maximum over rows >= i of each row statistic
  e = launch_scan_max(w.rowmax, w.Tq_pad, g.B * g.Hkv * kRowStats, w.Tq_pad, true, stream);
  if (e != hipSuccess) return e;
  // fp16 copies of u and dkbar (lo parts for rows < split)
  e = launch_stage_rows(w.u32, true, w.st.maxbits, kMaxU, w.u16, split > 0 ? w.u16lo : nullptr, g.B, g.Tq, w.Tq_pad,
                        g.Hq, split, w.lo_pad, stream, w.st.dh, w.st.dh);
  if (e != hipSuccess) return e;
  e = launch_stage_rows(w.dkb32, true, w.st.maxbits, kMaxDKB, w.e16, split > 0 ? w.e16lo : nullptr, g.B, g.Tq,
                        w.Tq_pad, g.Hq, split, w.lo_pad, stream, w.st.dh, w.st.dh);
  if (e != hipSuccess) return e;

  KeyParams kp{};
  kp.k16 = w.st.k16;
  kp.v16 = w.st.v16;
  kp.q16 = w.q16;
  kp.do16 = w.do16;
  kp.u16 = w.u16;
  kp.e16 = w.e16;
  kp.u16lo = w.u16lo;
  kp.e16lo = w.e16lo;
  kp.lse = lse;
  kp.alpha = w.alpha;
  kp.delta = w.delta;
  kp.rstat = w.rstat;
  kp.rowmax = w.rowmax;
  kp.dsscale = w.dsscale;
  kp.D = g.d;
  kp.qstride = w.do16 - w.q16;
  kp.maxbits = w.st.maxbits;
  kp.dk = dk;
  kp.dv = dv;
  kp.B = g.B;
  kp.Tq = g.Tq;
  kp.Tk = g.Tk;
  kp.Tk_pad = w.st.Tk_pad;
  kp.Tq_pad = w.Tq_pad;
  kp.lo_pad = w.lo_pad;
  kp.Hq = g.Hq;
  kp.Hkv = g.Hkv;
  kp.G = G;
  kp.causal = g.causal;
  kp.window = g.window;
  kp.scale = g.scale;
  kp.n_kb = (g.Tk + 127) / 128;
  kp.key_hi = g.Tk;
  kp.out_keys = g.Tk;
  // rows < split: only keys those rows can see, written to their own buffers by the hi + lo key kernel on
  // the side lane while the key-major kernel runs, and added to dk, dv after both
  const int off = g.Tk - g.Tq;
  int khi = g.causal ? split - 1 + off + 1 : g.Tk;
  khi = khi > g.Tk ? g.Tk : khi;
  const bool lo_keys = split > 0 && khi > 0;
  side = use_side ? side_fork(stream) : SideLane{stream, stream};
  if (lo_keys) {
    KeyParams k2 = kp;
    k2.row_lo = 0;
    k2.row_hi = split;
    k2.accumulate = 0;
    k2.key_hi = khi;
    k2.n_kb = (khi + 127) / 128;
    k2.dk = w.dklo;
    k2.dv = w.dvlo;
    k2.out_keys = w.lo_keys;
    if (d64) hipLaunchKernelGGL((k_bwd_keys_fast<true, 64>), dim3(g.B * g.Hkv * k2.n_kb), dim3(256), 0, side.stream, k2);
    else hipLaunchKernelGGL((k_bwd_keys_fast<true, kD>), dim3(g.B * g.Hkv * k2.n_kb), dim3(256), 0, side.stream, k2);
  }
  {
    // every key block, rows >= split, writing
    KeyParams k2 = kp;
    k2.row_lo = split;
    k2.row_hi = g.Tq;
    k2.accumulate = 0;
    k2.ds = w.ds;
    mark_begin(PLX_KERNEL_BWD_KEYS, stream);
    if (d64) hipLaunchKernelGGL(k_bwd_keys_pipe<64>, dim3(g.B * g.Hkv * k2.n_kb), dim3(512), 0, stream, k2);
    else hipLaunchKernelGGL(k_bwd_keys_pipe<kD>, dim3(g.B * g.Hkv * k2.n_kb), dim3(512), 0, stream, k2);
    mark_end(PLX_KERNEL_BWD_KEYS, stream);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (split < g.Tq) {
    DqParams dp{};
    dp.ds = w.ds;
    dp.dsscale = w.dsscale;
    dp.k16t = w.st.k16t;
    dp.maxbits = w.st.maxbits;
    dp.dq = dq;
    dp.D = g.d;
    dp.B = g.B;
    dp.Tq = g.Tq;
    dp.Tk = g.Tk;
    dp.Tk_pad = w.st.Tk_pad;
    dp.Tq_pad = w.Tq_pad;
    dp.Hq = g.Hq;
    dp.Hkv = g.Hkv;
    dp.G = G;
    dp.causal = g.causal;
    dp.window = g.window;
    dp.row_lo = split;
    dp.row_hi = g.Tq;
    dp.row_begin = (split / 32) * 32;   // ds tiles are 32-row aligned
    dp.rows_per_block = 32 * 8 / G;
    dp.n_rb = (g.Tq - dp.row_begin + dp.rows_per_block - 1) / dp.rows_per_block;
    dp.scale = g.scale;
    mark_begin(PLX_KERNEL_BWD_DQ, stream);
    if (d64) hipLaunchKernelGGL(k_bwd_dq<64>, dim3(g.B * g.Hkv * dp.n_rb), dim3(512), 0, stream, dp);
    else hipLaunchKernelGGL(k_bwd_dq<kD>, dim3(g.B * g.Hkv * dp.n_rb), dim3(512), 0, stream, dp);
    mark_end(PLX_KERNEL_BWD_DQ, stream);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = side_join(dpl);   // (the dP work, and whatever followed it on the side lane)
  if (e != hipSuccess) return e;
  e = side_join(side);
  if (e != hipSuccess) return e;
  if (lo_keys) {
    const int64_t n4 = static_cast<int64_t>(g.Hkv) * g.d / 4;
    hipLaunchKernelGGL(k_add_lo, dim3(256), dim3(256), 0, stream, dk, dv, w.dklo, w.dvlo, g.B,
                       static_cast<int64_t>(khi), static_cast<int64_t>(w.lo_keys), static_cast<int64_t>(g.Tk), n4);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_fast_bwd(const Geom& g, const void* q, const void* k, const void* v, const void* P,
                           const float* out, const void* dout, const float* lse, const float* kbar,
                           const float* osa, float* dq, float* dk, float* dv, float* dP, int split_rows,
                           void* ws, hipStream_t stream) {
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.P = P;
  a.dout = dout;
  a.out = out;
  a.lse = lse;
  a.kbar = kbar;
  a.osa = osa;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dP = dP;
  return bwd_impl(g, a, split_rows, ws, stream);
}

hipError_t launch_fast_probe_bwd(const Geom& g, const void* q, const void* k, const void* v, const void* rho,
                                 const float* out, const void* dout, const float* lse, const float* osa,
                                 const float* rk, float* dq, float* dk, float* dv, float* drho, int split_rows,
                                 void* ws, hipStream_t stream) {
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.rho = rho;
  a.dout = dout;
  a.out = out;
  a.lse = lse;
  a.osa = osa;
  a.rk = rk;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.drho = drho;
  return bwd_impl(g, a, split_rows, ws, stream);
}

}  // namespace plx
