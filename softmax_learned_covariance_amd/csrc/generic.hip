// Generic Parallax kernels: fp32 arithmetic on fp32 or bf16 inputs, any head_dim <= 128.
//
// One 64-lane wave owns one query row (forward, backward row passes) or one key
// row (backward key pass); lane l holds dimensions l and l + 64.  Dot products
// are butterfly reductions across the wave, so every lane ends with the same
// bits.  These kernels are the fp32 path of the library: fp32 inputs, per-query
// projectors, head dims other than 128 and 64, and query-head groups outside
// {1, 2, 4, 8}.  (The first query rows of the bf16 path, where few visible keys
// make the output large, run on that path's hi + lo operand-pair kernels.)
//
// Formulas: the output equation of the gist.science technical summary of
// "Parallax: Parameterized Local Linear Attention for Language Modeling",
// section "Core mechanism" (softmax output plus the key/value covariance applied
// to the probe u = P^T (q - kbar)), evaluated in its centred form
//   out_i = o_i + sum_j p_ij (u_i . (k_j - kbar_i)) (v_j - o_i);
// the backward is the chain rule of that definition (g = dout, alpha = u.kbar,
// t_ij = u_i.k_j):
//   du_i    = sum_j p_ij (g_i.v_j) (k_j - kbar_i)
//   dkbar_i = -(g_i.o_i) u_i - P du_i,   dq_i = P du_i + scale sum_j ds_ij k_j
//   Delta_i = g_i.out_i + dkbar_i.kbar_i
//   ds_ij   = p_ij ((g_i.v_j)(t_ij + 1 - alpha_i) + dkbar_i.k_j - Delta_i)
//   dk_j    = sum_i p_ij (g_i.v_j) u_i + p_ij dkbar_i + scale ds_ij q_i
//   dv_j    = sum_i p_ij (t_ij + 1 - alpha_i) g_i
//   dP      = sum_i (q_i - kbar_i) du_i^T
#include <math.h>

#include "plx_internal.h"

namespace plx {
namespace {

constexpr int kWaves = 4;  // waves per 256-thread block

template <bool BF16>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  if constexpr (BF16) {
    uint32_t bits = static_cast<const uint16_t*>(p)[i];
    return __uint_as_float(bits << 16);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Two independent reductions interleaved (more instruction-level parallelism).
__device__ __forceinline__ void wave_sum2(float& x, float& y) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float a = __shfl_xor(x, o, 64), b = __shfl_xor(y, o, 64);
    x += a;
    y += b;
  }
}

__device__ __forceinline__ void wave_sum4(float& x, float& y, float& z, float& w) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float a = __shfl_xor(x, o, 64), b = __shfl_xor(y, o, 64);
    float c = __shfl_xor(z, o, 64), e = __shfl_xor(w, o, 64);
    x += a;
    y += b;
    z += c;
    w += e;
  }
}

struct Args {
  const void *q, *k, *v, *P, *dout;
  const int32_t* seqlens;
  const float *out_in, *lse_in, *kbar_in, *osa_in;
  float *out, *lse, *kbar, *osa;
  float *dq, *dk, *dv, *dP;
  float *X, *DU, *DKB, *U, *ALPHA, *DELTA;  // backward workspace
  int B, Tq, Tk, Hq, Hkv, d, causal, window, p_per_query;
  float scale;
  int row_begin, row_end;
};

// Visible key range [lo, hi) of query row i when the sequence holds Tk keys.
__device__ __forceinline__ void key_range(const Args& a, int i, int Tk, int& lo, int& hi) {
  const int off = Tk - a.Tq;
  hi = a.causal ? min(Tk, i + off + 1) : Tk;
  lo = a.window > 0 ? max(0, i + off - a.window + 1) : 0;
  hi = max(hi, lo);
}

// Index of element (b, t, head, dim) in a [B][T][H][d] tensor.
__device__ __forceinline__ int64_t idx4(int b, int t, int T, int head, int H, int d, int dim) {
  return ((static_cast<int64_t>(b) * T + t) * H + head) * d + dim;
}

// ------------------------------- forward -----------------------------------
template <bool BF16, int DPL>
__global__ __launch_bounds__(256) void k_fwd(Args a) {
  __shared__ float xs[kWaves][128];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int i = a.row_begin + blockIdx.x * kWaves + wave;
  const int h = blockIdx.y, b = blockIdx.z;
  const bool valid = i < a.row_end;
  const int d = a.d, g = h / (a.Hq / a.Hkv);
  int Tk = a.Tk;
  if (a.seqlens) Tk = min(max(a.seqlens[b], 0), a.Tk);
  int lo = 0, hi = 0;
  if (valid) key_range(a, i, Tk, lo, hi);

  float qv[DPL], o[DPL], kb[DPL], u[DPL];
  float m = -INFINITY, l = 0.f;
#pragma unroll
  for (int r = 0; r < DPL; ++r) {
    const int dim = lane + 64 * r;
    qv[r] = (valid && dim < d) ? ld<BF16>(a.q, idx4(b, i, a.Tq, h, a.Hq, d, dim)) : 0.f;
    o[r] = 0.f;
    kb[r] = 0.f;
    u[r] = 0.f;
  }
  // pass 1: online softmax accumulating o and kbar together
  for (int j = lo; j < hi; ++j) {
    float kv[DPL], vv[DPL], s = 0.f;
#pragma unroll
    for (int r = 0; r < DPL; ++r) {
      const int dim = lane + 64 * r;
      const int64_t e = idx4(b, j, a.Tk, g, a.Hkv, d, dim);
      kv[r] = dim < d ? ld<BF16>(a.k, e) : 0.f;
      vv[r] = dim < d ? ld<BF16>(a.v, e) : 0.f;
      s += qv[r] * kv[r];
    }
    s = wave_sum(s) * a.scale;
    const float mn = fmaxf(m, s);
    const float corr = expf(m - mn), p = expf(s - mn);
    l = l * corr + p;
#pragma unroll
    for (int r = 0; r < DPL; ++r) {
      o[r] = o[r] * corr + p * vv[r];
      kb[r] = kb[r] * corr + p * kv[r];
    }
    m = mn;
  }
  float lse_i = -INFINITY;
  if (hi > lo) {
    const float inv = 1.f / l;
#pragma unroll
    for (int r = 0; r < DPL; ++r) {
      o[r] *= inv;
      kb[r] *= inv;
    }
    lse_i = m + logf(l);
  }
#pragma unroll
  for (int r = 0; r < DPL; ++r) {
    const int dim = lane + 64 * r;
    if (dim < 128) xs[wave][dim] = dim < d ? qv[r] - kb[r] : 0.f;
  }
  __syncthreads();
  // probe u[a] = sum_b P[b][a] (q - kbar)[b]
  const int64_t pbase = a.p_per_query ? idx4(b, i, a.Tq, h, a.Hq, d, 0) * d
                                      : static_cast<int64_t>(h) * d * d;
  if (valid && hi > lo) {
    for (int bb = 0; bb < d; ++bb) {
      const float xb = xs[wave][bb];
#pragma unroll
      for (int r = 0; r < DPL; ++r) {
        const int dim = lane + 64 * r;
        if (dim < d) u[r] += ld<BF16>(a.P, pbase + static_cast<int64_t>(bb) * d + dim) * xb;
      }
    }
  }
  float alpha = 0.f;
#pragma unroll
  for (int r = 0; r < DPL; ++r) alpha += u[r] * kb[r];
  alpha = wave_sum(alpha);
  // pass 2: c = sum_j p_j (u.(k_j - kbar)) (v_j - o)
  float c[DPL];
#pragma unroll
  for (int r = 0; r < DPL; ++r) c[r] = 0.f;
  for (int j = lo; j < hi; ++j) {
    float kv[DPL], vv[DPL], s = 0.f, t = 0.f;
#pragma unroll
    for (int r = 0; r < DPL; ++r) {
      const int dim = lane + 64 * r;
      const int64_t e = idx4(b, j, a.Tk, g, a.Hkv, d, dim);
      kv[r] = dim < d ? ld<BF16>(a.k, e) : 0.f;
      vv[r] = dim < d ? ld<BF16>(a.v, e) : 0.f;
      s += qv[r] * kv[r];
      t += u[r] * kv[r];
    }
    wave_sum2(s, t);
    const float p = expf(s * a.scale - lse_i);
    const float w = p * (t - alpha);
#pragma unroll
    for (int r = 0; r < DPL; ++r) c[r] += w * (vv[r] - o[r]);
  }
  if (!valid) return;
#pragma unroll
  for (int r = 0; r < DPL; ++r) {
    const int dim = lane + 64 * r;
    if (dim < d) {
      const int64_t e = idx4(b, i, a.Tq, h, a.Hq, d, dim);
      a.out[e] = o[r] + c[r];
      if (a.kbar) a.kbar[e] = kb[r];
      if (a.osa) a.osa[e] = o[r];
    }
  }
  if (a.lse && lane == 0) a.lse[(static_cast<int64_t>(b) * a.Hq + h) * a.Tq + i] = lse_i;
}

// --------------------------- backward, row pass A ---------------------------
template <bool BF16, int DPL>
__global__ __launch_bounds__(256) void k_bwd_rows(Args a) {
  __shared__ float xs[kWaves][128];
  __shared__ float dus[kWaves][128];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int i = blockIdx.x * kWaves + wave;
  const int h = blockIdx.y, b = blockIdx.z;
  const bool valid = i < a.Tq;
  const int d = a.d, g = h / (a.Hq / a.Hkv);
  int lo = 0, hi = 0;
  if (valid) key_range(a, i, a.Tk, lo, hi);
  const int64_t row = valid ? idx4(b, i, a.Tq, h, a.Hq, d, 0) : 0;
  const float lse_i = valid ? a.lse_in[(static_cast<int64_t>(b) * a.Hq + h) * a.Tq + i] : 0.f;

  float qv[DPL], gv[DPL], o[DPL], kb[DPL], ov[DPL], u[DPL], du[DPL];
#pragma unroll
  for (int r = 0; r < DPL; ++r) {
    const int dim = lane + 64 * r;
    const bool on = valid && dim < d;
    qv[r] = on ? ld<BF16>(a.q, row + dim) : 0.f;
    gv[r] = on ? ld<BF16>(a.dout, row + dim) : 0.f;
    o[r] = on ? a.osa_in[row + dim] : 0.f;
    kb[r] = on ? a.kbar_in[row + dim] : 0.f;
    ov[r] = on ? a.out_in[row + dim] : 0.f;
    u[r] = 0.f;
    du[r] = 0.f;
    if (dim < 128) xs[wave][dim] = qv[r] - kb[r];
  }
  __syncthreads();
  const int64_t pbase = static_cast<int64_t>(h) * d * d;
  if (valid) {
    for (int bb = 0; bb < d; ++bb) {
      const float xb = xs[wave][bb];
#pragma unroll
      for (int r = 0; r < DPL; ++r) {
        const int dim = lane + 64 * r;
        if (dim < d) u[r] += ld<BF16>(a.P, pbase + static_cast<int64_t>(bb) * d + dim) * xb;
      }
    }
  }
  float alpha = 0.f, go = 0.f, gout = 0.f;
#pragma unroll
  for (int r = 0; r < DPL; ++r) {
    alpha += u[r] * kb[r];
    go += gv[r] * o[r];
    gout += gv[r] * ov[r];
  }
  float dummy = 0.f;
  wave_sum4(alpha, go, gout, dummy);
  // du = sum_j p_j (g.v_j) (k_j - kbar)
  for (int j = lo; j < hi; ++j) {
    float kv[DPL], s = 0.f, G = 0.f;
#pragma unroll
    for (int r = 0; r < DPL; ++r) {
      const int dim = lane + 64 * r;
      const int64_t e = idx4(b, j, a.Tk, g, a.Hkv, d, dim);
      kv[r] = dim < d ? ld<BF16>(a.k, e) : 0.f;
      const float vv = dim < d ? ld<BF16>(a.v, e) : 0.f;
      s += qv[r] * kv[r];
      G += gv[r] * vv;
    }
    wave_sum2(s, G);
    const float pg = expf(s * a.scale - lse_i) * G;
#pragma unroll
    for (int r = 0; r < DPL; ++r) du[r] += pg * (kv[r] - kb[r]);
  }
#pragma unroll
  for (int r = 0; r < DPL; ++r) {
    const int dim = lane + 64 * r;
    if (dim < 128) dus[wave][dim] = du[r];
  }
  __syncthreads();
  // (P du)[b] = sum_a P[b][a] du[a]; lane holds rows b = lane, lane + 64
  float pdu[DPL];
#pragma unroll
  for (int r = 0; r < DPL; ++r) {
    const int bb = lane + 64 * r;
    float acc = 0.f;
    if (valid && bb < d)
      for (int aa = 0; aa < d; ++aa)
        acc += ld<BF16>(a.P, pbase + static_cast<int64_t>(bb) * d + aa) * dus[wave][aa];
    pdu[r] = acc;
  }
  float dkb[DPL], dkk = 0.f;
#pragma unroll
  for (int r = 0; r < DPL; ++r) {
    dkb[r] = -go * u[r] - pdu[r];
    dkk += dkb[r] * kb[r];
  }
  dkk = wave_sum(dkk);
  if (!valid) return;
#pragma unroll
  for (int r = 0; r < DPL; ++r) {
    const int dim = lane + 64 * r;
    if (dim < d) {
      a.dq[row + dim] = pdu[r];
      a.X[row + dim] = qv[r] - kb[r];
      a.DU[row + dim] = du[r];
      a.DKB[row + dim] = dkb[r];
      a.U[row + dim] = u[r];
    }
  }
  if (lane == 0) {
    const int64_t rs = (static_cast<int64_t>(b) * a.Hq + h) * a.Tq + i;
    a.ALPHA[rs] = alpha;
    a.DELTA[rs] = gout + dkk;
  }
}

// --------------------------- backward, key pass B ---------------------------
template <bool BF16, int DPL>
__global__ __launch_bounds__(256) void k_bwd_keys(Args a) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int j = blockIdx.x * kWaves + wave;
  const int g = blockIdx.y, b = blockIdx.z;
  if (j >= a.Tk) return;  // no block barrier in this kernel
  const int d = a.d, grp = a.Hq / a.Hkv, off = a.Tk - a.Tq;
  float kv[DPL], vv[DPL], dk[DPL], dv[DPL];
#pragma unroll
  for (int r = 0; r < DPL; ++r) {
    const int dim = lane + 64 * r;
    const int64_t e = idx4(b, j, a.Tk, g, a.Hkv, d, dim);
    kv[r] = dim < d ? ld<BF16>(a.k, e) : 0.f;
    vv[r] = dim < d ? ld<BF16>(a.v, e) : 0.f;
    dk[r] = 0.f;
    dv[r] = 0.f;
  }
  const int i_lo = a.causal ? max(0, j - off) : 0;
  const int i_hi = a.window > 0 ? min(a.Tq, j - off + a.window) : a.Tq;
  for (int hh = 0; hh < grp; ++hh) {
    const int h = g * grp + hh;
    for (int i = i_lo; i < i_hi; ++i) {
      const int64_t row = idx4(b, i, a.Tq, h, a.Hq, d, 0);
      const int64_t rs = (static_cast<int64_t>(b) * a.Hq + h) * a.Tq + i;
      float qv[DPL], gv[DPL], uv[DPL], ev[DPL];
      float s = 0.f, t = 0.f, G = 0.f, E = 0.f;
#pragma unroll
      for (int r = 0; r < DPL; ++r) {
        const int dim = lane + 64 * r;
        const bool on = dim < d;
        qv[r] = on ? ld<BF16>(a.q, row + dim) : 0.f;
        gv[r] = on ? ld<BF16>(a.dout, row + dim) : 0.f;
        uv[r] = on ? a.U[row + dim] : 0.f;
        ev[r] = on ? a.DKB[row + dim] : 0.f;
        s += qv[r] * kv[r];
        t += uv[r] * kv[r];
        G += gv[r] * vv[r];
        E += ev[r] * kv[r];
      }
      wave_sum4(s, t, G, E);
      const float p = expf(s * a.scale - a.lse_in[rs]);
      const float tt = t + 1.f - a.ALPHA[rs];
      const float ds = p * (G * tt + E - a.DELTA[rs]);
#pragma unroll
      for (int r = 0; r < DPL; ++r) {
        dv[r] += p * tt * gv[r];
        dk[r] += p * G * uv[r] + p * ev[r] + a.scale * ds * qv[r];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < DPL; ++r) {
    const int dim = lane + 64 * r;
    if (dim < d) {
      const int64_t e = idx4(b, j, a.Tk, g, a.Hkv, d, dim);
      a.dk[e] = dk[r];
      a.dv[e] = dv[r];
    }
  }
}

// --------------------------- backward, row pass C ---------------------------
template <bool BF16, int DPL>
__global__ __launch_bounds__(256) void k_bwd_dq(Args a) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int i = blockIdx.x * kWaves + wave;
  const int h = blockIdx.y, b = blockIdx.z;
  if (i >= a.Tq) return;  // no block barrier in this kernel
  const int d = a.d, g = h / (a.Hq / a.Hkv);
  int lo, hi;
  key_range(a, i, a.Tk, lo, hi);
  const int64_t row = idx4(b, i, a.Tq, h, a.Hq, d, 0);
  const int64_t rs = (static_cast<int64_t>(b) * a.Hq + h) * a.Tq + i;
  const float lse_i = a.lse_in[rs], alpha = a.ALPHA[rs], delta = a.DELTA[rs];
  float qv[DPL], gv[DPL], uv[DPL], ev[DPL], acc[DPL];
#pragma unroll
  for (int r = 0; r < DPL; ++r) {
    const int dim = lane + 64 * r;
    const bool on = dim < d;
    qv[r] = on ? ld<BF16>(a.q, row + dim) : 0.f;
    gv[r] = on ? ld<BF16>(a.dout, row + dim) : 0.f;
    uv[r] = on ? a.U[row + dim] : 0.f;
    ev[r] = on ? a.DKB[row + dim] : 0.f;
    acc[r] = 0.f;
  }
  for (int j = lo; j < hi; ++j) {
    float kv[DPL], s = 0.f, t = 0.f, G = 0.f, E = 0.f;
#pragma unroll
    for (int r = 0; r < DPL; ++r) {
      const int dim = lane + 64 * r;
      const int64_t e = idx4(b, j, a.Tk, g, a.Hkv, d, dim);
      kv[r] = dim < d ? ld<BF16>(a.k, e) : 0.f;
      const float vv = dim < d ? ld<BF16>(a.v, e) : 0.f;
      s += qv[r] * kv[r];
      t += uv[r] * kv[r];
      G += gv[r] * vv;
      E += ev[r] * kv[r];
    }
    wave_sum4(s, t, G, E);
    const float p = expf(s * a.scale - lse_i);
    const float ds = p * (G * (t + 1.f - alpha) + E - delta);
#pragma unroll
    for (int r = 0; r < DPL; ++r) acc[r] += ds * kv[r];
  }
#pragma unroll
  for (int r = 0; r < DPL; ++r) {
    const int dim = lane + 64 * r;
    if (dim < d) a.dq[row + dim] += a.scale * acc[r];
  }
}

// ------------------- dP = sum over batch and rows of x du^T -------------------
__global__ __launch_bounds__(256) void k_bwd_dP(Args a) {
  __shared__ float part[256];
  const int bb = blockIdx.x, h = blockIdx.y;
  const int t = threadIdx.x, aa = t & 127, half = t >> 7;
  const int d = a.d;
  const int64_t R = static_cast<int64_t>(a.B) * a.Tq;
  float acc = 0.f;
  if (aa < d) {
    for (int64_t r = half; r < R; r += 2) {
      const int64_t row = (r * a.Hq + h) * d;
      acc += a.X[row + bb] * a.DU[row + aa];
    }
  }
  part[t] = acc;
  __syncthreads();
  if (half == 0 && aa < d) a.dP[(static_cast<int64_t>(h) * d + bb) * d + aa] = part[t] + part[t + 128];
}

Args make_args(const Geom& g) {
  Args a{};
  a.B = g.B;
  a.Tq = g.Tq;
  a.Tk = g.Tk;
  a.Hq = g.Hq;
  a.Hkv = g.Hkv;
  a.d = g.d;
  a.causal = g.causal;
  a.window = g.window;
  a.p_per_query = g.p_per_query;
  a.scale = g.scale;
  return a;
}

__global__ __launch_bounds__(256) void k_fill(float* p, int64_t n, float val) {
  for (int64_t e = blockIdx.x * 256LL + threadIdx.x; e < n; e += 256LL * gridDim.x) p[e] = val;
}

}  // namespace

hipError_t launch_generic_fwd(const Geom& g, const void* q, const void* k, const void* v,
                              const void* P, const int32_t* seqlens, float* out, float* lse,
                              float* kbar, float* osa, int row_begin, int row_end,
                              hipStream_t stream, bool mark, int mark_id) {
  if (row_end <= row_begin || g.B == 0) return hipSuccess;
  Args a = make_args(g);
  a.q = q;
  a.k = k;
  a.v = v;
  a.P = P;
  a.seqlens = seqlens;
  a.out = out;
  a.lse = lse;
  a.kbar = kbar;
  a.osa = osa;
  a.row_begin = row_begin;
  a.row_end = row_end;
  dim3 grid((row_end - row_begin + kWaves - 1) / kWaves, g.Hq, g.B);
  const bool two = g.d > 64;
  if (mark) mark_begin(mark_id, stream);
  if (g.bf16) {
    if (two) hipLaunchKernelGGL((k_fwd<true, 2>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((k_fwd<true, 1>), grid, dim3(256), 0, stream, a);
  } else {
    if (two) hipLaunchKernelGGL((k_fwd<false, 2>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((k_fwd<false, 1>), grid, dim3(256), 0, stream, a);
  }
  if (mark) mark_end(mark_id, stream);
  return hipGetLastError();
}

size_t generic_bwd_workspace(const Geom& g) {
  const size_t rows = static_cast<size_t>(g.B) * g.Tq * g.Hq;
  return align_up(4 * rows * g.d * sizeof(float), 256) + align_up(2 * rows * sizeof(float), 256);
}

hipError_t launch_generic_bwd(const Geom& g, const void* q, const void* k, const void* v,
                              const void* P, const float* out, const void* dout,
                              const float* lse, const float* kbar, const float* osa,
                              float* dq, float* dk, float* dv, float* dP, void* ws,
                              hipStream_t stream) {
  Args a = make_args(g);
  a.q = q;
  a.k = k;
  a.v = v;
  a.P = P;
  a.dout = dout;
  a.out_in = out;
  a.lse_in = lse;
  a.kbar_in = kbar;
  a.osa_in = osa;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dP = dP;
  const size_t rows = static_cast<size_t>(g.B) * g.Tq * g.Hq;
  float* w = static_cast<float*>(ws);
  a.X = w;
  a.DU = a.X + rows * g.d;
  a.DKB = a.DU + rows * g.d;
  a.U = a.DKB + rows * g.d;
  a.ALPHA = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                     align_up(4 * rows * g.d * sizeof(float), 256));
  a.DELTA = a.ALPHA + rows;
  const bool two = g.d > 64;
  dim3 rgrid((g.Tq + kWaves - 1) / kWaves, g.Hq, g.B);
  dim3 kgrid((g.Tk + kWaves - 1) / kWaves, g.Hkv, g.B);
  dim3 pgrid(g.d, g.Hq);
  if (g.Tq > 0 && g.B > 0) {
#define PLX_LAUNCH(KER, GRID)                                                        \
  do {                                                                               \
    if (g.bf16) {                                                                    \
      if (two) hipLaunchKernelGGL((KER<true, 2>), GRID, dim3(256), 0, stream, a);    \
      else hipLaunchKernelGGL((KER<true, 1>), GRID, dim3(256), 0, stream, a);        \
    } else {                                                                         \
      if (two) hipLaunchKernelGGL((KER<false, 2>), GRID, dim3(256), 0, stream, a);   \
      else hipLaunchKernelGGL((KER<false, 1>), GRID, dim3(256), 0, stream, a);       \
    }                                                                                \
  } while (0)
    PLX_LAUNCH(k_bwd_rows, rgrid);
    if (g.Tk > 0) {
      mark_begin(PLX_KERNEL_BWD_KEYS, stream);
      PLX_LAUNCH(k_bwd_keys, kgrid);
      mark_end(PLX_KERNEL_BWD_KEYS, stream);
    }
    PLX_LAUNCH(k_bwd_dq, rgrid);
#undef PLX_LAUNCH
  } else if (g.Tk > 0 && g.B > 0) {
    // no query rows: dk = dv = 0 (a fill kernel, so the call stays graph-capturable)
    const int64_t n = static_cast<int64_t>(g.B) * g.Tk * g.Hkv * g.d;
    const int64_t nb = (n + 255) / 256;
    const int blocks = static_cast<int>(nb < 4096 ? nb : 4096);
    hipLaunchKernelGGL(k_fill, dim3(blocks), dim3(256), 0, stream, dk, n, 0.f);
    hipLaunchKernelGGL(k_fill, dim3(blocks), dim3(256), 0, stream, dv, n, 0.f);
  }
  hipLaunchKernelGGL(k_bwd_dP, pgrid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace plx
