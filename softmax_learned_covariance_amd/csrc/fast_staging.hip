// Staging kernels of the fast path: max-abs of the inputs, then fp16 copies of
// K, V and P in the MFMA operand layouts described in fast_common.h.
#include "fast_common.h"

namespace plx {
namespace {

__global__ __launch_bounds__(64) void k_zero_max(uint32_t* maxbits) {
  if (threadIdx.x < 16) maxbits[threadIdx.x] = 0u;
}

// Blocks per tensor slice.  Every block ends in one atomicMax on the same few words, and those
// serialise in L2, so fewer and longer blocks are faster than many short ones.
constexpr int kAbsmaxBlocks = 256;

// Up to eight bf16 tensor slices, each with the maxbits slot its max |x| goes to.
struct AbsmaxJob {
  const u16* src[8];
  int64_t n[8];   // elements, a multiple of 8
  int slot[8];
  int parts;
};

// Adds the slices of `t` to the job: large tensors in two halves, so that the slices of one launch
// are about even (q and dout are G times larger than k and v).
__host__ inline void absmax_add(AbsmaxJob& j, const void* t, int64_t n, int slot, bool halve) {
  if (t == nullptr || n <= 0) return;
  const u16* p = static_cast<const u16*>(t);
  const int64_t h = halve ? (n / 16) * 8 : n;   // whole 16-byte vectors
  j.src[j.parts] = p;
  j.n[j.parts] = h;
  j.slot[j.parts++] = slot;
  if (h < n) {
    j.src[j.parts] = p + h;
    j.n[j.parts] = n - h;
    j.slot[j.parts++] = slot;
  }
}

// Max |x| of each slice (grid.y) into maxbits[slot].
__global__ __launch_bounds__(256) void k_absmax(AbsmaxJob job, uint32_t* maxbits) {
  const int part = blockIdx.y;
  const u16* src = job.src[part];
  const int64_t n = job.n[part];
  const int which = job.slot[part];
  float m = 0.f;
  if (src) {
    const int64_t nvec = n / 8;
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    // a block reads 16 KB contiguous per step, four independent 16-byte loads in flight per thread
    for (int64_t i = blockIdx.x * 1024LL + threadIdx.x; i < nvec; i += 1024LL * gridDim.x) {
      uint4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = i + 256 * u < nvec ? s4[i + 256 * u] : uint4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          m = fmaxf(m, fabsf(__uint_as_float(ws[j] << 16)));
          m = fmaxf(m, fabsf(__uint_as_float(ws[j] & 0xffff0000u)));
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float b = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(&maxbits[which], __float_as_uint(b));
  }
}

// One block per (64-key tile, kv head, batch): K16 (and V16) row tiles, K16t (and V16t) column tiles at the
// staged head dim DH (rows of D < DH zero-padded), and the Euclidean norm of every key and value row (knorm,
// vnorm [B][Hkv][Tk_pad], 0 past Tk).
template <int DH>
__global__ __launch_bounds__(256) void k_stage_kv(const u16* k, const u16* v, const uint32_t* maxbits,
                                                  _Float16* k16, _Float16* k16t, _Float16* v16t,
                                                  _Float16* v16, float* knorm, float* vnorm, int Tk, int Tk_pad,
                                                  int Hkv, int D) {
  constexpr int LD = DH + 2;   // padded LDS row (halves) for conflict-light column reads
  constexpr int NC = DH / 8;   // 16-byte chunks per row
  __shared__ _Float16 ks[kKeyTile * LD];
  __shared__ _Float16 vs[kKeyTile * LD];
  // the kv heads of one key tile are consecutive blocks, so they read the same rows together
  const int g = blockIdx.x % Hkv, kt = blockIdx.x / Hkv, b = blockIdx.z, t = threadIdx.x;
  const int key0 = kt * kKeyTile;
  const float sK = range_scale(__uint_as_float(maxbits[1]));
  const float sV = range_scale(__uint_as_float(maxbits[2]));
  // load 64 rows x NC chunks of 8 bf16, scale, store fp16 (natural order); the chunks of a row are held by
  // NC consecutive threads, which also sum the row's squares
  for (int ci = t; ci < kKeyTile * NC; ci += 256) {
    const int r = ci / NC, c = ci % NC;
    const int key = key0 + r;
    uint4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
    if (key < Tk && c * 8 < D) {
      const int64_t off = ((static_cast<int64_t>(b) * Tk + key) * Hkv + g) * D + c * 8;
      kw = *reinterpret_cast<const uint4*>(k + off);
      vw = *reinterpret_cast<const uint4*>(v + off);
    }
    const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w};
    const uint32_t vv[4] = {vw.x, vw.y, vw.z, vw.w};
    float k2 = 0.f, v2 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float k0 = __uint_as_float(kk[j] << 16), k1 = __uint_as_float(kk[j] & 0xffff0000u);
      const float v0 = __uint_as_float(vv[j] << 16), v1 = __uint_as_float(vv[j] & 0xffff0000u);
      k2 = fmaf(k0, k0, fmaf(k1, k1, k2));
      v2 = fmaf(v0, v0, fmaf(v1, v1, v2));
      ks[r * LD + c * 8 + 2 * j] = static_cast<_Float16>(k0 * sK);
      ks[r * LD + c * 8 + 2 * j + 1] = static_cast<_Float16>(k1 * sK);
      vs[r * LD + c * 8 + 2 * j] = static_cast<_Float16>(v0 * sV);
      vs[r * LD + c * 8 + 2 * j + 1] = static_cast<_Float16>(v1 * sV);
    }
#pragma unroll
    for (int o = NC / 2; o > 0; o >>= 1) {
      k2 += __shfl_xor(k2, o, 64);
      v2 += __shfl_xor(v2, o, 64);
    }
    if (c == 0 && knorm) {
      const int64_t ni = (static_cast<int64_t>(b) * Hkv + g) * Tk_pad + key;
      knorm[ni] = sqrtf(k2);
      vnorm[ni] = sqrtf(v2);
    }
  }
  __syncthreads();
  const int64_t tb = kv_tile(b, g, kt, Hkv, Tk_pad / kKeyTile, DH);
  // K16: key rows with d permuted within groups of 16
  for (int ci = t; ci < kKeyTile * NC; ci += 256) {
    const int r = ci / NC, c = ci % NC;
    f16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = ks[r * LD + 16 * (c >> 1) + perm16(8 * (c & 1) + e)];
    *reinterpret_cast<f16x8*>(k16 + tb + c * (kKeyTile * 8) + r * 8) = o;
    if (v16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = vs[r * LD + 16 * (c >> 1) + perm16(8 * (c & 1) + e)];
      *reinterpret_cast<f16x8*>(v16 + tb + c * (kKeyTile * 8) + r * 8) = o;
    }
  }
  // K16t, V16t: d rows, keys permuted within groups of 16
  for (int ci = t; ci < DH * 8; ci += 256) {
    const int d = ci >> 3, c = ci & 7;
    f16x8 ok, ov;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = 16 * (c >> 1) + perm16(8 * (c & 1) + e);
      ok[e] = ks[key * LD + d];
      ov[e] = vs[key * LD + d];
    }
    const int64_t off = tb + c * (DH * 8) + d * 8;
    *reinterpret_cast<f16x8*>(k16t + off) = ok;
    if (v16t) *reinterpret_cast<f16x8*>(v16t + off) = ov;
  }
}

// Running maximum along each series (one block per series of n floats, series `stride` apart), in place:
// x[i] = max(x[0..i]) (with SUFFIX, max(x[i..n))).  Thread t owns the t-th run of ceil(n / 256) positions in
// scan order: it takes its run's maximum, the 256 maxima are scanned (within each wave by shuffles, then
// across the four waves through LDS), and each thread rewrites its run with the running maximum started
// from the maxima of the runs before it.  The values are >= 0 (norms and their bounds).
template <bool SUFFIX>
__global__ __launch_bounds__(256) void k_scan_max(float* x, int n, int64_t stride) {
  __shared__ float wmax[4];
  float* s = x + blockIdx.x * stride;
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const int run = (n + 255) / 256;
  const int b0 = min(n, t * run), b1 = min(n, b0 + run);   // positions in scan order
  float m = 0.f;
#pragma unroll 8
  for (int i = b0; i < b1; ++i) m = fmaxf(m, s[SUFFIX ? n - 1 - i : i]);
  float inc = m;   // inclusive scan over the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(inc, o, 64);
    if (l >= o) inc = fmaxf(inc, y);
  }
  if (l == 63) wmax[w] = inc;
  __syncthreads();
  float before = __shfl_up(inc, 1, 64);
  if (l == 0) before = 0.f;
  for (int j = 0; j < w; ++j) before = fmaxf(before, wmax[j]);
#pragma unroll 8
  for (int i = b0; i < b1; ++i) {
    const int k = SUFFIX ? n - 1 - i : i;
    before = fmaxf(before, s[k]);
    s[k] = before;
  }
}

// DH / (256 / (DH / 8)) blocks per query head (8 at DH = 128, 2 at 64), each writing 256 / (DH / 8) rows a
// of P16t[h][a][b'] = sP * P[h][perm(b')][a] (and, with p16, of P16[h][a][b'] = sP * P[h][a][perm(b')]) from
// the whole projector staged in LDS (a D x D projector zero-padded to DH x DH).
template <int DH>
__global__ __launch_bounds__(256) void k_stage_p(const u16* P, const uint32_t* maxbits, _Float16* p16t,
                                                 _Float16* p16, int D) {
  constexpr int LD = DH + 2, NC = DH / 8, RPB = 256 / NC;
  __shared__ _Float16 ps[DH * LD];
  const int h = blockIdx.x, part = blockIdx.y, t = threadIdx.x;
  const float sP = range_scale(__uint_as_float(maxbits[3]));
  const u16* src = P + static_cast<int64_t>(h) * D * D;
  if (D == DH) {   // 16-byte loads (8 values) per thread
    for (int e8 = t; e8 < DH * DH / 8; e8 += 256) {
      const int r = e8 / (DH / 8), c8 = (e8 % (DH / 8)) * 8;
      const uint4 wv = *reinterpret_cast<const uint4*>(src + r * DH + c8);
      const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ps[r * LD + c8 + 2 * j] = static_cast<_Float16>(__uint_as_float(ws[j] << 16) * sP);
        ps[r * LD + c8 + 2 * j + 1] = static_cast<_Float16>(__uint_as_float(ws[j] & 0xffff0000u) * sP);
      }
    }
  } else {
    for (int e = t; e < DH * DH; e += 256) {
      const int r = e / DH, c = e % DH;
      ps[r * LD + c] = r < D && c < D ? static_cast<_Float16>(bf16_to_f32(src[r * D + c]) * sP) : static_cast<_Float16>(0.f);
    }
  }
  __syncthreads();
  const int a = RPB * part + t / NC, c = t % NC;   // one 16-byte chunk per thread
  f16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = ps[(16 * (c >> 1) + perm16(8 * (c & 1) + e)) * LD + a];
  *reinterpret_cast<f16x8*>(p16t + (static_cast<int64_t>(h) * DH + a) * DH + c * 8) = o;
  if (p16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = ps[a * LD + 16 * (c >> 1) + perm16(8 * (c & 1) + e)];
    *reinterpret_cast<f16x8*>(p16 + (static_cast<int64_t>(h) * DH + a) * DH + c * 8) = o;
  }
}

// Query-side fp16 copies in the row-tile layout [DH/8 chunks][32 rows][8] (d permuted within groups of 16,
// tiles ordered [batch][head][tile]), times the tensor's range scale, and optionally the low halves
// x - fp16(x) for rows < lo_rows (tiles of a [B][Hq][lo_pad] index space).  src is [B][Tq][Hq][row]: bf16
// caller rows of D elements (zero-padded to DH) or fp32 workspace rows of DH.  One block per 32-row tile:
// each thread reads 8 consecutive d of a row (coalesced), the two 4-d runs go through LDS to their chunks
// (a run of 4 d is a run of 4 positions), and each thread writes whole 16-byte chunks (consecutive rows of
// a chunk are contiguous).
template <bool F32, int DH>
__global__ __launch_bounds__(256) void k_stage_rows(const void* src, const uint32_t* maxbits, int max_idx,
                                                    _Float16* dst, _Float16* lo, int Tq, int Tq_pad, int Hq,
                                                    int lo_rows, int lo_pad, int D) {
  constexpr int NC = DH / 8;                  // chunks per row
  constexpr int REPS = 32 * NC / 256;         // 16-byte items per thread
  __shared__ uint2 hs[NC * 32 * 2];   // [chunk][row][half of the chunk]
  __shared__ uint2 ls[NC * 32 * 2];
  // the heads of one row tile are consecutive blocks, so they read the same rows together
  const int h = blockIdx.x % Hq, qt = blockIdx.x / Hq, b = blockIdx.z, t = threadIdx.x;
  const int r0 = qt * 32;
  const float sc = range_scale(__uint_as_float(maxbits[max_idx]));
  const bool want_lo = lo != nullptr && r0 < lo_rows;
#pragma unroll
  for (int rep = 0; rep < REPS; ++rep) {
    const int i = t + 256 * rep, r = i / NC, k = i % NC, row = r0 + r;   // d = 8 k .. 8 k + 7
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (row < Tq && (F32 || 8 * k < D)) {
      const int64_t off = ((static_cast<int64_t>(b) * Tq + row) * Hq + h) * (F32 ? DH : D) + 8 * k;
      if constexpr (F32) {
        const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + off);
        const float4 c = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + off + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
      } else {
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const u16*>(src) + off);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[2 * j] = __uint_as_float(ws[j] << 16);
          x[2 * j + 1] = __uint_as_float(ws[j] & 0xffff0000u);
        }
      }
    }
    f16x8 hi, lw;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = x[e] * sc;
      hi[e] = static_cast<_Float16>(v);
      lw[e] = static_cast<_Float16>(v - static_cast<float>(hi[e]));
    }
    // d 8k + [0,4) and 8k + [4,8) are position runs 4 (k&1) + [0,4) of chunks 2 (k/2) and 2 (k/2) + 1
    const int c0 = 2 * (k >> 1), half = k & 1;
    const uint4 hv = __builtin_bit_cast(uint4, hi), lv = __builtin_bit_cast(uint4, lw);
    hs[(c0 * 32 + r) * 2 + half] = uint2{hv.x, hv.y};
    hs[((c0 + 1) * 32 + r) * 2 + half] = uint2{hv.z, hv.w};
    if (want_lo) {
      ls[(c0 * 32 + r) * 2 + half] = uint2{lv.x, lv.y};
      ls[((c0 + 1) * 32 + r) * 2 + half] = uint2{lv.z, lv.w};
    }
  }
  __syncthreads();
  const int64_t tb = q_tile(b, h, qt, Hq, Tq_pad / kQTile, DH);
  const int64_t tbl = want_lo ? q_tile(b, h, qt, Hq, lo_pad / kQTile, DH) : 0;
#pragma unroll
  for (int rep = 0; rep < REPS; ++rep) {
    const int j = t + 256 * rep, c = j >> 5, r = j & 31;
    const uint2 a = hs[(c * 32 + r) * 2], a2 = hs[(c * 32 + r) * 2 + 1];
    *reinterpret_cast<uint4*>(dst + tb + c * (kQTile * 8) + r * 8) = uint4{a.x, a.y, a2.x, a2.y};
    if (want_lo) {
      const uint2 m = ls[(c * 32 + r) * 2], m2 = ls[(c * 32 + r) * 2 + 1];
      *reinterpret_cast<uint4*>(lo + tbl + c * (kQTile * 8) + r * 8) = uint4{m.x, m.y, m2.x, m2.y};
    }
  }
}

}  // namespace

hipError_t launch_staging(const Staging& s, const void* q, int64_t q_elems, const void* k,
                          const void* v, const void* P, int B, int Tk, int Hkv, int Hq,
                          hipStream_t stream, const void* extra, int64_t extra_elems, int extra_slot, int D) {
  const int64_t nkv = static_cast<int64_t>(B) * Tk * Hkv * D;
  const int64_t np = static_cast<int64_t>(Hq) * D * D;
  hipLaunchKernelGGL(k_zero_max, dim3(1), dim3(64), 0, stream, s.maxbits);
  AbsmaxJob job{};
  absmax_add(job, q, q_elems, kMaxQ, true);
  absmax_add(job, k, nkv, kMaxK, false);
  absmax_add(job, v, nkv, kMaxV, false);
  absmax_add(job, P, np, kMaxP, false);
  absmax_add(job, extra, extra_elems, extra_slot, true);
  if (job.parts > 0)
    hipLaunchKernelGGL(k_absmax, dim3(kAbsmaxBlocks, job.parts), dim3(256), 0, stream, job, s.maxbits);
  if (B > 0 && s.Tk_pad > 0) {
    const dim3 grid(Hkv * (s.Tk_pad / kKeyTile), 1, B);
    if (s.dh == 64)
      hipLaunchKernelGGL(k_stage_kv<64>, grid, dim3(256), 0, stream, static_cast<const u16*>(k),
                         static_cast<const u16*>(v), s.maxbits, s.k16, s.k16t, s.v16t, s.v16, s.knorm, s.vnorm, Tk,
                         s.Tk_pad, Hkv, D);
    else
      hipLaunchKernelGGL(k_stage_kv<kD>, grid, dim3(256), 0, stream, static_cast<const u16*>(k),
                         static_cast<const u16*>(v), s.maxbits, s.k16, s.k16t, s.v16t, s.v16, s.knorm, s.vnorm, Tk,
                         s.Tk_pad, Hkv, D);
    // running maxima of the key and value norms along each sequence (the two arrays are consecutive)
    hipLaunchKernelGGL(k_scan_max<false>, dim3(2 * B * Hkv), dim3(256), 0, stream, s.knorm, s.Tk_pad,
                       static_cast<int64_t>(s.Tk_pad));
  }
  if (P) {
    if (s.dh == 64)
      hipLaunchKernelGGL(k_stage_p<64>, dim3(Hq, 2), dim3(256), 0, stream, static_cast<const u16*>(P), s.maxbits,
                         s.p16t, s.p16, D);
    else
      hipLaunchKernelGGL(k_stage_p<kD>, dim3(Hq, 8), dim3(256), 0, stream, static_cast<const u16*>(P), s.maxbits,
                         s.p16t, s.p16, D);
  }
  return hipGetLastError();
}


hipError_t launch_scan_max(float* x, int n, int series, int64_t stride, bool suffix, hipStream_t stream) {
  if (series <= 0 || n <= 0) return hipSuccess;
  if (suffix)
    hipLaunchKernelGGL(k_scan_max<true>, dim3(series), dim3(256), 0, stream, x, n, stride);
  else
    hipLaunchKernelGGL(k_scan_max<false>, dim3(series), dim3(256), 0, stream, x, n, stride);
  return hipGetLastError();
}

hipError_t launch_stage_rows(const void* src, bool f32, const uint32_t* maxbits, int max_idx, _Float16* dst,
                             _Float16* lo, int B, int Tq, int Tq_pad, int Hq, int lo_rows, int lo_pad,
                             hipStream_t stream, int D, int dh) {
  if (B == 0 || Tq_pad == 0) return hipSuccess;
  dim3 grid(Hq * (Tq_pad / 32), 1, B);
  if (dh == 64) {
    if (f32)
      hipLaunchKernelGGL((k_stage_rows<true, 64>), grid, dim3(256), 0, stream, src, maxbits, max_idx, dst, lo, Tq,
                         Tq_pad, Hq, lo_rows, lo_pad, D);
    else
      hipLaunchKernelGGL((k_stage_rows<false, 64>), grid, dim3(256), 0, stream, src, maxbits, max_idx, dst, lo, Tq,
                         Tq_pad, Hq, lo_rows, lo_pad, D);
  } else {
    if (f32)
      hipLaunchKernelGGL((k_stage_rows<true, kD>), grid, dim3(256), 0, stream, src, maxbits, max_idx, dst, lo, Tq,
                         Tq_pad, Hq, lo_rows, lo_pad, D);
    else
      hipLaunchKernelGGL((k_stage_rows<false, kD>), grid, dim3(256), 0, stream, src, maxbits, max_idx, dst, lo, Tq,
                         Tq_pad, Hq, lo_rows, lo_pad, D);
  }
  return hipGetLastError();
}

}  // namespace plx
