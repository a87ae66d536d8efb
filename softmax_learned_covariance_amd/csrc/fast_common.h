// Shared pieces of the MFMA fast path (head_dim 128 or 64; bf16 inputs): operand types, the fp16 staging
// layout, power-of-two range scales and wave helpers.
//
// Staging.  The MFMA kernels compute with fp16 operands (11 significant bits)
// and fp32 accumulation.  K, V, P (and, for the backward, q, dout, u, dkbar)
// are converted once per call into fp16 copies laid out tile by tile for the
// v_mfma_f32_32x32x16_f16 operand registers.  A tile is one contiguous block
// stored "chunk-major": its 16-byte chunks (8 fp16 values) are grouped by
// chunk index, so, for a staged head dim DH (128, or 64 in the forwards' native layout)
//   key rows    [DH/8 chunks][64 keys][8] (K16, V16: d permuted within groups of 16)
//   key columns [8 chunks][DH d][8]       (K16t, V16t: keys permuted within groups of 16)
//   query rows  [DH/8 chunks][32 rows][8]
// with tiles ordered [batch][head][tile].  Copying a tile to LDS is then one
// contiguous DMA, and an MFMA operand read (32 lanes reading the same chunk of
// 32 consecutive rows) is a contiguous 512-byte LDS access: no bank conflicts,
// and the chunk index becomes an immediate offset.
//   P16t  [Hq][DH][DH]           P16t[h][a][b'] = P[h][b][a], b permuted within groups of 16
//   P16   [Hq][DH][DH]           P16[h][b][a'] = P[h][b][a], a permuted within groups of 16
// A head of 64 is staged at DH = 64 (the kernels are instantiated for both head dims).
// The permutation of a group of 16 is the involution
//   position 8*hh + e  <->  element 8*(e/4) + 4*hh + (e%4)      (hh in {0,1}, e in 0..7)
// which is exactly the order in which a 32x32 accumulator tile holds its rows
// (lane half hh, register r: row 8*(r/4) + 4*hh + r%4), so an accumulator tile
// converted to fp16 is directly the B operand of the next MFMA over that index.
//
// Range.  bf16 has fp32's exponent range, fp16 does not.  Each tensor X in
// {Q, K, V, P} is multiplied by s_X = 2^(15 - E(max|X|)) (E(m) = exponent with
// 2^(E-1) <= m < 2^E), so its largest magnitude lies in [2^14, 2^15): exact
// (a power of two), never overflows fp16 and keeps small values out of the
// subnormal range.  Per-row quantities (q - kbar, the probe u) get per-row
// scales of the same form; results are unscaled in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace plx {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16;

constexpr int kD = 128;        // largest head_dim of the fast path
constexpr int kKeyTile = 64;   // keys per LDS tile
constexpr int kQTile = 32;     // query rows per tile of the key-major backward

// First element of key tile kt of (batch b, kv head g) in K16 / V16 / K16t / V16t staged at head dim dh.
__host__ __device__ inline int64_t kv_tile(int b, int g, int kt, int Hkv, int ntiles, int dh = kD) {
  return ((static_cast<int64_t>(b) * Hkv + g) * ntiles + kt) * (kKeyTile * dh);
}
// First element of query tile qt of (batch b, query head h) in the query-side copies staged at head dim dh.
__host__ __device__ inline int64_t q_tile(int b, int h, int qt, int Hq, int nqt, int dh = kD) {
  return ((static_cast<int64_t>(b) * Hq + h) * nqt + qt) * (kQTile * dh);
}

// permuted position <-> element within a group of 16 (an involution)
__host__ __device__ constexpr int perm16(int p) { return 8 * ((p & 7) >> 2) + 4 * (p >> 3) + (p & 3); }

__device__ __forceinline__ float bf16_to_f32(u16 b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// fp32 -> bf16 bits, rounded to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Four consecutive output values at element index i of an fp32 or a bf16 output array.
__device__ __forceinline__ void store_out4(void* out, int64_t i, bool bf16, float a, float b, float c, float d) {
  if (bf16)
    *reinterpret_cast<uint2*>(static_cast<u16*>(out) + i) =
        uint2{f32_to_bf16(a) | (f32_to_bf16(b) << 16), f32_to_bf16(c) | (f32_to_bf16(d) << 16)};
  else
    *reinterpret_cast<float4*>(static_cast<float*>(out) + i) = float4{a, b, c, d};
}

// 2^(15 - E(m)) for the magnitude bound m (1 for m == 0 or non-finite m).
__device__ __forceinline__ float range_scale(float m) {
  const uint32_t bits = __float_as_uint(m);
  const int ex = static_cast<int>((bits >> 23) & 0xff);
  if (m <= 0.f || ex == 0xff) return 1.f;
  const int E = (ex == 0) ? -126 : ex - 126;   // m < 2^E (subnormals: bound by 2^-126)
  return __builtin_ldexpf(1.f, 15 - E);
}

// 15 - E(m) as an integer, so that range_scale(m) == 2^range_exp(m) (0 for m == 0 or non-finite m).
__device__ __forceinline__ int range_exp(float m) {
  const uint32_t bits = __float_as_uint(m);
  const int ex = static_cast<int>((bits >> 23) & 0xff);
  if (m <= 0.f || ex == 0xff) return 0;
  const int E = (ex == 0) ? -126 : ex - 126;
  return 15 - E;
}

// x from lane l ^ 32 combined with x (sum / max) via the gfx950 half-wave swap.
// 2^x on the FMA pipe, without the transcendental unit, for x <= 100: x = n + f with n = floor(x), 2^f
// from a degree-3 polynomial on [0, 1] fitted for the least maximum relative error (iteratively
// reweighted least squares; 7.5e-5, below fp16's rounding of 2^-11), and n added to the exponent field.
// Inputs below -60 (masked scores included) give 2^-60, which rounds to zero in fp16.
__device__ __forceinline__ float exp2_fma(float x) {
  x = fmaxf(x, -60.f);
  const float n = floorf(x);
  const float f = x - n;
  const float q = fmaf(fmaf(fmaf(0.07802428f, f, 0.22606727f), f, 0.69583362f), f, 0.99992520f);
  return __int_as_float(__float_as_int(q) + (static_cast<int>(n) << 23));
}

__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Index of the calling wave in its workgroup, known to the compiler as wave-uniform (so values and
// branches derived from it stay scalar).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6); }

__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Packs 8 floats to an fp16 x8 operand (round to nearest even).
__device__ __forceinline__ f16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5,
                                       float a6, float a7) {
  f16x8 r;
  r[0] = static_cast<_Float16>(a0);
  r[1] = static_cast<_Float16>(a1);
  r[2] = static_cast<_Float16>(a2);
  r[3] = static_cast<_Float16>(a3);
  r[4] = static_cast<_Float16>(a4);
  r[5] = static_cast<_Float16>(a5);
  r[6] = static_cast<_Float16>(a6);
  r[7] = static_cast<_Float16>(a7);
  return r;
}

// fp16 of (x - hi) for the 8 values whose rounded fp16 is hi: the low half of a hi + lo pair.
__device__ __forceinline__ f16x8 pack_lo(const float* x, f16x8 hi) {
  return pack8(x[0] - static_cast<float>(hi[0]), x[1] - static_cast<float>(hi[1]),
               x[2] - static_cast<float>(hi[2]), x[3] - static_cast<float>(hi[3]),
               x[4] - static_cast<float>(hi[4]), x[5] - static_cast<float>(hi[5]),
               x[6] - static_cast<float>(hi[6]), x[7] - static_cast<float>(hi[7]));
}

// Makes 8 fp32 values opaque to the optimiser at this point (no instruction is emitted).  A hi + lo pair is
// formed from pinned values: otherwise the compiler may fold the multiply that produced a value into the
// hi conversion and into the lo subtraction separately (a mixed-precision fma rounds the exact product
// once, a multiply followed by a conversion rounds it twice), and for a product next to the midpoint of
// two fp16 values the two roundings pick different neighbours, leaving hi + lo one fp16 step off.
__device__ __forceinline__ void pin8(float* x) {
#pragma unroll
  for (int j = 0; j < 8; ++j) asm("" : "+v"(x[j]));
}

// Sum of the 8 fp16 values of an operand, accumulated in fp32 (v_dot2 with ones).
__device__ __forceinline__ float sum8(f16x8 v, float acc) {
  const f16x2 one = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  acc = __builtin_amdgcn_fdot2(f16x2{v[0], v[1]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2(f16x2{v[2], v[3]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2(f16x2{v[4], v[5]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2(f16x2{v[6], v[7]}, one, acc, false);
  return acc;
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane l's bytes land at
// lds_base + 16 * l, so one wave instruction fills 1024 contiguous LDS bytes.  lds_base must be
// wave-uniform.  Completion is waited for with lds_dma_wait() before the barrier that publishes the data.
// The instruction is issued from inline assembly: the compiler then does not track it, and does not
// make every later LDS read (of the other buffer) wait for the copy in flight, which it cannot tell
// apart from the copy's destination.  The instruction has no register results; its address operands
// (the global address and M0, the LDS base) are read at issue.
// M0 is a register the compiler reserves for itself, so the statement leaves it as it found it: the
// old value is saved in an SGPR of the statement's own (an early-clobber output, so it shares no
// register with the inputs) and restored after the issue.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lds_base);
  uint32_t saved_m0;
  // one wait state between the M0 write and the LDS DMA that reads it (s_nop 0)
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved_m0)
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
// The same copy with the global address split into a wave-uniform base (scalar registers) and a 32-bit
// per-lane byte offset: the scalar-base addressing form, which needs no 64-bit address per lane.
__device__ __forceinline__ void lds_dma16_sbase(const void* base, uint32_t voff, void* lds_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lds_base);
  const uint64_t bv = reinterpret_cast<uintptr_t>(base);
  const uint64_t bs = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bv >> 32))) << 32) |
                      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bv)));
  uint32_t saved_m0;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved_m0)
               : "v"(voff), "s"(bs), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
// The wait is issued twice: as assembly (always kept) and as the builtin, so that the compiler also
// knows that its own loads issued before it have completed.
__device__ __forceinline__ void lds_dma_wait() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// s_waitcnt vmcnt(0) that the compiler sees (lds_dma_wait is opaque to it): placed after a kernel's
// own global loads that precede a loop, so that the loop carries no waits for them -- which at run
// time would also wait for the tile copies the compiler does not track.
__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier that publishes this wave's LDS writes only.  __syncthreads() also fences global
// memory, which makes every wave first wait for its outstanding loads -- including a tile copy that
// was started early to overlap with this phase.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Column-layout operand (lane = d = 32 mt + l % 32, 8 query rows per lane in the permuted order of
// a column tile: chunk 2 t + hh) read from a query-row tile ([16 chunks][32 rows][8]) in LDS with two
// gfx950 transpose loads.  ds_read_b64_tr_b16 transposes 4 x 4 blocks of 16-bit values within each
// group of 16 lanes: lane i of a group receives element i % 4 of the 8 bytes addressed by lane
// 4 j + i / 4, as its element j.  Source lane 4 j + a of group G therefore points at the 4
// consecutive d 16 (2 mt + G % 2) + 4 a + [0, 4) (a run of 4 positions of the row layout) of row
// 16 t + 4 (G / 2) + j (and + 8 for the second load).
__device__ __forceinline__ int tr_lane_offset(int l) {
  const int G = l >> 4, s = l & 15, j = s >> 2, a = s & 3;
  return (2 * (G & 1) + (a & 1)) * 256 + (4 * (G >> 1) + j) * 8 + 4 * (a >> 1);
}
__device__ __forceinline__ f16x8 tr_cols(const _Float16* rows, int lane_off, int mt, int t) {
  const _Float16* src = rows + lane_off + mt * 1024 + t * 128;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)src);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(src + 64));
  // whole-vector casts (a bit cast of an element of a vector is not reliable here)
  const f16x4 lo_h = __builtin_bit_cast(f16x4, lo), hi_h = __builtin_bit_cast(f16x4, hi);
  return __builtin_shufflevector(lo_h, hi_h, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The same operand from a row tile whose rows are stored XOR-swizzled per chunk: row r of chunk c sits
// in row slot r ^ 4 (c % 4).  The unswizzled tile puts the four chunks of a d tile 512 bytes apart,
// so the 16 lanes of a group, which read two chunks, meet in the same banks (and 32 lanes, four
// chunks, four times); with the swizzle every lane of a transpose load hits its own banks.  Returns
// the lane's element offsets of the first load (rows r) and the second (rows r + 8).
__device__ __forceinline__ int2 tr_lane_offsets_swz(int l) {
  const int G = l >> 4, s = l & 15, j = s >> 2, a = s & 3;
  const int c = 2 * (G & 1) + (a & 1), r = 4 * (G >> 1) + j, x = 4 * c;
  return int2{c * 256 + (r ^ x) * 8 + 4 * (a >> 1), c * 256 + ((r + 8) ^ x) * 8 + 4 * (a >> 1)};
}
__device__ __forceinline__ f16x8 tr_cols_swz(const _Float16* rows, int2 lane_off, int mt, int t) {
  const _Float16* base = rows + mt * 1024 + t * 128;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(base + lane_off.x));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(base + lane_off.y));
  const f16x4 lo_h = __builtin_bit_cast(f16x4, lo), hi_h = __builtin_bit_cast(f16x4, hi);
  return __builtin_shufflevector(lo_h, hi_h, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Row slot of row r of chunk c in a swizzled row tile (an involution: also the row held by slot r).
__device__ __forceinline__ int row_slot_swz(int r, int c) { return r ^ (4 * (c & 3)); }

// Row-vector transfers between memory and the accumulator layout (register 4 j + e of d tile mt is d =
// 32 mt + 8 j + 4 hh + e of row ql) through a wave-private LDS block of 32 rows x kWR floats: a 32-wide d
// tile of the wave's 32 rows moves as eight rows of 128 contiguous bytes per instruction, instead of 16
// bytes of each of 32 rows.  Rows at or past row_end read as zeros and are not written.
constexpr int kWR = 36;   // LDS row stride in floats
struct WaveRows {
  float* lds;             // the wave's 32 x kWR floats
  int64_t base;           // element offset of (row i0, d 0); rows are rstride elements apart
  int64_t rstride;
  int nrows;              // rows of the wave that exist (i0 + r < row_end)
  int l, ql, hh;

  __device__ __forceinline__ void lds_sync() const { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
  // tile mt of an fp32 array (F32) or a bf16 array into v
  template <bool F32>
  __device__ __forceinline__ void load(const void* src, int mt, float (&v)[16]) const {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int rr = 8 * it + (l >> 3), c4 = 4 * (l & 7);
      float4 x = {0.f, 0.f, 0.f, 0.f};
      if (rr < nrows) {
        const int64_t o = base + rr * rstride + 32 * mt + c4;
        if constexpr (F32) {
          x = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + o);
        } else {
          const uint2 g = *reinterpret_cast<const uint2*>(static_cast<const u16*>(src) + o);
          x = float4{__uint_as_float(g.x << 16), __uint_as_float(g.x & 0xffff0000u), __uint_as_float(g.y << 16),
                     __uint_as_float(g.y & 0xffff0000u)};
        }
      }
      *reinterpret_cast<float4*>(lds + rr * kWR + c4) = x;
    }
    lds_sync();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 y = *reinterpret_cast<const float4*>(lds + ql * kWR + 8 * j + 4 * hh);
      v[4 * j] = y.x;
      v[4 * j + 1] = y.y;
      v[4 * j + 2] = y.z;
      v[4 * j + 3] = y.w;
    }
    lds_sync();
  }
  // v as tile mt of an fp32 array, or (BF16) of a bf16 array (rounded to nearest even)
  template <bool BF16 = false>
  __device__ __forceinline__ void store(void* dst, int mt, const float (&v)[16]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(lds + ql * kWR + 8 * j + 4 * hh) = float4{v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
    lds_sync();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int rr = 8 * it + (l >> 3), c4 = 4 * (l & 7);
      const float4 x = *reinterpret_cast<const float4*>(lds + rr * kWR + c4);
      if (rr < nrows) {
        const int64_t o = base + rr * rstride + 32 * mt + c4;
        if constexpr (BF16)
          *reinterpret_cast<uint2*>(static_cast<u16*>(dst) + o) =
              uint2{f32_to_bf16(x.x) | (f32_to_bf16(x.y) << 16), f32_to_bf16(x.z) | (f32_to_bf16(x.w) << 16)};
        else
          *reinterpret_cast<float4*>(static_cast<float*>(dst) + o) = x;
      }
    }
    lds_sync();
  }
};

// ---- staging buffers inside the caller's workspace ----
// Slots of the max-abs array (float bits; non-negative floats order like their bits).
enum MaxSlot { kMaxQ = 0, kMaxK = 1, kMaxV = 2, kMaxP = 3, kMaxDO = 4, kMaxU = 5, kMaxDKB = 6, kMaxDelta = 7,
               kMaxAlpha = 8, kMaxRho = 9 };

struct Staging {
  uint32_t* maxbits;   // [16] max-abs values, see MaxSlot
  _Float16* k16;
  _Float16* k16t;
  _Float16* v16t;      // forward only (nullptr otherwise)
  _Float16* v16;       // backward only: V rows, d permuted (nullptr otherwise)
  _Float16* p16t;
  _Float16* p16;       // backward only: P rows, columns permuted (nullptr otherwise)
  float* knorm;        // [B][Hkv][Tk_pad]: running maximum over keys 0..j of |k_j| (Euclidean, unscaled)
  float* vnorm;        // the same for |v_j|; directly after knorm
  int Tk_pad;
  int dh;              // staged head dim (128 or 64)
  size_t bytes;        // total workspace used
};

inline size_t ws_take(size_t& off, size_t n) {
  const size_t at = off;
  off += (n + 255) / 256 * 256;
  return at;
}

// Staging buffers at the start of `ws` (ws may be nullptr to size them), for head dim dh.
inline Staging staging_layout(void* ws, int B, int Tk, int Hkv, int Hq, bool backward = false, int dh = kD) {
  Staging s{};
  s.Tk_pad = (Tk + kKeyTile - 1) / kKeyTile * kKeyTile;
  s.dh = dh;
  const size_t kv = static_cast<size_t>(B) * s.Tk_pad * Hkv * dh * sizeof(_Float16);
  const size_t p = static_cast<size_t>(Hq) * dh * dh * sizeof(_Float16);
  char* base = static_cast<char*>(ws);
  size_t off = 0;
  s.maxbits = reinterpret_cast<uint32_t*>(base + ws_take(off, 256));
  s.k16 = reinterpret_cast<_Float16*>(base + ws_take(off, kv));
  s.k16t = reinterpret_cast<_Float16*>(base + ws_take(off, kv));
  if (backward) s.v16 = reinterpret_cast<_Float16*>(base + ws_take(off, kv));
  else s.v16t = reinterpret_cast<_Float16*>(base + ws_take(off, kv));
  s.p16t = reinterpret_cast<_Float16*>(base + ws_take(off, p));
  if (backward) s.p16 = reinterpret_cast<_Float16*>(base + ws_take(off, p));
  const size_t nrm = static_cast<size_t>(B) * Hkv * s.Tk_pad * sizeof(float);
  s.knorm = reinterpret_cast<float*>(base + ws_take(off, 2 * nrm));
  s.vnorm = s.knorm + static_cast<size_t>(B) * Hkv * s.Tk_pad;
  s.bytes = off;
  return s;
}

// In-place running maximum (suffix: from the end) along `series` series of n floats, `stride` apart.
hipError_t launch_scan_max(float* x, int n, int series, int64_t stride, bool suffix, hipStream_t stream);

// Query-side fp16 copies in the row-tile layout at head dim dh (see k_stage_rows in fast_staging.hip).
hipError_t launch_stage_rows(const void* src, bool f32, const uint32_t* maxbits, int max_idx, _Float16* dst,
                             _Float16* lo, int B, int Tq, int Tq_pad, int Hq, int lo_rows, int lo_pad,
                             hipStream_t stream, int D, int dh);   // D: row length of a bf16 src (fp32 src rows are dh)

// Launches the staging kernels: max-abs of q (rows [0, Tq)), k, v, P (and of one more bf16 tensor,
// `extra`, into maxbits[extra_slot]) in one launch, then the fp16 copies.  q may be nullptr (decode
// stages q itself).
hipError_t launch_staging(const Staging& s, const void* q, int64_t q_elems, const void* k,
                          const void* v, const void* P, int B, int Tk, int Hkv, int Hq,
                          hipStream_t stream, const void* extra = nullptr, int64_t extra_elems = 0,
                          int extra_slot = 0, int D = kD);   // D: head dim of k, v, P (zero-padded to s.dh)

}  // namespace plx
