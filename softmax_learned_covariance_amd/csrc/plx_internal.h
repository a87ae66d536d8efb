// Internal declarations shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "parallax.h"

namespace plx {

// Problem geometry after validation (all counts are non-negative, Hq % Hkv == 0).
struct Geom {
  int B, Tq, Tk, Hq, Hkv, d;
  int causal, window;
  float scale;
  int bf16;          // 1: inputs are bf16, 0: fp32
  int p_per_query;
  int out_bf16;      // 1: `out` of the forwards and decodes is bf16 (fast paths only)
};

// Query rows that see no key: with a causal mask (bottom-right aligned) and more query rows than keys, the
// rows below Tq - Tk.  split_rows counts rows from the first one that sees a key, since the rows that see
// only a handful of keys are the ones that need hi + lo operand pairs.
inline int rows_without_keys(const Geom& g) { return g.causal && g.Tq > g.Tk ? g.Tq - g.Tk : 0; }

// bf16 fast path: the first query rows see only a few keys, and their correction terms cancel
// badly in single fp16 operands (max|err|/rms near 4e-2 in the first rows' dq and the first
// keys' dk when they do).  Rows below this bound always take the hi + lo operand pairs, whatever
// split the caller asks for.
constexpr int kMinSplitRows = 16;


// ---- generic kernels: fp32 arithmetic on fp32 or bf16 inputs, any head_dim <= 128 ----

// Forward rows [row_begin, row_end) of every (batch, query head).  seqlens (nullable)
// overrides Tk per batch (decode); q/out/kbar/osa row stride is Hq*d, lse is [B][Hq][Tq].
hipError_t launch_generic_fwd(const Geom& g, const void* q, const void* k, const void* v,
                              const void* P, const int32_t* seqlens, float* out, float* lse,
                              float* kbar, float* osa, int row_begin, int row_end,
                              hipStream_t stream, bool mark, int mark_id = PLX_KERNEL_FWD);

// Workspace of the generic backward in bytes.
size_t generic_bwd_workspace(const Geom& g);

hipError_t launch_generic_bwd(const Geom& g, const void* q, const void* k, const void* v,
                              const void* P, const float* out, const void* dout,
                              const float* lse, const float* kbar, const float* osa,
                              float* dq, float* dk, float* dv, float* dP, void* ws,
                              hipStream_t stream);

// ---- bf16 MFMA fast path (head_dim 128) ----
// Probe form (the caller supplies rho per query row): out = o - Sigma_KV rho, one pass over K/V.
bool fast_probe_supported(const Geom& g);
size_t fast_probe_workspace(const Geom& g);
hipError_t launch_fast_probe(const Geom& g, const void* q, const void* k, const void* v, const void* rho,
                             void* out, float* lse, float* osa, float* rk, float* cor, int split_rows, void* ws,
                             hipStream_t stream);
// Its backward (u = -rho, no projector): dq, dk, dv and drho.
bool fast_probe_bwd_supported(const Geom& g);
size_t fast_probe_bwd_workspace(const Geom& g);
hipError_t launch_fast_probe_bwd(const Geom& g, const void* q, const void* k, const void* v, const void* rho,
                                 const float* out, const void* dout, const float* lse, const float* osa,
                                 const float* rk, float* dq, float* dk, float* dv, float* drho, int split_rows,
                                 void* ws, hipStream_t stream);
hipError_t launch_zero_f32(float* x, int64_t n, hipStream_t stream);   // n a multiple of 4

bool fast_fwd_supported(const Geom& g);
size_t fast_fwd_workspace(const Geom& g);
hipError_t launch_fast_fwd(const Geom& g, const void* q, const void* k, const void* v,
                           const void* P, void* out, float* lse, float* kbar, float* osa, float* cor,
                           int split_rows, void* ws, hipStream_t stream);

bool fast_bwd_supported(const Geom& g);
size_t fast_bwd_workspace(const Geom& g);
hipError_t launch_fast_bwd(const Geom& g, const void* q, const void* k, const void* v,
                           const void* P, const float* out, const void* dout,
                           const float* lse, const float* kbar, const float* osa,
                           float* dq, float* dk, float* dv, float* dP, int split_rows, void* ws,
                           hipStream_t stream);

bool fast_decode_supported(const Geom& g);
size_t fast_decode_workspace(const Geom& g);
// A paged key/value cache: pages [num_pages][page_size][Hkv][d] (page_size a power of two) and a block
// table [B][max_pages] of page indices; max_pages is the table's row stride, >= ceil(L / page_size).
struct PagedCache {
  const int32_t* block_table;
  int num_pages, page_size, max_pages;
};
hipError_t launch_fast_decode(const Geom& g, const void* q, const void* kc, const void* vc,
                              const int32_t* seqlens, const void* P, void* out, float* cor, void* ws,
                              hipStream_t stream, const PagedCache* paged = nullptr);
// Single-read decode: one workgroup per (sequence, kv head) reads the cache once and accumulates the
// softmax-weighted key/value moment on the matrix cores; no workspace.  Applies to bf16, d = 128, one new
// token, 1 or 2 query heads per kv head, at least 256 (sequence, kv head) pairs, pages of >= 64 keys.
// launch_fast_decode takes it by itself where it applies, unless the two-pass path is forced.
bool moment_decode_supported(const Geom& g, const PagedCache* paged);
hipError_t launch_moment_decode(const Geom& g, const void* q, const void* kc, const void* vc, const int32_t* seqlens,
                                const void* P, void* out, float* cor, hipStream_t stream, const PagedCache* paged);
// The decode path in force (a plx_decode_path value; parallax_set_decode_path sets it for the process).
int decode_path();

// Records the profiling hook's `before` / `after` event on `stream` when `kernel` (a plx_kernel)
// is the one selected (no-op otherwise).
void mark_begin(int kernel, hipStream_t stream);
void mark_end(int kernel, hipStream_t stream);

// A second lane of work beside the caller's stream: small kernels that do not depend on the
// main kernel running at the same time go there.  side_fork makes the helper stream wait for
// everything enqueued on `main` so far; side_join makes `main` wait for everything enqueued on the
// helper stream so far.  Without a helper stream (creation failed) `stream` is `main` itself.
struct SideLane {
  hipStream_t stream;
  hipStream_t main;
};
SideLane side_fork(hipStream_t main);
hipError_t side_join(const SideLane& lane);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace plx
