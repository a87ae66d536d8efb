/*
 * parallax.h -- C ABI of the Parallax attention operator for AMD Instinct MI355X (gfx950).
 *
 * The operator (gist.science technical summary of "Parallax: Parameterized Local
 * Linear Attention for Language Modeling", section "Core mechanism": softmax
 * attention plus the softmax-weighted key/value covariance applied to a probe
 * vector; the probe comes from a learned projector instead of the per-query
 * linear solve of exact local linear attention).  Per batch b, query head h
 * (key/value head g = h / (heads_q / heads_kv)) and query row i:
 *
 *   p_ij   = softmax_j (scale * q_i . k_j)      over the keys j visible to i
 *   o_i    = sum_j p_ij v_j                      kbar_i = sum_j p_ij k_j
 *   u_i    = P_h^T (q_i - kbar_i)                u_i[a] = sum_b P_h[b][a] (q_i - kbar_i)[b]
 *   out_i  = o_i + sum_j p_ij (u_i . (k_j - kbar_i)) (v_j - o_i)
 *
 * P = 0 gives plain softmax attention (encorp.ai blog, "Parallax keeps softmax"
 * and its FAQ).  The probe's form u = P^T (q - kbar) with one d x d projector
 * per query head is this library's reading of "a learned map produces the probe".
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates no device memory; scratch space is the caller's `workspace`.
 *   - Tensors are dense and contiguous in the layouts stated per argument
 *     (row-major, last index fastest).  Inputs q, k, v, P, dout have the dtype
 *     `desc->dtype` (fp32 or bf16); every output is fp32.
 *   - Masks are bottom-right aligned: with off = seqlen_k - seqlen_q, key j is
 *     visible to query i iff (!causal || j <= i + off) && (window <= 0 ||
 *     j > i + off - window).  A row that sees no key gets out = o = kbar = 0 and
 *     lse = -inf.
 *   - Arguments are validated before anything is launched; on any error status
 *     nothing is launched and no output is written.  parallax_last_error()
 *     then returns a description (thread-local).
 *   - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL is
 *     the default stream).  Faults during execution surface at the caller's next
 *     synchronisation, not as a status here.  Every call is safe from several
 *     threads.
 *   - State kept between calls: the thread-local profiling hook below, and per
 *     device one helper stream (non-blocking, default priority) with two events,
 *     created by the first forward or backward on that device that uses it and
 *     kept until the process ends.  The forward and backward run their small
 *     first-row kernels on it, ordered after everything the call enqueued on
 *     `hip_stream` before them; before the call returns, `hip_stream` is made to
 *     wait for them, so later work on `hip_stream` sees the call complete, as
 *     with any single-stream call.  Calls on different caller
 *     streams or threads share the helper stream, so their side kernels can run
 *     one after another; this orders work and never changes a result.  If the
 *     helper stream cannot be created, everything runs on `hip_stream`.
 */
#ifndef PARALLAX_H
#define PARALLAX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PARALLAX_ABI_VERSION 5

typedef enum {
  PLX_OK = 0,
  PLX_ERR_INVALID = 1,      /* null pointer, negative size, heads_q % heads_kv != 0, ... */
  PLX_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. head_dim > 128) */
  PLX_ERR_WORKSPACE = 3,    /* workspace_bytes smaller than the matching *_workspace() query */
  PLX_ERR_HIP = 4           /* a HIP launch call returned an error */
} plx_status;

typedef enum { PLX_F32 = 0, PLX_BF16 = 1 } plx_dtype;

typedef struct {
  int32_t batch;          /* B  >= 0 */
  int32_t seqlen_q;       /* Tq >= 0 (decode: must be 1) */
  int32_t seqlen_k;       /* Tk >= 0 (decode: cache capacity Lmax) */
  int32_t heads_q;        /* Hq >= 1 */
  int32_t heads_kv;       /* Hkv >= 1, Hq % Hkv == 0; query head h uses key/value head h / (Hq/Hkv) */
  int32_t head_dim;       /* d, 1..128 (bf16 with d = 128 or 64 runs the MFMA paths; other d and fp32 the generic fp32 kernels) */
  int32_t causal;         /* nonzero: bottom-right aligned causal mask (ignored by decode) */
  int32_t window;         /* <= 0: no window; > 0: keep only the `window` newest visible keys (the query's own included) */
  float   softmax_scale;  /* <= 0 selects 1/sqrt(head_dim) */
  int32_t dtype;          /* plx_dtype of q, k, v, P, dout */
  int32_t p_per_query;    /* 0: P is [Hq][d][d]; 1: P is [B][Tq][Hq][d][d] (forward only) */
  int32_t split_rows;     /* bf16 fast path: the first max(split_rows, 16) query rows that see a key (causal with Tq > Tk: counted from row Tq - Tk) use hi + lo fp16 operand pairs (about 22 bits); < 0 selects the default, 256 */
  int32_t out_dtype;      /* plx_dtype of `out` in the forwards and decodes (0 = PLX_F32). PLX_BF16 (rounded to
                             nearest even from the fp32 result) needs the bf16 fast path; the backwards read
                             an fp32 `out` and require PLX_F32 */
} plx_attn_desc;

/* Kernels the profiling hook can bracket. */
typedef enum {
  PLX_KERNEL_FWD = 0,          /* forward: the fused two-pass MFMA kernel (generic kernel on the fp32 path) */
  PLX_KERNEL_BWD_ROWS = 1,     /* backward: query-major kernel (du, dkbar, Delta, P du) */
  PLX_KERNEL_BWD_KEYS = 2,     /* backward: key-major kernel (dk, dv, ds); the generic key kernel on the fp32 path */
  PLX_KERNEL_DECODE_PASS1 = 3, /* decode: first split-KV pass (generic kernel on the fp32 path) */
  PLX_KERNEL_DECODE_PASS2 = 4, /* decode: second split-KV pass */
  PLX_KERNEL_BWD_DQ = 5,       /* backward: dq = P du + scale ds K from the stored ds (bf16 fast path) */
  PLX_KERNEL_FWD_PROBE = 6,    /* probe-form forward: the one-pass MFMA kernel */
  PLX_KERNEL_DECODE_MOMENT = 7 /* decode: the single-read kernel (one read of the cache, key/value moment on MFMA) */
} plx_kernel;

/*
 * Profiling hook.  While set, calls made on this thread record `before` (a
 * hipEvent_t) on their stream immediately before launching the kernel
 * `kernel` (a plx_kernel) and `after` immediately after it, so the caller can
 * time that one kernel with hipEventElapsedTime.  Calls that do not launch that
 * kernel record nothing.  Pass NULL, NULL to turn it off.  The setting is
 * thread-local.
 */
void parallax_set_kernel_events(int kernel, void* before, void* after);

/* Decode paths (parallax_set_decode_path). */
typedef enum {
  PLX_DECODE_AUTO = 0,     /* the single-read kernel where it applies (see parallax_attn_decode), else two-pass */
  PLX_DECODE_TWO_PASS = 1  /* always the two-pass split-KV kernels (for comparison and timing) */
} plx_decode_path;

/*
 * Selects the decode path for every later decode call of the process (all threads, all devices; the
 * default is PLX_DECODE_AUTO).  Both paths compute the same operator to the bf16 tolerance; their results
 * are not bit-identical.  Returns PLX_ERR_INVALID for a value outside plx_decode_path.
 */
plx_status parallax_set_decode_path(int32_t path);

/* Library version of this header's ABI (PARALLAX_ABI_VERSION). */
int parallax_abi_version(void);

/* Static description of a status code. */
const char* parallax_status_string(plx_status s);

/* Thread-local detail of the last non-OK status returned on this thread ("" if none). */
const char* parallax_last_error(void);

/*
 * Forward.  Bytes of workspace needed for `desc` (0 if none); returns 0 for an invalid desc.
 */
size_t parallax_attn_fwd_workspace(const plx_attn_desc* desc);

/*
 * Forward: the output equation above for every query row.
 *   q     [B][Tq][Hq][d]              k, v  [B][Tk][Hkv][d]
 *   P     [Hq][d][d], or [B][Tq][Hq][d][d] when desc->p_per_query
 *   out   [B][Tq][Hq][d] fp32, or bf16 when desc->out_dtype is PLX_BF16 (required)
 *   lse   [B][Hq][Tq]    fp32, natural-log softmax denominator of the scaled scores (nullable)
 *   kbar  [B][Tq][Hq][d] fp32 softmax-weighted key mean (nullable)
 *   o_sa  [B][Tq][Hq][d] fp32 softmax-attention output o (nullable)
 *   cor   [B][Hq][Tq]    fp32 correction-to-output ratio |out_i - o_i| / |out_i| (Euclidean norms over
 *                        d, from the fp32 result; 0 where out_i = 0), the pages' diagnostic of how much the
 *                        covariance branch moves the output (nullable; bf16 fast path only)
 * The backward needs lse, kbar and o_sa from the same call, and an fp32 out.
 */
plx_status parallax_attn_fwd(const plx_attn_desc* desc,
                             const void* q, const void* k, const void* v, const void* P,
                             void* out, float* lse, float* kbar, float* o_sa, float* cor,
                             void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Probe-form forward.  Bytes of workspace needed for `desc` (0 if none); returns 0 for an
 * invalid desc.
 */
size_t parallax_attn_fwd_probe_workspace(const plx_attn_desc* desc);

/*
 * Probe-form forward: the pages' own statement of the output (gist.science technical
 * summary, "Core mechanism"; the intensity argument of its "Hardware-aware algorithm"
 * section), with the probe rho_i supplied per query row instead of built from P:
 *
 *   out_i = o_i - Sigma_i rho_i,   Sigma_i = sum_j p_ij (v_j - o_i)(k_j - kbar_i)^T
 *         = o_i - sum_j p_ij (rho_i . (k_j - kbar_i)) (v_j - o_i)
 *
 * (the forward above with u_i = -rho_i).  rho_i = W_R x_i is the caller's projection of the
 * layer input.  Because rho does not depend on kbar, one pass over the keys suffices.
 *   q, rho [B][Tq][Hq][d]     k, v [B][Tk][Hkv][d]     dtype desc->dtype
 *   out    [B][Tq][Hq][d] fp32, or bf16 when desc->out_dtype is PLX_BF16 (required)
 *   lse    [B][Hq][Tq]    fp32 as in the forward (nullable)
 *   o_sa   [B][Tq][Hq][d] fp32 softmax-attention output o (nullable)
 *   rk     [B][Hq][Tq]    fp32 rho_i . kbar_i (nullable)
 *   cor    [B][Hq][Tq]    fp32 correction-to-output ratio as in the forward (nullable)
 * The probe-form backward needs lse, o_sa and rk from the same call.
 * Supported: bf16, head_dim 128 or 64, heads_q / heads_kv in {1, 2, 4, 8}, p_per_query 0; any other
 * valid desc returns PLX_ERR_UNSUPPORTED.  Masks, empty rows and split_rows as in the forward.
 */
plx_status parallax_attn_fwd_probe(const plx_attn_desc* desc,
                                   const void* q, const void* k, const void* v, const void* rho,
                                   void* out, float* lse, float* o_sa, float* rk, float* cor,
                                   void* workspace, size_t workspace_bytes, void* hip_stream);

/* Probe-form backward.  Bytes of workspace needed for `desc`; returns 0 for an invalid desc. */
size_t parallax_attn_bwd_probe_workspace(const plx_attn_desc* desc);

/*
 * Probe-form backward: gradients of sum(dout * out) of parallax_attn_fwd_probe.  The pages give
 * no backward; this is the chain rule of that forward with rho an input:
 *   drho_i = (g_i.o_i) kbar_i - sum_j p_ij (g_i.v_j) k_j      (g = dout)
 * and dq, dk, dv as in the backward above with u_i = -rho_i and no projector term.
 *   q, k, v, rho        as in the probe-form forward
 *   out, lse, o_sa, rk  that forward's outputs for the same inputs (all required)
 *   dout  [B][Tq][Hq][d]   dtype desc->dtype
 *   dq, drho [B][Tq][Hq][d] fp32     dk, dv [B][Tk][Hkv][d] fp32 (summed over the query heads of each group)
 * Every gradient is overwritten.  Results are deterministic.
 * Supported: bf16, head_dim 128 or 64, heads_q / heads_kv in {1, 2, 4, 8}, p_per_query 0; any other
 * valid desc returns PLX_ERR_UNSUPPORTED.  Empty problems write zero gradients.
 */
plx_status parallax_attn_bwd_probe(const plx_attn_desc* desc,
                                   const void* q, const void* k, const void* v, const void* rho,
                                   const float* out, const void* dout,
                                   const float* lse, const float* o_sa, const float* rk,
                                   float* dq, float* dk, float* dv, float* drho,
                                   void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Backward.  Bytes of workspace needed for `desc`; returns 0 for an invalid desc.
 * On the bf16 fast path the workspace holds, besides O(B*T*H*d) staging copies, one fp16 value per
 * visible (query, key) pair and query head: the key-major kernel stores its ds tiles for the
 * query-major dq kernel.  The size therefore grows as 2 * B * Hq * Tq_pad * Tk_pad bytes (Tq_pad, Tk_pad:
 * Tq, Tk rounded up to 32 and 64): about 4.3 GB at B = 2, Hq = 16, T = 8192, and 137 GB at B = 1, Hq = 16,
 * T = 65536.  Callers that cannot provide it can split the batch or the heads over several calls.
 */
size_t parallax_attn_bwd_workspace(const plx_attn_desc* desc);

/*
 * Backward: gradients of sum(dout * out).  The pages give no backward; this is
 * the chain rule of the forward definition.
 *   q, k, v, P        as in the forward (p_per_query must be 0)
 *   out, lse, kbar, o_sa   the forward's outputs for the same inputs (all required)
 *   dout  [B][Tq][Hq][d]   dtype desc->dtype
 *   dq    [B][Tq][Hq][d] fp32     dk, dv [B][Tk][Hkv][d] fp32 (summed over the query heads of each group)
 *   dP    [Hq][d][d] fp32 (summed over batch and rows; same orientation as P)
 * Every gradient is overwritten (not accumulated).  Results are deterministic.
 */
plx_status parallax_attn_bwd(const plx_attn_desc* desc,
                             const void* q, const void* k, const void* v, const void* P,
                             const float* out, const void* dout,
                             const float* lse, const float* kbar, const float* o_sa,
                             float* dq, float* dk, float* dv, float* dP,
                             void* workspace, size_t workspace_bytes, void* hip_stream);

/* Decode.  Bytes of workspace needed for `desc`; returns 0 for an invalid desc. */
size_t parallax_attn_decode_workspace(const plx_attn_desc* desc);

/*
 * Decode: T = desc->seqlen_q new queries per sequence against a key/value cache (the
 * decode path of the pages' hardware section; T > 1 for speculative or chunked
 * decoding).  The new tokens' keys and values are already the last T entries of their
 * sequence, so new token t of sequence b sees cache rows [max(0, e - window), e) with
 * e = L_b - (T - 1 - t) and L_b = seqlens_k[b] (or Lmax when seqlens_k is NULL).
 * desc->seqlen_k is Lmax, desc->causal is ignored, desc->p_per_query must be 0.
 * seqlens_k values are clamped to [0, Lmax]; a token that sees no key gets out = 0.
 * T > 1 needs the bf16 fast path (else PLX_ERR_UNSUPPORTED).
 *   q        [B][T][Hq][d] (for T = 1 also read as [B][Hq][d])
 *   k_cache, v_cache [B][Lmax][Hkv][d]
 *   seqlens_k [B] int32 device array (nullable)
 *   P        [Hq][d][d]            out [B][T][Hq][d] fp32, or bf16 when desc->out_dtype is PLX_BF16
 *   cor      [B][T][Hq] fp32 correction-to-output ratio as in the forward (nullable; bf16 fast path only)
 * Kernels.  With T = 1, bf16, head_dim 128, heads_q / heads_kv of 1 or 2 and at least 256 (sequence, kv
 * head) pairs, one workgroup per pair reads its cache rows once: it accumulates o, kbar and the
 * softmax-weighted moment sum_j p_j v_j k_j^T (fp16 products with power-of-two scales, fp32 sums, on the
 * matrix cores) and forms the correction from them, c = (sum_j p_j v_j k_j^T) u - (u.kbar) o; no
 * workspace is used.  A head where the two terms exceed the output by more than 2^11 (a key far larger
 * than the rest dominating the softmax) has its correction formed directly from a second read of its keys.
 * Otherwise (or with PLX_DECODE_TWO_PASS) two split-KV passes run: o and kbar first, the correction with the
 * finished u second.
 */
plx_status parallax_attn_decode(const plx_attn_desc* desc,
                                const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* seqlens_k, const void* P, void* out, float* cor,
                                void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Paged decode.  Bytes of workspace needed for `desc` (the same as parallax_attn_decode's); returns 0
 * for an invalid or unsupported desc.
 */
size_t parallax_attn_decode_paged_workspace(const plx_attn_desc* desc);

/*
 * Decode against a paged key/value cache (serving caches that grow page by page; the pages' decode
 * benchmark spans batch sizes and context lengths): the same result as parallax_attn_decode on the
 * sequences the block table describes.  Key j of sequence b is slot j % page_size of page
 * block_table[b][j / page_size].
 *   q            [B][T][Hq][d], T = desc->seqlen_q  dtype desc->dtype
 *   k_pages, v_pages [num_pages][page_size][Hkv][d]   dtype desc->dtype
 *   block_table  [B][block_table_stride] int32 device array: row b lists the pages of sequence b;
 *                only the entries that cover keys < seqlens_k[b] are read
 *   block_table_stride  entries per row of block_table (a table sized for the cache's capacity may be
 *                wider than the sequences need); must be >= ceil(desc->seqlen_k / page_size), else
 *                PLX_ERR_INVALID
 *   seqlens_k    [B] int32 device array (nullable: every sequence has desc->seqlen_k keys)
 *   P [Hq][d][d]     out [B][T][Hq][d] fp32 (bf16 when desc->out_dtype is PLX_BF16)     cor [B][T][Hq] (nullable)
 * New tokens as in parallax_attn_decode; desc->seqlen_k is the longest sequence the table can describe.
 * page_size must be a power of two (1 .. 65536) and num_pages >= 1.  Block-table entries outside
 * [0, num_pages) are clamped into the pool: that sequence's output is then wrong, but nothing is
 * read outside the caller's arrays.
 * Supported: bf16, head_dim 128 or 64, heads_q / heads_kv in {1, 2, 4, 8}, p_per_query 0; any other
 * valid desc returns PLX_ERR_UNSUPPORTED.  window as in parallax_attn_decode.  The single-read kernel (see
 * parallax_attn_decode) runs here too when page_size >= 64.
 */
plx_status parallax_attn_decode_paged(const plx_attn_desc* desc, const void* q,
                                      const void* k_pages, const void* v_pages,
                                      int32_t num_pages, int32_t page_size,
                                      const int32_t* block_table, int32_t block_table_stride,
                                      const int32_t* seqlens_k,
                                      const void* P, void* out, float* cor,
                                      void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * No-allocation decode, for callers that cannot allocate device memory or pass a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.  Same arguments, results
 * and kernels as parallax_attn_decode (bit-identical outputs), without the workspace: its scratch is a
 * fixed device array inside the library, parallax_attn_decode_noalloc_max_scratch() bytes (64 MiB) on
 * each GPU it runs on, held until the process ends.  A desc whose decode needs more scratch than that
 * (parallax_attn_decode_workspace(desc) > the maximum) returns PLX_ERR_WORKSPACE and launches nothing.
 * The call allocates nothing (no hipMalloc, no allocating library routine); the first call on a device
 * looks the array's address up once.  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (on different streams, or from several threads) race on it and give undefined
 * results; calls ordered on one stream are safe.  The kernels overwrite every scratch value they read,
 * so no clearing is needed between calls.
 */
size_t parallax_attn_decode_noalloc_max_scratch(void);

plx_status parallax_attn_decode_noalloc(const plx_attn_desc* desc,
                                        const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* seqlens_k, const void* P, void* out, float* cor,
                                        void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* PARALLAX_H */
