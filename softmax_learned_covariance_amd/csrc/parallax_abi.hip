// C ABI of the Parallax attention library: argument validation, workspace sizing,
// and dispatch between the bf16 MFMA fast path and the generic fp32 kernels.
// Declarations and the argument contract live in include/parallax.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "plx_internal.h"

namespace {

thread_local char g_last_error[512] = "";
thread_local hipEvent_t g_ev_before = nullptr;
thread_local hipEvent_t g_ev_after = nullptr;
thread_local int g_ev_kernel = -1;
std::atomic<int> g_decode_path{PLX_DECODE_AUTO};

plx_status fail(plx_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

plx_status ok() {
  g_last_error[0] = '\0';
  return PLX_OK;
}

constexpr int kDefaultSplitRows = 256;

// Checks the descriptor and fills the geometry.  `what` names the entry point.
plx_status check_desc(const plx_attn_desc* d, const char* what, plx::Geom* g) {
  if (!d) return fail(PLX_ERR_INVALID, "%s: desc is NULL", what);
  if (d->batch < 0 || d->seqlen_q < 0 || d->seqlen_k < 0)
    return fail(PLX_ERR_INVALID, "%s: negative size (batch=%d seqlen_q=%d seqlen_k=%d)", what,
                d->batch, d->seqlen_q, d->seqlen_k);
  if (d->heads_q < 1 || d->heads_kv < 1)
    return fail(PLX_ERR_INVALID, "%s: heads_q=%d heads_kv=%d must be >= 1", what, d->heads_q,
                d->heads_kv);
  if (d->heads_q % d->heads_kv != 0)
    return fail(PLX_ERR_INVALID, "%s: heads_q=%d is not a multiple of heads_kv=%d", what,
                d->heads_q, d->heads_kv);
  if (d->head_dim < 1) return fail(PLX_ERR_INVALID, "%s: head_dim=%d < 1", what, d->head_dim);
  if (d->head_dim > 128)
    return fail(PLX_ERR_UNSUPPORTED, "%s: head_dim=%d > 128 is not supported", what, d->head_dim);
  if (d->dtype != PLX_F32 && d->dtype != PLX_BF16)
    return fail(PLX_ERR_INVALID, "%s: unknown dtype %d", what, d->dtype);
  if (d->out_dtype != PLX_F32 && d->out_dtype != PLX_BF16)
    return fail(PLX_ERR_INVALID, "%s: unknown out_dtype %d", what, d->out_dtype);
  if (d->p_per_query != 0 && d->p_per_query != 1)
    return fail(PLX_ERR_INVALID, "%s: p_per_query must be 0 or 1", what);
  if (!(d->softmax_scale == d->softmax_scale) || isinf(d->softmax_scale))
    return fail(PLX_ERR_INVALID, "%s: softmax_scale is not finite", what);
  g->B = d->batch;
  g->Tq = d->seqlen_q;
  g->Tk = d->seqlen_k;
  g->Hq = d->heads_q;
  g->Hkv = d->heads_kv;
  g->d = d->head_dim;
  g->causal = d->causal != 0;
  g->window = d->window > 0 ? d->window : 0;
  g->scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.f / sqrtf(static_cast<float>(d->head_dim));
  g->bf16 = d->dtype == PLX_BF16;
  g->p_per_query = d->p_per_query;
  g->out_bf16 = d->out_dtype == PLX_BF16;
  return PLX_OK;
}

int split_rows_of(const plx_attn_desc* d) {
  return d->split_rows < 0 ? kDefaultSplitRows : d->split_rows;
}

plx_status check_ws(size_t need, const void* ws, size_t have, const char* what) {
  if (have < need)
    return fail(PLX_ERR_WORKSPACE, "%s: workspace_bytes=%zu < required %zu", what, have, need);
  if (need > 0 && !ws) return fail(PLX_ERR_INVALID, "%s: workspace is NULL but %zu bytes are required", what, need);
  return PLX_OK;
}

plx_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PLX_ERR_HIP, "%s: HIP error %d (%s)", what, static_cast<int>(e), hipGetErrorString(e));
  return ok();
}

size_t fwd_ws(const plx::Geom& g) {
  return plx::fast_fwd_supported(g) ? plx::fast_fwd_workspace(g) : 0;
}

size_t bwd_ws(const plx::Geom& g) {
  return plx::fast_bwd_supported(g) ? plx::fast_bwd_workspace(g) : plx::generic_bwd_workspace(g);
}

size_t dec_ws(const plx::Geom& g) {
  return plx::fast_decode_supported(g) ? plx::fast_decode_workspace(g) : 0;
}

}  // namespace

namespace plx {

namespace {
// One non-blocking helper stream per device (default priority), created on first use together with
// two events that order it against the caller's stream, and kept until the process ends.  Fork and
// join each record one of those events and make the other stream wait for it; the pair runs under
// the device's mutex, so a wait always refers to the record made by the same call (a stream wait
// takes the event's most recent record at the time of the wait).
constexpr int kMaxDevices = 64;
struct SideState {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool tried = false;
  std::mutex mutex;
};
SideState g_side[kMaxDevices];

SideState* side_state() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  SideState& s = g_side[dev];
  std::lock_guard<std::mutex> lock(s.mutex);
  if (!s.tried) {
    s.tried = true;
    bool good = hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) == hipSuccess;
    good = good && hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) == hipSuccess;
    good = good && hipEventCreateWithFlags(&s.join, hipEventDisableTiming) == hipSuccess;
    if (!good) s.stream = nullptr;   // (whatever was created stays until exit; the lane is not used)
  }
  return s.stream ? &s : nullptr;
}
}  // namespace

SideLane side_fork(hipStream_t main) {
  SideLane lane{main, main};
  SideState* s = side_state();
  if (!s) return lane;
  std::lock_guard<std::mutex> lock(s->mutex);
  if (hipEventRecord(s->fork, main) == hipSuccess && hipStreamWaitEvent(s->stream, s->fork, 0) == hipSuccess)
    lane.stream = s->stream;
  return lane;
}

hipError_t side_join(const SideLane& lane) {
  if (lane.stream == lane.main) return hipSuccess;
  SideState* s = side_state();
  if (!s) return hipErrorInvalidHandle;
  std::lock_guard<std::mutex> lock(s->mutex);
  hipError_t e = hipEventRecord(s->join, lane.stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(lane.main, s->join, 0);
  return e;
}

int decode_path() { return g_decode_path.load(); }

void mark_begin(int kernel, hipStream_t stream) {
  if (g_ev_before && kernel == g_ev_kernel) (void)hipEventRecord(g_ev_before, stream);
}
void mark_end(int kernel, hipStream_t stream) {
  if (g_ev_after && kernel == g_ev_kernel) (void)hipEventRecord(g_ev_after, stream);
}
}  // namespace plx

namespace {
// Scratch of the no-allocation decode entry point: a fixed device array instead of the caller's
// workspace.  Every GPU the library runs on holds its own copy until the process ends.  Host code
// never uses the array's name as an address (in host code it is only a stand-in for the symbol):
// the device address is looked up once per device with hipGetSymbolAddress, with that device current,
// and kept.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
void* g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mutex;

// The scratch array's device address on the current device (looked up on first use per device).
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" {

void parallax_set_kernel_events(int kernel, void* before, void* after) {
  g_ev_kernel = kernel;
  g_ev_before = static_cast<hipEvent_t>(before);
  g_ev_after = static_cast<hipEvent_t>(after);
}

plx_status parallax_set_decode_path(int32_t path) {
  if (path != PLX_DECODE_AUTO && path != PLX_DECODE_TWO_PASS)
    return fail(PLX_ERR_INVALID, "parallax_set_decode_path: path must be PLX_DECODE_AUTO or PLX_DECODE_TWO_PASS");
  g_decode_path.store(path);
  return PLX_OK;
}

int parallax_abi_version(void) { return PARALLAX_ABI_VERSION; }

const char* parallax_status_string(plx_status s) {
  switch (s) {
    case PLX_OK: return "PLX_OK";
    case PLX_ERR_INVALID: return "PLX_ERR_INVALID: invalid argument";
    case PLX_ERR_UNSUPPORTED: return "PLX_ERR_UNSUPPORTED: valid but not supported";
    case PLX_ERR_WORKSPACE: return "PLX_ERR_WORKSPACE: workspace too small";
    case PLX_ERR_HIP: return "PLX_ERR_HIP: HIP runtime error";
  }
  return "unknown plx_status";
}

const char* parallax_last_error(void) { return g_last_error; }

size_t parallax_attn_fwd_workspace(const plx_attn_desc* desc) {
  plx::Geom g;
  if (check_desc(desc, "parallax_attn_fwd_workspace", &g) != PLX_OK) return 0;
  return fwd_ws(g);
}

plx_status parallax_attn_fwd(const plx_attn_desc* desc, const void* q, const void* k,
                             const void* v, const void* P, void* out, float* lse, float* kbar,
                             float* o_sa, float* cor, void* workspace, size_t workspace_bytes,
                             void* hip_stream) {
  const char* what = "parallax_attn_fwd";
  plx::Geom g;
  plx_status st = check_desc(desc, what, &g);
  if (st != PLX_OK) return st;
  const bool empty = g.B == 0 || g.Tq == 0;
  if (!empty && (!q || !P || !out))
    return fail(PLX_ERR_INVALID, "%s: q, P and out must not be NULL", what);
  if (!empty && g.Tk > 0 && (!k || !v)) return fail(PLX_ERR_INVALID, "%s: k and v must not be NULL", what);
  st = check_ws(fwd_ws(g), workspace, workspace_bytes, what);
  if (st != PLX_OK) return st;
  if (empty) return ok();
  if (!plx::fast_fwd_supported(g) && (g.out_bf16 || cor))
    return fail(PLX_ERR_UNSUPPORTED, "%s: bf16 out and cor need the bf16 fast path", what);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t e;
  if (plx::fast_fwd_supported(g))
    e = plx::launch_fast_fwd(g, q, k, v, P, out, lse, kbar, o_sa, cor, split_rows_of(desc), workspace, stream);
  else
    e = plx::launch_generic_fwd(g, q, k, v, P, nullptr, static_cast<float*>(out), lse, kbar, o_sa, 0, g.Tq,
                                stream, true);
  return hip_status(e, what);
}

size_t parallax_attn_fwd_probe_workspace(const plx_attn_desc* desc) {
  plx::Geom g;
  if (check_desc(desc, "parallax_attn_fwd_probe_workspace", &g) != PLX_OK) return 0;
  return plx::fast_probe_supported(g) ? plx::fast_probe_workspace(g) : 0;
}

plx_status parallax_attn_fwd_probe(const plx_attn_desc* desc, const void* q, const void* k,
                                   const void* v, const void* rho, void* out, float* lse, float* o_sa,
                                   float* rk, float* cor, void* workspace, size_t workspace_bytes,
                                   void* hip_stream) {
  const char* what = "parallax_attn_fwd_probe";
  plx::Geom g;
  plx_status st = check_desc(desc, what, &g);
  if (st != PLX_OK) return st;
  if (!plx::fast_probe_supported(g))
    return fail(PLX_ERR_UNSUPPORTED,
                "%s: only bf16, head_dim 128 or 64, heads_q/heads_kv in {1,2,4,8} and p_per_query 0 are supported",
                what);
  const bool empty = g.B == 0 || g.Tq == 0;
  if (!empty && (!q || !rho || !out))
    return fail(PLX_ERR_INVALID, "%s: q, rho and out must not be NULL", what);
  if (!empty && g.Tk > 0 && (!k || !v)) return fail(PLX_ERR_INVALID, "%s: k and v must not be NULL", what);
  st = check_ws(plx::fast_probe_workspace(g), workspace, workspace_bytes, what);
  if (st != PLX_OK) return st;
  if (empty) return ok();
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  return hip_status(plx::launch_fast_probe(g, q, k, v, rho, out, lse, o_sa, rk, cor, split_rows_of(desc), workspace,
                                           stream),
                    what);
}

size_t parallax_attn_bwd_probe_workspace(const plx_attn_desc* desc) {
  plx::Geom g;
  if (check_desc(desc, "parallax_attn_bwd_probe_workspace", &g) != PLX_OK) return 0;
  if (!plx::fast_probe_bwd_supported(g)) return 0;
  return plx::fast_probe_bwd_workspace(g);
}

plx_status parallax_attn_bwd_probe(const plx_attn_desc* desc, const void* q, const void* k, const void* v,
                                   const void* rho, const float* out, const void* dout, const float* lse,
                                   const float* o_sa, const float* rk, float* dq, float* dk, float* dv,
                                   float* drho, void* workspace, size_t workspace_bytes, void* hip_stream) {
  const char* what = "parallax_attn_bwd_probe";
  plx::Geom g;
  plx_status st = check_desc(desc, what, &g);
  if (st != PLX_OK) return st;
  if (g.out_bf16) return fail(PLX_ERR_UNSUPPORTED, "%s: the backward reads an fp32 out (out_dtype PLX_F32)", what);
  // the empty cases only write zeros; the kernels need every extent >= 1
  plx::Geom gs = g;
  gs.B = gs.Tq = gs.Tk = 1;
  if (!plx::fast_probe_bwd_supported(gs))
    return fail(PLX_ERR_UNSUPPORTED,
                "%s: only bf16, head_dim 128 or 64, heads_q/heads_kv in {1,2,4,8} and p_per_query 0 are supported",
                what);
  const bool rows = g.B > 0 && g.Tq > 0;
  const bool keys = g.B > 0 && g.Tk > 0;
  if (rows && (!q || !rho || !out || !dout || !lse || !o_sa || !rk || !dq || !drho))
    return fail(PLX_ERR_INVALID, "%s: q, rho, out, dout, lse, o_sa, rk, dq and drho must not be NULL", what);
  if (keys && (!k || !v || !dk || !dv)) return fail(PLX_ERR_INVALID, "%s: k, v, dk and dv must not be NULL", what);
  const size_t need = plx::fast_probe_bwd_supported(g) ? plx::fast_probe_bwd_workspace(g) : 0;
  st = check_ws(need, workspace, workspace_bytes, what);
  if (st != PLX_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t e = hipSuccess;
  if (rows && keys) {
    e = plx::launch_fast_probe_bwd(g, q, k, v, rho, out, dout, lse, o_sa, rk, dq, dk, dv, drho,
                                   split_rows_of(desc), workspace, stream);
  } else {
    // no pair is visible: every gradient is zero
    const int64_t nq = static_cast<int64_t>(g.B) * g.Tq * g.Hq * g.d;
    const int64_t nk = static_cast<int64_t>(g.B) * g.Tk * g.Hkv * g.d;
    if (rows && e == hipSuccess) e = plx::launch_zero_f32(dq, nq, stream);
    if (rows && e == hipSuccess) e = plx::launch_zero_f32(drho, nq, stream);
    if (keys && e == hipSuccess) e = plx::launch_zero_f32(dk, nk, stream);
    if (keys && e == hipSuccess) e = plx::launch_zero_f32(dv, nk, stream);
  }
  return hip_status(e, what);
}

size_t parallax_attn_bwd_workspace(const plx_attn_desc* desc) {
  plx::Geom g;
  if (check_desc(desc, "parallax_attn_bwd_workspace", &g) != PLX_OK) return 0;
  return bwd_ws(g);
}

plx_status parallax_attn_bwd(const plx_attn_desc* desc, const void* q, const void* k,
                             const void* v, const void* P, const float* out, const void* dout,
                             const float* lse, const float* kbar, const float* o_sa, float* dq,
                             float* dk, float* dv, float* dP, void* workspace,
                             size_t workspace_bytes, void* hip_stream) {
  const char* what = "parallax_attn_bwd";
  plx::Geom g;
  plx_status st = check_desc(desc, what, &g);
  if (st != PLX_OK) return st;
  if (g.p_per_query)
    return fail(PLX_ERR_UNSUPPORTED, "%s: per-query projectors have no backward", what);
  if (g.out_bf16) return fail(PLX_ERR_UNSUPPORTED, "%s: the backward reads an fp32 out (out_dtype PLX_F32)", what);
  if (!P || !dP) return fail(PLX_ERR_INVALID, "%s: P and dP must not be NULL", what);
  const bool rows = g.B > 0 && g.Tq > 0;
  const bool keys = g.B > 0 && g.Tk > 0;
  if (rows && (!q || !out || !dout || !lse || !kbar || !o_sa || !dq))
    return fail(PLX_ERR_INVALID, "%s: q, out, dout, lse, kbar, o_sa and dq must not be NULL", what);
  if (keys && (!k || !v || !dk || !dv))
    return fail(PLX_ERR_INVALID, "%s: k, v, dk and dv must not be NULL", what);
  st = check_ws(bwd_ws(g), workspace, workspace_bytes, what);
  if (st != PLX_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t e;
  if (plx::fast_bwd_supported(g))
    e = plx::launch_fast_bwd(g, q, k, v, P, out, dout, lse, kbar, o_sa, dq, dk, dv, dP,
                             split_rows_of(desc), workspace, stream);
  else
    e = plx::launch_generic_bwd(g, q, k, v, P, out, dout, lse, kbar, o_sa, dq, dk, dv, dP,
                                workspace, stream);
  return hip_status(e, what);
}

size_t parallax_attn_decode_workspace(const plx_attn_desc* desc) {
  plx::Geom g;
  if (check_desc(desc, "parallax_attn_decode_workspace", &g) != PLX_OK) return 0;
  if (g.Tq < 1 || g.p_per_query) return 0;
  if (g.Tq > 1 && !plx::fast_decode_supported(g)) return 0;
  g.causal = 1;
  return dec_ws(g);
}

plx_status parallax_attn_decode(const plx_attn_desc* desc, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* seqlens_k, const void* P,
                                void* out, float* cor, void* workspace, size_t workspace_bytes,
                                void* hip_stream) {
  const char* what = "parallax_attn_decode";
  plx::Geom g;
  plx_status st = check_desc(desc, what, &g);
  if (st != PLX_OK) return st;
  if (g.Tq < 1) return fail(PLX_ERR_INVALID, "%s: seqlen_q must be >= 1 (got %d)", what, g.Tq);
  if (g.p_per_query) return fail(PLX_ERR_UNSUPPORTED, "%s: per-query projectors are not supported", what);
  if (g.Tq > 1 && !plx::fast_decode_supported(g))
    return fail(PLX_ERR_UNSUPPORTED, "%s: several new tokens per sequence need the bf16 fast path", what);
  g.causal = 1;  // the new token is the last entry of its sequence: it sees all of it
  if (g.B == 0) {
    st = check_ws(dec_ws(g), workspace, workspace_bytes, what);
    return st != PLX_OK ? st : ok();
  }
  if (!q || !P || !out) return fail(PLX_ERR_INVALID, "%s: q, P and out must not be NULL", what);
  if (g.Tk > 0 && (!k_cache || !v_cache))
    return fail(PLX_ERR_INVALID, "%s: k_cache and v_cache must not be NULL", what);
  st = check_ws(dec_ws(g), workspace, workspace_bytes, what);
  if (st != PLX_OK) return st;
  if (!plx::fast_decode_supported(g) && (g.out_bf16 || cor))
    return fail(PLX_ERR_UNSUPPORTED, "%s: bf16 out and cor need the bf16 fast path", what);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t e;
  if (plx::fast_decode_supported(g))
    e = plx::launch_fast_decode(g, q, k_cache, v_cache, seqlens_k, P, out, cor, workspace, stream);
  else
    e = plx::launch_generic_fwd(g, q, k_cache, v_cache, P, seqlens_k, static_cast<float*>(out), nullptr, nullptr,
                                nullptr, 0, 1, stream, true, PLX_KERNEL_DECODE_PASS1);
  return hip_status(e, what);
}

size_t parallax_attn_decode_paged_workspace(const plx_attn_desc* desc) {
  plx::Geom g;
  if (check_desc(desc, "parallax_attn_decode_paged_workspace", &g) != PLX_OK) return 0;
  if (g.Tq < 1 || g.p_per_query || !plx::fast_decode_supported(g)) return 0;
  g.causal = 1;
  return plx::fast_decode_workspace(g);
}

plx_status parallax_attn_decode_paged(const plx_attn_desc* desc, const void* q, const void* k_pages,
                                      const void* v_pages, int32_t num_pages, int32_t page_size,
                                      const int32_t* block_table, int32_t block_table_stride,
                                      const int32_t* seqlens_k, const void* P,
                                      void* out, float* cor, void* workspace, size_t workspace_bytes,
                                      void* hip_stream) {
  const char* what = "parallax_attn_decode_paged";
  plx::Geom g;
  plx_status st = check_desc(desc, what, &g);
  if (st != PLX_OK) return st;
  if (g.Tq < 1) return fail(PLX_ERR_INVALID, "%s: seqlen_q must be >= 1 (got %d)", what, g.Tq);
  if (page_size < 1 || page_size > 65536 || (page_size & (page_size - 1)) != 0)
    return fail(PLX_ERR_INVALID, "%s: page_size=%d is not a power of two in [1, 65536]", what, page_size);
  if (num_pages < 1) return fail(PLX_ERR_INVALID, "%s: num_pages=%d < 1", what, num_pages);
  const int64_t pages_needed = (static_cast<int64_t>(desc->seqlen_k) + page_size - 1) / page_size;
  if (block_table_stride < pages_needed)
    return fail(PLX_ERR_INVALID, "%s: block_table_stride=%d < %lld pages needed for seqlen_k=%d", what,
                block_table_stride, static_cast<long long>(pages_needed), desc->seqlen_k);
  if (!plx::fast_decode_supported(g))
    return fail(PLX_ERR_UNSUPPORTED,
                "%s: only bf16, head_dim 128 or 64, heads_q/heads_kv in {1,2,4,8} and p_per_query 0 are supported",
                what);
  g.causal = 1;
  const size_t need = plx::fast_decode_workspace(g);
  if (g.B == 0) {
    st = check_ws(need, workspace, workspace_bytes, what);
    return st != PLX_OK ? st : ok();
  }
  if (!q || !P || !out) return fail(PLX_ERR_INVALID, "%s: q, P and out must not be NULL", what);
  if (g.Tk > 0 && (!k_pages || !v_pages || !block_table))
    return fail(PLX_ERR_INVALID, "%s: k_pages, v_pages and block_table must not be NULL", what);
  st = check_ws(need, workspace, workspace_bytes, what);
  if (st != PLX_OK) return st;
  plx::PagedCache pc{block_table, num_pages, page_size, block_table_stride};
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  return hip_status(plx::launch_fast_decode(g, q, k_pages, v_pages, seqlens_k, P, out, cor, workspace, stream, &pc),
                    what);
}

size_t parallax_attn_decode_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

plx_status parallax_attn_decode_noalloc(const plx_attn_desc* desc, const void* q, const void* k_cache,
                                        const void* v_cache, const int32_t* seqlens_k, const void* P, void* out,
                                        float* cor, void* hip_stream) {
  const char* what = "parallax_attn_decode_noalloc";
  plx::Geom g;
  plx_status st = check_desc(desc, what, &g);
  if (st != PLX_OK) return st;
  if (g.Tq < 1) return fail(PLX_ERR_INVALID, "%s: seqlen_q must be >= 1 (got %d)", what, g.Tq);
  if (g.p_per_query) return fail(PLX_ERR_UNSUPPORTED, "%s: per-query projectors are not supported", what);
  if (g.Tq > 1 && !plx::fast_decode_supported(g))
    return fail(PLX_ERR_UNSUPPORTED, "%s: several new tokens per sequence need the bf16 fast path", what);
  g.causal = 1;
  const size_t need = dec_ws(g);
  if (need > kNoAllocScratchBytes)
    return fail(PLX_ERR_WORKSPACE, "%s: needs %zu bytes of scratch, more than the fixed %zu (use parallax_attn_decode "
                "with a workspace)", what, need, kNoAllocScratchBytes);
  if (g.B == 0) return ok();
  if (!q || !P || !out) return fail(PLX_ERR_INVALID, "%s: q, P and out must not be NULL", what);
  if (g.Tk > 0 && (!k_cache || !v_cache))
    return fail(PLX_ERR_INVALID, "%s: k_cache and v_cache must not be NULL", what);
  if (!plx::fast_decode_supported(g) && (g.out_bf16 || cor))
    return fail(PLX_ERR_UNSUPPORTED, "%s: bf16 out and cor need the bf16 fast path", what);
  void* ws = nullptr;
  hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) return hip_status(e, what);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (plx::fast_decode_supported(g))
    e = plx::launch_fast_decode(g, q, k_cache, v_cache, seqlens_k, P, out, cor, ws, stream);
  else
    e = plx::launch_generic_fwd(g, q, k_cache, v_cache, P, seqlens_k, static_cast<float*>(out), nullptr, nullptr,
                                nullptr, 0, 1, stream, true, PLX_KERNEL_DECODE_PASS1);
  return hip_status(e, what);
}

}  // extern "C"
