// C ABI of libep.so: argument checks, workspace carving and kernel launches.
//
// Every check runs on the host before anything is launched; a failed check
// returns an error code and records a message for ep_last_error() ("DeepEP
// topk_idx_t Custom Dtype Requirements", Runtime Validation: validation halts
// before any GPU work).  The numeric limits are those of the "Low-Latency
// Mode API" page, Constraints: top-k in (0, 16], experts in (0, 512], hidden a
// positive multiple of 32; the token count may not exceed the capacity.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "common.hpp"
#include "dispatch.hpp"
#include "moe.hpp"
#include "static_ws.hpp"

namespace {

thread_local char g_err[512] = "";

ep_status_t fail(ep_status_t code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

ep_status_t hip_fail(hipError_t e, const char *where) {
  return fail(EP_ERR_HIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_quant(int q) {
  const int mode = q & ep::kQuantMask;
  return (q & ~(ep::kQuantMask | EP_RECV_INTERLEAVED)) == 0 && mode >= EP_QUANT_NONE &&
         mode <= EP_QUANT_FP8_B128_UE8M0;
}

constexpr int32_t kMaxHidden = 65536;

ep_status_t check_hidden(int32_t hidden, int quant, const char *fn) {
  if (!valid_quant(quant)) return fail(EP_ERR_INVALID_ARG, "%s: unknown quant mode %d", fn, quant);
  if (hidden <= 0 || hidden % 32 != 0)
    return fail(EP_ERR_INVALID_ARG, "%s: hidden must be a positive multiple of 32 (got %d)", fn, hidden);
  if (hidden > kMaxHidden) return fail(EP_ERR_UNSUPPORTED, "%s: hidden %d exceeds %d", fn, hidden, kMaxHidden);
  if (ep::is_b128(quant & ep::kQuantMask) && hidden % 128 != 0)
    return fail(EP_ERR_INVALID_ARG, "%s: per-128 e4m3 needs hidden %% 128 == 0 (got %d)", fn, hidden);
  return EP_OK;
}

ep_status_t check_handle(const ep_handle_t *h, const char *fn) {
  if (!h) return fail(EP_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  if (h->num_topk <= 0 || h->num_topk > ep::kMaxTopk || h->num_experts <= 0 ||
      h->num_experts > ep::kMaxExperts || h->num_tokens < 0 || h->num_tokens > h->num_max_tokens ||
      h->max_rows < 0 ||
      h->max_rows != ep::layout_rows(h->num_max_tokens, h->num_topk, h->num_experts, h->row_align,
                                     h->expert_capacity))
    return fail(EP_ERR_INVALID_ARG, "%s: handle fields are inconsistent (not made by ep_layout?)", fn);
  if (!h->offsets || !h->slot || !h->row_src || !h->status)
    return fail(EP_ERR_INVALID_ARG, "%s: handle holds NULL pointers", fn);
  return EP_OK;
}

size_t buffer_bytes(int64_t rows, int32_t hidden, int quant, size_t *scale_off) {
  const ep::RecvGeom g = ep::recv_geom(rows, hidden, quant);
  if (scale_off) *scale_off = g.scale_off;
  return g.total;
}

}  // namespace

extern "C" {

int32_t ep_abi_version(void) { return EP_ABI_VERSION; }

const char *ep_last_error(void) { return g_err; }

size_t ep_workspace_bytes(int64_t num_max_dispatch_tokens, int32_t num_topk, int32_t num_experts) {
  if (num_max_dispatch_tokens < 0 || num_topk <= 0 || num_topk > ep::kMaxTopk || num_experts <= 0 ||
      num_experts > ep::kMaxExperts || num_max_dispatch_tokens * num_topk > INT32_MAX)
    return 0;
  return ep::workspace_layout(num_max_dispatch_tokens, num_topk, num_experts,
                              num_max_dispatch_tokens * num_topk).total;
}

int64_t ep_layout_rows(int64_t num_max_dispatch_tokens, int32_t num_topk, int32_t num_experts, int32_t row_align,
                       int32_t expert_capacity) {
  if (num_max_dispatch_tokens < 0 || num_topk <= 0 || num_topk > ep::kMaxTopk || num_experts <= 0 ||
      num_experts > ep::kMaxExperts || num_max_dispatch_tokens * num_topk > INT32_MAX)
    return -1;
  return ep::layout_rows(num_max_dispatch_tokens, num_topk, num_experts, row_align, expert_capacity);
}

size_t ep_workspace_bytes_ex(int64_t num_max_dispatch_tokens, int32_t num_topk, int32_t num_experts,
                             int32_t row_align, int32_t expert_capacity) {
  const int64_t rows = ep_layout_rows(num_max_dispatch_tokens, num_topk, num_experts, row_align, expert_capacity);
  if (rows < 0) return 0;
  return ep::workspace_layout(num_max_dispatch_tokens, num_topk, num_experts, rows).total;
}

ep_status_t ep_buffer_bytes(int64_t rows, int32_t hidden, ep_quant_t quant, size_t *total_bytes,
                            size_t *scale_offset) {
  if (rows < 0 || rows > INT32_MAX) return fail(EP_ERR_INVALID_ARG, "ep_buffer_bytes: rows out of range");
  const ep_status_t st = check_hidden(hidden, quant, "ep_buffer_bytes");
  if (st != EP_OK) return st;
  const size_t total = buffer_bytes(rows, hidden, quant, scale_offset);
  if (total_bytes) *total_bytes = total;
  return EP_OK;
}

}  // extern "C"

namespace {

// Checks the layout arguments and fills `h` (the handle the layout will
// produce) and `wl`; launches nothing.
ep_status_t layout_prepare(const char *fn, const void *topk_idx, ep_idx_dtype_t idx_dtype, int64_t num_tokens,
                           int32_t num_topk, int64_t num_max_dispatch_tokens, int32_t num_experts, int32_t row_align,
                           int32_t expert_capacity, int64_t *recv_count, int32_t *cumulative_recv_stats,
                           void *workspace, size_t workspace_bytes, ep_handle_t *handle, ep_handle_t &h,
                           ep::WsLayout &wl) {
  if (idx_dtype != EP_IDX_INT32 && idx_dtype != EP_IDX_INT64)
    return fail(EP_ERR_INVALID_ARG, "%s: topk_idx dtype must be int32 or int64", fn);
  if (num_topk <= 0 || num_topk > ep::kMaxTopk)
    return fail(EP_ERR_INVALID_ARG, "%s: num_topk must be in (0, 16] (got %d)", fn, num_topk);
  if (num_experts <= 0 || num_experts > ep::kMaxExperts)
    return fail(EP_ERR_INVALID_ARG, "%s: num_experts must be in (0, 512] (got %d)", fn, num_experts);
  if (num_tokens < 0 || num_max_dispatch_tokens < 0)
    return fail(EP_ERR_INVALID_ARG, "%s: negative token count", fn);
  if (num_tokens > num_max_dispatch_tokens)
    return fail(EP_ERR_INVALID_ARG, "%s: num_tokens %lld exceeds num_max_dispatch_tokens %lld", fn,
                (long long)num_tokens, (long long)num_max_dispatch_tokens);
  if (num_max_dispatch_tokens > INT32_MAX / num_topk)
    return fail(EP_ERR_INVALID_ARG, "%s: num_max_dispatch_tokens * num_topk exceeds 2^31-1", fn);
  if (row_align < 1 || row_align > ep::kMaxRowAlign)
    return fail(EP_ERR_INVALID_ARG, "%s: row_align must be in [1, %d] (got %d)", fn, ep::kMaxRowAlign, row_align);
  if (expert_capacity < 0) return fail(EP_ERR_INVALID_ARG, "%s: negative expert_capacity", fn);
  if (expert_capacity > 0 && row_align > 1)
    return fail(EP_ERR_INVALID_ARG, "%s: expert_capacity and row_align > 1 are exclusive", fn);
  const int64_t max_rows = ep::layout_rows(num_max_dispatch_tokens, num_topk, num_experts, row_align,
                                           expert_capacity);
  if (max_rows < 0) return fail(EP_ERR_INVALID_ARG, "%s: receive rows exceed 2^31-1", fn);
  if (num_tokens > 0 && !topk_idx) return fail(EP_ERR_INVALID_ARG, "%s: topk_idx is NULL", fn);
  if (topk_idx && !aligned(topk_idx, idx_dtype == EP_IDX_INT64 ? 8 : 4))
    return fail(EP_ERR_INVALID_ARG, "%s: topk_idx is not aligned to its dtype", fn);
  if (!recv_count || !aligned(recv_count, 8))
    return fail(EP_ERR_INVALID_ARG, "%s: recv_count is NULL or misaligned", fn);
  if (cumulative_recv_stats && !aligned(cumulative_recv_stats, 4))
    return fail(EP_ERR_INVALID_ARG, "%s: cumulative_recv_stats is misaligned", fn);
  if (!workspace || !aligned(workspace, ep::kWsAlign))
    return fail(EP_ERR_INVALID_ARG, "%s: workspace is NULL or not 256-byte aligned", fn);
  if (!handle) return fail(EP_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  wl = ep::workspace_layout(num_max_dispatch_tokens, num_topk, num_experts, max_rows);
  if (workspace_bytes < wl.total)
    return fail(EP_ERR_BUFFER_TOO_SMALL, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes, wl.total);

  char *ws = (char *)workspace;
  h.num_tokens = num_tokens;
  h.num_max_tokens = num_max_dispatch_tokens;
  h.max_rows = max_rows;
  h.num_topk = num_topk;
  h.num_experts = num_experts;
  h.row_align = row_align;
  h.expert_capacity = expert_capacity;
  h.offsets = (int32_t *)(ws + wl.offsets);
  h.slot = (int32_t *)(ws + wl.slot);
  h.row_src = (int32_t *)(ws + wl.row_src);
  h.status = (uint32_t *)(ws + wl.status);
  return EP_OK;
}

ep_status_t layout_impl(const char *fn, const void *topk_idx, ep_idx_dtype_t idx_dtype, int64_t num_tokens,
                        int32_t num_topk, int64_t num_max_dispatch_tokens, int32_t num_experts, int32_t row_align,
                        int32_t expert_capacity, int64_t *recv_count, int32_t *cumulative_recv_stats,
                        void *workspace, size_t workspace_bytes, ep_handle_t *handle, void *stream) {
  ep_handle_t h;
  ep::WsLayout wl;
  const ep_status_t st = layout_prepare(fn, topk_idx, idx_dtype, num_tokens, num_topk, num_max_dispatch_tokens,
                                        num_experts, row_align, expert_capacity, recv_count, cumulative_recv_stats,
                                        workspace, workspace_bytes, handle, h, wl);
  if (st != EP_OK) return st;
  const hipError_t e = ep::launch_layout(topk_idx, idx_dtype == EP_IDX_INT64, num_tokens, num_topk, num_experts,
                                         h.max_rows, row_align, expert_capacity, recv_count, cumulative_recv_stats,
                                         (char *)workspace, wl, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  *handle = h;
  return EP_OK;
}

// The dispatch arguments against a handle; launches nothing.
ep_status_t check_dispatch(const char *fn, const ep_handle_t *handle, const void *x, int32_t hidden,
                           const float *topk_weights, int quant, const void *recv_buf, size_t recv_buf_bytes,
                           const float *recv_weights) {
  ep_status_t st = check_handle(handle, fn);
  if (st != EP_OK) return st;
  st = check_hidden(hidden, quant, fn);
  if (st != EP_OK) return st;
  if (handle->num_tokens > 0 && !x) return fail(EP_ERR_INVALID_ARG, "%s: x is NULL", fn);
  if (x && !aligned(x, 16)) return fail(EP_ERR_INVALID_ARG, "%s: x is not 16-byte aligned", fn);
  if (!recv_buf || !aligned(recv_buf, 16))
    return fail(EP_ERR_INVALID_ARG, "%s: recv_buf is NULL or not 16-byte aligned", fn);
  const size_t need = buffer_bytes(handle->max_rows, hidden, quant, nullptr);
  if (recv_buf_bytes < need)
    return fail(EP_ERR_BUFFER_TOO_SMALL, "%s: recv_buf has %zu bytes, needs %zu", fn, recv_buf_bytes, need);
  if (recv_weights && !topk_weights && handle->num_tokens > 0)
    return fail(EP_ERR_INVALID_ARG, "%s: recv_weights given without topk_weights", fn);
  if ((topk_weights && !aligned(topk_weights, 4)) || (recv_weights && !aligned(recv_weights, 4)))
    return fail(EP_ERR_INVALID_ARG, "%s: weights are misaligned", fn);
  return EP_OK;
}

}  // namespace

extern "C" {

ep_status_t ep_layout_ex(const void *topk_idx, ep_idx_dtype_t idx_dtype, int64_t num_tokens, int32_t num_topk,
                         int64_t num_max_dispatch_tokens, int32_t num_experts, int32_t row_align,
                         int32_t expert_capacity, int64_t *recv_count, int32_t *cumulative_recv_stats,
                         void *workspace, size_t workspace_bytes, ep_handle_t *handle, void *stream) {
  return layout_impl("ep_layout_ex", topk_idx, idx_dtype, num_tokens, num_topk, num_max_dispatch_tokens,
                     num_experts, row_align, expert_capacity, recv_count, cumulative_recv_stats, workspace,
                     workspace_bytes, handle, stream);
}

ep_status_t ep_layout(const void *topk_idx, ep_idx_dtype_t idx_dtype, int64_t num_tokens, int32_t num_topk,
                      int64_t num_max_dispatch_tokens, int32_t num_experts, int64_t *recv_count,
                      int32_t *cumulative_recv_stats, void *workspace, size_t workspace_bytes,
                      ep_handle_t *handle, void *stream) {
  return layout_impl("ep_layout", topk_idx, idx_dtype, num_tokens, num_topk, num_max_dispatch_tokens, num_experts,
                     1, 0, recv_count, cumulative_recv_stats, workspace, workspace_bytes, handle, stream);
}

ep_status_t ep_dispatch(const ep_handle_t *handle, const void *x, int32_t hidden, const float *topk_weights,
                        ep_quant_t quant, void *recv_buf, size_t recv_buf_bytes, float *recv_weights,
                        void *stream) {
  const char *fn = "ep_dispatch";
  const ep_status_t st = check_dispatch(fn, handle, x, hidden, topk_weights, quant, recv_buf, recv_buf_bytes,
                                        recv_weights);
  if (st != EP_OK) return st;
  const hipError_t e = ep::launch_dispatch(*handle, x, hidden, topk_weights, quant, (char *)recv_buf,
                                           recv_weights, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return EP_OK;
}

}  // extern "C"

namespace {

ep_status_t layout_dispatch_impl(const char *fn, const void *topk_idx, ep_idx_dtype_t idx_dtype, int64_t num_tokens,
                                 int32_t num_topk, int64_t num_max_dispatch_tokens, int32_t num_experts,
                                 int32_t row_align, int32_t expert_capacity, int64_t *recv_count,
                                 int32_t *cumulative_recv_stats, void *workspace, size_t workspace_bytes,
                                 const void *x, int32_t hidden, const float *topk_weights, ep_quant_t quant,
                                 void *recv_buf, size_t recv_buf_bytes, float *recv_weights, ep_handle_t *handle,
                                 void *stream) {
  ep_handle_t h;
  ep::WsLayout wl;
  ep_status_t st = layout_prepare(fn, topk_idx, idx_dtype, num_tokens, num_topk, num_max_dispatch_tokens,
                                  num_experts, row_align, expert_capacity, recv_count, cumulative_recv_stats,
                                  workspace, workspace_bytes, handle, h, wl);
  if (st != EP_OK) return st;
  st = check_dispatch(fn, &h, x, hidden, topk_weights, quant, recv_buf, recv_buf_bytes, recv_weights);
  if (st != EP_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (ep::fused_layout_dispatch_fits(num_tokens * num_topk, row_align, expert_capacity, h.max_rows)) {
    e = ep::launch_layout_dispatch(h, topk_idx, idx_dtype == EP_IDX_INT64, recv_count, cumulative_recv_stats, x,
                                   hidden, topk_weights, quant, (char *)recv_buf, recv_weights, s);
  } else {
    e = ep::launch_layout(topk_idx, idx_dtype == EP_IDX_INT64, num_tokens, num_topk, num_experts, h.max_rows,
                          row_align, expert_capacity, recv_count, cumulative_recv_stats, (char *)workspace, wl, s);
    if (e == hipSuccess)
      e = ep::launch_dispatch(h, x, hidden, topk_weights, quant, (char *)recv_buf, recv_weights, s);
  }
  if (e != hipSuccess) return hip_fail(e, fn);
  *handle = h;
  return EP_OK;
}

}  // namespace

extern "C" {

ep_status_t ep_layout_dispatch(const void *topk_idx, ep_idx_dtype_t idx_dtype, int64_t num_tokens, int32_t num_topk,
                               int64_t num_max_dispatch_tokens, int32_t num_experts, int32_t row_align,
                               int32_t expert_capacity, int64_t *recv_count, int32_t *cumulative_recv_stats,
                               void *workspace, size_t workspace_bytes, const void *x, int32_t hidden,
                               const float *topk_weights, ep_quant_t quant, void *recv_buf, size_t recv_buf_bytes,
                               float *recv_weights, ep_handle_t *handle, void *stream) {
  return layout_dispatch_impl("ep_layout_dispatch", topk_idx, idx_dtype, num_tokens, num_topk,
                              num_max_dispatch_tokens, num_experts, row_align, expert_capacity, recv_count,
                              cumulative_recv_stats, workspace, workspace_bytes, x, hidden, topk_weights, quant,
                              recv_buf, recv_buf_bytes, recv_weights, handle, stream);
}

ep_status_t ep_layout_dispatch_noalloc(const void *topk_idx, ep_idx_dtype_t idx_dtype, int64_t num_tokens,
                                       int32_t num_topk, int64_t num_max_dispatch_tokens, int32_t num_experts,
                                       int32_t row_align, int32_t expert_capacity, int64_t *recv_count,
                                       int32_t *cumulative_recv_stats, const void *x, int32_t hidden,
                                       const float *topk_weights, ep_quant_t quant, void *recv_buf,
                                       size_t recv_buf_bytes, float *recv_weights, ep_handle_t *handle,
                                       void *stream) {
  const char *fn = "ep_layout_dispatch_noalloc";
  // the workspace this layout needs, against the library's static one
  // (argument errors are reported by the shared checks below)
  const int64_t rows = ep_layout_rows(num_max_dispatch_tokens, num_topk, num_experts, row_align, expert_capacity);
  if (rows >= 0) {
    const size_t need = ep::workspace_layout(num_max_dispatch_tokens, num_topk, num_experts, rows).total;
    if (need > ep::static_workspace_bytes())
      return fail(EP_ERR_BUFFER_TOO_SMALL, "%s: the layout needs %zu bytes of workspace, the static one holds %zu",
                  fn, need, ep::static_workspace_bytes());
  }
  void *ws = nullptr;
  const hipError_t e = ep::static_workspace(&ws);
  if (e != hipSuccess) return hip_fail(e, fn);
  return layout_dispatch_impl(fn, topk_idx, idx_dtype, num_tokens, num_topk, num_max_dispatch_tokens, num_experts,
                              row_align, expert_capacity, recv_count, cumulative_recv_stats, ws,
                              ep::static_workspace_bytes(), x, hidden, topk_weights, quant, recv_buf,
                              recv_buf_bytes, recv_weights, handle, stream);
}

ep_status_t ep_combine(const ep_handle_t *handle, const void *expert_out, size_t expert_out_bytes,
                       ep_quant_t in_quant, int32_t hidden, const void *topk_idx, ep_idx_dtype_t idx_dtype,
                       const float *topk_weights, void *out, void *stream) {
  const char *fn = "ep_combine";
  ep_status_t st = check_handle(handle, fn);
  if (st != EP_OK) return st;
  st = check_hidden(hidden, in_quant, fn);
  if (st != EP_OK) return st;
  if (idx_dtype != EP_IDX_INT32 && idx_dtype != EP_IDX_INT64)
    return fail(EP_ERR_INVALID_ARG, "%s: topk_idx dtype must be int32 or int64", fn);
  if (handle->num_tokens > 0 && !topk_idx)
    return fail(EP_ERR_INVALID_ARG, "%s: topk_idx is NULL (it must be the one given to dispatch)", fn);
  if (topk_idx && !aligned(topk_idx, idx_dtype == EP_IDX_INT64 ? 8 : 4))
    return fail(EP_ERR_INVALID_ARG, "%s: topk_idx is not aligned to its dtype", fn);
  if (!expert_out || !aligned(expert_out, 16))
    return fail(EP_ERR_INVALID_ARG, "%s: expert_out is NULL or not 16-byte aligned", fn);
  const size_t need = buffer_bytes(handle->max_rows, hidden, in_quant, nullptr);
  if (expert_out_bytes < need)
    return fail(EP_ERR_BUFFER_TOO_SMALL, "%s: expert_out has %zu bytes, needs %zu", fn, expert_out_bytes, need);
  if (handle->num_tokens > 0 && (!topk_weights || !aligned(topk_weights, 4)))
    return fail(EP_ERR_INVALID_ARG, "%s: topk_weights is NULL or misaligned (it is required)", fn);
  if (handle->num_tokens > 0 && (!out || !aligned(out, 16)))
    return fail(EP_ERR_INVALID_ARG, "%s: out is NULL or not 16-byte aligned", fn);
  const hipError_t e = ep::launch_combine(*handle, (const char *)expert_out, in_quant, hidden, topk_idx,
                                          idx_dtype == EP_IDX_INT64, topk_weights, out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return EP_OK;
}

ep_status_t ep_combine_backward(const ep_handle_t *handle, const void *grad_out, int32_t hidden,
                                const float *topk_weights, ep_quant_t quant, void *grad_buf, size_t grad_buf_bytes,
                                void *stream) {
  const char *fn = "ep_combine_backward";
  ep_status_t st = check_handle(handle, fn);
  if (st != EP_OK) return st;
  st = check_hidden(hidden, quant, fn);
  if (st != EP_OK) return st;
  if (handle->num_tokens > 0 && !grad_out) return fail(EP_ERR_INVALID_ARG, "%s: grad_out is NULL", fn);
  if (grad_out && !aligned(grad_out, 16))
    return fail(EP_ERR_INVALID_ARG, "%s: grad_out is not 16-byte aligned", fn);
  if (!grad_buf || !aligned(grad_buf, 16))
    return fail(EP_ERR_INVALID_ARG, "%s: grad_buf is NULL or not 16-byte aligned", fn);
  const size_t need = buffer_bytes(handle->max_rows, hidden, quant, nullptr);
  if (grad_buf_bytes < need)
    return fail(EP_ERR_BUFFER_TOO_SMALL, "%s: grad_buf has %zu bytes, needs %zu", fn, grad_buf_bytes, need);
  if (topk_weights && !aligned(topk_weights, 4))
    return fail(EP_ERR_INVALID_ARG, "%s: topk_weights is misaligned", fn);
  const hipError_t e = ep::launch_combine_backward(*handle, grad_out, hidden, topk_weights, quant, (char *)grad_buf,
                                                   (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return EP_OK;
}

ep_status_t ep_moe_packed_bytes(int32_t num_experts, int32_t rows, int32_t k, size_t *codes_bytes,
                                size_t *scales_bytes) {
  const char *fn = "ep_moe_packed_bytes";
  if (num_experts <= 0 || num_experts > ep::kMaxExperts || rows <= 0 || rows % 32 != 0 || k <= 0 || k % 64 != 0)
    return fail(EP_ERR_INVALID_ARG, "%s: need 0 < experts <= 512, rows %% 32 == 0, k %% 64 == 0", fn);
  size_t c, sc;
  ep::moe_packed_bytes(num_experts, rows, k, &c, &sc);
  if (codes_bytes) *codes_bytes = c;
  if (scales_bytes) *scales_bytes = sc;
  return EP_OK;
}

ep_status_t ep_moe_pack_weights(const void *codes, const void *scales, int32_t num_experts, int32_t rows, int32_t k,
                                int32_t gate_up, void *packed_codes, void *packed_scales, void *stream) {
  const char *fn = "ep_moe_pack_weights";
  const ep_status_t st = ep_moe_packed_bytes(num_experts, rows, k, nullptr, nullptr);
  if (st != EP_OK) return fail(st, "%s: need 0 < experts <= 512, rows %% 32 == 0, k %% 64 == 0", fn);
  if (gate_up != 0 && gate_up != 1) return fail(EP_ERR_INVALID_ARG, "%s: gate_up must be 0 or 1", fn);
  if (gate_up && rows % 64 != 0) return fail(EP_ERR_INVALID_ARG, "%s: gate/up weights need rows %% 64 == 0", fn);
  if (!codes || !scales || !packed_codes || !packed_scales || !aligned(codes, 16) || !aligned(packed_codes, 16) ||
      !aligned(packed_scales, 4))
    return fail(EP_ERR_INVALID_ARG, "%s: NULL or misaligned buffer", fn);
  const hipError_t e = ep::launch_moe_pack(codes, scales, num_experts, rows, k, gate_up, packed_codes, packed_scales,
                                           (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return EP_OK;
}

ep_status_t ep_moe_gmm1(const ep_handle_t *handle, const int64_t *recv_count, const void *x_buf, size_t x_buf_bytes,
                        int32_t hidden, int32_t inter, const void *w1, const void *w1_scales, ep_quant_t out_quant,
                        void *out_buf, size_t out_buf_bytes, void *stream) {
  const char *fn = "ep_moe_gmm1";
  ep_status_t st = check_handle(handle, fn);
  if (st != EP_OK) return st;
  if (hidden <= 0 || hidden % 128 != 0 || inter <= 0 || inter % 64 != 0)
    return fail(EP_ERR_INVALID_ARG, "%s: need hidden a positive multiple of 128 and inter of 64 (got %d, %d)", fn,
                hidden, inter);
  if (hidden > kMaxHidden || inter > kMaxHidden)
    return fail(EP_ERR_UNSUPPORTED, "%s: hidden / inter above %d", fn, kMaxHidden);
  if (out_quant != EP_QUANT_MXFP8 && out_quant != EP_QUANT_NONE)
    return fail(EP_ERR_INVALID_ARG, "%s: out_quant must be EP_QUANT_MXFP8 or EP_QUANT_NONE", fn);
  if (!x_buf || !aligned(x_buf, 16) || !out_buf || !aligned(out_buf, 16))
    return fail(EP_ERR_INVALID_ARG, "%s: x_buf / out_buf NULL or not 16-byte aligned", fn);
  if (!w1 || !w1_scales || !aligned(w1, 16) || !aligned(w1_scales, 4))
    return fail(EP_ERR_INVALID_ARG, "%s: w1 / w1_scales NULL or misaligned", fn);
  if (recv_count && !aligned(recv_count, 8)) return fail(EP_ERR_INVALID_ARG, "%s: recv_count misaligned", fn);
  const size_t need_x = buffer_bytes(handle->max_rows, hidden, EP_QUANT_MXFP8, nullptr);
  const size_t need_o = buffer_bytes(handle->max_rows, inter, out_quant, nullptr);
  if (x_buf_bytes < need_x || out_buf_bytes < need_o)
    return fail(EP_ERR_BUFFER_TOO_SMALL, "%s: x_buf needs %zu bytes, out_buf %zu", fn, need_x, need_o);
  const hipError_t e = ep::launch_moe_gmm1(*handle, recv_count, (const char *)x_buf, hidden, inter, w1, w1_scales,
                                           out_quant, (char *)out_buf, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return EP_OK;
}

ep_status_t ep_moe_gmm2(const ep_handle_t *handle, const int64_t *recv_count, const void *a_buf, size_t a_buf_bytes,
                        int32_t inter, int32_t hidden, const void *w2, const void *w2_scales, void *out_buf,
                        size_t out_buf_bytes, void *stream) {
  const char *fn = "ep_moe_gmm2";
  ep_status_t st = check_handle(handle, fn);
  if (st != EP_OK) return st;
  if (inter <= 0 || inter % 128 != 0 || hidden <= 0 || hidden % 128 != 0)
    return fail(EP_ERR_INVALID_ARG, "%s: inter and hidden must be positive multiples of 128 (got %d, %d)", fn, inter,
                hidden);
  if (hidden > kMaxHidden || inter > kMaxHidden)
    return fail(EP_ERR_UNSUPPORTED, "%s: hidden / inter above %d", fn, kMaxHidden);
  if (!a_buf || !aligned(a_buf, 16) || !out_buf || !aligned(out_buf, 16))
    return fail(EP_ERR_INVALID_ARG, "%s: a_buf / out_buf NULL or not 16-byte aligned", fn);
  if (!w2 || !w2_scales || !aligned(w2, 16) || !aligned(w2_scales, 4))
    return fail(EP_ERR_INVALID_ARG, "%s: w2 / w2_scales NULL or misaligned", fn);
  if (recv_count && !aligned(recv_count, 8)) return fail(EP_ERR_INVALID_ARG, "%s: recv_count misaligned", fn);
  const size_t need_a = buffer_bytes(handle->max_rows, inter, EP_QUANT_MXFP8, nullptr);
  const size_t need_o = buffer_bytes(handle->max_rows, hidden, EP_QUANT_NONE, nullptr);
  if (a_buf_bytes < need_a || out_buf_bytes < need_o)
    return fail(EP_ERR_BUFFER_TOO_SMALL, "%s: a_buf needs %zu bytes, out_buf %zu", fn, need_a, need_o);
  const hipError_t e = ep::launch_moe_gmm2(*handle, recv_count, (const char *)a_buf, inter, hidden, w2, w2_scales,
                                           (char *)out_buf, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return EP_OK;
}

ep_status_t ep_read_status(const ep_handle_t *handle, uint32_t *flags, void *stream) {
  const char *fn = "ep_read_status";
  if (!handle || !handle->status) return fail(EP_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  if (!flags) return fail(EP_ERR_INVALID_ARG, "%s: flags is NULL", fn);
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  e = hipMemcpy(flags, handle->status, sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, fn);
  return EP_OK;
}

}  // extern "C"
