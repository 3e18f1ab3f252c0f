/*
 * ep.h -- C ABI of the MI355X (gfx950) MoE token dispatch / combine library
 * (libep.so).
 *
 * The operation is the one the "Low-Latency Mode API" page (DeepEP-Ascend,
 * sections `low_latency_dispatch` and `low_latency_combine`) states for many
 * devices, done on one GPU that holds every expert:
 *
 *   ep_layout    routing layout from topk_idx: per-expert receive counts, the
 *                exclusive scan of those counts and a stable token-order row
 *                for every (token, j) pair.
 *   ep_dispatch  quantises each bf16 token row once and writes it to the
 *                receive row of every expert it is routed to.
 *   ep_combine   gathers each token's expert-output rows, dequantises them and
 *                reduces them in float32, weighted by topk_weights, in
 *                ascending j, rounding once to bf16.
 *
 * Conventions for every function below:
 *   - Array arguments are DEVICE pointers unless marked "host".  The caller
 *     owns every buffer; the library never allocates and never frees.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call is asynchronous on that stream, except ep_read_status, which
 *     waits for it.
 *   - All arguments are checked on the host before anything is launched.  On
 *     failure a call returns a non-zero ep_status_t, launches nothing, and
 *     ep_last_error() describes the failing check (the "Runtime Validation"
 *     rule of the "DeepEP topk_idx_t Custom Dtype Requirements" page).
 *   - Arrays are dense and row-major; "[T, k]" means T rows of k elements.
 *
 * Receive buffer format (ep_dispatch output and ep_combine input).  One
 * caller buffer holds a data region followed by a scale region ("EP dispatch
 * with unfused MXFP8 quantization", Changes: data and block scales share one
 * buffer sliced into data then scales):
 *   data region   rows x Dq bytes, row r at byte r*Dq
 *   scale region  starts at align_up(rows*Dq, 256); rows x Sq bytes
 *                 (EP_QUANT_NONE has no scale region and no padding)
 * with rows = handle.max_rows (num_max_tokens * k for the compact layout of
 * ep_layout; see ep_layout_rows for the others) and, for hidden size H:
 *   EP_QUANT_NONE        Dq = 2H (bf16)             Sq = 0
 *   EP_QUANT_INT8_TOKEN  Dq = H  (int8)             Sq = 4   (one float32)
 *   EP_QUANT_FP8_B128    Dq = H  (e4m3fn)           Sq = H/32 (H/128 float32)
 *   EP_QUANT_MXFP8       Dq = H  (e4m3fn)           Sq = H/32 (e8m0 bytes)
 *   EP_QUANT_FP8_B128_POW2  Dq = H (e4m3fn)         Sq = H/32 (H/128 float32)
 *   EP_QUANT_FP8_B128_UE8M0 Dq = H (e4m3fn)         Sq = H/128 (e8m0 bytes)
 *   EP_QUANT_MXFP4       Dq = H/2 (e2m1, element 2i in the low nibble)
 *                                                   Sq = H/32 (e8m0 bytes)
 * Interleaved form (quant OR-ed with EP_RECV_INTERLEAVED): row r starts at
 * byte r * align_up(Dq + Sq, 128) (rows on 128-byte cache lines) and holds its
 * Dq data bytes, then its Sq scale bytes, then padding -- the per-token message of "DeepEP FP8 Dispatch
 * and Combine Operations", Message Transmission via IBGDA (the payload
 * followed by its scales).
 * Expert e owns rows [offsets[e], offsets[e] + recv_count[e]); rows of one
 * expert are in ascending (token, j) order.  Rows that hold no pair (rows at
 * or past offsets[E], the padding of aligned or capacity-padded blocks) and
 * the padding between the regions are left unspecified.
 */
#ifndef EP_H_
#define EP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EP_ABI_VERSION 4

typedef enum {
  EP_OK = 0,
  EP_ERR_INVALID_ARG = 1,      /* a shape, enum, pointer or alignment check failed */
  EP_ERR_UNSUPPORTED = 2,      /* a valid request this library does not implement */
  EP_ERR_BUFFER_TOO_SMALL = 3, /* a caller buffer is smaller than required        */
  EP_ERR_HIP = 4               /* the HIP runtime reported an error                */
} ep_status_t;

/* Index dtype of topk_idx ("DeepEP topk_idx_t Custom Dtype Requirements":
 * int32 or int64; here chosen per call instead of at build time). */
typedef enum { EP_IDX_INT32 = 0, EP_IDX_INT64 = 1 } ep_idx_dtype_t;

/* Quantisation of a receive row ("Low-Latency Mode API", Parameters use_fp8,
 * use_ue8m0, use_mxfp4; "DeepEP FP8 Dispatch and Combine Operations", The
 * Dispatch Stage, for the per-128-channel e4m3 mode, and Advanced
 * Configuration Options, for its round_scale and use_ue8m0 variants).
 * Per-128 power-of-two scale: s0 = amax/448 rounded UP to a power of two 2^e
 * (e read off the float32 bits of s0), codes e4m3(clamp(x * 2^-e, +-448));
 * a block with amax 0 or e < -127 stores scale 0 (byte 0) and zero codes;
 * the e8m0 byte is e + 127, four consecutive blocks per int32. */
typedef enum {
  EP_QUANT_NONE = 0,       /* bf16 copy                                          */
  EP_QUANT_INT8_TOKEN = 1, /* int8, scale amax/127 per token                      */
  EP_QUANT_FP8_B128 = 2,   /* e4m3fn, scale amax/448 per 128 channels             */
  EP_QUANT_MXFP8 = 3,      /* e4m3fn, e8m0 power-of-two scale per 32 elements     */
  EP_QUANT_MXFP4 = 4,      /* e2m1 x2 per byte, e8m0 scale per 32 elements        */
  EP_QUANT_FP8_B128_POW2 = 5,  /* e4m3fn, power-of-two float32 scale per 128     */
  EP_QUANT_FP8_B128_UE8M0 = 6  /* e4m3fn, power-of-two e8m0 scale per 128        */
} ep_quant_t;

/* Receive-format flag OR-ed into the quant argument of ep_buffer_bytes,
 * ep_dispatch, ep_combine and ep_combine_backward (C++ callers cast the
 * result back to ep_quant_t): rows in the interleaved form above.  No other
 * bits above the low byte are accepted. */
#define EP_RECV_INTERLEAVED 0x100

/* Layout handle ("Low-Latency Mode API": the handle returned by dispatch is
 * passed unchanged to combine).  Plain data filled in by ep_layout; its
 * pointers point into the caller's workspace and stay valid while that
 * workspace lives and is not reused by another ep_layout call. */
typedef struct {
  int64_t num_tokens;     /* T                                               */
  int64_t num_max_tokens; /* capacity num_max_dispatch_tokens (>= T)         */
  int64_t max_rows;       /* receive rows: ep_layout_rows(num_max_tokens, k, */
                          /* E, row_align, expert_capacity)                  */
  int32_t num_topk;       /* k                                               */
  int32_t num_experts;    /* E                                               */
  int32_t row_align;      /* 1, or the alignment of every expert block       */
  int32_t expert_capacity;/* 0, or the rows of every expert block            */
  int32_t *offsets;       /* device [E+1]: block starts; offsets[E] = rows   */
                          /* up to the end of the last block                 */
  int32_t *slot;          /* device [T*k]: receive row of (t, j), or -1      */
  int32_t *row_src;       /* device [max_rows]: t*k + j of the pair in each  */
                          /* row, -1 for a row that holds none               */
  uint32_t *status;       /* device [1]: EP_STATUS_* bits                    */
} ep_handle_t;

/* Status bits of *handle.status.  The layout calls write the word (bits 0
 * and 1); ep_combine ORs in bit 2, which then stays set until the next layout
 * call on the same workspace. */
#define EP_STATUS_ID_OUT_OF_RANGE 1u   /* some id outside [-1, E), dropped     */
#define EP_STATUS_CAPACITY_OVERFLOW 2u /* some expert got more pairs than its  */
                                       /* capacity; the later ones dropped     */
#define EP_STATUS_COMBINE_MISMATCH 4u  /* ep_combine was given a topk_idx that */
                                       /* does not match the handle's layout   */

/* Bytes of workspace ep_layout needs for the given capacity; 0 if the
 * arguments are out of range.  Host-only; no device work. */
size_t ep_workspace_bytes(int64_t num_max_dispatch_tokens, int32_t num_topk, int32_t num_experts);

/* Receive rows (handle.max_rows) of a layout made by ep_layout_ex:
 *   expert_capacity == 0: num_max_dispatch_tokens * num_topk
 *                         + num_experts * (row_align - 1)
 *   expert_capacity  > 0: num_experts * expert_capacity
 * -1 if the arguments are out of range (see ep_layout_ex).  Host-only. */
int64_t ep_layout_rows(int64_t num_max_dispatch_tokens, int32_t num_topk, int32_t num_experts,
                       int32_t row_align, int32_t expert_capacity);

/* Workspace bytes of ep_layout_ex; 0 if the arguments are out of range.
 * Host-only. */
size_t ep_workspace_bytes_ex(int64_t num_max_dispatch_tokens, int32_t num_topk, int32_t num_experts,
                             int32_t row_align, int32_t expert_capacity);

/* Size of a receive buffer of `rows` rows (format above): writes the total
 * byte count and the scale offset to the host pointers (either may be NULL):
 * the start of the scale region, or for the interleaved form the offset of
 * the scales inside each row (Dq).  Host-only. */
ep_status_t ep_buffer_bytes(int64_t rows, int32_t hidden, ep_quant_t quant, size_t *total_bytes,
                            size_t *scale_offset);

/* Routing layout ("Low-Latency Mode API", Parameters topk_idx,
 * num_max_dispatch_tokens_per_rank, num_experts,
 * cumulative_local_expert_recv_stats; Return Values recv_count).
 *   topk_idx         device [T, k] of idx_dtype; -1 = no expert.  Ids outside
 *                    [-1, E) are dropped like -1 and set status bit 0.
 *                    May be NULL when num_tokens == 0.
 *   num_tokens       T, 0 <= T <= num_max_dispatch_tokens
 *   num_topk         k, 0 < k <= 16
 *   num_max_dispatch_tokens  capacity; max_rows = capacity * k <= 2^31 - 1
 *   num_experts      E, 0 < E <= 512
 *   recv_count       device int64 [E], written: rows received per expert
 *   cumulative_recv_stats  device int32 [E] or NULL: += recv_count
 *   workspace        device, 256-byte aligned, >= ep_workspace_bytes(...)
 *   handle           host, written on success
 * The receive-row order is deterministic: ascending (t, j) within an
 * expert, independent of timing. */
ep_status_t ep_layout(const void *topk_idx, ep_idx_dtype_t idx_dtype, int64_t num_tokens,
                      int32_t num_topk, int64_t num_max_dispatch_tokens, int32_t num_experts,
                      int64_t *recv_count, int32_t *cumulative_recv_stats, void *workspace,
                      size_t workspace_bytes, ep_handle_t *handle, void *stream);

/* Routing layout with per-expert blocks that are aligned or padded to a fixed
 * capacity -- the receive forms a grouped GEMM reads ("EP dispatch with
 * unfused MXFP8 quantization", Tests: the grouped path fixes one per-expert
 * alignment; "Low-Latency Mode API", low_latency_combine Parameters: x is
 * [num_local_experts, capacity, hidden]).  Arguments as ep_layout, plus:
 *   row_align        1 <= row_align <= 1024: every expert block starts at a
 *                    multiple of row_align rows; block e has
 *                    align_up(recv_count[e], row_align) rows.
 *   expert_capacity  0, or C > 0: block e is rows [e*C, (e+1)*C) (row_align
 *                    must then be 1).  Pairs past the C-th of an expert (in
 *                    (token, j) order) get slot -1 and set
 *                    EP_STATUS_CAPACITY_OVERFLOW; recv_count reports the rows
 *                    kept (<= C), cumulative_recv_stats adds the full demand.
 *   workspace        >= ep_workspace_bytes_ex(...)
 * ep_layout is ep_layout_ex with row_align 1 and expert_capacity 0.  The
 * other calls read only the handle, so they take any of these layouts. */
ep_status_t ep_layout_ex(const void *topk_idx, ep_idx_dtype_t idx_dtype, int64_t num_tokens,
                         int32_t num_topk, int64_t num_max_dispatch_tokens, int32_t num_experts,
                         int32_t row_align, int32_t expert_capacity, int64_t *recv_count,
                         int32_t *cumulative_recv_stats, void *workspace, size_t workspace_bytes,
                         ep_handle_t *handle, void *stream);

/* Dispatch ("Low-Latency Mode API", low_latency_dispatch; "DeepEP FP8
 * Dispatch and Combine Operations", The Dispatch Stage).
 *   handle         host, from ep_layout on the same stream (or ordered after it)
 *   x              device bf16 [T, H], 16-byte aligned.  Only bf16 input is
 *                  accepted: pre-quantised input is not a valid x.
 *   hidden         H > 0, H % 32 == 0 (H % 128 == 0 for the three per-128 modes)
 *   topk_weights   device float32 [T, k] or NULL
 *   recv_buf       device, 16-byte aligned, >= ep_buffer_bytes(max_rows, H, quant)
 *   recv_weights   device float32 [max_rows] or NULL; if given (and
 *                  topk_weights too) row slot[t, j] receives topk_weights[t, j]
 * Each token row is read once and quantised once; its packed row and scales
 * are written to every routed row. */
ep_status_t ep_dispatch(const ep_handle_t *handle, const void *x, int32_t hidden,
                        const float *topk_weights, ep_quant_t quant, void *recv_buf,
                        size_t recv_buf_bytes, float *recv_weights, void *stream);

/* Layout and dispatch in one call ("Low-Latency Mode API",
 * low_latency_dispatch, which takes the token rows and topk_idx together).
 * Arguments as ep_layout_ex followed by ep_dispatch; the results (handle,
 * recv_count, cumulative_recv_stats, status, receive buffer, receive
 * weights) are identical to that pair of calls, and every argument of both
 * is checked before anything is launched.  Compact layouts (row_align 1, no
 * capacity) and capacity blocks (row_align 1, at most 2^18 receive rows) of
 * at most 2048 (token, j) pairs run as a single launch, in which each
 * dispatch workgroup derives its own receive rows from topk_idx (a
 * decode-sized step saves one launch); aligned blocks and larger inputs run
 * the two launches of the separate calls.  The workspace must outlive every
 * call that uses the returned handle, as for ep_layout. */
ep_status_t ep_layout_dispatch(const void *topk_idx, ep_idx_dtype_t idx_dtype, int64_t num_tokens,
                               int32_t num_topk, int64_t num_max_dispatch_tokens, int32_t num_experts,
                               int32_t row_align, int32_t expert_capacity, int64_t *recv_count,
                               int32_t *cumulative_recv_stats, void *workspace, size_t workspace_bytes,
                               const void *x, int32_t hidden, const float *topk_weights, ep_quant_t quant,
                               void *recv_buf, size_t recv_buf_bytes, float *recv_weights,
                               ep_handle_t *handle, void *stream);

/* ep_layout_dispatch for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call without the workspace arguments.  The
 * workspace is the library's own static device array of 4 MiB (4194304
 * bytes) per GPU, held from the first call until the process ends; a layout
 * whose ep_workspace_bytes_ex(num_max_dispatch_tokens, num_topk,
 * num_experts, row_align, expert_capacity) exceeds it returns
 * EP_ERR_BUFFER_TOO_SMALL and launches nothing (4 MiB holds a compact
 * layout of up to 465472 (token, j) pairs with 512 experts, e.g. 58184
 * tokens at top-8, and 493120 with 256 experts).  The call allocates nothing
 * (no hipMalloc, no allocating library routine); it uses the current
 * device's array.  Every call on one device shares that array and leaves
 * its contents behind: the returned handle (its offsets, slot, row_src and
 * status point into the array) is valid until the next call of this
 * function on the same device, and calls that overlap on one device (other
 * streams or threads) race.  Results are those of ep_layout_dispatch. */
ep_status_t ep_layout_dispatch_noalloc(const void *topk_idx, ep_idx_dtype_t idx_dtype, int64_t num_tokens,
                                       int32_t num_topk, int64_t num_max_dispatch_tokens, int32_t num_experts,
                                       int32_t row_align, int32_t expert_capacity, int64_t *recv_count,
                                       int32_t *cumulative_recv_stats, const void *x, int32_t hidden,
                                       const float *topk_weights, ep_quant_t quant, void *recv_buf,
                                       size_t recv_buf_bytes, float *recv_weights, ep_handle_t *handle,
                                       void *stream);

/* Combine ("Low-Latency Mode API", low_latency_combine; "DeepEP FP8 Dispatch
 * and Combine Operations", The FP8 Combine Operation).
 *   handle          host, from the ep_layout of the matching dispatch
 *   expert_out      device receive-format buffer (format above, rows =
 *                   max_rows) of in_quant, 16-byte aligned
 *   hidden          H, as for ep_dispatch
 *   topk_idx        device [T, k] of idx_dtype: the ids given to the layout
 *                   call that made the handle (low_latency_combine
 *                   Parameters: topk_idx must match dispatch).  Aligned to
 *                   its dtype; may be NULL when T == 0.
 *   topk_weights    device float32 [T, k], required
 *   out             device bf16 [T, H], 16-byte aligned, written
 * out[t] = bf16_rne( sum over j = 0..k-1 with slot[t, j] >= 0 of
 *                    fl32(w[t, j] * dequant(row slot[t, j])) ), accumulated in
 * float32 in ascending j with one rounding per multiply and per add; a token
 * with no routed pair gets +0.  Dequantisation: int8 and e4m3-per-128 codes
 * times their float32 scale (one rounding); MX and per-128 e8m0 codes times
 * 2^(byte-127) (exact unless the product leaves float32's range); e8m0 byte
 * 0xFF is NaN.
 * The rows reduced are the handle's.  The kernel checks topk_idx against
 * them: pair (t, j) with a valid id e must sit in expert e's block (or be
 * dropped, slot -1, when blocks have a capacity) and a pair with any other
 * id must hold no row.  A pair that fails sets EP_STATUS_COMBINE_MISMATCH
 * (read it with ep_read_status); the output is still the handle's sum. */
ep_status_t ep_combine(const ep_handle_t *handle, const void *expert_out, size_t expert_out_bytes,
                       ep_quant_t in_quant, int32_t hidden, const void *topk_idx, ep_idx_dtype_t idx_dtype,
                       const float *topk_weights, void *out, void *stream);

/* Backward of combine with respect to the expert outputs, as a reverse
 * dispatch ("EP dispatch with unfused MXFP8 quantization", Description and
 * Changes: the result gradient is scattered back to the expert rows through
 * the same dispatch operation, quantised).
 *   handle         host, from the ep_layout of the forward pass
 *   grad_out       device bf16 [T, H] (gradient of combine's output), 16-byte aligned
 *   hidden         H, as for ep_dispatch
 *   topk_weights   device float32 [T, k] or NULL
 *   quant          format of the gradient rows (any ep_quant_t)
 *   grad_buf       device receive-format buffer (rows = max_rows), 16-byte
 *                  aligned, >= ep_buffer_bytes(max_rows, H, quant)
 * With topk_weights, row slot[t, j] receives the quantised
 * bf16_rne(fl32(topk_weights[t, j] * grad_out[t])) -- the gradient of the
 * weighted sum with respect to expert row j -- quantised once per routed
 * pair.  Without, it receives the quantised grad_out[t] (exactly
 * ep_dispatch of grad_out).  Rows that hold no pair are left unspecified. */
ep_status_t ep_combine_backward(const ep_handle_t *handle, const void *grad_out, int32_t hidden,
                                const float *topk_weights, ep_quant_t quant, void *grad_buf,
                                size_t grad_buf_bytes, void *stream);

/* Expert MLP between dispatch and combine ("[feat] A5 deep fused moe": the
 * fused operator runs dispatch, GMM1, SwiGLU, requant, GMM2 and combine; its
 * GMM1 A operand is e4m3 with one e8m0 scale per 32 elements).  Each expert e
 * multiplies the receive rows of its block (the first recv_count[e] rows,
 * clamped to [0, block size], or the whole block when recv_count is NULL) by
 * its own weights.  Weights are
 * MXFP8 -- codes [E, N, K] (e4m3) and scale bytes [E, N, K/32] (e8m0, one
 * per 32 consecutive codes of a row) -- packed once by ep_moe_pack_weights
 * into the matrix cores' fragment order (a permutation of the same bytes;
 * the GEMMs read only the packed form).  Products are
 * summed by the MX-scaled matrix cores in float32 accumulators; the
 * instruction adds each 64-product block with less than float32 precision
 * (about 3e-4 of the block's sum of |products|).
 *
 * ep_moe_gmm1: GMM1 + SwiGLU.
 *   x_buf      MXFP8 receive buffer of ep_dispatch (region form), rows = max_rows
 *   hidden     H (K of GMM1), H % 128 == 0
 *   inter      I, I % 64 == 0
 *   w1         packed codes of [E, 2I, H] (gate_up = 1): rows 0..I-1 are the
 *              gate rows, I..2I-1 the up rows;
 *   w1_scales  packed scales of [E, 2I, H/32]
 *   out_quant  EP_QUANT_MXFP8: row r of out_buf (an MXFP8 receive buffer of
 *              width I, region form) gets MXFP8(a) with the MX rule of
 *              dispatch; EP_QUANT_NONE: bf16(a) [max_rows, I]
 *   where a_n = silu(g_n) * u_n in float32, g = gate rows . x, u = up rows . x,
 *   silu(z) = z / (1 + exp(-z)).  Rows holding no pair are not written.
 * ep_moe_gmm2: GMM2.
 *   a_buf      MXFP8 receive buffer of width I (ep_moe_gmm1's output);
 *              I % 128 == 0
 *   w2         packed codes of [E, H, I] (gate_up = 0), w2_scales packed
 *              scales of [E, H, I/32]; H % 128 == 0
 *   out_buf    bf16 [max_rows, H]: row r gets bf16(W2[e] . a_r), the
 *              expert-output rows ep_combine reads (in_quant EP_QUANT_NONE)
 */
/* Bytes of packed codes and packed scales for E experts of N rows of K
 * codes (host only); EP_ERR_INVALID_ARG unless N % 32 == 0, K % 64 == 0. */
ep_status_t ep_moe_packed_bytes(int32_t num_experts, int32_t rows, int32_t k, size_t *codes_bytes,
                                size_t *scales_bytes);

/* Packs MXFP8 weights codes [E, N, K] and scales [E, N, K/32] (device,
 * dense) into packed_codes / packed_scales (device, sizes from
 * ep_moe_packed_bytes, 16-byte aligned).  gate_up = 1 for W1 (N = 2I: a
 * wave's 32 rows are 16 gate rows and the matching 16 up rows), 0 for W2.
 * Layout: for each group of 32 rows and 64-wide K step a 2048-byte
 * fragment, lane l = 32g + r holding K bytes [16g, 16g+16) of the group's
 * row r at 16l and K bytes [32+16g, 48+16g) at 1024 + 16l; for each group
 * and span of four K steps 256 scale bytes, lane l's four at 4l (step
 * 4t+u's K-block 2(4t+u)+g of row r, zero past the last step).  Fragments
 * are ordered by K step, then expert, then group (scale blocks by span,
 * then expert, then group), so the GEMMs need the weights packed for
 * exactly the handle's num_experts experts. */
ep_status_t ep_moe_pack_weights(const void *codes, const void *scales, int32_t num_experts, int32_t rows,
                                int32_t k, int32_t gate_up, void *packed_codes, void *packed_scales,
                                void *stream);

ep_status_t ep_moe_gmm1(const ep_handle_t *handle, const int64_t *recv_count, const void *x_buf,
                        size_t x_buf_bytes, int32_t hidden, int32_t inter, const void *w1,
                        const void *w1_scales, ep_quant_t out_quant, void *out_buf, size_t out_buf_bytes,
                        void *stream);
ep_status_t ep_moe_gmm2(const ep_handle_t *handle, const int64_t *recv_count, const void *a_buf,
                        size_t a_buf_bytes, int32_t inter, int32_t hidden, const void *w2,
                        const void *w2_scales, void *out_buf, size_t out_buf_bytes, void *stream);

/* Waits for `stream` and copies the status word of `handle` (EP_STATUS_*
 * bits) to host *flags. */
ep_status_t ep_read_status(const ep_handle_t *handle, uint32_t *flags, void *stream);

/* Text of the last failed check or runtime error on the calling thread. */
const char *ep_last_error(void);

/* EP_ABI_VERSION of the built library. */
int32_t ep_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EP_H_ */
