// Shared definitions of the HIP library: vector types, wave64 helpers and the
// internal launcher interface between the C ABI (ep_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ep.h"

namespace ep {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxTopk = 16;
constexpr int kMaxExperts = 512;

// the three e4m3 modes with one scale per 128 channels
__host__ __device__ constexpr bool is_b128(int q) {
  return q == EP_QUANT_FP8_B128 || q == EP_QUANT_FP8_B128_POW2 || q == EP_QUANT_FP8_B128_UE8M0;
}
constexpr size_t kScaleAlign = 256;   // scale region alignment inside a receive buffer
constexpr size_t kWsAlign = 256;      // alignment of each workspace sub-array

__host__ __device__ constexpr size_t align_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

// Per-row byte sizes of the receive format (see include/ep.h).
__host__ __device__ inline void row_bytes(int quant, int hidden, size_t *dq, size_t *sq) {
  const size_t H = (size_t)hidden;
  switch (quant) {
    case EP_QUANT_NONE: *dq = 2 * H; *sq = 0; break;
    case EP_QUANT_INT8_TOKEN: *dq = H; *sq = 4; break;
    case EP_QUANT_FP8_B128:
    case EP_QUANT_FP8_B128_POW2: *dq = H; *sq = 4 * (H / 128); break;
    case EP_QUANT_FP8_B128_UE8M0: *dq = H; *sq = H / 128; break;
    case EP_QUANT_MXFP8: *dq = H; *sq = H / 32; break;
    default: *dq = H / 2; *sq = H / 32; break;   // EP_QUANT_MXFP4
  }
}

// Byte offset of the scale region in a receive buffer of `rows` rows (no
// padding when there is no scale region).
__host__ __device__ inline size_t scale_offset(int64_t rows, size_t dq, size_t sq) {
  return sq ? align_up((size_t)rows * dq, kScaleAlign) : (size_t)rows * dq;
}

// A quant argument is the mode in the low byte, possibly OR-ed with
// EP_RECV_INTERLEAVED.
constexpr int kQuantMask = 0xff;
constexpr size_t kInterleavedRowAlign = 128;   // interleaved rows start on cache lines

// Geometry of a receive buffer: byte strides of data rows and of scale rows,
// where the scales start (the scale region, or inside each interleaved row),
// and the total size.
struct RecvGeom {
  int64_t data_stride, scale_stride;
  size_t scale_off, total;
};
__host__ inline RecvGeom recv_geom(int64_t rows, int hidden, int quant) {
  size_t dq, sq;
  row_bytes(quant & kQuantMask, hidden, &dq, &sq);
  RecvGeom g;
  if (quant & EP_RECV_INTERLEAVED) {
    const size_t stride = align_up(dq + sq, kInterleavedRowAlign);
    g.data_stride = g.scale_stride = (int64_t)stride;
    g.scale_off = dq;
    g.total = (size_t)rows * stride;
  } else {
    g.data_stride = (int64_t)dq;
    g.scale_stride = (int64_t)sq;
    g.scale_off = scale_offset(rows, dq, sq);
    g.total = g.scale_off + (size_t)rows * sq;
  }
  return g;
}

// Makes a value opaque to the optimizer at this point (an empty asm that
// claims to modify it).  Used (a) so that codes computed once are not
// re-derived inside every per-row store branch and (b) so that a store built
// from bit-cast conversion results keeps its non-temporal hint (without it the
// optimizer rewrites such a store and drops the hint).
template <typename T>
__device__ __forceinline__ T pin(T v) {
  asm volatile("" : "+v"(v));
  return v;
}

// DPP lane exchanges (wave64, no LDS traffic).  Controls: quad_perm
// [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E; row_ror:n = 0x120 + n (rotate within a
// row of 16 lanes).
__device__ __forceinline__ uint32_t dpp_quad_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_quad_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_row_ror4(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_row_ror8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_row_ror12(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x12C, 0xF, 0xF, false);
}

// max over the 4 lanes of a quad / the 16 lanes of a row, on unsigned values
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = max(v, dpp_quad_xor1(v));
  return max(v, dpp_quad_xor2(v));
}
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = quad_max(v);
  v = max(v, dpp_row_ror4(v));
  return max(v, dpp_row_ror8(v));
}

// ---------------------------------------------------------------------------
// internal launchers (defined in layout.hip / dispatch.hip / combine.hip)
// ---------------------------------------------------------------------------

struct WsLayout {      // byte offsets of the workspace sub-arrays
  size_t offsets, slot, row_src, status, hist, bstat, total;
  int64_t nblocks;     // blocks of the multi-block layout path (0 = single block)
};

// Receive rows of a layout: num_max_tokens * k (+ E * (align - 1) when
// blocks are aligned), or E * cap when every block has cap rows; -1 when
// the arguments are out of range (align outside [1, kMaxRowAlign], cap < 0,
// both set, or more than 2^31 - 1 rows).
constexpr int32_t kMaxRowAlign = 1024;
__host__ inline int64_t layout_rows(int64_t max_tokens, int32_t k, int32_t E, int32_t align, int32_t cap) {
  if (max_tokens < 0 || k <= 0 || E <= 0 || align < 1 || align > kMaxRowAlign || cap < 0 || (cap > 0 && align > 1))
    return -1;
  const int64_t rows = cap > 0 ? (int64_t)E * cap : max_tokens * k + (int64_t)E * (align - 1);
  return rows > INT32_MAX ? -1 : rows;
}

WsLayout workspace_layout(int64_t max_tokens, int32_t k, int32_t E, int64_t max_rows);

hipError_t launch_layout(const void *idx, int idx64, int64_t T, int32_t k, int32_t E, int64_t max_rows, int32_t align,
                         int32_t cap, int64_t *recv_count, int32_t *cum, char *ws, const WsLayout &wl,
                         hipStream_t s);

hipError_t launch_dispatch(const ep_handle_t &h, const void *x, int hidden, const float *w, int quant,
                           char *recv, float *recv_w, hipStream_t s);

hipError_t launch_combine(const ep_handle_t &h, const char *in, int quant, int hidden, const void *idx, int idx64,
                          const float *w, void *out, hipStream_t s);

hipError_t launch_combine_backward(const ep_handle_t &h, const void *grad, int hidden, const float *w, int quant,
                                   char *buf, hipStream_t s);

}  // namespace ep
