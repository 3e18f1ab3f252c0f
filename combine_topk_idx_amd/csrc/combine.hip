// Combine kernel for gfx950: gather each token's expert-output rows,
// dequantise them and reduce them weighted by topk_weights.
//
// ("Low-Latency Mode API", low_latency_combine: the result is the bf16
// weighted sum over the token's experts; "DeepEP FP8 Dispatch and Combine
// Operations", The FP8 Combine Operation: codes times the stored inverse
// scale, through float32.)  Per element:
//   acc = +0;  for j = 0..k-1 with slot[t, j] >= 0:  acc = acc + fl(w[t, j] * y_j)
//   out = bf16_rne(acc)
// in float32 with one rounding per multiply and per add (the library is built
// with -ffp-contract=off, so no fused multiply-add and no reassociation).
//
// Mapping: a workgroup handles one token and a span of its row; a lane owns 8
// consecutive output elements.  Slots and weights are workgroup-uniform
// (scalar loads).  All k row loads of a lane are issued before the first add,
// so a lane has up to k independent 4-16 byte loads in flight; the adds then
// run in ascending j.
#include "common.hpp"
#include "formats.hpp"
#include "tuning.hpp"

namespace ep {

namespace {

template <int Q> struct Raw;
template <> struct Raw<EP_QUANT_NONE> { using T = u32x4; };
template <> struct Raw<EP_QUANT_INT8_TOKEN> { using T = u32x2; };
template <> struct Raw<EP_QUANT_FP8_B128> { using T = u32x2; };
template <> struct Raw<EP_QUANT_MXFP8> { using T = u32x2; };
template <> struct Raw<EP_QUANT_MXFP4> { using T = uint32_t; };

template <int Q> constexpr int kBytesPerVec = sizeof(typename Raw<Q>::T);

// dequantised 8 elements of one row vector; `scale` is the row's float32
// scale (int8), the block's float32 scale (e4m3 per 128) or the block's
// power of two 2^(byte-127) (MX)
template <int Q>
__device__ __forceinline__ void dequant8(const typename Raw<Q>::T &r, float scale, float (&y)[8]) {
  if constexpr (Q == EP_QUANT_NONE) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[2 * i] = bf16_lo(r[i]);
      y[2 * i + 1] = bf16_hi(r[i]);
    }
  } else if constexpr (Q == EP_QUANT_INT8_TOKEN) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = (int)(int8_t)((r[i >> 2] >> (8 * (i & 3))) & 0xffu);
      y[i] = (float)q * scale;
    }
  } else if constexpr (Q == EP_QUANT_FP8_B128) {
    e4m3x8_decode(r, y);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = y[i] * scale;
  } else if constexpr (Q == EP_QUANT_MXFP8) {
    e4m3x8_decode_scaled(r, scale, y);
  } else {
    e2m1x8_decode_scaled(r, scale, y);
  }
}

template <int Q, int NT, int VPT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void combine_kernel(const char *__restrict__ data, const char *__restrict__ scales,
                                                     int64_t dq, int64_t sq, int nvec, int k, int chunks,
                                                     const int *__restrict__ slot, const float *__restrict__ w,
                                                     u32x4 *__restrict__ out) {
  using RawT = typename Raw<Q>::T;
  const int t = blockIdx.x / chunks;
  const int c = blockIdx.x - t * chunks;
  const int64_t pair0 = (int64_t)t * k;

  int s[kMaxTopk];
  float wt[kMaxTopk];
#pragma unroll
  for (int j = 0; j < kMaxTopk; ++j) {
    s[j] = j < k ? slot[pair0 + j] : -1;
    wt[j] = j < k ? w[pair0 + j] : 0.0f;
  }
  // per-row int8 scales are workgroup-uniform
  float rs[kMaxTopk];
  if constexpr (Q == EP_QUANT_INT8_TOKEN) {
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) rs[j] = s[j] >= 0 ? *(const float *)(scales + s[j] * sq) : 0.0f;
  }

  const int v0 = c * NT * VPT + threadIdx.x;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = v0 + i * NT;
    if (v >= nvec) continue;
    // phase 1: issue every row load (data and scale) of this vector
    RawT raw[kMaxTopk];
    uint32_t sraw[kMaxTopk];
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      raw[j] = RawT{};
      sraw[j] = 0;
      if (s[j] < 0) continue;
      const RawT *src = (const RawT *)(data + s[j] * dq + (int64_t)v * kBytesPerVec<Q>);
#if EP_COMBINE_NT_LOAD
      raw[j] = __builtin_nontemporal_load(src);
#else
      raw[j] = *src;
#endif
      if constexpr (Q == EP_QUANT_FP8_B128) {
        sraw[j] = *(const uint32_t *)(scales + s[j] * sq + (int64_t)(v >> 4) * 4);
      } else if constexpr (Q == EP_QUANT_MXFP8 || Q == EP_QUANT_MXFP4) {
        sraw[j] = *(const uint8_t *)(scales + s[j] * sq + (int64_t)(v >> 2));
      }
    }
    // phase 2: dequantise and accumulate in ascending j
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxTopk; ++j) {
      if (s[j] < 0) continue;
      float sc = 1.0f;
      if constexpr (Q == EP_QUANT_INT8_TOKEN) sc = rs[j];
      else if constexpr (Q == EP_QUANT_FP8_B128) sc = __uint_as_float(sraw[j]);
      else if constexpr (Q == EP_QUANT_MXFP8 || Q == EP_QUANT_MXFP4) sc = e8m0_decode(sraw[j]);
      float y[8];
      dequant8<Q>(raw[j], sc, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] + wt[j] * y[e];
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
#if EP_COMBINE_NT_STORE
    __builtin_nontemporal_store(o, out + (int64_t)t * nvec + v);
#else
    out[(int64_t)t * nvec + v] = o;
#endif
  }
}

template <int Q, int NT, int VPT>
hipError_t launch_q(const ep_handle_t &h, const char *in, int hidden, const float *w, void *out, hipStream_t s) {
  size_t dq, sq;
  row_bytes(Q, hidden, &dq, &sq);
  const size_t scale_off = scale_offset(h.max_rows, dq, sq);
  const int nvec = hidden / 8;
  const int chunks = (nvec + NT * VPT - 1) / (NT * VPT);
  const int64_t blocks = h.num_tokens * chunks;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((combine_kernel<Q, NT, VPT>), dim3((unsigned)blocks), dim3(NT), 0, s, in, in + scale_off,
                     (int64_t)dq, (int64_t)sq, nvec, h.num_topk, chunks, h.slot, w, (u32x4 *)out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const ep_handle_t &h, const char *in, int quant, int hidden, const float *w, void *out,
                          hipStream_t s) {
  constexpr int NT = EP_COMBINE_THREADS, VPT = EP_COMBINE_VPT;
  switch (quant) {
    case EP_QUANT_NONE: return launch_q<EP_QUANT_NONE, NT, VPT>(h, in, hidden, w, out, s);
    case EP_QUANT_INT8_TOKEN: return launch_q<EP_QUANT_INT8_TOKEN, NT, VPT>(h, in, hidden, w, out, s);
    case EP_QUANT_FP8_B128: return launch_q<EP_QUANT_FP8_B128, NT, VPT>(h, in, hidden, w, out, s);
    case EP_QUANT_MXFP8: return launch_q<EP_QUANT_MXFP8, NT, VPT>(h, in, hidden, w, out, s);
    default: return launch_q<EP_QUANT_MXFP4, NT, VPT>(h, in, hidden, w, out, s);
  }
}

}  // namespace ep
