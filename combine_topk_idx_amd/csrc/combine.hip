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
//
// The topk_idx given to combine must be the one dispatch was given ("Low-
// Latency Mode API", low_latency_combine Parameters).  The first span
// workgroup of each token checks its k pairs against the handle: a valid id e
// must have its slot inside expert e's block [offsets[e], offsets[e+1]) (or
// slot -1 when blocks have a capacity, for a pair dropped past it), and any
// other id must have slot -1.  A mismatch sets EP_STATUS_COMBINE_MISMATCH; the
// reduction itself always follows the handle's slots.  The ids' loads are
// issued before the row loads and the block bounds' loads after them, so the
// check adds no memory round trip of its own.
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
template <> struct Raw<EP_QUANT_FP8_B128_POW2> { using T = u32x2; };
template <> struct Raw<EP_QUANT_FP8_B128_UE8M0> { using T = u32x2; };

template <int Q> constexpr int kBytesPerVec = sizeof(typename Raw<Q>::T);

// dequantised 8 elements of one row vector; `scale` is the row's float32
// scale (int8), the block's float32 scale (e4m3 per 128, also when it is a
// power of two) or the block's power of two 2^(byte-127) (MX, per-128 e8m0)
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
  } else if constexpr (Q == EP_QUANT_FP8_B128 || Q == EP_QUANT_FP8_B128_POW2) {
    e4m3x8_decode(r, y);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = y[i] * scale;
  } else if constexpr (Q == EP_QUANT_MXFP8 || Q == EP_QUANT_FP8_B128_UE8M0) {
    e4m3x8_decode_scaled(r, scale, y);
  } else {
    e2m1x8_decode_scaled(r, scale, y);
  }
}

// What the routing check needs: the ids and the handle's block bounds.
struct IdCheck {
  const void *idx;              // [T, k] int32 or int64
  int idx64, E, cap;            // cap: the handle's expert_capacity (0: none)
  const int *offsets;           // [E + 1] block starts
  uint32_t *status;
};

template <int Q, int NT, int KMAX, int CV, bool EXACT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void combine_kernel(
    const char *__restrict__ data, const char *__restrict__ scales, int64_t dq, int64_t sq, int nvec, int k,
    int chunks, const int *__restrict__ slot, const float *__restrict__ w, u32x4 *__restrict__ out, IdCheck ic) {
  using RawT = typename Raw<Q>::T;
  const int t = blockIdx.x / chunks;
  const int c = blockIdx.x - t * chunks;
  const int64_t pair0 = (int64_t)t * k;
  // lane j < k of the token's first span workgroup checks pair j
  const bool checker = c == 0 && (int)threadIdx.x < k;
  int64_t my_id = -1;
  if (checker) {
    my_id = ic.idx64 ? ((const int64_t *)ic.idx)[pair0 + threadIdx.x]
                     : (int64_t)((const int32_t *)ic.idx)[pair0 + threadIdx.x];
  }

  // routed rows and weights: loads from valid addresses first, then masking,
  // so the loads are in flight together (with k == KMAX they are contiguous
  // and become one wide scalar load each)
  int s[KMAX];
  float wt[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int jj = EXACT ? j : min(j, k - 1);
    s[j] = slot[pair0 + jj];
    wt[j] = w[pair0 + jj];
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) s[j] = j < k ? s[j] : -1;
  // per-row int8 scales are workgroup-uniform
  float rs[KMAX];
  if constexpr (Q == EP_QUANT_INT8_TOKEN) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) rs[j] = *(const float *)(scales + max(s[j], 0) * sq);
  }

  // this lane's CV consecutive 8-element vectors
  const int v0 = (c * NT + threadIdx.x) * CV;
  const bool active = v0 < nvec;
  if (!active && !checker) return;

  // phase 1: issue every row load (data and scale)
  RawT raw[KMAX][CV];
  uint32_t sraw[KMAX][CV];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
#pragma unroll
    for (int h = 0; h < CV; ++h) {
      raw[j][h] = RawT{};
      sraw[j][h] = 0;
    }
    if (s[j] < 0 || !active) continue;
#pragma unroll
    for (int h = 0; h < CV; ++h) {
      const int v = v0 + h;
      const RawT *src = (const RawT *)(data + s[j] * dq + (int64_t)v * kBytesPerVec<Q>);
#if EP_COMBINE_NT_LOAD
      raw[j][h] = __builtin_nontemporal_load(src);
#else
      raw[j][h] = *src;
#endif
      if constexpr (Q == EP_QUANT_FP8_B128 || Q == EP_QUANT_FP8_B128_POW2) {
        sraw[j][h] = *(const uint32_t *)(scales + s[j] * sq + (int64_t)(v >> 4) * 4);
      } else if constexpr (Q == EP_QUANT_FP8_B128_UE8M0) {
        sraw[j][h] = *(const uint8_t *)(scales + s[j] * sq + (int64_t)(v >> 4));
      } else if constexpr (Q == EP_QUANT_MXFP8 || Q == EP_QUANT_MXFP4) {
        sraw[j][h] = *(const uint8_t *)(scales + s[j] * sq + (int64_t)(v >> 2));
      }
    }
  }
  // the routing check: this lane's slot is s[threadIdx.x] (uniform values)
  if (checker) {
    int my_slot = -1;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) my_slot = j == (int)threadIdx.x ? s[j] : my_slot;
    bool bad;
    if (my_id >= 0 && my_id < (int64_t)ic.E) {
      const int lo = ic.offsets[my_id], hi = ic.offsets[my_id + 1];
      bad = my_slot < 0 ? ic.cap == 0 : (my_slot < lo || my_slot >= hi);
    } else {
      bad = my_slot >= 0;
    }
    if (bad) atomicOr(ic.status, (uint32_t)EP_STATUS_COMBINE_MISMATCH);
  }
  if (!active) return;

  // phase 2: dequantise and accumulate in ascending j
  float acc[CV][8];
#pragma unroll
  for (int h = 0; h < CV; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (s[j] < 0) continue;
#pragma unroll
    for (int h = 0; h < CV; ++h) {
      float sc = 1.0f;
      if constexpr (Q == EP_QUANT_INT8_TOKEN) sc = rs[j];
      else if constexpr (Q == EP_QUANT_FP8_B128 || Q == EP_QUANT_FP8_B128_POW2) sc = __uint_as_float(sraw[j][h]);
      else if constexpr (Q == EP_QUANT_MXFP8 || Q == EP_QUANT_MXFP4 || Q == EP_QUANT_FP8_B128_UE8M0)
        sc = e8m0_decode(sraw[j][h]);
      float y[8];
      dequant8<Q>(raw[j][h], sc, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = acc[h][e] + wt[j] * y[e];
    }
  }
#pragma unroll
  for (int h = 0; h < CV; ++h) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[h][2 * e], acc[h][2 * e + 1]);
#if EP_COMBINE_NT_STORE
    __builtin_nontemporal_store(pin(o), out + (int64_t)t * nvec + v0 + h);
#else
    out[(int64_t)t * nvec + v0 + h] = o;
#endif
  }
}

// `quant` is Q possibly OR-ed with EP_RECV_INTERLEAVED; the kernel takes the
// row strides of data and scales (equal for interleaved rows) and the scale base.
template <int Q, int NT, int KMAX, int CV, bool EXACT>
hipError_t launch_q(const ep_handle_t &h, const char *in, int hidden, const float *w, void *out, int quant,
                    const IdCheck &ic, hipStream_t s) {
  const RecvGeom g = recv_geom(h.max_rows, hidden, quant);
  const int64_t dq = g.data_stride, sq = g.scale_stride;
  const size_t scale_off = g.scale_off;
  const int nvec = hidden / 8;                      // a multiple of 4 (hidden % 32 == 0)
  const int per_block = NT * CV;
  const int chunks = (nvec + per_block - 1) / per_block;
  const int64_t blocks = h.num_tokens * chunks;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((combine_kernel<Q, NT, KMAX, CV, EXACT>), dim3((unsigned)blocks), dim3(NT), EP_COMBINE_LDS_CAP, s, in,
                     in + scale_off, (int64_t)dq, (int64_t)sq, nvec, h.num_topk, chunks, h.slot, w, (u32x4 *)out, ic);
  return hipGetLastError();
}

template <int Q>
hipError_t launch_mode(const ep_handle_t &h, const char *in, int hidden, const float *w, void *out, int quant,
                       const IdCheck &ic, hipStream_t s) {
  constexpr int NT = EP_COMBINE_THREADS, CV = EP_COMBINE_CV;
  if (EP_COMBINE_KMAX_MIN <= 8 && h.num_topk == 8)
    return launch_q<Q, NT, 8, CV, true>(h, in, hidden, w, out, quant, ic, s);
  if (EP_COMBINE_KMAX_MIN <= 8 && h.num_topk < 8)
    return launch_q<Q, NT, 8, CV, false>(h, in, hidden, w, out, quant, ic, s);
  if (h.num_topk == kMaxTopk) return launch_q<Q, NT, kMaxTopk, CV, true>(h, in, hidden, w, out, quant, ic, s);
  return launch_q<Q, NT, kMaxTopk, CV, false>(h, in, hidden, w, out, quant, ic, s);
}

}  // namespace

hipError_t launch_combine(const ep_handle_t &h, const char *in, int quant, int hidden, const void *idx, int idx64,
                          const float *w, void *out, hipStream_t s) {
  const IdCheck ic{idx, idx64, h.num_experts, h.expert_capacity, h.offsets, h.status};
  switch (quant & kQuantMask) {
    case EP_QUANT_NONE: return launch_mode<EP_QUANT_NONE>(h, in, hidden, w, out, quant, ic, s);
    case EP_QUANT_INT8_TOKEN: return launch_mode<EP_QUANT_INT8_TOKEN>(h, in, hidden, w, out, quant, ic, s);
    case EP_QUANT_FP8_B128: return launch_mode<EP_QUANT_FP8_B128>(h, in, hidden, w, out, quant, ic, s);
    case EP_QUANT_MXFP8: return launch_mode<EP_QUANT_MXFP8>(h, in, hidden, w, out, quant, ic, s);
    case EP_QUANT_FP8_B128_POW2: return launch_mode<EP_QUANT_FP8_B128_POW2>(h, in, hidden, w, out, quant, ic, s);
    case EP_QUANT_FP8_B128_UE8M0: return launch_mode<EP_QUANT_FP8_B128_UE8M0>(h, in, hidden, w, out, quant, ic, s);
    default: return launch_mode<EP_QUANT_MXFP4>(h, in, hidden, w, out, quant, ic, s);
  }
}

}  // namespace ep
