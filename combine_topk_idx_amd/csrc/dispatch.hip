// Dispatch kernel for gfx950: read each bf16 token row once, quantise it once,
// write the packed row (and its scales) to every receive row it is routed to.
//
// Quantisation ("Low-Latency Mode API", Parameters use_fp8 / use_ue8m0 /
// use_mxfp4; "DeepEP FP8 Dispatch and Combine Operations", The Dispatch
// Stage), all in float32 with one rounding per operation:
//   INT8_TOKEN  amax over the row;  m = 127/amax, scale = amax/127,
//               code = clamp(rint(x*m), +-127)
//   FP8_B128    the same per 128 channels with 448, code = e4m3(clamp(x*m))
//   FP8_B128_POW2 / _UE8M0  per 128 channels: s0 = amax/448, scale 2^e with
//               e = ceil(log2 s0) (bits of s0), code = e4m3(clamp(x*2^-e));
//               the scale is stored as float32 or as the byte e+127; e < -127
//               counts as a zero block
//   MXFP8/MXFP4 per 32 elements: shared exponent clamp(floor(log2 amax) -
//               emax, +-127) (emax 8 for e4m3, 2 for e2m1), byte = exp+127,
//               code = enc(clamp(x * 2^-exp, +-max))
// A block whose amax is 0, or whose multiplier overflows, stores scale 0 and
// zero codes.
//
// Mapping: a workgroup handles one token and a contiguous span of its row; a
// lane owns 8 consecutive elements (one 16-byte load).  An MX block is 4
// adjacent lanes and a 128-channel block 16 adjacent lanes, so block maxima
// are DPP exchanges inside a quad or a 16-lane row; the int8 row maximum is a
// workgroup reduction.  Routed rows and weights are read once per workgroup
// (scalar loads).  Code rows are written with non-temporal stores, scale
// pieces through L2.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "dispatch.hpp"
#include "formats.hpp"
#include "tuning.hpp"

namespace ep {

namespace {

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// largest |x| of the 8 bf16 elements of a vector, as the bits of a
// non-negative bf16 (unsigned order == float order for these); packed
// 16-bit max over the four words, then the two halves
__device__ __forceinline__ uint32_t vec_absmax_bits(const u32x4 &r) {
  u16x2 m = __builtin_bit_cast(u16x2, r[0] & 0x7fff7fffu);
#pragma unroll
  for (int i = 1; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, r[i] & 0x7fff7fffu));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

__device__ __forceinline__ void unpack8(const u32x4 &r, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(r[i]);
    f[2 * i + 1] = bf16_hi(r[i]);
  }
}

// Scaled-integer style block (INT8 / FP8_B128): multiplier and stored scale.
struct ScaledBlock {
  float m, scale;
  bool zero;
};
__device__ __forceinline__ ScaledBlock scaled_block(uint32_t amax_bits, float qmax) {
  const float amax = __uint_as_float(amax_bits << 16);
  ScaledBlock b;
  b.m = qmax / amax;
  b.scale = amax / qmax;
  b.zero = (amax_bits == 0) || __builtin_isinf(b.m);
  if (b.zero) b.scale = 0.0f;
  return b;
}

// Per-128 power-of-two block: s0 = fl(amax/448) rounded up to 2^e.  m = 2^-e
// and scale = 2^e are exact float32 (e >= -127 keeps 2^-e finite; e <= 120
// for finite bf16 input); `byte` receives the e8m0 code e + 127.
__device__ __forceinline__ ScaledBlock pow2_block(uint32_t amax_bits, uint32_t &byte) {
  const float amax = __uint_as_float(amax_bits << 16);
  const uint32_t s0 = __float_as_uint(amax / 448.0f);
  const int e = s0 ? ceil_log2_bits(s0) : 0;
  ScaledBlock b;
  b.zero = amax_bits == 0 || e < -127;
  const int ec = b.zero ? 0 : e;
  b.m = __uint_as_float((uint32_t)(127 - ec) << 23);
  b.scale = b.zero ? 0.0f : (ec == -127 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)(ec + 127) << 23));
  byte = b.zero ? 0u : (uint32_t)(ec + 127);
  return b;
}

__device__ __forceinline__ u32x2 codes_int8(const float (&f)[8], const ScaledBlock &b) {
  uint32_t w[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float v = fminf(fmaxf(f[i] * b.m, -127.0f), 127.0f);
    const int q = b.zero ? 0 : (int)__builtin_rintf(v);
    w[i >> 2] |= ((uint32_t)q & 0xffu) << (8 * (i & 3));
  }
  return u32x2{w[0], w[1]};
}

// e4m3 codes of fl(x*m) clamped to +-448; a zero block stores +0 codes
__device__ __forceinline__ u32x2 codes_e4m3_scaled(const float (&f)[8], const ScaledBlock &b) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = fminf(fmaxf(f[i] * b.m, -448.0f), 448.0f);
    v[i] = b.zero ? 0.0f : v[i];
  }
  return e4m3x8_encode(v);
}

// MX shared exponent of a block from its amax bits (bf16 pattern): returns
// the e8m0 byte, 2^-exp in `mult` and 2^exp in `scale` (both exact float32;
// exp = -127 makes `scale` the subnormal 2^-127).
__device__ __forceinline__ uint32_t mx_scale(uint32_t amax_bits, int emax, float &mult, float &scale) {
  int se = -127;
  if (amax_bits != 0) {
    se = floor_log2_bits(amax_bits << 16) - emax;
    se = se < -127 ? -127 : (se > 127 ? 127 : se);
  }
  // se <= 127 - emax for finite bf16 input, so 2^-se is a normal float32
  mult = __uint_as_float((uint32_t)(127 - se) << 23);
  scale = se == -127 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)(se + 127) << 23);
  return (uint32_t)(se + 127);
}

__device__ __forceinline__ u32x2 codes_mxfp8(const float (&f)[8], float mult) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = fminf(fmaxf(f[i] * mult, -448.0f), 448.0f);
  return e4m3x8_encode(v);
}

// Code rows are written once and read by a later kernel: non-temporal stores
// keep them from displacing other lines on the way.  A scale piece is 1-4
// bytes of a 32-128 byte scale row that 4-16 workgroups on different XCDs
// write, so it goes through L2, which merges the pieces into whole lines.
template <typename T>
__device__ __forceinline__ void st_data(char *p, const T &v) {
#if EP_DISPATCH_NT_DATA
  __builtin_nontemporal_store(v, (T *)p);
#else
  *(T *)p = v;
#endif
}
template <typename T>
__device__ __forceinline__ void st_scale(char *p, const T &v) {
  *(T *)p = v;
}

// Workgroup max of one unsigned per thread (NT threads).
template <int NT>
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t *red) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, d));
  const int w = threadIdx.x / kWave;
  __syncthreads();   // `red` may still be read by a previous call
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) m = max(m, red[i]);
  return m;
}

// bf16(fl32(w * x)) of the 8 bf16 elements of a vector (round to nearest even)
__device__ __forceinline__ u32x4 scale_bf16x8(const u32x4 &r, float w) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(w * bf16_lo(r[i]), w * bf16_hi(r[i]));
  return o;
}

// Reverse dispatch in MXFP8: row s[j] receives, per 32-element block, the
// MX codes of bf16(fl32(w[j] * g)).  Worked from the float32 products, with
// no unpacking of rounded values: the block maximum of |w g| rounded to bf16
// is the maximum of the rounded values (rounding is monotonic), and clamping
// to +-448 * 2^se before the rounding gives what clamping after it gives
// (448 * 2^se is itself a bf16 value), so the clamped, rounded pairs go
// straight to the scaled e4m3 conversion, which divides by 2^se exactly and
// rounds to nearest even (tests/test_gpu_codecs.py compares it with the
// software encoder of the exact quotient for every finite bf16 pattern and
// every se; past +-448 it would give NaN, hence the clamp).
typedef short s16x2 __attribute__((ext_vector_type(2)));
template <int NT, int VPT, int KMAX, bool PACK>
__device__ __forceinline__ void weighted_mxfp8_store(const u32x4 (&raw)[VPT], int v0, int nvec, const int (&s)[KMAX],
                                                     const float (&wj)[KMAX], char *__restrict__ data,
                                                     char *__restrict__ scales, int64_t dq, int64_t sq) {
  float g[VPT][8];
#pragma unroll
  for (int i = 0; i < VPT; ++i) unpack8(raw[i], g[i]);
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (s[j] < 0) continue;   // uniform
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = v0 + i * NT;
      float p[8];
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = wj[j] * g[i][e];
        m = fmaxf(m, fabsf(p[e]));
      }
      float mult, scale;
      const uint32_t sbyte = mx_scale(quad_max(pack_bf16x2(m, 0.0f) & 0xffffu), 8, mult, scale);
      // scale bytes of the row's four blocks into its first lane (a row
      // rotation by n hands lane l the value of lane l - n, modulo 16)
      const uint32_t sword = PACK ? sbyte | (dpp_row_ror12(sbyte) << 8) | (dpp_row_ror8(sbyte) << 16) |
                                        (dpp_row_ror4(sbyte) << 24)
                                  : sbyte;
      if (v >= nvec) continue;
      const float lim = 448.0f * scale;
      uint32_t wd[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        wd[k] = pack_bf16x2(__builtin_amdgcn_fmed3f(p[2 * k], -lim, lim), __builtin_amdgcn_fmed3f(p[2 * k + 1], -lim, lim));
      s16x2 o0 = {0, 0}, o1 = {0, 0};
      o0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o0, __builtin_bit_cast(bf16x2, wd[0]), scale, false);
      o0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o0, __builtin_bit_cast(bf16x2, wd[1]), scale, true);
      o1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o1, __builtin_bit_cast(bf16x2, wd[2]), scale, false);
      o1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o1, __builtin_bit_cast(bf16x2, wd[3]), scale, true);
      const u32x2 q = pin(u32x2{__builtin_bit_cast(uint32_t, o0), __builtin_bit_cast(uint32_t, o1)});
      st_data(data + s[j] * dq + (int64_t)v * 8, q);
      if (PACK ? (v & 15) == 0 : (v & 3) == 0) {
        char *sp = scales + s[j] * sq + (int64_t)(v >> 2);
        if constexpr (PACK) st_scale(sp, sword);
        else st_scale(sp, (uint8_t)sbyte);
      }
    }
  }
}

// Quantises this thread's VPT row vectors (vector v0 + i*NT of one token row)
// and stores the packed codes and scales to every receive row s[j] >= 0 with
// j0 <= j < j1.  Every thread of the workgroup calls it (the int8 row maximum
// is a workgroup reduction through `red`).
template <int Q, int NT, int VPT, int KMAX, bool PACK>
__device__ __forceinline__ void quantize_store(const u32x4 (&raw)[VPT], int v0, int nvec, const int (&s)[KMAX],
                                               int j0, int j1, char *__restrict__ data, char *__restrict__ scales,
                                               int64_t dq, int64_t sq, uint32_t *red) {
  auto routed = [&](int j) { return j >= j0 && j < j1 && s[j] >= 0; };
  if constexpr (Q == EP_QUANT_NONE) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = v0 + i * NT;
      if (v >= nvec) continue;
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (routed(j)) st_data(data + s[j] * dq + (int64_t)v * 16, raw[i]);
    }
  } else if constexpr (Q == EP_QUANT_INT8_TOKEN) {
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < VPT; ++i) am = max(am, vec_absmax_bits(raw[i]));
    const ScaledBlock b = scaled_block(block_max<NT>(am, red), 127.0f);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = v0 + i * NT;
      if (v >= nvec) continue;
      float f[8];
      unpack8(raw[i], f);
      const u32x2 q = pin(codes_int8(f, b));
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (routed(j)) st_data(data + s[j] * dq + (int64_t)v * 8, q);
    }
    if (threadIdx.x == 0) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (routed(j)) st_scale(scales + s[j] * sq, b.scale);
    }
  } else {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = v0 + i * NT;
      const uint32_t am = vec_absmax_bits(raw[i]);
      if constexpr (is_b128(Q)) {
        float f[8];
        unpack8(raw[i], f);
        const uint32_t bmax = row16_max(am);                          // all 16 lanes
        uint32_t sbyte = 0;
        ScaledBlock b;
        if constexpr (Q == EP_QUANT_FP8_B128) b = scaled_block(bmax, 448.0f);
        else b = pow2_block(bmax, sbyte);
        if (v >= nvec) continue;
        const u32x2 q = pin(codes_e4m3_scaled(f, b));
        const bool lead = (v & 15) == 0;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (!routed(j)) continue;
          st_data(data + s[j] * dq + (int64_t)v * 8, q);
          if (lead) {
            if constexpr (Q == EP_QUANT_FP8_B128_UE8M0) st_scale(scales + s[j] * sq + (int64_t)(v >> 4), (uint8_t)sbyte);
            else st_scale(scales + s[j] * sq + (int64_t)(v >> 4) * 4, b.scale);
          }
        }
      } else {
        constexpr int emax = Q == EP_QUANT_MXFP8 ? 8 : 2;
        float mult, scale;
        const uint32_t sbyte = mx_scale(quad_max(am), emax, mult, scale);
        uint32_t sword = sbyte;
        if constexpr (PACK) {
          // gather the scale bytes of 4 consecutive blocks (lanes 0, 4, 8, 12
          // of each 16-lane row) into one dword held by the row's first lane;
          // only used when every 16-lane row is fully inside the row
          // (hidden % 128 == 0), which also makes the dword store aligned
          const int lane = threadIdx.x & (kWave - 1);
          const int rbase = lane & ~15;
          const uint32_t b1 = (uint32_t)__shfl((int)sbyte, rbase + 4);
          const uint32_t b2 = (uint32_t)__shfl((int)sbyte, rbase + 8);
          const uint32_t b3 = (uint32_t)__shfl((int)sbyte, rbase + 12);
          sword = sbyte | (b1 << 8) | (b2 << 16) | (b3 << 24);
        }
        if (v >= nvec) continue;
        const bool lead = PACK ? (v & 15) == 0 : (v & 3) == 0;
        constexpr int kBytes = Q == EP_QUANT_MXFP8 ? 8 : 4;
        using Codes = typename std::conditional<Q == EP_QUANT_MXFP8, u32x2, uint32_t>::type;
        Codes q;
        if constexpr (Q == EP_QUANT_MXFP8) {
          float f[8];
          unpack8(raw[i], f);
          q = pin(codes_mxfp8(f, mult));
        } else {
          q = pin(e2m1x8_encode_bf16(raw[i], scale));
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (!routed(j)) continue;
          st_data(data + s[j] * dq + (int64_t)v * kBytes, q);
          if (lead) {
            char *sp = scales + s[j] * sq + (int64_t)(v >> 2);
            if constexpr (PACK) st_scale(sp, sword);
            else st_scale(sp, (uint8_t)sbyte);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Layout fused into dispatch (compact rows or capacity blocks, few pairs).
//
// In the compact arrangement the receive row of pair f with expert e is
// (pairs with an expert below e) + (earlier pairs with expert e): the
// exclusive scan of the expert counts plus the stable rank ("Low-Latency Mode
// API", Return Values recv_count and the receive layout it describes).  With
// blocks of a fixed capacity C (the page's [experts, max tokens, hidden]
// receive buffer) it is e * C + (earlier pairs with expert e), and a pair whose
// rank reaches C is dropped.  Both are counts over the ids, so a dispatch
// workgroup can find the rows of its token's pairs by itself, with no wait on
// another workgroup, while its span of the token row is in flight.
//
// The first `lwg` workgroups are layout workgroups.  Compact (lwg = 1): it
// writes the per-expert outputs (counts, block starts, running statistics,
// status) and marks the rows past the last routed one free up to n = T * k;
// every span workgroup marks a share of the rows from n to the end free.
// Capacity: each layout workgroup counts the ids per expert and marks the
// free tail of every lwg-th block; the first also writes the per-expert
// outputs.  The first span workgroup of each token writes the token's slots,
// row_src entries and receive weights.
struct FusedArgs {
  const void *idx;     // [n] int32 or int64 ids
  int idx64, n, E, max_rows;
  int cap;             // 0 (compact rows) or the rows of every expert block
  int lwg;             // layout workgroups at the front of the grid
  int64_t *recv_count; // [E]
  int32_t *cum;        // [E] or null
  int32_t *offsets;    // [E + 1]
  int32_t *slot;       // [n]
  int32_t *row_src;    // [max_rows]
  uint32_t *status;
};

// Expert of an id, or `none` for -1 and for ids outside [-1, E) (`bad`).
template <typename IdT>
__device__ __forceinline__ int expert_or(IdT v, int E, int none, bool &bad) {
  if (v >= 0 && (int64_t)v < (int64_t)E) return (int)v;
  bad |= v != -1;
  return none;
}
constexpr int kIdBatch = 8;   // id loads a thread keeps in flight

// Sum of v over the 64 lanes of the wave (every lane gets it), by DPP steps:
// row_shr 1, 2, 4, 8 leave in lane 15 of each 16-lane row the row's sum
// (with zero for sources past the row start), row_bcast 15 adds row r's last
// lane into row r + 1 and row_bcast 31 adds lane 31 into rows 2 and 3, so
// lane 63 ends with the total.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);   // row_bcast:15, rows 1, 3
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);   // row_bcast:31, rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Exclusive scan of one int per thread over an NT-thread workgroup; `total`
// receives the sum.  `wsum` is LDS of NT / 64 ints.
template <int NT>
__device__ __forceinline__ int block_exclusive_sum(int v, int *wsum, int &total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) wsum[w] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) {
    const int c = wsum[i];
    all += c;
    before += i < w ? c : 0;
  }
  total = all;
  return before + x - v;
}

// Layout workgroup lw of the fused launch: expert histogram (LDS atomics).
// Compact (lw = 0 only): its exclusive scan, the per-expert outputs, the
// status word and the free rows below n (all of them when there is no token,
// hence no span workgroup).  Capacity: the free tail of every lwg-th block
// from block lw, and from lw = 0 the per-expert outputs and the status word.
template <int NT, bool CAPM, typename IdT>
__device__ __forceinline__ void fused_layout_outputs(const FusedArgs &a, int lw) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int wsum[NT / kWave];
  __shared__ uint32_t sbad;
  const IdT *idx = (const IdT *)a.idx;
  for (int e = threadIdx.x; e < a.E; e += NT) cnt[e] = 0;
  if (threadIdx.x == 0) sbad = 0;
  __syncthreads();
  bool bad = false;
  for (int base = threadIdx.x; base < a.n; base += kIdBatch * NT) {
    IdT v[kIdBatch];
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) v[u] = idx[min(base + u * NT, a.n - 1)];
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      if (base + u * NT >= a.n) break;
      const int e = expert_or(v[u], a.E, -1, bad);
      if (e >= 0) atomicAdd(&cnt[e], 1);
    }
  }
  if (bad) atomicOr(&sbad, EP_STATUS_ID_OUT_OF_RANGE);
  __syncthreads();
  if constexpr (CAPM) {
    // block e holds rows [e * cap, (e + 1) * cap); the first min(count, cap)
    // hold pairs
    for (int e = lw; e < a.E; e += a.lwg) {
      const int hi = (e + 1) * a.cap;
      for (int r = e * a.cap + min(cnt[e], a.cap) + (int)threadIdx.x; r < hi; r += NT) a.row_src[r] = -1;
    }
    if (lw != 0) return;
    bool over = false;
    for (int e = threadIdx.x; e < a.E; e += NT) {
      const int c = cnt[e];
      a.offsets[e] = e * a.cap;
      a.recv_count[e] = min(c, a.cap);
      if (a.cum) a.cum[e] += c;
      over |= c > a.cap;
    }
    if (over) atomicOr(&sbad, EP_STATUS_CAPACITY_OVERFLOW);
    __syncthreads();
    if (threadIdx.x == 0) {
      a.offsets[a.E] = a.E * a.cap;
      *a.status = sbad;
    }
    return;
  }
  // thread i owns experts [i * per, (i + 1) * per)
  const int per = (a.E + NT - 1) / NT;
  const int e0 = threadIdx.x * per, e1 = min(e0 + per, a.E);
  int mine = 0;
  for (int e = e0; e < e1; ++e) mine += cnt[e];
  int nrows;
  int run = block_exclusive_sum<NT>(mine, wsum, nrows);
  for (int e = e0; e < e1; ++e) {
    const int c = cnt[e];
    a.offsets[e] = run;
    a.recv_count[e] = c;
    if (a.cum) a.cum[e] += c;
    run += c;
  }
  if (threadIdx.x == 0) {
    a.offsets[a.E] = nrows;
    *a.status = sbad;
  }
  // free rows below n; the span workgroups clear [n, max_rows), unless there
  // are none (no tokens)
  const int end = gridDim.x > 1 ? a.n : a.max_rows;
  for (int r = nrows + threadIdx.x; r < end; r += NT) a.row_src[r] = -1;
}

// Receive rows of the pairs of token t (s[j] = -1 past k and for pairs with
// no valid expert).  With n < 4096, pair f with expert e has the order key
// e * 4096 + f, and the ids that order before pair j are those with a smaller
// key (ids with no valid expert get a key above all others).  Every thread counts,
// over its share of the ids, the keys below each pair's key (one compare and
// one add per id and pair); the counts are packed two per word (16 bits
// each) and summed over the wave (DPP) and then, through `red` (LDS of NT / 64 *
// KMAX / 2 words), over the workgroup.
template <int NT, int KMAX, bool EXACT, typename IdT>
__device__ __forceinline__ void fused_slots(const FusedArgs &a, int t, int k, int (&s)[KMAX], uint32_t *red) {
  static_assert(kFusedMaxPairs < 4096, "order keys hold the pair index in 12 bits; counts fit 16 bits");
  const IdT *idx = (const IdT *)a.idx;
  const int f0 = t * k;
  // the first batch of ids is loaded before the token's own ids, so that the
  // two loads are in flight together (this workgroup is called with n >= 1)
  IdT v[kIdBatch];
#pragma unroll
  for (int u = 0; u < kIdBatch; ++u) v[u] = idx[min(u * NT + (int)threadIdx.x, a.n - 1)];
  int key[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const IdT e = idx[f0 + (EXACT ? j : min(j, k - 1))];
    const bool ok = j < k && e >= 0 && (int64_t)e < (int64_t)a.E;
    key[j] = ok ? (int)e * 4096 + f0 + j : -1;   // -1: nothing orders before it
  }
  int cnt[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) cnt[j] = 0;
  for (int b0 = 0;;) {
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      const int f = b0 + u * NT + threadIdx.x;
      const bool ok = f < a.n && v[u] >= 0 && (int64_t)v[u] < (int64_t)a.E;
      const int kf = ok ? (int)v[u] * 4096 + f : 1 << 30;   // above every valid key
      // kf < key[j] as the sign of a difference that cannot overflow (keys
      // lie in [-1, 2^21)): plain vector arithmetic, no lane masks
#pragma unroll
      for (int j = 0; j < KMAX; ++j) cnt[j] += (int)(((uint32_t)kf - (uint32_t)key[j]) >> 31);
    }
    b0 += kIdBatch * NT;
    if (b0 >= a.n) break;
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) v[u] = idx[min(b0 + u * NT + (int)threadIdx.x, a.n - 1)];
  }
  uint32_t acc[KMAX / 2];
#pragma unroll
  for (int i = 0; i < KMAX / 2; ++i) {
    acc[i] = wave_sum((uint32_t)cnt[2 * i] | ((uint32_t)cnt[2 * i + 1] << 16));
  }
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
#pragma unroll
    for (int i = 0; i < KMAX / 2; ++i) red[w * (KMAX / 2) + i] = acc[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < KMAX / 2; ++i) {
    uint32_t sum = 0;
#pragma unroll
    for (int ww = 0; ww < NT / kWave; ++ww) sum += red[ww * (KMAX / 2) + i];
    acc[i] = sum;
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) s[j] = key[j] >= 0 ? (int)((acc[j / 2] >> (16 * (j & 1))) & 0xffffu) : -1;
}

// Capacity blocks: the receive rows of the pairs of token t as above, but
// counting only the keys in [e * 4096, key) -- the earlier pairs with the same
// expert -- so that the row is e * cap + that rank, or -1 once the rank
// reaches cap.  (Kept apart from the compact form, whose code it would
// otherwise change.)
template <int NT, int KMAX, bool EXACT, typename IdT>
__device__ __forceinline__ void fused_slots_cap(const FusedArgs &a, int t, int k, int (&s)[KMAX], uint32_t *red) {
  static_assert(kFusedMaxPairs < 4096, "order keys hold the pair index in 12 bits; counts fit 16 bits");
  const IdT *idx = (const IdT *)a.idx;
  const int f0 = t * k;
  // the first batch of ids is loaded before the token's own ids, so that the
  // two loads are in flight together (this workgroup is called with n >= 1)
  IdT v[kIdBatch];
#pragma unroll
  for (int u = 0; u < kIdBatch; ++u) v[u] = idx[min(u * NT + (int)threadIdx.x, a.n - 1)];
  int key[KMAX], lo[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const IdT e = idx[f0 + (EXACT ? j : min(j, k - 1))];
    const bool ok = j < k && e >= 0 && (int64_t)e < (int64_t)a.E;
    key[j] = ok ? (int)e * 4096 + f0 + j : -1;   // -1: nothing orders before it
    lo[j] = ok ? (int)e * 4096 : 0;
  }
  int cnt[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) cnt[j] = 0;
  for (int b0 = 0;;) {
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      const int f = b0 + u * NT + threadIdx.x;
      const bool ok = f < a.n && v[u] >= 0 && (int64_t)v[u] < (int64_t)a.E;
      const int kf = ok ? (int)v[u] * 4096 + f : 1 << 30;   // above every valid key
      // kf < key[j] as the sign of a difference that cannot overflow (keys
      // lie in [-1, 2^21)): plain vector arithmetic, no lane masks
#pragma unroll
      for (int j = 0; j < KMAX; ++j)   // lo[j] <= kf < key[j], both as signs of differences
        cnt[j] += (int)((((uint32_t)kf - (uint32_t)key[j]) >> 31) & ~(((uint32_t)kf - (uint32_t)lo[j]) >> 31));
    }
    b0 += kIdBatch * NT;
    if (b0 >= a.n) break;
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) v[u] = idx[min(b0 + u * NT + (int)threadIdx.x, a.n - 1)];
  }
  uint32_t acc[KMAX / 2];
#pragma unroll
  for (int i = 0; i < KMAX / 2; ++i) {
    acc[i] = wave_sum((uint32_t)cnt[2 * i] | ((uint32_t)cnt[2 * i + 1] << 16));
  }
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
#pragma unroll
    for (int i = 0; i < KMAX / 2; ++i) red[w * (KMAX / 2) + i] = acc[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < KMAX / 2; ++i) {
    uint32_t sum = 0;
#pragma unroll
    for (int ww = 0; ww < NT / kWave; ++ww) sum += red[ww * (KMAX / 2) + i];
    acc[i] = sum;
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int c = (int)((acc[j / 2] >> (16 * (j & 1))) & 0xffffu);
    s[j] = key[j] >= 0 && c < a.cap ? (key[j] >> 12) * a.cap + c : -1;
  }
}


// FUSED: workgroups b < lwg are the layout workgroups (above) and workgroup
// b >= lwg is span workgroup b - lwg, which derives its token's slots from
// the ids instead of reading them.
// FUSED (compact rows): workgroup 0 writes the layout's per-expert outputs
// and workgroup b > 0 is span workgroup b - 1, which derives its token's
// slots from the ids (above) instead of reading them.
template <int Q, int NT, int VPT, int KMAX, bool EXACT, bool PACK, bool WEIGHTED, bool FUSED>
__global__ __launch_bounds__(NT) void dispatch_kernel(const u32x4 *__restrict__ x, int nvec, int k, int chunks,
                                                      const int *__restrict__ slot,
                                                      const float *__restrict__ w, float *__restrict__ recv_w,
                                                      char *__restrict__ data, char *__restrict__ scales,
                                                      int64_t dq, int64_t sq, FusedArgs fa) {
  __shared__ uint32_t red[NT / kWave * (FUSED ? KMAX / 2 : 1)];
  int b = blockIdx.x;
  if constexpr (FUSED) {
    if (b == 0) {
      if (fa.idx64) fused_layout_outputs<NT, false, int64_t>(fa, 0);
      else fused_layout_outputs<NT, false, int32_t>(fa, 0);
      return;
    }
    b -= 1;
    // rows at or past n (= T * k) never hold a pair; with a capacity far
    // above T there can be many, so every span workgroup clears a share
    const int stride = ((int)gridDim.x - 1) * NT;
    for (int r = fa.n + b * NT + (int)threadIdx.x; r < fa.max_rows; r += stride) fa.row_src[r] = -1;
  }
  const int t = b / chunks;
  const int c = b - t * chunks;
  const int64_t pair0 = (int64_t)t * k;

  // the token's span is loaded first and the routed rows right after, before
  // either is needed, so the two loads are in flight together (at decode
  // sizes each is a memory round trip of the kernel's short life)
  const u32x4 *xr = x + (int64_t)t * nvec;
  const int v0 = c * NT * VPT + threadIdx.x;
  u32x4 raw[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = v0 + i * NT;
    raw[i] = v < nvec ? xr[v] : u32x4{0u, 0u, 0u, 0u};
  }
  // routed rows: loads from valid addresses first, then masking, so the loads
  // are in flight together (with k == KMAX they are one wide scalar load)
  int s[KMAX];
  float wj[KMAX];
  if constexpr (FUSED) {
    if (fa.idx64) fused_slots<NT, KMAX, EXACT, int64_t>(fa, t, k, s, red);
    else fused_slots<NT, KMAX, EXACT, int32_t>(fa, t, k, s, red);
    if (c == 0 && threadIdx.x < k) {
      int r = -1;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) r = j == (int)threadIdx.x ? s[j] : r;
      fa.slot[pair0 + threadIdx.x] = r;
      if (r >= 0) {
        fa.row_src[r] = (int)pair0 + threadIdx.x;
        if (recv_w != nullptr) recv_w[r] = w[pair0 + threadIdx.x];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int jj = EXACT ? j : min(j, k - 1);
      s[j] = slot[pair0 + jj];
      if constexpr (WEIGHTED) wj[j] = w[pair0 + jj];
    }
  }
  bool any = false;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    s[j] = j < k ? s[j] : -1;
    any |= s[j] >= 0;
  }
  if (!any) return;   // uniform: the token is routed nowhere
  if (!FUSED && !WEIGHTED && recv_w != nullptr && c == 0 && threadIdx.x < k) {
    const int r = slot[pair0 + threadIdx.x];
    if (r >= 0) recv_w[r] = w[pair0 + threadIdx.x];
  }

  if constexpr (!WEIGHTED) {
    quantize_store<Q, NT, VPT, KMAX, PACK>(raw, v0, nvec, s, 0, KMAX, data, scales, dq, sq, red);
  } else if constexpr (Q == EP_QUANT_MXFP8) {
    weighted_mxfp8_store<NT, VPT, KMAX, PACK>(raw, v0, nvec, s, wj, data, scales, dq, sq);
  } else {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (s[j] < 0) continue;   // uniform
      u32x4 sr[VPT];
#pragma unroll
      for (int i = 0; i < VPT; ++i) sr[i] = scale_bf16x8(raw[i], wj[j]);
      quantize_store<Q, NT, VPT, KMAX, PACK>(sr, v0, nvec, s, j, j + 1, data, scales, dq, sq, red);
    }
  }
}

// The one launch of layout + dispatch for capacity blocks: workgroups b <
// fa.lwg are layout workgroups, workgroup b >= fa.lwg is span workgroup
// b - fa.lwg.  The same steps as the fused form of dispatch_kernel, with the
// capacity rows; kept as a kernel of its own (rather than a flag of a shared
// body) because sharing the body changed the compact kernel's register
// allocation and cost it 0.3 us per decode step.
template <int Q, int NT, int VPT, int KMAX, bool EXACT, bool PACK>
__global__ __launch_bounds__(NT) void dispatch_cap_kernel(const u32x4 *__restrict__ x, int nvec, int k, int chunks,
                                                          const float *__restrict__ w, float *__restrict__ recv_w,
                                                          char *__restrict__ data, char *__restrict__ scales,
                                                          int64_t dq, int64_t sq, FusedArgs fa) {
  __shared__ uint32_t red[NT / kWave * (KMAX / 2)];
  int b = blockIdx.x;
  if (b < fa.lwg) {
    if (fa.idx64) fused_layout_outputs<NT, true, int64_t>(fa, b);
    else fused_layout_outputs<NT, true, int32_t>(fa, b);
    return;
  }
  b -= fa.lwg;
  const int t = b / chunks;
  const int c = b - t * chunks;
  const int64_t pair0 = (int64_t)t * k;
  const u32x4 *xr = x + (int64_t)t * nvec;
  const int v0 = c * NT * VPT + threadIdx.x;
  u32x4 raw[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int v = v0 + i * NT;
    raw[i] = v < nvec ? xr[v] : u32x4{0u, 0u, 0u, 0u};
  }
  int s[KMAX];
  if (fa.idx64) fused_slots_cap<NT, KMAX, EXACT, int64_t>(fa, t, k, s, red);
  else fused_slots_cap<NT, KMAX, EXACT, int32_t>(fa, t, k, s, red);
  if (c == 0 && threadIdx.x < k) {
    int r = -1;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) r = j == (int)threadIdx.x ? s[j] : r;
    fa.slot[pair0 + threadIdx.x] = r;
    if (r >= 0) {
      fa.row_src[r] = (int)pair0 + threadIdx.x;
      if (recv_w != nullptr) recv_w[r] = w[pair0 + threadIdx.x];
    }
  }
  bool any = false;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    s[j] = j < k ? s[j] : -1;
    any |= s[j] >= 0;
  }
  if (!any) return;   // uniform: every pair of the token dropped or routed nowhere
  quantize_store<Q, NT, VPT, KMAX, PACK>(raw, v0, nvec, s, 0, KMAX, data, scales, dq, sq, red);
}

// fa != null: the fused launch (layout workgroups first), forward dispatch only.
template <int Q, int NT, int VPT, bool PACK, bool WEIGHTED>
hipError_t launch_q(const ep_handle_t &h, const void *x, int nvec, const float *w, char *recv, float *recv_w,
                    int64_t dq, int64_t sq, size_t scale_off, const FusedArgs *fa, hipStream_t s) {
  const int chunks = (nvec + NT * VPT - 1) / (NT * VPT);
  const int64_t blocks = h.num_tokens * chunks + (fa ? fa->lwg : 0);
  if (blocks == 0) return hipSuccess;
#define EP_LAUNCH_DISPATCH(KMAX, EXACT, FUSED)                                                                 \
  hipLaunchKernelGGL((dispatch_kernel<Q, NT, VPT, KMAX, EXACT, PACK, WEIGHTED, FUSED>), dim3((unsigned)blocks), \
                     dim3(NT), EP_DISPATCH_LDS_CAP, s, (const u32x4 *)x, nvec, h.num_topk, chunks, h.slot, w,    \
                     recv_w, recv, recv + scale_off, dq, sq, fa ? *fa : FusedArgs{})
#define EP_LAUNCH_K(FUSED)                                                  \
  if (h.num_topk == 8) EP_LAUNCH_DISPATCH(8, true, FUSED);                  \
  else if (h.num_topk < 8) EP_LAUNCH_DISPATCH(8, false, FUSED);             \
  else if (h.num_topk == kMaxTopk) EP_LAUNCH_DISPATCH(kMaxTopk, true, FUSED); \
  else EP_LAUNCH_DISPATCH(kMaxTopk, false, FUSED);
#define EP_LAUNCH_CAP(KMAX, EXACT)                                                                          \
  hipLaunchKernelGGL((dispatch_cap_kernel<Q, NT, VPT, KMAX, EXACT, PACK>), dim3((unsigned)blocks), dim3(NT),  \
                     EP_DISPATCH_LDS_CAP, s, (const u32x4 *)x, nvec, h.num_topk, chunks, w, recv_w, recv,     \
                     recv + scale_off, dq, sq, *fa)
  if constexpr (!WEIGHTED) {
    if (fa && fa->cap > 0) {
      if (h.num_topk == 8) EP_LAUNCH_CAP(8, true);
      else if (h.num_topk < 8) EP_LAUNCH_CAP(8, false);
      else if (h.num_topk == kMaxTopk) EP_LAUNCH_CAP(kMaxTopk, true);
      else EP_LAUNCH_CAP(kMaxTopk, false);
      return hipGetLastError();
    }
    if (fa) {
      EP_LAUNCH_K(true)
      return hipGetLastError();
    }
  }
  EP_LAUNCH_K(false)
#undef EP_LAUNCH_CAP
#undef EP_LAUNCH_K
#undef EP_LAUNCH_DISPATCH
  return hipGetLastError();
}

// `quant` is Q possibly OR-ed with EP_RECV_INTERLEAVED; the kernels take the
// row strides of data and scales (equal for interleaved rows) and the scale base.
template <int Q, bool WEIGHTED>
hipError_t launch_mode(const ep_handle_t &h, const void *x, int hidden, const float *w, char *recv,
                       float *recv_w, int quant, const FusedArgs *fa, hipStream_t s) {
  const RecvGeom g = recv_geom(h.max_rows, hidden, quant);
  const int64_t dq = g.data_stride, sq = g.scale_stride;
  const size_t scale_off = g.scale_off;
  const int nvec = hidden / 8;
  if constexpr (Q == EP_QUANT_INT8_TOKEN) {
    // the whole row must sit in one workgroup (its amax is a row reduction)
    if (nvec <= 256) return launch_q<Q, 256, 1, false, WEIGHTED>(h, x, nvec, w, recv, recv_w, dq, sq, scale_off, fa, s);
    if (nvec <= 512) return launch_q<Q, 256, 2, false, WEIGHTED>(h, x, nvec, w, recv, recv_w, dq, sq, scale_off, fa, s);
    if (nvec <= 1024) return launch_q<Q, 256, 4, false, WEIGHTED>(h, x, nvec, w, recv, recv_w, dq, sq, scale_off, fa, s);
    if (nvec <= 2048) return launch_q<Q, 256, 8, false, WEIGHTED>(h, x, nvec, w, recv, recv_w, dq, sq, scale_off, fa, s);
    return launch_q<Q, 1024, 8, false, WEIGHTED>(h, x, nvec, w, recv, recv_w, dq, sq, scale_off, fa, s);
  } else if constexpr (Q == EP_QUANT_MXFP8 || Q == EP_QUANT_MXFP4) {
    constexpr int NT = EP_DISPATCH_THREADS, VPT = EP_DISPATCH_VPT;
    if (hidden % 128 == 0)
      return launch_q<Q, NT, VPT, true, WEIGHTED>(h, x, nvec, w, recv, recv_w, dq, sq, scale_off, fa, s);
    return launch_q<Q, NT, VPT, false, WEIGHTED>(h, x, nvec, w, recv, recv_w, dq, sq, scale_off, fa, s);
  } else {
    return launch_q<Q, EP_DISPATCH_THREADS, EP_DISPATCH_VPT, false, WEIGHTED>(h, x, nvec, w, recv, recv_w, dq, sq,
                                                                          scale_off, fa, s);
  }
}

template <bool WEIGHTED>
hipError_t launch_any(const ep_handle_t &h, const void *x, int hidden, const float *w, int quant, char *recv,
                      float *recv_w, const FusedArgs *fa, hipStream_t s) {
#define EP_MODE(QQ) launch_mode<QQ, WEIGHTED>(h, x, hidden, w, recv, recv_w, quant, fa, s)
  switch (quant & kQuantMask) {
    case EP_QUANT_NONE: return EP_MODE(EP_QUANT_NONE);
    case EP_QUANT_INT8_TOKEN: return EP_MODE(EP_QUANT_INT8_TOKEN);
    case EP_QUANT_FP8_B128: return EP_MODE(EP_QUANT_FP8_B128);
    case EP_QUANT_MXFP8: return EP_MODE(EP_QUANT_MXFP8);
    case EP_QUANT_FP8_B128_POW2: return EP_MODE(EP_QUANT_FP8_B128_POW2);
    case EP_QUANT_FP8_B128_UE8M0: return EP_MODE(EP_QUANT_FP8_B128_UE8M0);
    default: return EP_MODE(EP_QUANT_MXFP4);
  }
#undef EP_MODE
}

}  // namespace

hipError_t launch_dispatch(const ep_handle_t &h, const void *x, int hidden, const float *w, int quant,
                           char *recv, float *recv_w, hipStream_t s) {
  return launch_any<false>(h, x, hidden, w, quant, recv, recv_w, nullptr, s);
}

hipError_t launch_layout_dispatch(const ep_handle_t &h, const void *idx, int idx64, int64_t *recv_count,
                                  int32_t *cum, const void *x, int hidden, const float *w, int quant, char *recv,
                                  float *recv_w, hipStream_t s) {
  FusedArgs fa;
  fa.idx = idx;
  fa.idx64 = idx64;
  fa.n = (int)(h.num_tokens * h.num_topk);
  fa.E = h.num_experts;
  fa.max_rows = (int)h.max_rows;
  fa.cap = h.expert_capacity;
  fa.lwg = h.expert_capacity > 0
               ? (int)std::min<int64_t>(std::max<int64_t>((h.max_rows + kFusedRowsPerLayoutWg - 1) /
                                                               kFusedRowsPerLayoutWg, 1),
                                        h.num_experts)
               : 1;
  fa.recv_count = recv_count;
  fa.cum = cum;
  fa.offsets = h.offsets;
  fa.slot = h.slot;
  fa.row_src = h.row_src;
  fa.status = h.status;
  return launch_any<false>(h, x, hidden, w, quant, recv, recv_w, &fa, s);
}

hipError_t launch_combine_backward(const ep_handle_t &h, const void *grad, int hidden, const float *w, int quant,
                                   char *buf, hipStream_t s) {
  if (w == nullptr) return launch_any<false>(h, grad, hidden, nullptr, quant, buf, nullptr, nullptr, s);
  return launch_any<true>(h, grad, hidden, w, quant, buf, nullptr, nullptr, s);
}

}  // namespace ep
