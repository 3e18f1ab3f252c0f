// Measurement probes (libep_probe.so, not part of the dispatch/combine
// library): the smallest kernels of the access patterns the path is built
// from, timed by `bench.py --probes` to give the floors and ceilings its
// kernels are compared against.
//
//   ep_probe_empty      a grid of workgroups that do nothing: the cost of a
//                       launch of that shape
//   ep_probe_gather     per workgroup (token t, span c): read the k row
//                       numbers of token t, then k row spans of 2 KB (16
//                       bytes per lane), add them in float32, write 2 KB --
//                       combine's dependent loads with no dequantisation
//   ep_probe_scatter    per workgroup (token t, span c): read the k row
//                       numbers of token t and the token's 2 KB span (16
//                       bytes per lane), write one byte per element (8
//                       bytes per lane) to each of the k rows -- dispatch's
//                       access pattern for one-byte codes, with no
//                       quantisation and no scale bytes
//   ep_probe_stream     grid-stride 16-byte accesses over n bytes: read only
//                       (one 16-byte value per workgroup written), write only,
//                       or copy
//   ep_probe_wave_stream  each wave reads its own contiguous range in 2 KB
//                       steps (two 1 KB loads per step) with a fixed number
//                       of steps in flight -- the expert GEMMs' weight
//                       stream, without the matrix-core work
//   ep_probe_mixed_stream  the weight stream plus, per step, two 16-byte
//                       pieces per thread of an activation buffer shared by
//                       all workgroups -- the GEMMs' whole fetch per CU
//   ep_probe_mfma_rate  back-to-back independent matrix-core instructions
//                       (MX-scaled e4m3 32x32x64, or bf16 32x32x16) on
//                       every wave of a grid: the sustained rate per SIMD
//   ep_probe_mfma       one v_mfma_scale_f32_32x32x64_f8f6f4 step (e4m3 x
//                       e4m3) per case: the raw float32 result of a given
//                       64-product block, to check a model of its precision
//   ep_probe_codec      the element converters of formats.hpp (and the
//                       scaled bf16 -> e4m3 conversion of the weighted reverse
//                       dispatch) over arrays of inputs, to check them against
//                       software codecs over their whole input domains
//
// All pointers are device pointers; every call is asynchronous on `stream`.
// Sizes are checked on the host (a call with a bad size launches nothing and
// returns -1).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "formats.hpp"

namespace {

using ep::u32x2;

using ep::u32x4;

__global__ void empty_kernel() {}

// rows: [max_rows, nvec] 16-byte vectors (bf16 x 8); slot: [T, k] int32
template <int K>
__global__ __launch_bounds__(128) void gather_kernel(const u32x4 *__restrict__ rows, const int *__restrict__ slot,
                                                     int nvec, int chunks, u32x4 *__restrict__ out) {
  const int t = blockIdx.x / chunks, c = blockIdx.x - t * chunks;
  int s[K];
#pragma unroll
  for (int j = 0; j < K; ++j) s[j] = slot[t * K + j];
  const int v = c * 128 + threadIdx.x;
  if (v >= nvec) return;
  u32x4 r[K];
#pragma unroll
  for (int j = 0; j < K; ++j) r[j] = __builtin_nontemporal_load(rows + (int64_t)max(s[j], 0) * nvec + v);
  float acc[8] = {};
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (s[j] < 0) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(r[j][e] << 16);
      acc[2 * e + 1] += __uint_as_float(r[j][e] & 0xffff0000u);
    }
  }
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = (__float_as_uint(acc[2 * e]) >> 16) | (__float_as_uint(acc[2 * e + 1]) & 0xffff0000u);
  __builtin_nontemporal_store(o, out + (int64_t)t * nvec + v);
}

// x: [T, nvec] 16-byte vectors (bf16 x 8); slot: [T, K] int32; rows:
// [max_rows, nvec] 8-byte pieces.  Lane v of workgroup (t, c) writes the
// high bytes of its eight bf16 values to every routed row of token t.
template <int K>
__global__ __launch_bounds__(128) void scatter_kernel(const u32x4 *__restrict__ x, const int *__restrict__ slot,
                                                     int nvec, int chunks, u32x2 *__restrict__ rows) {
  const int t = blockIdx.x / chunks, c = blockIdx.x - t * chunks;
  const int v = c * 128 + threadIdx.x;
  int s[K];
#pragma unroll
  for (int j = 0; j < K; ++j) s[j] = slot[t * K + j];
  if (v >= nvec) return;
  const u32x4 r = __builtin_nontemporal_load(x + (int64_t)t * nvec + v);
  const u32x2 o = {(r.x >> 8 & 0xffu) | (r.x >> 16 & 0xff00u) | (r.y << 8 & 0xff0000u) | (r.y & 0xff000000u),
                   (r.z >> 8 & 0xffu) | (r.z >> 16 & 0xff00u) | (r.w << 8 & 0xff0000u) | (r.w & 0xff000000u)};
#pragma unroll
  for (int j = 0; j < K; ++j)
    if (s[j] >= 0) __builtin_nontemporal_store(o, rows + (int64_t)s[j] * nvec + v);
}

// mode 0: read `src` (each workgroup writes one vector to dst[blockIdx]);
// mode 1: write dst; mode 2: copy src -> dst.  n16 = 16-byte vectors.
template <int MODE>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                     int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 x = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    if constexpr (MODE == 1) {
      const u32x4 w = {(uint32_t)i, 1u, 2u, 3u};
#pragma unroll
      for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(w, dst + i + u * stride);
    } else {
      u32x4 r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) r[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (MODE == 2) __builtin_nontemporal_store(r[u], dst + i + u * stride);
        else x ^= r[u];
      }
    }
  }
  for (; i < n16; i += stride) {
    if constexpr (MODE == 1) {
      __builtin_nontemporal_store(u32x4{(uint32_t)i, 1u, 2u, 3u}, dst + i);
    } else {
      const u32x4 r = __builtin_nontemporal_load(src + i);
      if constexpr (MODE == 2) __builtin_nontemporal_store(r, dst + i);
      else x ^= r;
    }
  }
  if constexpr (MODE == 0) {
    // one vector per workgroup, so the loads cannot be dropped
    for (int d = 1; d < 64; d <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] ^= (uint32_t)__shfl_xor((int)x[e], d);
    if (threadIdx.x == 0) dst[blockIdx.x] = x;
  }
}

// Each wave w of the grid reads steps x 2 KB from src + w * steps * 2 KB:
// lane l loads bytes [16l, 16l + 16) and [1024 + 16l, ...) of every step,
// DEPTH steps ahead; lane 0 of each wave writes the XOR of what it read to
// out[w].  ONE_PER_CU reserves 96 KB of LDS, so that no two workgroups share
// a CU (160 KB of LDS per CU).  steps is a multiple of DEPTH.
// APIECES > 0 adds the activation side of the GEMMs' fetch: with every
// weight step each thread also loads APIECES 16-byte pieces of a shared
// buffer `a` (a_vecs vectors, a power of two) that every workgroup walks in
// the same order, so that after the first workgroup of an XCD they come from
// its L2.
template <int DEPTH, bool ONE_PER_CU, int APIECES = 0>
__global__ __launch_bounds__(1024) void wave_stream_kernel(const u32x4 *__restrict__ src, int steps,
                                                           u32x4 *__restrict__ out, const u32x4 *__restrict__ a = nullptr,
                                                           int a_vecs = 1) {
  __shared__ u32x4 pad[ONE_PER_CU ? 6144 : 1];
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const u32x4 *p = src + w * (int64_t)steps * 128 + lane;
  u32x4 r0[DEPTH], r1[DEPTH], ra[DEPTH][APIECES > 0 ? APIECES : 1];
  auto load_a = [&](int step, int d) {
#pragma unroll
    for (int q = 0; q < APIECES; ++q)
      ra[d][q] = a[((step * APIECES + q) * (int)blockDim.x + (int)threadIdx.x) & (a_vecs - 1)];
  };
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    r0[d] = __builtin_nontemporal_load(p + d * 128);
    r1[d] = __builtin_nontemporal_load(p + d * 128 + 64);
    load_a(d, d);
  }
  u32x4 x = {0u, 0u, 0u, 0u};
  for (int s = DEPTH; s < steps; s += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      x ^= r0[d] ^ r1[d];
#pragma unroll
      for (int q = 0; q < APIECES; ++q) x ^= ra[d][q];
      r0[d] = __builtin_nontemporal_load(p + (int64_t)(s + d) * 128);
      r1[d] = __builtin_nontemporal_load(p + (int64_t)(s + d) * 128 + 64);
      load_a(s + d, d);
    }
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    x ^= r0[d] ^ r1[d];
#pragma unroll
    for (int q = 0; q < APIECES; ++q) x ^= ra[d][q];
  }
  if (steps < 0) {                              // never taken: keeps the LDS reservation
    pad[threadIdx.x % (ONE_PER_CU ? 6144 : 1)] = x;
    __syncthreads();
    x = pad[(threadIdx.x + 1) % (ONE_PER_CU ? 6144 : 1)];
  }
  if (lane == 0) out[w] = x;
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Every wave issues iters x 8 matrix-core instructions on CHAINS independent
// accumulators (8 or 4; with 4 each accumulator takes two instructions per
// iteration, four instructions apart) -- KIND 0: MX-scaled e4m3 32x32x64,
// scale bytes 127; KIND 1: bf16 32x32x16 -- and writes one float per lane.
// ONE_PER_CU reserves 96 KB of LDS so that no two workgroups share a CU.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
template <int KIND, int CHAINS, bool ONE_PER_CU>
__global__ __launch_bounds__(512) void mfma_rate_kernel(int iters, float *__restrict__ out) {
  __shared__ float pad[ONE_PER_CU ? 24576 : 1];
  const int l = threadIdx.x & 63;
  v16f c[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {                  // distinct, so that no two chains can be merged
    c[u] = v16f{};
    c[u][0] = (float)(u + 8 * l);
  }
  if constexpr (KIND == 0) {
    const int x = 0x38383838 ^ (l & 7) ^ (iters << 8);
    const v8i a = {x, x + 1, x + 2, x + 3, x + 4, x + 5, x + 6, x + 7};
    const v8i b = {x ^ 1, x ^ 2, x ^ 3, x ^ 4, x ^ 5, x ^ 6, x ^ 7, x};
    v8i au[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) au[u] = a ^ u;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        c[u % CHAINS] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(au[u], b, c[u % CHAINS], 0, 0, 0, 127, 0, 127);
    }
  } else {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(float)(l + e + iters);
      b[e] = (__bf16)(float)(l - e);
    }
    bf16x8 au[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      au[u] = a;
      au[u][0] = (__bf16)(float)(u + l);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u % CHAINS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(au[u], b, c[u % CHAINS], 0, 0, 0);
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += c[u][e];
  if (iters < 0) {                               // never taken: keeps the LDS reservation
    pad[threadIdx.x] = sum;
    __syncthreads();
    sum = pad[(threadIdx.x + 1) % (ONE_PER_CU ? 24576 : 1)];
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

// One case: row 0 of A holds a[0..63] and column 0 of B holds b[0..63]
// (e4m3 codes), the K-blocks [0, 32) and [32, 64) scaled by the e8m0 bytes
// sa[0] / sb[0] and sa[1] / sb[1]; the accumulator starts at c0 in row 0,
// column 0 and at 0 elsewhere.  Operand layout of the instruction: lane
// (r = l % 32, g = l / 32) holds K bytes [16g, 16g + 16) and [32 + 16g,
// 48 + 16g) of row / column r, and its scale register's byte scales K-block
// g of row / column r; accumulator 0 of lane 0 is row 0, column 0.
struct MfmaCase {
  uint8_t a[64], b[64];
  uint8_t sa[2], sb[2];
  float c0;
};

__global__ __launch_bounds__(64) void mfma_kernel(const MfmaCase *__restrict__ cs, float *__restrict__ out) {
  const MfmaCase &c = cs[blockIdx.x];
  const int l = threadIdx.x, r = l & 31, g = l >> 5;
  v8i av, bv;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t wa = 0, wb = 0;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int byte = 4 * q + y;                                   // 0..15: K 16g.., 16..31: K 32+16g..
      const int kk = (byte < 16 ? 16 * g : 32 + 16 * g) + (byte & 15);
      wa |= (uint32_t)(r == 0 ? c.a[kk] : 0) << (8 * y);
      wb |= (uint32_t)(r == 0 ? c.b[kk] : 0) << (8 * y);
    }
    av[q] = (int)wa;
    bv[q] = (int)wb;
  }
  const int as = r == 0 ? c.sa[g] : 127, bs = r == 0 ? c.sb[g] : 127;
  v16f acc = {};
  acc[0] = l == 0 ? c.c0 : 0.0f;
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, as, 0, bs);
  // every lane stores (a store from lane 0 alone lets the compiler move the
  // instruction into that lane's branch, where the other lanes' operands
  // are never formed)
  out[(size_t)blockIdx.x * 64 + l] = acc[0];
}

// Converter checks; thread i handles input group i (see ep_probe_codec).
typedef short s16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x2 scaled_e4m3(const u32x4 &r, float scale) {
  const uint32_t w0 = r.x, w1 = r.y, w2 = r.z, w3 = r.w;
  s16x2 o0 = {0, 0}, o1 = {0, 0};
  o0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o0, __builtin_bit_cast(ep::bf16x2, w0), scale, false);
  o0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o0, __builtin_bit_cast(ep::bf16x2, w1), scale, true);
  o1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o1, __builtin_bit_cast(ep::bf16x2, w2), scale, false);
  o1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o1, __builtin_bit_cast(ep::bf16x2, w3), scale, true);
  return u32x2{__builtin_bit_cast(uint32_t, o0), __builtin_bit_cast(uint32_t, o1)};
}

__global__ void codec_kernel(int kind, const void *__restrict__ in, void *__restrict__ out, int64_t groups,
                             float scale_arg) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= groups) return;
  // the kernels compute their scales per lane, so the instructions read them
  // from vector registers; kind 6 passes the same value as a scalar operand
  float scale = scale_arg;
  asm volatile("" : "+v"(scale));
  switch (kind) {
    case 0: {   // e4m3 encode: 8 float32 (already within +-448) -> 8 codes
      const float *f = (const float *)in + 8 * i;
      float v[8];
      for (int e = 0; e < 8; ++e) v[e] = f[e];
      ((u32x2 *)out)[i] = ep::e4m3x8_encode(v);
      break;
    }
    case 1: {   // e4m3 decode scaled: (code | scale byte << 8) -> float32
      const uint16_t c = ((const uint16_t *)in)[i];
      float y[8];
      ep::e4m3x8_decode_scaled(u32x2{(uint32_t)(c & 0xff), 0u}, ep::e8m0_decode(c >> 8), y);
      ((float *)out)[i] = y[0];
      break;
    }
    case 2: {   // e2m1 encode: 8 bf16 divided by `scale` -> 8 nibbles
      ((uint32_t *)out)[i] = ep::e2m1x8_encode_bf16(((const u32x4 *)in)[i], scale);
      break;
    }
    case 3: {   // e2m1 decode scaled: (nibble | scale byte << 8) -> float32
      const uint16_t c = ((const uint16_t *)in)[i];
      float y[8];
      ep::e2m1x8_decode_scaled((uint32_t)(c & 0xf), ep::e8m0_decode(c >> 8), y);
      ((float *)out)[i] = y[0];
      break;
    }
    case 4: {   // bf16 pack: 2 float32 -> 2 bf16 in one word
      const float *f = (const float *)in + 2 * i;
      ((uint32_t *)out)[i] = ep::pack_bf16x2(f[0], f[1]);
      break;
    }
    case 5:     // scaled e4m3 from bf16 (the reverse dispatch's conversion): 8 bf16 / `scale` -> 8 codes
      ((u32x2 *)out)[i] = scaled_e4m3(((const u32x4 *)in)[i], scale);
      break;
    default:    // the same with the scale as a scalar operand
      ((u32x2 *)out)[i] = scaled_e4m3(((const u32x4 *)in)[i], scale_arg);
      break;
  }
}

}  // namespace

extern "C" {

// kind 0: e4m3 encode, in float32[8 groups], out bytes[8 groups]
// kind 1: e4m3 decode scaled, in uint16 (code | byte << 8)[groups], out float32[groups]
// kind 2: e2m1 encode of bf16 / scale, in bf16[8 groups], out uint32 (8 nibbles)[groups]
// kind 3: e2m1 decode scaled, in uint16 (nibble | byte << 8)[groups], out float32[groups]
// kind 4: bf16 pack, in float32[2 groups], out uint32[groups]
// kind 5: scaled e4m3 of bf16 / scale, in bf16[8 groups], out bytes[8 groups]
// kind 6: kind 5 with the scale read from a scalar register
// `scale` (kinds 2, 5 and 6) is the float32 power of two the instructions take.
int ep_probe_codec(int kind, const void *in, void *out, int64_t groups, float scale, void *stream) {
  if (kind < 0 || kind > 6 || groups <= 0 || groups > (int64_t)1 << 31) return -1;
  const int threads = 256;
  hipLaunchKernelGGL(codec_kernel, dim3((unsigned)((groups + threads - 1) / threads)), dim3(threads), 0,
                     (hipStream_t)stream, kind, in, out, groups, scale);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// cases: n records of 136 bytes (64 A codes, 64 B codes, 2 A scale bytes,
// 2 B scale bytes, float32 c0); out: n * 64 floats, out[64 i] the result of
// case i.
int ep_probe_mfma(const void *cases, int n, float *out, void *stream) {
  static_assert(sizeof(MfmaCase) == 136, "case record layout");
  if (n <= 0) return -1;
  hipLaunchKernelGGL(mfma_kernel, dim3(n), dim3(64), 0, (hipStream_t)stream, (const MfmaCase *)cases, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int ep_probe_empty(int blocks, int threads, void *stream) {
  if (blocks <= 0 || threads <= 0 || threads > 1024) return -1;
  hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(threads), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// rows: [max_rows, hidden] bf16; slot: [T, k] int32 with values in
// [-1, max_rows); out: [T, hidden] bf16; hidden % 8 == 0; k in {1, 8}.
int ep_probe_gather(const void *rows, const int *slot, int T, int k, int hidden, void *out, void *stream) {
  if (T <= 0 || hidden <= 0 || hidden % 8 != 0 || (k != 1 && k != 8)) return -1;
  const int nvec = hidden / 8, chunks = (nvec + 127) / 128;
  const dim3 grid((unsigned)(T * chunks));
  if (k == 1)
    hipLaunchKernelGGL(gather_kernel<1>, grid, dim3(128), 0, (hipStream_t)stream, (const u32x4 *)rows, slot, nvec,
                       chunks, (u32x4 *)out);
  else
    hipLaunchKernelGGL(gather_kernel<8>, grid, dim3(128), 0, (hipStream_t)stream, (const u32x4 *)rows, slot, nvec,
                       chunks, (u32x4 *)out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// x: [T, hidden] bf16; slot: [T, k] int32 with values in [-1, max_rows);
// rows: [max_rows, hidden] bytes; hidden % 8 == 0; k in {1, 8}.
int ep_probe_scatter(const void *x, const int *slot, int T, int k, int hidden, void *rows, void *stream) {
  if (T <= 0 || hidden <= 0 || hidden % 8 != 0 || (k != 1 && k != 8)) return -1;
  const int nvec = hidden / 8, chunks = (nvec + 127) / 128;
  const dim3 grid((unsigned)(T * chunks));
  if (k == 1)
    hipLaunchKernelGGL(scatter_kernel<1>, grid, dim3(128), 0, (hipStream_t)stream, (const u32x4 *)x, slot, nvec,
                       chunks, (u32x2 *)rows);
  else
    hipLaunchKernelGGL(scatter_kernel<8>, grid, dim3(128), 0, (hipStream_t)stream, (const u32x4 *)x, slot, nvec,
                       chunks, (u32x2 *)rows);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// mode 0 read (dst needs `blocks` vectors), 1 write, 2 copy; n = bytes, a
// multiple of 16; blocks workgroups of 256 threads.
int ep_probe_stream(int mode, const void *src, void *dst, int64_t n, int blocks, void *stream) {
  if (n <= 0 || n % 16 != 0 || blocks <= 0 || mode < 0 || mode > 2) return -1;
  const int64_t n16 = n / 16;
  const dim3 grid((unsigned)blocks), block(256);
  if (mode == 0)
    hipLaunchKernelGGL(stream_kernel<0>, grid, block, 0, (hipStream_t)stream, (const u32x4 *)src, (u32x4 *)dst, n16);
  else if (mode == 1)
    hipLaunchKernelGGL(stream_kernel<1>, grid, block, 0, (hipStream_t)stream, (const u32x4 *)src, (u32x4 *)dst, n16);
  else
    hipLaunchKernelGGL(stream_kernel<2>, grid, block, 0, (hipStream_t)stream, (const u32x4 *)src, (u32x4 *)dst, n16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// out: blocks * waves * 64 floats; kind 0 (MX e4m3) or 1 (bf16); chains 8
// or 4; waves 1..8.
int ep_probe_mfma_rate(int kind, int chains, int blocks, int waves, int iters, int one_per_cu, float *out,
                       void *stream) {
  if (blocks <= 0 || waves <= 0 || waves > 8 || iters <= 0 || kind < 0 || kind > 1 || (chains != 4 && chains != 8))
    return -1;
  const dim3 grid((unsigned)blocks), block((unsigned)(64 * waves));
  const hipStream_t st = (hipStream_t)stream;
#define EP_RATE(K, C, O) hipLaunchKernelGGL((mfma_rate_kernel<K, C, O>), grid, block, 0, st, iters, out)
  if (one_per_cu) {
    if (kind == 0) { if (chains == 8) EP_RATE(0, 8, true); else EP_RATE(0, 4, true); }
    else { if (chains == 8) EP_RATE(1, 8, true); else EP_RATE(1, 4, true); }
  } else {
    if (kind == 0) { if (chains == 8) EP_RATE(0, 8, false); else EP_RATE(0, 4, false); }
    else { if (chains == 8) EP_RATE(1, 8, false); else EP_RATE(1, 4, false); }
  }
#undef EP_RATE
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// src: blocks * waves * steps * 2048 bytes; out: blocks * waves vectors;
// waves 1..16, depth 4 or 8, steps a positive multiple of depth.
int ep_probe_wave_stream(const void *src, int blocks, int waves, int steps, int depth, int one_per_cu, void *out,
                         void *stream) {
  if (blocks <= 0 || waves <= 0 || waves > 16 || steps <= 0 || (depth != 4 && depth != 8) || steps % depth != 0)
    return -1;
  const dim3 grid((unsigned)blocks), block((unsigned)(64 * waves));
  const u32x4 *s = (const u32x4 *)src;
  u32x4 *o = (u32x4 *)out;
  const hipStream_t st = (hipStream_t)stream;
  if (depth == 4 && one_per_cu)
    hipLaunchKernelGGL((wave_stream_kernel<4, true>), grid, block, 0, st, s, steps, o);
  else if (depth == 4)
    hipLaunchKernelGGL((wave_stream_kernel<4, false>), grid, block, 0, st, s, steps, o);
  else if (one_per_cu)
    hipLaunchKernelGGL((wave_stream_kernel<8, true>), grid, block, 0, st, s, steps, o);
  else
    hipLaunchKernelGGL((wave_stream_kernel<8, false>), grid, block, 0, st, s, steps, o);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// src as for ep_probe_wave_stream (depth 4, one workgroup per CU); a:
// a_bytes of activations, a power of two and at least 16; out: blocks *
// waves vectors.
int ep_probe_mixed_stream(const void *src, const void *a, int64_t a_bytes, int blocks, int waves, int steps,
                          void *out, void *stream) {
  if (blocks <= 0 || waves <= 0 || waves > 16 || steps <= 0 || steps % 4 != 0 || a_bytes < 16 ||
      (a_bytes & (a_bytes - 1)) != 0 || a_bytes / 16 > (int64_t)1 << 30)
    return -1;
  hipLaunchKernelGGL((wave_stream_kernel<4, true, 2>), dim3((unsigned)blocks), dim3((unsigned)(64 * waves)), 0,
                     (hipStream_t)stream, (const u32x4 *)src, steps, (u32x4 *)out, (const u32x4 *)a,
                     (int)(a_bytes / 16));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
