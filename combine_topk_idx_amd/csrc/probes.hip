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
//   ep_probe_stream     grid-stride 16-byte accesses over n bytes: read only
//                       (one 16-byte value per workgroup written), write only,
//                       or copy
//   ep_probe_mfma       one v_mfma_scale_f32_32x32x64_f8f6f4 step (e4m3 x
//                       e4m3) per case: the raw float32 result of a given
//                       64-product block, to check a model of its precision
//
// All pointers are device pointers; every call is asynchronous on `stream`.
// Sizes are checked on the host (a call with a bad size launches nothing and
// returns -1).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

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

}  // namespace

extern "C" {

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

}  // extern "C"
