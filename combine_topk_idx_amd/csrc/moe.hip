// Grouped MXFP8 matrix multiplies of the expert MLP for gfx950: GMM1 with a
// SwiGLU (+ MXFP8 requant) epilogue and GMM2 with a bf16 epilogue.
//
// What is computed ("[feat] A5 deep fused moe": dispatch, GMM1, SwiGLU,
// requant, GMM2, combine; the GMM1 A operand is e4m3 with one e8m0 scale per
// 32 elements): for expert e and each of its receive rows r,
//   GMM1  g_n = sum_h W1[e][n][h] x[r][h], u_n = sum_h W1[e][I+n][h] x[r][h]
//         a_n = silu(g_n) * u_n                  (float32, silu = g / (1 + e^-g))
//         out = MXFP8(a) per 32 along I (the MX rule of dispatch) or bf16(a)
//   GMM2  y_m = sum_i W2[e][m][i] a[r][i],  out = bf16(y)
// with every operand MXFP8 (e4m3 codes, e8m0 scale per 32 along the
// reduction axis) and the products summed by the MX-scaled matrix cores.
//
// Matrix-core operand layout (v_mfma_scale_f32_32x32x64_f8f6f4, checked on
// the device): lane (r = l % 32, g = l / 32) holds, for row/column r, the 16
// K-bytes [16g, 16g + 16) and [32 + 16g, 48 + 16g) of the 64-wide K step; the
// e8m0 byte in lane (r, g)'s scale register scales K-block g (K [32g, 32g +
// 32)) of row/column r.  The 16 accumulators of lane l are column l % 32,
// rows 8b + 4(l / 32) + i (b, i in 0..3).  The instruction sums each block of
// products with less than float32 precision (about 3e-4 of sum |a b| per
// instruction, measured), which bounds how closely any result here can
// follow an exact dot product.
//
// Mapping: a workgroup (4 waves) owns one (expert, chunk of up to 256 rows,
// N tile).  The chunk's A rows are staged through double-buffered LDS one
// 64-wide K step at a time and shared by the 4 waves; every wave streams its
// own 32 weight rows (B) straight into registers, kPrefetch K steps ahead
// (weights are read once from HBM: they are the traffic that bounds the
// kernel at the shapes of the benchmark).  GMM1 gives each wave 16 gate and
// the matching 16 up rows, so lane c < 16 and lane c + 16 hold g and u of the
// same output; GMM2 gives each wave 32 output columns.
#include <math.h>

#include "common.hpp"
#include "formats.hpp"

namespace ep {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxFrags = 8;                      // 32-row fragments per chunk
constexpr int kChunkRows = kMaxFrags * 32;        // rows per work item
constexpr int kKStep = 64;                        // K per matrix-core step
constexpr int kRowStride = 80;                    // LDS bytes per staged A row (64 + pad)
constexpr int kStage = kChunkRows * kRowStride;   // bytes of one staged A step
constexpr int kScaleStage = kChunkRows * 2;       // scale bytes of one staged A step
constexpr int kPrefetch = 4;                      // weight K steps in flight per wave
constexpr int kEpiCols = 64;                      // GMM1 SwiGLU columns per workgroup
constexpr int kEpiStride = kEpiCols + 1;          // floats per LDS row of the epilogue tile

enum Mode { kGmm1Mx = 0, kGmm1Bf16 = 1, kGmm2 = 2 };

struct Item {
  int expert, row0, rows;                         // rows <= kChunkRows
};

// The work item of work index `item` (an (expert, 256-row chunk) pair in
// expert order), or expert -1 past the last one.  Row counts are recv_count
// when given, else the expert block sizes.  Every thread takes two experts;
// their chunk counts are scanned across the workgroup (wave scans, then the
// four wave totals through LDS).
__device__ Item find_item(int item, int E, const int *__restrict__ offsets, const int64_t *__restrict__ recv_count) {
  __shared__ int wsum[kWaves];
  __shared__ Item found;
  if (threadIdx.x == 0) found.expert = -1;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  int cnt[2], ch[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * threadIdx.x + q;
    cnt[q] = 0;
    if (e < E) cnt[q] = recv_count ? (int)recv_count[e] : offsets[e + 1] - offsets[e];
    ch[q] = (cnt[q] + kChunkRows - 1) / kChunkRows;
  }
  int x = ch[0] + ch[1];
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) wsum[wv] = x;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) before += i < wv ? wsum[i] : 0;
  int start = before + x - ch[0] - ch[1];                          // exclusive prefix of expert 2t
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * threadIdx.x + q;
    if (e < E && item >= start && item < start + ch[q]) {
      const int c = item - start;
      found.expert = e;
      found.row0 = offsets[e] + c * kChunkRows;
      found.rows = min(kChunkRows, cnt[q] - c * kChunkRows);
    }
    start += ch[q];
  }
  __syncthreads();
  return found;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

template <int MODE>
__global__ __launch_bounds__(kThreads) void mx_gmm_kernel(
    const uint8_t *__restrict__ a_data, const uint8_t *__restrict__ a_scales, int K,
    const uint8_t *__restrict__ w, const uint8_t *__restrict__ w_scales, int N_w, int n_tiles, int inter,
    const int *__restrict__ offsets, const int64_t *__restrict__ recv_count, int E,
    uint8_t *__restrict__ out_data, uint8_t *__restrict__ out_scales, int out_cols) {
  constexpr int kStaging = 2 * (kStage + kScaleStage);
  constexpr int kTile = MODE == kGmm2 ? 0 : kChunkRows * kEpiStride * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStaging > kTile ? kStaging : kTile];
  const Item it = find_item(blockIdx.x / n_tiles, E, offsets, recv_count);
  if (it.expert < 0 || it.rows <= 0) return;                     // uniform
  const int ntile = blockIdx.x % n_tiles;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int r = lane & 31, g = lane >> 5;
  const int nfrag = (it.rows + 31) / 32;
  const int ksteps = K / kKStep;
  const int kb = K / 32;                                          // scale bytes per row

  // this lane's weight row
  int wrow;
  if constexpr (MODE == kGmm2) {
    wrow = ntile * (kWaves * 32) + wv * 32 + r;
  } else {
    const int n0 = ntile * kEpiCols + wv * 16;
    wrow = r < 16 ? n0 + r : inter + n0 + (r - 16);
  }
  const uint8_t *wp = w + ((size_t)it.expert * N_w + wrow) * (size_t)K;
  const uint8_t *wsp = w_scales + ((size_t)it.expert * N_w + wrow) * (size_t)kb;

  // staging of A step s into LDS buffer s & 1: each thread moves 16-byte
  // pieces of the chunk's rows (4 per row per step) and one scale pair per row
  auto a_piece_count = nfrag * 32 * 4;
  auto load_a = [&](int s, u32x4 (&pieces)[4], uint32_t &sc) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = threadIdx.x + p * kThreads;
      pieces[p] = u32x4{0u, 0u, 0u, 0u};
      if (idx < a_piece_count) {
        const int row = idx >> 2, q = idx & 3;
        const int src = it.row0 + min(row, it.rows - 1);
        pieces[p] = *(const u32x4 *)(a_data + (size_t)src * K + (size_t)s * kKStep + q * 16);
      }
    }
    sc = 0;
    if (threadIdx.x < nfrag * 32) {
      const int src = it.row0 + min((int)threadIdx.x, it.rows - 1);
      const uint8_t *sp = a_scales + (size_t)src * kb + (size_t)s * 2;
      sc = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
    }
  };
  auto store_a = [&](int buf, const u32x4 (&pieces)[4], uint32_t sc) {
    uint8_t *base = smem + buf * (kStage + kScaleStage);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int idx = threadIdx.x + p * kThreads;
      if (idx < a_piece_count) {
        const int row = idx >> 2, q = idx & 3;
        *(u32x4 *)(base + row * kRowStride + q * 16) = pieces[p];
      }
    }
    if (threadIdx.x < nfrag * 32) *(uint16_t *)(base + kStage + threadIdx.x * 2) = (uint16_t)sc;
  };

  // weight ring: kPrefetch steps of (two 16-byte pieces, one scale byte)
  u32x4 wb0[kPrefetch], wb1[kPrefetch];
  uint32_t wsc[kPrefetch];
  auto load_w = [&](int s, int slot) {
    const int ss = min(s, ksteps - 1);                            // clamped: loads past the end are dropped
    wb0[slot] = *(const u32x4 *)(wp + (size_t)ss * kKStep + g * 16);
    wb1[slot] = *(const u32x4 *)(wp + (size_t)ss * kKStep + 32 + g * 16);
    wsc[slot] = wsp[ss * 2 + g];
  };

  v16f acc[kMaxFrags];
#pragma unroll
  for (int f = 0; f < kMaxFrags; ++f) acc[f] = v16f{};

  u32x4 ap[4];
  uint32_t asc;
  load_a(0, ap, asc);
  store_a(0, ap, asc);
  if (ksteps > 1) load_a(1, ap, asc);
#pragma unroll
  for (int p = 0; p < kPrefetch; ++p) load_w(p, p);
  __syncthreads();

  for (int s0 = 0; s0 < ksteps; s0 += kPrefetch) {
#pragma unroll
    for (int u = 0; u < kPrefetch; ++u) {
      const int s = s0 + u;
      if (s >= ksteps) break;                                     // uniform
      if (s + 1 < ksteps) store_a((s + 1) & 1, ap, asc);
      if (s + 2 < ksteps) load_a(s + 2, ap, asc);
      const u32x4 b0 = wb0[u], b1 = wb1[u];
      const int bsc = (int)wsc[u];
      load_w(s + kPrefetch, u);
      const v8i bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      const uint8_t *base = smem + (s & 1) * (kStage + kScaleStage);
#pragma unroll
      for (int f = 0; f < kMaxFrags; ++f) {
        if (f >= nfrag) break;                                    // uniform
        const int row = f * 32 + r;
        const u32x4 x0 = *(const u32x4 *)(base + row * kRowStride + g * 16);
        const u32x4 x1 = *(const u32x4 *)(base + row * kRowStride + 32 + g * 16);
        const int xs = (int)base[kStage + row * 2 + g];
        const v8i av = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        acc[f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[f], 0, 0, 0, xs, 0, bsc);
      }
      __syncthreads();
    }
  }

  // ---------------------------------------------------------------- epilogue
  if constexpr (MODE == kGmm2) {
    // bf16 rows: column l % 32 of this wave's 32, rows 8b + 4g + i of each fragment
    const int col = ntile * (kWaves * 32) + wv * 32 + r;
#pragma unroll
    for (int f = 0; f < kMaxFrags; ++f) {
      if (f >= nfrag) break;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = f * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
        if (row < it.rows) {
          const uint32_t bits = pack_bf16x2(acc[f][i], 0.0f) & 0xffffu;
          *(uint16_t *)(out_data + ((size_t)(it.row0 + row) * out_cols + col) * 2) = (uint16_t)bits;
        }
      }
    }
  } else {
    // SwiGLU: lane r < 16 holds gate column r, lane r + 16 the matching up
    // column; the 16 results of each wave go to an LDS tile [rows][64]
    float *tile = (float *)smem;
#pragma unroll
    for (int f = 0; f < kMaxFrags; ++f) {
      if (f >= nfrag) break;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float gate = acc[f][i];
        const float up = __shfl_xor(gate, 16);
        const int row = f * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
        if (r < 16) tile[row * kEpiStride + wv * 16 + r] = silu(gate) * up;
      }
    }
    __syncthreads();
    // each thread: one (row, 32-column block) of the tile
    const int n0 = ntile * kEpiCols;
    for (int job = threadIdx.x; job < it.rows * 2; job += kThreads) {
      const int row = job >> 1, blk = job & 1;
      const float *src = tile + row * kEpiStride + blk * 32;
      const size_t orow = (size_t)(it.row0 + row);
      if constexpr (MODE == kGmm1Bf16) {
        uint32_t o[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) o[e] = pack_bf16x2(src[2 * e], src[2 * e + 1]);
        u32x4 *dst = (u32x4 *)(out_data + (orow * out_cols + n0 + blk * 32) * 2);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = u32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
      } else {
        // MX rule: shared exponent clamp(floor(log2 amax) - 8, -127, 127);
        // codes e4m3(clamp(x * 2^-exp, +-448))
        uint32_t amax = 0;
#pragma unroll
        for (int e = 0; e < 32; ++e) amax = max(amax, __float_as_uint(src[e]) & 0x7fffffffu);
        int se = -127;
        if (amax != 0) {
          se = floor_log2_bits(amax) - 8;
          se = se < -127 ? -127 : (se > 127 ? 127 : se);
        }
        const float mult = __uint_as_float((uint32_t)(127 - se) << 23);
        u32x2 q[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = fminf(fmaxf(src[8 * c + e] * mult, -448.0f), 448.0f);
          q[c] = e4m3x8_encode(v);
        }
        u32x4 *dst = (u32x4 *)(out_data + orow * out_cols + n0 + blk * 32);
        dst[0] = u32x4{q[0].x, q[0].y, q[1].x, q[1].y};
        dst[1] = u32x4{q[2].x, q[2].y, q[3].x, q[3].y};
        out_scales[orow * (out_cols / 32) + (n0 >> 5) + blk] = (uint8_t)(se + 127);
      }
    }
  }
}

}  // namespace

hipError_t launch_moe_gmm1(const ep_handle_t &h, const int64_t *recv_count, const char *x_buf, int hidden, int inter,
                           const void *w1, const void *w1_scales, int out_quant, char *out_buf, hipStream_t s) {
  const RecvGeom gx = recv_geom(h.max_rows, hidden, EP_QUANT_MXFP8);
  const int n_tiles = inter / kEpiCols;
  const int64_t items = (h.max_rows + kChunkRows - 1) / kChunkRows + h.num_experts;
  const int64_t blocks = items * n_tiles;
  if (h.num_tokens == 0 || blocks == 0) return hipSuccess;
  if (out_quant == EP_QUANT_MXFP8) {
    const RecvGeom go = recv_geom(h.max_rows, inter, EP_QUANT_MXFP8);
    hipLaunchKernelGGL(mx_gmm_kernel<kGmm1Mx>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       (const uint8_t *)x_buf, (const uint8_t *)x_buf + gx.scale_off, hidden, (const uint8_t *)w1,
                       (const uint8_t *)w1_scales, 2 * inter, n_tiles, inter, h.offsets, recv_count, h.num_experts,
                       (uint8_t *)out_buf, (uint8_t *)out_buf + go.scale_off, inter);
  } else {
    hipLaunchKernelGGL(mx_gmm_kernel<kGmm1Bf16>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       (const uint8_t *)x_buf, (const uint8_t *)x_buf + gx.scale_off, hidden, (const uint8_t *)w1,
                       (const uint8_t *)w1_scales, 2 * inter, n_tiles, inter, h.offsets, recv_count, h.num_experts,
                       (uint8_t *)out_buf, (uint8_t *)nullptr, inter);
  }
  return hipGetLastError();
}

hipError_t launch_moe_gmm2(const ep_handle_t &h, const int64_t *recv_count, const char *a_buf, int inter, int hidden,
                           const void *w2, const void *w2_scales, char *out_buf, hipStream_t s) {
  const RecvGeom ga = recv_geom(h.max_rows, inter, EP_QUANT_MXFP8);
  const int n_tiles = hidden / (kWaves * 32);
  const int64_t items = (h.max_rows + kChunkRows - 1) / kChunkRows + h.num_experts;
  const int64_t blocks = items * n_tiles;
  if (h.num_tokens == 0 || blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_gmm_kernel<kGmm2>, dim3((unsigned)blocks), dim3(kThreads), 0, s, (const uint8_t *)a_buf,
                     (const uint8_t *)a_buf + ga.scale_off, inter, (const uint8_t *)w2, (const uint8_t *)w2_scales,
                     hidden, n_tiles, inter, h.offsets, recv_count, h.num_experts, (uint8_t *)out_buf,
                     (uint8_t *)nullptr, hidden);
  return hipGetLastError();
}

}  // namespace ep
