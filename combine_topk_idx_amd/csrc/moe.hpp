// Launchers and size helpers of the expert GEMMs (moe.hip), kept apart
// from common.hpp so that the dispatch/combine kernels do not depend on them.
#pragma once

#include "common.hpp"

namespace ep {

// Packed MXFP8 weights for the expert GEMMs: bytes of the codes and of the
// scales of E experts with N rows of K codes (K % 64 == 0, N % 32 == 0).
__host__ inline void moe_packed_bytes(int64_t E, int64_t N, int64_t K, size_t *codes, size_t *scales) {
  const int64_t ksteps = K / 64, spans = (ksteps + 3) / 4;
  *codes = (size_t)(E * N * K);
  *scales = (size_t)(E * (N / 32) * spans * 256);
}

hipError_t launch_moe_pack(const void *codes, const void *scales, int E, int N, int K, int gate_up, void *pcodes,
                           void *pscales, hipStream_t s);

hipError_t launch_moe_gmm1(const ep_handle_t &h, const int64_t *recv_count, const char *x_buf, int hidden, int inter,
                           const void *w1, const void *w1_scales, int out_quant, char *out_buf, hipStream_t s);

hipError_t launch_moe_gmm2(const ep_handle_t &h, const int64_t *recv_count, const char *a_buf, int inter, int hidden,
                           const void *w2, const void *w2_scales, char *out_buf, hipStream_t s);

}  // namespace ep
