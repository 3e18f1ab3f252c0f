// Launcher of the one-launch layout + dispatch (defined in dispatch.hip).
#pragma once

#include "common.hpp"

namespace ep {

// Layout (compact rows) and dispatch in one launch; the handle is the one the
// layout would produce.  Only for handles with row_align 1, no capacity and
// at most kFusedMaxPairs pairs: every span workgroup scans all the ids.
constexpr int64_t kFusedMaxPairs = 2048;
hipError_t launch_layout_dispatch(const ep_handle_t &h, const void *idx, int idx64, int64_t *recv_count,
                                  int32_t *cum, const void *x, int hidden, const float *w, int quant, char *recv,
                                  float *recv_w, hipStream_t s);

}  // namespace ep
