// Launcher of the one-launch layout + dispatch (defined in dispatch.hip).
#pragma once

#include "common.hpp"

namespace ep {

// Layout and dispatch in one launch; the handle is the one the layout would
// produce.  Only for compact rows or capacity blocks (row_align 1), at most
// kFusedMaxPairs pairs (every span workgroup scans all the ids) and, with a
// capacity, at most kFusedMaxCapRows receive rows (the layout workgroups mark
// the free rows of every block, kFusedRowsPerLayoutWg each).
constexpr int64_t kFusedMaxPairs = 2048;
constexpr int64_t kFusedMaxCapRows = 1 << 18;
constexpr int64_t kFusedRowsPerLayoutWg = 1024;
inline bool fused_layout_dispatch_fits(int64_t pairs, int32_t row_align, int32_t cap, int64_t max_rows) {
  return row_align == 1 && pairs <= kFusedMaxPairs && (cap == 0 || max_rows <= kFusedMaxCapRows);
}
hipError_t launch_layout_dispatch(const ep_handle_t &h, const void *idx, int idx64, int64_t *recv_count,
                                  int32_t *cum, const void *x, int hidden, const float *w, int quant, char *recv,
                                  float *recv_w, hipStream_t s);

}  // namespace ep
