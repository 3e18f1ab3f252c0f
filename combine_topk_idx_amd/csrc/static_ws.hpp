// The library's static device workspace (static_ws.hip), used by the layout
// + dispatch call that allocates nothing.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ep {

// Bytes of the static workspace.
size_t static_workspace_bytes();

// Its device address on the current device (resolved on the first call per
// device, kept per device).
hipError_t static_workspace(void **addr);

}  // namespace ep
