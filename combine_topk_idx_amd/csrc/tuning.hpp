// Launch shapes and memory hints of the dispatch and combine kernels.
// Defaults are the measured best on MI355X for hidden 7168; each can be
// overridden at build time with -D for tuning sweeps.
#pragma once

#ifndef EP_DISPATCH_THREADS
#define EP_DISPATCH_THREADS 128   // threads per workgroup (one token, a span of its row)
#endif
#ifndef EP_DISPATCH_VPT
#define EP_DISPATCH_VPT 1         // 16-byte input vectors per thread
#endif
#ifndef EP_DISPATCH_NT_STORE
#define EP_DISPATCH_NT_STORE 0    // non-temporal stores of receive rows
#endif
#ifndef EP_COMBINE_THREADS
#define EP_COMBINE_THREADS 128
#endif
#ifndef EP_COMBINE_VPT
#define EP_COMBINE_VPT 1          // 8-element output vectors per thread
#endif
#ifndef EP_COMBINE_NT_LOAD
#define EP_COMBINE_NT_LOAD 1      // non-temporal loads of expert rows
#endif
#ifndef EP_COMBINE_NT_STORE
#define EP_COMBINE_NT_STORE 1     // non-temporal stores of the output
#endif
