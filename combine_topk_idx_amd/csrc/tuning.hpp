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
#ifndef EP_DISPATCH_NT_DATA
#define EP_DISPATCH_NT_DATA 1     // non-temporal stores of the code rows (scale pieces always go through L2)
#endif
#ifndef EP_COMBINE_THREADS
#define EP_COMBINE_THREADS 128
#endif
#ifndef EP_COMBINE_CV
#define EP_COMBINE_CV 1           // consecutive 8-element output vectors per thread (1 or 2)
#endif
#ifndef EP_COMBINE_NT_LOAD
#define EP_COMBINE_NT_LOAD 1      // non-temporal loads of expert rows
#endif
#ifndef EP_COMBINE_NT_STORE
#define EP_COMBINE_NT_STORE 1     // non-temporal stores of the output
#endif
#ifndef EP_COMBINE_LDS_CAP
#define EP_COMBINE_LDS_CAP 0      // LDS bytes reserved per combine workgroup (caps resident workgroups per CU)
#endif
#ifndef EP_DISPATCH_LDS_CAP
#define EP_DISPATCH_LDS_CAP 0     // same for dispatch
#endif
#ifndef EP_COMBINE_KMAX_MIN
#define EP_COMBINE_KMAX_MIN 8     // smallest compile-time top-k bound used by combine (8 or 16)
#endif
#ifndef EP_LAYOUT_ITEMS
#define EP_LAYOUT_ITEMS 2         // pairs per thread of a multi-block layout chunk (chunk = 1024 * this)
#endif
#ifndef EP_LAYOUT_COLSCAN_MIN
#define EP_LAYOUT_COLSCAN_MIN 128 // chunk counts above which the layout scans its count table in a kernel of its own
#endif
