// Routing layout kernels: expert histogram, exclusive scan and stable
// token-order slot assignment for gfx950.
//
// What is computed ("Low-Latency Mode API", Parameters topk_idx and
// cumulative_local_expert_recv_stats, Return Values recv_count): for the T*k
// (token, j) pairs in (t, j) order, pair f = t*k + j with a valid expert e
// gets receive row offsets[e] + (number of earlier pairs with expert e).
//
// How: a workgroup of 16 wave64s owns a contiguous chunk of pairs; each wave
// walks its sub-range 64 pairs at a time.  For one step, the lanes holding the
// same expert find each other with one ballot per key bit (the AND of the
// matching ballots is the set of lanes with an equal key), so a lane's rank
// among equal lanes is the popcount of that set below it.  A per-wave LDS
// counter per expert carries the count across steps (the wave's LDS
// operations complete in program order, so every lane reads the counter
// before the leader of its group bumps it).  Per-wave counts are then turned
// into per-wave bases by a prefix over the 16 waves.  Nothing depends on the
// order in which atomics or waves happen to run: the result is deterministic.
//
// Receive rows are arranged in one of three ways: compact (expert e's block
// is exactly its count), aligned (every block is rounded up to a multiple of
// `align` rows) or capacity-padded (every block is `cap` rows; pairs past the
// cap-th of an expert are dropped and set a status bit).  Rows that hold no
// pair get row_src -1.
//
// Small problems (pairs <= 6144) run in one workgroup that also does the scan
// over experts and writes every output: one launch (padded arrangements with
// many rows add workgroups that only clear free rows).  (All of its waves share
// one CU, so its cost grows by about a microsecond per 64-pair step of a
// wave, against about four for a second launch.)  Larger ones run in two
// launches over 2048-pair chunks: rank (per-chunk counts and ranks), then
// finalize (each workgroup redoes the small scan over chunk counts itself).
// With more than 128 chunks (262144 pairs) that redone scan, which reads the
// whole chunk-count table in every workgroup, would grow with the square
// of the chunk count; a column-scan kernel between the two then turns the
// table into prefixes once, and each finalize workgroup reads two rows.
#include "common.hpp"
#include "tuning.hpp"

namespace ep {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kSingleItems = 6;                    // up to 6 * 1024 pairs in one workgroup
constexpr int kMultiItems = EP_LAYOUT_ITEMS;       // pairs per thread in a multi-block chunk
constexpr int kMultiChunk = kMultiItems * kThreads;
constexpr int64_t kSingleMaxPairs = (int64_t)kSingleItems * kThreads;
constexpr int64_t kSingleMaxRows = 65536;          // single workgroup also clears row_src tail
constexpr int kMaxFillBlocks = 512;                // finalize workgroups beyond the chunk count
constexpr int kHelperRows = 2048;                  // rows per clearing helper of the single-workgroup path
// Above this many chunks the count table's columns are scanned by a kernel
// of their own before finalize (three launches instead of two).
constexpr int kColscanMinChunks = EP_LAYOUT_COLSCAN_MIN;

// Expert of an id, or -1 for -1 / ids outside [-1, E) (which set `bad`).
template <typename IdxT>
__device__ __forceinline__ int expert_of(IdxT raw, int E, bool &bad) {
  const int64_t v = (int64_t)raw;
  if (v >= 0 && v < (int64_t)E) return (int)v;
  bad |= v != -1;
  return -1;
}

// Rows of expert block with `c` pairs: c rounded up to `align`, or `cap`.
__device__ __forceinline__ int block_rows(int c, int align, int cap) {
  return cap > 0 ? cap : (c + align - 1) / align * align;
}

// -1 into row_src for every row that holds no pair.  This thread is number
// `first` of `step` (both multiples of the wave size apart).  offs[e] (block
// start) and kept[e] (pairs the block holds) are in LDS.  Free rows are the
// rows at or past nrows (compact and aligned arrangements) and the end of
// every padded block, [offs[e] + kept[e], block end): each such tail is
// walked by a wave (by S waves together when there are S times more waves
// than experts), so no row has to search for its block.
__device__ __forceinline__ void clear_free_rows(int *__restrict__ row_src, int first, int step, int max_rows,
                                                int nrows, int E, int align, int cap, const int *offs,
                                                const int *kept) {
  for (int r = nrows + first; r < max_rows; r += step) row_src[r] = -1;
  if (align <= 1 && cap <= 0) return;
  const int lane = first & (kWave - 1);
  const int nw = step / kWave, gw = first / kWave;
  const int S = nw > E ? nw / E : 1;
  for (int u = gw; u < E * S; u += nw) {
    const int e = u / S, part = u - e * S;
    const int lo = offs[e] + kept[e];
    const int hi = offs[e] + (cap > 0 ? cap : block_rows(kept[e], align, 0));
    for (int r = lo + part * kWave + lane; r < hi; r += S * kWave) row_src[r] = -1;
  }
}

// Stable rank of each of this thread's pairs among the equal-expert pairs
// of its wave's sub-range (the wave clears its own counters first).  Wave w owns pairs [begin + w*steps*64, begin +
// (w+1)*steps*64) (steps <= ITEMS, uniform), walked 64 at a time.  On return
// cnt[w*E + e] is the number of wave-w pairs with expert e; ex[i] is the
// expert (or -1) and lr[i] the rank within the wave.  All ids are loaded
// before the matching starts, so a wave has its ITEMS loads in flight at once.
template <typename IdxT, int ITEMS>
__device__ __forceinline__ void wave_rank(const IdxT *__restrict__ idx, int begin, int n, int E, int nbits,
                                          int steps, int *cnt, int (&ex)[ITEMS], int (&lr)[ITEMS],
                                          bool &bad) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int *my = cnt + w * E;
  const uint64_t below = (1ull << lane) - 1ull;
  const int wbegin = begin + w * steps * kWave;
  // all loads first (clamped to a valid pair, so none sits in a branch and
  // they are in flight together), then the classification
  IdxT raw[ITEMS];
  if (n > 0) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) raw[it] = idx[min(wbegin + it * kWave + lane, n - 1)];
  }
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int f = wbegin + it * kWave + lane;
    ex[it] = (it < steps && f < n) ? expert_of(raw[it], E, bad) : -1;
  }
  // this wave's counters; only this wave touches them until the caller's
  // barrier, and a wave's LDS accesses complete in program order
  for (int e = lane; e < E; e += kWave) my[e] = 0;
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    lr[it] = 0;
    if (it >= steps) continue;                       // uniform
    const int e = ex[it];
    const int key = e < 0 ? E : e;
    uint64_t same = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int rank = __popcll(same & below);
    const int tot = __popcll(same);
    int r = 0;
    if (e >= 0) r = my[e] + rank;
    if (e >= 0 && rank == 0) my[e] = r + tot;
    lr[it] = r;
  }
}

// cnt[w*E + e] (counts) -> per-wave exclusive bases; total[e] = block count.
// All 16 counts of an expert are read before any is written, so the reads
// are in flight together.
__device__ __forceinline__ void wave_bases(int *cnt, int *total, int E) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) c[w] = cnt[w * E + e];
    int run = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      cnt[w * E + e] = run;
      run += c[w];
    }
    total[e] = run;
  }
}

// Exclusive scan of one int per thread over a 1024-thread block: a wave
// scan, then every thread adds the totals of the waves before its own (16
// broadcast LDS reads).  Returns the exclusive prefix and the block total.
__device__ __forceinline__ int block_exclusive_scan(int v, int *wsum, int &total) {
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
  for (int i = 0; i < kWaves; ++i) {
    const int c = wsum[i];
    all += c;
    before += i < w ? c : 0;
  }
  total = all;
  return before + x - v;
}

template <typename IdxT>
__global__ __launch_bounds__(kThreads) void layout_single_kernel(
    const IdxT *__restrict__ idx, int n, int E, int max_rows, int align, int cap,
    int64_t *__restrict__ recv_count, int *__restrict__ cum, int *__restrict__ offsets, int *__restrict__ slot,
    int *__restrict__ row_src, uint32_t *__restrict__ status) {
  __shared__ int cnt[kWaves * kMaxExperts];
  __shared__ int total[kMaxExperts];
  __shared__ int excl[kMaxExperts];
  __shared__ int kept[kMaxExperts];
  __shared__ int wsum[kWaves];
  __shared__ uint32_t sbad;
  if (blockIdx.x > 0) {
    // helper workgroups (padded arrangements with many rows): recount the
    // experts with LDS atomics (order-free, so the same counts as workgroup
    // 0), redo the scan over blocks and clear a share of the free rows --
    // one workgroup alone is limited by the stores it can keep in flight
    for (int e = threadIdx.x; e < E; e += kThreads) total[e] = 0;
    __syncthreads();
    bool ignored = false;
    for (int f = threadIdx.x; f < n; f += kThreads) {
      const int e = expert_of(idx[f], E, ignored);
      if (e >= 0) atomicAdd(&total[e], 1);
    }
    __syncthreads();
    const int c = threadIdx.x < E ? total[threadIdx.x] : 0;
    int nrows;
    const int pre = block_exclusive_scan(threadIdx.x < E ? block_rows(c, align, cap) : 0, wsum, nrows);
    if (threadIdx.x < E) {
      excl[threadIdx.x] = pre;
      kept[threadIdx.x] = cap > 0 ? min(c, cap) : c;
    }
    __syncthreads();
    clear_free_rows(row_src, (blockIdx.x - 1) * kThreads + threadIdx.x, (gridDim.x - 1) * kThreads, max_rows,
                    nrows, E, align, cap, excl, kept);
    return;
  }
  if (threadIdx.x == 0) sbad = 0;

  const int nbits = 32 - __builtin_clz((unsigned)E);   // keys 0..E
  const int steps = (n + kThreads - 1) / kThreads;     // 64-pair steps per wave, <= kSingleItems
  int ex[kSingleItems], lr[kSingleItems];
  bool bad = false;
  wave_rank<IdxT, kSingleItems>(idx, 0, n, E, nbits, steps, cnt, ex, lr, bad);
  __syncthreads();
  wave_bases(cnt, total, E);
  __syncthreads();

  const int c = threadIdx.x < E ? total[threadIdx.x] : 0;
  int nrows;
  const int pre = block_exclusive_scan(threadIdx.x < E ? block_rows(c, align, cap) : 0, wsum, nrows);
  const int k_e = cap > 0 ? min(c, cap) : c;
  if (threadIdx.x < E) {
    excl[threadIdx.x] = pre;
    kept[threadIdx.x] = k_e;
    recv_count[threadIdx.x] = k_e;
    offsets[threadIdx.x] = pre;
    if (cum) cum[threadIdx.x] += c;
  }
  if (threadIdx.x == 0) offsets[E] = nrows;
  if (bad) atomicOr(&sbad, EP_STATUS_ID_OUT_OF_RANGE);
  if (k_e < c) atomicOr(&sbad, EP_STATUS_CAPACITY_OVERFLOW);
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
#pragma unroll
  for (int it = 0; it < kSingleItems; ++it) {
    const int f = w * steps * kWave + it * kWave + lane;
    if (it >= steps || f >= n) continue;
    const int e = ex[it];
    const int local = e >= 0 ? cnt[w * E + e] + lr[it] : 0;
    if (e >= 0 && (cap <= 0 || local < cap)) {
      const int r = excl[e] + local;
      slot[f] = r;
      row_src[r] = f;
    } else {
      slot[f] = -1;
    }
  }
  if (gridDim.x == 1) clear_free_rows(row_src, threadIdx.x, kThreads, max_rows, nrows, E, align, cap, excl, kept);
  if (threadIdx.x == 0) *status = sbad;
}

// Multi-block pass 1 (chunk b): per-chunk counts hist[b*E + e] and, in
// slot[f], the pair's expert and chunk-local rank packed as (e << 16) | rank
// (-1 if not routed); bstat[b] = out-of-range flag of the chunk.  `cnt` is
// LDS of kWaves * E ints, `total` of E ints.
template <typename IdxT>
__device__ __forceinline__ void rank_chunk(const IdxT *__restrict__ idx, int n, int E, int b, int *__restrict__ hist,
                                           uint32_t *__restrict__ bstat, int *__restrict__ slot, int *cnt,
                                           int *total, uint32_t *sbad) {
  if (threadIdx.x == 0) *sbad = 0;
  const int nbits = 32 - __builtin_clz((unsigned)E);
  const int begin = b * kMultiChunk;
  int ex[kMultiItems], lr[kMultiItems];
  bool bad = false;
  wave_rank<IdxT, kMultiItems>(idx, begin, n, E, nbits, kMultiItems, cnt, ex, lr, bad);
  __syncthreads();
  wave_bases(cnt, total, E);
  if (bad) atomicOr(sbad, 1u);
  __syncthreads();

  for (int e = threadIdx.x; e < E; e += kThreads) hist[(int64_t)b * E + e] = total[e];
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
#pragma unroll
  for (int it = 0; it < kMultiItems; ++it) {
    const int f = begin + w * kMultiItems * kWave + it * kWave + lane;
    if (f >= n) continue;
    const int e = ex[it];
    slot[f] = e >= 0 ? (e << 16) | (cnt[w * E + e] + lr[it]) : -1;
  }
  if (threadIdx.x == 0) bstat[b] = *sbad;
}

template <typename IdxT>
__global__ __launch_bounds__(kThreads) void layout_rank_kernel(const IdxT *__restrict__ idx, int n, int E,
                                                               int *__restrict__ hist,
                                                               uint32_t *__restrict__ bstat,
                                                               int *__restrict__ slot) {
  __shared__ int cnt[kWaves * kMaxExperts];
  __shared__ int total[kMaxExperts];
  __shared__ uint32_t sbad;
  rank_chunk(idx, n, E, blockIdx.x, hist, bstat, slot, cnt, total, &sbad);
}

// Multi-block pass 2.  Every workgroup re-derives from hist (read through
// LDS, a few tens of KB from L2) the per-expert totals, the exclusive scan
// over experts and its own chunk's per-expert base, so no workgroup waits for
// another.  Workgroup b < nblocks finalises the slots of chunk b (loaded
// first, so that load overlaps the scan); workgroup 0 also writes counts,
// offsets, statistics and status; all of them clear row_src past R.  `tile`
// is LDS of kTileInts ints, `base` of E ints.
constexpr int kTileInts = 8192;
static_assert(kTileInts % kThreads == 0, "a tile is whole loads per thread");

template <bool SCANNED>
__device__ __forceinline__ void finalize_chunk(int n, int E, int max_rows, int align, int cap, int nblocks, int b,
                                               const int *__restrict__ hist, const uint32_t *__restrict__ bstat,
                                               int64_t *__restrict__ recv_count, int *__restrict__ cum,
                                               int *__restrict__ offsets, int *__restrict__ slot,
                                               int *__restrict__ row_src, uint32_t *__restrict__ status, int *tile,
                                               int *base, int *offs, int *kept, int *wsum, uint32_t *sbad) {
  const int e = threadIdx.x;
  if (threadIdx.x == 0) *sbad = 0;

  int v[kMultiItems];
  if (n > 0) {
#pragma unroll
    for (int it = 0; it < kMultiItems; ++it) v[it] = slot[min(b * kMultiChunk + it * kThreads + (int)threadIdx.x, n - 1)];
  }
#pragma unroll
  for (int it = 0; it < kMultiItems; ++it) {
    const int f = b * kMultiChunk + it * kThreads + threadIdx.x;
    v[it] = (b < nblocks && f < n) ? v[it] : -1;
  }
  uint32_t bad = 0;
  if (b == 0)
    for (int i = threadIdx.x; i < nblocks; i += kThreads) bad |= bstat[i];

  int tot = 0, pre = 0;
  if constexpr (SCANNED) {
    // hist holds inclusive prefixes down each expert's column (the column
    // scan): chunk b's base is row b - 1, the totals are the last row
    if (e < E && nblocks > 0) {
      tot = hist[(int64_t)(nblocks - 1) * E + e];
      pre = b == 0 ? 0 : (b < nblocks ? hist[(int64_t)(b - 1) * E + e] : tot);
    }
  } else {
  const int tile_rows = kTileInts / E;
  // this thread's share of a tile (rows * E <= kTileInts ints) is loaded
  // whole before any of it is stored, so the loads are in flight together;
  // the next tile's share is loaded before the current tile is summed
  constexpr int kPart = kTileInts / kThreads;
  int part[kPart];
  auto load_part = [&](int b0) {
    const int m = min(tile_rows, nblocks - b0) * E;
#pragma unroll
    for (int u = 0; u < kPart; ++u) part[u] = hist[(int64_t)b0 * E + min(u * kThreads + (int)threadIdx.x, m - 1)];
  };
  if (nblocks > 0) load_part(0);
  for (int b0 = 0; b0 < nblocks; b0 += tile_rows) {
    const int rows = min(tile_rows, nblocks - b0);
    const int m = rows * E;
#pragma unroll
    for (int u = 0; u < kPart; ++u)
      if (u * kThreads + (int)threadIdx.x < m) tile[u * kThreads + threadIdx.x] = part[u];
    __syncthreads();
    if (b0 + tile_rows < nblocks) load_part(b0 + tile_rows);
    if (e < E) {
      const int mine = min(max(b - b0, 0), rows);   // rows of this tile before chunk b
      int r = 0;
      for (; r + 4 <= rows; r += 4) {
        const int c0 = tile[r * E + e], c1 = tile[(r + 1) * E + e];
        const int c2 = tile[(r + 2) * E + e], c3 = tile[(r + 3) * E + e];
        tot += c0 + c1 + c2 + c3;
        pre += (r < mine ? c0 : 0) + (r + 1 < mine ? c1 : 0) + (r + 2 < mine ? c2 : 0) + (r + 3 < mine ? c3 : 0);
      }
      for (; r < rows; ++r) {
        const int c0 = tile[r * E + e];
        tot += c0;
        pre += r < mine ? c0 : 0;
      }
    }
    __syncthreads();
  }
  }
  int nrows;
  const int p = block_exclusive_scan(e < E ? block_rows(tot, align, cap) : 0, wsum, nrows);
  const int k_e = cap > 0 ? min(tot, cap) : tot;
  if (e < E) {
    base[e] = pre;
    offs[e] = p;
    kept[e] = k_e;
  }
  if (b == 0) {
    if (e < E) {
      recv_count[e] = k_e;
      offsets[e] = p;
      if (cum) cum[e] += tot;
    }
    if (k_e < tot) bad |= EP_STATUS_CAPACITY_OVERFLOW;
    if (bad) atomicOr(sbad, bad);
  }
  __syncthreads();
  if (b == 0 && threadIdx.x == 0) {
    offsets[E] = nrows;
    *status = *sbad;
  }
#pragma unroll
  for (int it = 0; it < kMultiItems; ++it) {
    if (v[it] < 0) continue;
    const int f = b * kMultiChunk + it * kThreads + threadIdx.x;
    const int e = v[it] >> 16;
    const int local = base[e] + (v[it] & 0xffff);
    if (cap > 0 && local >= cap) {
      slot[f] = -1;
      continue;
    }
    const int r = offs[e] + local;
    slot[f] = r;
    row_src[r] = f;
  }
  clear_free_rows(row_src, b * kThreads + threadIdx.x, gridDim.x * kThreads, max_rows, nrows, E, align, cap,
                  offs, kept);
}

template <bool SCANNED>
__global__ __launch_bounds__(kThreads) void layout_finalize_kernel(
    int n, int E, int max_rows, int align, int cap, int nblocks, const int *__restrict__ hist,
    const uint32_t *__restrict__ bstat, int64_t *__restrict__ recv_count, int *__restrict__ cum,
    int *__restrict__ offsets, int *__restrict__ slot, int *__restrict__ row_src, uint32_t *__restrict__ status) {
  __shared__ int tile[kTileInts];
  __shared__ int base[kMaxExperts];
  __shared__ int offs[kMaxExperts];
  __shared__ int kept[kMaxExperts];
  __shared__ int wsum[kWaves];
  __shared__ uint32_t sbad;
  finalize_chunk<SCANNED>(n, E, max_rows, align, cap, nblocks, blockIdx.x, hist, bstat, recv_count, cum, offsets,
                          slot, row_src, status, tile, base, offs, kept, wsum, &sbad);
}

// Column scan between the two passes of a layout with many chunks: the
// chunk counts hist[b*E + e] become inclusive prefixes down each expert's
// column, so that each finalize workgroup reads two rows of the table
// instead of all of it (whose cost grows with the square of the chunk
// count).  Workgroup g owns 16 experts [16g, 16g + 16) and splits the
// chunks into 64 runs of L = ceil(nblocks / 64): thread t handles expert
// 16g + t % 16 over run t / 16, so the 16 threads of one run read one
// contiguous 64-byte piece of a row.  Each thread sums its run, the runs'
// sums are added up through LDS in run order, and a second walk writes the
// prefixes in place.  (16 experts per workgroup spread the table's reads
// over E / 16 CUs; one CU per 64 experts was limited by its own fetch.)
constexpr int kScanCols = 16;                         // experts per column-scan workgroup
constexpr int kScanRuns = kThreads / kScanCols;       // runs of chunks per expert
constexpr int kScanBatch = 16;                        // loads in flight per thread
__global__ __launch_bounds__(kThreads) void layout_colscan_kernel(int *__restrict__ hist, int nblocks, int E) {
  __shared__ int part[kScanRuns][kScanCols];
  const int c = threadIdx.x % kScanCols, run_id = threadIdx.x / kScanCols;
  const int e = blockIdx.x * kScanCols + c;
  const bool on = e < E;
  const int L = (nblocks + kScanRuns - 1) / kScanRuns;
  const int b0 = min(run_id * L, nblocks), b1 = min(b0 + L, nblocks);
  int s = 0;
  for (int b = b0; b < b1; b += kScanBatch) {
    int v[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) v[u] = on && b + u < b1 ? hist[(int64_t)(b + u) * E + e] : 0;
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) s += v[u];
  }
  part[run_id][c] = s;
  __syncthreads();
  int run = 0;
  for (int i = 0; i < run_id; ++i) run += part[i][c];
  for (int b = b0; b < b1; b += kScanBatch) {
    int v[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) v[u] = on && b + u < b1 ? hist[(int64_t)(b + u) * E + e] : 0;
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      run += v[u];
      if (on && b + u < b1) hist[(int64_t)(b + u) * E + e] = run;
    }
  }
}

template <typename IdxT>
hipError_t launch_typed(const IdxT *idx, int n, int32_t E, int max_rows, int align, int cap, int64_t *recv_count,
                        int32_t *cum, char *ws, const WsLayout &wl, hipStream_t s) {
  int *offsets = (int *)(ws + wl.offsets);
  int *slot = (int *)(ws + wl.slot);
  int *row_src = (int *)(ws + wl.row_src);
  uint32_t *status = (uint32_t *)(ws + wl.status);
  if (n <= kSingleMaxPairs && max_rows <= kSingleMaxRows) {
    // padded arrangements with many rows add helper workgroups that clear
    // the free rows (about kHelperRows rows each)
    const bool padded = align > 1 || cap > 0;
    const int helpers = padded && max_rows > kHelperRows ? (max_rows + kHelperRows - 1) / kHelperRows : 0;
    hipLaunchKernelGGL(layout_single_kernel<IdxT>, dim3(1 + helpers), dim3(kThreads), 0, s, idx, n, E, max_rows,
                       align, cap, recv_count, cum, offsets, slot, row_src, status);
    return hipGetLastError();
  }
  int *hist = (int *)(ws + wl.hist);
  uint32_t *bstat = (uint32_t *)(ws + wl.bstat);
  const int nb = (n + kMultiChunk - 1) / kMultiChunk;
  // enough workgroups for the slots of every chunk and for clearing free rows
  // (capped: every workgroup re-reads the chunk counts, and a grid-stride
  // loop covers any number of rows)
  const int64_t want = (max_rows + kMultiChunk - 1) / kMultiChunk;
  const int fill_blocks = (int)(want < kMaxFillBlocks ? want : kMaxFillBlocks);
  const int grid = nb > fill_blocks ? nb : (fill_blocks > 0 ? fill_blocks : 1);
  if (nb > 0) {
    hipLaunchKernelGGL(layout_rank_kernel<IdxT>, dim3(nb), dim3(kThreads), 0, s, idx, n, E, hist, bstat, slot);
  }
  if (nb > kColscanMinChunks) {
    // many chunks: scan the count table's columns once, then each finalize
    // workgroup reads two of its rows
    hipLaunchKernelGGL(layout_colscan_kernel, dim3((E + kScanCols - 1) / kScanCols), dim3(kThreads), 0, s, hist, nb,
                       E);
    hipLaunchKernelGGL(layout_finalize_kernel<true>, dim3(grid), dim3(kThreads), 0, s, n, E, max_rows, align, cap,
                       nb, hist, bstat, recv_count, cum, offsets, slot, row_src, status);
  } else {
    hipLaunchKernelGGL(layout_finalize_kernel<false>, dim3(grid), dim3(kThreads), 0, s, n, E, max_rows, align, cap,
                       nb, hist, bstat, recv_count, cum, offsets, slot, row_src, status);
  }
  return hipGetLastError();
}

}  // namespace

WsLayout workspace_layout(int64_t max_tokens, int32_t k, int32_t E, int64_t max_rows) {
  WsLayout wl{};
  const int64_t pairs = max_tokens * k;
  const int64_t nb = (pairs + kMultiChunk - 1) / kMultiChunk;
  size_t off = 0;
  wl.offsets = off; off = align_up(off + sizeof(int32_t) * (size_t)(E + 1), kWsAlign);
  wl.slot = off;    off = align_up(off + sizeof(int32_t) * (size_t)pairs, kWsAlign);
  wl.row_src = off; off = align_up(off + sizeof(int32_t) * (size_t)max_rows, kWsAlign);
  wl.status = off;  off = align_up(off + sizeof(uint32_t), kWsAlign);
  wl.hist = off;    off = align_up(off + sizeof(int32_t) * (size_t)(nb * E), kWsAlign);
  wl.bstat = off;   off = align_up(off + sizeof(uint32_t) * (size_t)nb, kWsAlign);
  wl.total = off;
  wl.nblocks = nb;
  return wl;
}

hipError_t launch_layout(const void *idx, int idx64, int64_t T, int32_t k, int32_t E, int64_t max_rows, int32_t align,
                         int32_t cap, int64_t *recv_count, int32_t *cum, char *ws, const WsLayout &wl,
                         hipStream_t s) {
  const int n = (int)(T * k);
  if (idx64) return launch_typed((const int64_t *)idx, n, E, (int)max_rows, align, cap, recv_count, cum, ws, wl, s);
  return launch_typed((const int32_t *)idx, n, E, (int)max_rows, align, cap, recv_count, cum, ws, wl, s);
}

}  // namespace ep
