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
// Mapping: a workgroup (4 or 6 working waves) owns one (expert, chunk of up
// to 160 rows, N tile of one 32-row weight group per wave).  The chunk's A
// rows are staged through double-buffered LDS two 64-wide K steps at a time
// and shared by the waves; every wave streams its own weight group (B)
// straight into registers four K steps ahead (each weight byte is read once
// from HBM).  GMM1 gives each wave 16 gate and the matching 16 up rows, so
// lane c < 16 and lane c + 16 hold g and u of the same output; GMM2 gives
// each wave 32 output columns.
#include <math.h>

#include "common.hpp"
#include "moe.hpp"
#include "formats.hpp"

namespace ep {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// A tile is 4 or 6 groups of 32 weight rows, one per wave (an even count,
// so that a GMM1 tile covers whole 32-column MX blocks).  A CU moves data at
// a bounded rate, and its time is about the weight bytes of its tiles plus
// the activation bytes of their chunks, which every tile of a chunk reads
// again: wide tiles read the activations fewer times, narrow tiles make more
// work units.  Each launch picks the width whose busiest CU moves fewer
// bytes; workgroups are launched with the wide tile's waves, and with narrow
// tiles the last two waves leave at once.
constexpr int kNarrow = 4, kWide = 6;
constexpr int kThreads = kWide * kWave;
constexpr int kWaves = kWide;                     // waves launched per workgroup
constexpr int kMaxFrags = 5;                      // 32-row fragments per chunk
constexpr int kChunkRows = kMaxFrags * 32;        // rows per work item
constexpr int kKStep = 64;                        // K per matrix-core step
// The chunk's A rows are staged two K steps (128 bytes of a row, one full
// cache line) at a time; a padded row stride of 144 bytes puts the 16-byte
// fragment reads of 16 consecutive rows in distinct LDS banks.  Every thread
// moves the same number of 16-byte pieces per stage; pieces past the
// chunk's rows land in spare LDS rows that are never read.
constexpr int kStageSteps = 2;
constexpr int kStageK = kStageSteps * kKStep;     // K bytes of a row per stage
constexpr int kRowStride = kStageK + 16;          // LDS bytes per staged A row
constexpr int a_pieces(int nf, int waves) { return (nf * 32 * (kStageK / 16) + waves * kWave - 1) / (waves * kWave); }
constexpr int a_stage_rows(int waves) { return a_pieces(kMaxFrags, waves) * waves * kWave / (kStageK / 16); }
constexpr int kAStageRows = a_stage_rows(kNarrow) > a_stage_rows(kWide) ? a_stage_rows(kNarrow) : a_stage_rows(kWide);
constexpr int kAStage = kAStageRows * kRowStride; // bytes of one staged A block
// A scale bytes are loaded 16 per row (eight K steps) at a time into a
// double-buffered table of kThreads rows, padded to 20 bytes so that the
// dword reads of 32 consecutive rows fall in distinct banks.
constexpr int kBodySteps = 8;
constexpr int kScaleStride = 20;
constexpr int kScaleBuf = kThreads * kScaleStride;
constexpr int kStaging = 2 * kAStage + 2 * kScaleBuf;
constexpr int kEpiTileBytes = kChunkRows * (16 * kWide + 1) * 4;   // GMM1 SwiGLU tile of the wide tiles
// GMM2's bf16 tile: dwords per row, 16 past the data of the wide tiles so
// that the two rows one dword store writes start 16 banks apart
constexpr int kGmm2Stride = 16 * kWide + 16;
constexpr int kGmm2TileBytes = kChunkRows * kGmm2Stride * 4;

enum Mode { kGmm1Mx = 0, kGmm1Bf16 = 1, kGmm2 = 2 };

struct Item {
  int expert, row0, rows;                         // rows <= kChunkRows
  int waves;                                      // tile width of the unit
};

// The work of a launch.  Work units are (expert, chunk of up to kChunkRows
// rows, N tile) triples in expert-major order; their number comes from
// workgroup scans over the experts (rows from recv_count when given, else
// the expert block sizes; every thread takes two experts).  The grid is at
// most one workgroup per CU and each workgroup walks its units with a
// stride.  The hardware hands workgroups to the 8 XCDs round-robin, so
// workgroup b runs on XCD b % 8; giving XCD x the contiguous units
// [x * per, (x + 1) * per) keeps each XCD on one or two experts, whose
// activation rows then stay in that XCD's L2 instead of being fetched by
// every XCD.
//
// Tile widths.  A launch first takes one width for all chunks, counting
// every chunk as full (the cost rule above).  When that is the wide tile
// and every unit gets its own workgroup, chunks are then moved to narrow
// tiles, those with the most 32-row fragments first (their units cost the
// most), while the units still fit the grid: a 5-fragment chunk on narrow
// tiles costs less than a 4-fragment one on wide tiles, so the busiest CU
// gets cheaper at no cost to the others.  In such a mixed launch the
// chunks with at least `nf_narrow` fragments take narrow tiles.
constexpr int kXcds = 8;

struct Plan {                                     // uniform over the launch
  int units, per, n_tiles, waves;                 // one width: n_tiles per chunk, `waves` its width
  bool mixed;                                     // both widths (then the fields below)
  int nt_narrow, nt_wide, nf_narrow;
};

// per-expert rows and first chunk (first unit when mixed), for the unit lookups
__shared__ int s_rows[2 * kThreads], s_first[2 * kThreads];

__device__ __forceinline__ int frags_of(int rows) { return (rows + 31) / 32; }

// Units of an expert with `rows` rows in a mixed launch: its full chunks,
// then a partial one.
__device__ __forceinline__ int expert_units(int rows, int nf_narrow, int nt_narrow, int nt_wide) {
  const int full = rows / kChunkRows, rest = rows - full * kChunkRows;
  const int nt_full = kMaxFrags >= nf_narrow ? nt_narrow : nt_wide;
  return full * nt_full + (rest > 0 ? (frags_of(rest) >= nf_narrow ? nt_narrow : nt_wide) : 0);
}

// Exclusive scan of x over the workgroup (every thread one value); returns
// the thread's start and the total in `all`.  Ends with a barrier.
__device__ __forceinline__ int block_scan(int x, int *wsum, int &all) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int x0 = x;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) wsum[wv] = x;
  __syncthreads();
  int before = 0;
  all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    before += i < wv ? wsum[i] : 0;
    all += wsum[i];
  }
  __syncthreads();
  return before + x - x0;
}

// MIX: whether the launch may use both widths (see the kernel).
template <bool MIX>
__device__ __forceinline__ Plan make_plan(int nt_narrow, int nt_wide, int num_cus, int E,
                                          const int *__restrict__ offsets, const int64_t *__restrict__ recv_count) {
  __shared__ int wsum[kWaves];
  __shared__ int bins[kMaxFrags + 1];             // chunks by fragment count
  int cnt[2], ch[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * threadIdx.x + q;
    cnt[q] = 0;
    if (e < E) {
      // rows of expert e: recv_count when given, never more than its block
      const int block = offsets[e + 1] - offsets[e];
      cnt[q] = recv_count ? (int)min((int64_t)block, max(recv_count[e], (int64_t)0)) : block;
    }
    ch[q] = (cnt[q] + kChunkRows - 1) / kChunkRows;
  }
  if (threadIdx.x <= kMaxFrags) bins[threadIdx.x] = 0;
  int chunks;
  const int start = block_scan(ch[0] + ch[1], wsum, chunks);
  s_rows[2 * threadIdx.x] = cnt[0];
  s_rows[2 * threadIdx.x + 1] = cnt[1];
  s_first[2 * threadIdx.x] = start;
  s_first[2 * threadIdx.x + 1] = start + ch[0];
  Plan pl;
  chunks = __builtin_amdgcn_readfirstlane(chunks);
  // a CU's time ~ its units x (weight rows + activation rows) of K bytes
  // each, with chunks taken as full: the tile width with the smaller
  // busiest-CU cost wins (narrow on a tie)
  const int rounds_n = (chunks * nt_narrow + num_cus - 1) / num_cus;
  const int rounds_w = (chunks * nt_wide + num_cus - 1) / num_cus;
  pl.waves = rounds_n * (32 * kNarrow + kChunkRows) <= rounds_w * (32 * kWide + kChunkRows) ? kNarrow : kWide;
  pl.n_tiles = pl.waves == kNarrow ? nt_narrow : nt_wide;
  pl.units = chunks * pl.n_tiles;
  pl.mixed = false;
  pl.nt_narrow = nt_narrow;
  pl.nt_wide = nt_wide;
  pl.nf_narrow = kMaxFrags + 1;
  const int grid = (int)gridDim.x / kXcds * kXcds;   // units one round can take
  if (MIX && pl.waves == kWide && pl.units <= grid && nt_narrow > nt_wide) {
    // one unit per workgroup: move the chunks with the most fragments to
    // narrow tiles while the units still fit
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int full = cnt[q] / kChunkRows, rest = cnt[q] - full * kChunkRows;
      if (full > 0) atomicAdd(&bins[kMaxFrags], full);
      if (rest > 0) atomicAdd(&bins[frags_of(rest)], 1);
    }
    __syncthreads();
    int units = pl.units;
    for (int nf = kMaxFrags; nf >= 1; --nf) {
      const int more = bins[nf] * (nt_narrow - nt_wide);
      if (units + more > grid) break;
      units += more;
      if (more > 0) pl.nf_narrow = nf;
    }
    pl.nf_narrow = __builtin_amdgcn_readfirstlane(pl.nf_narrow);
    if (pl.nf_narrow <= kMaxFrags) {
      // first unit of every expert
      const int u0 = expert_units(cnt[0], pl.nf_narrow, nt_narrow, nt_wide);
      const int u1 = expert_units(cnt[1], pl.nf_narrow, nt_narrow, nt_wide);
      const int ustart = block_scan(u0 + u1, wsum, units);
      s_first[2 * threadIdx.x] = ustart;
      s_first[2 * threadIdx.x + 1] = ustart + u0;
      pl.mixed = true;
      pl.units = __builtin_amdgcn_readfirstlane(units);
    }
  }
  pl.per = (pl.units + kXcds - 1) / kXcds;
  return pl;
}

// The i-th unit of this workgroup, or expert -1 past its last one (uniform).
// Starts with a barrier, so the previous unit's LDS is no longer in use.
__device__ __forceinline__ Item find_item(const Plan &pl, int E, const int *__restrict__ offsets, int i, int &ntile) {
  __shared__ Item found;
  __shared__ int found_tile;
  __syncthreads();
  if (threadIdx.x == 0) found.expert = -1;
  __syncthreads();
  const int slot = blockIdx.x / kXcds + i * (gridDim.x / kXcds);
  const int unit = (blockIdx.x % kXcds) * pl.per + slot;
  if (slot < pl.per && unit < pl.units) {
    if (!pl.mixed) {
      const int item = unit / pl.n_tiles;
      for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int first = s_first[e], rows = s_rows[e];
        const int c = item - first;
        if (c >= 0 && c * kChunkRows < rows) {
          found.expert = e;
          found.row0 = offsets[e] + c * kChunkRows;
          found.rows = min(kChunkRows, rows - c * kChunkRows);
          found.waves = pl.waves;
          found_tile = unit - item * pl.n_tiles;
        }
      }
    } else {
      for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int first = s_first[e], rows = s_rows[e];
        const int u = unit - first;
        if (u >= 0 && u < expert_units(rows, pl.nf_narrow, pl.nt_narrow, pl.nt_wide)) {
          // full chunks first, then the partial one
          const int full = rows / kChunkRows;
          const bool full_narrow = kMaxFrags >= pl.nf_narrow;
          const int nt_full = full_narrow ? pl.nt_narrow : pl.nt_wide;
          const bool in_full = u < full * nt_full;
          const int c = in_full ? u / nt_full : full;
          found.expert = e;
          found.row0 = offsets[e] + c * kChunkRows;
          found.rows = min(kChunkRows, rows - c * kChunkRows);
          found.waves = (in_full ? full_narrow : frags_of(rows - full * kChunkRows) >= pl.nf_narrow) ? kNarrow : kWide;
          found_tile = u - c * nt_full;
        }
      }
    }
  }
  __syncthreads();
  Item it;                                        // the same in every lane: kept in scalar registers
  it.expert = __builtin_amdgcn_readfirstlane(found.expert);
  it.row0 = __builtin_amdgcn_readfirstlane(found.row0);
  it.rows = __builtin_amdgcn_readfirstlane(found.rows);
  it.waves = __builtin_amdgcn_readfirstlane(found.waves);
  ntile = __builtin_amdgcn_readfirstlane(found_tile);
  return it;
}

// silu(z) = z / (1 + e^-z), the quotient taken as z times the hardware
// reciprocal (v_rcp_f32, within 1 ulp) instead of a correctly rounded
// division: expf, the add, the reciprocal and the two products stay within a
// few float32 ulps of the exact a = silu(g)·u, far inside the 2^-20·|a|
// the tests allow for its float32 evaluation, at a sixth of the division's
// instructions (the epilogue is ALU-bound)
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + expf(-z)); }

// Packed weights.  A wave's 32 weight rows form a group: for GMM2 rows
// 32j .. 32j+31; for GMM1 ("gate/up" groups) the gate rows 16j .. 16j+15 and
// the matching up rows I+16j .. I+16j+15.  For each group and 64-wide K step
// the group's fragment is 2048 bytes in matrix-core lane order: bytes
// [0, 1024) hold, for lane l = 32g + r, K bytes [16g, 16g+16) of the
// group's row r at offset 16l; bytes [1024, 2048) hold K bytes [32+16g,
// 48+16g) at 1024 + 16l.  Each 16-byte load of a wave then reads 1 KB in
// one piece.  Scale bytes: for each group and span of four K steps, 256
// bytes where lane l's four bytes (offset 4l) are the e8m0 scales of K-block
// 2(4t+u) + g of row r for u = 0..3 (zero past the last step).  Fragments
// are stored step-major: the fragments of K step s of every group of every
// expert (expert-major, then group) lie together, and so do the scale
// blocks of span t.  The waves of a launch all start at step 0 and advance
// in step, so at any time they read one contiguous stretch of the weights
// (measured 1 % faster than one contiguous stream per group).
__host__ __device__ inline int packed_group_row(int j, int r, int gate_up, int inter) {
  return gate_up ? (r < 16 ? 16 * j + r : inter + 16 * j + (r - 16)) : 32 * j + r;
}

__global__ void pack_weights_kernel(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales, int E, int N,
                                    int K, int gate_up, uint8_t *__restrict__ pcodes, uint8_t *__restrict__ pscales) {
  const int ksteps = K / kKStep, spans = (ksteps + 3) / 4, groups = N / 32, kb = K / 32;
  const int inter = N / 2;
  // one thread per (expert, group, step, half, lane): a 16-byte piece
  const int64_t pieces = (int64_t)E * groups * ksteps * 128;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < pieces; i += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i & 63), half = (int)((i >> 6) & 1);
    const int64_t rest = i >> 7;
    const int s = (int)(rest % ksteps);
    const int64_t eg = rest / ksteps;
    const int j = (int)(eg % groups), e = (int)(eg / groups);
    const int r = lane & 31, g = lane >> 5;
    const int row = packed_group_row(j, r, gate_up, inter);
    const uint8_t *src = codes + ((int64_t)e * N + row) * K + s * kKStep + half * 32 + g * 16;
    const int64_t d = ((int64_t)s * E * groups + eg) * 128 + (i & 127);   // step-major
    *(u32x4 *)(pcodes + d * 16) = *(const u32x4 *)src;
  }
  // one thread per (expert, group, span, lane): four scale bytes
  const int64_t words = (int64_t)E * groups * spans * 64;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i & 63);
    const int64_t rest = i >> 6;
    const int t = (int)(rest % spans);
    const int64_t eg = rest / spans;
    const int j = (int)(eg % groups), e = (int)(eg / groups);
    const int r = lane & 31, g = lane >> 5;
    const int row = packed_group_row(j, r, gate_up, inter);
    uint32_t w = 0;
    for (int u = 0; u < 4; ++u) {
      const int step = 4 * t + u;
      if (step < ksteps) w |= (uint32_t)scales[((int64_t)e * N + row) * kb + step * 2 + g] << (8 * u);
    }
    const int64_t d = ((int64_t)t * E * groups + eg) * 64 + lane;          // span-major
    *(uint32_t *)(pscales + d * 4) = w;
  }
}

// Weight loads are streamed (each weight byte is read once per launch);
// activation rows are shared by the workgroups of an expert through L2.
// Build-time knobs (-D...) for measuring alternatives; the defaults are the
// measured best: EP_MOE_W_NT / EP_MOE_A_NT non-temporal weight / activation
// loads, EP_MOE_ASETS stages of A loads in flight per thread (1, 2 or 4).
#ifndef EP_MOE_W_NT
#define EP_MOE_W_NT 1
#endif
#ifndef EP_MOE_A_NT
#define EP_MOE_A_NT 0
#endif
#ifndef EP_MOE_ASETS
#define EP_MOE_ASETS 2
#endif
template <typename T>
__device__ __forceinline__ T ld_w(const uint8_t *p) {
#if EP_MOE_W_NT
  return __builtin_nontemporal_load((const T *)p);
#else
  return *(const T *)p;
#endif
}
template <typename T>
__device__ __forceinline__ T ld_a(const uint8_t *p) {
#if EP_MOE_A_NT
  return __builtin_nontemporal_load((const T *)p);
#else
  return *(const T *)p;
#endif
}

// The MX-scaled matrix-core step with the A scale taken from byte 2h of
// `as` and the B scale from byte `u` of `bs` (the instruction's op_sel picks
// the bytes, so no extraction is needed; h and u are constants wherever this
// is inlined in the unrolled loop).
template <int HA>
__device__ __forceinline__ v16f mfma_b_byte(int u, const v8i &a, const v8i &b, const v16f &c, int as, int bs) {
  switch (u) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, HA, as, 0, bs);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, HA, as, 1, bs);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, HA, as, 2, bs);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, HA, as, 3, bs);
  }
}
__device__ __forceinline__ v16f mfma_ab_byte(int h, int u, const v8i &a, const v8i &b, const v16f &c, int as,
                                             int bs) {
  return h == 0 ? mfma_b_byte<0>(u, a, b, c, as, bs) : mfma_b_byte<2>(u, a, b, c, as, bs);
}

// Workgroup barrier for LDS hand-offs only.  __syncthreads() carries a
// release fence, which on this target waits for every outstanding vector
// memory operation -- loads included -- and so would drain the weight loads
// in flight at every K step.  Every LDS write here is a ds_write whose data is
// already in registers, so waiting for this wave's LDS operations and then
// meeting at the barrier is enough; the "memory" clobber keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct GemmArgs {
  const uint8_t *a_data, *a_scales;
  int K;
  const uint8_t *w, *w_scales;
  int N_w, nt_narrow, nt_wide, num_cus, inter;
  int groups_all;                                 // weight groups of all experts (E * N_w / 32)
  uint8_t *out_data, *out_scales;
  int out_cols;
};

// Main loop and epilogue for a chunk of NF 32-row fragments.  K is a
// multiple of 128 (whole stages).
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

template <int MODE, int NF, int WE>
__device__ __forceinline__ void gemm_chunk(const GemmArgs &p, const Item &it, int ntile, uint8_t *smem, int tid) {
  constexpr int kThr = WE * kWave;                                // threads of the working waves
  constexpr int kPieces = a_pieces(NF, WE);                       // A pieces per thread per stage
  static_assert(kPieces * kThr / (kStageK / 16) <= kAStageRows, "A pieces fit the staged block");
  constexpr int kEpiCols = 16 * WE;                               // GMM1 SwiGLU columns of the tile
  constexpr int kEpiStride = kEpiCols + 1;                        // floats per LDS row of the epilogue tile
  const int lane = tid & (kWave - 1), wv = tid / kWave;
  const int r = lane & 31, g = lane >> 5;
  const int K = p.K, ksteps = K / kKStep, nstages = ksteps / kStageSteps, kb = K / 32;

  // this wave's packed weight group (see pack_weights_kernel): fragments of
  // 2048 bytes per K step, groups_all fragments apart, scale dwords per span
  // of four steps, groups_all blocks of 256 bytes apart
  // a tile's last waves may lie past N: they repeat the last group (their
  // loads hit the cache lines of the wave that owns it) and store nothing
  const int groups = p.N_w / 32;
  const int group = min(ntile * WE + wv, groups - 1);
  const int spans = (ksteps + 3) / 4;
  const size_t gidx = (size_t)it.expert * (p.N_w / 32) + group;
  const uint8_t *wp = p.w + gidx * (size_t)2048 + lane * 16;
  const uint8_t *wsp = p.w_scales + gidx * (size_t)256 + lane * 4;
  const size_t wstep = (size_t)p.groups_all * 2048, wspan_stride = (size_t)p.groups_all * 256;

  // A staging, branch-free: piece i of this thread is (row, 16-byte piece) =
  // (idx >> 3, idx & 7) of the stage, so 8 lanes read one 128-byte line;
  // rows past the chunk read its last row (their LDS rows are never read)
  const uint8_t *a_chunk = p.a_data + (size_t)it.row0 * K;
  uint32_t apiece[kPieces];                                       // byte offsets within the chunk
  int lpiece[kPieces];
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int idx = tid + i * kThr;
    const int row = idx >> 3, q = idx & 7;
    apiece[i] = (uint32_t)(min(row, it.rows - 1) * K + q * 16);
    lpiece[i] = row * kRowStride + q * 16;
  }
  constexpr int kASets = EP_MOE_ASETS;                            // A loads run kASets stages ahead
  static_assert(4 % kASets == 0, "sets are fixed within a body");
  u32x4 areg[kASets][kPieces];
  auto load_a = [&](int j, int set) {
    const int jj = min(j, nstages - 1);                           // loads past the end are never used
#pragma unroll
    for (int i = 0; i < kPieces; ++i) areg[set][i] = ld_a<u32x4>(a_chunk + apiece[i] + (size_t)jj * kStageK);
  };
  auto store_a = [&](int buf, int set) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) *(u32x4 *)(smem + buf * kAStage + lpiece[i]) = areg[set][i];
  };

  // A scales: thread t keeps row t's 16 scale bytes of the next eight K steps
  // (body b covers steps [8b, 8b + 8)); the table row of thread t is t.  A
  // body's 16 bytes start at byte min(16b, kb - 16) of the row, so a partial
  // last body reads in bounds and its reader adds back the shift.
  const uint8_t *srow = p.a_scales + (size_t)(it.row0 + min(tid, it.rows - 1)) * kb;
  uint32_t *sc_st = (uint32_t *)(smem + 2 * kAStage + tid * kScaleStride);
  u32x4_a4 sc;
  auto load_sc = [&](int body) { sc = ld_a<u32x4_a4>(srow + min(16 * body, kb - 16)); };
  auto store_sc = [&](int buf) {
    uint32_t *d = sc_st + buf * (kScaleBuf / 4);
    d[0] = sc.x;
    d[1] = sc.y;
    d[2] = sc.z;
    d[3] = sc.w;
  };
  const uint8_t *sc_rd0 = smem + 2 * kAStage + r * kScaleStride;  // dword-aligned (shift is a multiple of 4)
  auto sc_reader = [&](int body) {
    const int shift = body == 0 ? 0 : 16 * body - min(16 * body, kb - 16);
    return sc_rd0 + (body & 1) * kScaleBuf + shift;
  };

  // weight ring: kRing K steps of two 16-byte pieces (each wave load reads
  // 1 KB in one piece), and the scale dwords of the current and the next
  // span of four steps (span t in wspan[t & 1], loaded at the first step of
  // span t - 1).  Slot u is refilled only after the matrix-core instructions
  // that read it are issued, so a slot keeps one register across the loop:
  // no copy of a register a load is still writing (a copy would wait for
  // that load and every load before it).
  constexpr int kRing = 4;                                        // K steps of weights in flight per wave
  u32x4 wb0[kRing], wb1[kRing];
  uint32_t wspan[2];
  auto load_w = [&](int s, int slot) {
    const int ss = min(s, ksteps - 1);                             // loads past the end are never used
    wb0[slot] = ld_w<u32x4>(wp + (size_t)ss * wstep);
    wb1[slot] = ld_w<u32x4>(wp + (size_t)ss * wstep + 1024);
  };
  auto load_span = [&](int t, int slot) { wspan[slot] = ld_w<uint32_t>(wsp + (size_t)min(t, spans - 1) * wspan_stride); };

  v16f acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = v16f{};

  // prologue: A stage 0 and body 0's scales in LDS buffer 0 (the scales as
  // four dword loads clamped to the row, which may be shorter than 16 bytes);
  // A stages 1 .. kASets in register sets 1 .. kASets-1, 0; weight steps
  // 0 .. kRing-1 in flight
  load_a(0, 0);
#pragma unroll
  for (int d = 0; d < 4; ++d) sc[d] = *(const uint32_t *)(srow + min(4 * d, kb - 4));
  store_a(0, 0);
  store_sc(0);
#pragma unroll
  for (int q = 1; q < kASets; ++q) load_a(q, q);
  load_a(kASets, 0);
#pragma unroll
  for (int q = 0; q < kRing; ++q) load_w(q, q);
  load_span(0, 0);
  lds_barrier();

  // stage j (i = j % 4 within its body): write A(j+1) (register set
  // (j+1) % kASets, loaded kASets stages ago) to LDS buffer (j+1) & 1 and
  // reload the set with A(j+1+kASets); in a full body, stage 0 loads the next body's scales and
  // stage 3 writes them to their table; then the two K steps of stage j from
  // buffer j & 1, each followed by the refill of its weight slot; one barrier
  // per stage
  auto stage = [&](int j, int i, bool full, int body, const uint8_t *sc_rd) {
    store_a((i + 1) & 1, (i + 1) % kASets);
    load_a(j + 1 + kASets, (i + 1) % kASets);
    if (full && i == 0) load_sc(body + 1);
    if (full && i == 3) store_sc((body + 1) & 1);
    const uint8_t *abase = smem + (i & 1) * kAStage;
    // the stage's A scale bytes of each fragment row: one dword (blocks
    // 4i .. 4i+3 of the body), shifted so that byte 2h is lane (r, g)'s
    // block of step h
    int xsw[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f)
      xsw[f] = (int)(*(const uint32_t *)(sc_rd + f * 32 * kScaleStride + 4 * i) >> (8 * g));
#pragma unroll
    for (int h = 0; h < kStageSteps; ++h) {
      const int sb = kStageSteps * i + h;                          // step within the body
      const int u = sb % kRing;
      const v8i bv = {(int)wb0[u].x, (int)wb0[u].y, (int)wb0[u].z, (int)wb0[u].w,
                      (int)wb1[u].x, (int)wb1[u].y, (int)wb1[u].z, (int)wb1[u].w};
      const int bsc = (int)wspan[(sb >> 2) & 1];                   // byte sb & 3 of the span dword, by op_sel
      // A fragments in two register sets, so that the LDS read of fragment
      // f + 1 is in flight while the matrix core works on fragment f
      v8i av[2];
      auto read_a = [&](int f) {
        const int row = f * 32 + r;
        const u32x4 x0 = *(const u32x4 *)(abase + row * kRowStride + h * kKStep + g * 16);
        const u32x4 x1 = *(const u32x4 *)(abase + row * kRowStride + h * kKStep + 32 + g * 16);
        av[f & 1] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      };
      read_a(0);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (f + 1 < NF) read_a(f + 1);
        acc[f] = mfma_ab_byte(h, sb & 3, av[f & 1], bv, acc[f], xsw[f], bsc);
      }
      load_w(kStageSteps * j + h + kRing, u);
      if ((sb & 3) == 0) load_span((kStageSteps * j + h) / 4 + 1, ((sb >> 2) + 1) & 1);
    }
    lds_barrier();
  };
  int j0 = 0, body = 0;
  for (; (j0 + 4) * kStageSteps <= ksteps; j0 += 4, ++body) {
    const uint8_t *sc_rd = sc_reader(body);
#pragma unroll
    for (int i = 0; i < 4; ++i) stage(j0 + i, i, true, body, sc_rd);
  }
  {
    const uint8_t *sc_rd = sc_reader(body);
#pragma unroll
    for (int i = 0; i < 3; ++i)
      if (j0 + i < nstages) stage(j0 + i, i, false, body, sc_rd);  // uniform tail
  }
  // every load issued past the last step targets registers nobody reads;
  // let them land before the registers and the kernel go away
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---------------------------------------------------------------- epilogue
  if constexpr (MODE == kGmm2) {
    // bf16 rows through an LDS tile [rows][32 * WE], so that the stores to
    // HBM are 16-byte pieces of whole row segments.  Lane (r, g) holds
    // column r of this wave's 32 at rows 8b + 4g + i of each fragment.  The
    // last stage's barrier has retired every read of the staging buffers
    // this tile overwrites.
    uint32_t *tile = (uint32_t *)smem;
    constexpr int kDw = 16 * WE;                                  // dwords of a tile row's data
    uint16_t *tcol = (uint16_t *)smem + wv * 32 + r;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = f * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
        tcol[row * (2 * kGmm2Stride)] = (uint16_t)(pack_bf16x2(acc[f][i], 0.0f) & 0xffffu);
      }
    }
    lds_barrier();
    // each thread: 16-byte pieces (8 columns) of the tile's rows; pieces of
    // a wave group past N are not stored
    constexpr int kRowPieces = kDw / 4;
    const int c0 = ntile * (WE * 32);
    for (int job = tid; job < it.rows * kRowPieces; job += kThr) {
      const int row = job / kRowPieces, q = job - row * kRowPieces;
      if (ntile * WE + (q >> 2) >= groups) continue;
      const u32x4 v = *(const u32x4 *)(tile + row * kGmm2Stride + 4 * q);
      *(u32x4 *)(p.out_data + ((size_t)(it.row0 + row) * p.out_cols + c0 + 8 * q) * 2) = v;
    }
  } else {
    // SwiGLU: lane r < 16 holds gate column r, lane r + 16 the matching up
    // column.  For each pair of rows (i, i + 1), v_permlane16_swap exchanges
    // lanes 16..31 of row i with lanes 0..15 of row i + 1 (in each 32-lane
    // half), so that lane r < 16 then holds the gate and up of row i and
    // lane r + 16 those of row i + 1: every lane evaluates one silu per two
    // rows.  The 16 results of each wave go to an LDS tile [rows][16 * waves].
    float *tile = (float *)smem;
    const int hi = r >> 4;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const auto gu = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[f][i]), __float_as_uint(acc[f][i + 1]),
                                                         false, false);
        const int row = f * 32 + (i >> 2) * 8 + g * 4 + (i & 3) + hi;
        tile[row * kEpiStride + wv * 16 + (r & 15)] = silu(__uint_as_float(gu[0])) * __uint_as_float(gu[1]);
      }
    }
    lds_barrier();
    // each thread: one (row, 32-column block) of the tile
    const int n0 = ntile * kEpiCols;
    constexpr int kBlocks = kEpiCols / 32;
    for (int job = tid; job < it.rows * kBlocks; job += kThr) {
      const int row = job / kBlocks, blk = job - row * kBlocks;
      if (n0 + blk * 32 >= p.out_cols) continue;                  // past I (a partial last tile)
      const float *src = tile + row * kEpiStride + blk * 32;
      const size_t orow = (size_t)(it.row0 + row);
      if constexpr (MODE == kGmm1Bf16) {
        uint32_t o[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) o[e] = pack_bf16x2(src[2 * e], src[2 * e + 1]);
        u32x4 *dst = (u32x4 *)(p.out_data + (orow * p.out_cols + n0 + blk * 32) * 2);
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
        u32x4 *dst = (u32x4 *)(p.out_data + orow * p.out_cols + n0 + blk * 32);
        dst[0] = u32x4{q[0].x, q[0].y, q[1].x, q[1].y};
        dst[1] = u32x4{q[2].x, q[2].y, q[3].x, q[3].y};
        p.out_scales[orow * (p.out_cols / 32) + (n0 >> 5) + blk] = (uint8_t)(se + 127);
      }
    }
  }
}

template <int MODE, int WE>
__device__ __forceinline__ void gemm_frags(const GemmArgs &p, const Item &it, int ntile, uint8_t *smem, int tid) {
  static_assert(kMaxFrags == 5, "one instantiation per fragment count 1..kMaxFrags");
  switch ((it.rows + 31) / 32) {                                 // uniform: one instantiation per fragment count
    case 1: gemm_chunk<MODE, 1, WE>(p, it, ntile, smem, tid); break;
    case 2: gemm_chunk<MODE, 2, WE>(p, it, ntile, smem, tid); break;
    case 3: gemm_chunk<MODE, 3, WE>(p, it, ntile, smem, tid); break;
    case 4: gemm_chunk<MODE, 4, WE>(p, it, ntile, smem, tid); break;
    default: gemm_chunk<MODE, 5, WE>(p, it, ntile, smem, tid); break;
  }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void mx_gmm_kernel(GemmArgs p, const int *__restrict__ offsets,
                                                          const int64_t *__restrict__ recv_count, int E) {
  constexpr int kTile = MODE == kGmm2 ? kGmm2TileBytes : kEpiTileBytes;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStaging > kTile ? kStaging : kTile];
  // GMM2 launches keep one width: the exit below that a launch with both
  // widths needs made GMM2's compiled loop about 10 % slower, and at the
  // sizes measured GMM2 never had room for narrow tiles anyway
  constexpr bool kMix = MODE != kGmm2;
  const Plan pl = make_plan<kMix>(p.nt_narrow, p.nt_wide, p.num_cus, E, offsets, recv_count);
  // with narrow tiles the last waves have no weight group; a wave that has
  // ended no longer takes part in the workgroup's barriers (the wave index
  // is read as a scalar, so that these exits are branches of whole waves)
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  if (wave >= pl.waves) return;
  for (int i = 0;; ++i) {
    int ntile;
    const Item it = find_item(pl, E, offsets, i, ntile);
    if (it.expert < 0) return;                                   // uniform
    // a launch with both widths gives every workgroup at most one unit, so
    // the waves a narrow unit does not use are done
    if constexpr (kMix) {
      if (wave >= it.waves) return;
    }
    // the thread index passes through an empty asm in every iteration, so
    // that no address derived from it is hoisted out of this loop (held
    // across a whole unit, those would crowd out the GEMM's registers)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    if ((kMix ? it.waves : pl.waves) == kNarrow)
      gemm_frags<MODE, kNarrow>(p, it, ntile, smem, tid);
    else
      gemm_frags<MODE, kWide>(p, it, ntile, smem, tid);
  }
}

// CUs of the current device (cached per device).
int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace

// Workgroups of a GEMM launch: one per possible work unit, at most one per
// CU (a multiple of the XCD count, so that every XCD walks its units with the
// same stride); a workgroup with no unit leaves at once.
int64_t persistent_grid(int64_t units_upper) {
  const int cus = device_cus();
  const int64_t cap = cus >= kXcds ? cus / kXcds * kXcds : kXcds;
  const int64_t g = (units_upper + kXcds - 1) / kXcds * kXcds;
  return g < cap ? g : cap;
}

hipError_t launch_moe_pack(const void *codes, const void *scales, int E, int N, int K, int gate_up, void *pcodes,
                           void *pscales, hipStream_t s) {
  hipLaunchKernelGGL(pack_weights_kernel, dim3(1024), dim3(256), 0, s, (const uint8_t *)codes, (const uint8_t *)scales,
                     E, N, K, gate_up, (uint8_t *)pcodes, (uint8_t *)pscales);
  return hipGetLastError();
}

hipError_t launch_moe_gmm1(const ep_handle_t &h, const int64_t *recv_count, const char *x_buf, int hidden, int inter,
                           const void *w1, const void *w1_scales, int out_quant, char *out_buf, hipStream_t s) {
  const RecvGeom gx = recv_geom(h.max_rows, hidden, EP_QUANT_MXFP8);
  const int groups = inter / 16;                                  // 2I weight rows in groups of 32
  const int ntn = (groups + kNarrow - 1) / kNarrow, ntw = (groups + kWide - 1) / kWide;
  const int64_t items = (h.max_rows + kChunkRows - 1) / kChunkRows + h.num_experts;
  const int64_t blocks = persistent_grid(items * ntn);
  if (h.num_tokens == 0 || blocks == 0) return hipSuccess;
  GemmArgs p{(const uint8_t *)x_buf, (const uint8_t *)x_buf + gx.scale_off, hidden, (const uint8_t *)w1,
             (const uint8_t *)w1_scales, 2 * inter, ntn, ntw, device_cus(), inter, h.num_experts * (2 * inter / 32),
             (uint8_t *)out_buf, nullptr, inter};
  if (out_quant == EP_QUANT_MXFP8) {
    p.out_scales = (uint8_t *)out_buf + recv_geom(h.max_rows, inter, EP_QUANT_MXFP8).scale_off;
    hipLaunchKernelGGL(mx_gmm_kernel<kGmm1Mx>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, h.offsets,
                       recv_count, h.num_experts);
  } else {
    hipLaunchKernelGGL(mx_gmm_kernel<kGmm1Bf16>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, h.offsets,
                       recv_count, h.num_experts);
  }
  return hipGetLastError();
}

hipError_t launch_moe_gmm2(const ep_handle_t &h, const int64_t *recv_count, const char *a_buf, int inter, int hidden,
                           const void *w2, const void *w2_scales, char *out_buf, hipStream_t s) {
  const RecvGeom ga = recv_geom(h.max_rows, inter, EP_QUANT_MXFP8);
  const int groups = hidden / 32;
  const int ntn = (groups + kNarrow - 1) / kNarrow, ntw = (groups + kWide - 1) / kWide;
  const int64_t items = (h.max_rows + kChunkRows - 1) / kChunkRows + h.num_experts;
  const int64_t blocks = persistent_grid(items * ntn);
  if (h.num_tokens == 0 || blocks == 0) return hipSuccess;
  const GemmArgs p{(const uint8_t *)a_buf, (const uint8_t *)a_buf + ga.scale_off, inter, (const uint8_t *)w2,
                   (const uint8_t *)w2_scales, hidden, ntn, ntw, device_cus(), inter, h.num_experts * (hidden / 32),
                   (uint8_t *)out_buf, nullptr, hidden};
  hipLaunchKernelGGL(mx_gmm_kernel<kGmm2>, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, h.offsets, recv_count,
                     h.num_experts);
  return hipGetLastError();
}

}  // namespace ep
