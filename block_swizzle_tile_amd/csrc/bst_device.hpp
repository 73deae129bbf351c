// bst_device.hpp -- device side of the swizzled tiled GEMM for gfx950.
//
// One persistent kernel template serves every form (plain, batched, grouped
// slice-M, int8 with dequant) and every operand type:
//   * the block -> tile scheduler of GemmIdentityBlockSwizzle ("Block
//     Scheduler Code Explained", CATLASS docs: s4.1 loop counts, s4.4 batch
//     index, s4.5 Zn / Nz windows with snake reversal, s4.6 tail shapes, s6
//     runtime offset / direction) evaluated per task in scalar registers;
//   * an optional K split (unit u -> slice u / T, task u % T, in the manner
//     of GetBatchIdx) with an in-kernel, fixed-order fix-up;
//   * a double-buffered global -> LDS pipeline: 16-byte coalesced loads,
//     LDS rows of 128 bytes (one K stage) whose 16-byte chunks are
//     XOR-permuted by the row index so that MFMA fragment reads and stage
//     writes spread over all banks; B (row-major K x N) is transposed in
//     registers on its way into LDS so that every MFMA operand is K-packed;
//   * the 32x32 MFMA family of CDNA4 (f16 / bf16 x16, i8 x32, scaled fp8
//     x64) with operands swapped (B^T as src0, A^T as src1) so that each lane
//     ends up holding four consecutive output columns of one row;
//   * tail masking on every load and store, and an epilogue that converts to
//     f16 / bf16 / f32 / i32 and optionally applies the per-token x
//     per-channel dequant in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace bst {

enum AbKind { AB_F16 = 1, AB_BF16 = 2, AB_E4M3 = 3, AB_MXE4M3 = 4, AB_I8 = 5 };
// Problem forms a kernel instance is built for: plain or batched (the batch
// index of task t is t / tiles per batch), grouped slice-M (groups stacked
// along M, group table of first tasks and rows), grouped slice-K (K cut
// into groups, one output per group; tasks numbered like batches, group
// table of first K indices).
enum Form { FORM_DENSE = 0, FORM_SLICE_M = 1, FORM_SLICE_K = 2 };
enum OutKind { OUT_F16 = 1, OUT_BF16 = 2, OUT_I32 = 6, OUT_F32 = 7 };

constexpr int kRowBytes = 128;      // bytes of one LDS row = one K stage of one row
constexpr int kMaxGroups = 1024;
constexpr int kNumXcd = 8;          // MI355X: 8 accelerator dies, one L2 each

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_byte_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_out_t;

// ------------------------------------------------------------ arguments ---
// Division of 32-bit unsigned values by a divisor fixed for a launch,
// without a division instruction: q = (mulhi(n, mul) + n) >> shift with the
// multiplier and shift precomputed on the host (the round-up reciprocal
// method of Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994).  Exact for every n < 2^32 and 1 <= d < 2^31.
struct FastDiv {
  uint32_t d, mul, shift;
  __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t hi = __umulhi(n, mul);
#else
    const uint32_t hi = (uint32_t)(((uint64_t)n * mul) >> 32);
#endif
    return (uint32_t)(((uint64_t)hi + n) >> shift);
  }
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f{d, 0u, 0u};
  if (d == 0) return f;
  uint32_t l = 0;
  while (l < 32 && (1ull << l) < d) ++l;  // l = ceil(log2 d)
  f.shift = l;
  f.mul = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
  return f;
}

// The block map of one launch with fixed loop counts (plain, batched and
// slice-K problems), precomputed on the host: the window order of
// GetBlockCoord ("Block Scheduler Code Explained", s4.5) reduced to
// multiplications.  The direction's major dimension is cut into W windows
// of o tile-lines (the last one holds `last`); span = o x (tile-lines of the
// minor dimension).  RASTER is the Nz order with one window spanning every
// column (offset >= loopsN), which walks the tiles row by row.
struct MapConsts {
  uint32_t nz;        // 0: windows of tile-rows (Zn); 1: of tile-columns (Nz, RASTER)
  uint32_t o, W, last, loops_min;
  FastDiv span, by_o, by_last, core, tiles, nk_full;
};

struct GemmArgs {
  const uint8_t* A;
  const uint8_t* B;
  uint8_t* C;
  const uint8_t* X;                   // matmul-add: addend of C's type and shape, or null
  int64_t ldx;                        // its leading dimension (elements)
  int64_t lda, ldb, ldc;              // elements
  int64_t strideA, strideB, strideC;  // elements; batch (or group, for B) strides
  const uint8_t* sa;                  // MX scales of A [M][ldsa]
  const uint8_t* sb;                  // MX scales of B [K/32][ldsb]
  int64_t ldsa, ldsb;
  const float* row_scale;             // dequant, per stacked row
  const float* col_scale;             // dequant, [G][N]
  const int32_t* group_m;             // grouped slice-M: device int32[G] row counts
  const int32_t* group_k;             // grouped slice-K: device int32[G] K counts
  int32_t G;
  int64_t total_m;                    // grouped slice-M: rows allocated in A and C
  int64_t total_k;                    // grouped slice-K: K columns / rows allocated in A / B
  uint32_t M, N, K;                   // M unused when grouped
  uint32_t batch;
  uint32_t tiles;                     // non-grouped: batch * loopsM * loopsN
  uint32_t off, dir;
  uint32_t split;                     // K slices per tile (>= 1)
  uint32_t kslice;                    // K elements per slice (multiple of the stage depth)
  uint32_t remap;                     // XCD-contiguous renumbering of workgroups
  uint32_t shuffle_k;                 // rotate each whole-stage task's K-loop start (ShuffleK)
  uint32_t preload;                   // issue the next unit's first stages before the epilogue
  uint32_t* queue;                    // dynamic task allocation: 8 queue counters + exit count
                                      // (null: static stride)
  uint32_t grid;                      // workgroups launched (gridDim.x, passed here because the
                                      // kernel would read it from the dispatch packet in host
                                      // memory: about a microsecond at every kernel start)
  uint32_t cdtype;                    // OutKind
  float* ws_part;                     // split > 1: [split][tile capacity][BM*BN] partials
  uint32_t* ws_count;                 // split > 1: one arrival counter per tile
  uint32_t tile_cap;                  // tiles the workspace was sized for
  MapConsts mc;                       // plain, batched, slice-K: the map's constants
  uint32_t* map_out;                  // map-dump kernel only
  uint64_t* trace;                    // BST_TRACE builds only: per-wave cycle counts of workgroup 0
  uint64_t* clock;                    // measurement hook (null: off): per-workgroup clock record
  uint32_t clock_n;                   // workgroups recorded (the first clock_n)
};

// Clock record of a workgroup (LDS-DMA kernels, when a.clock is set):
// the 100 MHz reference counter at the workgroup's start and end and the
// shader cycles in between, so that shader cycles / reference ticks is the
// shader clock it ran at.
struct ClockMark {
  uint64_t ref0 = 0, sh0 = 0;
  __device__ __forceinline__ void start(const GemmArgs& a) {
    if (a.clock != nullptr) {
      ref0 = __builtin_amdgcn_s_memrealtime();
      sh0 = __builtin_amdgcn_s_memtime();
    }
  }
  __device__ __forceinline__ void stop(const GemmArgs& a) {
    if (a.clock != nullptr && threadIdx.x == 0 && blockIdx.x < a.clock_n) {
      __builtin_amdgcn_s_waitcnt(0);
      const uint64_t sh1 = __builtin_amdgcn_s_memtime();
      const uint64_t ref1 = __builtin_amdgcn_s_memrealtime();
      uint64_t* o = a.clock + 4 * blockIdx.x;
      o[0] = ref0;
      o[1] = ref1;
      o[2] = sh1 - sh0;
      o[3] = 1;
    }
  }
};

// ------------------------------------------------------------ scheduler ---
// Block coordinate of the `inner`-th task of one loopsM x loopsN problem
// (s4.5 GetBlockCoord).  An offset beyond the tile count gives the same
// order as one window, so it is clamped first; that keeps every product in
// 32 bits.
struct TileCoord {
  uint32_t m, n;
};

__host__ __device__ __forceinline__ TileCoord block_coord(uint32_t loopsM, uint32_t loopsN, uint32_t off,
                                                 uint32_t dir, uint32_t inner) {
  TileCoord c;
  if (dir == 0) {  // Zn
    const uint32_t o = off < loopsM ? off : loopsM;
    const uint32_t span = o * loopsN;
    const uint32_t w = inner / span;
    const uint32_t j = inner - w * span;
    const uint32_t windows = (loopsM + o - 1) / o;
    const uint32_t rows = (w == windows - 1) ? loopsM - o * w : o;
    c.m = w * o + j % rows;
    c.n = j / rows;
    if (w & 1u) c.n = loopsN - 1 - c.n;  // snake (s5.2)
  } else if (dir == 1) {  // Nz: Zn with the roles of M and N exchanged
    const uint32_t o = off < loopsN ? off : loopsN;
    const uint32_t span = o * loopsM;
    const uint32_t w = inner / span;
    const uint32_t j = inner - w * span;
    const uint32_t windows = (loopsN + o - 1) / o;
    const uint32_t cols = (w == windows - 1) ? loopsN - o * w : o;
    c.n = w * o + j % cols;
    c.m = j / cols;
    if (w & 1u) c.m = loopsM - 1 - c.m;
  } else {  // RASTER
    c.m = inner / loopsN;
    c.n = inner - c.m * loopsN;
  }
  return c;
}

// block_coord with the launch's precomputed constants (same results).
__host__ __device__ __forceinline__ TileCoord block_coord_fast(const MapConsts& mc, uint32_t inner) {
  const uint32_t w = mc.span.div(inner);
  const uint32_t j = inner - w * mc.span.d;
  const bool tail = w == mc.W - 1;
  const uint32_t q = tail ? mc.by_last.div(j) : mc.by_o.div(j);
  const uint32_t rows = tail ? mc.last : mc.o;
  const uint32_t maj = w * mc.o + (j - q * rows);
  const uint32_t mnr = (w & 1u) ? mc.loops_min - 1 - q : q;  // snake (s5.2)
  TileCoord c;
  c.m = mc.nz ? mnr : maj;
  c.n = mc.nz ? maj : mnr;
  return c;
}

// Everything a workgroup needs to know about one task.
struct Task {
  uint32_t idx;      // batch index or group index
  uint32_t m, n;     // block coordinate inside its problem
  uint32_t mAct, nAct;
  int64_t row0;      // first row of the tile in the (stacked) A / C
  uint32_t rows_valid;  // rows of the tile inside the allocation (<= mAct)
  uint32_t poison = 0;  // slice-K group the LDS-DMA kernels cannot take: NaN / INT32_MIN out
};

// Grouped problems: per-workgroup table in LDS of each group's first task
// and first row, built once from the device group sizes.  A group's rows are
// clamped to the rows still left in the allocation (negative sizes count as
// 0), so the task count never exceeds ceil(total_m / BM) + G tile-rows.
struct GroupTable {
  union {
    uint32_t first_task[kMaxGroups + 1];  // slice-M: each group's first task
    uint32_t order[kMaxGroups + 1];       // slice-K: the groups in run order (below)
  };
  int64_t first_row[kMaxGroups + 1];
};

__host__ __device__ inline void fill_group_table(GroupTable& gt, const int32_t* group_m, int G,
                                                 int64_t total_m, uint32_t BM, uint32_t loopsN) {
  uint32_t t = 0;
  int64_t r = 0;
  for (int g = 0; g < G; ++g) {
    gt.first_task[g] = t;
    gt.first_row[g] = r;
    int64_t mg = group_m[g] > 0 ? group_m[g] : 0;
    if (mg > total_m - r) mg = total_m - r;
    t += ((uint32_t)mg + BM - 1) / BM * loopsN;
    r += mg;
  }
  gt.first_task[G] = t;
  gt.first_row[G] = r;
}

__device__ __forceinline__ void build_group_table(GroupTable& gt, const GemmArgs& a, uint32_t BM,
                                                  uint32_t loopsN) {
  if (threadIdx.x == 0) fill_group_table(gt, a.group_m, a.G, a.total_m, BM, loopsN);
  __syncthreads();
}

// Grouped slice-K: first_row[g] holds the group's first K index (the
// earlier groups' sizes summed), first_row[G] the end of the last group.
// Sizes below 0 count as 0 and a group is cut to the K still left of
// total_k, so no group reads past the allocation.
__host__ __device__ inline void fill_k_prefix(GroupTable& gt, const int32_t* group_k, int G,
                                              int64_t total_k) {
  int64_t q = 0;
  for (int g = 0; g < G; ++g) {
    gt.first_row[g] = q;
    int64_t kg = group_k[g] > 0 ? group_k[g] : 0;
    if (kg > total_k - q) kg = total_k - q;
    q += kg;
  }
  gt.first_row[G] = q;
}

// Run order of slice-K groups: every tile of group g costs in proportion to
// its K size, so the tasks of the longest groups go first (largest K first,
// ties by index; the longest-processing-time-first rule): they start in the
// first round, and the short ones fill in behind them.
// order[r] is the group of rank r.  Ranking is O(G) per group, so beyond
// kOrderMaxGroups groups the index order is kept.  Only which workgroup runs
// a task, and when, changes: every task still computes its own tile.
constexpr int kOrderMaxGroups = 256;
__host__ __device__ inline void rank_k_group(GroupTable& gt, int G, int i) {
  if (G > kOrderMaxGroups) {
    gt.order[i] = (uint32_t)i;
    return;
  }
  const int64_t ki = gt.first_row[i + 1] - gt.first_row[i];
  int r = 0;
  for (int j = 0; j < G; ++j) {
    const int64_t kj = gt.first_row[j + 1] - gt.first_row[j];
    r += (kj > ki || (kj == ki && j < i)) ? 1 : 0;
  }
  gt.order[r] = (uint32_t)i;
}

__host__ inline void fill_k_table(GroupTable& gt, const int32_t* group_k, int G,
                                  int64_t total_k) {
  fill_k_prefix(gt, group_k, G, total_k);
  for (int i = 0; i < G; ++i) rank_k_group(gt, G, i);
}

__device__ __forceinline__ void build_k_table(GroupTable& gt, const GemmArgs& a) {
  if (threadIdx.x == 0) fill_k_prefix(gt, a.group_k, a.G, a.total_k);
  __syncthreads();
  for (int i = (int)threadIdx.x; i < a.G; i += (int)blockDim.x) rank_k_group(gt, a.G, i);
  __syncthreads();
}

// Task of position t in the run order of a slice-K launch: the groups'
// tasks are numbered like batches (t / tiles per group), and the group
// position maps through the run order.
__host__ __device__ __forceinline__ uint32_t slicek_task(const GemmArgs& a, const GroupTable* gt,
                                                         uint32_t t) {
  const uint32_t pos = a.mc.core.div(t);
  return gt->order[pos] * a.mc.core.d + (t - pos * a.mc.core.d);
}

// K range [k0, k1) of slice s of a task whose K runs over [kq, kq + kg):
// slices of ks elements (a multiple of the stage depth), the last one
// shorter, slices past the end empty (k0 >= k1).
struct KRange {
  uint32_t k0, k1;
};
__host__ __device__ __forceinline__ KRange slice_range(uint32_t kq, uint32_t kg, uint32_t ks,
                                                       uint32_t s) {
  const uint32_t lo = s * ks;
  const uint32_t hi = (lo >= kg || kg - lo < ks) ? kg : lo + ks;
  return KRange{kq + lo, kq + hi};
}

// Slice length of a slice-K group of kg elements cut into `split` slices of
// whole stages of depth bk.
__host__ __device__ __forceinline__ uint32_t group_kslice(uint32_t kg, uint32_t split, uint32_t bk) {
  const uint32_t stages = (kg + bk - 1) / bk;
  return (stages + split - 1) / split * bk;
}

__host__ __device__ __forceinline__ Task decode_task(const GemmArgs& a, uint32_t t, uint32_t BM, uint32_t BN,
                                            const GroupTable* gt) {
  Task k;
  const uint32_t loopsN = (a.N + BN - 1) / BN;
  uint32_t Mp, inner;
  if (gt) {
    // last group whose first task is <= t (binary search; empty groups own no task)
    int lo = 0, hi = a.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (gt->first_task[mid] <= t) lo = mid; else hi = mid - 1;
    }
    k.idx = (uint32_t)lo;
    inner = t - gt->first_task[lo];
    Mp = (uint32_t)(gt->first_row[lo + 1] - gt->first_row[lo]);
  } else {
    const uint32_t core = a.mc.core.d;  // s4.3 GetCoreLoops: loopsM * loopsN
    k.idx = a.mc.core.div(t);           // s4.4 GetBatchIdx
    inner = t - k.idx * core;
    Mp = a.M;
  }
  const uint32_t loopsM = (Mp + BM - 1) / BM;
  const TileCoord c = gt ? block_coord(loopsM, loopsN, a.off, a.dir, inner)
                         : block_coord_fast(a.mc, inner);
  k.m = c.m;
  k.n = c.n;
  k.mAct = (c.m == loopsM - 1) ? Mp - c.m * BM : BM;  // s4.6 GetActualBlockShape
  k.nAct = (c.n == loopsN - 1) ? a.N - c.n * BN : BN;
  if (gt) {
    k.row0 = gt->first_row[k.idx] + (int64_t)c.m * BM;
    const int64_t room = a.total_m - k.row0;
    k.rows_valid = room <= 0 ? 0u : (room < (int64_t)k.mAct ? (uint32_t)room : k.mAct);
  } else {
    k.row0 = (int64_t)c.m * BM;
    k.rows_valid = k.mAct;
  }
  return k;
}

// MapConsts of a problem with loopsM x loopsN tiles per batch / group,
// `tiles` tasks in all and nk_full stages in a full K slice.
inline MapConsts make_map_consts(uint32_t loopsM, uint32_t loopsN, uint32_t off, uint32_t dir,
                                 uint32_t tiles, uint32_t nk_full) {
  MapConsts mc{};
  const bool nz = dir != 0;
  const uint32_t maj = nz ? loopsN : loopsM, mnr = nz ? loopsM : loopsN;
  uint32_t o = dir == 2 ? maj : (off < maj ? off : maj);  // RASTER: one window
  if (o == 0) o = 1;
  mc.nz = nz ? 1u : 0u;
  mc.o = o;
  mc.W = maj == 0 ? 1u : (maj + o - 1) / o;
  mc.last = maj == 0 ? o : maj - o * (mc.W - 1);
  mc.loops_min = mnr;
  mc.span = make_fastdiv(o * (mnr ? mnr : 1u));
  mc.by_o = make_fastdiv(o);
  mc.by_last = make_fastdiv(mc.last ? mc.last : 1u);
  mc.core = make_fastdiv(loopsM * loopsN ? loopsM * loopsN : 1u);
  mc.tiles = make_fastdiv(tiles ? tiles : 1u);
  mc.nk_full = make_fastdiv(nk_full ? nk_full : 1u);
  return mc;
}

// Workgroup renumbering: hardware places workgroup w on XCD w % 8; with
// remap on, XCD x gets a contiguous block of logical indices.  G: the
// number of workgroups launched.
// Branch-free, so that the compiler issues every kernel-argument load of the
// kernel's start in one batch instead of waiting for `remap` first.
__device__ __forceinline__ uint32_t logical_wg(uint32_t remap, uint32_t G) {
  const uint32_t w = blockIdx.x;
  const uint32_t x = w % kNumXcd, q = w / kNumXcd;
  const uint32_t base = G / kNumXcd, rem = G % kNumXcd;
  const uint32_t lw = x * base + (x < rem ? x : rem) + q;
  return remap ? lw : w;
}

// The value x, as if computed at this point: whatever the compiler derives
// from the result stays after it.  Lane and wave indices pass through this
// at the start of each task's set-up and epilogue; otherwise the compiler
// hoists every per-lane address and mask (all loop-invariant across the
// tasks of a persistent workgroup) to the kernel's start, where they stay
// live across the K loop and the large tiles spill them to scratch.
__device__ __forceinline__ uint32_t fresh_v(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ uint32_t fresh_s(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

__device__ __forceinline__ uint32_t xcc_id() {
  // HW_REG_XCC_ID (hardware register 20), bits [3:0]
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 0xf;
}

// ------------------------------------------------------------- traits -----
template <int AB>
struct Traits;
template <>
struct Traits<AB_F16> {
  static constexpr int ES = 2, BK = 64, KBR = 4, MFMA_K = 16, FRAG_DW = 4;
  static constexpr bool IS_INT = false, SCALED = false;
};
template <>
struct Traits<AB_BF16> {
  static constexpr int ES = 2, BK = 64, KBR = 4, MFMA_K = 16, FRAG_DW = 4;
  static constexpr bool IS_INT = false, SCALED = false;
};
template <>
struct Traits<AB_I8> {
  static constexpr int ES = 1, BK = 128, KBR = 8, MFMA_K = 32, FRAG_DW = 4;
  static constexpr bool IS_INT = true, SCALED = false;
};
// fp8 e4m3 operands: plain (every block scale 2^0, fed as the constant
// 0x7f) and MX (e8m0 block scales from memory) are separate kernels, so that
// neither carries a run-time test on the scales.
template <>
struct Traits<AB_E4M3> {
  static constexpr int ES = 1, BK = 128, KBR = 8, MFMA_K = 64, FRAG_DW = 8;
  static constexpr bool IS_INT = false, SCALED = false;
};
template <>
struct Traits<AB_MXE4M3> {
  static constexpr int ES = 1, BK = 128, KBR = 8, MFMA_K = 64, FRAG_DW = 8;
  static constexpr bool IS_INT = false, SCALED = true;
};

// One 32x32 MFMA step: acc(32 n x 32 m) += Bt(32 n x k) * At(k x 32 m).
template <int AB, typename Acc, typename Frag>
__device__ __forceinline__ void mfma32(Acc& acc, const Frag& bt, const Frag& at, uint32_t sc_b,
                                       uint32_t sc_a) {
  if constexpr (AB == AB_F16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, bt),
                                                 __builtin_bit_cast(half8_t, at), acc, 0, 0, 0);
  } else if constexpr (AB == AB_BF16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bt),
                                                  __builtin_bit_cast(bf16x8_t, at), acc, 0, 0, 0);
  } else if constexpr (AB == AB_I8) {
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4_t, bt),
                                                __builtin_bit_cast(i32x4_t, at), acc, 0, 0, 0);
  } else {
    // operand format 0 = FP8 E4M3 for both sources; scale bytes from bits [7:0]
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8_t, bt),
                                                          __builtin_bit_cast(i32x8_t, at), acc, 0,
                                                          0, 0, (int)sc_b, 0, (int)sc_a);
  }
}

// XOR permutation of the eight 16-byte chunks of LDS row r.
__host__ __device__ __forceinline__ uint32_t swz(uint32_t r) { return (r ^ (r >> 3)) & 7u; }

__device__ __forceinline__ uint32_t lds_off(uint32_t row, uint32_t chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

// 16 bytes from global memory, `valid` of them kept (the rest read as 0).
// A 16-byte-aligned whole chunk is one vector load; anything else (a tail,
// or a chunk that starts mid-way, as slice-K groups of any size make) is
// read byte by byte.
__device__ __forceinline__ u32x4_t load16(const uint8_t* p, int valid) {
  if (valid >= 16 && ((uintptr_t)p & 15u) == 0) return *reinterpret_cast<const u32x4_t*>(p);
  if (valid > 16) valid = 16;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (valid > 0) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int e = 0; e < 16; ++e)
      if (e < valid) w[e >> 2] |= (uint32_t)p[e] << ((e & 3) * 8);
    v = u32x4_t{w[0], w[1], w[2], w[3]};
  }
  return v;
}

// ---------------------------------------------------------------- kernel --
// ------------------------------------------------------------ epilogue --
// Shared by both kernel families: the fixed-order split-K fix-up and the
// conversion / dequant / masked store of a wave's 32x32 sub-tiles.
// A call the epilogue makes before its first store: after its dequant scale
// loads are issued where it gathers them up front (no-op by default).  The
// dynamic allocation requests its next ticket there: a device-scope atomic
// issued before those loads would have to complete before the scales could
// be used, since vector-memory operations are counted in issue order.
struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

template <int AB, int BM, int BN, int WM, int WN, int FORM>
struct Epilogue {
  using T = Traits<AB>;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  using Acc = typename std::conditional<T::IS_INT, i32x16_t, f32x16_t>::type;

  // Split-K: every slice stores its partial tile; the last slice to arrive
  // adds the partials in slice order 0..split-1 (so the result does not
  // depend on arrival order) and returns true; the others return false.  The
  // tile's counter is back at zero when the last slice leaves.
  //
  // The slices of a tile may run on different XCDs, whose L2 caches are not
  // coherent with each other.  Partials are therefore written and read with
  // the device-scope cache policy (the L2 writes them through and never
  // serves them stale) and ordered by waiting for the stores to complete
  // before the arrival counter is bumped.  This avoids device-scope fences,
  // which write back and invalidate the whole L2 and so cost every other
  // workgroup on the XCD its cached A and B panels.  Partial tile layout:
  // [wave][sub-tile][quarter][lane][4 values], so every wave instruction
  // moves 1 KiB of contiguous memory.
  static constexpr int kDeviceScope = 16;  // cache policy bit sc1 on gfx950

  __device__ __attribute__((always_inline)) static bool fixup(const GemmArgs& a,
                                                              Acc (&acc)[FM][FN], uint32_t s,
                                                              uint32_t t) {
    if (a.split <= 1) return true;
    __shared__ uint32_t last_flag;
    const uint32_t wave = fresh_s(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    const uint32_t lane = fresh_v(threadIdx.x & 63u);
    const size_t tile_bytes = (size_t)BM * BN * 4;
    const uint32_t wave_off = wave * FM * FN * 4096u + lane * 16u;
    {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<uint8_t*>(a.ws_part) + ((size_t)s * a.tile_cap + t) * tile_bytes,
          (short)0, (int)tile_bytes, 0x00020000);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            u32x4_t v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // copy the element out first: a bit_cast of a vector-element
              // expression would read element 0
              const auto x = acc[i][j][4 * q + e];
              v[e] = __builtin_bit_cast(uint32_t, x);
            }
            __builtin_amdgcn_raw_buffer_store_b128(v, r, wave_off + (i * FN + j) * 4096u + q * 1024u,
                                                   0, kDeviceScope);
          }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t prev =
          __hip_atomic_fetch_add(&a.ws_count[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_flag = (prev == a.split - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (last_flag == 0) return false;
    // Sum in slice order.  A whole slice's partials (two slices' when the
    // wave's part of the tile is small enough to hold twice in registers)
    // are requested before any is added, so the loads overlap instead of
    // waiting one by one.
    constexpr uint32_t PAIR = (FM * FN <= 4) ? 2u : 1u;
    Acc sum[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum[i][j][e] = 0;
    for (uint32_t ss = 0; ss < a.split; ss += PAIR) {
      const bool two = PAIR == 2 && ss + 1 < a.split;
      u32x4_t v0[FM][FN][4], v1[FM][FN][4];
      const __amdgpu_buffer_rsrc_t r0 = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<uint8_t*>(a.ws_part) + ((size_t)ss * a.tile_cap + t) * tile_bytes,
          (short)0, (int)tile_bytes, 0x00020000);
      // the second slice's descriptor is range-limited to 0 bytes when absent
      const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<uint8_t*>(a.ws_part) +
              ((size_t)(two ? ss + 1 : ss) * a.tile_cap + t) * tile_bytes,
          (short)0, two ? (int)tile_bytes : 0, 0x00020000);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t off = wave_off + (i * FN + j) * 4096u + q * 1024u;
            v0[i][j][q] = __builtin_amdgcn_raw_buffer_load_b128(r0, off, 0, kDeviceScope);
            if constexpr (PAIR == 2)
              v1[i][j][q] = __builtin_amdgcn_raw_buffer_load_b128(r1, off, 0, kDeviceScope);
            else
              v1[i][j][q] = u32x4_t{0, 0, 0, 0};
          }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t x0 = v0[i][j][q][e], x1 = v1[i][j][q][e];
              if constexpr (T::IS_INT) {
                sum[i][j][4 * q + e] += __builtin_bit_cast(int, x0);
                if (two) sum[i][j][4 * q + e] += __builtin_bit_cast(int, x1);
              } else {
                sum[i][j][4 * q + e] += __builtin_bit_cast(float, x0);
                if (two) sum[i][j][4 * q + e] += __builtin_bit_cast(float, x1);
              }
            }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = sum[i][j];
    if (threadIdx.x == 0)
      __hip_atomic_store(&a.ws_count[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }

  // Rows per staging pass of a whole tile through SB bytes of LDS (rows of
  // PITCH bytes): the most rows, a multiple of 32 dividing BM, that fit and
  // that the NTH threads copy out in whole 16-byte chunks; 0 if none.
  static constexpr int stage_rows(int bm, int pitch, int sb, int cpr, int nth) {
    for (int rp = bm; rp >= 32; rp -= 32)
      if (bm % rp == 0 && rp * pitch <= sb && (rp * cpr) % nth == 0) return rp;
    return 0;
  }

  // Two output elements packed into one dword, rounded to nearest even
  // (the gfx950 conversions round that way in the default mode).
  template <int OUT>
  __device__ static __forceinline__ uint32_t pack2(float x, float y) {
    if constexpr (OUT == OUT_F16)
      return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y) << 16);
    else
      return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)y) << 16);
  }

  // Stores of a wave's sub-tiles as output kind OUT; lane holds rows l32,
  // columns 8g + 4*hi + {0..3} of each 32x32 sub-tile.  DEQ applies the
  // per-row and per-column scales, out = (float(acc) * row) * column.  FULL:
  // every row and column of the tile is inside the problem, so each lane
  // writes its 4 consecutive values with one vector store and no mask.
  //
  // SB > 0: `stage` is SB bytes of LDS the workgroup no longer needs.  A
  // whole tile goes through it, in passes of as many rows as fit (rows
  // padded by 16 bytes): the waves write the pass's values row-major into
  // LDS, then every thread stores consecutive 16-byte chunks, so a store
  // instruction writes whole cache lines instead of 16 bytes in each of 32
  // rows (those partial lines stay dirty in L2 and cost their write-back
  // when the kernel ends).  All waves of the workgroup call this together
  // (it has barriers).
  template <int OUT, bool DEQ, bool FULL, int SB, bool ADD, class Hook = NoHook>
  __device__ static __forceinline__ void store_as(const GemmArgs& a, const Task& tk,
                                                  const Acc (&acc)[FM][FN], uint32_t wm,
                                                  uint32_t wn, lds_byte_t* stage,
                                                  const Hook& hook = Hook()) {
    constexpr int OS = (OUT == OUT_F16 || OUT == OUT_BF16) ? 2 : 4;
    constexpr int PITCH = BN * OS + 16;
    constexpr int NTH = 64 * WM * WN;
    constexpr int CPR = BN * OS / 16;  // 16-byte chunks per row
    // Tile rows per staging pass.  Several passes only for 16-bit outputs
    // and without in-place dequant scale loads (PRE below): the other
    // combinations spilled over the pass loop.
    constexpr int RP0 = stage_rows(BM, PITCH, SB, CPR, NTH);
    constexpr bool MULTI = OS == 2 && !(DEQ && FN * 16 + FM > 40);
    constexpr int RP = (RP0 == BM || MULTI) ? RP0 : 0;
    constexpr bool STAGED = FULL && RP > 0;
    constexpr int NPASS = STAGED ? BM / RP : 1;
    const uint32_t lane = fresh_v(threadIdx.x & 63u);
    wm = fresh_s(__builtin_amdgcn_readfirstlane(wm));  // wave-uniform in both families
    wn = fresh_s(__builtin_amdgcn_readfirstlane(wn));
    const uint32_t l32 = lane & 31u, hi = lane >> 5;
    // slice-M tasks address C by their stacked row; batches and slice-K
    // groups own a C each, strideC apart
    uint8_t* cbase = a.C + ((int64_t)(FORM == FORM_SLICE_M ? 0 : tk.idx) * a.strideC +
                            tk.row0 * a.ldc + (int64_t)tk.n * BN) * OS;
    // dequant row scales: per stacked row (slice-M), per group and row
    // (slice-K), per row (plain)
    const int64_t rs0 = (FORM == FORM_SLICE_K ? (int64_t)tk.idx * a.M : 0) + tk.row0;
    // matmul-add (plain GEMM only, so the task's row0 is its first row of X)
    const uint8_t* xbase = ADD ? a.X + (tk.row0 * a.ldx + (int64_t)tk.n * BN) * OS : nullptr;
    // Dequant scales are gathered before the first store when they fit in a
    // few registers: a store counts in vmcnt too, so a scale load issued
    // after one waits for it (the compiler cannot hoist the loads itself,
    // since C may alias the scales).  Wide wave tiles load them in place.
    constexpr bool PRE = DEQ && FN * 16 + FM <= 40;
    float rsv[FM];
    float csv[FN][4][4];
    const float* csb = nullptr;
    if constexpr (DEQ)
      csb = a.col_scale + (int64_t)(FORM == FORM_DENSE ? 0 : tk.idx) * a.N + (int64_t)tk.n * BN;
    if constexpr (PRE) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint32_t ml = wm * TM + i * 32 + l32;
        rsv[i] = (FULL || ml < tk.rows_valid) ? a.row_scale[rs0 + ml] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t nl = wn * TN + j * 32 + 8 * g + 4 * hi;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            csv[j][g][r] = (FULL || nl + r < tk.nAct) ? csb[nl + r] : 0.0f;
        }
    }
    hook();
    // One pass: the wave's rows (those of staging pass `pass` when staged).
    auto emit = [&](uint32_t pass) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (STAGED)
          if ((wm * TM + i * 32) / RP != pass) continue;  // wave-uniform
        const uint32_t ml = wm * TM + i * 32 + l32;
        if (!FULL && ml >= tk.rows_valid) continue;
        uint8_t* crow = cbase + (int64_t)ml * a.ldc * OS;
        const uint8_t* xrow = ADD ? xbase + (int64_t)ml * a.ldx * OS : nullptr;
        float rs = 1.0f;
        if constexpr (PRE)
          rs = rsv[i];
        else if constexpr (DEQ)
          rs = a.row_scale[rs0 + ml];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint32_t nl = wn * TN + j * 32 + 8 * g + 4 * hi;  // column inside the tile
            if (!FULL && nl >= tk.nAct) continue;
            const bool whole = FULL || nl + 4 <= tk.nAct;
            float f[4];
            int32_t iv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const auto x = acc[i][j][4 * g + r];
              if constexpr (T::IS_INT) {
                iv[r] = x;
                f[r] = (float)iv[r];
              } else {
                f[r] = x;
                iv[r] = 0;
              }
            }
            if constexpr (PRE) {
#pragma unroll
              for (int r = 0; r < 4; ++r) f[r] = (f[r] * rs) * csv[j][g][r];
            } else if constexpr (DEQ) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float c = (whole || nl + r < tk.nAct) ? csb[nl + r] : 0.0f;
                f[r] = (f[r] * rs) * c;
              }
            }
            if constexpr (ADD) add_x<OUT>(f, iv, xrow + nl * OS, whole, tk.nAct - nl);
            if constexpr (FORM == FORM_SLICE_K) {
              if (tk.poison) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  f[r] = __builtin_nanf("");
                  iv[r] = (int32_t)0x80000000u;
                }
              }
            }
            uint8_t* p = crow + nl * OS;
            if constexpr (STAGED) {
              lds_byte_t* q = stage + (ml - pass * RP) * PITCH + nl * OS;
              if constexpr (OS == 2)
                *(__attribute__((address_space(3))) u32x2_t*)q =
                    u32x2_t{pack2<OUT>(f[0], f[1]), pack2<OUT>(f[2], f[3])};
              else if constexpr (OUT == OUT_F32)
                *(__attribute__((address_space(3))) f32x4_t*)q = f32x4_t{f[0], f[1], f[2], f[3]};
              else
                *(__attribute__((address_space(3))) i32x4_t*)q = i32x4_t{iv[0], iv[1], iv[2], iv[3]};
              (void)p;
            } else if (whole) {
              if constexpr (OS == 2)
                *(u32x2_t*)__builtin_assume_aligned(p, 8) =
                    u32x2_t{pack2<OUT>(f[0], f[1]), pack2<OUT>(f[2], f[3])};
              else if constexpr (OUT == OUT_F32)
                *(f32x4_t*)__builtin_assume_aligned(p, 16) = f32x4_t{f[0], f[1], f[2], f[3]};
              else
                *(i32x4_t*)__builtin_assume_aligned(p, 16) = i32x4_t{iv[0], iv[1], iv[2], iv[3]};
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                if (nl + r >= tk.nAct) continue;
                if constexpr (OS == 2)
                  ((uint16_t*)p)[r] = (uint16_t)pack2<OUT>(f[r], 0.0f);
                else if constexpr (OUT == OUT_F32)
                  ((float*)p)[r] = f[r];
                else
                  ((int32_t*)p)[r] = iv[r];
              }
            }
          }
      }
    };
    if constexpr (STAGED) {
      // The tile goes through the L2 to memory (device-scope cache policy):
      // its lines do not stay dirty in the XCD's L2, where they would take
      // the place of A and B panel lines and wait to be written back when
      // the kernel ends.  The buffer offsets are 31-bit: the host runs
      // these kernels only where a tile's rows of C span less than 2 GiB.
      const __amdgpu_buffer_rsrc_t crsrc =
          __builtin_amdgcn_make_buffer_rsrc(cbase, (short)0, (int)0x7fffffff, 0x00020000);
      // a loop, not unrolled: each wave writes in the passes that hold its
      // rows, and one copy of the code serves them all
#pragma unroll 1
      for (uint32_t pass = 0; pass < (uint32_t)NPASS; ++pass) {
        emit(pass);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < RP * CPR / NTH; ++i) {
          const uint32_t q = fresh_v(threadIdx.x) + (uint32_t)i * NTH;
          const uint32_t row = q / CPR, c = q % CPR;
          const u32x4_t v = *(const lds_u32x4_out_t*)(stage + row * PITCH + c * 16);
          __builtin_amdgcn_raw_buffer_store_b128(
              v, crsrc, (pass * RP + row) * (uint32_t)a.ldc * OS + c * 16, 0, kDeviceScope);
        }
        // the next pass (or the next task's prologue) refills the buffer
        __syncthreads();
      }
    } else {
      emit(0);
    }
  }

  template <bool DEQ, bool FULL, int SB, bool ADD = false, class Hook = NoHook>
  __device__ static __forceinline__ void store_kind(const GemmArgs& a, const Task& tk,
                                                    const Acc (&acc)[FM][FN], uint32_t wm,
                                                    uint32_t wn, lds_byte_t* stage,
                                                    const Hook& hook = Hook()) {
    if (a.cdtype == OUT_F16)
      store_as<OUT_F16, DEQ, FULL, SB, ADD>(a, tk, acc, wm, wn, stage, hook);
    else if (a.cdtype == OUT_BF16)
      store_as<OUT_BF16, DEQ, FULL, SB, ADD>(a, tk, acc, wm, wn, stage, hook);
    else if (a.cdtype == OUT_F32)
      store_as<OUT_F32, DEQ, FULL, SB, ADD>(a, tk, acc, wm, wn, stage, hook);
    else if constexpr (T::IS_INT && !DEQ)
      store_as<OUT_I32, false, FULL, SB, ADD>(a, tk, acc, wm, wn, stage, hook);
    else
      hook();
  }

  // matmul-add: the addend's four values at p (of the output kind OUT) are
  // added to the lane's values before they are rounded; `whole`: all four
  // columns are inside the problem, else only the first `left` are read.
  template <int OUT>
  __device__ static __forceinline__ void add_x(float (&f)[4], int32_t (&iv)[4],
                                               const uint8_t* p, bool whole, uint32_t left) {
    if constexpr (OUT == OUT_F16 || OUT == OUT_BF16) {
      uint16_t h[4] = {0, 0, 0, 0};
      if (whole) {
        const u32x2_t v = *(const u32x2_t*)__builtin_assume_aligned(p, 8);
        h[0] = (uint16_t)v[0];
        h[1] = (uint16_t)(v[0] >> 16);
        h[2] = (uint16_t)v[1];
        h[3] = (uint16_t)(v[1] >> 16);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if ((uint32_t)r < left) h[r] = ((const uint16_t*)p)[r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (OUT == OUT_F16)
          f[r] += (float)__builtin_bit_cast(_Float16, h[r]);
        else
          f[r] += __builtin_bit_cast(float, (uint32_t)h[r] << 16);
      }
    } else {
      uint32_t w[4] = {0, 0, 0, 0};
      if (whole) {
        const u32x4_t v = *(const u32x4_t*)__builtin_assume_aligned(p, 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t e = v[r];  // copy the element out before using it
          w[r] = e;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if ((uint32_t)r < left) w[r] = ((const uint32_t*)p)[r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (OUT == OUT_I32)
          iv[r] = (int32_t)((uint32_t)iv[r] + w[r]);  // int32 addition, wrapping
        else
          f[r] += __builtin_bit_cast(float, w[r]);
      }
    }
  }

  // The wave's whole output: one dispatch per task on the output kind, the
  // dequant and whether the tile is whole, then straight-line stores.
  // Dequantised outputs exist for int8 operands only.  SB, stage: LDS that
  // whole tiles may be staged through (see store_as; SB = 0: none).
  // ADD: the matmul-add instances, whose epilogue adds a.X (never with the
  // dequant, which the host rules out for them).
  template <int SB = 0, bool ADD = false, class Hook = NoHook>
  __device__ static __forceinline__ void store_tile(const GemmArgs& a, const Task& tk,
                                                    const Acc (&acc)[FM][FN], uint32_t wm,
                                                    uint32_t wn, lds_byte_t* stage = nullptr,
                                                    const Hook& hook = Hook()) {
    const bool full = tk.rows_valid >= (uint32_t)BM && tk.nAct >= (uint32_t)BN;
    if constexpr (T::IS_INT && !ADD) {
      if (a.row_scale != nullptr) {
        if (full)
          store_kind<true, true, SB, false, Hook>(a, tk, acc, wm, wn, stage, hook);
        else
          store_kind<true, false, SB, false, Hook>(a, tk, acc, wm, wn, stage, hook);
        return;
      }
    }
    if (full)
      store_kind<false, true, SB, ADD, Hook>(a, tk, acc, wm, wn, stage, hook);
    else
      store_kind<false, false, SB, ADD, Hook>(a, tk, acc, wm, wn, stage, hook);
  }

};

template <int AB, int BM, int BN, int WM, int WN, int FORM>
struct GemmKernel {
  using T = Traits<AB>;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 sub-tiles per wave
  static constexpr int CE = 16 / T::ES;             // elements per 16-byte chunk
  static constexpr int KSTEPS = T::BK / T::MFMA_K;  // MFMA steps per stage
  static constexpr int A_CHUNKS = BM * 8;           // 16-byte chunks of an A stage
  static constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
  static constexpr int NBC = BN / CE;               // 16-byte chunks across a B row
  static constexpr int KBLK = T::BK / T::KBR;       // B blocks along K (= 16)
  static constexpr int B_BLOCKS = KBLK * NBC;
  static constexpr int B_PER_T = (B_BLOCKS + NT - 1) / NT;
  static constexpr int KB_LO = T::ES == 2 ? 1 : 2;  // K-block bits varied fastest across lanes
  static constexpr int STAGE_BYTES = (BM + BN) * kRowBytes;
  static constexpr int SCALE_BYTES = T::SCALED ? (BM + BN) * 4 : 0;
  static constexpr int LDS_BYTES = 2 * (STAGE_BYTES + SCALE_BYTES);
  using Acc = typename std::conditional<T::IS_INT, i32x16_t, f32x16_t>::type;
  using Frag = typename std::conditional<T::FRAG_DW == 8, i32x8_t, u32x4_t>::type;
  using Epi = Epilogue<AB, BM, BN, WM, WN, FORM>;
  static constexpr bool GROUPED = FORM == FORM_SLICE_M;

  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(T::BK * T::ES == kRowBytes, "one stage = one 128-byte row");
  static_assert(KBLK == 16, "16 B-blocks of 8 bytes fill a 128-byte row");
  static_assert(!T::SCALED || (BM <= NT && BN <= NT), "one thread per scale row / column");

  // Registers holding one stage on its way from global memory to LDS.
  struct Stage {
    u32x4_t a[A_PER_T];
    u32x4_t b[B_PER_T][T::KBR];
    uint32_t sa, sb;  // MX: 4 scale bytes (one per 32-wide K block) of one A row / B column
  };

  // a_al: A's 16-byte chunks of this task start on 16-byte boundaries (a
  // slice-K group may start anywhere).
  __device__ static void load_stage(Stage& st, const GemmArgs& a, const uint8_t* Ab,
                                    const uint8_t* Bb, const Task& tk, uint32_t kb0,
                                    uint32_t kend, const uint8_t* sab, const uint8_t* sbb,
                                    bool a_al) {
    const uint32_t tid = threadIdx.x;
    const bool k_full = kb0 + T::BK <= kend;
    // Interior stages (the common case) issue every 16-byte load back to
    // back with no predicate; only stages that touch a tail take the masked
    // path.  Both conditions are uniform across the workgroup.
    if (k_full && a_al && tk.rows_valid == (uint32_t)BM) {
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) {
        const uint32_t q = tid + i * NT;
        if (A_CHUNKS % NT == 0 || q < (uint32_t)A_CHUNKS) {
          const uint32_t r = q >> 3, c = q & 7u;
          st.a[i] = *reinterpret_cast<const u32x4_t*>(Ab + ((int64_t)r * a.lda + kb0 + c * CE) * T::ES);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) {
        const uint32_t q = tid + i * NT;
        st.a[i] = u32x4_t{0u, 0u, 0u, 0u};
        if (A_CHUNKS % NT == 0 || q < (uint32_t)A_CHUNKS) {
          const uint32_t r = q >> 3, c = q & 7u;
          const uint32_t gk = kb0 + c * CE;
          if (r < tk.rows_valid && gk < kend) {
            const int valid = (int)((kend - gk) < (uint32_t)CE ? (kend - gk) : CE) * T::ES;
            st.a[i] = load16(Ab + ((int64_t)r * a.lda + gk) * T::ES, valid);
          }
        }
      }
    }
    if (k_full && tk.n * BN + BN <= a.N) {
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) {
        const uint32_t q = tid + i * NT;
        if (!(B_BLOCKS % NT == 0 || q < (uint32_t)B_BLOCKS)) continue;
        const uint32_t kb_lo = q & ((1u << KB_LO) - 1u);
        const uint32_t rest = q >> KB_LO;
        const uint32_t nb = rest % NBC;
        const uint32_t kb = (rest / NBC) * (1u << KB_LO) + kb_lo;
        const uint8_t* p = Bb + ((int64_t)(kb0 + kb * T::KBR) * a.ldb + tk.n * BN + nb * CE) * T::ES;
#pragma unroll
        for (int j = 0; j < T::KBR; ++j)
          st.b[i][j] = *reinterpret_cast<const u32x4_t*>(p + (int64_t)j * a.ldb * T::ES);
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) {
        const uint32_t q = tid + i * NT;
        const uint32_t kb_lo = q & ((1u << KB_LO) - 1u);
        const uint32_t rest = q >> KB_LO;
        const uint32_t nb = rest % NBC;
        const uint32_t kb = (rest / NBC) * (1u << KB_LO) + kb_lo;
        const uint32_t ncol = tk.n * BN + nb * CE;
        const bool live = (B_BLOCKS % NT == 0 || q < (uint32_t)B_BLOCKS);
        const int nvalid =
            ncol < a.N ? (int)((a.N - ncol) < (uint32_t)CE ? (a.N - ncol) : CE) * T::ES : 0;
#pragma unroll
        for (int j = 0; j < T::KBR; ++j) {
          const uint32_t gk = kb0 + kb * T::KBR + j;
          st.b[i][j] = u32x4_t{0u, 0u, 0u, 0u};
          if (live && gk < kend && nvalid > 0)
            st.b[i][j] = load16(Bb + ((int64_t)gk * a.ldb + ncol) * T::ES, nvalid);
        }
      }
    }
    if constexpr (T::SCALED) {
      // A scales: one row per thread, 4 K blocks; B scales: one column per thread.
      st.sa = 0x7f7f7f7fu;
      st.sb = 0x7f7f7f7fu;
      if (sab) {
        uint32_t va = 0, vb = 0;
        for (int e = 0; e < 4; ++e) {
          const uint32_t kblock = kb0 / 32 + e;
          const bool kin = kblock * 32 < kend;
          uint32_t x = 0x7f, y = 0x7f;
          if (tid < (uint32_t)BM && kin && tid < tk.rows_valid)
            x = sab[(int64_t)tid * a.ldsa + kblock];
          if (tid < (uint32_t)BN && kin && tk.n * BN + tid < a.N)
            y = sbb[(int64_t)kblock * a.ldsb + tk.n * BN + tid];
          va |= x << (8 * e);
          vb |= y << (8 * e);
        }
        st.sa = va;
        st.sb = vb;
      }
    }
  }

  __device__ static void store_stage(const Stage& st, uint8_t* lds) {
    const uint32_t tid = threadIdx.x;
    uint8_t* la = lds;
    uint8_t* lb = lds + BM * kRowBytes;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const uint32_t q = tid + i * NT;
      if (A_CHUNKS % NT == 0 || q < (uint32_t)A_CHUNKS)
        *reinterpret_cast<u32x4_t*>(la + lds_off(q >> 3, q & 7u)) = st.a[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const uint32_t q = tid + i * NT;
      if (!(B_BLOCKS % NT == 0 || q < (uint32_t)B_BLOCKS)) continue;
      const uint32_t kb_lo = q & ((1u << KB_LO) - 1u);
      const uint32_t rest = q >> KB_LO;
      const uint32_t nb = rest % NBC;
      const uint32_t kb = (rest / NBC) * (1u << KB_LO) + kb_lo;
      // transpose KBR rows x 16 bytes into (16 / KBR*... ) columns of 8 bytes
      if constexpr (T::ES == 2) {
        // 4 K-rows x 8 halves -> 8 columns x 4 halves
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t sel = h ? 0x07060302u : 0x05040100u;
            const uint32_t d0 = __builtin_amdgcn_perm(st.b[i][1][w], st.b[i][0][w], sel);
            const uint32_t d1 = __builtin_amdgcn_perm(st.b[i][3][w], st.b[i][2][w], sel);
            const uint32_t n = nb * 8 + w * 2 + h;
            *reinterpret_cast<u32x2_t*>(lb + lds_off(n, kb >> 1) + (kb & 1u) * 8) = u32x2_t{d0, d1};
          }
        }
      } else {
        // 8 K-rows x 16 bytes -> 16 columns x 8 bytes
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t col[2][4];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const uint32_t r0 = st.b[i][4 * half + 0][w], r1 = st.b[i][4 * half + 1][w];
            const uint32_t r2 = st.b[i][4 * half + 2][w], r3 = st.b[i][4 * half + 3][w];
            const uint32_t p01l = __builtin_amdgcn_perm(r1, r0, 0x05010400u);
            const uint32_t p01h = __builtin_amdgcn_perm(r1, r0, 0x07030602u);
            const uint32_t p23l = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
            const uint32_t p23h = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
            col[half][0] = __builtin_amdgcn_perm(p23l, p01l, 0x05040100u);
            col[half][1] = __builtin_amdgcn_perm(p23l, p01l, 0x07060302u);
            col[half][2] = __builtin_amdgcn_perm(p23h, p01h, 0x05040100u);
            col[half][3] = __builtin_amdgcn_perm(p23h, p01h, 0x07060302u);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t n = nb * 16 + w * 4 + e;
            *reinterpret_cast<u32x2_t*>(lb + lds_off(n, kb >> 1) + (kb & 1u) * 8) =
                u32x2_t{col[0][e], col[1][e]};
          }
        }
      }
    }
    if constexpr (T::SCALED) {
      uint32_t* ls = reinterpret_cast<uint32_t*>(lds + STAGE_BYTES);
      if (tid < (uint32_t)BM) ls[tid] = st.sa;
      if (tid < (uint32_t)BN) ls[BM + tid] = st.sb;
    }
  }

  // MFMAs of one stage held in LDS.  Operand lanes: 16-bit and int8 steps
  // take 16 consecutive bytes of K per lane (lane group hi = lane / 32 holds
  // the upper half of the step).  The scaled fp8 step of 64 K values takes
  // two 16-byte pieces per lane, K [16hi, 16hi+16) and [32+16hi, 48+16hi)
  // of the step, and the lane of group hi supplies the E8M0 scale of the
  // 32-wide block hi of its row (column) -- the operand layout of the
  // gfx950 scaled MFMA, established by an on-device lane probe.
  __device__ static void compute_stage(Acc (&acc)[FM][FN], const uint8_t* lds, uint32_t wm,
                                       uint32_t wn) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t l32 = lane & 31u, hi = lane >> 5;
    const uint8_t* la = lds;
    const uint8_t* lb = lds + BM * kRowBytes;
    const uint32_t* ls = reinterpret_cast<const uint32_t*>(lds + STAGE_BYTES);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      Frag fa[FM], fb[FN];
      uint32_t sca[FM], scb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint32_t row = wm * TM + i * 32 + l32;
        if constexpr (T::FRAG_DW == 4) {
          fa[i] = *reinterpret_cast<const u32x4_t*>(la + lds_off(row, 2 * kk + hi));
        } else {
          const u32x4_t x = *reinterpret_cast<const u32x4_t*>(la + lds_off(row, 4 * kk + hi));
          const u32x4_t y = *reinterpret_cast<const u32x4_t*>(la + lds_off(row, 4 * kk + 2 + hi));
          fa[i] = i32x8_t{(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                          (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
        }
        sca[i] = T::SCALED ? (ls[row] >> (8 * (2 * kk + hi))) & 0xffu : 0x7fu;
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint32_t row = wn * TN + j * 32 + l32;
        if constexpr (T::FRAG_DW == 4) {
          fb[j] = *reinterpret_cast<const u32x4_t*>(lb + lds_off(row, 2 * kk + hi));
        } else {
          const u32x4_t x = *reinterpret_cast<const u32x4_t*>(lb + lds_off(row, 4 * kk + hi));
          const u32x4_t y = *reinterpret_cast<const u32x4_t*>(lb + lds_off(row, 4 * kk + 2 + hi));
          fb[j] = i32x8_t{(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                          (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
        }
        scb[j] = T::SCALED ? (ls[BM + row] >> (8 * (2 * kk + hi))) & 0xffu : 0x7fu;
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mfma32<AB>(acc[i][j], fb[j], fa[i], scb[j], sca[i]);
    }
  }

  __device__ __attribute__((always_inline)) static void run(const GemmArgs& a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
    GroupTable* gt = nullptr;
    uint32_t T_tiles = a.tiles;
    if constexpr (FORM != FORM_DENSE) {
      __shared__ GroupTable gtab;
      gt = &gtab;
      if constexpr (FORM == FORM_SLICE_M) {
        build_group_table(gtab, a, BM, (a.N + BN - 1) / BN);
        T_tiles = gtab.first_task[a.G];
      } else {
        build_k_table(gtab, a);
      }
    }
    const uint32_t units = T_tiles * a.split;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t wm = wave / WN, wn = wave % WN;
    const uint32_t lane = threadIdx.x & 63u;

    for (uint32_t u = logical_wg(a.remap, a.grid); u < units; u += a.grid) {
      const uint32_t s = u / T_tiles;       // K slice (like GetBatchIdx over slices)
      uint32_t t = u - s * T_tiles;         // task
      if constexpr (FORM == FORM_SLICE_K) t = slicek_task(a, gt, t);
      const Task tk = decode_task(a, t, BM, BN, GROUPED ? gt : nullptr);
      // the task's K range: all of K, or its slice-K group's
      uint32_t kq = 0, kg = a.K, ks = a.kslice;
      if constexpr (FORM == FORM_SLICE_K) {
        kq = (uint32_t)gt->first_row[tk.idx];
        kg = (uint32_t)gt->first_row[tk.idx + 1] - kq;
        ks = group_kslice(kg, a.split, T::BK);
      }
      const KRange kr = slice_range(kq, kg, ks, s);
      const uint32_t k0 = kr.k0, k1 = kr.k1;
      const uint32_t klen = k0 < k1 ? k1 - k0 : 0u;
      const uint32_t nk = (klen + T::BK - 1) / T::BK;
      const bool a_al = FORM != FORM_SLICE_K || (kq * T::ES) % 16u == 0;

      const int64_t bidx = FORM == FORM_DENSE ? tk.idx : 0;
      const uint8_t* Ab = a.A + (bidx * a.strideA + tk.row0 * a.lda) * T::ES;
      const uint8_t* Bb = a.B + ((int64_t)(FORM == FORM_SLICE_K ? 0 : tk.idx) * a.strideB) * T::ES;
      const uint8_t* sab = a.sa ? a.sa + tk.row0 * a.ldsa : nullptr;
      const uint8_t* sbb = a.sb;

      Acc acc[FM][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

      if (nk > 0) {
        Stage st;
        load_stage(st, a, Ab, Bb, tk, k0, k1, sab, sbb, a_al);
        store_stage(st, lds);
        __syncthreads();
        for (uint32_t kt = 0; kt < nk; ++kt) {
          const uint8_t* cur = lds + (kt & 1u) * (STAGE_BYTES + SCALE_BYTES);
          uint8_t* nxt = lds + ((kt + 1) & 1u) * (STAGE_BYTES + SCALE_BYTES);
          const bool more = kt + 1 < nk;
          if (more) load_stage(st, a, Ab, Bb, tk, k0 + (kt + 1) * T::BK, k1, sab, sbb, a_al);
          compute_stage(acc, cur, wm, wn);
          if (more) store_stage(st, nxt);
          __syncthreads();
        }
      }

      if (!Epi::fixup(a, acc, s, t)) continue;
      Epi::store_tile(a, tk, acc, wm, wn);
    }
  }
};

template <int AB, int BM, int BN, int WM, int WN, int FORM>
__global__ void __launch_bounds__(64 * WM * WN) gemm_kernel(GemmArgs a) {
  GemmKernel<AB, BM, BN, WM, WN, FORM>::run(a);
}

// Map dump: the same scheduler, persistent loop and renumbering as the GEMM
// kernels, one wave per workgroup, one record of 8 words per task.
template <bool GROUPED>
__global__ void __launch_bounds__(64) tile_map_kernel(GemmArgs a, uint32_t BM, uint32_t BN) {
  GroupTable* gt = nullptr;
  uint32_t T_tiles = a.tiles;
  if constexpr (GROUPED) {
    __shared__ GroupTable gtab;
    gt = &gtab;
    build_group_table(gtab, a, BM, (a.N + BN - 1) / BN);
    T_tiles = gtab.first_task[a.G];
  }
  for (uint32_t t = logical_wg(a.remap, a.grid); t < T_tiles; t += a.grid) {
    const Task tk = decode_task(a, t, BM, BN, gt);
    if (threadIdx.x == 0) {
      uint32_t* o = a.map_out + (size_t)t * 8;
      o[0] = tk.idx;
      o[1] = tk.m;
      o[2] = tk.n;
      o[3] = tk.mAct;
      o[4] = tk.nAct;
      o[5] = GROUPED ? (uint32_t)tk.row0 : 0u;
      o[6] = xcc_id();
      o[7] = blockIdx.x;
    }
  }
}

}  // namespace bst
