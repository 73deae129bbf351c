// bst.hip -- host side of the C ABI declared in include/bst.h: argument
// validation (pure host code, no HIP call before it passes), kernel-instance
// selection, schedule resolution (default tiles, automatic K split,
// persistent grid size) and launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <unordered_map>

#include "bst.h"
#include "bst_instances.hpp"

using namespace bst;

namespace {

thread_local char g_err[512] = "";

// Measurement hook (bst_set_clock_record): device buffer and workgroup count.
uint64_t* g_clock = nullptr;
uint32_t g_clock_n = 0;

#ifdef BST_TRACE
uint64_t* g_trace = nullptr;  // device buffer for the K-loop cycle accounting
#endif

bst_status fail(bst_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

int kernel_ab(bst_dtype ab) { return (int)ab; }

const Instance* find_instance(bst_dtype ab, uint32_t bm, uint32_t bn, int form, bool dma,
                              bool add = false, int wgs = 1) {
  const InstanceList lists[] = {instances_f16(), instances_bf16(), instances_i8(),
                                instances_fp8(), instances_mxfp8(), instances_slicek()};
  for (const InstanceList& l : lists)
    for (int i = 0; i < l.count; ++i) {
      const Instance& in = l.begin[i];
      if (in.ab == kernel_ab(ab) && (uint32_t)in.bm == bm && (uint32_t)in.bn == bn &&
          in.form == form && in.dma == dma && in.add == add && in.wgs == wgs)
        return &in;
    }
  return nullptr;
}

size_t elem_size(bst_dtype t) {
  switch (t) {
    case BST_F16:
    case BST_BF16: return 2;
    case BST_E4M3:
    case BST_MXE4M3:
    case BST_I8: return 1;
    case BST_I32:
    case BST_F32: return 4;
    default: return 0;  // not a dtype
  }
}

bool is_ab(bst_dtype t) {
  return t == BST_F16 || t == BST_BF16 || t == BST_E4M3 || t == BST_MXE4M3 || t == BST_I8;
}

bool out_ok(bst_dtype ab, bst_dtype c) {
  if (c == BST_F16 || c == BST_BF16 || c == BST_F32) return true;
  return c == BST_I32 && ab == BST_I8;
}

// --------------------------------------------------------- device info ----
struct DevInfo {
  int cus = 0;
};

std::mutex g_mu;
std::unordered_map<int, DevInfo> g_dev;
std::unordered_map<uint64_t, int> g_occ;

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_dev.find(dev);
  if (it != g_dev.end()) return it->second.cus;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  g_dev[dev].cus = cus;
  return cus;
}

int occupancy(const Instance* in) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  const uint64_t key = ((uint64_t)(uintptr_t)in) ^ ((uint64_t)dev << 56);
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_occ.find(key);
  if (it != g_occ.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, in->fn, in->threads, 0) != hipSuccess ||
      n <= 0)
    n = 1;
  (void)hipGetLastError();
  g_occ[key] = n;
  return n;
}

// ------------------------------------------------------------ planning ----
constexpr int64_t kMaxU32 = 0x7fffffffLL;
// Workspace layout: a fixed counter area that partial tiles never
// overwrite -- one arrival counter per tile, then the dynamic allocation's
// eight queue counters and exit count -- followed by the fp32 / int32
// partial tiles.  The counter area must be zero before the first call;
// every call leaves the counters it used at zero, whatever its tile count,
// split or allocation.
constexpr uint32_t kMaxSplitTiles = 16384;
constexpr size_t kQueueOffset = kMaxSplitTiles * 4;
constexpr size_t kCounterBytes = kQueueOffset + 8192;  // 57 counters, one per 128-byte line

struct Plan {
  const Instance* inst = nullptr;
  uint32_t bm = 0, bn = 0, bk = 0;
  uint32_t off = 1, dir = 0, remap = 0, shuffle = 0, dynamic = 0, preload = 0;
  uint32_t split = 1, kslice = 0;
  uint64_t tile_cap = 0;  // tiles (upper bound for grouped)
  uint32_t grid = 0;
  size_t ws_bytes = 0;
  size_t part_bytes = 0;
};

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Resolves the schedule.  form FORM_DENSE: plain / batched (count = batch),
// FORM_SLICE_M: grouped slice-M (count = G, M = total_m), FORM_SLICE_K:
// grouped slice-K (count = G, K = total_k).  Validates the schedule fields
// and the sizes that bound the task count; pointer checks are the callers'.
// Layout facts that decide whether the LDS-DMA family can run a call.
struct Layout {
  int64_t lda = 0, ldb = 0;
  const void* sa = nullptr;
  const void* sb = nullptr;
  int64_t ldc_bytes = 0;  // C's row pitch in bytes (0: not known, the query calls)
};

bool dma_fits(bst_dtype ab, int64_t N, int64_t K, uint32_t bm, uint32_t bk, const Layout& L) {
  const int64_t es = (int64_t)elem_size(ab), ce = 16 / es;
  if (K % ce != 0 || N % ce != 0) return false;       // no 16-byte chunk straddles K or N
  // 31-bit panel offsets: lane offset (row / K row inside a stage) plus the
  // stage's scalar offset (K position) stay below 2^31
  if ((int64_t)bm * L.lda * es + K * es >= (1LL << 31)) return false;
  if ((K + bk) * L.ldb * es >= (1LL << 31)) return false;
  // the staged epilogue addresses a C tile with 31-bit offsets too
  if ((int64_t)bm * L.ldc_bytes >= (1LL << 31)) return false;
  if (ab == BST_MXE4M3 && (K / 32 + 4) * N >= (1LL << 31)) return false;  // B scales [K/32][N]
  if (ab == BST_MXE4M3 && (K % 128 != 0 || ((uintptr_t)L.sa & 3u) || ((uintptr_t)L.sb & 3u)))
    return false;
  return true;
}

bst_status make_plan(int form, bst_dtype ab, int64_t count, int64_t M, int64_t N, int64_t K,
                     const bst_sched* s, bool need_device, Plan& p, const Layout* L = nullptr,
                     bool add = false) {
  const bool grouped = form != FORM_DENSE;
  if (!is_ab(ab)) return fail(BST_E_INVAL, "unknown operand dtype %d", (int)ab);
  if (count < 0 || M < 0 || N < 0 || K < 0)
    return fail(BST_E_INVAL, "negative size (count %lld M %lld N %lld K %lld)", (long long)count,
                (long long)M, (long long)N, (long long)K);
  if (M > kMaxU32 || N > kMaxU32 || K > kMaxU32 || count > kMaxU32)
    return fail(BST_E_INVAL, "size above 2^31-1");
  if (grouped && (count < 1 || count > kMaxGroups))
    return fail(BST_E_INVAL, "group count %lld outside [1, %d]", (long long)count, kMaxGroups);
  if (ab == BST_MXE4M3 && K % 32 != 0)
    return fail(BST_E_INVAL, "MX operands need K %% 32 == 0 (K = %lld)", (long long)K);
  if (ab == BST_I8 && K > 131071)
    return fail(BST_E_INVAL, "int8 K = %lld could overflow the int32 accumulator (max 131071)",
                (long long)K);
  bst_sched d{};
  if (s) d = *s;
  if (d.swizzle_offset == 0 && s) return fail(BST_E_INVAL, "swizzle_offset must be >= 1");
  if (!s) d.swizzle_offset = 1;
  if (d.swizzle_direction > 2)
    return fail(BST_E_INVAL, "swizzle_direction %u not in {0 Zn, 1 Nz, 2 raster}",
                d.swizzle_direction);
  if (d.xcd_remap > 1) return fail(BST_E_INVAL, "xcd_remap must be 0 or 1");
  if (d.split_k > 64) return fail(BST_E_INVAL, "split_k %u above 64", d.split_k);
  if (d.tile_m == 0 && d.tile_n == 0) {
    d.tile_m = 128;
    d.tile_n = 128;
  }
  if (d.path > 3)
    return fail(BST_E_INVAL, "path %u not in {0 auto, 1 register, 2 dma, 3 dma pair}", d.path);
  if (d.shuffle_k > 1) return fail(BST_E_INVAL, "shuffle_k must be 0 or 1");
  if (d.dynamic > 1) return fail(BST_E_INVAL, "dynamic must be 0 or 1");
  if (d.preload > 1) return fail(BST_E_INVAL, "preload must be 0 or 1");
  // matmul-add runs only the LDS-DMA instances built with the addend epilogue
  const Instance* reg = add ? nullptr : find_instance(ab, d.tile_m, d.tile_n, form, false);
  const Instance* dma = find_instance(ab, d.tile_m, d.tile_n, form, true, add);
  const Instance* pair = add ? nullptr : find_instance(ab, d.tile_m, d.tile_n, form, true, false, 2);
  if (!reg && !dma && !pair)
    return fail(BST_E_UNSUPPORTED, "no %s kernel for dtype %d with tile %ux%u",
                add ? "matmul-add" : form == FORM_SLICE_M ? "grouped slice-M"
                : form == FORM_SLICE_K ? "grouped slice-K" : "plain", (int)ab, d.tile_m,
                d.tile_n);
  const Layout lay = L ? *L : Layout{K, N, nullptr, nullptr};
  // slice-K: the kernels check each group's chunk alignment on the device,
  // so the total K need not be whole chunks
  const int64_t ce = 16 / (int64_t)elem_size(ab);
  const int64_t kfit = form == FORM_SLICE_K ? (K + ce - 1) / ce * ce : K;
  const Instance* any_dma = dma ? dma : pair;  // both run the same stage depth (bk)
  const bool fits = any_dma && dma_fits(ab, N, kfit, d.tile_m, (uint32_t)any_dma->bk, lay);
  if ((d.path == 2 || d.path == 3) && !fits)
    return fail(BST_E_UNSUPPORTED, "the LDS-DMA kernels need K and N in whole 16-byte chunks "
                "(and K %% 128 == 0 for MX); use path 0 or 1");
  if (d.path == 3 && !pair)
    return fail(BST_E_UNSUPPORTED, "no two-workgroup LDS-DMA kernel for dtype %d with tile %ux%u "
                "in this problem form", (int)ab, d.tile_m, d.tile_n);
  // path 0 decides between dma and pair below, once the unit count is known
  p.inst = (d.path == 1 || !fits) ? reg : d.path == 3 ? pair : (dma ? dma : pair);
  if (!p.inst) return fail(BST_E_UNSUPPORTED, "no kernel of the requested family for this tile");
  if (d.tile_k != 0 && d.tile_k != (uint32_t)p.inst->bk)
    return fail(BST_E_UNSUPPORTED, "tile_k %u: this dtype runs tile_k %d", d.tile_k,
                p.inst->bk);
  p.bm = d.tile_m;
  p.bn = d.tile_n;
  p.bk = (uint32_t)p.inst->bk;
  p.off = d.swizzle_offset;
  p.dir = d.swizzle_direction;
  p.remap = d.xcd_remap;
  // ShuffleK, dynamic allocation and preload are LDS-DMA features; the
  // register-staged family runs stages in order over a static stride
  p.shuffle = p.inst->dma ? d.shuffle_k : 0u;
  p.dynamic = p.inst->dma ? d.dynamic : 0u;
  // with dynamic allocation the next task is known only after the epilogue
  p.preload = (p.inst->dma && !p.dynamic) ? d.preload : 0u;
  const int64_t loopsN = cdiv64(N, p.bn);
  const int64_t tiles = form == FORM_SLICE_M ? (cdiv64(M, p.bm) + count) * loopsN
                                             : count * cdiv64(M, p.bm) * loopsN;
  if (tiles > kMaxU32) return fail(BST_E_INVAL, "task count %lld above 2^31-1", (long long)tiles);
  p.tile_cap = (uint64_t)tiles;
  // slice-K groups split their own K on the device (whole stages per slice,
  // empty slices allowed); the automatic split judges by the mean group
  const int64_t nk = cdiv64(form == FORM_SLICE_K ? cdiv64(K, count) : K, p.bk);
  int64_t split = d.split_k;
  const int cus = need_device ? device_cus() : 256;
  if (split == 0) {
    split = 1;
    if (tiles > 0 && tiles < cus && nk >= 8)
      split = std::min<int64_t>({cus / tiles, nk / 4, 16});
    if (split < 1) split = 1;
  }
  if (nk == 0) split = 1;
  int64_t kslice_steps = nk > 0 ? cdiv64(nk, split) : 0;
  // no empty slices (slice-K groups differ in size: the requested split
  // stands, and a short group's surplus slices are empty)
  if (kslice_steps > 0 && form != FORM_SLICE_K) split = cdiv64(nk, kslice_steps);
  p.split = (uint32_t)split;
  p.kslice = (uint32_t)(kslice_steps * p.bk);
  // automatic family: two resident workgroups per CU when the launch has
  // more units than CUs (one workgroup's epilogue and set-up then overlap
  // the other's K loop), one deeper-pipelined workgroup otherwise
  if (d.path == 0 && p.inst->dma && pair && dma)
    p.inst = tiles * split > (int64_t)cus ? pair : dma;
  if (tiles * split > kMaxU32) return fail(BST_E_INVAL, "work-unit count above 2^31-1");
  if (p.split > 1) {
    if (tiles > (int64_t)kMaxSplitTiles)
      return fail(BST_E_INVAL, "split_k > 1 takes at most %u tiles (got %lld)", kMaxSplitTiles,
                  (long long)tiles);
    p.part_bytes = (size_t)p.split * (size_t)tiles * p.bm * p.bn * 4;
    p.ws_bytes = kCounterBytes + p.part_bytes;
  } else if (p.dynamic) {
    p.ws_bytes = kCounterBytes;  // the queue counters
  }
  const int64_t units = tiles * split;
  int64_t grid = d.grid;
  if (grid == 0) grid = (int64_t)cus * (need_device ? occupancy(p.inst) : 1);
  grid = std::max<int64_t>(1, std::min<int64_t>(grid, units > 0 ? units : 1));
  p.grid = (uint32_t)grid;
  return BST_OK;
}

// Problem form of a public `kind` code: 0 plain / batched, 1 grouped
// slice-M, 2 the GEMM of the padding matmul (a plain one), 3 grouped slice-K.
int kind_form(int kind) {
  return kind == 1 ? FORM_SLICE_M : kind == 3 ? FORM_SLICE_K : FORM_DENSE;
}

// The map's launch constants for a problem of M x N per batch / group.
MapConsts map_consts(const Plan& p, int64_t M, int64_t N) {
  return make_map_consts((uint32_t)cdiv64(M, p.bm), (uint32_t)cdiv64(N, p.bn), p.off, p.dir,
                         (uint32_t)p.tile_cap, p.bk ? p.kslice / p.bk : 0u);
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }
bool stride_ok(int64_t ld, size_t es) { return ((uint64_t)ld * es) % 16 == 0; }

bst_status check_ws(const Plan& p, void* ws, size_t ws_bytes) {
  if (p.ws_bytes == 0) return BST_OK;
  if (!ws || ws_bytes < p.ws_bytes)
    return fail(BST_E_WORKSPACE, "split %u%s needs %zu workspace bytes (got %zu)", p.split,
                p.dynamic ? " with dynamic allocation" : "", p.ws_bytes,
                ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(BST_E_ALIGN, "workspace not 16-byte aligned");
  return BST_OK;
}

void fill_ws(GemmArgs& a, const Plan& p, void* ws) {
  a.split = p.split;
  a.kslice = p.kslice;
  a.tile_cap = (uint32_t)p.tile_cap;
  a.ws_part = nullptr;
  a.ws_count = nullptr;
  a.queue = nullptr;
  a.preload = p.preload;
  if (p.split > 1) {
    a.ws_count = reinterpret_cast<uint32_t*>(ws);
    a.ws_part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + kCounterBytes);
  }
  if (p.dynamic) a.queue = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ws) + kQueueOffset);
}

bst_status launch(const Plan& p, const GemmArgs& a, void* stream) {
  GemmArgs b = a;
  b.grid = p.grid;
  b.clock = g_clock;
  b.clock_n = g_clock_n;
  const hipError_t e =
      p.inst->launch(dim3(p.grid), dim3(p.inst->threads), (hipStream_t)stream, b);
  if (e != hipSuccess) return fail(BST_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return BST_OK;
}

// Validation and set-up shared by gemm, gemm_add, gemm_padded and
// batched_gemm: checks every argument, resolves the plan and fills the
// kernel arguments, and enqueues nothing.  On BST_OK, `empty` tells that the
// problem has no output (nothing to launch).
bst_status prepare_dense(bst_dtype ab, bst_dtype c, int64_t batch, int64_t M, int64_t N,
                         int64_t K, const void* A, int64_t lda, int64_t strideA, const void* B,
                         int64_t ldb, int64_t strideB, void* C, int64_t ldc, int64_t strideC,
                         const uint8_t* sa, const uint8_t* sb, const float* rs, const float* cs,
                         const bst_sched* s, void* ws, size_t ws_bytes, const void* X,
                         int64_t ldx, Plan& p, GemmArgs& a, bool& empty) {
  empty = true;
  if (!is_ab(ab)) return fail(BST_E_INVAL, "unknown operand dtype %d", (int)ab);
  if (!out_ok(ab, c)) return fail(BST_E_UNSUPPORTED, "output dtype %d with operands %d", (int)c, (int)ab);
  bst_status st = make_plan(FORM_DENSE, ab, batch, M, N, K, s, false, p, nullptr, X != nullptr);
  if (st != BST_OK) return st;
  if (batch == 0 || M == 0 || N == 0) return BST_OK;
  const size_t es = elem_size(ab), ec = elem_size(c);
  if (!C) return fail(BST_E_INVAL, "C is NULL");
  const bool has_k = K > 0;  // with K == 0, A and B are never read
  if (has_k && (!A || !B)) return fail(BST_E_INVAL, "A or B is NULL");
  if ((has_k && (lda < K || ldb < N)) || ldc < N)
    return fail(BST_E_INVAL, "leading dimension too small (lda %lld K %lld, ldb %lld N %lld, ldc %lld)",
                (long long)lda, (long long)K, (long long)ldb, (long long)N, (long long)ldc);
  if (batch > 1 && (strideA < 0 || strideB < 0 || strideC < 0))
    return fail(BST_E_INVAL, "negative batch stride");
  // batches of C must not overlap (their tasks run concurrently); A and B
  // are only read, so theirs may
  if (batch > 1 && strideC < (M - 1) * ldc + N)
    return fail(BST_E_INVAL, "strideC %lld lets batches of C overlap (need >= %lld)",
                (long long)strideC, (long long)((M - 1) * ldc + N));
  if (ab == BST_MXE4M3 && has_k && (!sa || !sb)) return fail(BST_E_INVAL, "MX scales are NULL");
  if ((rs == nullptr) != (cs == nullptr)) return fail(BST_E_INVAL, "give both dequant scales or neither");
  if (X && (batch != 1 || rs)) return fail(BST_E_INVAL, "the addend is taken by bst_gemm_add only");
  if (X && ldx < N)
    return fail(BST_E_INVAL, "leading dimension too small (ldx %lld N %lld)", (long long)ldx,
                (long long)N);
  if (X && (!aligned16(X) || !stride_ok(ldx, ec)))
    return fail(BST_E_ALIGN, "the addend and its stride must be 16-byte multiples");
  if (!aligned16(C) || !stride_ok(ldc, ec) || (batch > 1 && !stride_ok(strideC, ec)) ||
      (has_k && (!aligned16(A) || !aligned16(B) || !stride_ok(lda, es) || !stride_ok(ldb, es) ||
                 (batch > 1 && (!stride_ok(strideA, es) || !stride_ok(strideB, es))))))
    return fail(BST_E_ALIGN, "pointers and strides must be 16-byte multiples");
  const Layout lay{lda, ldb, sa, sb, ldc * (int64_t)ec};
  st = make_plan(FORM_DENSE, ab, batch, M, N, K, s, true, p, &lay, X != nullptr);
  if (st != BST_OK) return st;
  st = check_ws(p, ws, ws_bytes);
  if (st != BST_OK) return st;

  a = GemmArgs{};
#ifdef BST_TRACE
  a.trace = g_trace;
#endif
  a.A = static_cast<const uint8_t*>(A);
  a.B = static_cast<const uint8_t*>(B);
  a.C = static_cast<uint8_t*>(C);
  a.X = static_cast<const uint8_t*>(X);
  a.ldx = ldx;
  a.lda = lda; a.ldb = ldb; a.ldc = ldc;
  a.strideA = batch > 1 ? strideA : 0;
  a.strideB = batch > 1 ? strideB : 0;
  a.strideC = batch > 1 ? strideC : 0;
  a.sa = ab == BST_MXE4M3 ? sa : nullptr;
  a.sb = ab == BST_MXE4M3 ? sb : nullptr;
  a.ldsa = K / 32;
  a.ldsb = N;
  a.row_scale = rs;
  a.col_scale = cs;
  a.M = (uint32_t)M; a.N = (uint32_t)N; a.K = (uint32_t)K;
  a.batch = (uint32_t)batch;
  a.tiles = (uint32_t)p.tile_cap;
  a.off = p.off; a.dir = p.dir; a.remap = p.remap; a.shuffle_k = p.shuffle;
  a.mc = map_consts(p, M, N);
  a.cdtype = (uint32_t)c;
  fill_ws(a, p, ws);
  empty = false;
  return BST_OK;
}

bst_status dense(bst_dtype ab, bst_dtype c, int64_t batch, int64_t M, int64_t N, int64_t K,
                 const void* A, int64_t lda, int64_t strideA, const void* B, int64_t ldb,
                 int64_t strideB, void* C, int64_t ldc, int64_t strideC, const uint8_t* sa,
                 const uint8_t* sb, const float* rs, const float* cs, const bst_sched* s,
                 void* ws, size_t ws_bytes, void* stream, const void* X = nullptr,
                 int64_t ldx = 0) {
  Plan p;
  GemmArgs a{};
  bool empty = true;
  const bst_status st = prepare_dense(ab, c, batch, M, N, K, A, lda, strideA, B, ldb, strideB, C,
                                      ldc, strideC, sa, sb, rs, cs, s, ws, ws_bytes, X, ldx, p, a,
                                      empty);
  if (st != BST_OK || empty) return st;
  return launch(p, a, stream);
}

// ------------------------------------------------------- padding GEMM ----
// Row repack of an operand into the workspace: dst[r][c] = src[r][c] for
// r < rows and c < cols, 0 elsewhere in drows x dld elements (drows >= rows).
// Reads stay inside the caller's rows x cols matrix, writes inside
// drows x dld.
// One workgroup per row at a time (rows strided over the grid), its threads
// over the row's elements, so that loads and stores are consecutive; each
// thread keeps four loads in flight before it stores.
template <typename E>
__global__ void repack_kernel(const E* __restrict__ src, int64_t sld, E* __restrict__ dst,
                              int64_t dld, int64_t rows, int64_t cols, int64_t drows) {
  const int64_t nt = blockDim.x;
  for (int64_t r = blockIdx.x; r < drows; r += gridDim.x) {
    const bool live = r < rows;  // rows past the source are all zeros
    const E* s = src + (live ? r : 0) * sld;
    E* d = dst + r * dld;
    for (int64_t c0 = threadIdx.x; c0 < dld; c0 += 4 * nt) {
      E v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t c = c0 + u * nt;
        v[u] = (live && c < cols) ? s[c] : E(0);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t c = c0 + u * nt;
        if (c < dld) d[c] = v[u];
      }
    }
  }
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Repacked layout: A as [M][lda] and B as [kp][ldb] with rows of whole
// 16-byte chunks, zeros in the padding; the GEMM then runs with K = kp (A's
// padding columns meet B's zero rows, so every added product is an exact 0),
// which lets the LDS-DMA kernels take it whatever K was.  The int8 bound on
// K is kept: kp stays K when padding would cross it.  Both copies start at a
// 256-byte boundary.
struct Padded {
  int64_t lda = 0, ldb = 0, kp = 0;
  size_t a_bytes = 0, bytes = 0;
};
Padded padded_layout(bst_dtype ab, int64_t M, int64_t N, int64_t K) {
  Padded q;
  const int64_t es = (int64_t)elem_size(ab), ce = 16 / es;
  q.lda = round_up(K, ce);
  q.ldb = round_up(N, ce);
  q.kp = (ab == BST_I8 && q.lda > 131071) ? K : q.lda;
  q.a_bytes = (size_t)round_up(M * q.lda * es, 256);
  q.bytes = q.a_bytes + (size_t)round_up(q.kp * q.ldb * es, 256);
  return q;
}

size_t padded_gemm_ws(const Plan& p) {
  return (size_t)round_up((int64_t)std::max(p.ws_bytes, kCounterBytes), 256);
}

bst_status repack(bst_dtype ab, const void* src, int64_t sld, void* dst, int64_t dld, int64_t rows,
                  int64_t cols, int64_t drows, void* stream) {
  if (drows * dld == 0) return BST_OK;
  const int64_t blocks = std::min<int64_t>(drows, 4096);
  if (elem_size(ab) == 2)
    hipLaunchKernelGGL((repack_kernel<uint16_t>), dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, static_cast<const uint16_t*>(src), sld,
                       static_cast<uint16_t*>(dst), dld, rows, cols, drows);
  else
    hipLaunchKernelGGL((repack_kernel<uint8_t>), dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, static_cast<const uint8_t*>(src), sld,
                       static_cast<uint8_t*>(dst), dld, rows, cols, drows);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BST_E_HIP, "repack launch failed: %s", hipGetErrorString(e));
  return BST_OK;
}

// ------------------------------------------------- static scratch -------
// The scratch of bst_gemm_noalloc: a workspace (counter area, then split-K
// partials) that lives in the library's own device memory, one copy per GPU
// for the life of the process.  In host code `scratch` names a host-side
// stand-in, not the device address: the address comes from
// hipGetSymbolAddress, once per device (scratch_ptr), and only that address
// is passed to kernels.
constexpr size_t kScratchBytes = 32u << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch;  // device -> address of its scratch

__global__ void zero_words(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    p[i] = 0u;
}

// The current device's scratch address; on the first call for a device, its
// counter area is cleared on `stream` (a fill kernel, so that a capturing
// caller records no memset node).
bst_status scratch_ptr(void* stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BST_E_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch.find(dev);
  if (it != g_scratch.end()) {
    *out = it->second;
    return BST_OK;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr)
    return fail(BST_E_HIP, "hipGetSymbolAddress of the scratch failed: %s", hipGetErrorString(e));
  hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, (hipStream_t)stream,
                     static_cast<uint32_t*>(ptr), (uint32_t)(kCounterBytes / 4));
  e = hipGetLastError();
  if (e != hipSuccess) return fail(BST_E_HIP, "scratch clear failed: %s", hipGetErrorString(e));
  g_scratch[dev] = ptr;
  *out = ptr;
  return BST_OK;
}

}  // namespace

extern "C" {

#ifdef BST_TRACE
void bst_debug_set_trace(void* dev_buf) { g_trace = (uint64_t*)dev_buf; }
#endif

const char* bst_last_error(void) { return g_err; }

bst_status bst_set_clock_record(void* dev_buf, int64_t n) {
  if (n < 0 || n > 0x7fffffff || (n > 0 && !dev_buf))
    return fail(BST_E_INVAL, "clock record: n %lld with buffer %p", (long long)n, dev_buf);
  g_clock = n > 0 ? static_cast<uint64_t*>(dev_buf) : nullptr;
  g_clock_n = (uint32_t)n;
  return BST_OK;
}

const char* bst_version(void) { return "bst 0.1 (gfx950)"; }

bst_status bst_gemm(bst_dtype ab, bst_dtype c, int64_t M, int64_t N, int64_t K, const void* A,
                    int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                    const uint8_t* scale_a, const uint8_t* scale_b, const bst_sched* s, void* ws,
                    size_t ws_bytes, void* stream) {
  if (ab != BST_MXE4M3 && (scale_a || scale_b))
    return fail(BST_E_INVAL, "block scales are only taken with BST_MXE4M3");
  return dense(ab, c, 1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, scale_a, scale_b, nullptr,
               nullptr, s, ws, ws_bytes, stream);
}

bst_status bst_gemm_noalloc(bst_dtype ab, bst_dtype c, int64_t M, int64_t N, int64_t K,
                            const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                            int64_t ldc, const uint8_t* scale_a, const uint8_t* scale_b,
                            const bst_sched* s, void* stream) {
  if (ab != BST_MXE4M3 && (scale_a || scale_b))
    return fail(BST_E_INVAL, "block scales are only taken with BST_MXE4M3");
  // every check first, against a stand-in address of the scratch's size
  Plan p;
  GemmArgs a{};
  bool empty = true;
  void* const stand_in = reinterpret_cast<void*>(uintptr_t{256});
  bst_status st = make_plan(FORM_DENSE, ab, 1, M, N, K, s, false, p);
  if (st != BST_OK) return st;
  if (p.ws_bytes > kScratchBytes)
    return fail(BST_E_WORKSPACE, "this schedule needs %zu workspace bytes; the static scratch of "
                "bst_gemm_noalloc holds %zu (use a smaller split_k, or bst_gemm with a workspace)",
                p.ws_bytes, kScratchBytes);
  st = prepare_dense(ab, c, 1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, scale_a, scale_b, nullptr,
                     nullptr, s, stand_in, kScratchBytes, nullptr, 0, p, a, empty);
  if (st != BST_OK || empty) return st;
  if (p.ws_bytes > kScratchBytes)  // the plan made with the device's CU count
    return fail(BST_E_WORKSPACE, "this schedule needs %zu workspace bytes; the static scratch of "
                "bst_gemm_noalloc holds %zu", p.ws_bytes, kScratchBytes);
  void* ws = nullptr;
  st = scratch_ptr(stream, &ws);
  if (st != BST_OK) return st;
  fill_ws(a, p, ws);
  return launch(p, a, stream);
}

bst_status bst_gemm_add(bst_dtype ab, bst_dtype c, int64_t M, int64_t N, int64_t K, const void* A,
                        int64_t lda, const void* B, int64_t ldb, const void* X, int64_t ldx,
                        void* C, int64_t ldc, const uint8_t* scale_a, const uint8_t* scale_b,
                        const bst_sched* s, void* ws, size_t ws_bytes, void* stream) {
  if (ab != BST_MXE4M3 && (scale_a || scale_b))
    return fail(BST_E_INVAL, "block scales are only taken with BST_MXE4M3");
  if (M > 0 && N > 0 && !X) return fail(BST_E_INVAL, "the addend X is NULL");
  return dense(ab, c, 1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, scale_a, scale_b, nullptr,
               nullptr, s, ws, ws_bytes, stream, X, ldx);
}

bst_status bst_gemm_padded(bst_dtype ab, bst_dtype c, int64_t M, int64_t N, int64_t K,
                           const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                           int64_t ldc, const uint8_t* scale_a, const uint8_t* scale_b,
                           const bst_sched* s, void* ws, size_t ws_bytes, void* stream) {
  if (!is_ab(ab)) return fail(BST_E_INVAL, "unknown operand dtype %d", (int)ab);
  if (ab != BST_MXE4M3 && (scale_a || scale_b))
    return fail(BST_E_INVAL, "block scales are only taken with BST_MXE4M3");
  if (M < 0 || N < 0 || K < 0) return fail(BST_E_INVAL, "negative size");
  if (M == 0 || N == 0) return BST_OK;
  if (K > 0 && (!A || !B)) return fail(BST_E_INVAL, "A or B is NULL");
  if (K > 0 && (lda < K || ldb < N))
    return fail(BST_E_INVAL, "leading dimension too small (lda %lld K %lld, ldb %lld N %lld)",
                (long long)lda, (long long)K, (long long)ldb, (long long)N);
  // the caller's K decides what is valid (MX blocks, the int8 bound); the
  // GEMM then runs at the padded depth
  Plan p;
  bst_status st = make_plan(FORM_DENSE, ab, 1, M, N, K, s, false, p);
  if (st != BST_OK) return st;
  const Padded q = padded_layout(ab, M, N, K);
  const Layout lay{q.lda, q.ldb, scale_a, scale_b, ldc * (int64_t)elem_size(c)};
  st = make_plan(FORM_DENSE, ab, 1, M, N, q.kp, s, true, p, &lay);
  if (st != BST_OK) return st;
  // The GEMM's own workspace comes first, its split-K counters at offset 0
  // whatever the split, so that a workspace shared with other calls keeps
  // its counter area zero; the repacked operands follow.
  const size_t gws = padded_gemm_ws(p);
  if (!ws || ws_bytes < gws + q.bytes)
    return fail(BST_E_WORKSPACE, "the padding GEMM needs %zu workspace bytes (got %zu)",
                gws + q.bytes, ws ? ws_bytes : (size_t)0);
  if (!aligned16(ws)) return fail(BST_E_ALIGN, "workspace not 16-byte aligned");
  uint8_t* w = static_cast<uint8_t*>(ws);
  uint8_t* ap = w + gws;
  uint8_t* bp = ap + q.a_bytes;
  // every remaining check (output dtype, C, ldc, scales, workspace) before
  // the first repack, so that a failing call has enqueued nothing
  GemmArgs a{};
  bool empty = true;
  st = prepare_dense(ab, c, 1, M, N, q.kp, ap, q.lda, 0, bp, q.ldb, 0, C, ldc, 0, scale_a,
                     scale_b, nullptr, nullptr, s, w, gws, nullptr, 0, p, a, empty);
  if (st != BST_OK || empty) return st;
  if (K > 0) {
    st = repack(ab, A, lda, ap, q.lda, M, K, M, stream);
    if (st != BST_OK) return st;
    st = repack(ab, B, ldb, bp, q.ldb, K, N, q.kp, stream);
    if (st != BST_OK) return st;
  }
  return launch(p, a, stream);
}

bst_status bst_batched_gemm(bst_dtype ab, bst_dtype c, int64_t batch, int64_t M, int64_t N,
                            int64_t K, const void* A, int64_t lda, int64_t strideA, const void* B,
                            int64_t ldb, int64_t strideB, void* C, int64_t ldc, int64_t strideC,
                            const bst_sched* s, void* ws, size_t ws_bytes, void* stream) {
  if (ab == BST_MXE4M3) return fail(BST_E_UNSUPPORTED, "batched MX GEMM is not provided");
  return dense(ab, c, batch, M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, nullptr,
               nullptr, nullptr, nullptr, s, ws, ws_bytes, stream);
}

bst_status bst_quant_gemm_per_token(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                                    const int8_t* B, int64_t ldb, const float* row_scale,
                                    const float* col_scale, void* C, int64_t ldc, bst_dtype c,
                                    const bst_sched* s, void* ws, size_t ws_bytes, void* stream) {
  if (c != BST_I32 && (!row_scale || !col_scale))
    return fail(BST_E_INVAL, "row_scale and col_scale are required for a dequantised output");
  const bool raw = c == BST_I32;
  return dense(BST_I8, c, 1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, nullptr, nullptr,
               raw ? nullptr : row_scale, raw ? nullptr : col_scale, s, ws, ws_bytes, stream);
}

bst_status bst_grouped_gemm_slice_m(bst_dtype ab, bst_dtype c, int32_t G, const int32_t* group_m,
                                    int64_t total_m, int64_t N, int64_t K, const void* A,
                                    int64_t lda, const void* B, int64_t ldb, int64_t strideB,
                                    void* C, int64_t ldc, const float* row_scale,
                                    const float* col_scale, const bst_sched* s, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (ab != BST_I8 && ab != BST_F16 && ab != BST_BF16)
    return fail(BST_E_UNSUPPORTED, "grouped GEMM takes int8, f16 or bf16 operands");
  if (!out_ok(ab, c)) return fail(BST_E_UNSUPPORTED, "output dtype %d with operands %d", (int)c, (int)ab);
  if ((row_scale == nullptr) != (col_scale == nullptr))
    return fail(BST_E_INVAL, "give both dequant scales or neither");
  if (row_scale && (ab != BST_I8 || c == BST_I32))
    return fail(BST_E_INVAL, "dequant scales need int8 operands and a floating output");
  Plan p;
  bst_status st = make_plan(FORM_SLICE_M, ab, G, total_m, N, K, s, false, p);
  if (st != BST_OK) return st;
  if (!group_m) return fail(BST_E_INVAL, "group_m is NULL");
  if (total_m == 0 || N == 0) return BST_OK;
  const size_t es = elem_size(ab), ec = elem_size(c);
  const bool has_k = K > 0;  // with K == 0, A and B are never read
  if (!C || (has_k && (!A || !B))) return fail(BST_E_INVAL, "A, B or C is NULL");
  if ((has_k && (lda < K || ldb < N || strideB < (int64_t)K * ldb)) || ldc < N)
    return fail(BST_E_INVAL, "leading dimension or group stride too small");
  if (!aligned16(C) || !stride_ok(ldc, ec) ||
      (has_k && (!aligned16(A) || !aligned16(B) || !stride_ok(lda, es) || !stride_ok(ldb, es) ||
                 !stride_ok(strideB, es))))
    return fail(BST_E_ALIGN, "pointers and strides must be 16-byte multiples");
  const Layout lay{lda, ldb, nullptr, nullptr, ldc * (int64_t)ec};
  st = make_plan(FORM_SLICE_M, ab, G, total_m, N, K, s, true, p, &lay);
  if (st != BST_OK) return st;
  st = check_ws(p, ws, ws_bytes);
  if (st != BST_OK) return st;
  GemmArgs a{};
#ifdef BST_TRACE
  a.trace = g_trace;
#endif
  a.A = static_cast<const uint8_t*>(A);
  a.B = static_cast<const uint8_t*>(B);
  a.C = static_cast<uint8_t*>(C);
  a.lda = lda; a.ldb = ldb; a.ldc = ldc;
  a.strideB = strideB;
  a.row_scale = row_scale;
  a.col_scale = col_scale;
  a.group_m = group_m;
  a.G = G;
  a.total_m = total_m;
  a.N = (uint32_t)N; a.K = (uint32_t)K;
  a.off = p.off; a.dir = p.dir; a.remap = p.remap; a.shuffle_k = p.shuffle;
  a.mc.nk_full = make_fastdiv(p.bk ? p.kslice / p.bk : 1u);  // the map itself is per group
  a.cdtype = (uint32_t)c;
  fill_ws(a, p, ws);
  return launch(p, a, stream);
}

bst_status bst_grouped_gemm_slice_k(bst_dtype ab, bst_dtype c, int32_t G, const int32_t* group_k,
                                    int64_t total_k, int64_t M, int64_t N, const void* A,
                                    int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                                    int64_t strideC, const float* row_scale,
                                    const float* col_scale, const bst_sched* s, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (ab != BST_I8 && ab != BST_F16 && ab != BST_BF16)
    return fail(BST_E_UNSUPPORTED, "grouped slice-K GEMM takes int8, f16 or bf16 operands");
  if (!out_ok(ab, c)) return fail(BST_E_UNSUPPORTED, "output dtype %d with operands %d", (int)c, (int)ab);
  if ((row_scale == nullptr) != (col_scale == nullptr))
    return fail(BST_E_INVAL, "give both dequant scales or neither");
  if (row_scale && (ab != BST_I8 || c == BST_I32))
    return fail(BST_E_INVAL, "dequant scales need int8 operands and a floating output");
  Plan p;
  bst_status st = make_plan(FORM_SLICE_K, ab, G, M, N, total_k, s, false, p);
  if (st != BST_OK) return st;
  if (!group_k) return fail(BST_E_INVAL, "group_k is NULL");
  if (M == 0 || N == 0) return BST_OK;
  const size_t es = elem_size(ab), ec = elem_size(c);
  const bool has_k = total_k > 0;  // with no K at all, A and B are never read
  if (!C || (has_k && (!A || !B))) return fail(BST_E_INVAL, "A, B or C is NULL");
  if ((has_k && (lda < total_k || ldb < N)) || ldc < N)
    return fail(BST_E_INVAL, "leading dimension too small (lda %lld total_k %lld, ldb %lld, "
                "ldc %lld, N %lld)", (long long)lda, (long long)total_k, (long long)ldb,
                (long long)ldc, (long long)N);
  if (G > 1 && (strideC < 0 || strideC < (M - 1) * ldc + N))
    return fail(BST_E_INVAL, "strideC %lld lets the groups' outputs overlap (need >= %lld)",
                (long long)strideC, (long long)((M - 1) * ldc + N));
  if (!aligned16(C) || !stride_ok(ldc, ec) || (G > 1 && !stride_ok(strideC, ec)) ||
      (has_k && (!aligned16(A) || !aligned16(B) || !stride_ok(lda, es) || !stride_ok(ldb, es))))
    return fail(BST_E_ALIGN, "pointers and strides must be 16-byte multiples");
  const Layout lay{lda, ldb, nullptr, nullptr, ldc * (int64_t)ec};
  st = make_plan(FORM_SLICE_K, ab, G, M, N, total_k, s, true, p, &lay);
  if (st != BST_OK) return st;
  st = check_ws(p, ws, ws_bytes);
  if (st != BST_OK) return st;
  GemmArgs a{};
#ifdef BST_TRACE
  a.trace = g_trace;
#endif
  a.A = static_cast<const uint8_t*>(A);
  a.B = static_cast<const uint8_t*>(B);
  a.C = static_cast<uint8_t*>(C);
  a.lda = lda; a.ldb = ldb; a.ldc = ldc;
  a.strideC = G > 1 ? strideC : 0;
  a.row_scale = row_scale;
  a.col_scale = col_scale;
  a.group_k = group_k;
  a.G = G;
  a.total_k = total_k;
  a.M = (uint32_t)M; a.N = (uint32_t)N; a.K = (uint32_t)total_k;
  a.batch = (uint32_t)G;
  a.tiles = (uint32_t)p.tile_cap;
  a.off = p.off; a.dir = p.dir; a.remap = p.remap; a.shuffle_k = p.shuffle;
  a.mc = map_consts(p, M, N);
  a.mc.nk_full = make_fastdiv(1);  // groups differ in K: ShuffleK does not apply
  a.cdtype = (uint32_t)c;
  fill_ws(a, p, ws);
  return launch(p, a, stream);
}

bst_status bst_tile_map(bst_dtype ab, int64_t batch, int64_t M, int64_t N, const bst_sched* s,
                        uint32_t* out, int64_t max_tasks, void* stream) {
  Plan p;
  bst_sched d{};
  if (s) d = *s;
  d.split_k = 1;
  bst_status st = make_plan(FORM_DENSE, ab, batch, M, N, 0, s ? &d : nullptr, false, p);
  if (st != BST_OK) return st;
  if (p.tile_cap == 0) return BST_OK;
  if (!out) return fail(BST_E_INVAL, "out is NULL");
  if ((int64_t)p.tile_cap > max_tasks)
    return fail(BST_E_INVAL, "%llu tasks do not fit max_tasks %lld",
                (unsigned long long)p.tile_cap, (long long)max_tasks);
  GemmArgs a{};
#ifdef BST_TRACE
  a.trace = g_trace;
#endif
  a.M = (uint32_t)M; a.N = (uint32_t)N;
  a.batch = (uint32_t)batch;
  a.tiles = (uint32_t)p.tile_cap;
  a.off = p.off; a.dir = p.dir; a.remap = p.remap; a.shuffle_k = p.shuffle;
  a.mc = map_consts(p, M, N);
  a.map_out = out;
  uint32_t grid = s && s->grid ? std::min<uint32_t>(s->grid, a.tiles)
                               : (uint32_t)std::min<int64_t>(device_cus(), a.tiles);
  a.grid = grid;
  hipLaunchKernelGGL((tile_map_kernel<false>), dim3(grid), dim3(64), 0, (hipStream_t)stream, a,
                     p.bm, p.bn);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BST_E_HIP, "map kernel launch failed: %s", hipGetErrorString(e));
  return BST_OK;
}

bst_status bst_grouped_tile_map(bst_dtype ab, int32_t G, const int32_t* group_m, int64_t total_m,
                                int64_t N, const bst_sched* s, uint32_t* out, int64_t max_tasks,
                                void* stream) {
  Plan p;
  bst_sched d{};
  if (s) d = *s;
  d.split_k = 1;
  bst_status st = make_plan(FORM_SLICE_M, ab, G, total_m, N, 0, s ? &d : nullptr, false, p);
  if (st != BST_OK) return st;
  if (!group_m || !out) return fail(BST_E_INVAL, "group_m or out is NULL");
  if ((int64_t)p.tile_cap > max_tasks)
    return fail(BST_E_INVAL, "max_tasks %lld below the bound %llu", (long long)max_tasks,
                (unsigned long long)p.tile_cap);
  if (p.tile_cap == 0) return BST_OK;
  GemmArgs a{};
#ifdef BST_TRACE
  a.trace = g_trace;
#endif
  a.N = (uint32_t)N;
  a.group_m = group_m;
  a.G = G;
  a.total_m = total_m;
  a.off = p.off; a.dir = p.dir; a.remap = p.remap; a.shuffle_k = p.shuffle;
  a.map_out = out;
  uint32_t grid = s && s->grid ? std::min<uint32_t>(s->grid, (uint32_t)p.tile_cap)
                               : (uint32_t)std::min<int64_t>(device_cus(), p.tile_cap);
  a.grid = grid;
  hipLaunchKernelGGL((tile_map_kernel<true>), dim3(grid), dim3(64), 0, (hipStream_t)stream, a,
                     p.bm, p.bn);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BST_E_HIP, "map kernel launch failed: %s", hipGetErrorString(e));
  return BST_OK;
}

size_t bst_workspace_bytes(int kind, bst_dtype ab, int64_t count, int64_t M, int64_t N, int64_t K,
                           const bst_sched* s) {
  Plan p;
  if (kind < 0 || kind > 3) {
    fail(BST_E_INVAL, "kind must be 0, 1, 2 or 3");
    return 0;
  }
  if (kind == 2) {  // bst_gemm_padded: the split-K workspace, then the repacked operands
    if (!is_ab(ab) || M < 0 || N < 0 || K < 0) return 0;
    if (make_plan(FORM_DENSE, ab, 1, M, N, K, s, false, p) != BST_OK) return 0;
    const Padded q = padded_layout(ab, M, N, K);
    const Layout lay{q.lda, q.ldb, nullptr, nullptr};
    if (make_plan(FORM_DENSE, ab, 1, M, N, q.kp, s, true, p, &lay) != BST_OK) return 0;
    return padded_gemm_ws(p) + q.bytes;
  }
  if (make_plan(kind_form(kind), ab, count, M, N, K, s, true, p) != BST_OK) return 0;
  return p.ws_bytes;
}

bst_status bst_effective_sched(int kind, bst_dtype ab, int64_t count, int64_t M, int64_t N,
                               int64_t K, const bst_sched* s, bst_sched* out) {
  if (!out) return fail(BST_E_INVAL, "out is NULL");
  if (kind < 0 || kind > 3) return fail(BST_E_INVAL, "kind must be 0, 1, 2 or 3");
  Plan p;
  bst_status st = make_plan(kind_form(kind), ab, count, M, N, K, s, true, p);
  if (st != BST_OK) return st;
  if (kind == 2) {  // the GEMM bst_gemm_padded runs on the repacked operands
    const Padded q = padded_layout(ab, M, N, K);
    const Layout lay{q.lda, q.ldb, nullptr, nullptr};
    st = make_plan(FORM_DENSE, ab, 1, M, N, q.kp, s, true, p, &lay);
    if (st != BST_OK) return st;
  }
  out->tile_m = p.bm;
  out->tile_n = p.bn;
  out->tile_k = p.bk;
  out->swizzle_offset = p.off;
  out->swizzle_direction = p.dir;
  out->split_k = p.split;
  out->xcd_remap = p.remap;
  out->grid = p.grid;
  out->path = !p.inst->dma ? 1u : p.inst->wgs == 2 ? 3u : 2u;
  out->shuffle_k = p.shuffle;
  out->dynamic = p.dynamic;
  out->preload = p.preload;
  return BST_OK;
}

bst_status bst_task_count(int kind, bst_dtype ab, int64_t count, int64_t M, int64_t N,
                          const bst_sched* s, int64_t* tasks) {
  if (!tasks) return fail(BST_E_INVAL, "tasks is NULL");
  if (kind != 0 && kind != 1 && kind != 3) return fail(BST_E_INVAL, "kind must be 0, 1 or 3");
  bst_sched d{};
  if (s) d = *s;
  d.split_k = 1;
  Plan p;
  const bst_status st = make_plan(kind_form(kind), ab, count, M, N, 0, s ? &d : nullptr, false, p);
  if (st != BST_OK) return st;
  *tasks = (int64_t)p.tile_cap;
  return BST_OK;
}

}  // extern "C"
