// Host-side bounds and coverage check of the LDS-DMA kernels' addressing.
//
// Runs, on the CPU, the same addressing code the GPU kernels run
// (DmaKernel::lane_setup / a_access / b_access / sa_access / sb_access and
// the LDS offset helpers, plus the scheduler's decode_task and
// fill_group_table) over every task, K slice, pipeline stage, wave and lane
// of many problems, and checks that
//   1. every enabled global access (16 bytes of A or B, 4 bytes of a scale
//      block) lies inside the valid rows and columns of its matrix;
//   2. every LDS destination lies inside the stage buffer;
//   3. each stage loads every valid chunk of the tile exactly once;
//   4. where whole MX tasks load A's scales a group of four stages at a time
//      (DmaKernel::SAG), every group load reads 16 bytes inside its row,
//      lands in its group slot, every stage's scale read finds its own
//      group there, and no slot is rewritten while a stage still reads it.
// Prints "ALL OK" and exits 0, or prints the first violation and exits 1.
// Build: hipcc --cuda-host-only -std=c++17 -I include -I <csrc> check_dma_bounds.hip
#include <cstdio>
#include <cstdlib>
#include <set>
#include <string>
#include <vector>

#include <algorithm>

#include "bst_kernel_dma.hpp"

using namespace bst;

static int g_fail = 0;
static long long g_checked = 0;

#define REQUIRE(cond, ...)                          \
  do {                                              \
    if (!(cond)) {                                  \
      if (g_fail < 10) {                            \
        printf("VIOLATION %s:%d: ", __FILE__, __LINE__); \
        printf(__VA_ARGS__);                        \
        printf("\n");                               \
      }                                             \
      ++g_fail;                                     \
    }                                               \
  } while (0)

struct Problem {
  std::string name;
  int64_t batch = 1, M = 0, N = 0, K = 0, lda = 0, ldb = 0, strideA = 0, strideB = 0;
  std::vector<int32_t> groups;  // non-empty: grouped (M = total_m)
  uint32_t split = 1;
  bool scaled = false;
};

template <int AB, int BM, int BN, int WM, int WN, int STAGES, int FORM>
void check(const Problem& p) {
  using KN = DmaKernel<AB, BM, BN, WM, WN, STAGES, FORM>;
  constexpr bool GROUPED = FORM == FORM_SLICE_M;
  constexpr bool SLICEK = FORM == FORM_SLICE_K;
  constexpr int ES = KN::ES, BK = KN::BK, CE = KN::CE, NW = KN::NW;
  // schedule: the same split resolution as the host planner (no empty
  // slices); slice-K groups cut their own K on the device, every slice
  // index up to the requested split exists (slices past a group's end are
  // empty)
  const int64_t nk_all = (p.K + BK - 1) / BK;
  int64_t split = p.split;
  if (nk_all == 0) split = 1;
  const int64_t ks_steps = nk_all > 0 ? (nk_all + split - 1) / split : 0;
  if (ks_steps > 0 && !SLICEK) split = (nk_all + ks_steps - 1) / ks_steps;
  const uint32_t kslice = (uint32_t)(ks_steps * BK);

  GemmArgs a{};
  a.M = (uint32_t)p.M;
  a.N = (uint32_t)p.N;
  a.K = (uint32_t)p.K;
  a.off = 2;
  a.dir = 0;
  a.lda = p.lda;
  a.ldb = p.ldb;
  a.ldsa = p.K / 32;
  a.ldsb = p.N;
  a.total_m = p.M;
  GroupTable gt;
  const GroupTable* gtp = nullptr;
  const uint32_t loopsN = (uint32_t)((p.N + BN - 1) / BN);
  uint32_t T;
  if (GROUPED) {
    a.G = (int)p.groups.size();
    fill_group_table(gt, p.groups.data(), a.G, p.M, BM, loopsN);
    gtp = &gt;
    T = gt.first_task[a.G];
  } else if (SLICEK) {
    a.G = (int)p.groups.size();
    a.total_k = p.K;
    fill_k_table(gt, p.groups.data(), a.G, p.K);
    T = (uint32_t)(a.G * ((p.M + BM - 1) / BM) * loopsN);
  } else {
    T = (uint32_t)(p.batch * ((p.M + BM - 1) / BM) * loopsN);
  }
  if (!GROUPED)
    a.mc = make_map_consts((uint32_t)((p.M + BM - 1) / BM), loopsN, a.off, a.dir, T,
                           (uint32_t)(kslice / BK));
  const int64_t rowbytesA = p.lda * ES, rowbytesB = p.ldb * ES;
  for (uint32_t s = 0; s < split; ++s) {
    for (uint32_t t = 0; t < T; ++t) {
      const Task tk = decode_task(a, t, BM, BN, gtp);
      // the kernel's own K-range code: all of K, or the slice-K group's
      uint32_t kq = 0, kg = a.K, ks = kslice;
      bool poison = false;
      if (SLICEK) {
        kq = (uint32_t)gt.first_row[tk.idx];
        kg = (uint32_t)gt.first_row[tk.idx + 1] - kq;
        ks = group_kslice(kg, (uint32_t)split, BK);
        poison = ((kq | kg) % (uint32_t)CE) != 0u;
      }
      const KRange kr = slice_range(kq, kg, ks, s);
      const uint32_t k0 = kr.k0, k1 = kr.k1;
      const uint32_t nk = (k0 < k1 && !poison) ? (k1 - k0 + BK - 1) / BK : 0u;
      REQUIRE(k1 <= kq + kg && (k0 >= k1 || k0 >= kq), "%s slice [%u,%u) outside group [%u,%u)",
              p.name.c_str(), k0, k1, kq, kq + kg);
      // valid rows of the tile in the stacked A (group or batch problem)
      int64_t row_lo = tk.row0, row_hi = tk.row0 + tk.rows_valid;
      int64_t prob_rows;  // rows of this problem / group, for the bound check
      int64_t prob_first;
      if (GROUPED) {
        prob_first = gt.first_row[tk.idx];
        prob_rows = gt.first_row[tk.idx + 1] - prob_first;
      } else {
        prob_first = 0;
        prob_rows = p.M;
      }
      const int64_t bidx = FORM == FORM_DENSE ? tk.idx : 0;
      const int64_t bsel = SLICEK ? 0 : tk.idx;
      const int64_t a_tile = (bidx * p.strideA + tk.row0 * p.lda) * ES;  // bytes from A
      const int64_t b_tile = (bsel * p.strideB + (int64_t)tk.n * BN) * ES;
      // a task without partial or padding stages runs the precomputed lane
      // offsets: they must equal the checked ones at every stage
      const bool full = nk > 0 && KN::full_task(k0, k1);
      auto same = [](uint32_t u, uint32_t v) { return u == v || (u >= kOob && v >= kOob); };
      // whole MX tasks starting on a group boundary load A's scales by groups
      if constexpr (KN::SAG) {
        if (p.scaled && full && (k0 / BK) % 4 == 0) {
          REQUIRE(nk % 4 == 0, "grouped task of %u stages", nk);
          check_scale_groups<KN, BM, STAGES>(p, tk, k0, nk, a);
        }
      }
      // padding stages (past nk, up to the unroll) must access nothing
      for (uint32_t kt = 0; kt < KN::padded_stages(nk); ++kt) {
        const uint32_t kb0 = k0 + kt * BK;
        std::vector<int> covA(BM * 8, 0), covB(BK * KN::NCH, 0);
        std::vector<int> covSA(BM, 0), covSB(4 * BN, 0);
        for (uint32_t w = 0; w < (uint32_t)NW; ++w) {
          for (uint32_t lane = 0; lane < 64; ++lane) {
            typename KN::Lanes ln;
            KN::lane_setup(ln, w, lane, tk.rows_valid, tk.n, a.N, a.lda, rowbytesB, a.ldsa,
                           a.ldsb);
            for (int i = 0; i < KN::A_IPW; ++i) {
              const uint32_t lds = KN::a_lds(w, i) + lane * 16;
              REQUIRE(lds + 16 <= (uint32_t)KN::A_BYTES, "A lds %u", lds);
              const auto x = KN::a_access(ln, i, kb0, k1);
              ++g_checked;
              if (full) REQUIRE(same(KN::full_voff(ln, i), x.voff), "A full voff");
              if (!x.ok) { REQUIRE(x.voff >= kOob, "disabled A lane in range"); continue; }
              REQUIRE(x.voff < kOob, "A voff %u", x.voff);
              const int64_t addr = a_tile + (int64_t)kb0 * ES + x.voff;  // from batch base
              const int64_t rel = addr - bidx * p.strideA * ES;
              const int64_t R = rel / rowbytesA, cb = rel % rowbytesA;
              REQUIRE(R >= row_lo && R < row_hi && R >= prob_first &&
                          R < prob_first + prob_rows,
                      "%s A row %lld outside [%lld,%lld)", p.name.c_str(), (long long)R,
                      (long long)row_lo, (long long)row_hi);
              // the whole chunk inside the task's K range (a slice-K chunk
              // may not reach into the next group)
              REQUIRE(cb + 16 <= p.K * ES && cb >= (int64_t)kb0 * ES &&
                          cb + 16 <= (int64_t)k1 * ES,
                      "%s A col byte %lld (K %lld, kb0 %u, kend %u)", p.name.c_str(),
                      (long long)cb, (long long)p.K, kb0, k1);
              // coverage: which (row, chunk) of the tile stage landed where
              const int64_t r = R - tk.row0, c = (cb - (int64_t)kb0 * ES) / 16;
              if (r >= 0 && r < BM && c >= 0 && c < 8) {
                covA[r * 8 + c]++;
                REQUIRE((lds / 128) == (uint32_t)r && ((lds % 128) / 16) == (c ^ swz(r)),
                        "A chunk (%lld,%lld) at lds %u", (long long)r, (long long)c, lds);
              }
            }
            for (int i = 0; i < KN::B_IPW; ++i) {
              const uint32_t lds = KN::b_lds(w, i) + lane * 16;
              REQUIRE(lds + 16 <= (uint32_t)(KN::A_BYTES + KN::B_BYTES), "B lds %u", lds);
              const auto x = KN::b_access(ln, i, kb0, k1);
              ++g_checked;
              if (full)
                REQUIRE(same(KN::full_voff(ln, KN::A_IPW + i), x.voff), "B full voff");
              if (!x.ok) { REQUIRE(x.voff >= kOob, "disabled B lane in range"); continue; }
              REQUIRE(x.voff < kOob, "B voff %u", x.voff);
              const int64_t rel = b_tile - bsel * p.strideB * ES +
                                  (int64_t)kb0 * rowbytesB + x.voff;
              const int64_t R = rel / rowbytesB, cb = rel % rowbytesB;
              REQUIRE(R >= kb0 && R < k1 && R < p.K, "%s B row %lld (kb0 %u kend %u)",
                      p.name.c_str(), (long long)R, kb0, k1);
              REQUIRE(cb + 16 <= p.N * ES && cb >= (int64_t)tk.n * BN * ES &&
                          cb < ((int64_t)tk.n * BN + BN) * ES,
                      "%s B col byte %lld (N %lld)", p.name.c_str(), (long long)cb,
                      (long long)p.N);
              const int64_t k = R - kb0, c = (cb - (int64_t)tk.n * BN * ES) / 16;
              covB[k * KN::NCH + c]++;
              const uint32_t lb = lds - KN::A_BYTES;
              REQUIRE(lb / KN::RB == (uint32_t)k && (lb % KN::RB) / 16 == (c ^ KN::swz_b(k)),
                      "B chunk (%lld,%lld) at lds %u", (long long)k, (long long)c, lb);
            }
            if (KN::T::SCALED && p.scaled) {
              for (int i = 0; i < KN::SC_IPW; ++i) {
                const auto sl = KN::sc_slot(w, i);
                const auto x = KN::sc_access(ln, i, kb0, k1);
                ++g_checked;
                if (full)
                  REQUIRE(same(KN::full_voff(ln, KN::A_IPW + KN::B_IPW + i), x.voff),
                          "scale full voff");
                if (sl.kind == 2) {  // padding slot: no access, writes the stage's dummy area
                  REQUIRE(!x.ok && x.voff == kOob, "padding scale slot accesses memory");
                  REQUIRE(KN::SD_BYTES == 256 &&
                              sl.lds == (uint32_t)(KN::A_BYTES + KN::B_BYTES + KN::SA_BYTES + KN::SB_BYTES) &&
                              sl.lds + 256 == (uint32_t)KN::STAGE_BYTES,
                          "padding slot lds %u", sl.lds);
                  continue;
                }
                const uint32_t lds = sl.lds + lane * 4;
                if (sl.kind == 0)
                  REQUIRE(lds >= (uint32_t)(KN::A_BYTES + KN::B_BYTES) &&
                              lds + 4 <= (uint32_t)(KN::A_BYTES + KN::B_BYTES + KN::SA_BYTES),
                          "SA lds %u", lds);
                else
                  REQUIRE(lds >= (uint32_t)(KN::A_BYTES + KN::B_BYTES + KN::SA_BYTES) &&
                              lds + 4 <= (uint32_t)KN::STAGE_BYTES, "SB lds %u", lds);
                if (!x.ok) continue;
                if (sl.kind == 0) {
                  const int64_t addr = tk.row0 * a.ldsa + kb0 / 32 + x.voff;
                  const int64_t R = addr / a.ldsa, c = addr % a.ldsa;
                  REQUIRE(R >= row_lo && R < row_hi && c + 4 <= a.ldsa && c == kb0 / 32,
                          "%s SA row %lld col %lld", p.name.c_str(), (long long)R, (long long)c);
                  // the row's dword lands where the MFMA operand read expects it
                  REQUIRE(lds == (uint32_t)(KN::A_BYTES + KN::B_BYTES + (R - tk.row0) * 4),
                          "SA row %lld at lds %u", (long long)R, lds);
                  covSA[R - tk.row0]++;
                } else {
                  const int64_t addr = (int64_t)tk.n * BN + (int64_t)(kb0 / 32) * a.ldsb + x.voff;
                  const int64_t R = addr / a.ldsb, c = addr % a.ldsb;
                  REQUIRE(R >= kb0 / 32 && R < kb0 / 32 + 4 && R < p.K / 32 && c + 4 <= p.N,
                          "%s SB row %lld col %lld", p.name.c_str(), (long long)R, (long long)c);
                  const int64_t e = R - kb0 / 32, cc = c - tk.n * BN;
                  REQUIRE(lds == (uint32_t)(KN::A_BYTES + KN::B_BYTES + KN::SA_BYTES + e * BN + cc),
                          "SB (%lld,%lld) at lds %u", (long long)e, (long long)cc, lds);
                  for (int q = 0; q < 4; ++q) covSB[e * BN + cc + q]++;
                }
              }
            }
          }
        }
        // coverage: every valid chunk exactly once, nothing else
        for (int r = 0; r < BM; ++r)
          for (int c = 0; c < 8; ++c) {
            const bool want = (uint32_t)r < tk.rows_valid && kb0 + c * CE < k1;
            REQUIRE(covA[r * 8 + c] == (want ? 1 : 0), "%s A coverage r %d c %d = %d",
                    p.name.c_str(), r, c, covA[r * 8 + c]);
          }
        for (int k = 0; k < BK; ++k)
          for (int c = 0; c < KN::NCH; ++c) {
            const bool want = kb0 + k < k1 && tk.n * BN + c * CE < a.N;
            REQUIRE(covB[k * KN::NCH + c] == (want ? 1 : 0), "%s B coverage k %d c %d = %d",
                    p.name.c_str(), k, c, covB[k * KN::NCH + c]);
          }
        if (KN::T::SCALED && p.scaled) {
          for (int r = 0; r < BM; ++r)
            REQUIRE(covSA[r] == ((uint32_t)r < tk.rows_valid && kb0 < k1 ? 1 : 0), "SA coverage %d", r);
          for (int e = 0; e < 4; ++e)
            for (int c = 0; c < BN; ++c)
              REQUIRE(covSB[e * BN + c] == (tk.n * BN + c < a.N && kb0 < k1 ? 1 : 0), "SB coverage");
        }
      }
    }
  }
}

// Whole MX tasks with A-scale groups: for the ShuffleK shifts given, walk
// the task's stages in issue order, check every group load's addresses, and
// replay the loads and the reads on a timeline of loop steps: a load goes out
// in the step that issues its group's first stage (j - (S - 1); the stages
// of the prologue before any read), and the waves read group g's slot into
// registers once, in the prologue for group 0 and in step 4g - 1 (the last
// step of the trip before, with stage 4g resident) for the others.  A read
// must find its group as the slot's last load from an earlier step, and no
// load may hit a slot in the step that reads it.
template <class KN, int BM, int S>
void check_scale_groups(const Problem& p, const Task& tk, uint32_t k0, uint32_t nk,
                        const GemmArgs& a) {
  constexpr int BK = KN::BK;
  const int64_t row_lo = tk.row0, row_hi = tk.row0 + tk.rows_valid;
  std::vector<uint32_t> shifts = {0u};
  if (nk >= 8) shifts.push_back(4u);
  if (nk >= 4) shifts.push_back(nk - 4);
  struct Load { int64_t t; uint32_t slot; int64_t group; };
  for (uint32_t kshift : shifts) {
    std::vector<Load> loads;
    for (uint32_t j = 0; j < nk; ++j) {
      // the kernel's own rule for which issue carries a group load
      const bool gst = j < (uint32_t)(S - 1) ? KN::sag_issue_prologue((int)j)
                                            : KN::sag_issue_step((int)((j - (S - 1)) % 4));
      REQUIRE(gst == (j % 4 == 0), "stage %u group load %d", j, (int)gst);
      if (!gst) continue;
      const uint32_t kb0 = k0 + ((j + kshift) % nk) * BK;
      const uint32_t slot = KN::sag_slot(j);
      REQUIRE(kb0 / 32 % 16 == 0, "group start stage %u not on a 16-scale boundary", j);
      for (uint32_t w = 0; w < (uint32_t)KN::NW; ++w)
        for (uint32_t lane = 0; lane < 64; ++lane) {
          typename KN::Lanes ln;
          KN::lane_setup(ln, w, lane, tk.rows_valid, tk.n, a.N, a.lda, 0, a.ldsa, a.ldsb);
          for (int i = 0; i < KN::SCA_IPW; ++i) {
            const auto sl = KN::sc_slot(w, i);
            const uint32_t v = KN::full_voff(ln, KN::A_IPW + KN::B_IPW + i);
            ++g_checked;
            if (sl.kind != 0) {  // a padding A slot: nothing read, zeros into the dummy kilobyte
              REQUIRE(sl.kind == 2 && v >= kOob, "padding A slot reads memory");
              continue;
            }
            const uint32_t lds = slot * KN::SAG_SLOT + KN::sag_lds(sl.idx) + lane * 16;
            const uint32_t r = sl.idx * 64 + lane;  // row inside the tile
            REQUIRE(lds + 16 <= 2u * KN::SAG_SLOT && lds == slot * KN::SAG_SLOT + r * 16,
                    "group row %u at lds %u", r, lds);
            if (v >= kOob) {
              REQUIRE(r >= tk.rows_valid, "valid row %u without its group", r);
              continue;
            }
            const int64_t addr = tk.row0 * a.ldsa + (int64_t)v + (kb0 / 32);
            const int64_t R = addr / a.ldsa, c = addr % a.ldsa;
            REQUIRE(R >= row_lo && R < row_hi && R - tk.row0 == (int64_t)r,
                    "%s group row %lld outside [%lld,%lld)", p.name.c_str(), (long long)R,
                    (long long)row_lo, (long long)row_hi);
            REQUIRE(c == kb0 / 32 && c + 16 <= a.ldsa, "%s group col %lld (ldsa %lld)",
                    p.name.c_str(), (long long)c, (long long)a.ldsa);
          }
        }
      const int64_t t = j < (uint32_t)(S - 1) ? -2 : (int64_t)j - (S - 1);
      loads.push_back(Load{t, slot, (int64_t)(kb0 / 32 / 16)});
    }
    for (uint32_t g = 0; g < nk / 4; ++g) {
      const uint32_t kb0 = k0 + ((4 * g + kshift) % nk) * BK;
      const uint32_t slot = KN::sag_slot(4 * g);
      const int64_t tr = g == 0 ? -1 : 4 * (int64_t)g - 1;
      // every stage of the group reads its scales from these registers: the
      // group's four stages are its 16 bytes in order
      for (uint32_t q = 0; q < 4; ++q)
        REQUIRE(k0 + ((4 * g + q + kshift) % nk) * BK == kb0 + q * BK && KN::sag_slot(4 * g + q) == slot,
                "group %u stage %u out of order", g, q);
      const Load* last = nullptr;
      for (const Load& l : loads) {
        if (l.slot != slot) continue;
        REQUIRE(l.t != tr, "slot %u loaded in step %lld, which reads it", slot, (long long)tr);
        if (l.t < tr && (!last || l.t > last->t)) last = &l;
      }
      ++g_checked;
      REQUIRE(last && last->group == (int64_t)(kb0 / 32 / 16),
              "%s group %u (step %lld) finds group %lld in slot %u, wants %u", p.name.c_str(), g,
              (long long)tr, last ? (long long)last->group : -1LL, slot, kb0 / 32 / 16);
    }
  }
}

static Problem plain(const char* n, int64_t M, int64_t N, int64_t K, int64_t pad_a, int64_t pad_b,
                     uint32_t split, int64_t batch = 1, bool scaled = false) {
  Problem p;
  p.name = n;
  p.M = M; p.N = N; p.K = K;
  p.lda = K + pad_a; p.ldb = N + pad_b;
  p.batch = batch;
  p.strideA = M * p.lda; p.strideB = K * p.ldb;
  p.split = split;
  p.scaled = scaled;
  return p;
}

static Problem grouped(const char* n, std::vector<int32_t> g, int64_t spare, int64_t N, int64_t K,
                       uint32_t split) {
  Problem p;
  p.name = n;
  int64_t tot = 0;
  for (int32_t x : g) tot += x > 0 ? x : 0;
  p.M = tot + spare; p.N = N; p.K = K;
  p.lda = K; p.ldb = N; p.strideB = K * N;
  p.groups = g;
  p.split = split;
  return p;
}

// Grouped slice-K: K cut into groups of the given sizes (total K = their
// sum plus `spare` unused columns), M x N outputs.
static Problem slicek(const char* n, std::vector<int32_t> g, int64_t spare, int64_t M, int64_t N,
                      uint32_t split) {
  Problem p;
  p.name = n;
  int64_t tot = 0;
  for (int32_t x : g) tot += x > 0 ? x : 0;
  p.M = M; p.N = N; p.K = tot + spare;
  p.lda = p.K; p.ldb = N;
  p.groups = g;
  p.split = split;
  return p;
}

template <int AB, int BM, int BN, int WM, int WN, int S>
void run_plain(const std::vector<Problem>& ps) {
  for (const Problem& p : ps) check<AB, BM, BN, WM, WN, S, FORM_DENSE>(p);
}
template <int AB, int BM, int BN, int WM, int WN, int S>
void run_grouped(const std::vector<Problem>& ps) {
  for (const Problem& p : ps) check<AB, BM, BN, WM, WN, S, FORM_SLICE_M>(p);
}
template <int AB, int BM, int BN, int WM, int WN, int S>
void run_slicek(const std::vector<Problem>& ps) {
  for (const Problem& p : ps) check<AB, BM, BN, WM, WN, S, FORM_SLICE_K>(p);
}

// The slice-K run order: a permutation of the groups, longest K first, ties
// by index (checked against a stable sort); the index order beyond the
// ranking limit; the task mapping a bijection of each launch's tasks.
static void check_k_order() {
  const std::vector<std::vector<int32_t>> cases = {
      {336, 208, 32, 80, 16, 5072, 912, 1536}, {0, 0, 48}, {64, 5, 200, 16, 64, 64},
      {1}, {-3, 7, 7, 0, 7}, std::vector<int32_t>(300, 16)};
  for (const auto& gk : cases) {
    const int G = (int)gk.size();
    int64_t total = 0;
    for (int32_t k : gk) total += k > 0 ? k : 0;
    GroupTable gt;
    fill_k_table(gt, gk.data(), G, total);
    std::vector<int> want(G);
    for (int i = 0; i < G; ++i) want[i] = i;
    if (G <= kOrderMaxGroups)
      std::stable_sort(want.begin(), want.end(), [&](int x, int y) {
        return (gt.first_row[x + 1] - gt.first_row[x]) > (gt.first_row[y + 1] - gt.first_row[y]);
      });
    for (int r = 0; r < G; ++r)
      REQUIRE((int)gt.order[r] == want[r], "k order G=%d rank %d: %u, want %d", G, r,
              gt.order[r], want[r]);
    GemmArgs a{};
    a.mc.core = make_fastdiv(6);  // 6 tiles per group
    std::vector<int> seen(6 * G, 0);
    for (uint32_t t = 0; t < 6u * G; ++t) ++seen[slicek_task(a, &gt, t)];
    for (int t = 0; t < 6 * G; ++t) REQUIRE(seen[t] == 1, "k order task %d seen %d times", t, seen[t]);
    ++g_checked;
  }
}

// The division by invariant integers against the hardware-free '/': every
// divisor up to 4096 and a spread of larger ones, each with the dividends
// that sit at and around its multiples and at the ends of the range.
static void check_fastdiv() {
  std::vector<uint32_t> ds;
  for (uint32_t d = 1; d <= 4096; ++d) ds.push_back(d);
  for (uint64_t d = 4097; d < (1ull << 31); d = d * 3 / 2 + 7) ds.push_back((uint32_t)d);
  ds.push_back(0x7fffffffu);
  uint64_t x = 88172645463325252ull;  // xorshift for pseudo-random dividends
  for (uint32_t d : ds) {
    const FastDiv f = make_fastdiv(d);
    std::vector<uint32_t> ns = {0u, 1u, d - 1, d, d + 1, 0xffffffffu, 0xfffffffeu, 0x80000000u};
    for (uint32_t k = 1; k < 64; ++k) {
      const uint64_t m = (uint64_t)d * k * 977u;
      if (m <= 0xffffffffull) { ns.push_back((uint32_t)m); ns.push_back((uint32_t)(m - 1)); }
      x ^= x << 13; x ^= x >> 7; x ^= x << 17;
      ns.push_back((uint32_t)x);
    }
    for (uint32_t n : ns) {
      ++g_checked;
      REQUIRE(f.div(n) == n / d, "fastdiv %u / %u = %u", n, d, f.div(n));
    }
  }
}

// The map with the launch's precomputed constants against block_coord (the
// reference the GPU map test pins to the oracle) over every task.
static void check_fast_map() {
  for (uint32_t lm = 1; lm <= 37; ++lm)
    for (uint32_t ln = 1; ln <= 37; ln += (ln < 12 ? 1 : 5))
      for (uint32_t off : {1u, 2u, 3u, 4u, 5u, 8u, 13u, 1000u})
        for (uint32_t dir = 0; dir < 3; ++dir) {
          const MapConsts mc = make_map_consts(lm, ln, off, dir, lm * ln, 1);
          for (uint32_t i = 0; i < lm * ln; ++i) {
            const TileCoord r = block_coord(lm, ln, off, dir, i);
            const TileCoord f = block_coord_fast(mc, i);
            ++g_checked;
            REQUIRE(r.m == f.m && r.n == f.n, "map %ux%u off %u dir %u task %u: (%u,%u) vs (%u,%u)",
                    lm, ln, off, dir, i, r.m, r.n, f.m, f.n);
          }
        }
}

// Random plain problems of the shape class the GPU tests draw at random:
// M in [1, 320), N and K whole 16-byte chunks up to a few hundred (MX: K in
// blocks of 128), splits 1-3; a fixed xorshift seed.
static std::vector<Problem> random_plain(int n, int q, int kq, bool scaled, uint64_t seed) {
  std::vector<Problem> v;
  uint64_t x = seed;
  auto next = [&]() {
    x ^= x << 13;
    x ^= x >> 7;
    x ^= x << 17;
    return x;
  };
  static char names[64][16];
  for (int i = 0; i < n && i < 64; ++i) {
    const int64_t M = 1 + (int64_t)(next() % 319);
    const int64_t N = q * (1 + (int64_t)(next() % (320 / q)));
    const int64_t K = kq * (1 + (int64_t)(next() % 19));
    const uint32_t split = 1 + (uint32_t)(next() % 3);
    snprintf(names[i], sizeof(names[i]), "rnd%d", i);
    v.push_back(plain(names[i], M, N, K, 0, 0, split, 1, scaled));
  }
  return v;
}

int main() {
  check_fastdiv();
  check_fast_map();
  check_k_order();
  // 16-bit operands: K and N multiples of 8 elements
  const std::vector<Problem> p16 = {
      plain("tails", 200, 136, 256, 0, 0, 1),      plain("tails-split", 200, 136, 256, 8, 16, 3),
      plain("tiny", 1, 8, 8, 0, 0, 1),             plain("ragged", 129, 264, 1000, 24, 8, 2),
      plain("2k", 1024, 1024, 2048, 0, 0, 4),      plain("kslice", 77, 8, 520, 8, 8, 5),
      plain("flat", 300, 1000, 64, 0, 0, 1),       plain("batch", 100, 200, 136, 8, 0, 2, 3),
      plain("k0", 33, 40, 0, 8, 0, 1)};
  const std::vector<Problem> g16 = {grouped("g16", {0, 1, 300, 0, 127, 129, 5}, 9, 136, 264, 1),
                                    grouped("g16s", {64, 0, 200}, 0, 128, 512, 3)};
  run_plain<AB_F16, 64, 64, 2, 2, 4>(p16);
  run_plain<AB_F16, 128, 128, 2, 2, 4>(p16);
  run_plain<AB_F16, 256, 128, 2, 2, 3>(p16);
  run_plain<AB_F16, 128, 256, 2, 2, 3>(p16);
  run_plain<AB_F16, 128, 192, 2, 2, 3>(p16);
  run_plain<AB_F16, 128, 64, 2, 2, 4>(p16);
  run_plain<AB_F16, 64, 128, 2, 2, 4>(p16);
  run_plain<AB_F16, 128, 64, 4, 2, 4>(p16);
  run_plain<AB_F16, 64, 128, 2, 4, 4>(p16);
  run_plain<AB_F16, 256, 256, 4, 2, 2>(p16);
  run_plain<AB_F16, 64, 64, 2, 2, 6>(p16);
  run_plain<AB_F16, 64, 64, 2, 2, 5>(p16);
  run_grouped<AB_F16, 128, 128, 2, 2, 4>(g16);
  // the two-workgroups-per-CU instances (two stages)
  run_plain<AB_F16, 128, 128, 2, 2, 2>(p16);
  run_grouped<AB_F16, 128, 128, 2, 2, 2>(g16);
  // slice-K: aligned groups (8 elements), an empty one, a group cut short by
  // the allocation, and groups that break the 16-byte chunks (no access)
  const std::vector<Problem> k16 = {slicek("k16", {64, 0, 200, 8, 136}, 16, 129, 264, 1),
                                    slicek("k16s", {64, 0, 200, 8, 136}, 0, 70, 136, 3),
                                    slicek("k16bad", {64, 5, 200, 16}, 3, 65, 72, 2),
                                    slicek("k16big", {1024, 512, 72}, 0, 256, 128, 4)};
  run_slicek<AB_F16, 64, 64, 2, 2, 4>(k16);
  run_slicek<AB_F16, 128, 128, 2, 2, 4>(k16);
  run_slicek<AB_F16, 256, 128, 2, 2, 3>(k16);
  // 8-bit operands: K and N multiples of 16
  const std::vector<Problem> p8 = {
      plain("tails8", 200, 144, 256, 0, 0, 1),   plain("t8split", 333, 528, 384, 16, 16, 3),
      plain("tiny8", 1, 16, 16, 0, 0, 1),        plain("big8", 1024, 1024, 1024, 0, 0, 2),
      plain("k8", 65, 32, 1040, 16, 0, 4),       plain("batch8", 50, 272, 256, 0, 16, 1, 2)};
  const std::vector<Problem> g8 = {
      grouped("g8", {0, 1, 300, 0, 0, 127, 129, 5, 0}, 9, 144, 96, 1),
      grouped("g8s", {1562, 1426, 784, 1108, 234, 823, 101, 154}, 0, 512, 256, 2),
      grouped("g8e", {0, 0}, 5, 64, 128, 1)};
  run_plain<AB_I8, 64, 64, 2, 2, 4>(p8);
  run_plain<AB_I8, 128, 128, 2, 2, 4>(p8);
  run_plain<AB_I8, 256, 128, 2, 2, 3>(p8);
  run_plain<AB_I8, 256, 256, 4, 2, 2>(p8);
  run_grouped<AB_I8, 64, 64, 2, 2, 4>(g8);
  run_grouped<AB_I8, 128, 128, 2, 2, 4>(g8);
  run_grouped<AB_I8, 256, 128, 2, 2, 3>(g8);
  run_grouped<AB_I8, 256, 256, 4, 2, 2>(g8);
  run_plain<AB_I8, 128, 128, 2, 2, 2>(p8);
  run_grouped<AB_I8, 128, 128, 2, 2, 2>(g8);
  const std::vector<Problem> k8 = {
      slicek("k8", {336, 208, 32, 80, 16, 512, 912, 1536}, 0, 200, 144, 1),
      slicek("k8s", {336, 208, 32, 80, 16, 512, 912, 1536}, 32, 64, 256, 3),
      slicek("k8e", {0, 0, 48}, 16, 40, 48, 2),
      slicek("k8bad", {48, 24, 64}, 0, 64, 64, 1)};
  run_slicek<AB_I8, 64, 64, 2, 2, 4>(k8);
  run_slicek<AB_I8, 128, 128, 2, 2, 4>(k8);
  run_slicek<AB_I8, 256, 128, 2, 2, 3>(k8);
  run_slicek<AB_I8, 256, 256, 4, 2, 2>(k8);
  // fp8: plain (no scales; their kernels issue no scale DMA) and MX (K a
  // multiple of 128, scales always present)
  run_plain<AB_E4M3, 64, 64, 2, 2, 4>(p8);
  run_plain<AB_E4M3, 128, 128, 2, 2, 4>(p8);
  run_plain<AB_E4M3, 256, 128, 2, 2, 3>(p8);
  run_plain<AB_E4M3, 256, 256, 4, 2, 2>(p8);
  const std::vector<Problem> pmx = {plain("mx", 256, 512, 1024, 0, 0, 1, 1, true),
                                    plain("mxtail", 200, 144, 384, 128, 16, 2, 1, true),
                                    plain("mxsplit", 130, 96, 1024, 0, 0, 3, 1, true),
                                    plain("mx4k", 1024, 2048, 4096, 0, 0, 2, 1, true),
                                    plain("mx2k3", 200, 256, 2048, 0, 0, 3, 1, true),
                                    plain("mx2k4", 72, 128, 2048, 0, 0, 4, 1, true)};
  run_plain<AB_MXE4M3, 64, 64, 2, 2, 4>(pmx);
  run_plain<AB_MXE4M3, 128, 64, 2, 2, 4>(pmx);
  run_plain<AB_MXE4M3, 64, 128, 2, 2, 4>(pmx);
  run_plain<AB_MXE4M3, 128, 64, 4, 2, 4>(pmx);
  run_plain<AB_MXE4M3, 64, 128, 2, 4, 4>(pmx);
  run_plain<AB_MXE4M3, 64, 128, 2, 2, 6>(pmx);
  run_plain<AB_MXE4M3, 128, 64, 2, 2, 6>(pmx);
  run_plain<AB_MXE4M3, 64, 128, 2, 2, 5>(pmx);
  run_plain<AB_E4M3, 128, 64, 2, 2, 4>(p8);
  run_plain<AB_E4M3, 64, 128, 2, 2, 4>(p8);
  run_plain<AB_MXE4M3, 128, 128, 2, 2, 4>(pmx);
  run_plain<AB_MXE4M3, 128, 128, 2, 2, 2>(pmx);
  run_plain<AB_MXE4M3, 256, 128, 2, 2, 3>(pmx);
  run_plain<AB_MXE4M3, 256, 256, 4, 2, 2>(pmx);
  // random shapes on every plain instance of both operand widths and the MX one
  const std::vector<Problem> r16 = random_plain(24, 8, 8, false, 0x9E3779B97F4A7C15ull);
  const std::vector<Problem> r8 = random_plain(24, 16, 16, false, 0xD1B54A32D192ED03ull);
  const std::vector<Problem> rmx = random_plain(16, 16, 128, true, 0x8CB92BA72F3D8DD7ull);
  run_plain<AB_F16, 64, 64, 2, 2, 4>(r16);
  run_plain<AB_F16, 128, 128, 2, 2, 4>(r16);
  run_plain<AB_F16, 128, 128, 2, 2, 2>(r16);
  run_plain<AB_F16, 256, 128, 2, 2, 3>(r16);
  run_plain<AB_F16, 128, 256, 2, 2, 3>(r16);
  run_plain<AB_F16, 128, 192, 2, 2, 3>(r16);
  run_plain<AB_F16, 128, 64, 2, 2, 4>(r16);
  run_plain<AB_F16, 64, 128, 2, 2, 4>(r16);
  run_plain<AB_F16, 256, 256, 4, 2, 2>(r16);
  run_plain<AB_I8, 64, 64, 2, 2, 4>(r8);
  run_plain<AB_I8, 128, 128, 2, 2, 4>(r8);
  run_plain<AB_I8, 128, 128, 2, 2, 2>(r8);
  run_plain<AB_I8, 256, 128, 2, 2, 3>(r8);
  run_plain<AB_I8, 256, 256, 4, 2, 2>(r8);
  run_plain<AB_E4M3, 128, 64, 2, 2, 4>(r8);
  run_plain<AB_E4M3, 64, 128, 2, 2, 4>(r8);
  run_plain<AB_MXE4M3, 64, 64, 2, 2, 4>(rmx);
  run_plain<AB_MXE4M3, 128, 128, 2, 2, 4>(rmx);
  run_plain<AB_MXE4M3, 128, 128, 2, 2, 2>(rmx);
  run_plain<AB_MXE4M3, 256, 128, 2, 2, 3>(rmx);
  run_plain<AB_MXE4M3, 256, 256, 4, 2, 2>(rmx);
  run_plain<AB_MXE4M3, 128, 64, 2, 2, 4>(rmx);
  run_plain<AB_MXE4M3, 64, 128, 2, 2, 4>(rmx);
  if (g_fail) {
    printf("FAILED: %d violations (%lld accesses checked)\n", g_fail, g_checked);
    return 1;
  }
  printf("ALL OK (%lld accesses checked)\n", g_checked);
  return 0;
}
