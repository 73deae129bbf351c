// bst_kernel_dma.hpp -- the fast kernel family: a multi-stage LDS-DMA
// pipeline for gfx950.
//
// Every stage of A (BM x BK, K-contiguous rows of 128 bytes) and of B
// (BK x BN, kept in its natural N-contiguous layout) is copied from global
// memory straight into LDS with 16-byte `buffer_load ... lds` instructions:
// no registers are spent on staging, so STAGES-1 stages can be in flight
// while the MFMAs work on the oldest one (the buffering that "Block Dispatch
// Policies" describes as ping-pong / preload between global memory and the
// on-chip buffers, with the capacity rule stages x tile bytes <= LDS).
// Out-of-range lanes of a buffer load write zeros, which masks every tail
// (rows past the problem or group, K past the slice, columns past N) without
// a branch.  Each lane picks the global 16-byte chunk that lands on its LDS
// slot through an XOR permutation of the chunk index by the row, so the
// MFMA operand reads below spread over the banks.
//
// Operand fetch per 32x32 MFMA: A with ds_read_b128 from the K-contiguous
// rows; B^T with the gfx950 transposing reads ds_read_b64_tr_b16 /
// ds_read_b64_tr_b8, each of which turns a 16-lane group's row-major 4 x 16
// (16-bit) or 8 x 16 (8-bit) patch of B into one K-run of 4 / 8 values per
// lane (lane layout established by an on-device probe).
//
// The MFMA, tail-shape, scheduler and epilogue code is shared with the
// register-staged kernel of bst_device.hpp, which remains the path for
// shapes whose K or N do not fill whole 16-byte chunks.
#pragma once

#include <type_traits>
#include <utility>

#include "bst_device.hpp"

namespace bst {

typedef __attribute__((address_space(3))) uint8_t lds_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) uint32_t lds_u32_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

constexpr uint32_t kOob = 0x80000000u;  // a voffset that fails the buffer range check
constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor word 3: raw 32-bit data

// One LDS array per pipeline stage, so that the compiler's wait-count pass
// sees each stage as a separate object and only waits for the DMA into the
// stage about to be read.
template <int S, int BYTES>
__device__ __forceinline__ lds_t* stage_buf() {
  __shared__ __attribute__((aligned(16))) uint8_t buf[BYTES];
  return (lds_t*)buf;
}

// The ring of A-scale groups (see DmaKernel::SAG): an LDS array of its
// own, apart from the stage buffers.
template <int BYTES>
__device__ __forceinline__ lds_t* sag_buf() {
  __shared__ __attribute__((aligned(16))) uint8_t buf[BYTES];
  return (lds_t*)buf;
}

// Buffer descriptor over [base, base + 2^31): raw (stride 0) 32-bit data.
__device__ __forceinline__ u32x4_t make_desc(const uint8_t* base) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return u32x4_t{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, kOob, (uint32_t)kRsrcWord3};
}

// Global -> LDS copies: lane i writes bytes [lds + 16i, +16) (or [lds + 4i,
// +4)) from base + soff + voff; a lane whose voff fails the descriptor's
// range check writes zeros.  Issued as inline assembly so that the
// compiler does not insert its own conservative wait for these LDS writes
// before every LDS read; the pipeline's explicit vmcnt waits and barriers
// order them instead.
// The descriptor and the scalar offset are wave-uniform by construction;
// readfirstlane states it, so that they always live in scalar registers.
//
// The compiler does not look inside inline assembly for hazards, and it
// often writes these scalar operands (readfirstlane, or a reload of a
// spilled scalar through v_readlane) with a vector instruction right
// before the asm; the hardware needs 5 wait states between a vector-ALU
// write of an SGPR and a vector-memory instruction reading it, and 1
// between a write of M0 and an LDS DMA.  The asm therefore starts with
// s_nop 4 (5 wait states).
__device__ __forceinline__ u32x4_t uniform(const u32x4_t& d) {
  return u32x4_t{(uint32_t)__builtin_amdgcn_readfirstlane(d[0]),
                 (uint32_t)__builtin_amdgcn_readfirstlane(d[1]),
                 (uint32_t)__builtin_amdgcn_readfirstlane(d[2]),
                 (uint32_t)__builtin_amdgcn_readfirstlane(d[3])};
}
__device__ __forceinline__ void dma16(const u32x4_t& desc, const lds_t* lds, uint32_t voff,
                                      uint32_t soff) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "{m0}"((uint32_t)(uintptr_t)lds), "v"(voff), "s"(uniform(desc)),
                 "s"((uint32_t)__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}
__device__ __forceinline__ void dma4(const u32x4_t& desc, const lds_t* lds, uint32_t voff,
                                     uint32_t soff) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "{m0}"((uint32_t)(uintptr_t)lds), "v"(voff), "s"(uniform(desc)),
                 "s"((uint32_t)__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}

// Wait for every outstanding LDS access of this wave (vmcnt and expcnt
// fields at their maxima: no wait on those).
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

// Workgroup barrier that the compiler may not move memory accesses across.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Compile-time loops: f(std::integral_constant<int, i>) for i in [B, E).
template <int B, typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, B + Is>{}), ...);
}
template <int B, int E, typename F>
__device__ __forceinline__ void static_for_range(F&& f) {
  if constexpr (E > B) static_for_impl<B>(f, std::make_integer_sequence<int, E - B>{});
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_range<0, N>(f);
}

// The kernel's argument block, read in place in the kernarg segment (the
// kernels take GemmArgs as their only argument, so it starts there).  Each
// call yields a new pointer, so the loads through it are issued after this
// point: a phase of the kernel (a unit's set-up, its epilogue) loads the
// fields it uses there, together, instead of the compiler loading every
// field at the kernel's start and keeping (spilling) the values across the
// K loop.  The cast back to a generic pointer keeps the constant address
// space visible to the compiler, so the loads stay scalar.
__device__ __forceinline__ const GemmArgs* kernel_args() {
  auto p = (const __attribute__((address_space(4))) GemmArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return (const GemmArgs*)p;
}

// Brings every 64-byte line of the argument block into the scalar cache in
// one round trip (one word of each, combined into an empty asm operand), so
// that the set-up's dependent reads of the arguments hit in it.
__device__ __forceinline__ void warm_args(const GemmArgs* ap) {
  static_assert(sizeof(GemmArgs) <= 6 * 64, "the argument block spans at most six lines");
  const uint32_t* w = (const uint32_t*)ap;
  const uint32_t x = w[0] ^ w[16] ^ w[32] ^ w[48] ^ w[64] ^ w[80];
  asm volatile("" ::"s"(x));
}

// Shader-clock stamp for the BST_TRACE cycle accounting (0 otherwise).
__device__ __forceinline__ uint64_t trace_stamp() {
#ifdef BST_TRACE
  return __builtin_amdgcn_s_memtime();
#else
  return 0;
#endif
}

// Cycle accounting of the K loop (BST_TRACE builds only; empty otherwise):
// time in the wait + barrier at the top of each step, and in the step bodies.
struct LoopTrace {
#ifdef BST_TRACE
  uint64_t wait = 0, body = 0, mark = 0, start = 0, prologue = 0;
#endif
  __device__ __forceinline__ void begin() {
#ifdef BST_TRACE
    start = mark = __builtin_amdgcn_s_memtime();
#endif
  }
  __device__ __forceinline__ void top() {  // before the wait of a step
#ifdef BST_TRACE
    const uint64_t t = __builtin_amdgcn_s_memtime();
    body += t - mark;
    mark = t;
#endif
  }
  __device__ __forceinline__ void released() {  // after the barrier of a step
#ifdef BST_TRACE
    const uint64_t t = __builtin_amdgcn_s_memtime();
    wait += t - mark;
    mark = t;
#endif
  }
  __device__ __forceinline__ void prologue_done() {
#ifdef BST_TRACE
    const uint64_t t = __builtin_amdgcn_s_memtime();
    prologue = t - start;
    mark = t;
#endif
  }
  __device__ __forceinline__ void finish(uint64_t* out) {
#ifdef BST_TRACE
    const uint64_t t = __builtin_amdgcn_s_memtime();
    body += t - mark;
    if (out != nullptr && blockIdx.x == 0 && (threadIdx.x & 63u) == 0) {
      const uint32_t w = threadIdx.x >> 6;
      out[w * 4 + 0] += wait;
      out[w * 4 + 1] += body;
      out[w * 4 + 2] += prologue;
      out[w * 4 + 3] += t - start;
    }
#else
    (void)out;
#endif
  }
};

// Largest power of two (at most 16) dividing n: the size of the aligned
// chunk blocks inside which a B row is permuted.
constexpr int pow2_block(int n) { return (n % 16 == 0) ? 16 : (n % 8 == 0) ? 8 : (n % 4 == 0) ? 4 : (n % 2 == 0) ? 2 : 1; }

template <int AB, int BM, int BN, int WM, int WN, int STAGES, int FORM, bool ADD = false>
struct DmaKernel {
  using T = Traits<AB>;
  using Epi = Epilogue<AB, BM, BN, WM, WN, FORM>;
  static constexpr bool GROUPED = FORM == FORM_SLICE_M;
  using Acc = typename Epi::Acc;
  using Frag = typename std::conditional<T::FRAG_DW == 8, i32x8_t, u32x4_t>::type;
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  static constexpr int ES = T::ES, BK = T::BK, CE = 16 / ES;
  static constexpr int KSTEPS = BK / T::MFMA_K;
  static constexpr int RB = BN * ES;     // bytes of one B row (one K index) in LDS
  static constexpr int NCH = RB / 16;    // 16-byte chunks per B row
  static constexpr uint32_t BSWZ = pow2_block(NCH) - 1;
  static constexpr int A_BYTES = BM * kRowBytes;
  static constexpr int B_BYTES = BK * RB;
  static constexpr int A_IPW = A_BYTES / 1024 / NW;  // 1 KiB DMA instructions per wave
  static constexpr int B_IPW = B_BYTES / 1024 / NW;
  static constexpr int UNR = STAGES;  // steps per loop trip: buffer index stays compile-time
  // A's scales in whole tasks (SAG).  A row's scales lie in one line of
  // memory, 4 bytes per stage, so per-stage loads read a line per row for 4
  // useful bytes.  In four-stage kernels (a trip of four steps holds one
  // group of four stages, so a group starts at a fixed step), whole tasks
  // starting on a group boundary load them a group at a time instead: 16
  // bytes per row (dword-by-4 DMA, 64 rows per instruction) at the group's
  // first stage, into one of two group slots ([row][16 bytes], group g in
  // slot g mod 2); at the group's other stages the A slots load nothing and
  // write zeros to their places in the stage, which these tasks do not
  // read.  The instruction count per stage stays the same.
  static constexpr bool SAG = T::SCALED && STAGES == 4;
  static constexpr int SAG_SLOT = SAG ? BM * 16 : 0;
  static constexpr uint32_t SAG_DUMMY = 2u * SAG_SLOT;  // a dummy kilobyte
  static constexpr int SAG_BYTES = SAG ? 2 * SAG_SLOT + 1024 : 16;
  // MX scales: A as [BM rows][4 bytes] (one dword = the stage's 4 K blocks
  // of a row), B as [4][BN] bytes; dword DMA, 256 bytes per instruction:
  // SA_N instructions for A (64 rows each) and SB_N for B.  They are dealt
  // out as slots, SC_IPW per wave: with A-scale groups A's and B's apart
  // (SCA_IPW A slots per wave, wave w taking A instructions w*SCA_IPW + i,
  // then SCB_IPW B slots), so that a slot's matrix, and with it the
  // instruction form, is fixed at compile time; otherwise together (wave w
  // takes slots w*SC_IPW + i of A's, then B's), which needs fewer slots.  A
  // slot past its instructions issues an all-out-of-range instruction (it
  // writes zeros) into the stage's 256-byte dummy area, so that every wave
  // issues the same count for the vmcnt arithmetic.
  static constexpr int SA_N = T::SCALED ? BM / 64 : 0;
  static constexpr int SB_N = T::SCALED ? BN / 64 : 0;
  static constexpr int SCA_IPW = SAG ? (SA_N + NW - 1) / NW : 0;
  static constexpr int SCB_IPW = SAG ? (SB_N + NW - 1) / NW : 0;
  static constexpr int SC_IPW = SAG ? SCA_IPW + SCB_IPW : (SA_N + SB_N + NW - 1) / NW;
  static constexpr int SA_BYTES = SA_N * 256;
  static constexpr int SB_BYTES = SB_N * 256;
  static constexpr int SD_BYTES = (SAG ? (SCA_IPW * NW > SA_N || SCB_IPW * NW > SB_N)
                                       : SC_IPW * NW > SA_N + SB_N) ? 256 : 0;
  static constexpr int LPS = A_IPW + B_IPW + SC_IPW;  // DMA instructions / wave / stage
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES + SD_BYTES;

  static_assert(STAGES >= 2 && STAGES <= 6, "2..6 stages");
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "whole DMA waves");
  static_assert(!T::SCALED || (BM % 64 == 0 && BN % 64 == 0), "whole 256-byte scale instructions");
  static_assert(LPS * STAGES < 64, "vmcnt holds 6 bits");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "32x32 MFMA sub-tiles");
  static_assert(STAGES * STAGE_BYTES + (SAG ? SAG_BYTES : 0) <=
                    160 * 1024 - (FORM != FORM_DENSE ? (int)sizeof(GroupTable) : 0) - 16,
                "LDS budget");
  // a group slot is rewritten STAGES-1 stages ahead of its group; the group
  // two back must be done with by then
  static_assert(!SAG || STAGES <= 5, "A-scale groups need at most five stages");

  static __host__ __device__ __forceinline__ uint32_t swz_b(uint32_t k) {
    if constexpr (ES == 2)
      return (((k & 1u) * 10u) + (((k >> 1) & 1u) * 4u)) & BSWZ;
    else
      return ((k & 7u) + (k & 1u) * 8u) & BSWZ;
  }

  // Per-task, per-lane DMA addressing (offsets inside the tile panels).
  struct Lanes {
    uint32_t a_off[A_IPW];   // byte offset of the chunk in the A panel (row, chunk)
    uint32_t a_kc[A_IPW];    // K index of the chunk's first element inside the stage
    uint32_t a_ok;           // bit i: the chunk's row is inside the problem / group
    uint32_t b_off[B_IPW];   // byte offset inside one stage of the B panel
    uint32_t b_k[B_IPW];     // K row inside the stage
    uint32_t b_ok;           // bit i: the chunk's columns are inside N
    uint32_t sc_off[SC_IPW > 0 ? SC_IPW : 1];  // scale slots (see sc_slot)
    uint32_t sc_ok;
  };

  struct Ctx {
    const uint8_t* a_tile;   // A panel of the task (first row, K = 0)
    const uint8_t* b_tile;   // B panel of the task (K = 0, first column)
    const uint8_t* sa_tile;  // MX: first scale of the task's first row
    const uint8_t* sb_tile;  // MX: first scale column of the task
    int64_t ldb_bytes, ldsb;
    uint32_t ldb_bytes32, ldsb32;  // the same, known below 2^31 per panel
    uint32_t k0;             // first K index of the task's slice
    uint32_t kend;
    uint32_t kshift, nks;    // ShuffleK: stage j runs K stage (j + kshift) mod nks (nks = ~0: off)
    uint32_t wave;
    Lanes ln;
  };

  // One DMA lane access: enabled, and its byte offset from the panel base of
  // the stage (A: a_tile + kb0*ES, B: b_tile + kb0*ldb*ES, scales: the
  // stage's first scale).  A disabled access gets an offset that fails the
  // buffer range check, so the lane writes zeros.
  struct Access {
    bool ok;
    uint32_t voff;
  };

  // Per-task, per-lane addressing.  Host-callable so that a CPU check can
  // run exactly this code over every lane, wave, stage and task.
  __host__ __device__ __forceinline__ static void lane_setup(Lanes& ln, uint32_t wave, uint32_t lane,
                                             uint32_t rows_valid, uint32_t n_tile, uint32_t N,
                                             int64_t lda, int64_t ldb_bytes, int64_t ldsa,
                                             int64_t ldsb) {
    ln.a_ok = 0;
    for (int i = 0; i < A_IPW; ++i) {
      const uint32_t r = (wave * A_IPW + i) * 8 + (lane >> 3);
      const uint32_t ch = (lane & 7u) ^ swz(r);
      ln.a_off[i] = (uint32_t)((int64_t)r * lda * ES) + ch * 16;
      ln.a_kc[i] = ch * CE;
      if (r < rows_valid) ln.a_ok |= 1u << i;
    }
    ln.b_ok = 0;
    for (int i = 0; i < B_IPW; ++i) {
      const uint32_t byte = (wave * B_IPW + i) * 1024 + lane * 16;
      const uint32_t k = byte / RB;
      const uint32_t ch = ((byte % RB) / 16) ^ swz_b(k);
      ln.b_off[i] = (uint32_t)((int64_t)k * ldb_bytes) + ch * 16;
      ln.b_k[i] = k;
      if (n_tile * BN + ch * CE < N) ln.b_ok |= 1u << i;
    }
    ln.sc_ok = 0;
    for (int i = 0; i < SC_IPW; ++i) {
      const ScSlot sl = sc_slot(wave, i);
      ln.sc_off[i] = kOob;
      if (sl.kind == 0) {
        const uint32_t r = sl.idx * 64 + lane;
        ln.sc_off[i] = (uint32_t)((int64_t)r * ldsa);
        if (r < rows_valid) ln.sc_ok |= 1u << i;
      } else if (sl.kind == 1) {
        const uint32_t byte = sl.idx * 256 + lane * 4;
        const uint32_t e = byte / BN, col = byte % BN;
        ln.sc_off[i] = (uint32_t)((int64_t)e * ldsb) + col;
        if (n_tile * BN + col < N) ln.sc_ok |= 1u << i;
      }
    }
  }

  __host__ __device__ __forceinline__ static Access a_access(const Lanes& ln, int i, uint32_t kb0, uint32_t kend) {
    const bool kfull = kb0 + BK <= kend;
    const bool ok = ((ln.a_ok >> i) & 1u) && (kfull || kb0 + ln.a_kc[i] < kend);
    return Access{ok, ok ? ln.a_off[i] : kOob};
  }
  __host__ __device__ __forceinline__ static Access b_access(const Lanes& ln, int i, uint32_t kb0, uint32_t kend) {
    const bool kfull = kb0 + BK <= kend;
    const bool ok = ((ln.b_ok >> i) & 1u) && (kfull || kb0 + ln.b_k[i] < kend);
    return Access{ok, ok ? ln.b_off[i] : kOob};
  }
  // Scales: this family runs MX only with K a multiple of the stage depth,
  // so a stage inside [0, kend) has all 4 blocks; a padding stage past kend
  // reads none.
  __host__ __device__ __forceinline__ static Access sc_access(const Lanes& ln, int i, uint32_t kb0, uint32_t kend) {
    const bool ok = ((ln.sc_ok >> i) & 1u) && kb0 < kend;
    return Access{ok, ok ? ln.sc_off[i] : kOob};
  }
  // LDS byte offsets, inside a stage, of DMA instruction i of a wave.
  __host__ __device__ __forceinline__ static uint32_t a_lds(uint32_t wave, int i) { return (wave * A_IPW + i) * 1024; }
  __host__ __device__ __forceinline__ static uint32_t b_lds(uint32_t wave, int i) {
    return A_BYTES + (wave * B_IPW + i) * 1024;
  }
  // Scale slot i of a wave: kind 0 = A instruction idx (rows 64*idx ..),
  // 1 = B instruction idx (bytes 256*idx .. of the [4][BN] block), 2 = none;
  // lds: its byte offset inside the stage (for none, the dummy area).
  struct ScSlot {
    int kind;
    uint32_t idx, lds;
  };
  __host__ __device__ __forceinline__ static ScSlot sc_slot(uint32_t wave, int i) {
    constexpr uint32_t dummy = (uint32_t)(A_BYTES + B_BYTES + SA_BYTES + SB_BYTES);
    if (!SAG) {
      const uint32_t x = wave * SC_IPW + (uint32_t)i;
      if (x < (uint32_t)SA_N) return ScSlot{0, x, A_BYTES + B_BYTES + x * 256u};
      if (x < (uint32_t)(SA_N + SB_N))
        return ScSlot{1, x - SA_N, A_BYTES + B_BYTES + SA_BYTES + (x - SA_N) * 256u};
      return ScSlot{2, 0u, dummy};
    }
    if (i < SCA_IPW) {  // an A slot
      const uint32_t x = wave * SCA_IPW + (uint32_t)i;
      return x < (uint32_t)SA_N ? ScSlot{0, x, A_BYTES + B_BYTES + x * 256u} : ScSlot{2, 0u, dummy};
    }
    const uint32_t y = wave * SCB_IPW + (uint32_t)(i - SCA_IPW);
    return y < (uint32_t)SB_N ? ScSlot{1, y, A_BYTES + B_BYTES + SA_BYTES + y * 256u}
                              : ScSlot{2, 0u, dummy};
  }
  // A-scale groups: group slot of the task's stage j, and the LDS offset of
  // A scale instruction idx (rows 64 idx ..) inside a group slot.
  // Host-callable for the CPU check.
  __host__ __device__ __forceinline__ static uint32_t sag_slot(uint32_t j) { return (j >> 2) & 1u; }
  // Whether the stage a prologue issue (stage J) or step I of a trip (stage
  // trip + I + STAGES - 1) sends out starts a group, i.e. carries its load.
  static constexpr bool sag_issue_prologue(int J) { return SAG && J % 4 == 0; }
  static constexpr bool sag_issue_step(int I) { return SAG && (I + STAGES - 1) % 4 == 0; }
  __host__ __device__ __forceinline__ static uint32_t sag_lds(uint32_t idx) { return idx * 1024u; }

  // Per-task DMA state: buffer descriptors over the task's panels and, for
  // a task whose every stage lies inside its K slice (no partial and no
  // padding stage), each instruction's lane offset with the lane's row /
  // column validity folded in (kOob outside).  The K position of a stage
  // reaches the address through the instruction's scalar offset, so a
  // steady-state DMA is an M0 write and the load.  Kernels without block
  // scales have no scale slots.
  struct Dma {
    u32x4_t ra, rb;
    u32x4_t rsc[SC_IPW > 0 ? SC_IPW : 1];   // scale slot i: its matrix's descriptor,
    uint32_t sclds[SC_IPW > 0 ? SC_IPW : 1];  // its byte offset inside a stage,
    uint32_t scb;                             // bit i: slot i reads B's scales
    uint32_t sag[2][SCA_IPW > 0 ? SCA_IPW : 1];  // A slot i: its group destination per slot
    uint32_t vo[LPS];
  };

  // Lane offset of DMA instruction X when the stage is entirely inside the
  // slice (host-callable, so the CPU check compares it with the checked
  // per-stage offsets).
  __host__ __device__ __forceinline__ static uint32_t full_voff(const Lanes& ln, int X) {
    if (X < A_IPW) return ((ln.a_ok >> X) & 1u) ? ln.a_off[X] : kOob;
    if (X < A_IPW + B_IPW) {
      const int i = X - A_IPW;
      return ((ln.b_ok >> i) & 1u) ? ln.b_off[i] : kOob;
    }
    const int i = X - A_IPW - B_IPW;
    return ((ln.sc_ok >> i) & 1u) ? ln.sc_off[i] : kOob;
  }

  template <bool FULL>
  __device__ static __forceinline__ Dma make_dma(const Ctx& c) {
    Dma d;
    d.ra = make_desc(c.a_tile);
    d.rb = make_desc(c.b_tile);
    d.scb = 0;
    if constexpr (T::SCALED) {
      const u32x4_t rsa = make_desc(c.sa_tile), rsb = make_desc(c.sb_tile);
#pragma unroll
      for (int i = 0; i < SC_IPW; ++i) {
        const ScSlot sl = sc_slot(c.wave, i);
        d.rsc[i] = sl.kind == 1 ? rsb : rsa;
        d.sclds[i] = sl.lds;
        if (sl.kind == 1) d.scb |= 1u << i;
        if (i < SCA_IPW) {
          // a padding A slot loads its (all out-of-range) group into the
          // dummy kilobyte
          d.sag[0][i] = sl.kind == 0 ? sag_lds(sl.idx) : SAG_DUMMY;
          d.sag[1][i] = sl.kind == 0 ? SAG_SLOT + sag_lds(sl.idx) : SAG_DUMMY;
        }
      }
    }
    if constexpr (FULL) {
#pragma unroll
      for (int x = 0; x < LPS; ++x) d.vo[x] = full_voff(c.ln, x);
    }
    return d;
  }

  // Scalar byte offsets of the stage at K index kb0 inside each panel.
  struct Soff {
    uint32_t kb0, a, b, sa, sb;
    uint32_t gslot;  // A-scale groups: the stage's group slot
  };
  // K index of the task's stage j.  With ShuffleK (whole-stage tasks only)
  // the stages start at kshift and wrap around; otherwise nks = ~0 and the
  // stages, padding included, run in order.
  __device__ static __forceinline__ uint32_t stage_k(const Ctx& c, uint32_t j) {
    const uint32_t r = j + c.kshift;
    return c.k0 + (r >= c.nks ? r - c.nks : r) * BK;
  }

  __device__ static __forceinline__ Soff stage_soff(const Ctx& c, uint32_t kb0) {
    return Soff{kb0, kb0 * (uint32_t)ES, kb0 * c.ldb_bytes32, kb0 / 32u, (kb0 / 32u) * c.ldsb32,
                0u};
  }
  // The offsets of the task's stage j.
  __device__ static __forceinline__ Soff stage_so(const Ctx& c, uint32_t j) {
    Soff so = stage_soff(c, stage_k(c, j));
    so.gslot = sag_slot(j);
    return so;
  }

  // DMA instruction X (0 <= X < LPS) of this wave for the stage of `so`,
  // into stage buffer S.  GST: whole tasks with A-scale groups, the stage
  // starts a group.
  template <int S, int X, bool FULL, bool GST>
  __device__ static __forceinline__ void dma_one(const Ctx& c, const Dma& d, const Soff& so) {
    lds_t* base = stage_buf<S, STAGE_BYTES>();
    if constexpr (X < A_IPW) {
      const uint32_t v = FULL ? d.vo[X] : a_access(c.ln, X, so.kb0, c.kend).voff;
      dma16(d.ra, base + a_lds(c.wave, X), v, so.a);
    } else if constexpr (X < A_IPW + B_IPW) {
      constexpr int i = X - A_IPW;
      const uint32_t v = FULL ? d.vo[X] : b_access(c.ln, i, so.kb0, c.kend).voff;
      dma16(d.rb, base + b_lds(c.wave, i), v, so.b);
    } else {
      // a scale slot: which matrix is fixed by the slot index, a padding slot
      // differs only in its offsets, so no branch enters the step
      constexpr int i = X - A_IPW - B_IPW;
      const uint32_t v = FULL ? d.vo[X] : sc_access(c.ln, i, so.kb0, c.kend).voff;
      if constexpr (!SAG) {
        dma4(d.rsc[i], base + d.sclds[i], v, ((d.scb >> i) & 1u) ? so.sb : so.sa);
      } else if constexpr (i >= SCA_IPW) {
        dma4(d.rsc[i], base + d.sclds[i], v, so.sb);
      } else if constexpr (!FULL) {
        dma4(d.rsc[i], base + d.sclds[i], v, so.sa);
      } else if constexpr (GST) {
        // the group's 16 bytes of each row, from its first scale
        dma16(d.rsc[i], sag_buf<SAG_BYTES>() + (so.gslot ? d.sag[1][i] : d.sag[0][i]), v,
              so.sa & ~15u);
      } else {
        dma4(d.rsc[i], base + d.sclds[i], kOob, 0u);
      }
    }
  }

  // Enqueue the whole DMA of the task's stage j into stage buffer S.
  template <int S, bool FULL, bool GST>
  __device__ static __forceinline__ void issue(const Ctx& c, const Dma& d, uint32_t j) {
    const Soff so = stage_so(c, j);
    static_for<LPS>([&](auto x) { dma_one<S, decltype(x)::value, FULL, GST>(c, d, so); });
  }

  // MFMA operands of one K step of a wave, held in registers.
  struct KFrag {
    Frag a[FM];
    Frag b[FN];
    uint32_t sa[FM];
    uint32_t sb[FN];
  };

  // LDS -> registers, one operand fragment at a time: A fragment I and B
  // fragment J of K step KK of stage buffer S, with their block scales.
  // The A scales of one stage for the rows of a wave's A fragments, held in
  // registers (whole tasks with A-scale groups): one dword (4 K blocks) each.
  struct Scw {
    uint32_t d[FM];
  };
  // A wave reads a group's 16 bytes for each of its fragment rows from the
  // group slot of stage j: 32 consecutive rows of 16 bytes, conflict-free,
  // once per group instead of a dword per stage and K step (rows 16 bytes
  // apart put 32 lanes' dwords on 8 banks).
  __device__ static __forceinline__ void read_sag(u32x4_t (&sg)[FM], uint32_t j, uint32_t wm) {
    const uint32_t l32 = threadIdx.x & 31u;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      sg[i] = *(const lds_u32x4_t*)(sag_buf<SAG_BYTES>() + sag_slot(j) * SAG_SLOT +
                                    (wm * TM + i * 32 + l32) * 16u);
  }
  __device__ static __forceinline__ Scw scw_of(const u32x4_t (&sg)[FM], int q) {
    Scw w;
#pragma unroll
    for (int i = 0; i < FM; ++i) w.d[i] = sg[i][q];
    return w;
  }

  // w: whole tasks with A-scale groups, the stage's A scales (Scw).
  template <int S, int KK, int I, bool FULL>
  __device__ static __forceinline__ void load_a(KFrag& f, uint32_t wm, const Scw& w) {
    const lds_t* base = stage_buf<S, STAGE_BYTES>();
    const lds_t* la = base;
    const lds_t* lsa = base + A_BYTES + B_BYTES;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t l32 = lane & 31u, hi = lane >> 5;
    const uint32_t row = wm * TM + I * 32 + l32;
    const lds_t* rp = la + row * kRowBytes;
    if constexpr (T::FRAG_DW == 4) {
      f.a[I] = *(const lds_u32x4_t*)(rp + (((2 * KK + hi) ^ swz(row)) << 4));
    } else {
      const u32x4_t x = *(const lds_u32x4_t*)(rp + (((4 * KK + hi) ^ swz(row)) << 4));
      const u32x4_t y = *(const lds_u32x4_t*)(rp + (((4 * KK + 2 + hi) ^ swz(row)) << 4));
      f.a[I] = i32x8_t{(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                       (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
    }
    if constexpr (SAG && FULL)
      f.sa[I] = (w.d[I] >> (8 * (2 * KK + hi))) & 0xffu;
    else if constexpr (T::SCALED)
      f.sa[I] = (*(const lds_u32_t*)(lsa + row * 4) >> (8 * (2 * KK + hi))) & 0xffu;
    else
      f.sa[I] = 0x7fu;  // 2^0 (the scale operand only matters to fp8 MFMAs)
    (void)w;
  }

  template <int S, int KK, int J>
  __device__ static __forceinline__ void load_b(KFrag& f, uint32_t wn) {
    const lds_t* base = stage_buf<S, STAGE_BYTES>();
    const lds_t* lb = base + A_BYTES;
    const lds_t* lsb = base + A_BYTES + B_BYTES + SA_BYTES;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t l32 = lane & 31u, hi = lane >> 5;
    const uint32_t L = lane & 15u, half_group = (lane >> 4) & 1u;
    const uint32_t cbase = wn * TN + J * 32 + 16 * half_group;  // first column of the group
    if constexpr (ES == 2) {
      // two transposing reads: K rows 16kk + 8hi + {0..3} and {4..7}
      const uint32_t colb = (cbase + 4 * (L & 3u)) * 2;
      i16x4_t v[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t k = 16 * KK + 8 * hi + 4 * t + (L >> 2);
        const lds_t* p = lb + k * RB + ((((colb >> 4) ^ swz_b(k))) << 4) + (colb & 8u);
        v[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
      }
      f.b[J] = __builtin_bit_cast(u32x4_t, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3,
                                                                   4, 5, 6, 7));
    } else {
      const uint32_t colb = cbase + 8 * (L & 1u);
      constexpr int NR = T::FRAG_DW / 2;  // 8-byte transposing reads per operand
      i32x2_t v[NR];
#pragma unroll
      for (int t = 0; t < NR; ++t) {
        // int8: K rows 32kk + 16hi + 8t + {0..7}; fp8: the two 16-byte
        // pieces of a lane come from the two halves of the 64-wide step
        const uint32_t k = (NR == 2) ? 32 * KK + 16 * hi + 8 * t + (L >> 1)
                                     : 64 * KK + 32 * (t >> 1) + 16 * hi + 8 * (t & 1) + (L >> 1);
        const lds_t* p = lb + k * RB + ((((colb >> 4) ^ swz_b(k))) << 4) + (colb & 8u);
        v[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)p);
      }
      if constexpr (NR == 2)
        f.b[J] = u32x4_t{(uint32_t)v[0][0], (uint32_t)v[0][1], (uint32_t)v[1][0], (uint32_t)v[1][1]};
      else
        f.b[J] = Frag{v[0][0], v[0][1], v[1][0], v[1][1], v[2][0], v[2][1], v[3][0], v[3][1]};
    }
    if constexpr (T::SCALED)
      f.sb[J] = lsb[(2 * KK + hi) * BN + wn * TN + J * 32 + l32];
    else
      f.sb[J] = 0x7fu;
  }

  // Fragment load X of K step KK: A fragments 0..FM-1, then B fragments 0..FN-1.
  static constexpr int NLK = FM + FN;       // fragment loads per K step
  static constexpr int NMK = FM * FN;       // MFMAs per K step
  static constexpr int NMF = KSTEPS * NMK;  // MFMAs per stage

  template <int S, int KK, int X, bool FULL>
  __device__ static __forceinline__ void load_one(KFrag& f, uint32_t wm, uint32_t wn,
                                                 const Scw& w) {
    if constexpr (X < FM)
      load_a<S, KK, X, FULL>(f, wm, w);
    else
      load_b<S, KK, X - FM>(f, wn);
  }
  template <int S, int KK, bool FULL>
  __device__ static __forceinline__ void load_kstep(KFrag& f, uint32_t wm, uint32_t wn,
                                                   const Scw& w) {
    static_for<NLK>([&](auto x) { load_one<S, KK, decltype(x)::value, FULL>(f, wm, wn, w); });
  }

  // MFMA Q of a K step (A fragment major).
  template <int Q>
  __device__ static __forceinline__ void mfma_one(Acc (&acc)[FM][FN], const KFrag& f) {
    constexpr int I = Q / FN, J = Q % FN;
    mfma32<AB>(acc[I][J], f.b[J], f.a[I], f.sb[J], f.sa[I]);
  }

  // The DMA instructions that MFMA slot Q of a stage carries.  A wave
  // blocks while it issues a DMA instruction and its MFMA pipe drains
  // meanwhile, so each one sits right behind an MFMA instead of in a burst.
  // With 4 or more stages the LPS instructions are dealt out evenly over the
  // NMF slots: the stage issued in step kt must be resident two steps later.
  // With 2 or 3 stages it has only one step's compute to land in (with 3,
  // the ring reads stage kt+2 from the top of step kt+1 on), so its
  // instructions go one per slot from the first.
  static constexpr int DSLOTS = (STAGES <= 3 && LPS < NMF) ? LPS : NMF;
  template <int SD, int Q, bool FULL, bool GST>
  __device__ static __forceinline__ void slot_dma(const Ctx& c, const Dma& d, const Soff& so) {
    if constexpr (Q < DSLOTS)
      static_for_range<(Q * LPS) / DSLOTS, ((Q + 1) * LPS) / DSLOTS>(
          [&](auto x) { dma_one<SD, decltype(x)::value, FULL, GST>(c, d, so); });
  }

  template <int N>
  __device__ static __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  }

  // Two schedules.  Every step runs its MFMAs unconditionally: the stage
  // count is padded up to the unroll (padding stages hold zeros) and the
  // last unroll group is peeled with its DMA and wait pattern fixed at
  // compile time, so the accumulators never pass through a branch and the
  // steady state carries no per-instruction conditions.
  //
  // Ring (3 to 6 stages): the MFMAs of K step g carry the LDS reads of K
  // step g+PD, which may lie in the next stage (resident from the top of
  // the step on), and the step's share of the DMA of stage kt+STAGES-1.
  // PD+1 K steps of operands live in registers, in a ring of sets.
  //
  // K-step (2 stages): the next stage is still in flight during a step, so
  // the reads run inside the stage only: the MFMAs of K step kk carry the
  // reads of K step kk+1.
  static constexpr int RING_K = UNR * KSTEPS;  // K steps per loop trip (ring schedule)
  // The ring's read-ahead: as far as 3 K steps (and never past the next
  // stage), with a set count that divides the K steps of one trip so that
  // every set index is a compile-time constant, and with the accumulators
  // and operand sets together in at most half of a wave's share of the
  // SIMD's 512 registers (the rest holds addresses and DMA offsets; wide
  // MX tiles at read-ahead 2 spilled inside the K loop).
  static constexpr int SET_REGS = (FM + FN) * T::FRAG_DW + (T::SCALED ? FM + FN : 0);
  static constexpr int ring_pd() {
    for (int dd = (KSTEPS < 3 ? KSTEPS : 3); dd > 1; --dd)
      if (RING_K % (dd + 1) == 0 && FM * FN * 16 + (dd + 1) * SET_REGS <= 256 * 4 / NW) return dd;
    return 1;
  }
  static constexpr int PD = ring_pd();
  static constexpr int NSET = PD + 1;
  static_assert(STAGES == 2 || (RING_K % NSET == 0 && PD <= KSTEPS), "ring shape");

  __host__ __device__ __forceinline__ static uint32_t padded_stages(uint32_t nk) {
    return (nk + UNR - 1) / UNR * UNR;
  }
  // A task runs the unchecked DMA offsets when no stage is partial or padding.
  __host__ __device__ __forceinline__ static bool full_task(uint32_t k0, uint32_t k1) {
    const uint32_t nk = (k1 - k0) / BK;
    return (k1 - k0) % BK == 0 && nk % UNR == 0;
  }

  // One step of the ring schedule.  WAITN: outstanding DMA instructions
  // allowed at the top (-1: no wait and no barrier, the task's last step);
  // LAST: skip the reads that would run past the task's last stage.
  template <int I, bool FULL, bool DMA, int WAITN, bool LAST>
  // sgc / sgn (whole tasks with A-scale groups): the current and the next
  // group's A scales of the wave's fragment rows.
  __device__ static __forceinline__ void step_ring(Acc (&acc)[FM][FN], KFrag (&f)[NSET],
                                                   const Ctx& c, const Dma& d, uint32_t kt,
                                                   uint32_t wm, uint32_t wn, LoopTrace& tr,
                                                   u32x4_t (&sgc)[FM], u32x4_t (&sgn)[FM]) {
    constexpr int S = I % STAGES, SD = (S + STAGES - 1) % STAGES;
    // Stage kt+1 resident: own DMA done, then the barrier (which also tells
    // that every wave has finished reading stage kt-1, whose buffer the DMA
    // below refills).
    tr.top();
    if constexpr (WAITN >= 0) {
      wait_vm<WAITN>();
      barrier_lds();
    }
    tr.released();
    const Soff so = stage_so(c, kt + STAGES - 1);
    // whole tasks with A-scale groups: a trip of four steps is one group, so
    // the stage issued here starts a group at a fixed step (I = 1), and
    // stage kt is the group's stage I.  The last step reads the next
    // group's scales (its first stage, kt+1, is resident now).
    constexpr bool GST = FULL && sag_issue_step(I);
    if constexpr (SAG && FULL && I == 3 && !LAST) read_sag(sgn, kt + 1, wm);
    const Scw w0 = (SAG && FULL) ? scw_of(sgc, I % 4) : Scw{};
    const Scw w1 = (SAG && FULL) ? (I < 3 ? scw_of(sgc, (I + 1) % 4) : scw_of(sgn, 0)) : Scw{};
    static_for<NMF>([&](auto q) {
      constexpr int Q = decltype(q)::value;
      constexpr int KK = Q / NMK, R = Q % NMK;
      constexpr int G = I * KSTEPS + KK;  // K step inside the trip
      mfma_one<R>(acc, f[G % NSET]);
      if constexpr (DMA) slot_dma<SD, Q, FULL, GST>(c, d, so);
      constexpr int GL = G + PD;  // the K step whose operands are read now
      if constexpr (!(LAST && GL >= RING_K)) {
        constexpr int SB = (GL / KSTEPS) % STAGES, KL = GL % KSTEPS;
        constexpr bool NEXT = GL / KSTEPS > I;  // the read lies in stage kt+1
        static_for_range<(R * NLK) / NMK, ((R + 1) * NLK) / NMK>([&](auto x) {
          load_one<SB, KL, decltype(x)::value, FULL>(f[GL % NSET], wm, wn, NEXT ? w1 : w0);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (SAG && FULL && I == 3) {
#pragma unroll
      for (int i = 0; i < FM; ++i) sgc[i] = sgn[i];
    }
  }

  template <int I, bool FULL, bool DMA, int WAITN>
  __device__ static __forceinline__ void step_kstep(Acc (&acc)[FM][FN], const Ctx& c,
                                                    const Dma& d, uint32_t kt, uint32_t wm,
                                                    uint32_t wn, LoopTrace& tr) {
    constexpr int S = I % STAGES, SD = (S + STAGES - 1) % STAGES;
    // Issued so far: stages up to kt+STAGES-2.  Stage kt resident.
    tr.top();
    wait_vm<WAITN>();
    barrier_lds();
    tr.released();
    const Soff so = stage_so(c, kt + STAGES - 1);
    constexpr bool GST = SAG && FULL && (I + STAGES - 1) % 4 == 0;
    static_assert(!SAG, "A-scale groups run with the ring schedule");
    const Scw w{};
    KFrag g0, g1;
    load_kstep<S, 0, FULL>(g0, wm, wn, w);
    static_for<NMF>([&](auto q) {
      constexpr int Q = decltype(q)::value;
      constexpr int KK = Q / NMK, R = Q % NMK;
      mfma_one<R>(acc, (KK & 1) ? g1 : g0);
      if constexpr (DMA) slot_dma<SD, Q, FULL, GST>(c, d, so);
      if constexpr (KK + 1 < KSTEPS) {
        static_for_range<(R * NLK) / NMK, ((R + 1) * NLK) / NMK>([&](auto x) {
          load_one<S, KK + 1, decltype(x)::value, FULL>((KK & 1) ? g0 : g1, wm, wn, w);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  // The first stage of a task, into buffer 0, issued ahead of its K loop
  // while the previous task's epilogue runs (which stages through buffer
  // STAGES-1).
  template <bool FULL>
  __device__ static __forceinline__ void preload_stage0(const Ctx& c) {
    const Dma d = make_dma<FULL>(c);
    issue<0, FULL, FULL && sag_issue_prologue(0)>(c, d, 0u);
  }

  // The K loop of one task: nkp (padded, >= UNR) stages from K index c.k0.
  // pre: stage 0 was issued ahead (preload_stage0).  The epilogue stores
  // issued after it count in vmcnt too; the first wait still allows only
  // the stages issued here to stay in flight, so it covers stage 0 (and the
  // stores, in whatever order they complete).
  template <bool FULL>
  __device__ static __forceinline__ void kloop(Acc (&acc)[FM][FN], const Ctx& c, uint32_t nkp,
                                               uint32_t wm, uint32_t wn, uint64_t* trace_out,
                                               bool pre) {
    LoopTrace tr;
    tr.begin();
    const Dma d = make_dma<FULL>(c);
    uint32_t kt = 0;
    if constexpr (STAGES > 2) {
      // stages 0..STAGES-2 in flight, then stage 0 resident
      if (!pre) issue<0, FULL, FULL && sag_issue_prologue(0)>(c, d, 0u);
      static_for_range<1, STAGES - 1>([&](auto i) {
        constexpr int I = decltype(i)::value;
        issue<I, FULL, FULL && sag_issue_prologue(I)>(c, d, (uint32_t)I);
      });
      wait_vm<(STAGES - 2) * LPS>();
      barrier_lds();
      u32x4_t sgc[FM], sgn[FM];  // A-scale groups: the current and the next group's scales
      if constexpr (SAG && FULL) read_sag(sgc, 0u, wm);
      KFrag f[NSET];
      static_for<PD>([&](auto g) {
        constexpr int GG = decltype(g)::value;
        load_kstep<0, GG, FULL>(f[GG], wm, wn, (SAG && FULL) ? scw_of(sgc, 0) : Scw{});
      });
      tr.prologue_done();
      // At the top of step kt the stages up to kt+STAGES-2 have been
      // issued and kt+1 must be resident: STAGES-3 stages may stay in flight.
      constexpr int WSTEADY = (STAGES - 3) * LPS;
      for (; kt + UNR < nkp; kt += UNR) {
        static_for<UNR>([&](auto i) {
          constexpr int I = decltype(i)::value;
          step_ring<I, FULL, true, WSTEADY, false>(acc, f, c, d, kt + I, wm, wn, tr, sgc, sgn);
        });
      }
      // Last group: only its first step has a stage left to issue (the
      // last one), so from its second step on STAGES-2-I stages remain in
      // flight, and the last step waits for nothing.
      static_for<UNR>([&](auto i) {
        constexpr int I = decltype(i)::value;
        constexpr int W = (I == UNR - 1) ? -1 : (I == 0 ? WSTEADY : (STAGES - 2 - I) * LPS);
        step_ring<I, FULL, I == 0, W, I == UNR - 1>(acc, f, c, d, kt + I, wm, wn, tr, sgc, sgn);
      });
    } else {
      if (!pre) issue<0, FULL, SAG && FULL>(c, d, 0u);
      tr.prologue_done();
      constexpr int U = STAGES;
      for (; kt + U < nkp; kt += U) {
        static_for<U>([&](auto i) {
          constexpr int I = decltype(i)::value;
          step_kstep<I, FULL, true, 0>(acc, c, d, kt + I, wm, wn, tr);
        });
      }
      // last trip: every step but the last has a stage left to issue
      static_for<U>([&](auto i) {
        constexpr int I = decltype(i)::value;
        step_kstep<I, FULL, I + 1 < U, 0>(acc, c, d, kt + I, wm, wn, tr);
      });
    }
    // every wave is done with the stage buffers before the next task's
    // prologue refills them
    __builtin_amdgcn_s_waitcnt(0);
    barrier_lds();
    tr.finish(trace_out);
  }

  // One work unit (a K slice of a task) as the persistent loop sees it.
  struct Unit {
    Task tk;
    uint32_t s, t;  // K slice, task
    uint32_t nk;    // stages (0: nothing to load)
    bool whole;     // no partial or padding stage: precomputed DMA offsets
  };

  // Decodes unit u and fills the per-task part of the DMA context.
  __device__ static __forceinline__ void setup_unit(const GemmArgs& a, const GroupTable* gt,
                                                    uint32_t T_tiles, uint32_t u, Unit& un,
                                                    Ctx& c) {
    un.s = GROUPED ? u / T_tiles : a.mc.tiles.div(u);
    un.t = u - un.s * T_tiles;
    if constexpr (FORM == FORM_SLICE_K)
      un.t = __builtin_amdgcn_readfirstlane(slicek_task(a, gt, un.t));
    Task tk = decode_task(a, un.t, BM, BN, GROUPED ? gt : nullptr);
    if constexpr (GROUPED) {
      // the group table lives in LDS: make the task wave-uniform so that
      // the buffer descriptors below stay in scalar registers
      tk.idx = __builtin_amdgcn_readfirstlane(tk.idx);
      tk.m = __builtin_amdgcn_readfirstlane(tk.m);
      tk.n = __builtin_amdgcn_readfirstlane(tk.n);
      tk.mAct = __builtin_amdgcn_readfirstlane(tk.mAct);
      tk.nAct = __builtin_amdgcn_readfirstlane(tk.nAct);
      tk.rows_valid = __builtin_amdgcn_readfirstlane(tk.rows_valid);
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)tk.row0);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)tk.row0 >> 32));
      tk.row0 = (int64_t)(((uint64_t)hi << 32) | lo);
    }
    // the task's K range: all of K, or its slice-K group's
    uint32_t kq = 0, kg = a.K, ks = a.kslice;
    if constexpr (FORM == FORM_SLICE_K) {
      kq = __builtin_amdgcn_readfirstlane((uint32_t)gt->first_row[tk.idx]);
      kg = __builtin_amdgcn_readfirstlane((uint32_t)gt->first_row[tk.idx + 1]) - kq;
      ks = group_kslice(kg, a.split, BK);
      // A's 16-byte chunks must not straddle a group boundary: a group
      // that does not start and end on one is not computed, its output
      // reads NaN (INT32_MIN for raw accumulators)
      tk.poison = ((kq | kg) % (uint32_t)CE) != 0u;
    }
    const KRange kr = slice_range(kq, kg, ks, un.s);
    const uint32_t k0 = kr.k0, k1 = kr.k1;
    un.nk = (k0 < k1 && !tk.poison) ? (k1 - k0 + BK - 1) / BK : 0u;
    const int64_t bidx = FORM == FORM_DENSE ? tk.idx : 0;
    const int64_t bsel = FORM == FORM_SLICE_K ? 0 : tk.idx;
    c.a_tile = a.A + (bidx * a.strideA + tk.row0 * a.lda) * ES;
    c.b_tile = a.B + (bsel * a.strideB + (int64_t)tk.n * BN) * ES;
    c.sa_tile = T::SCALED ? a.sa + tk.row0 * a.ldsa : nullptr;
    c.sb_tile = T::SCALED ? a.sb + (int64_t)tk.n * BN : nullptr;
    c.k0 = k0;
    c.kend = k1;
    // kernels with A-scale groups run whole tasks only from a group
    // boundary (their stage count is a whole number of groups already)
    un.whole = un.nk > 0 && full_task(k0, k1) && (!SAG || (k0 / BK) % 4u == 0u);
    // ShuffleK: tasks of the launch's full stage count S start at stage t mod
    // S (with A-scale groups: rounded down to a group boundary)
    const bool shuffle = a.shuffle_k != 0 && un.whole && un.nk == a.mc.nk_full.d;
    c.kshift = shuffle ? un.t - a.mc.nk_full.div(un.t) * un.nk : 0u;
    if constexpr (SAG) c.kshift &= ~3u;
    c.nks = shuffle ? un.nk : 0xFFFFFFFFu;
    lane_setup(c.ln, c.wave, fresh_v(threadIdx.x & 63u), tk.rows_valid, tk.n, a.N, a.lda,
               c.ldb_bytes, a.ldsa, a.ldsb);
    un.tk = tk;
  }

  // Dynamic task allocation ("Block Scheduler Code Explained", s1, names it
  // among the scheduler's policies): the first round of units, one per
  // workgroup, is assigned as in the static stride; the rest are split into
  // eight contiguous ranges, one queue per XCD.  A workgroup takes tickets
  // (device-scope atomic increments of its queue's counter) from the queue
  // of the XCD it runs on, then from the others in turn, so the work of a
  // slow or short-staffed XCD is taken over.  Only the order in which
  // workgroups meet the units changes: each unit computes exactly what it
  // computes under the static stride.  Thread 0 of a workgroup holds its
  // queue and ticket.  Vector-memory operations are counted in issue order,
  // so an atomic in flight holds back every later wait: a ticket requested
  // before the K loop would delay the stage loads, one requested right after
  // it the fix-up and the dequant scale loads, and one used right after the
  // epilogue would wait for its stores.  Tickets are therefore taken one
  // unit ahead: requested in a unit's epilogue, once the scale loads are out,
  // and used after the next unit's K loop (by which time it has long
  // returned) to decide the unit after that.
  //
  // Counter area: one counter per 128-byte line (device-scope atomics on
  // one line are served one at a time): lines 0-7 the queues, line 8 the
  // count of exit groups done, lines 9.. one exit count per group of at
  // least 32 workgroups (counting all exits on one word would serialise
  // every workgroup's exit).  The last workgroup of each group bumps line
  // 8, and the last group's last workgroup sets every counter back to zero
  // for the next call in stream order.
  struct Queues {
    uint32_t first, count;  // dynamic units: [first, first + count)
    __device__ __forceinline__ uint32_t lo(uint32_t x) const {
      return first + x * (count / kNumXcd) + (x < count % kNumXcd ? x : count % kNumXcd);
    }
    __device__ __forceinline__ uint32_t len(uint32_t x) const {
      return count / kNumXcd + (x < count % kNumXcd ? 1u : 0u);
    }
  };
  static constexpr uint32_t kNoUnit = 0xFFFFFFFFu;
  static constexpr uint32_t kLine = 32;  // uint32 words per 128-byte line
  static constexpr uint32_t kGroupsDone = 8 * kLine, kGroupBase = 9 * kLine, kMaxExitGroups = 48;

  // Thread 0: the unit the held ticket of queue q stands for, or the next
  // queue's, ...; kNoUnit once every queue is spent.  q is left on the queue
  // the unit came from.
  __device__ static __forceinline__ uint32_t take(const GemmArgs& a, const Queues& Q, uint32_t& q,
                                                  uint32_t ticket) {
    for (uint32_t tries = 0;; ++tries) {
      if (ticket < Q.len(q)) return Q.lo(q) + ticket;
      if (tries + 1 == (uint32_t)kNumXcd) return kNoUnit;
      q = (q + 1) % kNumXcd;
      ticket = __hip_atomic_fetch_add(&a.queue[q * kLine], 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // Thread 0, once its workgroup has no unit left: the exit count, and the
  // reset by the last workgroup out.
  __device__ static __forceinline__ void queue_exit(const GemmArgs& a) {
    const uint32_t G = a.grid;
    uint32_t gsz = (G + kMaxExitGroups - 1) / kMaxExitGroups;
    if (gsz < 32u) gsz = 32u;
    const uint32_t ngroups = (G + gsz - 1) / gsz;
    const uint32_t grp = blockIdx.x / gsz;
    const uint32_t members = (grp + 1 == ngroups) ? G - grp * gsz : gsz;
    const uint32_t in_grp = __hip_atomic_fetch_add(&a.queue[kGroupBase + grp * kLine], 1u,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (in_grp + 1 != members) return;
    const uint32_t done = __hip_atomic_fetch_add(&a.queue[kGroupsDone], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (done + 1 != ngroups) return;
    for (uint32_t x = 0; x < (uint32_t)kNumXcd; ++x)
      __hip_atomic_store(&a.queue[x * kLine], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.queue[kGroupsDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (uint32_t g = 0; g < ngroups; ++g)
      __hip_atomic_store(&a.queue[kGroupBase + g * kLine], 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }

  // Grouped slice-M kernels keep the compiler's own argument handling (all
  // loaded at the start): reading them per phase raised their vector
  // register use past the budget of the two-workgroup and 256x256 builds.
  static constexpr bool kPhaseArgs = FORM != FORM_SLICE_M;

  __device__ __attribute__((always_inline)) static void run(const GemmArgs& a0) {
    const GemmArgs* ap = kPhaseArgs ? kernel_args() : &a0;
    uint64_t t_start = trace_stamp();
    if constexpr (kPhaseArgs) warm_args(ap);
    ClockMark clk;
    clk.start(*ap);
#ifdef BST_TRACE
    const uint64_t clk_ref0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t clk_sh0 = t_start;
#endif
    GroupTable* gt = nullptr;
    uint32_t T_tiles = ap->tiles;
    if constexpr (FORM != FORM_DENSE) {
      __shared__ GroupTable gtab;
      gt = &gtab;
      if constexpr (FORM == FORM_SLICE_M) {
        build_group_table(gtab, *ap, BM, (ap->N + BN - 1) / BN);
        T_tiles = gtab.first_task[ap->G];
      } else {
        build_k_table(gtab, *ap);
      }
    }
    const uint32_t units = T_tiles * ap->split;
    Ctx c;
    c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    c.ldb_bytes = ap->ldb * ES;
    c.ldsb = ap->ldsb;
    c.ldb_bytes32 = (uint32_t)c.ldb_bytes;
    c.ldsb32 = (uint32_t)ap->ldsb;
    const uint32_t wm = c.wave / WN, wn = c.wave % WN;
    // dynamic allocation, when there are units past the first round
    const Queues Q{ap->grid, units > ap->grid ? units - ap->grid : 0u};
    const bool dyn = ap->queue != nullptr && Q.count > 0;
    const bool preload = !dyn && ap->preload != 0;
    uint32_t q = xcc_id(), ticket = 0;  // thread 0's queue and held ticket
    bool held = false;                  // thread 0: a ticket was requested ahead
    uint32_t decided = kNoUnit;         // thread 0: the unit after the current one
    // thread 0 publishes the next unit here, alternating slots, so that a
    // slot is rewritten only after a later barrier that every wave passed
    // after reading it
    __shared__ uint32_t next_unit[2];
    uint32_t round = 0;

    // The host launches at most one workgroup per unit, so a plain launch's
    // first unit exists (a grouped launch learns its unit count here).
    uint32_t u = logical_wg(ap->remap, ap->grid);
    bool have = !GROUPED || u < units;
    bool pre = false;  // the unit's first stages were issued ahead
    Unit un;
    if (have) setup_unit(*ap, gt, T_tiles, u, un, c);
    while (have) {
      const uint64_t t_loop = trace_stamp();
      Acc acc[FM][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;
      if (un.nk > 0) {
        if (un.whole)
          kloop<true>(acc, c, padded_stages(un.nk), wm, wn, ap->trace, pre);
        else
          kloop<false>(acc, c, padded_stages(un.nk), wm, wn, ap->trace, pre);
      }
      const uint64_t t_epi = trace_stamp();
      if constexpr (kPhaseArgs) ap = kernel_args();
      // dynamic allocation: the unit after this one comes from the ticket
      // requested during the previous unit's epilogue, complete by now (this
      // unit's K loop waited for every load issued after it); the first
      // unit's ticket is requested here
      if (dyn && threadIdx.x == 0) {
        if (!held)
          ticket = __hip_atomic_fetch_add(&ap->queue[q * kLine], 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        decided = take(*ap, Q, q, ticket);
        next_unit[round & 1u] = decided;
        held = false;
      }
      const bool last = Epi::fixup(*ap, acc, un.s, un.t);
      const uint64_t t_fix = trace_stamp();
      // static stride: the next unit is known now, and with preload its
      // first stage goes out before this unit's epilogue, whose staging
      // uses a buffer the stage does not.  Only the unit index is kept across
      // the epilogue (its set-up is redone after it), so that the
      // epilogue's registers stay its own.
      uint32_t nu = dyn ? kNoUnit : u + ap->grid;
      pre = false;
      if (preload && nu < units) {
        Unit nx;
        Ctx cn = c;
        setup_unit(*ap, gt, T_tiles, nu, nx, cn);
        if (nx.nk > 0) {
          if (nx.whole)
            preload_stage0<true>(cn);
          else
            preload_stage0<false>(cn);
          pre = true;
        }
      }
      // dynamic allocation: the ticket for the unit after the next is
      // requested once the epilogue's scale loads are out (its latency then
      // overlaps the stores and the next K loop), or here when this slice
      // stores nothing; none once the queues are spent
      auto request = [&]() {
        if (dyn && threadIdx.x == 0 && decided != kNoUnit) {
          ticket = __hip_atomic_fetch_add(&ap->queue[q * kLine], 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
          held = true;
        }
      };
      if (last)
        Epi::template store_tile<STAGE_BYTES, ADD>(*ap, un.tk, acc, wm, wn,
                                                   stage_buf<STAGES - 1, STAGE_BYTES>(), request);
      else
        request();
      if (dyn) {
        __syncthreads();
        nu = __builtin_amdgcn_readfirstlane(next_unit[round & 1u]);
        ++round;
      }
      have = nu < units;
#ifdef BST_TRACE
      {
        const uint64_t t_end = trace_stamp();
        __builtin_amdgcn_s_waitcnt(0);
        const uint64_t t_done = trace_stamp();
        if (ap->trace != nullptr && blockIdx.x == 0 && (threadIdx.x & 63u) == 0) {
          uint64_t* o = ap->trace + 32 + (threadIdx.x >> 6) * 4;
          o[0] += t_loop - t_start;  // unit set-up (first unit: from kernel start)
          o[1] += t_epi - t_loop;    // K loop
          o[2] += t_end - t_epi;     // fix-up, preload, epilogue, next ticket
          o[3] += 1;                 // units
          uint64_t* r = ap->trace + 64 + (threadIdx.x >> 6) * 4;
          r[0] += t_fix - t_epi;     // fix-up
          r[1] += t_end - t_fix;     // preload, stores issued, next ticket
          r[2] += t_done - t_end;    // stores complete
        }
      }
#else
      (void)t_loop;
      (void)t_epi;
      (void)t_fix;
#endif
      if (have) {
        setup_unit(*ap, gt, T_tiles, nu, un, c);
        u = nu;
      }
      t_start = trace_stamp();
    }
    if (dyn && threadIdx.x == 0) queue_exit(*ap);
    clk.stop(*ap);
#ifdef BST_TRACE
    // Clock record of the first 256 workgroups at trace[128 + 4 w]: the
    // 100 MHz reference counter at the start and at the end, and the shader
    // cycles in between, so shader cycles / reference ticks gives the shader
    // clock the workgroup ran at.
    if (ap->trace != nullptr && threadIdx.x == 0 && blockIdx.x < 256) {
      __builtin_amdgcn_s_waitcnt(0);
      const uint64_t sh1 = __builtin_amdgcn_s_memtime();
      const uint64_t ref1 = __builtin_amdgcn_s_memrealtime();
      uint64_t* o = ap->trace + 128 + 4 * blockIdx.x;
      o[0] = clk_ref0;
      o[1] = ref1;
      o[2] = sh1 - clk_sh0;
      o[3] = 1;
    }
#endif
  }
};

// ADD: the matmul-add instances (C = A.B + X; plain GEMM only).
template <int AB, int BM, int BN, int WM, int WN, int STAGES, int FORM, bool ADD = false>
__global__ void __launch_bounds__(64 * WM * WN) gemm_dma_kernel(GemmArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses gfx950-only builtins: device pass only
  DmaKernel<AB, BM, BN, WM, WN, STAGES, FORM, ADD>::run(a);
#endif
}

// The same kernel built for two resident workgroups per CU: its waves may
// use at most half of a SIMD's registers (256 per lane, so two waves share
// each SIMD), and its instances take two pipeline stages, so two
// workgroups' LDS fits in one CU.  While one workgroup stores a tile or sets
// up its next one, the other's K loop keeps the CU's loads and matrix cores
// busy; the host sizes the persistent grid from the occupancy the runtime
// reports.
template <int AB, int BM, int BN, int WM, int WN, int STAGES, int FORM>
__global__ void __launch_bounds__(64 * WM * WN)
    __attribute__((amdgpu_waves_per_eu(2 * WM * WN / 4))) gemm_dma_kernel_pair(GemmArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  DmaKernel<AB, BM, BN, WM, WN, STAGES, FORM, false>::run(a);
#endif
}

}  // namespace bst
