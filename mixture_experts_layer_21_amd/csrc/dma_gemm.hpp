// Building blocks of the direct-to-LDS bf16 MFMA GEMM main loop on gfx950,
// shared by the forward's large-tile grouped GEMM and the backward's GEMMs.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace dma {

// Threads that take part in a block's tile scan.
constexpr int kScanThreads = 256;

// ---------------------------------------------------------------------------
// Large-tile bf16 kernel: 512 threads (8 waves, two per SIMD), operands moved
// global -> LDS by buffer_load ... lds (no register staging), an S-stage LDS
// ring (loads for k-step kt+S-1 are in flight while kt is multiplied), and
// MFMA fragments double-buffered in registers.
//
// Each 1 KB wave load fills 64 consecutive 16-byte LDS slots (slot = base +
// lane*16); the lane fetches the global chunk that the swizzled layout puts in
// that slot, so the fragment reads stay bank-conflict free.  Every stage lives
// in its own LDS array and stage indices are compile-time constants, so the
// wait for stage kt is an exact vmcnt and later stages stay in flight.

typedef __attribute__((address_space(3))) void lds_void_t;


// Swizzle of 16-byte chunk c in row r for KCH chunks per row.  The LDS serves
// a 16-byte read for 16 lanes per cycle (64 four-byte banks); these XOR
// patterns keep the 32-row fragment reads conflict-free, as measured with
// SQ_LDS_BANK_CONFLICT on gfx950 (plain layouts conflict 5-12x per read).
template <int KCH>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (KCH == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return (r >> 2) & 3;
}

// s_waitcnt with only the vector-memory counter limited to n (gfx9 encoding:
// vmcnt[3:0] | expcnt << 4 | lgkmcnt << 8 | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the release fence of __syncthreads(): the fence
// would wait for every load in flight, including later stages.  The wave's
// own stage is already complete (wait_vmcnt), LDS reads of the previous stage
// have returned (their MFMAs consumed them), and the empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int BM, int BNB, int BK_, int S_, int WGM, int NWV, bool GATEUP>
struct DmaCfg {
  static constexpr int NT = 64 * NWV, NW = NWV, WGN = NW / WGM;
  static constexpr int BK = BK_, KCH = BK / 8, S = S_;
  static constexpr int A_LD = BM * KCH / 64 / NW;   // 1 KB wave loads per stage
  static constexpr int B_LD = BNB * KCH / 64 / NW;
  static constexpr int LPS = A_LD + B_LD;            // loads per thread per stage
  static constexpr int WM = BM / WGM;
  static constexpr int NB = GATEUP ? 2 : 1;
  static constexpr int BN = BNB / NB;                // output columns of the tile
  static constexpr int WN = BN / WGN;                // output columns per wave
  static constexpr int MI = WM / 32, NI = WN / 32;
  static_assert(A_LD >= 1 && B_LD >= 1 && MI >= 1 && NI >= 1, "tile shape");
  static_assert(BM * KCH % (64 * NW) == 0 && BNB * KCH % (64 * NW) == 0, "tile shape");
  static_assert(S_ >= 2 && S_ <= 4 && (S_ - 2) * LPS < 64, "stages");
  static_assert(NT >= kScanThreads, "the tile decode scans the expert offsets with 256 threads");
};

template <class C, bool GATEUP>
struct DmaLoads {
  __amdgpu_buffer_rsrc_t rA, rG, rU;
  const uint32_t* a_off;
  const uint32_t* b_off;
  int wave;
  // k-major B only: bytes per k row, and the k from which rows come from rU
  uint32_t b_kbytes;
  int k_split;
  // k-major A only: bytes per k row
  uint32_t a_kbytes;
};

// One wave load (1 KB) of the B tile of k-step kt into stage buffer sb, with
// cache policy BCPOL (a template parameter of the caller): 0, or 2 for
// non-temporal (streaming) loads of a B slice that no other block reads.
// K-contiguous B (BTR false): 16-byte chunks along k of BNB rows, GATEUP
// taking the second half of the rows from rU.  k-major B (BTR true, "B
// transposed": row k holds the N columns): BK rows of BNB columns, the rows
// at and past k_split from rU; the k advance goes into the lane offset, so
// the resource's range check sees it (rows past the range read as zeros).
#define MOE_DMA_B(C, GATEUP, BTR, ld, sb, kt, i)                                             \
  do {                                                                                      \
    const int blk_ = (ld).wave + C::NW * (i);                                               \
    if constexpr (BTR) {                                                                    \
      const int k_ = (kt) * C::BK;                                                          \
      const bool hi_ = k_ >= (ld).k_split;                                                  \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                             \
          hi_ ? (ld).rU : (ld).rG, (lds_void_t*)((sb) + blk_ * 512), 16,                    \
          (ld).b_off[i] + (uint32_t)(hi_ ? k_ - (ld).k_split : k_) * (ld).b_kbytes, 0, 0,    \
          BCPOL);                                                                           \
    } else {                                                                                \
      const bool up_ = (GATEUP) && blk_ * 64 >= C::BN * C::KCH;                             \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(up_ ? (ld).rU : (ld).rG,                     \
                                               (lds_void_t*)((sb) + blk_ * 512), 16,        \
                                               (ld).b_off[i], (kt) * C::BK * 2, 0, BCPOL);  \
    }                                                                                       \
  } while (0)

// Issue all LPS global -> LDS loads (A loads first, then B) of k-step kt into
// one stage's buffers.  (A macro: the host pass of hipcc rejects this body as
// a device function template called from the k-loop.)
// One wave load of the A tile: k-contiguous (ATR false) or k-major (BK rows
// of BM columns, the k advance in the lane offset as for B).
#define MOE_DMA_A(C, ATR, ld, sa, kt, i)                                                     \
  do {                                                                                      \
    if constexpr (ATR)                                                                      \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                             \
          (ld).rA, (lds_void_t*)((sa) + ((ld).wave + C::NW * (i)) * 512), 16,               \
          (ld).a_off[i] + (uint32_t)((kt) * C::BK) * (ld).a_kbytes, 0, 0, 0);                \
    else                                                                                    \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                             \
          (ld).rA, (lds_void_t*)((sa) + ((ld).wave + C::NW * (i)) * 512), 16,               \
          (ld).a_off[i], (kt) * C::BK * 2, 0, 0);                                           \
  } while (0)

#define MOE_DMA_ISSUE(C, GATEUP, ATR, BTR, ld, sa, sb, kt)                                   \
  do {                                                                                      \
    _Pragma("unroll") for (int i_ = 0; i_ < C::A_LD; ++i_)                                  \
        MOE_DMA_A(C, ATR, ld, sa, kt, i_);                                                  \
    _Pragma("unroll") for (int i_ = 0; i_ < C::B_LD; ++i_)                                  \
        MOE_DMA_B(C, GATEUP, BTR, ld, sb, kt, i_);                                          \
  } while (0)

// Multiply one stage (BK/16 k-steps of MI x NB*NI 32x32x16 MFMAs per wave)
// after issuing the loads of a later k-step into another stage's buffers
// (spreading them over the k-steps measured slower on gfx950).
template <class C, bool PARTIAL>
__device__ __forceinline__ void dma_mfmas(const bf16x8 (&af)[C::MI], const bf16x8 (&bfr)[C::NB][C::NI],
                                          f32x16 (&acc)[C::NB][C::MI][C::NI], int mi_n) {
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi) {
        if (PARTIAL && mi >= mi_n) continue;
        acc[nb][mi][ni] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[nb][ni], acc[nb][mi][ni], 0, 0, 0);
      }
}

// s_waitcnt lgkmcnt(0) with the other counters left open.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));
}

// With MOE_DEFER the MFMAs of a stage's last k16 step run after the next
// stage's barrier (their fragments are already in registers), so they cover
// the latency of the next stage's first fragment reads.
#ifndef MOE_DEFER
#define MOE_DEFER 1
#endif

// Two ds_read_b64_tr_b16 give one MFMA operand fragment (8 consecutive k of
// one column) from a k-major tile whose rows hold `cols` bf16 with 16-byte
// chunk c of row k at c ^ 4*(k%4): in each group of 16 lanes, lane 4j+q
// points at row k0+j, columns n0+4q..n0+4q+3, and lane i receives rows
// k0..k0+3 of column n0+i, the first or second half of its 8 k values.
template <int COLS>
__device__ __forceinline__ bf16x8 tr_fragment(const uint16_t* tile, int kk, int col0, int lr,
                                              int lk) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef short v8s __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const int j = (lr >> 2) & 3, q = lr & 3;
  const int row = kk * 16 + 8 * lk + j;  // + 4 for the second read
  const int col = col0 + 16 * ((lr >> 4) & 1) + 4 * q;
  const int byte = row * (COLS * 2) + (((col >> 3) ^ (4 * j)) << 4) + ((q & 1) << 3);
  const char* base = reinterpret_cast<const char*>(tile);
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + byte));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + byte + 4 * COLS * 2));
  const v8s v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

template <class C, bool GATEUP, bool PARTIAL, bool BTR, bool ATR = false, int BCPOL = 0>
__device__ __forceinline__ void dma_compute(const uint16_t* sa, const uint16_t* sb, int wm,
                                            int wn, int lr, int lk,
                                            f32x16 (&acc)[C::NB][C::MI][C::NI],
                                            const DmaLoads<C, GATEUP>& ld, uint16_t* na,
                                            uint16_t* nb_, int kt_next, int mi_n,
                                            bf16x8 (&af)[2][C::MI],
                                            bf16x8 (&bfr)[2][C::NB][C::NI]) {
  constexpr int BK = C::BK, KCH = C::KCH, KS = BK / 16;
  static_assert(KS % 2 == 0, "the deferred k16 step uses fragment buffer 1");
  constexpr int NRD = C::MI + C::NB * C::NI;          // fragment reads per k16 step
  constexpr int NMF = C::MI * C::NB * C::NI;          // MFMAs per k16 step
  static_assert(NMF >= 4, "the scheduling hint places four MFMAs ahead of the reads");
  constexpr int NLD = C::LPS;                         // all loads before the first k16 step
  auto frags = [&](int kk, int buf) {
    const int ch = kk * 2 + lk;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
      if (PARTIAL && mi >= mi_n) continue;
      if constexpr (ATR) {
        af[buf][mi] = tr_fragment<C::WM * (C::NW / C::WGN)>(sa, kk, wm * C::WM + mi * 32,
                                                                 lr, lk);
      } else {
        const int r = wm * C::WM + mi * 32 + lr;
        af[buf][mi] = *reinterpret_cast<const bf16x8*>(sa + r * BK + (ch ^ swz_k<KCH>(r)) * 8);
      }
    }
    if (PARTIAL && mi_n == 0) return;
    if constexpr (BTR) {
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni)
          bfr[buf][nb][ni] =
              tr_fragment<C::NB * C::BN>(sb, kk, nb * C::BN + wn * C::WN + ni * 32, lr, lk);
    } else {
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni) {
          const int r = nb * C::BN + wn * C::WN + ni * 32 + lr;
          bfr[buf][nb][ni] =
              *reinterpret_cast<const bf16x8*>(sb + r * BK + (ch ^ swz_k<KCH>(r)) * 8);
        }
    }
  };
  frags(0, 0);
  if (MOE_DEFER) dma_mfmas<C, PARTIAL>(af[1], bfr[1], acc, mi_n);
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    constexpr int LPS = C::LPS;
    const int i1 = (kk + 1) * NLD < LPS ? (kk + 1) * NLD : LPS;
    {  // loads [kk*NLD, i1) of k-step kt_next (A loads first, then B)
      const int i0 = kk * NLD;
#pragma unroll
      for (int i = 0; i < C::A_LD; ++i)
        if (i >= i0 && i < i1) MOE_DMA_A(C, ATR, ld, na, kt_next, i);
#pragma unroll
      for (int i = 0; i < C::B_LD; ++i) {
        if (C::A_LD + i < i0 || C::A_LD + i >= i1) continue;
        MOE_DMA_B(C, GATEUP, BTR, ld, nb_, kt_next, i);
      }
    }
    // Fragments of the next k16 step are read while this step's MFMAs run.
    if (kk + 1 < KS) frags(kk + 1, (kk + 1) & 1);
    if (MOE_DEFER && kk + 1 == KS) {
      wait_lgkmcnt0();  // the deferred fragments are in registers before the barrier
      continue;
    }
    dma_mfmas<C, PARTIAL>(af[kk & 1], bfr[kk & 1], acc, mi_n);
    if (PARTIAL) continue;  // no fixed instruction pattern to schedule
    // Scheduling hint: four MFMAs, then all fragment reads of the next k16
    // step, then the remaining MFMAs (on the 256x256 tile: 2-3% ahead of a
    // 1:1 interleave, 10% ahead of no hint, ~1% ahead of two MFMAs first).
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    if (kk + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NMF - 4, 0);
  }
}

// The pipelined k-loop.  The stage buffers come in as __restrict__ pointers:
// once this is inlined, every LDS access and every LDS-bound load carries
// scoped no-alias information, so the compiler's own wait before a fragment
// read covers only the load into that same buffer (issued S-1 stages earlier)
// instead of every load in flight.
template <class C, bool GATEUP, bool PARTIAL, bool BTR = false, bool ATR = false,
          int BCPOL = 0>
__device__ __forceinline__ void dma_mainloop(
    const DmaLoads<C, GATEUP>& ld, int nk, int mi_n, int wm, int wn, int lr, int lk,
    f32x16 (&acc)[C::NB][C::MI][C::NI], uint16_t* __restrict__ a0, uint16_t* __restrict__ a1,
    uint16_t* __restrict__ a2, uint16_t* __restrict__ a3, uint16_t* __restrict__ b0,
    uint16_t* __restrict__ b1, uint16_t* __restrict__ b2, uint16_t* __restrict__ b3) {
  constexpr int S = C::S;
  // Fragment buffers; buffer 1 starts at zero so that the first stage's
  // deferred MFMAs add nothing.
  bf16x8 af[2][C::MI], bfr[2][C::NB][C::NI];
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi) af[1][mi] = bf16x8{};
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni) bfr[1][nb][ni] = bf16x8{};
  // Prologue: stages 0 .. S-2 in flight.
  MOE_DMA_ISSUE(C, GATEUP, ATR, BTR, ld, a0, b0, 0);
  if (S > 2) MOE_DMA_ISSUE(C, GATEUP, ATR, BTR, ld, a1, b1, min(1, nk - 1));
  if (S > 3) MOE_DMA_ISSUE(C, GATEUP, ATR, BTR, ld, a2, b2, min(2, nk - 1));

  // Every step issues one stage of loads, so exactly S-2 stages are in flight
  // behind the one being waited for.  Past the end the loads repeat the last
  // k-step into a buffer nobody reads again, and steps past the end skip the
  // multiply; keeping the issue unconditional keeps the compiler's view of
  // the in-flight LDS writes precise.
#define MOE_SA(i) ((i) == 0 ? a0 : (i) == 1 ? a1 : (i) == 2 ? a2 : a3)
#define MOE_SB(i) ((i) == 0 ? b0 : (i) == 1 ? b1 : (i) == 2 ? b2 : b3)
#define MOE_STEP(SI)                                                                        \
  if constexpr (SI < S) {                                                                   \
    const int kt = kb + SI;                                                                 \
    wait_vmcnt<(S - 2) * C::LPS>();                                                         \
    stage_barrier();                                                                        \
    if (kt < nk)                                                                            \
      dma_compute<C, GATEUP, PARTIAL, BTR, ATR, BCPOL>(MOE_SA(SI), MOE_SB(SI), wm, wn, lr, lk, acc, \
                                                ld,                                         \
                                      MOE_SA((SI + S - 1) % S), MOE_SB((SI + S - 1) % S),   \
                                      min(kt + S - 1, nk - 1), mi_n, af, bfr);              \
    else                                                                                    \
      MOE_DMA_ISSUE(C, GATEUP, ATR, BTR, ld, MOE_SA((SI + S - 1) % S),                     \
                    MOE_SB((SI + S - 1) % S), nk - 1);                                      \
  }
  for (int kb = 0; kb < nk; kb += S) {
    MOE_STEP(0)
    MOE_STEP(1)
    MOE_STEP(2)
    MOE_STEP(3)
  }
#undef MOE_STEP
#undef MOE_SA
#undef MOE_SB
  if (MOE_DEFER && nk > 0) dma_mfmas<C, PARTIAL>(af[1], bfr[1], acc, mi_n);
  // No LDS write may still be in flight when the block ends.
  wait_vmcnt<0>();
}

}  // namespace dma
}  // namespace moe
