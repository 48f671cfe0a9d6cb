// Backward pass of the MoE layer on gfx950.
//
// The objective is the training loss of "Lab: build a tiny MoE in PyTorch"
// ("Smoke test and backward pass"): a task term whose gradient dout reaches
// the layer output, plus alpha * balance + beta * z.  As in "2.9
// Mixture-of-Experts (MoE) Architectures" ("The Router": top-k is a
// stop-gradient on the index decision; "The auxiliary load-balancing loss":
// the dispatch fractions f are detached), the routes, drops and counts of the
// forward are constants; gradients reach the router through the kept gate
// weights, through P_e and through z.
//
// Every GEMM of the backward runs on one grouped bf16 MFMA kernel whose two
// operands are K-contiguous (the forward's layout): weights are transposed
// once ([D,H] -> [H,D] etc.), and the operands of the weight gradients, whose
// contraction runs over the rows of an expert, are written transposed with
// each expert's rows padded to a multiple of 64 columns, so every k-step lies
// inside one expert.
//
//   recompute  g, u = x_t W_g^T, x_t W_u^T  ->  act, p1 = d act/d g, p2 = d act/d u
//   down dgrad dact = dout_t W_d;  dg = w dact p1, du = w dact p2;  dL/dw = act . dact
//   router     dh from dL/dw, the balance and z terms        (router_bwd_kernel)
//   up dgrad   dz = [dg du] [W_g; W_u];  dx_router = dh W_r;  dx = gather-sum (dx_kernel)
//   wgrad      dW_d = (w dout)^T act,  [dW_g; dW_u] = [dg du]^T x,  dW_r = dh^T x
#include <algorithm>

#include "common.hpp"
#include "dma_gemm.hpp"
#include "kernels.hpp"

// Non-temporal stores of the fp32 results of the direct-to-LDS backward
// GEMMs: mostly the weight gradients (twice the weights' bytes), written once
// (backward -1.7% on the Mixtral shape, -2.7% DeepSeek, -6% decode).
#ifndef MOE_BWD_NT_F32
#define MOE_BWD_NT_F32 1
#endif

namespace moe {
namespace {

constexpr int BT = 256;                  // threads of the GEMM block: 4 waves
constexpr int BBM = 128, BBN = 128, BBK = 64;
constexpr int BKCH = BBK / 8;            // 16-byte chunks per LDS row
constexpr int BCH = BBM * BKCH / BT;     // chunks per thread and operand (4)

// XOR swizzle of the 16-byte chunk inside a 128-byte LDS row (as the forward:
// conflict-free 32-row fragment reads).
__device__ __forceinline__ int bswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ float sigm(float v) { return sigmoid_f32(v); }

// Tile of the block: group, first row (MROWS: global row), row end, column
// tile, and the k range.  Returns false when the block has no tile.
struct BTile {
  int g, m0, m_end, nt, k0, k1;
};

// BM rows and bn output columns per tile.  Every thread of the block calls
// it (MROWS has barriers); the first 256 threads scan.
template <int BM>
__device__ bool bwd_tile(const BwdGemmParams& p, int bn, BTile& t, int* s_scan) {
  // Logical tile b.  DENSE and MROWS: block i runs on XCD i % 8, and each XCD
  // takes a contiguous run of logical tiles, so the blocks that share a B
  // slice (the row tiles of one column tile, consecutive below) share that
  // XCD's L2.  KRAGGED (short k ranges, fp32 tiles out) keeps the block
  // order: measured faster spread over the XCDs.
  const int nb = gridDim.x, xcd = blockIdx.x & 7, q = nb >> 3, rem = nb & 7;
  const int b = p.grouping == BWD_KRAGGED ? (int)blockIdx.x
                                          : xcd * q + min(xcd, rem) + (int)(blockIdx.x >> 3);
  if (p.grouping == BWD_DENSE) {
    const int ntn = (p.N + bn - 1) / bn, ntm = (p.M + BM - 1) / BM;
    if (b >= ntn * ntm) return false;
    t.g = 0;
    t.m0 = (b % ntm) * BM;
    t.nt = b / ntm;
    t.m_end = p.M;
    t.k0 = 0;
    t.k1 = p.K;
    return true;
  }
  if (p.grouping == BWD_KRAGGED) {
    const int ntn = (p.N + bn - 1) / bn, ntm = (p.M + BM - 1) / BM;
    const int per = ntn * ntm;
    if (b >= per * p.G) return false;
    t.g = b / per;
    const int q = b % per;
    t.m0 = (q % ntm) * BM;
    t.nt = q / ntm;
    t.m_end = p.M;
    t.k0 = p.offsets[t.g];
    t.k1 = p.offsets[t.g + 1];
    return true;
  }
  // MROWS: the row tiles of all groups, column tile major; one scan of the
  // per-group row-tile counts (G <= 256) finds the block's group.
  const int tid = threadIdx.x;
  int cnt = 0;
  if (tid < p.G) cnt = (p.offsets[tid + 1] - p.offsets[tid] + BM - 1) / BM;
  if (tid < BT) s_scan[tid] = cnt;
  __syncthreads();
  for (int d = 1; d < p.G; d <<= 1) {  // prefixes of the groups only
    const int v = (tid < BT && tid >= d) ? s_scan[tid - d] : 0;
    __syncthreads();
    if (tid < BT) s_scan[tid] += v;
    __syncthreads();
  }
  const int total = s_scan[p.G - 1];
  const int mt_bound = (p.max_rows + BM - 1) / BM + p.G;
  const int ml = b % mt_bound;
  t.nt = b / mt_bound;
  if (ml >= total || t.nt * bn >= p.N) return false;  // uniform across the block
  if (tid < p.G) {
    const int hi = s_scan[tid], lo = hi - cnt;
    if (ml >= lo && ml < hi) {
      s_scan[BT] = tid;
      s_scan[BT + 1] = p.offsets[tid] + (ml - lo) * BM;
      s_scan[BT + 2] = p.offsets[tid + 1];
    }
  }
  __syncthreads();
  t.g = s_scan[BT];
  t.m0 = s_scan[BT + 1];
  t.m_end = s_scan[BT + 2];
  t.k0 = 0;
  t.k1 = p.K;
  return true;
}

// 128x128 output tile, 4 waves stacked along M (each 32 rows x 128 columns:
// four 32x32 accumulators), BK = 64, LDS double-buffered through registers.
template <int EPI>
__global__ __launch_bounds__(BT) void bwd_gemm_kernel(BwdGemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BBM * BBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BBN * BBK];
  __shared__ int s_scan[BT + 4];
  BTile t;
  if (!bwd_tile<BBM>(p, EPI == BWD_EPI_GATEUP_SAVE ? BBN / 2 : BBN, t, s_scan)) return;
  const int tid = threadIdx.x;
  const bool kr = p.grouping == BWD_KRAGGED;

  // Row pointers of this thread's chunks (rows past the end load a valid row).
  const uint16_t* a_src[BCH];
  const uint16_t* b_src[BCH];
  int dst[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int c = tid + BT * i, r = c / BKCH, kc = c % BKCH;
    dst[i] = r * BBK + (kc ^ bswz(r)) * 8;
    int m = t.m0 + r;
    if (m >= t.m_end) m = t.m0;
    long long arow;
    if (kr) {
      arow = (long long)m * p.lda + t.k0;
    } else {
      const int src = p.gather ? p.gather[m] / p.gdiv : m;
      arow = (long long)src * p.lda;
    }
    a_src[i] = p.a_kmajor ? nullptr : p.A + arow + kc * 8;
    const uint16_t* bb;
    if (p.b_kmajor) {  // chunk c: k row c / 16, columns 8*(c % 16) .. +7
      b_src[i] = nullptr;
      continue;
    }
    if (EPI == BWD_EPI_GATEUP_SAVE) {
      // 64 gate rows then the same 64 up rows of column tile nt
      int n = t.nt * (BBN / 2) + (r % (BBN / 2));
      if (n >= p.N) n = 0;
      bb = (r < BBN / 2 ? p.B : p.B2) + (long long)t.g * p.b_gstride + (long long)n * p.ldb;
    } else {
      int n = t.nt * BBN + r;
      if (n >= p.N) n = 0;
      bb = kr ? p.B + (long long)n * p.ldb + t.k0
              : p.B + (long long)t.g * p.b_gstride + (long long)n * p.ldb;
    }
    b_src[i] = bb + kc * 8;
  }

  f32x16 acc[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[ni][i] = 0.f;

  const int nk = (t.k1 - t.k0) / BBK;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 31, lk = lane >> 5;
  u32x4 ra[BCH], rb[BCH];
  // k-major operands: chunk c of a stage is k row c / 16, columns
  // 8*(c % 16) .. +7 of the tile; rows past the operand's rows (the group's,
  // for KRAGGED; else past its byte extent) load as zeros.
  const long long a_rows = kr ? 0 : p.a_bytes / (2 * p.lda);
  const long long b_rows = kr ? 0 : p.b_bytes / (2 * p.ldb);
  const int kg0 = kr && p.krows ? p.krows[t.g] : 0;
  const int kg1 = kr && p.krows ? p.krows[t.g + 1] : 0;
  auto kmajor_load = [&](const uint16_t* base, const uint16_t* base2, long long ld, long long rows,
                         int k, int col, int ncols) -> u32x4 {
    if (col >= ncols) col = 0;
    long long row;
    const uint16_t* src = base;
    if (kr) {
      row = kg0 + (long long)k;
      if (row >= kg1) return u32x4{0u, 0u, 0u, 0u};
    } else {
      row = k;
      if (base2 && k >= p.k_split) {
        src = base2;
        row = k - p.k_split;
      }
      if (row >= rows) return u32x4{0u, 0u, 0u, 0u};
    }
    return *reinterpret_cast<const u32x4*>(src + row * ld + col);
  };
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int c = tid + BT * i, k = kt * BBK + c / (BBN / 8), c8 = (c % (BBN / 8)) * 8;
      if (p.a_kmajor)
        ra[i] = kmajor_load(p.A, nullptr, p.lda, a_rows, k, t.m0 + c8, p.M);
      else
        ra[i] = *reinterpret_cast<const u32x4*>(a_src[i] + (size_t)kt * BBK);
      if (p.b_kmajor) {
        const long long gs = kr ? 0 : (long long)t.g * p.b_gstride;
        rb[i] = kmajor_load(p.B + gs, p.B2 ? p.B2 + gs : nullptr, p.ldb, b_rows, k,
                            t.nt * BBN + c8, p.N);
      } else {
        rb[i] = *reinterpret_cast<const u32x4*>(b_src[i] + (size_t)kt * BBK);
      }
    }
  };
  // 8 columns of one k row into the row-major (k-contiguous) swizzled tile
  auto scatter8 = [&](uint16_t* tile, const u32x4& v, int c) {
    const int k = c / (BBN / 8), n0 = (c % (BBN / 8)) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int n = n0 + e;
      const uint32_t w = v[e >> 1];
      tile[n * BBK + ((k >> 3) ^ bswz(n)) * 8 + (k & 7)] =
          (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      if (p.a_kmajor)
        scatter8(As[buf], ra[i], tid + BT * i);
      else
        *reinterpret_cast<u32x4*>(&As[buf][dst[i]]) = ra[i];
      if (p.b_kmajor)
        scatter8(Bs[buf], rb[i], tid + BT * i);
      else
        *reinterpret_cast<u32x4*>(&Bs[buf][dst[i]]) = rb[i];
    }
  };
  if (nk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BBK / 16; ++kk) {
      const int ch = kk * 2 + lk;
      const int ra_ = wave * 32 + lr;
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(&As[cur][ra_ * BBK + (ch ^ bswz(ra_)) * 8]);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int rb_ = ni * 32 + lr;
        const bf16x8 bfr =
            *reinterpret_cast<const bf16x8*>(&Bs[cur][rb_ * BBK + (ch ^ bswz(rb_)) * 8]);
        acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr, acc[ni], 0, 0, 0);
      }
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  Accumulator element i of lane l: row 8*(i/4) + 4*(l/32) + (i%4)
  // of the wave's 32 rows, column l%32 of the 32-column block ni.
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = t.m0 + wave * 32 + 8 * (i >> 2) + 4 * lk + (i & 3);
    const bool row_ok = m < t.m_end;
    if (EPI == BWD_EPI_F32) {
      if (!row_ok) continue;
      if (p.Cb) {
        uint16_t* cb = p.Cb + (long long)t.g * p.c_gstride + (long long)m * p.ldc;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int n = t.nt * BBN + ni * 32 + lr;
          if (n < p.N) cb[n] = f32_to_bf16_bits(acc[ni][i]);
        }
        continue;
      }
      float* base;
      long long row = m;
      if (m >= p.c_split) {
        base = p.C2;
        row = m - p.c_split;
      } else {
        base = p.C;
      }
      base += (long long)t.g * p.c_gstride + row * p.ldc;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int n = t.nt * BBN + ni * 32 + lr;
        if (n < p.N) base[n] = acc[ni][i];
      }
    } else if (EPI == BWD_EPI_GATEUP_SAVE) {
      if (!row_ok) continue;
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int h = t.nt * (BBN / 2) + ni * 32 + lr;
        if (h >= p.N) continue;
        const float g = acc[ni][i], u = acc[ni + 2][i];
        float gc = g, uc = u, mg = 1.f, mu = 1.f;
        if (p.limit > 0.f) {
          gc = fminf(fmaxf(g, -p.limit), p.limit);
          uc = fminf(fmaxf(u, -p.limit), p.limit);
          mg = fabsf(g) < p.limit ? 1.f : 0.f;
          mu = fabsf(u) < p.limit ? 1.f : 0.f;
        }
        const float s = sigm(gc);
        const long long o = (long long)m * p.ldh + h;
        p.act[o] = f32_to_bf16_bits(gc * s * uc);
        p.p1[o] = f32_to_bf16_bits(mg * uc * (s + gc * s * (1.f - s)));
        p.p2[o] = f32_to_bf16_bits(mu * gc * s);
      }
    }
  }
}

// The same GEMM on the forward's 256x256 direct-to-LDS main loop: 512
// threads, BK = 64, two LDS stages, operands fetched straight into the
// swizzled LDS tiles by buffer loads with 32-bit offsets.  With the paired
// gate/up tile the B tile is 128 gate rows then the same 128 up rows.
template <int EPI, bool ATR, bool BTR>
__global__ __launch_bounds__(512) void bwd_dma_kernel(BwdGemmParams p) {
  constexpr bool PAIRED = EPI == BWD_EPI_GATEUP_SAVE;
  using C = dma::DmaCfg<256, 256, 64, 2, 2, 8, PAIRED>;
  constexpr int BM = 256, BK = 64, KCH = C::KCH, MI = C::MI, NI = C::NI, NB = C::NB;
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[BM * BK];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[BM * BK];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[256 * BK];
  __shared__ __attribute__((aligned(1024))) uint16_t sB1[256 * BK];
  __shared__ __attribute__((aligned(1024))) uint16_t sX[8];  // unused stages
  __shared__ int s_scan[BT + 4];
  BTile t;
  if (!bwd_tile<BM>(p, C::BN, t, s_scan)) return;
  const bool kr = p.grouping == BWD_KRAGGED;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // A k-major operand of a ragged-K group starts at the group's first row and
  // its resource covers exactly the group's rows (past them: zeros).
  const int kr0 = kr && (ATR || BTR) ? p.krows[t.g] : 0;
  const long long krn = kr && (ATR || BTR) ? p.krows[t.g + 1] - kr0 : 0;
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.A + (ATR && kr ? (long long)kr0 * p.lda : 0)), 0,
      (int)(ATR && kr ? krn * p.lda * 2 : p.a_bytes), 0x00020000);
  const long long bg = kr ? (BTR ? (long long)kr0 * p.ldb : 0) : (long long)t.g * p.b_gstride;
  const __amdgpu_buffer_rsrc_t rG = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.B + bg), 0, (int)(BTR && kr ? krn * p.ldb * 2 : p.b_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rU =
      (PAIRED || (BTR && p.B2))
          ? __builtin_amdgcn_make_buffer_rsrc((void*)(p.B2 + bg), 0, (int)p.b_bytes, 0x00020000)
          : rG;
  uint32_t a_off[C::A_LD];
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) {
    if constexpr (ATR) {  // k-major tile, as the B tile below
      const int k = 2 * (wave + C::NW * i) + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (k & 3));
      int m = t.m0 + c * 8;
      if (m >= p.M) m = 0;
      a_off[i] = (uint32_t)(((long long)k * p.lda + m) * 2);
      continue;
    }
    const int slot = (wave + C::NW * i) * 64 + lane;
    const int r = slot / KCH, lc = (slot % KCH) ^ dma::swz_k<KCH>(r);
    int m = t.m0 + r;
    if (m >= t.m_end) m = t.m0;
    const long long row = kr ? (long long)m * p.lda + t.k0
                             : (long long)(p.gather ? p.gather[m] / p.gdiv : m) * p.lda;
    a_off[i] = (uint32_t)(row * 2) + (uint32_t)lc * 16u;
  }
  uint32_t b_off[C::B_LD];
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) {
    if constexpr (BTR) {
      // k-major tile: a wave load is two k rows of 32 chunks (8 columns
      // each); chunk c of row k sits at c ^ 4*(k%4) (the layout the
      // transposed fragment reads expect)
      const int k = 2 * (wave + C::NW * i) + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (k & 3));
      int n = t.nt * C::BN + c * 8;
      if (n >= p.N) n = 0;
      b_off[i] = (uint32_t)(((long long)k * p.ldb + n) * 2);
    } else {
      const int slot = (wave + C::NW * i) * 64 + lane;
      const int r = slot / KCH, lc = (slot % KCH) ^ dma::swz_k<KCH>(r);
      int n = t.nt * C::BN + (PAIRED ? r % C::BN : r);
      if (n >= p.N) n = 0;
      const long long row = (long long)n * p.ldb + (kr ? t.k0 : 0);
      b_off[i] = (uint32_t)(row * 2) + (uint32_t)lc * 16u;
    }
  }
  const dma::DmaLoads<C, PAIRED> ld{rA, rG, rU, a_off, b_off, wave,
                                    (uint32_t)(p.ldb * 2), BTR ? p.k_split : 0,
                                    (uint32_t)(p.lda * 2)};
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int lr = lane & 31, lk = lane >> 5;
  f32x16 acc[NB][MI][NI];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[nb][mi][ni][i] = 0.f;
  const int nk = (t.k1 - t.k0) / BK;
  // (Device pass only: the host pass of hipcc rejects this call's template
  // deduction; kernel bodies are never run on the host.)
  // Waves whose 32-row blocks lie past the tile's rows (the last row tile of
  // an expert) skip those blocks' fragment reads and MFMAs.
  const int mi_n = min(MI, max(0, (t.m_end - t.m0 - wm * C::WM + 31) / 32));
#if defined(__HIP_DEVICE_COMPILE__)
  if (nk > 0) {
    if (mi_n == MI)
      dma::dma_mainloop<C, PAIRED, false, BTR, ATR>(ld, nk, MI, wm, wn, lr, lk, acc, sA0, sA1, sX,
                                                    sX, sB0, sB1, sX, sX);
    else
      dma::dma_mainloop<C, PAIRED, true, BTR, ATR>(ld, nk, mi_n, wm, wn, lr, lk, acc, sA0, sA1,
                                                   sX, sX, sB0, sB1, sX, sX);
  }
#endif

  // Epilogue: element i of accumulator (nb, mi, ni) of lane l is row
  // wm*WM + mi*32 + 8*(i/4) + 4*(l/32) + (i%4), column wn*WN + ni*32 + l%32.
  const int n_base = t.nt * C::BN + wn * C::WN;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rloc = wm * C::WM + mi * 32 + 8 * (i >> 2) + 4 * lk + (i & 3);
      const int m = t.m0 + rloc;
      const bool row_ok = m < t.m_end;
      if (EPI == BWD_EPI_F32) {
        if (!row_ok) continue;
        if (p.Cb) {
          uint16_t* cb = p.Cb + (long long)t.g * p.c_gstride + (long long)m * p.ldc;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const int n = n_base + ni * 32 + lr;
            if (n < p.N) cb[n] = f32_to_bf16_bits(acc[0][mi][ni][i]);
          }
          continue;
        }
        float* base = m >= p.c_split ? p.C2 : p.C;
        const long long row = m >= p.c_split ? m - p.c_split : m;
        base += (long long)t.g * p.c_gstride + row * p.ldc;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int n = n_base + ni * 32 + lr;
          if (n < p.N) {
            if (MOE_BWD_NT_F32)  // fp32 results, mostly weight gradients written once
              __builtin_nontemporal_store(acc[0][mi][ni][i], base + n);
            else
              base[n] = acc[0][mi][ni][i];
          }
        }
      } else if (EPI == BWD_EPI_GATEUP_SAVE) {
        if (!row_ok) continue;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int h = n_base + ni * 32 + lr;
          if (h >= p.N) continue;
          const float g = acc[0][mi][ni][i], u = acc[NB - 1][mi][ni][i];
          float gc = g, uc = u, mg = 1.f, mu = 1.f;
          if (p.limit > 0.f) {
            gc = fminf(fmaxf(g, -p.limit), p.limit);
            uc = fminf(fmaxf(u, -p.limit), p.limit);
            mg = fabsf(g) < p.limit ? 1.f : 0.f;
            mu = fabsf(u) < p.limit ? 1.f : 0.f;
          }
          const float s = sigm(gc);
          const long long o = (long long)m * p.ldh + h;
          p.act[o] = f32_to_bf16_bits(gc * s * uc);
          p.p1[o] = f32_to_bf16_bits(mg * uc * (s + gc * s * (1.f - s)));
          p.p2[o] = f32_to_bf16_bits(mu * gc * s);
        }
      }
    }
  }
}

bool bwd_dma_fits(const BwdGemmParams& p) {
  const long long lim = 1ll << 31;
  return p.a_bytes > 0 && p.b_bytes > 0 && p.a_bytes < lim && p.b_bytes < lim;
}

// SwiGLU backward, one wave per row, 16-byte chunks along H (see
// SwigluBwdParams).  The dL/dw sum runs per lane in chunk order, then over
// the lanes in a fixed butterfly.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(SwigluBwdParams p) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int rows = p.offsets ? p.offsets[p.G] : p.n;
  if (r >= rows) return;  // whole wave
  const float w = p.gate_w ? p.gate_w[p.r2a ? p.r2a[r] : r] : 1.f;
  const long long base = (long long)r * p.H;
  const long long based = (long long)r * 2 * p.H;
  float rs = 0.f;
  for (int c = lane * 8; c < p.H; c += 64 * 8) {
    const u32x4 d4 = *reinterpret_cast<const u32x4*>(p.dact + base + c);
    const u32x4 a4 = *reinterpret_cast<const u32x4*>(p.act + base + c);
    const u32x4 q4 = *reinterpret_cast<const u32x4*>(p.p1 + base + c);
    const u32x4 v4 = *reinterpret_cast<const u32x4*>(p.p2 + base + c);
    u32x4 g4, u4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d0 = __uint_as_float(d4[e] << 16), d1 = __uint_as_float(d4[e] & 0xffff0000u);
      rs += __uint_as_float(a4[e] << 16) * d0;
      rs += __uint_as_float(a4[e] & 0xffff0000u) * d1;
      g4[e] = (uint32_t)f32_to_bf16_bits(w * d0 * __uint_as_float(q4[e] << 16)) |
              ((uint32_t)f32_to_bf16_bits(w * d1 * __uint_as_float(q4[e] & 0xffff0000u)) << 16);
      u4[e] = (uint32_t)f32_to_bf16_bits(w * d0 * __uint_as_float(v4[e] << 16)) |
              ((uint32_t)f32_to_bf16_bits(w * d1 * __uint_as_float(v4[e] & 0xffff0000u)) << 16);
    }
    *reinterpret_cast<u32x4*>(p.dgu + based + c) = g4;
    *reinterpret_cast<u32x4*>(p.dgu + based + p.H + c) = u4;
  }
  if (p.dw) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) rs += __shfl_xor(rs, off);
    if (lane == 0) p.dw[r] = rs;
  }
}

// 64x64 tiled transpose through LDS (see TransposeParams), 16-byte global
// accesses on both sides (every row stride and column offset is a multiple
// of 8 elements).  With skip_rows, a batch b whose group has no rows
// (skip_rows[b+1] == skip_rows[b]) is left untouched: its weights feed no
// gradient.
__global__ __launch_bounds__(256) void transpose_kernel(TransposeParams p) {
  __shared__ uint16_t tile[64][66];
  __shared__ int s_group;
  const int b = blockIdx.z;
  if (p.skip_rows && p.skip_rows[b + 1] == p.skip_rows[b]) return;
  const int jc0 = blockIdx.x * 64;           // first destination column (padded space)
  const int c0 = blockIdx.y * 64;            // first source column
  if (jc0 >= p.out_cols) return;
  const int tid = threadIdx.x;
  // Source rows j of this tile: with ragged groups a 64-column tile lies in
  // one group (padded offsets are multiples of 64), found by one thread per
  // group (G <= 256); -1: past the last group, the tile is zeros.
  int j0 = jc0, j_end = p.rows;
  if (p.offsets) {
    if (tid == 0) s_group = -1;
    __syncthreads();
    if (tid < p.G && p.padoff[tid] <= jc0 && jc0 < p.padoff[tid + 1]) s_group = tid;
    __syncthreads();
    const int g = s_group;
    if (g < 0) {
      j0 = 0;
      j_end = 0;
    } else {
      j0 = p.offsets[g] + (jc0 - p.padoff[g]);
      j_end = p.offsets[g + 1];
    }
  }
  // load: 64 source rows x 64 columns; a thread takes 16-byte chunks
  const int per = p.src_f32 ? 4 : 8;           // elements per chunk
  const int cpr = 64 / per;                    // chunks per row
  for (int q = tid; q < 64 * cpr; q += 256) {
    const int jj = q / cpr, cc = (q % cpr) * per;
    const int j = j0 + jj, c = c0 + cc;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (j < j_end && c < p.cols) {
      const int src_row = p.gather ? p.gather[j] / p.gdiv : j;
      const long long o = (long long)b * p.src_bstride + (long long)src_row * p.ld_src + c;
      if (p.src_f32) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.src) + o);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = x[e];
      } else {
        const u32x4 x = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.src) + o);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = __uint_as_float(x[e] << 16);
          v[2 * e + 1] = __uint_as_float(x[e] & 0xffff0000u);
        }
      }
      if (p.scale) {
        const float sc = p.scale[p.scale_idx ? p.scale_idx[j] : j];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= sc;
      }
    }
    for (int e = 0; e < per; ++e) tile[jj][cc + e] = f32_to_bf16_bits(v[e]);
  }
  __syncthreads();
  // store: 64 destination rows (source columns) x 64 columns, 8 per chunk
  for (int q = tid; q < 64 * 8; q += 256) {
    const int cc = q / 8, jj = (q % 8) * 8;
    const int c = c0 + cc, jc = jc0 + jj;
    if (c >= p.cols || jc >= p.out_cols) continue;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[jj + 2 * e][cc] | ((uint32_t)tile[jj + 2 * e + 1][cc] << 16);
    *reinterpret_cast<u32x4*>(p.dst + (long long)b * p.dst_bstride + (long long)c * p.ld_dst +
                              p.dst_col0 + jc) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// padoff[g] = sum over g' < g of the rows of g' rounded up to 64.
__global__ __launch_bounds__(256) void pad_offsets_kernel(int G, const int32_t* offsets,
                                                          int32_t* padoff) {
  __shared__ int s[257];
  const int tid = threadIdx.x;
  s[tid + 1] = tid < G ? (offsets[tid + 1] - offsets[tid] + 63) / 64 * 64 : 0;
  if (tid == 0) s[0] = 0;
  __syncthreads();
  if (tid == 0)
    for (int g = 1; g <= G; ++g) s[g] += s[g - 1];
  __syncthreads();
  // G + 1 values: with G = 256 groups the end offset is the 257th
  for (int i = tid; i <= G; i += blockDim.x) padoff[i] = s[i];
}

// dL/dh for one token per wave (experts lane + 64j, j < 4).
__global__ __launch_bounds__(256) void router_bwd_kernel(RouterBwdParams p) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const int E = p.E, k = p.k;
  uint16_t* dh_row = p.dh + (long long)t * p.Epad;
  if (p.ids[(long long)t * k] < 0) {  // masked token: no gradient
    for (int e = lane; e < p.Epad; e += 64) dh_row[e] = 0;
    if (p.dgw && lane < k) p.dgw[(long long)t * k + lane] = 0.f;
    return;
  }
  float h[4], sc[4], smx[4];
  bool ok[4];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    ok[j] = e < E;
    h[j] = ok[j] ? p.logits[(long long)t * E + e] : -INFINITY;
    m = fmaxf(m, h[j]);
  }
  m = wave_max(m);
  float S = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    smx[j] = ok[j] ? __expf(h[j] - m) : 0.f;
    S += smx[j];
  }
  S = wave_sum(S);
  const float lse = m + __logf(S);
  float ssum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    smx[j] /= S;
    if (!ok[j]) {
      sc[j] = 0.f;
    } else if (p.score_func == 0) {
      sc[j] = smx[j];
    } else if (p.score_func == 1) {
      sc[j] = sigm(h[j]);
    } else {
      const float sp = h[j] > 20.f ? h[j] : log1pf(__expf(h[j]));
      sc[j] = sqrtf(sp);
    }
    ssum += sc[j];
  }
  ssum = wave_sum(ssum);

  // dL/dw of each slot: that of its kept row (0 when dropped).
  float dw[kMaxTopK];
  float csum = 0.f, dwc = 0.f;
  for (int s = 0; s < k; ++s) {
    const int r = p.a2r[(long long)t * k + s];
    const float v = r >= 0 ? p.dw[r] : 0.f;
    dw[s] = v;
    const int e = p.ids[(long long)t * k + s];
    float cj = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (e >> 6 == j) cj = __shfl(sc[j], e & 63);
    csum += cj;
    dwc += v * cj;
  }
  if (p.dgw && lane < k) {
    float mine = 0.f;
    for (int s = 0; s < k; ++s)
      if (s == lane) mine = dw[s];
    p.dgw[(long long)t * k + lane] = mine;
  }
  // dL/d score
  float dsc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < k; ++s) {
    const int e = p.ids[(long long)t * k + s];
    const float dc = p.renormalize ? p.route_scale / csum * (dw[s] - dwc / csum)
                                   : p.route_scale * dw[s];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == e) dsc[j] += dc;
  }
  // balance: E * sum f_e P_e with f = counts / (n_valid k) held constant
  int tot = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) tot += ok[j] ? p.counts[lane + 64 * j] : 0;
  tot = wave_sum_int(tot);
  const float n_valid = (float)(tot / k);
  if (p.alpha != 0.f && tot > 0) {
    float dq[4], dqq = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dq[j] = ok[j] ? p.alpha * (float)E * ((float)p.counts[lane + 64 * j] / (float)tot) / n_valid
                    : 0.f;
      dqq += dq[j] * sc[j];
    }
    dqq = wave_sum(dqq);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (p.score_func == 0)
        dsc[j] += dq[j];
      else
        dsc[j] += (dq[j] - dqq / ssum) / ssum;
    }
  }
  // scores -> logits, then z = mean lse^2
  float dss = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) dss += dsc[j] * sc[j];
  dss = wave_sum(dss);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float d;
    if (!ok[j]) {
      d = 0.f;
    } else if (p.score_func == 0) {
      d = sc[j] * (dsc[j] - dss);
    } else if (p.score_func == 1) {
      d = dsc[j] * sc[j] * (1.f - sc[j]);
    } else {
      d = dsc[j] * sigm(h[j]) / (2.f * sc[j]);
    }
    if (ok[j] && p.beta != 0.f && tot > 0) d += p.beta * 2.f * lse * smx[j] / n_valid;
    const int e = lane + 64 * j;
    if (e < p.Epad) dh_row[e] = f32_to_bf16_bits(ok[j] ? d : 0.f);
  }
}

// dx[t] = sum over kept slots (slot order) of dz[row] + dzs[t] + dxr[t]
template <typename T>
__global__ __launch_bounds__(256) void dx_kernel(DxParams p) {
  const long long n4 = (long long)p.T * p.D / 4;
  for (long long q = blockIdx.x * 256ll + threadIdx.x; q < n4; q += (long long)gridDim.x * 256) {
    const long long o = q * 4;
    const int t = (int)(o / p.D), d = (int)(o % p.D);
    f32x4 s = *reinterpret_cast<const f32x4*>(p.dxr + o);
    for (int j = 0; j < p.k; ++j) {
      const int r = p.a2r[(long long)t * p.k + j];
      if (r >= 0) s += *reinterpret_cast<const f32x4*>(p.dz + (long long)r * p.D + d);
    }
    if (p.dzs) s += *reinterpret_cast<const f32x4*>(p.dzs + o);
    if (p.sg) {
      const float g = p.sg[t], dl = g * (1.f - g) * p.sdw[t];
      const uint2 w2 = *reinterpret_cast<const uint2*>(p.wsg + d);
      s[0] += dl * __uint_as_float(w2.x << 16);
      s[1] += dl * __uint_as_float(w2.x & 0xffff0000u);
      s[2] += dl * __uint_as_float(w2.y << 16);
      s[3] += dl * __uint_as_float(w2.y & 0xffff0000u);
    }
    if (p.dx_f32) {
      *reinterpret_cast<f32x4*>(p.dx_f32 + o) = s;
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) Elem<T>::store(static_cast<T*>(p.dx), o + i, s[i]);
  }
}

// Gate of the shared expert: one wave per token, the fp32 dot product of
// 8-element chunks per lane, then a butterfly over the lanes.
__global__ __launch_bounds__(256) void shared_gate_kernel(int T, int D, const uint16_t* x,
                                                          const uint16_t* wsg, float* g) {
  const int lane = threadIdx.x & 63, t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  float acc = 0.f;
  for (int c = lane * 8; c < D; c += 64 * 8) {
    const u32x4 xv = *reinterpret_cast<const u32x4*>(x + (long long)t * D + c);
    const u32x4 wv = *reinterpret_cast<const u32x4*>(wsg + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc += __uint_as_float(xv[e] << 16) * __uint_as_float(wv[e] << 16);
      acc += __uint_as_float(xv[e] & 0xffff0000u) * __uint_as_float(wv[e] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) g[t] = sigm(acc);
}

// Weight gradient of the gate: each block sums a chunk of rows for 256
// columns in row order; a second pass adds the chunks in order.
constexpr int kGateRowsPerChunk = 256;

int gate_rows_per_chunk(int T) {
  const int per = (T + 65534) / 65535;  // the grid's y extent stays within 65535
  return per > kGateRowsPerChunk ? per : kGateRowsPerChunk;
}

__global__ __launch_bounds__(256) void gate_dw_part_kernel(int T, int D, const uint16_t* x,
                                                           const float* g, const float* sdw,
                                                           int per, float* part) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  if (d >= D) return;
  const long long t0 = (long long)blockIdx.y * per;
  const long long t1 = min((long long)T, t0 + per);
  float acc = 0.f;
  for (long long t = t0; t < t1; ++t) {
    const float dl = g[t] * (1.f - g[t]) * sdw[t];
    acc += dl * __uint_as_float((uint32_t)x[t * D + d] << 16);
  }
  part[(long long)blockIdx.y * D + d] = acc;
}

__global__ __launch_bounds__(256) void colsum_final_kernel(int D, int nchunk, const float* part,
                                                           float* out) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  if (d >= D) return;
  float acc = part[d];
  for (int c = 1; c < nchunk; ++c) acc += part[(long long)c * D + d];
  out[d] = acc;
}

}  // namespace

int gate_dw_chunks(int T) { return (T + gate_rows_per_chunk(T) - 1) / gate_rows_per_chunk(T); }

hipError_t launch_shared_gate(int T, int D, const uint16_t* x, const uint16_t* wsg, float* g,
                              hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(shared_gate_kernel, dim3((T + 3) / 4), dim3(256), 0, s, T, D, x, wsg, g);
  return hipGetLastError();
}

hipError_t launch_gate_dw(int T, int D, const uint16_t* x, const float* g, const float* sdw,
                          float* part, float* dwsg, hipStream_t s) {
  const dim3 grid((D + 255) / 256, gate_dw_chunks(T));
  hipLaunchKernelGGL(gate_dw_part_kernel, grid, dim3(256), 0, s, T, D, x, g, sdw,
                     gate_rows_per_chunk(T), part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(colsum_final_kernel, dim3((D + 255) / 256), dim3(256), 0, s, D,
                     gate_dw_chunks(T), part, dwsg);
  return hipGetLastError();
}

hipError_t launch_bwd_gemm(const BwdGemmParams& p, hipStream_t s) {
  if (bwd_dma_fits(p)) {
    const int bn = p.epilogue == BWD_EPI_GATEUP_SAVE ? 128 : 256, nN = (p.N + bn - 1) / bn;
    long long blocks;
    if (p.grouping == BWD_DENSE)
      blocks = (long long)nN * ((p.M + 255) / 256);
    else if (p.grouping == BWD_KRAGGED)
      blocks = (long long)nN * ((p.M + 255) / 256) * p.G;
    else
      blocks = (long long)nN * ((p.max_rows + 255) / 256 + p.G);
    if (blocks <= 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(512);
    if (p.epilogue != BWD_EPI_F32)
      hipLaunchKernelGGL((bwd_dma_kernel<BWD_EPI_GATEUP_SAVE, false, false>), grid, block, 0, s, p);
    else if (p.a_kmajor && p.b_kmajor)
      hipLaunchKernelGGL((bwd_dma_kernel<BWD_EPI_F32, true, true>), grid, block, 0, s, p);
    else if (p.a_kmajor)
      hipLaunchKernelGGL((bwd_dma_kernel<BWD_EPI_F32, true, false>), grid, block, 0, s, p);
    else if (p.b_kmajor)
      hipLaunchKernelGGL((bwd_dma_kernel<BWD_EPI_F32, false, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((bwd_dma_kernel<BWD_EPI_F32, false, false>), grid, block, 0, s, p);
    return hipGetLastError();
  }
  long long blocks;
  const int nN = p.epilogue == BWD_EPI_GATEUP_SAVE ? (p.N + BBN / 2 - 1) / (BBN / 2)
                                                  : (p.N + BBN - 1) / BBN;
  if (p.grouping == BWD_DENSE)
    blocks = (long long)nN * ((p.M + BBM - 1) / BBM);
  else if (p.grouping == BWD_KRAGGED)
    blocks = (long long)nN * ((p.M + BBM - 1) / BBM) * p.G;
  else
    blocks = (long long)nN * ((p.max_rows + BBM - 1) / BBM + p.G);
  if (blocks <= 0) return hipSuccess;
  if (p.epilogue == BWD_EPI_F32)
    hipLaunchKernelGGL(bwd_gemm_kernel<BWD_EPI_F32>, dim3((unsigned)blocks), dim3(BT), 0, s, p);
  else
    hipLaunchKernelGGL(bwd_gemm_kernel<BWD_EPI_GATEUP_SAVE>, dim3((unsigned)blocks), dim3(BT), 0,
                       s, p);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const SwigluBwdParams& p, hipStream_t s) {
  if (p.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((p.n + 3) / 4), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_transpose(const TransposeParams& p, hipStream_t s) {
  if (p.out_cols <= 0 || p.cols <= 0 || p.batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_kernel, dim3((p.out_cols + 63) / 64, (p.cols + 63) / 64, p.batch),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_pad_offsets(int G, const int32_t* offsets, int32_t* padoff, hipStream_t s) {
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(256), 0, s, G, offsets, padoff);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const RouterBwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL(router_bwd_kernel, dim3((p.T + 3) / 4), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_dx(const DxParams& p, bool bf16, hipStream_t s) {
  const long long n4 = (long long)p.T * p.D / 4;
  const unsigned blocks = (unsigned)std::min<long long>((n4 + 255) / 256, 8192);
  if (bf16)
    hipLaunchKernelGGL(dx_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(dx_kernel<float>, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
