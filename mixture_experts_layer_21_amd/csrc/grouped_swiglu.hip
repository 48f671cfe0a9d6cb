// Grouped SwiGLU expert GEMMs over the expert-major row list.
//
// The expert is SwiGLUExpert of "Lab: build a tiny MoE in PyTorch" ("Full
// implementation"): down(silu(gate(x)) * up(x)) with bias-free Linears; the
// per-expert loop there becomes one launch over all (expert, row-tile,
// column-tile) triples, the grouped-GEMM form named in "2.9 Mixture-of-Experts
// (MoE) Architectures" ("MoE in Practice").
//
//   kernel 1 (GATEUP): Hb[r, :] = silu(x_t W_gate^T) * (x_t W_up^T), rounded
//            once to the activation dtype; x rows are gathered through
//            row_to_assign (t = a / top_k), never copied;
//   kernel 2 (DOWN):   Y[r, :]  = g(r) * (Hb[r, :] W_down^T), the gate weight
//            applied to the fp32 accumulators before rounding.
//
// bf16: 256 threads = 4 waves; a BM x BN output tile (GATEUP: BN gate and BN
// up columns) is built from v_mfma_f32_32x32x16_bf16; A and B tiles of BK = 64
// are staged through LDS (double-buffered, one barrier per k-step) with an XOR
// swizzle of the 16-byte chunks so the MFMA fragment reads are bank-conflict
// free.  The host never reads the expert offsets: the grid covers an upper
// bound of row tiles and each block finds its (expert, row tile) from the
// device-side offsets, exiting when it has none.  Block indices are remapped
// so that blocks sharing a weight tile run on the same XCD (one L2).
// fp32: the same tiling with plain FMA (small layers only).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int NTHREADS = 256;

struct Tile {
  int e, m0, m_end, nt;
};

// Map blockIdx.x to (expert, first row, row end, column tile).  Returns false
// when the block has no tile.  Row tiles of one column tile are consecutive in
// the logical order, and consecutive logical tiles share an XCD.
template <int BM>
__device__ bool find_tile(const GemmParams& p, int max_mtiles, Tile& t, int* s_scan) {
  const int G = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, q = G >> 3, rem = G & 7;
  const int L = xcd * q + min(xcd, rem) + (b >> 3);
  const int ml = L % max_mtiles;
  t.nt = L / max_mtiles;
  if (p.expert_offsets == nullptr) {  // identity rows: one group of T rows
    t.e = 0;
    t.m0 = ml * BM;
    t.m_end = p.T;
    return t.m0 < p.T;
  }
  // Inclusive scan of the per-expert row-tile counts (n_groups <= 256).
  const int tid = threadIdx.x;
  int cnt = 0;
  if (tid < p.n_groups) {
    const int rows = p.expert_offsets[tid + 1] - p.expert_offsets[tid];
    cnt = (rows + BM - 1) / BM;
  }
  s_scan[tid] = cnt;
  __syncthreads();
  for (int d = 1; d < NTHREADS; d <<= 1) {
    const int v = tid >= d ? s_scan[tid - d] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  const int total = s_scan[NTHREADS - 1];
  if (ml >= total) return false;  // uniform across the block
  if (tid < p.n_groups) {
    const int hi = s_scan[tid], lo = hi - cnt;
    if (ml >= lo && ml < hi) {
      s_scan[NTHREADS] = tid;
      s_scan[NTHREADS + 1] = p.expert_offsets[tid] + (ml - lo) * BM;
      s_scan[NTHREADS + 2] = p.expert_offsets[tid + 1];
    }
  }
  __syncthreads();
  t.e = s_scan[NTHREADS];
  t.m0 = s_scan[NTHREADS + 1];
  t.m_end = s_scan[NTHREADS + 2];
  return true;
}

// XOR swizzle of the 16-byte chunk index inside a 64-element (128-byte) row:
// any 8 consecutive rows, and the even or odd rows of any 16 consecutive
// rows, land on distinct chunk positions.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int BM, int BN, int WGM, bool GATEUP>
__global__ __launch_bounds__(NTHREADS) void gemm_bf16_kernel(GemmParams p, int max_mtiles) {
  constexpr int BK = 64;
  constexpr int WGN = 4 / WGM;
  constexpr int NB = GATEUP ? 2 : 1;
  constexpr int BROWS = NB * BN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int KCH = BK / 8;
  constexpr int AC = BM * KCH / NTHREADS, BC = BROWS * KCH / NTHREADS;
  static_assert(MI >= 1 && NI >= 1 && AC >= 1 && BC >= 1, "tile too small");
  static_assert(BM * KCH % NTHREADS == 0 && BROWS * KCH % NTHREADS == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BROWS * BK];
  __shared__ int s_scan[NTHREADS + 4];

  Tile tile;
  if (!find_tile<BM>(p, max_mtiles, tile, s_scan)) return;

  const int K = GATEUP ? p.D : p.hidden;
  const int N = GATEUP ? p.hidden : p.D;
  const int n0 = tile.nt * BN;
  const int tid = threadIdx.x;
  const uint16_t* x = static_cast<const uint16_t*>(p.x);
  const uint16_t* hb = static_cast<const uint16_t*>(p.hbuf);

  // Global sources and LDS destinations of this thread's 16-byte chunks.
  const uint16_t* a_src[AC];
  int a_dst[AC];
#pragma unroll
  for (int i = 0; i < AC; ++i) {
    const int c = tid + NTHREADS * i, r = c / KCH, kc = c % KCH;
    int grow = tile.m0 + r;
    if (grow >= tile.m_end) grow = tile.m0;
    const uint16_t* base;
    if constexpr (GATEUP) {
      const int tok = p.row_to_assign ? p.row_to_assign[grow] / p.k : grow;
      base = x + (size_t)tok * K;
    } else {
      base = hb + (size_t)grow * K;
    }
    a_src[i] = base + kc * 8;
    a_dst[i] = r * BK + (kc ^ swz(r)) * 8;
  }
  const uint16_t* b_src[BC];
  int b_dst[BC];
#pragma unroll
  for (int i = 0; i < BC; ++i) {
    const int c = tid + NTHREADS * i, r = c / KCH, kc = c % KCH;
    const uint16_t* w;
    int n;
    if constexpr (GATEUP) {
      w = static_cast<const uint16_t*>(r < BN ? p.w_gate : p.w_up);
      n = n0 + (r % BN);
    } else {
      w = static_cast<const uint16_t*>(p.w_down);
      n = n0 + r;
    }
    if (n >= N) n = n0;
    b_src[i] = w + ((size_t)tile.e * N + n) * K + kc * 8;
    b_dst[i] = r * BK + (kc ^ swz(r)) * 8;
  }

  f32x16 acc[NB][MI][NI];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[nb][mi][ni][i] = 0.f;

  u32x4 ra[AC], rb[BC];
#define MOE_GLOAD(k0)                                                                     \
  do {                                                                                    \
    _Pragma("unroll") for (int i = 0; i < AC; ++i) ra[i] =                                \
        *reinterpret_cast<const u32x4*>(a_src[i] + (k0));                                 \
    _Pragma("unroll") for (int i = 0; i < BC; ++i) rb[i] =                                \
        *reinterpret_cast<const u32x4*>(b_src[i] + (k0));                                 \
  } while (0)
#define MOE_SSTORE(buf)                                                                   \
  do {                                                                                    \
    _Pragma("unroll") for (int i = 0; i < AC; ++i)                                        \
        *reinterpret_cast<u32x4*>(&As[buf][a_dst[i]]) = ra[i];                            \
    _Pragma("unroll") for (int i = 0; i < BC; ++i)                                        \
        *reinterpret_cast<u32x4*>(&Bs[buf][b_dst[i]]) = rb[i];                            \
  } while (0)

  const int wave = tid / MOE_WAVE, lane = lane_id();
  const int wm = wave / WGN, wn = wave % WGN;
  const int lr = lane & 31, lk = lane >> 5;

  MOE_GLOAD(0);
  MOE_SSTORE(0);
  __syncthreads();
  const int nk = K / BK;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) MOE_GLOAD((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = kk * 2 + lk;
      bf16x8 af[MI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int r = wm * WM + mi * 32 + lr;
        af[mi] = *reinterpret_cast<const bf16x8*>(&As[cur][r * BK + (ch ^ swz(r)) * 8]);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int r = nb * BN + wn * WN + ni * 32 + lr;
          const bf16x8 bfr = *reinterpret_cast<const bf16x8*>(&Bs[cur][r * BK + (ch ^ swz(r)) * 8]);
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
            acc[nb][mi][ni] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr, acc[nb][mi][ni], 0, 0, 0);
        }
    }
    if (kt + 1 < nk) MOE_SSTORE(cur ^ 1);
    __syncthreads();
  }
#undef MOE_GLOAD
#undef MOE_SSTORE

  // Epilogue.  32x32 accumulator layout: element i of lane l is row
  // 8*(i/4) + 4*(l/32) + (i%4), column l%32.
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int grow = tile.m0 + wm * WM + mi * 32 + 8 * (i >> 2) + 4 * lk + (i & 3);
      if (grow >= tile.m_end) continue;
      if constexpr (GATEUP) {
        uint16_t* out = static_cast<uint16_t*>(p.hbuf) + (size_t)grow * N;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int col = n0 + wn * WN + ni * 32 + lr;
          if (col < N) {
            const float g = acc[0][mi][ni][i], u = acc[1][mi][ni][i];
            out[col] = f32_to_bf16_bits(silu_f32(g) * u);
          }
        }
      } else {
        float gw = 1.f;
        if (p.gate_w && p.row_to_assign) gw = p.gate_w[p.row_to_assign[grow]];
        uint16_t* out = static_cast<uint16_t*>(p.y) + (size_t)grow * N;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int col = n0 + wn * WN + ni * 32 + lr;
          if (col < N) out[col] = f32_to_bf16_bits(gw * acc[0][mi][ni][i]);
        }
      }
    }
  }
}

// fp32 path: 64x64 tiles, 16x16 threads with 4x4 outputs each (rows ty+16i,
// columns tx+16j), K staged 16 at a time, any K.
template <bool GATEUP>
__global__ __launch_bounds__(NTHREADS) void gemm_f32_kernel(GemmParams p, int max_mtiles) {
  constexpr int BM = 64, BN = 64, BK = 16;
  constexpr int NB = GATEUP ? 2 : 1;
  __shared__ float As[BK][BM + 1];
  __shared__ float Bs[NB][BK][BN + 1];
  __shared__ int s_scan[NTHREADS + 4];
  Tile tile;
  if (!find_tile<BM>(p, max_mtiles, tile, s_scan)) return;
  const int K = GATEUP ? p.D : p.hidden;
  const int N = GATEUP ? p.hidden : p.D;
  const int n0 = tile.nt * BN;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float* x = static_cast<const float*>(p.x);
  const float* hb = static_cast<const float*>(p.hbuf);

  float acc[NB][4][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[nb][i][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < BM * BK / NTHREADS; ++i) {
      const int c = tid + NTHREADS * i, r = c / BK, kk = c % BK;
      int grow = tile.m0 + r;
      if (grow >= tile.m_end) grow = tile.m0;
      float v = 0.f;
      if (k0 + kk < K) {
        if constexpr (GATEUP) {
          const int tok = p.row_to_assign ? p.row_to_assign[grow] / p.k : grow;
          v = x[(size_t)tok * K + k0 + kk];
        } else {
          v = hb[(size_t)grow * K + k0 + kk];
        }
      }
      As[kk][r] = v;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < BN * BK / NTHREADS; ++i) {
        const int c = tid + NTHREADS * i, r = c / BK, kk = c % BK;
        const int n = n0 + r;
        float v = 0.f;
        if (n < N && k0 + kk < K) {
          const float* w = static_cast<const float*>(GATEUP ? (nb ? p.w_up : p.w_gate) : p.w_down);
          v = w[((size_t)tile.e * N + n) * K + k0 + kk];
        }
        Bs[nb][kk][r] = v;
      }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float b = Bs[nb][kk][tx + 16 * j];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[nb][i][j] = fmaf(a[i], b, acc[nb][i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int grow = tile.m0 + ty + 16 * i;
    if (grow >= tile.m_end) continue;
    float gw = 1.f;
    if (!GATEUP && p.gate_w && p.row_to_assign) gw = p.gate_w[p.row_to_assign[grow]];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx + 16 * j;
      if (col >= N) continue;
      if constexpr (GATEUP) {
        static_cast<float*>(p.hbuf)[(size_t)grow * N + col] =
            silu_f32(acc[0][i][j]) * acc[NB - 1][i][j];
      } else {
        static_cast<float*>(p.y)[(size_t)grow * N + col] = gw * acc[0][i][j];
      }
    }
  }
}

int mtiles_bound(const GemmParams& p, int bm) {
  if (p.expert_offsets == nullptr) return (p.T + bm - 1) / bm;
  return (p.max_rows + bm - 1) / bm + p.n_groups;
}

template <int BM, int BN, int WGM, bool GATEUP>
hipError_t launch_bf16(const GemmParams& p, hipStream_t s) {
  const int N = GATEUP ? p.hidden : p.D;
  const int mt = mtiles_bound(p, BM);
  const long long nblocks = (long long)mt * ((N + BN - 1) / BN);
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, GATEUP>), dim3((unsigned)nblocks),
                     dim3(NTHREADS), 0, s, p, mt);
  return hipGetLastError();
}

template <bool GATEUP>
hipError_t launch_f32(const GemmParams& p, hipStream_t s) {
  const int N = GATEUP ? p.hidden : p.D;
  const int mt = mtiles_bound(p, 64);
  const long long nblocks = (long long)mt * ((N + 63) / 64);
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_f32_kernel<GATEUP>), dim3((unsigned)nblocks), dim3(NTHREADS), 0, s,
                     p, mt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_swiglu(const GemmParams& p, bool bf16, hipStream_t s) {
  hipError_t err;
  if (!bf16) {
    if ((err = launch_f32<true>(p, s)) != hipSuccess) return err;
    return launch_f32<false>(p, s);
  }
  // Rows per group decide the row-tile height: decode-sized groups use 32-row
  // tiles so that MFMA work is not spent on padding.
  const int rows = p.expert_offsets ? p.max_rows : p.T;
  const bool small_m = (long long)rows < 64LL * (p.expert_offsets ? p.n_groups : 1);
  if (small_m) {
    if ((err = launch_bf16<32, 128, 1, true>(p, s)) != hipSuccess) return err;
    return launch_bf16<32, 256, 1, false>(p, s);
  }
  if ((err = launch_bf16<128, 128, 2, true>(p, s)) != hipSuccess) return err;
  return launch_bf16<128, 256, 2, false>(p, s);
}

}  // namespace moe
