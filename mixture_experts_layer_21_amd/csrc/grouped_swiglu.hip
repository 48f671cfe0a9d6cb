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
#include <type_traits>

#include <algorithm>

#include "common.hpp"
#include "dma_gemm.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

using namespace dma;

constexpr int NTHREADS = 256;

// silu(g) * u, with both projections first clamped to [-limit, limit] when
// limit > 0 (the clamped SwiGLU of the NeMo MLP, swiglu_limit).
__device__ __forceinline__ float swiglu_act(float g, float u, float limit) {
  if (limit > 0.f) {
    g = fminf(fmaxf(g, -limit), limit);
    u = fminf(fmaxf(u, -limit), limit);
  }
  return silu_f32(g) * u;
}

// The two factors of d act = p1 dg + p2 du for act = silu(g) u (each input
// clamped to [-limit, limit] first when limit > 0, with no gradient where it
// clamps), rounded to bf16 at element o of save_p1 / save_p2.
__device__ __forceinline__ void save_factors(const GemmParams& p, size_t o, float g, float u) {
  float gc = g, uc = u, mg = 1.f, mu = 1.f;
  if (p.swiglu_limit > 0.f) {
    gc = fminf(fmaxf(g, -p.swiglu_limit), p.swiglu_limit);
    uc = fminf(fmaxf(u, -p.swiglu_limit), p.swiglu_limit);
    mg = fabsf(g) < p.swiglu_limit ? 1.f : 0.f;
    mu = fabsf(u) < p.swiglu_limit ? 1.f : 0.f;
  }
  const float s = sigmoid_f32(gc);
  p.save_p1[o] = f32_to_bf16_bits(mg * uc * (s + gc * s * (1.f - s)));
  p.save_p2[o] = f32_to_bf16_bits(mu * gc * s);
}

struct Tile {
  int e, m0, m_end, nt;
  int rt;  // row tiles of the expert (decode_job only)
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
  for (int d = 1; d < p.n_groups; d <<= 1) {  // prefixes of the groups only
    const int v = tid >= d ? s_scan[tid - d] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  const int total = s_scan[p.n_groups - 1];
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

// Blocks per XCD of the split-K tail reduce of the large and 128-row tiles.
#ifndef MOE_REDUCE_BLOCKS
#define MOE_REDUCE_BLOCKS 128
#endif

// The weights of a layer stream through with non-temporal loads when all
// its experts' weights together exceed this many bytes (MI355X: a 256 MB
// Infinity Cache; a smaller set stays there from one call to the next, and
// streaming loads would give that up).
#ifndef MOE_STREAM_MIN_BYTES
#define MOE_STREAM_MIN_BYTES (256ll << 20)
#endif

// Most pieces a split tail tile is cut into (at most 16: the reduce kernels
// hold one vector per piece).
#ifndef MOE_TAIL_MAX_PIECES
#define MOE_TAIL_MAX_PIECES 16
#endif
static_assert(MOE_TAIL_MAX_PIECES >= 1 && MOE_TAIL_MAX_PIECES <= 16, "tail pieces");

// Column tiles per rasterisation band of the large-tile kernel.
#ifndef MOE_BAND
#define MOE_BAND 4
#endif

// Tile decode shared by the grouped GEMM kernels (blockDim >= 256; every
// thread must call it, it contains barriers).  The active tiles (row tiles of
// every expert x column tiles) are dealt to the XCDs in contiguous runs;
// block b runs on XCD b%8 as that XCD's (b/8)-th block.  Each XCD runs its
// whole rounds of tail_slots tiles at full depth; the r tiles left over are
// each cut along K (64-deep k-steps) into nsplit pieces, so the last round is
// short.  Pieces write fp32 partial tiles that a reduce kernel adds in piece
// order.  Returns false when the block has no work.
template <int BM, int BN, bool GATEUP>
__device__ bool decode_job(const GemmParams& p, int tail_slots, int* s_scan, Tile& tile,
                           int& piece, int& nsplit, int& tail_slot) {
  piece = -1;
  nsplit = 1;
  tail_slot = 0;
  int tail_tile = 0;
  {
    const int tid = threadIdx.x;
    const int ntiles = ((GATEUP ? p.hidden : p.D) + BN - 1) / BN;
    const int nk = (GATEUP ? p.D : p.hidden) / 64;
    int total, cnt = 0;
    if (p.expert_offsets == nullptr) {
      total = (p.T + BM - 1) / BM;
    } else {
      // Inclusive scan of the per-expert row-tile counts; the first 256
      // threads scan, all threads take part in the barriers.
      if (tid < p.n_groups) {
        const int rows = p.expert_offsets[tid + 1] - p.expert_offsets[tid];
        cnt = (rows + BM - 1) / BM;
      }
      if (tid < NTHREADS) s_scan[tid] = cnt;
      __syncthreads();
      for (int d = 1; d < p.n_groups; d <<= 1) {  // prefixes of the groups only
        const int v = (tid < NTHREADS && tid >= d) ? s_scan[tid - d] : 0;
        __syncthreads();
        if (tid < NTHREADS) s_scan[tid] += v;
        __syncthreads();
      }
      total = s_scan[p.n_groups - 1];
    }
    const int A = total * ntiles;
    const int b = blockIdx.x, xcd = b % kXcds, i = b / kXcds;
    const int ax = A / kXcds + (xcd < A % kXcds ? 1 : 0);
    const int start = xcd * (A / kXcds) + min(xcd, A % kXcds);
    int nfull = ax, r = 0;
    if (tail_slots > 0) {
      nfull = ax / tail_slots * tail_slots;
      r = ax - nfull;
      nsplit = r > 0 ? min(min(tail_slots / r, MOE_TAIL_MAX_PIECES), nk) : 1;
      if (nsplit < 2) {
        nfull = ax;
        r = 0;
        nsplit = 1;
      }
      if (i == 0 && tid == 0) {
        p.tail_meta[2 * xcd] = r;
        p.tail_meta[2 * xcd + 1] = nsplit;
      }
    }
    int L;
    if (i < nfull) {
      L = start + i;
    } else if (i < nfull + r * nsplit) {
      tail_tile = (i - nfull) / nsplit;
      piece = (i - nfull) % nsplit;
      tail_slot = xcd * kTailSlots + (i - nfull);
      L = start + nfull + tail_tile;
    } else {
      return false;  // uniform across the block
    }
    // Logical tiles run in bands of GN column tiles; inside a band the GN
    // column tiles of one row tile are consecutive.  The blocks an XCD holds
    // at once then cover about (32/GN) row tiles x GN column tiles, so each
    // A slice is fetched into that XCD's L2 once for GN blocks and each B
    // slice once for the row tiles of its expert.
    constexpr int GN = MOE_BAND;
    const int full = ntiles / GN;
    int ml;
    if (L < full * total * GN) {
      const int rr = L % (total * GN);
      ml = rr / GN;
      tile.nt = (L / (total * GN)) * GN + rr % GN;
    } else {
      const int w = ntiles - full * GN;
      const int rr = L - full * total * GN;
      ml = rr / w;
      tile.nt = full * GN + rr % w;
    }
    if (p.expert_offsets == nullptr) {
      tile.e = 0;
      tile.m0 = ml * BM;
      tile.m_end = p.T;
      tile.rt = total;
    } else {
      if (tid < p.n_groups) {
        const int hi = s_scan[tid], lo = hi - cnt;
        if (ml >= lo && ml < hi) {
          s_scan[NTHREADS] = tid;
          s_scan[NTHREADS + 1] = p.expert_offsets[tid] + (ml - lo) * BM;
          s_scan[NTHREADS + 2] = p.expert_offsets[tid + 1];
          s_scan[NTHREADS + 3] = cnt;
        }
      }
      __syncthreads();
      tile.e = s_scan[NTHREADS];
      tile.m0 = s_scan[NTHREADS + 1];
      tile.m_end = s_scan[NTHREADS + 2];
      tile.rt = s_scan[NTHREADS + 3];
    }
    if (piece == 0 && tid == 0) {
      int32_t* d = p.tail_desc + (size_t)(xcd * kTailSlots + tail_tile) * 4;
      d[0] = tile.e;
      d[1] = tile.m0;
      d[2] = tile.m_end;
      d[3] = tile.nt;
    }
  }

  return true;
}

// XOR swizzle of the 16-byte chunk index inside a 64-element (128-byte) row:
// any 8 consecutive rows, and the even or odd rows of any 16 consecutive
// rows, land on distinct chunk positions.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int BM, int BN, int WGM, bool GATEUP, bool NT>
__global__ __launch_bounds__(NTHREADS) void gemm_bf16_kernel(GemmParams p, int tail_slots) {
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
  int piece, nsplit, tail_slot;
  if (!decode_job<BM, BN, GATEUP>(p, tail_slots, s_scan, tile, piece, nsplit, tail_slot))
    return;

  const int K = GATEUP ? p.D : p.hidden;
  const int N = GATEUP ? p.hidden : p.D;
  const int n0 = tile.nt * BN;
  const int tid = threadIdx.x;
  // K range: all k-steps, or this piece's share of a split tail tile.
  const int nk_all = K / BK;
  const int kb = piece < 0 ? 0 : piece * nk_all / nsplit;
  const int ke = piece < 0 ? nk_all : (piece + 1) * nk_all / nsplit;
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
    a_src[i] = base + kc * 8 + (size_t)kb * BK;
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
    b_src[i] = w + ((size_t)tile.e * N + n) * K + kc * 8 + (size_t)kb * BK;
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

  // The weights: each byte of a tile's B slice is read by this block only;
  // with NT they stream through as non-temporal loads.
  auto load_b = [](const uint16_t* q) -> u32x4 {
    if constexpr (NT)
      return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q));
    else
      return *reinterpret_cast<const u32x4*>(q);
  };
  u32x4 ra[AC], rb[BC];
#define MOE_GLOAD(k0)                                                                     \
  do {                                                                                    \
    _Pragma("unroll") for (int i = 0; i < AC; ++i) ra[i] =                                \
        *reinterpret_cast<const u32x4*>(a_src[i] + (k0));                                 \
    _Pragma("unroll") for (int i = 0; i < BC; ++i) rb[i] = load_b(b_src[i] + (k0));        \
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
  const int nk = ke - kb;
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
  if (piece >= 0) {
    // A piece of a split tail tile: the raw fp32 sums, row-major over the
    // tile's BM rows and NB*BN columns (gate columns, then up columns); rows
    // past the tile's end are not stored (the reduce reads none of them).
    float* part = p.tail_part + (size_t)tail_slot * p.tail_slot_floats;
    const int vrows = tile.m_end - tile.m0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int rl = wm * WM + mi * 32 + 8 * (i >> 2) + 4 * lk + (i & 3);
            if (rl < vrows) part[rl * BROWS + nb * BN + wn * WN + ni * 32 + lr] = acc[nb][mi][ni][i];
          }
    return;
  }
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
            out[col] = f32_to_bf16_bits(swiglu_act(g, u, p.swiglu_limit));
            if (p.save_p1) save_factors(p, (size_t)grow * N + col, g, u);
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

// Reduce of the split tail tiles of gemm_bf16_kernel.  Each XCD's blocks
// (block b runs on XCD b % 8, whose L2 holds the partials) stride over that
// XCD's tail tiles x 4-column vectors of their rows: a thread loads the
// vector of every piece (gate and up halves for gate/up) before it adds them
// in piece order, then runs the epilogue on the four columns.
template <int BM, int BN, bool GATEUP>
__global__ __launch_bounds__(NTHREADS) void gemm_tail_reduce_flat_kernel(GemmParams p) {
  constexpr int NB = GATEUP ? 2 : 1, W = NB * BN, V = BN / 4;
  static_assert(BN % 4 == 0, "4-column vectors");
  const int xcd = blockIdx.x % kXcds, bx = blockIdx.x / kXcds, nbx = gridDim.x / kXcds;
  const int r = p.tail_meta[2 * xcd], ns = p.tail_meta[2 * xcd + 1];
  const int N = GATEUP ? p.hidden : p.D;
  const size_t SLOT = p.tail_slot_floats;
  for (int idx = bx * NTHREADS + threadIdx.x; idx < r * BM * V; idx += nbx * NTHREADS) {
    const int j = idx / (BM * V), w = idx % (BM * V);
    const int rl = w / V, cl = 4 * (w % V);
    const int32_t* d = p.tail_desc + (size_t)(xcd * kTailSlots + j) * 4;
    const int m0 = d[1], m_end = d[2], col = d[3] * BN + cl;
    const int row = m0 + rl;
    if (row >= m_end || col >= N) continue;  // N is a multiple of 64: all 4 columns valid
    // (the row's assignment index goes out ahead of the partials)
    const int ra = (!GATEUP && p.gate_w && p.row_to_assign) ? p.row_to_assign[row] : -1;
    const float* part0 = p.tail_part + (size_t)(xcd * kTailSlots + j * ns) * SLOT + rl * W + cl;
    f32x4 v[NB][16];
#pragma unroll
    for (int pc = 0; pc < 16; ++pc)
      if (pc < ns) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          v[nb][pc] = *reinterpret_cast<const f32x4*>(part0 + (size_t)pc * SLOT + nb * BN);
      }
    f32x4 a[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      a[nb] = v[nb][0];
#pragma unroll
      for (int pc = 1; pc < 16; ++pc)
        if (pc < ns) a[nb] += v[nb][pc];
    }
    const size_t o = (size_t)row * N + col;
    uint16_t q[4];
    if constexpr (GATEUP) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        q[u] = f32_to_bf16_bits(swiglu_act(a[0][u], a[NB - 1][u], p.swiglu_limit));
        if (p.save_p1) save_factors(p, o + u, a[0][u], a[NB - 1][u]);
      }
    } else {
      const float gw = ra >= 0 ? p.gate_w[ra] : 1.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) q[u] = f32_to_bf16_bits(gw * a[0][u]);
    }
    uint16_t* out = static_cast<uint16_t*>(GATEUP ? p.hbuf : p.y) + o;
    *reinterpret_cast<uint2*>(out) = make_uint2((uint32_t)q[0] | ((uint32_t)q[1] << 16),
                                                (uint32_t)q[2] | ((uint32_t)q[3] << 16));
  }
}

// Epilogue of a finished tile (32x32 accumulator layout: element i of lane l
// is row 8*(i/4) + 4*(l/32) + (i%4), column l%32): SiLU(gate)*up into Hb, or
// the gate weight times the down product into Y, rounded once to bf16.
template <class C, bool GATEUP>
__device__ __forceinline__ void dma_epilogue(const GemmParams& p, int m0, int m_end, int n0,
                                             int wm, int wn, int lr, int lk,
                                             const f32x16 (&acc)[C::NB][C::MI][C::NI],
                                             const float* row_gw) {
  const int N = GATEUP ? p.hidden : p.D;
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int grow = m0 + wm * C::WM + mi * 32 + 8 * (i >> 2) + 4 * lk + (i & 3);
      if (grow >= m_end) continue;
      if constexpr (GATEUP) {
        uint16_t* out = static_cast<uint16_t*>(p.hbuf) + (size_t)grow * N;
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni) {
          const int col = n0 + wn * C::WN + ni * 32 + lr;
          if (col < N) {
            out[col] = f32_to_bf16_bits(
                swiglu_act(acc[0][mi][ni][i], acc[1][mi][ni][i], p.swiglu_limit));
            if (p.save_p1)
              save_factors(p, (size_t)grow * N + col, acc[0][mi][ni][i], acc[1][mi][ni][i]);
          }
        }
      } else {
        const float gw = row_gw[grow - m0];
        uint16_t* out = static_cast<uint16_t*>(p.y) + (size_t)grow * N;
#pragma unroll
        for (int ni = 0; ni < C::NI; ++ni) {
          const int col = n0 + wn * C::WN + ni * 32 + lr;
          if (col < N) out[col] = f32_to_bf16_bits(gw * acc[0][mi][ni][i]);
        }
      }
    }
  }
}

// Partial tiles are stored in accumulator order, vector v of thread t at
// [v][t], so every store and load of a wave covers 1 KB contiguously.
template <class C>
constexpr int partial_vectors() { return C::NB * C::MI * C::NI * 4; }

// The same epilogue through LDS, for tiles of BM rows x BN output columns
// whose bf16 result fits the four 32 KB stage buffers: each wave writes its
// results as [row][column] bf16 (16-byte chunk c of row r at c ^ 4*((r/4)%4),
// so the two rows one write touches use different banks), then every thread
// stores whole 16-byte row chunks, full 128-byte lines per row.  The caller
// has passed the k-loop; the first barrier makes the stage buffers free.
//
// The LDS address of accumulator element (mi, i, ni) splits into a per-lane
// part, computed once, and a compile-time part that goes into the write's
// immediate offset: a 32-row block (mi) starts at a multiple of 16 rows, so
// the row's swizzle term 4*((r/4)%4) is 4*((2*(i/4) + lane/32) % 4), which
// depends on the lane and on the parity of i/4 only.  The clamp of the
// SwiGLU (swiglu_limit) is decided once per tile, not per element.
template <class C, bool GATEUP, bool CLAMP>
__device__ __forceinline__ void staged_write(const GemmParams& p, int wm, int wn, int lr, int lk,
                                             const f32x16 (&acc)[C::NB][C::MI][C::NI],
                                             const float* row_gw, uint16_t* s0, uint16_t* s1,
                                             uint16_t* s2, uint16_t* s3) {
  constexpr int BN = C::BN;
  constexpr int ROWS_PER = 16384 / BN;  // rows of one 32 KB buffer
  static_assert(ROWS_PER % 32 == 0, "a 32-row block lies in one buffer");
  // per-lane element offsets (uint16 units) inside a buffer, by i/4 parity
  int off[C::NI][2];
#pragma unroll
  for (int ni = 0; ni < C::NI; ++ni) {
    const int col = wn * C::WN + ni * 32 + lr;
#pragma unroll
    for (int g = 0; g < 2; ++g)
      off[ni][g] = 4 * lk * BN + (((col >> 3) ^ (4 * ((2 * g + lk) & 3))) << 3) + (col & 7);
  }
  const float lim = p.swiglu_limit;
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi) {
    const int rb = wm * C::WM + mi * 32;  // first row of the block (wave-uniform)
    const int b = rb / ROWS_PER;
    uint16_t* base = (b == 0 ? s0 : b == 1 ? s1 : b == 2 ? s2 : s3) + (rb % ROWS_PER) * BN;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rc = 8 * (i >> 2) + (i & 3);  // row inside the block, less 4*lk
      const float gw = GATEUP ? 1.f : row_gw[rb + rc + 4 * lk];
#pragma unroll
      for (int ni = 0; ni < C::NI; ++ni) {
        float v;
        if constexpr (GATEUP) {
          float g = acc[0][mi][ni][i], u = acc[C::NB - 1][mi][ni][i];
          if constexpr (CLAMP) {
            g = fminf(fmaxf(g, -lim), lim);
            u = fminf(fmaxf(u, -lim), lim);
          }
          v = silu_f32(g) * u;
        } else {
          v = gw * acc[0][mi][ni][i];
        }
        base[off[ni][(i >> 2) & 1] + rc * BN] = f32_to_bf16_bits(v);
      }
    }
  }
}

// NTS: the rows leave as non-temporal stores (the large tiles' hidden and
// expert rows, hundreds of MB, would only displace cached operands).
template <class C, bool GATEUP, bool NTS>
__device__ __forceinline__ void dma_epilogue_staged(
    const GemmParams& p, int m0, int m_end, int n0, int wm, int wn, int lr, int lk,
    const f32x16 (&acc)[C::NB][C::MI][C::NI], const float* row_gw, uint16_t* s0, uint16_t* s1,
    uint16_t* s2, uint16_t* s3) {
  constexpr int BM = C::WM * (C::NW / C::WGN), BN = C::BN;
  constexpr int ROWS_PER = 16384 / BN;   // rows of one 32 KB buffer
  constexpr int CPR = BN / 8;            // 16-byte chunks per row
  static_assert(BM <= 4 * ROWS_PER && CPR >= 16, "staged epilogue shape");
  auto at = [&](int r, int c) -> uint16_t* {  // chunk c of tile row r
    const int b = r / ROWS_PER, rl = r % ROWS_PER;
    uint16_t* base = b == 0 ? s0 : b == 1 ? s1 : b == 2 ? s2 : s3;
    return base + rl * BN + ((c ^ (4 * ((r >> 2) & 3))) << 3);
  };
  const int N = GATEUP ? p.hidden : p.D;
  __syncthreads();
  if (GATEUP && p.swiglu_limit > 0.f)
    staged_write<C, GATEUP, true>(p, wm, wn, lr, lk, acc, row_gw, s0, s1, s2, s3);
  else
    staged_write<C, GATEUP, false>(p, wm, wn, lr, lk, acc, row_gw, s0, s1, s2, s3);
  __syncthreads();
  uint16_t* out = static_cast<uint16_t*>(GATEUP ? p.hbuf : p.y);
  for (int q = threadIdx.x; q < BM * CPR; q += C::NT) {
    const int r = q / CPR, c = q % CPR;
    const int row = m0 + r, col = n0 + c * 8;
    if (row >= m_end || col >= N) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(at(r, c));
    if constexpr (NTS)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + (size_t)row * N + col));
    else
      *reinterpret_cast<u32x4*>(out + (size_t)row * N + col) = v;
  }
}

// Only the 32-row blocks that hold rows of the tile are stored (wave_rows:
// the tile's rows from this wave's first row on); the reduce reads no others.
template <class C, bool GATEUP>
__device__ __forceinline__ void dma_store_partial(float* slot, int tid, int wave_rows,
                                                  const f32x16 (&acc)[C::NB][C::MI][C::NI]) {
  static_assert((size_t)partial_vectors<C>() * C::NT * 16 <= kTailSlotBytes, "tail slot size");
  f32x4* dst = reinterpret_cast<f32x4*>(slot);
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
      if (mi * 32 < wave_rows)
#pragma unroll
      for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int v = ((nb * C::MI + mi) * C::NI + ni) * 4 + q;
          dst[v * C::NT + tid] = f32x4{acc[nb][mi][ni][4 * q], acc[nb][mi][ni][4 * q + 1],
                                       acc[nb][mi][ni][4 * q + 2], acc[nb][mi][ni][4 * q + 3]};
        }
}

// Sum of a split tail tile's pieces and its epilogue.  Each XCD's blocks
// (block b runs on XCD b % 8, whose L2 holds the partials) stride over that
// XCD's tail tiles x the f32x4 accumulator vectors of the GEMM block: a
// thread loads one vector of every piece (both halves for gate/up) before
// adding them in piece order, and writes the 4 rows x 1 column they hold.
template <int BM, int BNB, int BK, int S, int WGM, int NWV, bool GATEUP>
__global__ __launch_bounds__(256) void gemm_tail_reduce_kernel(GemmParams p) {
  using C = DmaCfg<BM, BNB, BK, S, WGM, NWV, GATEUP>;
  constexpr int VPT = C::MI * C::NI * 4;  // f32x4 vectors of one GEMM thread per NB part
  constexpr int PER_TILE = VPT * C::NT;
  const size_t SLOT = p.tail_slot_floats;
  const int xcd = blockIdx.x % kXcds, bx = blockIdx.x / kXcds, nbx = gridDim.x / kXcds;
  const int r = p.tail_meta[2 * xcd], ns = p.tail_meta[2 * xcd + 1];
  const int N = GATEUP ? p.hidden : p.D;
  for (int idx = bx * 256 + threadIdx.x; idx < r * PER_TILE; idx += nbx * 256) {
    const int j = idx / PER_TILE, w = idx % PER_TILE;
    const int vv = w / C::NT, tid = w % C::NT;
    const int mi = vv / (C::NI * 4), ni = (vv / 4) % C::NI, q = vv % 4;
    const int32_t* d = p.tail_desc + (size_t)(xcd * kTailSlots + j) * 4;
    const int m0 = d[1], m_end = d[2], nt = d[3];
    const int lane = tid & 63, wv = tid >> 6, wm = wv / C::WGN, wn = wv % C::WGN;
    // accumulator element 4q+u of (mi, ni): row 8q + 4*(lane/32) + u of the
    // 32-row block, column lane % 32 (as in dma_store_partial's order)
    const int row0 = m0 + wm * C::WM + mi * 32 + 8 * q + 4 * (lane >> 5);
    const int col = nt * C::BN + wn * C::WN + ni * 32 + (lane & 31);
    if (row0 >= m_end || col >= N) continue;
    // The down GEMM's gate weights of the four rows: their index loads go
    // out ahead of the partials so that the two dependent lookups overlap
    // the partial loads instead of following them.
    int ra[4];
    const bool gated = !GATEUP && p.gate_w && p.row_to_assign;
    if (gated) {
#pragma unroll
      for (int u = 0; u < 4; ++u) ra[u] = row0 + u < m_end ? p.row_to_assign[row0 + u] : -1;
    }
    const float* base = p.tail_part + (size_t)(xcd * kTailSlots + j * ns) * SLOT;
    f32x4 x[C::NB][16];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      const int v = ((nb * C::MI + mi) * C::NI + ni) * 4 + q;
#pragma unroll
      for (int pc = 0; pc < 16; ++pc)
        if (pc < ns)
          x[nb][pc] = reinterpret_cast<const f32x4*>(base + pc * SLOT)[v * C::NT + tid];
    }
    float gw[4] = {1.f, 1.f, 1.f, 1.f};
    if (gated) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (ra[u] >= 0) gw[u] = p.gate_w[ra[u]];
    }
    f32x4 sum[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      sum[nb] = x[nb][0];
#pragma unroll
      for (int pc = 1; pc < 16; ++pc)
        if (pc < ns) sum[nb] += x[nb][pc];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = row0 + u;
      if (row >= m_end) break;
      const size_t o = (size_t)row * N + col;
      if constexpr (GATEUP) {
        const float g = sum[0][u], up = sum[C::NB - 1][u];
        static_cast<uint16_t*>(p.hbuf)[o] = f32_to_bf16_bits(swiglu_act(g, up, p.swiglu_limit));
        if (p.save_p1) save_factors(p, o, g, up);
      } else {
        static_cast<uint16_t*>(p.y)[o] = f32_to_bf16_bits(gw[u] * sum[0][u]);
      }
    }
  }
}

template <int BM, int BNB, int BK, int S, int WGM, int NWV, bool GATEUP>
__global__ __launch_bounds__(64 * NWV) void gemm_dma_kernel(GemmParams p, int tail_slots) {
  using C = DmaCfg<BM, BNB, BK, S, WGM, NWV, GATEUP>;
  constexpr int KCH = C::KCH, MI = C::MI, NI = C::NI, NB = C::NB;
  __shared__ __attribute__((aligned(1024))) uint16_t sA0[BM * BK];
  __shared__ __attribute__((aligned(1024))) uint16_t sA1[BM * BK];
  __shared__ __attribute__((aligned(1024))) uint16_t sA2[S > 2 ? BM * BK : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t sA3[S > 3 ? BM * BK : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t sB0[BNB * BK];
  __shared__ __attribute__((aligned(1024))) uint16_t sB1[BNB * BK];
  __shared__ __attribute__((aligned(1024))) uint16_t sB2[S > 2 ? BNB * BK : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t sB3[S > 3 ? BNB * BK : 8];
  __shared__ int s_scan[NTHREADS + 4];
  __shared__ float s_gw[GATEUP ? 1 : BM];

  Tile tile;
  int piece, nsplit, tail_slot;
  if (!decode_job<BM, C::BN, GATEUP>(p, tail_slots, s_scan, tile, piece, nsplit, tail_slot))
    return;
  if constexpr (!GATEUP) {
    // The gate weight of each of the tile's rows for the epilogue, fetched
    // once ahead of the k-loop rather than per row at the end.
    if (threadIdx.x < BM) {
      const int row = tile.m0 + (int)threadIdx.x;
      s_gw[threadIdx.x] = (p.gate_w && p.row_to_assign && row < tile.m_end)
                              ? p.gate_w[p.row_to_assign[row]]
                              : 1.f;
    }
    __syncthreads();
  }

  const int K = GATEUP ? p.D : p.hidden;
  const int N = GATEUP ? p.hidden : p.D;
  const int n0 = tile.nt * C::BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)

  // Buffer resources: A is x (gathered rows) or this tile's rows of Hb; B is
  // this expert's weight slice.  Offsets stay below 4 GB (checked on the host).
  const uint16_t* a_base = GATEUP ? static_cast<const uint16_t*>(p.x)
                                  : static_cast<const uint16_t*>(p.hbuf) + (size_t)tile.m0 * K;
  const uint32_t a_bytes = GATEUP ? (uint32_t)((size_t)p.T * K * 2)
                                  : (uint32_t)((size_t)(tile.m_end - tile.m0) * K * 2);
  const __amdgpu_buffer_rsrc_t rA =
      __builtin_amdgcn_make_buffer_rsrc((void*)a_base, 0, (int)a_bytes, 0x00020000);
  const uint16_t* wg = static_cast<const uint16_t*>(GATEUP ? p.w_gate : p.w_down) +
                       (size_t)tile.e * N * K;
  const uint16_t* wu = GATEUP ? static_cast<const uint16_t*>(p.w_up) + (size_t)tile.e * N * K
                              : wg;
  const uint32_t w_bytes = (uint32_t)((size_t)N * K * 2);
  const __amdgpu_buffer_rsrc_t rG =
      __builtin_amdgcn_make_buffer_rsrc((void*)wg, 0, (int)w_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rU =
      __builtin_amdgcn_make_buffer_rsrc((void*)wu, 0, (int)w_bytes, 0x00020000);

  // Per-lane byte offsets of each 1 KB wave load (k-step 0).
  uint32_t a_off[C::A_LD];
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) {
    const int slot = (wave + C::NW * i) * 64 + lane;
    const int r = slot / KCH, pc = slot % KCH, lc = pc ^ swz_k<KCH>(r);
    int grow = tile.m0 + r;
    if (grow >= tile.m_end) grow = tile.m0;
    uint32_t rowoff;
    if constexpr (GATEUP) {
      const int tok = p.row_to_assign ? p.row_to_assign[grow] / p.k : grow;
      rowoff = (uint32_t)tok * (uint32_t)K * 2u;
    } else {
      rowoff = (uint32_t)(grow - tile.m0) * (uint32_t)K * 2u;
    }
    a_off[i] = rowoff + (uint32_t)lc * 16u;
  }
  uint32_t b_off[C::B_LD];
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) {
    const int slot = (wave + C::NW * i) * 64 + lane;
    const int r = slot / KCH, pc = slot % KCH, lc = pc ^ swz_k<KCH>(r);
    int n = n0 + (GATEUP ? (r % C::BN) : r);
    if (n >= N) n = n0;
    b_off[i] = (uint32_t)n * (uint32_t)K * 2u + (uint32_t)lc * 16u;
  }
  // B rows [0, BN) come from rG, [BN, 2BN) from rU (GATEUP); wave loads never
  // straddle the two halves because BN*KCH is a multiple of 64.

  // K range: all k-steps, or this piece's share of a split tail tile.
  const int nk = K / BK;
  const int kb = piece < 0 ? 0 : piece * nk / nsplit;
  const int ke = piece < 0 ? nk : (piece + 1) * nk / nsplit;
#pragma unroll
  for (int i = 0; i < C::A_LD; ++i) a_off[i] += (uint32_t)kb * BK * 2u;
#pragma unroll
  for (int i = 0; i < C::B_LD; ++i) b_off[i] += (uint32_t)kb * BK * 2u;

  const DmaLoads<C, GATEUP> ld{rA, rG, rU, a_off, b_off, wave};
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

  // Row blocks of this wave that hold valid rows (the last row tile of an
  // expert is usually partial); the others skip their reads and MFMAs.  Only
  // tiles with four row blocks per wave take the second path: with fewer the
  // saving is small and the extra code makes the kernel spill.
  const int mi_n = min(C::MI, max(0, (tile.m_end - tile.m0 - wm * C::WM + 31) / 32));
  // The only row tile of its expert is the only block that reads this B
  // slice: its weights stream through with non-temporal loads (several row
  // tiles of one expert share the slice through L2 and keep the default).
  if (!(p.stream_weights && tile.rt == 1)) {
    if (C::MI < 4 || mi_n == C::MI)
      dma_mainloop<C, GATEUP, false>(ld, ke - kb, C::MI, wm, wn, lr, lk, acc, sA0, sA1, sA2,
                                     sA3, sB0, sB1, sB2, sB3);
    else if constexpr (C::MI >= 4)
      dma_mainloop<C, GATEUP, true>(ld, ke - kb, mi_n, wm, wn, lr, lk, acc, sA0, sA1, sA2, sA3,
                                    sB0, sB1, sB2, sB3);
  } else {
    if (C::MI < 4 || mi_n == C::MI)
      dma_mainloop<C, GATEUP, false, false, false, 2>(ld, ke - kb, C::MI, wm, wn, lr, lk, acc,
                                                      sA0, sA1, sA2, sA3, sB0, sB1, sB2, sB3);
    else if constexpr (C::MI >= 4)
      dma_mainloop<C, GATEUP, true, false, false, 2>(ld, ke - kb, mi_n, wm, wn, lr, lk, acc,
                                                     sA0, sA1, sA2, sA3, sB0, sB1, sB2, sB3);
  }
  if (piece >= 0) {
    dma_store_partial<C, GATEUP>(p.tail_part + (size_t)tail_slot * p.tail_slot_floats, tid,
                                 tile.m_end - tile.m0 - wm * C::WM, acc);
    return;
  }
  // The bf16 results go out through the free stage buffers when those hold
  // them (saving the SwiGLU factors stores per element instead).
  if (!(GATEUP && p.save_p1)) {
    constexpr int OUT_BYTES = BM * C::BN * 2;
    if constexpr (BM == 256 && BNB == 256 && BK == 64 && S == 2) {
      dma_epilogue_staged<C, GATEUP, true>(p, tile.m0, tile.m_end, n0, wm, wn, lr, lk, acc,
                                           s_gw, sA0, sA1, sB0, sB1);
      return;
    } else if constexpr (BNB * BK * 2 == 32768 && OUT_BYTES <= 2 * 32768) {
      // 32 KB B stage buffers (the 128-row tiles): two of them hold the tile
      dma_epilogue_staged<C, GATEUP, false>(p, tile.m0, tile.m_end, n0, wm, wn, lr, lk, acc,
                                            s_gw, sB0, sB1, sB0, sB1);
      return;
    }
  }
  dma_epilogue<C, GATEUP>(p, tile.m0, tile.m_end, n0, wm, wn, lr, lk, acc, s_gw);
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
            swiglu_act(acc[0][i][j], acc[NB - 1][i][j], p.swiglu_limit);
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

// Resident blocks per XCD of one kernel on the current device (0 when the
// CUs do not split evenly over the XCDs); cached per device.
template <class Kern>
int slots_per_xcd(Kern kern, int threads) {
  static int cache[64];
  static bool have[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!have[dev]) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, 0) != hipSuccess)
      return 0;
    cache[dev] = (cus % kXcds == 0) ? std::min(kTailSlots, occ * cus / kXcds) : 0;
    have[dev] = true;
  }
  return cache[dev];
}

template <int BM, int BN, int WGM, bool GATEUP, bool NT>
hipError_t launch_bf16_nt(const GemmParams& p, hipStream_t s) {
  const auto kern = gemm_bf16_kernel<BM, BN, WGM, GATEUP, NT>;
  const int N = GATEUP ? p.hidden : p.D;
  const int mt = mtiles_bound(p, BM);
  const long long tiles = (long long)mt * ((N + BN - 1) / BN);
  if (tiles <= 0) return hipSuccess;
  constexpr size_t part_floats = (size_t)BM * (GATEUP ? 2 : 1) * BN;
  const int slots =
      p.tail_part && part_floats <= p.tail_slot_floats ? slots_per_xcd(kern, NTHREADS) : 0;
  // Every XCD gets at most ceil(tiles/8) tiles plus at most `slots` extra
  // blocks for the pieces of its split tail.
  const long long nblocks = kXcds * ((tiles + kXcds - 1) / kXcds + slots);
  hipLaunchKernelGGL(kern, dim3((unsigned)nblocks), dim3(NTHREADS), 0, s, p, slots);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || slots == 0) return err;
  hipLaunchKernelGGL((gemm_tail_reduce_flat_kernel<BM, BN, GATEUP>), dim3(kXcds * MOE_REDUCE_BLOCKS),
                     dim3(NTHREADS), 0, s, p);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, bool GATEUP>
hipError_t launch_bf16(const GemmParams& p, hipStream_t s) {
  return p.stream_weights ? launch_bf16_nt<BM, BN, WGM, GATEUP, true>(p, s)
                          : launch_bf16_nt<BM, BN, WGM, GATEUP, false>(p, s);
}

template <int BM, int BNB, int BK, int S, int WGM, int NWV, bool GATEUP>
hipError_t launch_dma(const GemmParams& p, hipStream_t s) {
  using C = DmaCfg<BM, BNB, BK, S, WGM, NWV, GATEUP>;
  const auto kern = gemm_dma_kernel<BM, BNB, BK, S, WGM, NWV, GATEUP>;
  const int N = GATEUP ? p.hidden : p.D;
  const int mt = mtiles_bound(p, BM);
  const long long tiles = (long long)mt * ((N + C::BN - 1) / C::BN);
  if (tiles <= 0) return hipSuccess;
  constexpr size_t part_floats = (size_t)partial_vectors<C>() * C::NT * 4;
  const int slots =
      p.tail_part && part_floats <= p.tail_slot_floats ? slots_per_xcd(kern, C::NT) : 0;
  // Every XCD gets at most ceil(tiles/8) tiles plus at most `slots` extra
  // blocks for the pieces of its split tail.
  const long long nblocks = kXcds * ((tiles + kXcds - 1) / kXcds + slots);
  hipLaunchKernelGGL(kern, dim3((unsigned)nblocks), dim3(C::NT), 0, s, p, slots);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || slots == 0) return err;
  hipLaunchKernelGGL((gemm_tail_reduce_kernel<BM, BNB, BK, S, WGM, NWV, GATEUP>),
                     dim3(kXcds * MOE_REDUCE_BLOCKS), dim3(256), 0, s, p);
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

// Large-tile configuration (rows, B-tile rows, k-step, stages, wave rows,
// waves);
// overridable at build time for tuning sweeps.
#ifndef MOE_GU_CFG
#define MOE_GU_CFG 256, 256, 64, 2, 2, 8
#endif
#ifndef MOE_DN_CFG
#define MOE_DN_CFG 256, 256, 64, 2, 2, 8
#endif
// Average rows per group from which the 256-row tiles are used.
#ifndef MOE_LARGE_MIN_ROWS
#define MOE_LARGE_MIN_ROWS 192
#endif
// Smaller groups of 64 or more rows on average: 128-row tiles, three stages
// (on the capacity-limited Switch-shaped layer, whose short k-loops wait on
// HBM, 15% ahead of two; 256-column down tiles 9% ahead of 512).
#ifndef MOE_GU_CFG_M
#define MOE_GU_CFG_M 128, 512, 32, 3, 2, 8
#endif
#ifndef MOE_DN_CFG_M
#define MOE_DN_CFG_M 128, 256, 64, 3, 2, 8
#endif

// Groups under this many rows on average use the 32-row register-staged
// tiles (gate/up: MOE_SMALL_GU_BN output columns, down: MOE_SMALL_DN_BN).
#ifndef MOE_SMALL_MAX_ROWS
#define MOE_SMALL_MAX_ROWS 64
#endif
#ifndef MOE_SMALL_GU_BN
#define MOE_SMALL_GU_BN 128
#endif
#ifndef MOE_SMALL_DN_BN
#define MOE_SMALL_DN_BN 256
#endif

// Offsets inside the buffer resources of the large-tile kernel are 32-bit, and
// its k-loop needs K (D for gate/up, hidden for down) to be a multiple of BK.
template <class C1, class C2>
bool dma_fits(const GemmParams& p) {
  if (p.D % C1::BK || p.hidden % C2::BK) return false;
  const size_t lim = (size_t)1 << 31;
  const size_t x_bytes = (size_t)p.T * p.D * 2;
  const size_t w_bytes = (size_t)p.hidden * p.D * 2;
  const size_t hb_tile = (size_t)256 * p.hidden * 2;
  return x_bytes < lim && w_bytes < lim && hb_tile < lim;
}

hipError_t launch_grouped_swiglu(const GemmParams& p_in, bool bf16, hipStream_t s) {
  hipError_t err;
  GemmParams p = p_in;
  p.stream_weights = (double)p.n_groups * 3.0 * p.D * p.hidden * 2.0 >
                     (double)MOE_STREAM_MIN_BYTES;
  if (!bf16) {
    if ((err = launch_f32<true>(p, s)) != hipSuccess) return err;
    return launch_f32<false>(p, s);
  }
  // Rows per group decide the row-tile height: decode-sized groups use 32-row
  // tiles so that MFMA work is not spent on padding.
  const int rows = p.expert_offsets ? p.max_rows : p.T;
  const int groups = p.expert_offsets ? p.n_groups : 1;
  if ((long long)rows < (long long)MOE_SMALL_MAX_ROWS * groups) {
    if ((err = launch_bf16<32, MOE_SMALL_GU_BN, 1, true>(p, s)) != hipSuccess) return err;
    return launch_bf16<32, MOE_SMALL_DN_BN, 1, false>(p, s);
  }
  using GU = DmaCfg<MOE_GU_CFG, true>;
  using DN = DmaCfg<MOE_DN_CFG, false>;
  using GUM = DmaCfg<MOE_GU_CFG_M, true>;
  using DNM = DmaCfg<MOE_DN_CFG_M, false>;
  if ((long long)rows >= (long long)MOE_LARGE_MIN_ROWS * groups && dma_fits<GU, DN>(p)) {
    if ((err = launch_dma<MOE_GU_CFG, true>(p, s)) != hipSuccess) return err;
    return launch_dma<MOE_DN_CFG, false>(p, s);
  }
  // Groups of 64-191 rows on average: a capacity limit with a skewed router
  // can leave rows in a few experts only, whose weights then stay in the
  // Infinity Cache from one call to the next; their loads keep the default
  // policy (streaming loads measured 26% slower on the Switch-shaped layer).
  p.stream_weights = 0;
  if (dma_fits<GUM, DNM>(p)) {
    if ((err = launch_dma<MOE_GU_CFG_M, true>(p, s)) != hipSuccess) return err;
    return launch_dma<MOE_DN_CFG_M, false>(p, s);
  }
  if ((err = launch_bf16<128, 128, 2, true>(p, s)) != hipSuccess) return err;
  return launch_bf16<128, 256, 2, false>(p, s);
}

}  // namespace moe
