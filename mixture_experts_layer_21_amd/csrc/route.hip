// Routing: router GEMM, fp32 scores, optional group limit, top-k, gate
// weights, and per-block partial sums for the balance and z losses.
//
// Follows "Lab: build a tiny MoE in PyTorch" ("Full implementation": Linear
// router, float32 softmax, topk, renormalised weights, bincount, balance and
// z losses) and "2.9 Mixture-of-Experts (MoE) Architectures" ("The Router":
// selection-only per-expert bias), with the NeMo Gate switches score_func,
// n_groups / topk_groups and route_scale.
//
// Routers of at most 64 experts whose weights fit route_fused run as one
// kernel, route_fused_kernel (below): each block computes its tokens' logits
// over all of K and selects from them.  Larger routers take two kernels:
//  * route_logits_kernel: the [T x E] logits as split-K partial sums.  A
//    256-thread block covers 32 tokens x up to 64 experts x one K range; each
//    wave runs 16x16 MFMA tiles (bf16 x bf16: 16x16x32 bf16, products exact;
//    bf16 x with fp32 W: the same MFMAs on an exact three-term bf16 split of
//    W; fp32 x: 16x16x4 fp32).  Waves sharing an expert tile split the
//    k-steps and are summed through LDS in a fixed order.
//  * route_select_kernel: the block first adds the K-split partials of its
//    tokens (route_tile: 8 or 32) in split order into LDS; then one wave per token does the
//    scores, group limit, k arg-max rounds (ties to the lower expert index)
//    and weights.  Lane l holds experts l, l+64, l+128, l+192.  Every
//    reduction has a fixed order, so results are bit-reproducible.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int RT = kRouteTile;
constexpr int NTHREADS = 256;
constexpr int NWAVES = NTHREADS / MOE_WAVE;

// Four consecutive elements starting at p (16-byte or 8-byte aligned) as fp32.
__device__ __forceinline__ f32x4 load4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ f32x4 load4(const uint16_t* p) {
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xffff0000u),
               __uint_as_float(q.y << 16), __uint_as_float(q.y & 0xffff0000u)};
}

// Partial logits part[ks][t][e] = sum over this block's K range of x[t,k] W[e,k].
// MFMA operand mapping (both operands alike, so any fixed k permutation inside
// a step gives the same products): 16x16x32 bf16: lane l holds row l%16 and
// k = 8*(l/16) .. +7; 16x16x4 fp32 (four per 16-wide step): lane l holds row
// l%16 and k = 4*(l/16) + j in the j-th MFMA.  Output element i of lane l is
// row 4*(l/16) + i, column l%16.
// Exact split of eight fp32 values into three bf16 terms, w = hi + mid + lo:
// hi is w rounded to bf16, mid the rounded remainder, lo the remainder of
// that, which has at most eight significant bits and is therefore exact in
// bf16 (for |w| far above the bf16 underflow threshold, as router weights
// are).  A bf16 x times each term is exact in fp32.
__device__ __forceinline__ void split3_bf16(const f32x4 a, const f32x4 b, bf16x8& hi, bf16x8& mid,
                                            bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float w = i < 4 ? a[i] : b[i - 4];
    const __bf16 h = static_cast<__bf16>(w);
    const float r = w - static_cast<float>(h);
    const __bf16 m = static_cast<__bf16>(r);
    hi[i] = h;
    mid[i] = m;
    lo[i] = static_cast<__bf16>(r - static_cast<float>(m));
  }
}

// SPLIT3 (bf16 x, fp32 W): each fp32 weight is split into three bf16 terms
// and the products go through 16x16x32 bf16 MFMAs (exact products, fp32
// sums), a sixteenth of the matrix-core time of 16x16x4 fp32 MFMAs each.
template <typename XT, typename WT, bool BF16, bool SPLIT3 = false>
__global__ __launch_bounds__(NTHREADS) void route_logits_kernel(RouteParams p) {
  constexpr int KSTEP = (BF16 || SPLIT3) ? 32 : 16;
  const XT* x = static_cast<const XT*>(p.x);
  const WT* w = static_cast<const WT*>(p.w_router);
  const int NT = (p.E + 15) / 16;
  const int NTB = NT >= 4 ? 4 : (NT >= 2 ? 2 : 1);
  const int WPN = NWAVES / NTB;  // waves per expert tile (they split the k-steps)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  const int nt = blockIdx.y * NTB + wave / WPN;
  const int phase = wave % WPN;
  const int t0 = blockIdx.x * RT;
  const int nsteps = p.D / KSTEP;
  const int per = (nsteps + p.ksplit - 1) / p.ksplit;
  const int s0 = blockIdx.z * per, s1 = min(nsteps, s0 + per);
  const bool active = nt < NT;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  if (active) {
    const int r = lane & 15, kq = lane >> 4;
    const int ta = min(t0 + r, p.T - 1), tb = min(t0 + 16 + r, p.T - 1);
    const int e = min(nt * 16 + r, p.E - 1);
    if constexpr (BF16) {
      const uint16_t* pa = reinterpret_cast<const uint16_t*>(x) + (size_t)ta * p.D + kq * 8;
      const uint16_t* pb = reinterpret_cast<const uint16_t*>(x) + (size_t)tb * p.D + kq * 8;
      const uint16_t* pw = reinterpret_cast<const uint16_t*>(w) + (size_t)e * p.D + kq * 8;
      int s = s0 + phase;
      // Four k-steps in flight per iteration.
      for (; s + 3 * WPN < s1; s += 4 * WPN) {
        bf16x8 A0[4], A1[4], B[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k0 = (s + u * WPN) * 32;
          A0[u] = *reinterpret_cast<const bf16x8*>(pa + k0);
          A1[u] = *reinterpret_cast<const bf16x8*>(pb + k0);
          B[u] = *reinterpret_cast<const bf16x8*>(pw + k0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0[u], B[u], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[u], B[u], acc1, 0, 0, 0);
        }
      }
      for (; s < s1; s += WPN) {
        const int k0 = s * 32;
        const bf16x8 A0 = *reinterpret_cast<const bf16x8*>(pa + k0);
        const bf16x8 A1 = *reinterpret_cast<const bf16x8*>(pb + k0);
        const bf16x8 B = *reinterpret_cast<const bf16x8*>(pw + k0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B, acc1, 0, 0, 0);
      }
    } else if constexpr (SPLIT3) {
      const uint16_t* pa = reinterpret_cast<const uint16_t*>(x) + (size_t)ta * p.D + kq * 8;
      const uint16_t* pb = reinterpret_cast<const uint16_t*>(x) + (size_t)tb * p.D + kq * 8;
      const float* pw = reinterpret_cast<const float*>(w) + (size_t)e * p.D + kq * 8;
      int s = s0 + phase;
      // Two k-steps in flight per iteration.
      for (; s + WPN < s1; s += 2 * WPN) {
        bf16x8 A0[2], A1[2];
        f32x4 W0[2], W1[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int k0 = (s + u * WPN) * 32;
          A0[u] = *reinterpret_cast<const bf16x8*>(pa + k0);
          A1[u] = *reinterpret_cast<const bf16x8*>(pb + k0);
          W0[u] = *reinterpret_cast<const f32x4*>(pw + k0);
          W1[u] = *reinterpret_cast<const f32x4*>(pw + k0 + 4);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          bf16x8 h, m, l;
          split3_bf16(W0[u], W1[u], h, m, l);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0[u], h, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[u], h, acc1, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0[u], m, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[u], m, acc1, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0[u], l, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1[u], l, acc1, 0, 0, 0);
        }
      }
      for (; s < s1; s += WPN) {
        const int k0 = s * 32;
        const bf16x8 A0 = *reinterpret_cast<const bf16x8*>(pa + k0);
        const bf16x8 A1 = *reinterpret_cast<const bf16x8*>(pb + k0);
        bf16x8 h, m, l;
        split3_bf16(*reinterpret_cast<const f32x4*>(pw + k0),
                    *reinterpret_cast<const f32x4*>(pw + k0 + 4), h, m, l);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, h, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, h, acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, m, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, m, acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, l, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, l, acc1, 0, 0, 0);
      }
    } else {
      const XT* pa = x + (size_t)ta * p.D + kq * 4;
      const XT* pb = x + (size_t)tb * p.D + kq * 4;
      const WT* pw = w + (size_t)e * p.D + kq * 4;
      for (int s = s0 + phase; s < s1; s += WPN) {
        const int k0 = s * 16;
        const f32x4 a0 = load4(pa + k0), a1 = load4(pb + k0), b = load4(pw + k0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[j], b[j], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[j], b[j], acc1, 0, 0, 0);
        }
      }
    }
  }
  __shared__ f32x4 red[NWAVES][2][MOE_WAVE];
  if (WPN > 1) {  // block-uniform
    red[wave][0][lane] = acc0;
    red[wave][1][lane] = acc1;
    __syncthreads();
    if (phase == 0) {
      for (int ph = 1; ph < WPN; ++ph) {
        acc0 += red[wave + ph][0][lane];
        acc1 += red[wave + ph][1][lane];
      }
    }
  }
  if (active && phase == 0) {
    const int e = nt * 16 + (lane & 15);
    float* out = p.logits_part + (size_t)blockIdx.z * p.T * p.E;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ta = t0 + 4 * (lane >> 4) + i, tb = ta + 16;
      if (e < p.E && ta < p.T) out[(size_t)ta * p.E + e] = acc0[i];
      if (e < p.E && tb < p.T) out[(size_t)tb * p.E + e] = acc1[i];
    }
  }
}

// LDS-tiled router GEMM for bf16 x and W: a block computes BM tokens x 256
// experts over its K range (BK-deep k-steps staged through LDS in two
// buffers, the next k-step's operands in registers meanwhile; a second
// register set for the k-step after that measured no faster); its BM/16
// waves in a (BM/32) x 2 grid each hold 32 tokens x 128 experts as four
// 32x32x16 MFMA tiles.  x is read once per K range instead of once per
// expert tile, the router once per BM tokens.  The 16-byte chunk c of row r
// sits at c ^ rswz(r) in LDS, which keeps the fragment reads conflict-free
// (64-byte rows: (r >> 2) & 3; 128-byte rows: the grouped GEMM's pattern).
template <int KCH>
__device__ __forceinline__ int rswz(int r) {
  if constexpr (KCH == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return (r >> 2) & 3;
}

template <int BM, int BK>
__global__ __launch_bounds__(BM * 4) void route_logits_tiled_kernel(RouteParams p) {
  constexpr int BN = kRouteTiledN, NT = BM * 4, KCH = BK / 8;
  constexpr int AC = BM * KCH / NT, BC = BN * KCH / NT;  // chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];
  const uint16_t* x = static_cast<const uint16_t*>(p.x);
  const uint16_t* w = static_cast<const uint16_t*>(p.w_router);
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;
  const int t0 = blockIdx.x * BM, e0 = blockIdx.y * BN;
  const int nsteps = p.D / BK;
  const int per = (nsteps + p.ksplit - 1) / p.ksplit;
  const int s0 = blockIdx.z * per, s1 = min(nsteps, s0 + per);

  // This thread's 16-byte chunks: AC of A, BC of B (chunk c: row c / KCH).
  const uint16_t* asrc[AC];
  int adst[AC];
#pragma unroll
  for (int i = 0; i < AC; ++i) {
    const int c = tid + NT * i, r = c / KCH, cc = c % KCH;
    asrc[i] = x + (size_t)min(t0 + r, p.T - 1) * p.D + cc * 8;
    adst[i] = r * BK + (cc ^ rswz<KCH>(r)) * 8;
  }
  const uint16_t* bsrc[BC];
  int bdst[BC];
#pragma unroll
  for (int i = 0; i < BC; ++i) {
    const int c = tid + NT * i, r = c / KCH, cc = c % KCH;
    bsrc[i] = w + (size_t)min(e0 + r, p.E - 1) * p.D + cc * 8;
    bdst[i] = r * BK + (cc ^ rswz<KCH>(r)) * 8;
  }
  f32x16 acc[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[ni][i] = 0.f;

  if (s0 < s1) {
    u32x4 ra[AC], rb[BC];
#define MOE_RLOAD(s)                                                                        \
  do {                                                                                      \
    const int k0_ = (s) * BK;                                                               \
    _Pragma("unroll") for (int i = 0; i < AC; ++i) ra[i] =                                  \
        *reinterpret_cast<const u32x4*>(asrc[i] + k0_);                                     \
    _Pragma("unroll") for (int i = 0; i < BC; ++i) rb[i] =                                  \
        *reinterpret_cast<const u32x4*>(bsrc[i] + k0_);                                     \
  } while (0)
#define MOE_RSTORE(buf)                                                                     \
  do {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < AC; ++i)                                          \
        *reinterpret_cast<u32x4*>(&As[buf][adst[i]]) = ra[i];                               \
    _Pragma("unroll") for (int i = 0; i < BC; ++i)                                          \
        *reinterpret_cast<u32x4*>(&Bs[buf][bdst[i]]) = rb[i];                               \
  } while (0)
    MOE_RLOAD(s0);
    MOE_RSTORE(0);
    __syncthreads();
    for (int s = s0; s < s1; ++s) {
      const int cur = (s - s0) & 1;
      if (s + 1 < s1) MOE_RLOAD(s + 1);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int ch = kk * 2 + lk;
        const int r = wm * 32 + lr;
        const bf16x8 af =
            *reinterpret_cast<const bf16x8*>(&As[cur][r * BK + (ch ^ rswz<KCH>(r)) * 8]);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int rb_ = wn * 128 + ni * 32 + lr;
          const bf16x8 bfr =
              *reinterpret_cast<const bf16x8*>(&Bs[cur][rb_ * BK + (ch ^ rswz<KCH>(rb_)) * 8]);
          acc[ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr, acc[ni], 0, 0, 0);
        }
      }
      if (s + 1 < s1) MOE_RSTORE(cur ^ 1);
      __syncthreads();
    }
#undef MOE_RLOAD
#undef MOE_RSTORE
  }
  // Partial logits (an empty K range writes zeros).  32x32 accumulator
  // layout: element i of lane l is row 8*(i/4) + 4*(l/32) + (i%4), column l%32.
  float* out = p.logits_part + (size_t)blockIdx.z * p.T * p.E;
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int e = e0 + wn * 128 + ni * 32 + lr;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = t0 + wm * 32 + 8 * (i >> 2) + 4 * lk + (i & 3);
      if (t < p.T && e < p.E) out[(size_t)t * p.E + e] = acc[ni][i];
    }
  }
}

// ---------------------------------------------------------------------------
// Selection.  Cross-lane steps use DPP inside 16-lane rows (quad permutes,
// half-row and row mirrors) and v_readlane across the four rows, instead of
// LDS permutes: each all-reduce below is four DPP steps plus four readlanes.

constexpr int SEL_THREADS = 512;
constexpr int SEL_WAVES = SEL_THREADS / MOE_WAVE;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <-> 7-i inside each 8 lanes
constexpr int DPP_ROW_MIRROR = 0x140;   // lane i <-> 15-i inside each 16 lanes

__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Sum over the wave; every lane of a row holds the same row sum (partners
// always hold disjoint lane sets, and IEEE addition is commutative), and the
// four row sums are added in the fixed order (r0 + r1) + (r2 + r3).
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<DPP_XOR1>(v);
  v += dpp_f<DPP_XOR2>(v);
  v += dpp_f<DPP_HALF_MIRROR>(v);
  v += dpp_f<DPP_ROW_MIRROR>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f<DPP_XOR1>(v));
  v = fmaxf(v, dpp_f<DPP_XOR2>(v));
  v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)),
               fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ uint32_t wave_max_key(uint32_t v) {
  v = max(v, dpp_u<DPP_XOR1>(v));
  v = max(v, dpp_u<DPP_XOR2>(v));
  v = max(v, dpp_u<DPP_HALF_MIRROR>(v));
  v = max(v, dpp_u<DPP_ROW_MIRROR>(v));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

// Order-preserving unsigned key of a non-NaN float (-0 and +0 equal, as in a
// float comparison).  Key 0 is below every float, including -inf: it marks
// "not selectable".
__device__ __forceinline__ uint32_t okey(float v) {
  const uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-2 of two disjoint sets, each given as (first, second).
__device__ __forceinline__ void top2_merge(float& a1, float& a2, float b1, float b2) {
  if (a1 >= b1) {
    a2 = fmaxf(a2, b1);
  } else {
    a2 = fmaxf(a1, b2);
    a1 = b1;
  }
}
template <int CTRL>
__device__ __forceinline__ void top2_step(float& a1, float& a2) {
  top2_merge(a1, a2, dpp_f<CTRL>(a1), dpp_f<CTRL>(a2));
}

// One arg-max round over the wave: among the keys of this lane's four slots
// (slot j is expert lane + 64 j), the largest key wins; equal keys go to the
// lower expert index.  Returns the winner's lane and slot (wave-uniform).
template <int NS>
__device__ __forceinline__ void wave_argmax_key(const uint32_t (&key)[NS], int& wl, int& wj) {
  uint32_t lk = key[0];
  int lj = 0;
#pragma unroll
  for (int j = 1; j < NS; ++j)
    if (key[j] > lk) {
      lk = key[j];
      lj = j;
    }
  const uint32_t M = wave_max_key(lk);
  wl = 0;
  wj = 0;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const uint64_t m = __ballot(lk == M && lj == j);
    if (m) {
      wl = __ffsll((unsigned long long)m) - 1;
      wj = j;
      break;
    }
  }
}

// Slot j of lane l of a (j and l wave-uniform): every slot is read from lane
// l and the choice is made on the scalar side, so that no register array is
// indexed at run time.
template <int NS>
__device__ __forceinline__ float readlane_slot(const float (&a)[NS], int j, int l) {
  float v = readlane_f(a[0], l);
#pragma unroll
  for (int i = 1; i < NS; ++i) {
    const float u = readlane_f(a[i], l);
    if (j == i) v = u;
  }
  return v;
}

template <int TILE>
struct SelectSmem {
  float lg[TILE * kMaxExperts];    // summed logits of the block's tokens, row stride E
  float pe[SEL_WAVES][kMaxExperts];
  float zw[SEL_WAVES];
  int nv[SEL_WAVES];
  int hist[kMaxExperts];
};

// sqrt(softplus(h)), softplus(h) = log(1 + e^h) written without overflow.
__device__ __forceinline__ float sqrt_softplus(float h) {
  return sqrtf(fmaxf(h, 0.f) + log1pf(expf(-fabsf(h))));
}

// The biases of the experts this lane holds in the selection (lane + 64 j),
// loaded at the start of a kernel so that the loads overlap its first phase.
__device__ __forceinline__ void load_biases(const RouteParams p, float (&lb)[4], float (&sb)[4]) {
  const int lane = lane_id();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    lb[j] = (e < p.E && p.logit_bias) ? p.logit_bias[e] : 0.f;
    sb[j] = (e < p.E && p.select_bias) ? p.select_bias[e] : 0.f;
  }
}

// Selection of a block's nt tokens (t0 ..) from their logits in sm.lg (row
// stride E), published with sm.hist zeroed by a barrier before the call: one
// wave per token computes the scores, group limit, k arg-max rounds (ties to
// the lower expert index) and weights; then the block's P_e and z partial
// sums and expert histogram go to column blk of the per-block arrays.  Lane
// l holds experts l, l+64, l+128, l+192.  Every reduction has a fixed order,
// so results are bit-reproducible.
template <int TILE, int NS>
__device__ __forceinline__ void select_tokens(const RouteParams p, SelectSmem<TILE>& sm, int blk,
                                              int t0, int nt, const float (&lb)[4],
                                              const float (&sb)[4]) {
  const int wave = threadIdx.x / MOE_WAVE, lane = lane_id();
  const int E = p.E, k = p.k;
  // softmax scores are a distribution over the experts; sigmoid and
  // sqrt-softplus scores are per expert and normalised where a sum is needed.
  const bool per_expert = p.score_func != 0;
  const bool by_score = per_expert || p.select_bias != nullptr;
  const int gsz = p.n_groups > 1 ? E / p.n_groups : E;
  // Group limit with a segmented reduction: groups are aligned runs of gsz
  // lanes in one slot when gsz is a power of two below 64.
  const bool seg_groups = p.n_groups > 1 && gsz < 64 && (gsz & (gsz - 1)) == 0;
  bool ok[NS];
  float pacc[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    ok[j] = lane + 64 * j < E;
    pacc[j] = 0.f;
  }
  float zacc = 0.f;
  int nvalid = 0;

  for (int tl = wave; tl < nt; tl += SEL_WAVES) {
    const int t = t0 + tl;
    if (p.token_mask && !p.token_mask[t]) {  // padding token: not routed
      if (lane < k) {
        p.ids[(size_t)t * k + lane] = -1;
        p.gate_w[(size_t)t * k + lane] = 0.f;
      }
      continue;
    }
    ++nvalid;
    float h[NS], sc[NS], sel[NS];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      h[j] = ok[j] ? sm.lg[tl * E + lane + 64 * j] + lb[j] : -INFINITY;
      mloc = fmaxf(mloc, h[j]);
      if (p.logits_out && ok[j]) p.logits_out[(size_t)t * E + lane + 64 * j] = h[j];
    }
    const float m = wave_max_dpp(mloc);
    float ex[NS], sloc = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      ex[j] = ok[j] ? expf(h[j] - m) : 0.f;
      sloc += ex[j];
    }
    const float S = wave_sum_dpp(sloc);
    const float lse = m + logf(S);
    zacc += lse * lse;
    if (!per_expert) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        sc[j] = ex[j] / S;
        pacc[j] += sc[j];
      }
    } else {
      float ssl = 0.f;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        if (!ok[j])
          sc[j] = 0.f;
        else
          sc[j] = p.score_func == 1 ? 1.0f / (1.0f + expf(-h[j])) : sqrt_softplus(h[j]);
        ssl += sc[j];
      }
      const float ss = wave_sum_dpp(ssl);
#pragma unroll
      for (int j = 0; j < NS; ++j) pacc[j] += sc[j] / ss;
    }
    // NaN scores rank as -inf so that every round still picks a valid expert.
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const float v = by_score ? sc[j] + sb[j] : h[j];
      sel[j] = (!ok[j] || v != v) ? -INFINITY : v;
    }

    bool allowed[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) allowed[j] = ok[j];
    if (p.n_groups > 1) {
      // Group scores are taken over the selection scores themselves: for
      // softmax the probabilities, not the logits the expert rounds may rank
      // by (a sum of two probabilities is not ordered like the sum of their
      // logits).
      float gin[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const float v = by_score ? sel[j] : sc[j];
        gin[j] = (!ok[j] || v != v) ? -INFINITY : v;
      }
      // Group score of every group, then group g's key in lane g.
      uint32_t gkey = 0;
      if (seg_groups) {
        float a1[NS], a2[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          a1[j] = gin[j];
          a2[j] = -INFINITY;
          if (gsz >= 2) top2_step<DPP_XOR1>(a1[j], a2[j]);
          if (gsz >= 4) top2_step<DPP_XOR2>(a1[j], a2[j]);
          if (gsz >= 8) top2_step<DPP_HALF_MIRROR>(a1[j], a2[j]);
          if (gsz >= 16) top2_step<DPP_ROW_MIRROR>(a1[j], a2[j]);
          if (gsz >= 32)
            top2_merge(a1[j], a2[j], __shfl_xor(a1[j], 16, MOE_WAVE),
                       __shfl_xor(a2[j], 16, MOE_WAVE));
        }
        // Group g lives in slot g / (64/gsz), lanes of segment g % (64/gsz).
        const int per_slot = MOE_WAVE / gsz;
        const int g = lane;
        const int gj = min(g / per_slot, NS - 1), src = (g % per_slot) * gsz;
        float gs = -INFINITY;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const float s1 = __shfl(a1[j], src, MOE_WAVE), s2 = __shfl(a2[j], src, MOE_WAVE);
          if (gj == j) gs = p.group_rule == 0 ? s1 + s2 : s1;
        }
        if (g < p.n_groups) gkey = okey(gs != gs ? -INFINITY : gs);
      } else {
        for (int g = 0; g < p.n_groups; ++g) {
          float a1 = -INFINITY, a2 = -INFINITY;
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            if (ok[j] && (lane + 64 * j) / gsz == g) top2_merge(a1, a2, gin[j], -INFINITY);
          }
#pragma unroll
          for (int msk = 32; msk >= 1; msk >>= 1)
            top2_merge(a1, a2, __shfl_xor(a1, msk, MOE_WAVE), __shfl_xor(a2, msk, MOE_WAVE));
          const float gs = p.group_rule == 0 ? a1 + a2 : a1;
          if (lane == g) gkey = okey(gs != gs ? -INFINITY : gs);
        }
      }
      uint64_t gmask = 0;
      uint32_t gk[1] = {gkey};
      for (int r = 0; r < p.topk_groups; ++r) {
        int wl, wj;
        wave_argmax_key(gk, wl, wj);
        gmask |= 1ull << wl;
        if (lane == wl) gk[0] = 0u;
      }
#pragma unroll
      for (int j = 0; j < NS; ++j)
        allowed[j] = ok[j] && ((gmask >> ((lane + 64 * j) / gsz)) & 1ull);
    }

    uint32_t key[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) key[j] = allowed[j] ? okey(sel[j]) : 0u;
    int my_id = 0;
    float my_sc = 0.f;
    for (int r = 0; r < k; ++r) {
      int wl, wj;
      wave_argmax_key(key, wl, wj);
      const float wsc = readlane_slot(sc, wj, wl);
      if (lane == r) {
        my_id = wl + 64 * wj;
        my_sc = wsc;
      }
      if (lane == wl) {
#pragma unroll
        for (int j = 0; j < NS; ++j)
          if (j == wj) key[j] = 0u;
      }
    }
    my_id = min(max(my_id, 0), E - 1);  // always a valid expert (see NaN note)
    const float ssel = wave_sum_dpp(lane < k ? my_sc : 0.f);
    if (lane < k) {
      const float wgt = p.renormalize ? p.route_scale * (my_sc / ssel) : p.route_scale * my_sc;
      p.ids[(size_t)t * k + lane] = my_id;
      p.gate_w[(size_t)t * k + lane] = wgt;
      atomicAdd(&sm.hist[my_id], 1);
    }
  }

  // Per-block partials, reduced across waves in a fixed order.
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int e = lane + 64 * j;
    if (e < E) sm.pe[wave][e] = pacc[j];
  }
  if (lane == 0) {
    sm.zw[wave] = zacc;
    sm.nv[wave] = nvalid;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += SEL_THREADS) {
    float s = sm.pe[0][e];
#pragma unroll
    for (int w = 1; w < SEL_WAVES; ++w) s += sm.pe[w][e];
    const int nblk = gridDim.x;  // expert-major: column e holds the tiles in order
    p.pe_part[(size_t)e * nblk + blk] = s;
    p.hist[(size_t)e * nblk + blk] = sm.hist[e];
  }
  if (threadIdx.x == 0) {
    float s = sm.zw[0];
    int nv = sm.nv[0];
#pragma unroll
    for (int w = 1; w < SEL_WAVES; ++w) {
      s += sm.zw[w];
      nv += sm.nv[w];
    }
    p.z_part[blk] = s;
    p.valid_part[blk] = nv;
  }
}

// select_tokens with as many 64-expert slots per lane as E needs.
template <int TILE>
__device__ __forceinline__ void select_slots(const RouteParams p, SelectSmem<TILE>& sm, int blk,
                                             int t0, int nt, const float (&lb)[4],
                                             const float (&sb)[4]) {
  if (p.E <= 64)
    select_tokens<TILE, 1>(p, sm, blk, t0, nt, lb, sb);
  else if (p.E <= 128)
    select_tokens<TILE, 2>(p, sm, blk, t0, nt, lb, sb);
  else
    select_tokens<TILE, 4>(p, sm, blk, t0, nt, lb, sb);
}

// Adds the KS split-K partials of n 16-byte groups of logits (group i of
// split s at b4[s * s4 + i]) in split order into lg4[i]; each thread takes
// EPT groups per pass with all their KS * EPT loads in flight (a thread past
// the end reloads the last group and stores nothing).
template <int KS, int EPT>
__device__ __forceinline__ void sum_partials(const f32x4* __restrict__ b4, size_t s4, int n,
                                             f32x4* lg4) {
  for (int i0 = threadIdx.x; i0 < n; i0 += EPT * SEL_THREADS) {
    f32x4 a[EPT][KS];
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int i = min(i0 + u * SEL_THREADS, n - 1);
#pragma unroll
      for (int sp = 0; sp < KS; ++sp) a[u][sp] = b4[sp * s4 + i];
    }
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      f32x4 v = a[u][0];
#pragma unroll
      for (int sp = 1; sp < KS; ++sp) v += a[u][sp];
      if (i0 + u * SEL_THREADS < n) lg4[i0 + u * SEL_THREADS] = v;
    }
  }
}

// The block's [tile x E] logits: the K-split partials (a power of two, at
// most 16) added in split order into LDS, all of a group's loads in flight;
// then the selection above.
template <int TILE>
__global__ __launch_bounds__(SEL_THREADS) void route_select_kernel(RouteParams p) {
  __shared__ SelectSmem<TILE> sm;
  const int blk = blockIdx.x, t0 = blk * TILE;
  const int E = p.E;
  const int nt = min(TILE, p.T - t0);
  float lb[4], sb[4];
  load_biases(p, lb, sb);
  for (int e = threadIdx.x; e < E; e += SEL_THREADS) sm.hist[e] = 0;
  {
    const int ks = p.ksplit;
    const int L = nt * E;
    const size_t stride = (size_t)p.T * E;
    const float* base = p.logits_part + (size_t)t0 * E;
    if ((E & 3) == 0) {
      const f32x4* b4 = reinterpret_cast<const f32x4*>(base);
      f32x4* lg4 = reinterpret_cast<f32x4*>(sm.lg);
      const size_t s4 = stride >> 2;
      const int L4 = L >> 2;
      switch (ks) {
        case 1: sum_partials<1, 4>(b4, s4, L4, lg4); break;
        case 2: sum_partials<2, 4>(b4, s4, L4, lg4); break;
        case 4: sum_partials<4, 4>(b4, s4, L4, lg4); break;
        case 8: sum_partials<8, 2>(b4, s4, L4, lg4); break;
        default: sum_partials<16, 1>(b4, s4, L4, lg4); break;
      }
    } else {
      for (int i = threadIdx.x; i < L; i += SEL_THREADS) {
        float s = 0.f;
        for (int k0 = 0; k0 < ks; k0 += 8) {
          float a[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (k0 + u < ks) a[u] = base[(k0 + u) * stride + i];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (k0 + u < ks) s = (k0 + u == 0) ? a[u] : s + a[u];
        }
        sm.lg[i] = s;
      }
    }
  }
  __syncthreads();
  select_slots<TILE>(p, sm, blk, t0, nt, lb, sb);
}

// ---------------------------------------------------------------------------
// Fused routing for routers small enough to stream through one block (at most
// kFusedMaxE experts, route_fused below): a block owns its tile of tokens,
// computes their logits against every expert over the whole of K, and selects
// from them, in one launch and with no split-K partials in HBM.  The waves
// split the k-steps evenly; each holds the block's whole [tile x E] output as
// 16x16 MFMA tiles (token tile ts, expert tile et).  The waves' partial tiles
// go through LDS and are added in wave (= K) order.
// MODE 0: bf16 x and W, 16x16x32 bf16; 1: bf16 x and fp32 W on the exact
// three-term bf16 split of W (three MFMAs per tile and k-step, products
// exact, fp32 sums); 2: an fp32 operand, 16x16x4 fp32.
// ETM: expert tiles held per wave (E <= 16 * ETM).  U = 2 k-steps of
// operands are loaded at once: with every wave of every block loading at
// the same time, more in flight measured slower (Mixtral-shaped router: 18.5
// us at two k-steps, 19.5 at four, 21.4 at eight; one: 21.9).

template <typename XT, typename WT, int MODE, int TILE, int ETM>
__global__ __launch_bounds__(SEL_THREADS) void route_fused_kernel(RouteParams p) {
  constexpr int TS = (TILE + 15) / 16;
  constexpr int KSTEP = MODE == 2 ? 16 : 32;
  constexpr int KLANE = MODE == 2 ? 4 : 8;  // k elements per lane per k-step
  // Per-wave LDS region (in 1 KB units): the bf16 operand tiles of one
  // k-step on their way into the MFMA layout (MODE 0 and 1; an fp32 W tile
  // takes 2 KB), later the wave's partial output tiles.
  constexpr int STG = MODE == 2 ? 0 : TS + (MODE == 1 ? 2 : 1) * ETM;
  constexpr int WT_ = STG > TS * ETM ? STG : TS * ETM;
  __shared__ SelectSmem<TILE> sm;
  __shared__ f32x4 red[SEL_WAVES][WT_][MOE_WAVE];
  const int blk = blockIdx.x, t0 = blk * TILE;
  const int E = p.E, ET = (E + 15) / 16;
  const int nt = min(TILE, p.T - t0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
  float lb[4], sb[4];
  load_biases(p, lb, sb);
  for (int e = threadIdx.x; e < E; e += SEL_THREADS) sm.hist[e] = 0;

  const XT* x = static_cast<const XT*>(p.x);
  const WT* w = static_cast<const WT*>(p.w_router);
  const int nsteps = p.D / KSTEP;
  const int per = (nsteps + SEL_WAVES - 1) / SEL_WAVES;
  const int s0 = min(nsteps, wave * per), s1 = min(nsteps, s0 + per);
  const int r = lane & 15, kq = lane >> 4;
  // MODE 2: this lane's row of token tile ts and of expert tile et
  // (clamped), at its k offset inside a k-step.
  auto xr = [&](int ts) { return x + (size_t)min(t0 + ts * 16 + r, p.T - 1) * p.D + kq * KLANE; };
  auto wr = [&](int et) { return w + (size_t)min(et * 16 + r, E - 1) * p.D + kq * KLANE; };
  // MODE 0 and 1 load coalesced: four consecutive lanes read one row's 64
  // contiguous bytes of a k-step (row lane/4, 16-byte chunk lane%4), and
  // the tile goes through the wave's LDS region into the MFMA layout (lane
  // l: row l%16, k chunk l/16).  The 16-byte slots are XOR-swizzled so
  // that the fragment reads are free of bank conflicts.
  const int lr = lane >> 2, lc = lane & 3;
  auto xc = [&](int ts) { return x + (size_t)min(t0 + ts * 16 + lr, p.T - 1) * p.D + lc * 8; };
  auto wc = [&](int et) {
    return w + (size_t)min(et * 16 + lr, E - 1) * p.D + lc * (MODE == 1 ? 4 : 8);
  };
  // bf16 tiles: chunk c of row q in slot 4q + (c ^ (q/4 % 4)); fp32 W
  // tiles (eight 4-float chunks a row): chunk m of row q in slot
  // 8q + (m ^ (q/2 % 8)).
  const int wslot = lr * 4 + (lc ^ ((lr >> 2) & 3));
  const int rslot = r * 4 + (kq ^ ((r >> 2) & 3));
  const int wslot_f0 = lr * 8 + (lc ^ ((lr >> 1) & 7));
  const int wslot_f1 = lr * 8 + ((4 + lc) ^ ((lr >> 1) & 7));
  const int rslot_f0 = r * 8 + ((2 * kq) ^ ((r >> 1) & 7));
  const int rslot_f1 = r * 8 + ((2 * kq + 1) ^ ((r >> 1) & 7));
  bf16x8* stb = reinterpret_cast<bf16x8*>(&red[wave][0][0]);
  f32x4* stf = reinterpret_cast<f32x4*>(&red[wave][0][0]) + TS * 64;
  f32x4 acc[TS][ETM];
#pragma unroll
  for (int ts = 0; ts < TS; ++ts)
#pragma unroll
    for (int et = 0; et < ETM; ++et) acc[ts][et] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (MODE == 0) {
    constexpr int U = 2;  // k-steps of operands in flight per wave (see above)
    // One k-step from registers (coalesced layout) through LDS into MFMAs.
    auto step = [&](const bf16x8 (&A)[TS], const bf16x8 (&B)[ETM]) {
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) stb[ts * 64 + wslot] = A[ts];
#pragma unroll
      for (int et = 0; et < ETM; ++et)
        if (et < ET) stb[(TS + et) * 64 + wslot] = B[et];
      bf16x8 a[TS];
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) a[ts] = stb[ts * 64 + rslot];
#pragma unroll
      for (int et = 0; et < ETM; ++et)
        if (et < ET) {
          const bf16x8 b = stb[(TS + et) * 64 + rslot];
#pragma unroll
          for (int ts = 0; ts < TS; ++ts)
            acc[ts][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ts], b, acc[ts][et], 0, 0, 0);
        }
    };
    int s = s0;
    for (; s + U <= s1; s += U) {
      bf16x8 A[U][TS], B[U][ETM];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int ts = 0; ts < TS; ++ts)
          A[u][ts] = *reinterpret_cast<const bf16x8*>(xc(ts) + (s + u) * KSTEP);
#pragma unroll
        for (int et = 0; et < ETM; ++et)
          if (et < ET) B[u][et] = *reinterpret_cast<const bf16x8*>(wc(et) + (s + u) * KSTEP);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) step(A[u], B[u]);
    }
    for (; s < s1; ++s) {
      bf16x8 A[TS], B[ETM];
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) A[ts] = *reinterpret_cast<const bf16x8*>(xc(ts) + s * KSTEP);
#pragma unroll
      for (int et = 0; et < ETM; ++et)
        if (et < ET) B[et] = *reinterpret_cast<const bf16x8*>(wc(et) + s * KSTEP);
      step(A, B);
    }
  } else if constexpr (MODE == 1) {
    constexpr int U = 2;
    auto step = [&](const bf16x8 (&A)[TS], const f32x4 (&W0)[ETM], const f32x4 (&W1)[ETM]) {
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) stb[ts * 64 + wslot] = A[ts];
#pragma unroll
      for (int et = 0; et < ETM; ++et)
        if (et < ET) {
          stf[et * 128 + wslot_f0] = W0[et];
          stf[et * 128 + wslot_f1] = W1[et];
        }
      bf16x8 a[TS];
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) a[ts] = stb[ts * 64 + rslot];
#pragma unroll
      for (int et = 0; et < ETM; ++et)
        if (et < ET) {
          bf16x8 h, m, l;
          split3_bf16(stf[et * 128 + rslot_f0], stf[et * 128 + rslot_f1], h, m, l);
#pragma unroll
          for (int ts = 0; ts < TS; ++ts) {
            acc[ts][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ts], h, acc[ts][et], 0, 0, 0);
            acc[ts][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ts], m, acc[ts][et], 0, 0, 0);
            acc[ts][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ts], l, acc[ts][et], 0, 0, 0);
          }
        }
    };
    int s = s0;
    for (; s + U <= s1; s += U) {
      bf16x8 A[U][TS];
      f32x4 W0[U][ETM], W1[U][ETM];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int ts = 0; ts < TS; ++ts)
          A[u][ts] = *reinterpret_cast<const bf16x8*>(xc(ts) + (s + u) * KSTEP);
#pragma unroll
        for (int et = 0; et < ETM; ++et)
          if (et < ET) {
            W0[u][et] = *reinterpret_cast<const f32x4*>(wc(et) + (s + u) * KSTEP);
            W1[u][et] = *reinterpret_cast<const f32x4*>(wc(et) + (s + u) * KSTEP + 16);
          }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) step(A[u], W0[u], W1[u]);
    }
    for (; s < s1; ++s) {
      bf16x8 A[TS];
      f32x4 W0[ETM], W1[ETM];
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) A[ts] = *reinterpret_cast<const bf16x8*>(xc(ts) + s * KSTEP);
#pragma unroll
      for (int et = 0; et < ETM; ++et)
        if (et < ET) {
          W0[et] = *reinterpret_cast<const f32x4*>(wc(et) + s * KSTEP);
          W1[et] = *reinterpret_cast<const f32x4*>(wc(et) + s * KSTEP + 16);
        }
      step(A, W0, W1);
    }
  } else {
    for (int s = s0; s < s1; ++s) {
      f32x4 a[TS];
#pragma unroll
      for (int ts = 0; ts < TS; ++ts) a[ts] = load4(xr(ts) + s * KSTEP);
#pragma unroll
      for (int et = 0; et < ETM; ++et)
        if (et < ET) {
          const f32x4 b = load4(wr(et) + s * KSTEP);
#pragma unroll
          for (int ts = 0; ts < TS; ++ts)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[ts][et] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[ts][j], b[j], acc[ts][et], 0, 0, 0);
        }
    }
  }
#pragma unroll
  for (int ts = 0; ts < TS; ++ts)
#pragma unroll
    for (int et = 0; et < ETM; ++et)
      if (et < ET) red[wave][ts * ETM + et][lane] = acc[ts][et];
  __syncthreads();
  // Element i of lane l of tile (ts, et) is token ts*16 + 4*(l/16) + i,
  // expert et*16 + l%16.
  for (int idx = threadIdx.x; idx < nt * E; idx += SEL_THREADS) {
    const int tl = idx / E, e = idx - tl * E;
    const int tile = (tl >> 4) * ETM + (e >> 4);
    const int ln = ((tl & 15) >> 2) * 16 + (e & 15), i = tl & 3;
    const float* rv = reinterpret_cast<const float*>(&red[0][tile][ln]) + i;
    constexpr int WSTRIDE = WT_ * MOE_WAVE * 4;  // floats between two waves' regions
    float v = rv[0];
#pragma unroll
    for (int wv = 1; wv < SEL_WAVES; ++wv) v += rv[wv * WSTRIDE];
    sm.lg[idx] = v;
  }
  __syncthreads();
  select_tokens<TILE, 1>(p, sm, blk, t0, nt, lb, sb);  // E <= 64: one slot
}

template <int TILE, int ETM>
void launch_fused_etm(const RouteParams& p, hipStream_t s) {
  const dim3 grid(route_blocks(p.T)), block(SEL_THREADS);
  if (p.act_bf16 && p.router_bf16)
    hipLaunchKernelGGL((route_fused_kernel<uint16_t, uint16_t, 0, TILE, ETM>), grid, block, 0, s,
                       p);
  else if (p.act_bf16)
    hipLaunchKernelGGL((route_fused_kernel<uint16_t, float, 1, TILE, ETM>), grid, block, 0, s, p);
  else if (p.router_bf16)
    hipLaunchKernelGGL((route_fused_kernel<float, uint16_t, 2, TILE, ETM>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((route_fused_kernel<float, float, 2, TILE, ETM>), grid, block, 0, s, p);
}

template <int TILE>
void launch_fused(const RouteParams& p, hipStream_t s) {
  static_assert(kFusedMaxE == 64, "expert tiles per wave: 1, 2 or 4");
  if (p.E <= 16)
    launch_fused_etm<TILE, 1>(p, s);
  else if (p.E <= 32)
    launch_fused_etm<TILE, 2>(p, s);
  else
    launch_fused_etm<TILE, 4>(p, s);
}

}  // namespace

hipError_t launch_route(const RouteParams& p, hipStream_t s) {
  if (route_fused(p.D, p.E, p.router_bf16)) {
    if (p.tile == kSmallRouteTile)
      launch_fused<kSmallRouteTile>(p, s);
    else
      launch_fused<kRouteTile>(p, s);
    return hipGetLastError();
  }
  const int NT = (p.E + 15) / 16;
  const int NTB = NT >= 4 ? 4 : (NT >= 2 ? 2 : 1);
  const dim3 grid(logits_blocks(p.T), (NT + NTB - 1) / NTB, p.ksplit), block(NTHREADS);
  if (route_tiled(p.T, p.E, p.act_bf16 && p.router_bf16)) {
    const dim3 tgrid((p.T + kRouteTiledM - 1) / kRouteTiledM,
                     (p.E + kRouteTiledN - 1) / kRouteTiledN, p.ksplit);
    hipLaunchKernelGGL((route_logits_tiled_kernel<kRouteTiledM, kRouteTiledK>), tgrid,
                       dim3(kRouteTiledM * 4), 0, s, p);
  } else if (p.act_bf16 && p.router_bf16) {
    hipLaunchKernelGGL((route_logits_kernel<uint16_t, uint16_t, true>), grid, block, 0, s, p);
  } else if (p.act_bf16) {
    hipLaunchKernelGGL((route_logits_kernel<uint16_t, float, false, true>), grid, block, 0, s, p);
  } else if (p.router_bf16) {
    hipLaunchKernelGGL((route_logits_kernel<float, uint16_t, false>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((route_logits_kernel<float, float, false>), grid, block, 0, s, p);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (p.tile == kSmallRouteTile)
    hipLaunchKernelGGL(route_select_kernel<kSmallRouteTile>, dim3(route_blocks(p.T)),
                       dim3(SEL_THREADS), 0, s, p);
  else
    hipLaunchKernelGGL(route_select_kernel<kRouteTile>, dim3(route_blocks(p.T)),
                       dim3(SEL_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
