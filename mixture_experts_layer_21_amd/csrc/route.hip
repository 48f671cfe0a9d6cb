// Routing: router GEMM, fp32 scores, optional group limit, top-k, gate
// weights, and per-block partial sums for the balance and z losses.
//
// Follows "Lab: build a tiny MoE in PyTorch" ("Full implementation": Linear
// router, float32 softmax, topk, renormalised weights, bincount, balance and
// z losses) and "2.9 Mixture-of-Experts (MoE) Architectures" ("The Router":
// selection-only per-expert bias), with the NeMo Gate switches score_func,
// n_groups / topk_groups and route_scale.
//
// Two kernels:
//  * route_logits_kernel: the [T x E] logits as split-K partial sums.  A
//    256-thread block covers 32 tokens x up to 64 experts x one K range; each
//    wave runs 16x16 MFMA tiles (bf16 x bf16: 16x16x32 bf16, products exact;
//    any fp32 operand: 16x16x4 fp32).  Waves sharing an expert tile split the
//    k-steps and are summed through LDS in a fixed order.
//  * route_select_kernel: the block first adds the K-split partials of its
//    32 tokens in split order into LDS; then one wave per token does the
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
template <typename XT, typename WT, bool BF16>
__global__ __launch_bounds__(NTHREADS) void route_logits_kernel(RouteParams p) {
  constexpr int KSTEP = BF16 ? 32 : 16;
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

// LDS-tiled router GEMM for bf16 x and W: a block computes 64 tokens x 256
// experts over its K range (32-deep k-steps staged through LDS in two
// buffers); four waves in a 2 x 2 grid each hold 32 tokens x 128 experts as
// four 32x32x16 MFMA tiles.  x is read once per K range instead of once per
// expert tile.  Rows are 64 bytes in LDS; the 16-byte chunk c of row r sits
// at c ^ ((r >> 2) & 3), which keeps the fragment reads conflict-free.
__device__ __forceinline__ int rswz(int r) { return (r >> 2) & 3; }

__global__ __launch_bounds__(NTHREADS) void route_logits_tiled_kernel(RouteParams p) {
  constexpr int BM = kRouteTiledM, BN = kRouteTiledN, BK = 32;
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

  // This thread's 16-byte chunks: one of A (row tid/4), four of B.
  const int ar = tid >> 2, ac = tid & 3;
  const uint16_t* asrc = x + (size_t)min(t0 + ar, p.T - 1) * p.D + ac * 8;
  const int adst = ar * BK + (ac ^ rswz(ar)) * 8;
  const uint16_t* bsrc[4];
  int bdst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + NTHREADS * i, r = c >> 2, cc = c & 3;
    bsrc[i] = w + (size_t)min(e0 + r, p.E - 1) * p.D + cc * 8;
    bdst[i] = r * BK + (cc ^ rswz(r)) * 8;
  }
  f32x16 acc[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[ni][i] = 0.f;

  if (s0 < s1) {
    u32x4 ra, rb[4];
#define MOE_RLOAD(s)                                                                        \
  do {                                                                                      \
    const int k0_ = (s) * BK;                                                               \
    ra = *reinterpret_cast<const u32x4*>(asrc + k0_);                                       \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) rb[i] =                                   \
        *reinterpret_cast<const u32x4*>(bsrc[i] + k0_);                                     \
  } while (0)
#define MOE_RSTORE(buf)                                                                     \
  do {                                                                                      \
    *reinterpret_cast<u32x4*>(&As[buf][adst]) = ra;                                         \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                           \
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
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(&As[cur][r * BK + (ch ^ rswz(r)) * 8]);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int rb_ = wn * 128 + ni * 32 + lr;
          const bf16x8 bfr =
              *reinterpret_cast<const bf16x8*>(&Bs[cur][rb_ * BK + (ch ^ rswz(rb_)) * 8]);
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
__device__ __forceinline__ void wave_argmax_key(const uint32_t (&key)[4], int& wl, int& wj) {
  uint32_t lk = key[0];
  int lj = 0;
#pragma unroll
  for (int j = 1; j < 4; ++j)
    if (key[j] > lk) {
      lk = key[j];
      lj = j;
    }
  const uint32_t M = wave_max_key(lk);
  wl = 0;
  wj = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t m = __ballot(lk == M && lj == j);
    if (m) {
      wl = __ffsll((unsigned long long)m) - 1;
      wj = j;
      break;
    }
  }
}

template <typename V>
__device__ __forceinline__ V pick4(const V (&a)[4], int j) {
  return j == 0 ? a[0] : j == 1 ? a[1] : j == 2 ? a[2] : a[3];
}

struct SelectSmem {
  float lg[RT * kMaxExperts];      // summed logits of the block's tokens, row stride E
  float pe[SEL_WAVES][kMaxExperts];
  float zw[SEL_WAVES];
  int nv[SEL_WAVES];
  int hist[kMaxExperts];
};

// sqrt(softplus(h)), softplus(h) = log(1 + e^h) written without overflow.
__device__ __forceinline__ float sqrt_softplus(float h) {
  return sqrtf(fmaxf(h, 0.f) + log1pf(expf(-fabsf(h))));
}

// Phase 1: the block's [RT x E] logits, the K-split partials added in split
// order, into LDS (all threads, 16-byte loads, up to 16 loads in flight).
// Phase 2: one wave per token: scores, group limit, k arg-max rounds,
// weights; per-block P_e and z partials and the expert histogram.
__global__ __launch_bounds__(SEL_THREADS) void route_select_kernel(RouteParams p) {
  __shared__ SelectSmem sm;
  const int blk = blockIdx.x, t0 = blk * RT;
  const int wave = threadIdx.x / MOE_WAVE, lane = lane_id();
  const int E = p.E, k = p.k;
  const int nt = min(RT, p.T - t0);
  for (int e = threadIdx.x; e < E; e += SEL_THREADS) sm.hist[e] = 0;
  {
    const int ks = p.ksplit;
    const int L = nt * E;
    const size_t stride = (size_t)p.T * E;
    const float* base = p.logits_part + (size_t)t0 * E;
    if ((E & 3) == 0) {
      const int L4 = L >> 2;
      const f32x4* b4 = reinterpret_cast<const f32x4*>(base);
      const size_t s4 = stride >> 2;
      for (int i0 = threadIdx.x; i0 < L4; i0 += 2 * SEL_THREADS) {
        const int i1 = i0 + SEL_THREADS;
        const bool has1 = i1 < L4;
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
        for (int k0 = 0; k0 < ks; k0 += 8) {
          f32x4 a[8], b[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            if (k0 + u < ks) {
              a[u] = b4[(k0 + u) * s4 + i0];
              if (has1) b[u] = b4[(k0 + u) * s4 + i1];
            }
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            if (k0 + u < ks) {
              s0 = (k0 + u == 0) ? a[u] : s0 + a[u];
              if (has1) s1 = (k0 + u == 0) ? b[u] : s1 + b[u];
            }
          }
        }
        *reinterpret_cast<f32x4*>(&sm.lg[4 * i0]) = s0;
        if (has1) *reinterpret_cast<f32x4*>(&sm.lg[4 * i1]) = s1;
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

  // softmax scores are a distribution over the experts; sigmoid and
  // sqrt-softplus scores are per expert and normalised where a sum is needed.
  const bool per_expert = p.score_func != 0;
  const bool by_score = per_expert || p.select_bias != nullptr;
  const int gsz = p.n_groups > 1 ? E / p.n_groups : E;
  // Group limit with a segmented reduction: groups are aligned runs of gsz
  // lanes in one slot when gsz is a power of two below 64.
  const bool seg_groups = p.n_groups > 1 && gsz < 64 && (gsz & (gsz - 1)) == 0;
  float lb[4], sb[4];
  bool ok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    ok[j] = e < E;
    lb[j] = (ok[j] && p.logit_bias) ? p.logit_bias[e] : 0.f;
    sb[j] = (ok[j] && p.select_bias) ? p.select_bias[e] : 0.f;
  }
  float pacc[4] = {0.f, 0.f, 0.f, 0.f};
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
    float h[4], sc[4], sel[4];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = ok[j] ? sm.lg[tl * E + lane + 64 * j] + lb[j] : -INFINITY;
      mloc = fmaxf(mloc, h[j]);
      if (p.logits_out && ok[j]) p.logits_out[(size_t)t * E + lane + 64 * j] = h[j];
    }
    const float m = wave_max_dpp(mloc);
    float ex[4], sloc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ex[j] = ok[j] ? expf(h[j] - m) : 0.f;
      sloc += ex[j];
    }
    const float S = wave_sum_dpp(sloc);
    const float lse = m + logf(S);
    zacc += lse * lse;
    if (!per_expert) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[j] = ex[j] / S;
        pacc[j] += sc[j];
      }
    } else {
      float ssl = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!ok[j])
          sc[j] = 0.f;
        else
          sc[j] = p.score_func == 1 ? 1.0f / (1.0f + expf(-h[j])) : sqrt_softplus(h[j]);
        ssl += sc[j];
      }
      const float ss = wave_sum_dpp(ssl);
#pragma unroll
      for (int j = 0; j < 4; ++j) pacc[j] += sc[j] / ss;
    }
    // NaN scores rank as -inf so that every round still picks a valid expert.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = by_score ? sc[j] + sb[j] : h[j];
      sel[j] = (!ok[j] || v != v) ? -INFINITY : v;
    }

    bool allowed[4] = {ok[0], ok[1], ok[2], ok[3]};
    if (p.n_groups > 1) {
      // Group score of every group, then group g's key in lane g.
      uint32_t gkey = 0;
      if (seg_groups) {
        float a1[4], a2[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a1[j] = sel[j];
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
        const int gj = min(g / per_slot, 3), src = (g % per_slot) * gsz;
        float gs = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float s1 = __shfl(a1[j], src, MOE_WAVE), s2 = __shfl(a2[j], src, MOE_WAVE);
          if (gj == j) gs = p.group_rule == 0 ? s1 + s2 : s1;
        }
        if (g < p.n_groups) gkey = okey(gs != gs ? -INFINITY : gs);
      } else {
        for (int g = 0; g < p.n_groups; ++g) {
          float a1 = -INFINITY, a2 = -INFINITY;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (ok[j] && (lane + 64 * j) / gsz == g) top2_merge(a1, a2, sel[j], -INFINITY);
          }
#pragma unroll
          for (int msk = 32; msk >= 1; msk >>= 1)
            top2_merge(a1, a2, __shfl_xor(a1, msk, MOE_WAVE), __shfl_xor(a2, msk, MOE_WAVE));
          const float gs = p.group_rule == 0 ? a1 + a2 : a1;
          if (lane == g) gkey = okey(gs != gs ? -INFINITY : gs);
        }
      }
      uint64_t gmask = 0;
      uint32_t gk[4] = {gkey, 0u, 0u, 0u};
      for (int r = 0; r < p.topk_groups; ++r) {
        int wl, wj;
        wave_argmax_key(gk, wl, wj);
        gmask |= 1ull << wl;
        if (lane == wl) gk[0] = 0u;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        allowed[j] = ok[j] && ((gmask >> ((lane + 64 * j) / gsz)) & 1ull);
    }

    uint32_t key[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = allowed[j] ? okey(sel[j]) : 0u;
    int my_id = 0;
    float my_sc = 0.f;
    for (int r = 0; r < k; ++r) {
      int wl, wj;
      wave_argmax_key(key, wl, wj);
      const float wsc = readlane_f(pick4(sc, wj), wl);
      if (lane == r) {
        my_id = wl + 64 * wj;
        my_sc = wsc;
      }
      if (lane == wl) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
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
  for (int j = 0; j < 4; ++j) {
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

}  // namespace

hipError_t launch_route(const RouteParams& p, hipStream_t s) {
  const int NT = (p.E + 15) / 16;
  const int NTB = NT >= 4 ? 4 : (NT >= 2 ? 2 : 1);
  const dim3 grid(route_blocks(p.T), (NT + NTB - 1) / NTB, p.ksplit), block(NTHREADS);
  if (route_tiled(p.T, p.E, p.act_bf16 && p.router_bf16)) {
    const dim3 tgrid((p.T + kRouteTiledM - 1) / kRouteTiledM,
                     (p.E + kRouteTiledN - 1) / kRouteTiledN, p.ksplit);
    hipLaunchKernelGGL(route_logits_tiled_kernel, tgrid, block, 0, s, p);
  } else if (p.act_bf16 && p.router_bf16) {
    hipLaunchKernelGGL((route_logits_kernel<uint16_t, uint16_t, true>), grid, block, 0, s, p);
  } else if (p.act_bf16) {
    hipLaunchKernelGGL((route_logits_kernel<uint16_t, float, false>), grid, block, 0, s, p);
  } else if (p.router_bf16) {
    hipLaunchKernelGGL((route_logits_kernel<float, uint16_t, false>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((route_logits_kernel<float, float, false>), grid, block, 0, s, p);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_select_kernel, dim3(route_blocks(p.T)), dim3(SEL_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
