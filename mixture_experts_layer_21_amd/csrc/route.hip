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
//  * route_select_kernel: one wave per token adds the K-split partials in a
//    fixed order and does the scores, group limit, k arg-max rounds (butterfly
//    shuffles; ties to the lower expert index) and weights.  Lane l holds
//    experts l, l+64, l+128, l+192.  Every reduction has a fixed order, so
//    results are bit-reproducible.
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

// Arg-max over the wave of (value, index): larger value wins, equal values go
// to the lower index.  `extra` travels with the winner.
__device__ __forceinline__ void wave_argmax(float& v, int& idx, float& extra) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(v, m, MOE_WAVE);
    const int oi = __shfl_xor(idx, m, MOE_WAVE);
    const float ox = __shfl_xor(extra, m, MOE_WAVE);
    if (ov > v || (ov == v && oi < idx)) {
      v = ov;
      idx = oi;
      extra = ox;
    }
  }
}

struct SelectSmem {
  float pe[NWAVES][kMaxExperts];
  float zw[NWAVES];
  int hist[kMaxExperts];
};

__global__ __launch_bounds__(NTHREADS) void route_select_kernel(RouteParams p) {
  __shared__ SelectSmem sm;
  const int blk = blockIdx.x, t0 = blk * RT;
  const int wave = threadIdx.x / MOE_WAVE, lane = lane_id();
  for (int e = threadIdx.x; e < p.E; e += NTHREADS) sm.hist[e] = 0;
  __syncthreads();

  const int E = p.E, k = p.k;
  const bool sigm = p.score_func == 1;
  const bool by_score = sigm || p.select_bias != nullptr;
  const int gsz = p.n_groups > 1 ? E / p.n_groups : E;
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

  for (int tl = wave; tl < RT; tl += NWAVES) {
    const int t = t0 + tl;
    if (t >= p.T) break;  // wave-uniform
    float h[4], sc[4], sel[4];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = -INFINITY;
      if (ok[j]) {
        // K-split partials added in split order; loads issued 8 at a time.
        const float* q = p.logits_part + (size_t)t * E + lane + 64 * j;
        const size_t stride = (size_t)p.T * E;
        v = 0.f;
        for (int k0 = 0; k0 < p.ksplit; k0 += 8) {
          float part[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) part[u] = k0 + u < p.ksplit ? q[(k0 + u) * stride] : 0.f;
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (k0 + u < p.ksplit) v = (k0 + u == 0) ? part[u] : v + part[u];
        }
        v += lb[j];
      }
      h[j] = v;
      mloc = fmaxf(mloc, h[j]);
    }
    const float m = wave_max(mloc);
    float ex[4], sloc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ex[j] = ok[j] ? expf(h[j] - m) : 0.f;
      sloc += ex[j];
    }
    const float S = wave_sum(sloc);
    const float lse = m + logf(S);
    zacc += lse * lse;
    if (!sigm) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[j] = ex[j] / S;
        pacc[j] += sc[j];
      }
    } else {
      float ssl = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[j] = ok[j] ? 1.0f / (1.0f + expf(-h[j])) : 0.f;
        ssl += sc[j];
      }
      const float ss = wave_sum(ssl);
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
      float gmine = -INFINITY;
      for (int g = 0; g < p.n_groups; ++g) {
        float a1 = -INFINITY, a2 = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (ok[j] && (lane + 64 * j) / gsz == g) {
            const float v = sel[j];
            if (v > a1) {
              a2 = a1;
              a1 = v;
            } else if (v > a2) {
              a2 = v;
            }
          }
        }
#pragma unroll
        for (int msk = 32; msk >= 1; msk >>= 1) {
          const float b1 = __shfl_xor(a1, msk, MOE_WAVE);
          const float b2 = __shfl_xor(a2, msk, MOE_WAVE);
          if (a1 >= b1) {
            a2 = fmaxf(a2, b1);
          } else {
            a2 = fmaxf(a1, b2);
            a1 = b1;
          }
        }
        const float gs = p.group_rule == 0 ? a1 + a2 : a1;
        if (lane == g) gmine = gs != gs ? -INFINITY : gs;
      }
      uint64_t gmask = 0;
      bool gtaken = false;
      for (int r = 0; r < p.topk_groups; ++r) {
        float v = (lane < p.n_groups && !gtaken) ? gmine : -INFINITY;
        int gi = (lane < p.n_groups && !gtaken) ? lane : 0x7fffffff;
        float dummy = 0.f;
        wave_argmax(v, gi, dummy);
        gmask |= 1ull << gi;
        if (lane == gi) gtaken = true;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        allowed[j] = ok[j] && ((gmask >> ((lane + 64 * j) / gsz)) & 1ull);
    }

    uint32_t taken = 0;
    int my_id = 0;
    float my_sc = 0.f;
    for (int r = 0; r < k; ++r) {
      float bv = -INFINITY, bsc = 0.f;
      int be = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (allowed[j] && !((taken >> j) & 1u)) {
          const int e = lane + 64 * j;
          if (sel[j] > bv || (sel[j] == bv && e < be)) {
            bv = sel[j];
            be = e;
            bsc = sc[j];
          }
        }
      }
      wave_argmax(bv, be, bsc);
      if (lane == r) {
        my_id = be;
        my_sc = bsc;
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
    }
    my_id = min(max(my_id, 0), E - 1);  // always a valid expert (see NaN note)
    const float ssel = wave_sum(lane < k ? my_sc : 0.f);
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
  if (lane == 0) sm.zw[wave] = zacc;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += NTHREADS) {
    float s = sm.pe[0][e];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) s += sm.pe[w][e];
    const int nblk = gridDim.x;  // expert-major: column e holds the tiles in order
    p.pe_part[(size_t)e * nblk + blk] = s;
    p.hist[(size_t)e * nblk + blk] = sm.hist[e];
  }
  if (threadIdx.x == 0) {
    float s = sm.zw[0];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) s += sm.zw[w];
    p.z_part[blk] = s;
  }
}

}  // namespace

hipError_t launch_route(const RouteParams& p, hipStream_t s) {
  const int NT = (p.E + 15) / 16;
  const int NTB = NT >= 4 ? 4 : (NT >= 2 ? 2 : 1);
  const dim3 grid(route_blocks(p.T), (NT + NTB - 1) / NTB, p.ksplit), block(NTHREADS);
  if (p.act_bf16 && p.router_bf16) {
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
  hipLaunchKernelGGL(route_select_kernel, dim3(route_blocks(p.T)), block, 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
