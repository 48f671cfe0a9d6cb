// Routing kernel: router GEMM, fp32 scores, optional group limit, top-k,
// gate weights, and per-block partial sums for the balance and z losses.
//
// Follows "Lab: build a tiny MoE in PyTorch" ("Full implementation": Linear
// router, float32 softmax, topk, renormalised weights, bincount, balance and
// z losses) and "2.9 Mixture-of-Experts (MoE) Architectures" ("The Router":
// selection-only per-expert bias), with the NeMo Gate switches score_func,
// n_groups / topk_groups and route_scale.
//
// One 256-thread block routes kRouteTile tokens.  Phase 1 computes the
// [tile x E] logits into LDS: bf16 x and bf16 W_r use 16x16x32 bf16 MFMA
// (exact products, fp32 accumulation); any fp32 operand uses fp32 FMA.
// Phase 2 gives each wave one token at a time: lane l holds experts
// l, l+64, l+128, l+192; max, sums and the k arg-max rounds are butterfly
// shuffles, so every reduction has a fixed order and results are
// bit-reproducible.  Ties go to the lower expert index.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int RT = kRouteTile;
constexpr int NTHREADS = 256;
constexpr int NWAVES = NTHREADS / MOE_WAVE;
constexpr int LSTR = kMaxExperts + 4;  // LDS row stride of the logit tile
constexpr int KC = 32;                 // k chunk of the fp32 path

struct RouteSmem {
  float logits[RT][LSTR];
  union {
    struct {
      float xs[RT][KC + 1];
      float ws[KC][kMaxExperts];
    } simt;
    float pe[NWAVES][kMaxExperts];
  } u;
  float zw[NWAVES];
  int hist[kMaxExperts];
};

// bf16 x bf16 logits with v_mfma_f32_16x16x32_bf16.  Lane l supplies row
// (l % 16) and k-slice 8*(l / 16) .. +7 of both operands; it receives output
// rows 4*(l / 16) .. +3 of column (l % 16).
__device__ void logits_mfma(const RouteParams& p, int t0, RouteSmem& sm) {
  const uint16_t* x = static_cast<const uint16_t*>(p.x);
  const uint16_t* w = static_cast<const uint16_t*>(p.w_router);
  const int wave = threadIdx.x / MOE_WAVE, lane = lane_id();
  const int NT = (p.E + 15) / 16;
  const int r = lane & 15, kq = (lane >> 4) * 8;
  const int ta = min(t0 + r, p.T - 1), tb = min(t0 + 16 + r, p.T - 1);
  const uint16_t* pa = x + (size_t)ta * p.D + kq;
  const uint16_t* pb = x + (size_t)tb * p.D + kq;
  const uint16_t* pw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = min((wave + NWAVES * j) * 16 + r, p.E - 1);
    pw[j] = w + (size_t)e * p.D + kq;
  }
  f32x4 acc[2][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc[0][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[1][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int k0 = 0; k0 < p.D; k0 += 32) {
    const bf16x8 A0 = *reinterpret_cast<const bf16x8*>(pa + k0);
    const bf16x8 A1 = *reinterpret_cast<const bf16x8*>(pb + k0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (wave + NWAVES * j < NT) {  // wave-uniform
        const bf16x8 B = *reinterpret_cast<const bf16x8*>(pw[j] + k0);
        acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B, acc[0][j], 0, 0, 0);
        acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B, acc[1][j], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int nt = wave + NWAVES * j;
    if (nt < NT) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.logits[mt * 16 + (lane >> 4) * 4 + i][nt * 16 + (lane & 15)] = acc[mt][j][i];
    }
  }
}

// fp32 logits (any fp32 operand): thread (tg, eg) accumulates tokens
// 8*tg .. 8*tg+7 against experts eg + 64*j, in k order.
template <typename XT, typename WT>
__device__ void logits_simt(const RouteParams& p, int t0, RouteSmem& sm) {
  const XT* x = static_cast<const XT*>(p.x);
  const WT* w = static_cast<const WT*>(p.w_router);
  const int tid = threadIdx.x, eg = tid & 63, tg = tid >> 6;
  float acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < p.D; k0 += KC) {
    for (int idx = tid; idx < RT * KC; idx += NTHREADS) {
      const int rr = idx / KC, c = idx % KC;
      const int t = t0 + rr, kk = k0 + c;
      sm.u.simt.xs[rr][c] = (t < p.T && kk < p.D) ? Elem<XT>::load(x, (size_t)t * p.D + kk) : 0.f;
    }
    for (int idx = tid; idx < p.E * KC; idx += NTHREADS) {
      const int e = idx / KC, c = idx % KC, kk = k0 + c;
      sm.u.simt.ws[c][e] = kk < p.D ? Elem<WT>::load(w, (size_t)e * p.D + kk) : 0.f;
    }
    __syncthreads();
    for (int c = 0; c < KC; ++c) {
      float wv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = eg + 64 * j;
        wv[j] = e < p.E ? sm.u.simt.ws[c][e] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xv = sm.u.simt.xs[tg * 8 + i][c];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xv, wv[j], acc[i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = eg + 64 * j;
      if (e < p.E) sm.logits[tg * 8 + i][e] = acc[i][j];
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

template <typename XT, typename WT, bool MFMA>
__global__ __launch_bounds__(NTHREADS) void route_kernel(RouteParams p) {
  __shared__ RouteSmem sm;
  const int blk = blockIdx.x, t0 = blk * RT;
  const int wave = threadIdx.x / MOE_WAVE, lane = lane_id();
  for (int e = threadIdx.x; e < p.E; e += NTHREADS) sm.hist[e] = 0;

  if constexpr (MFMA) {
    logits_mfma(p, t0, sm);
  } else {
    logits_simt<XT, WT>(p, t0, sm);
  }
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
      h[j] = ok[j] ? sm.logits[tl][lane + 64 * j] + lb[j] : -INFINITY;
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
  __syncthreads();  // the SIMT staging area is reused for the P_e partials
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    if (e < E) sm.u.pe[wave][e] = pacc[j];
  }
  if (lane == 0) sm.zw[wave] = zacc;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += NTHREADS) {
    float s = sm.u.pe[0][e];
#pragma unroll
    for (int w = 1; w < NWAVES; ++w) s += sm.u.pe[w][e];
    p.pe_part[(size_t)blk * E + e] = s;
    p.hist[(size_t)blk * E + e] = sm.hist[e];
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
  const dim3 grid(route_blocks(p.T)), block(NTHREADS);
  if (p.act_bf16 && p.router_bf16) {
    hipLaunchKernelGGL((route_kernel<uint16_t, uint16_t, true>), grid, block, 0, s, p);
  } else if (p.act_bf16) {
    hipLaunchKernelGGL((route_kernel<uint16_t, float, false>), grid, block, 0, s, p);
  } else if (p.router_bf16) {
    hipLaunchKernelGGL((route_kernel<float, uint16_t, false>), grid, block, 0, s, p);
  } else {
    hipLaunchKernelGGL((route_kernel<float, float, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace moe
