// Internal launchers of the gfx950 kernels.  Host code in moe_api.hip checks
// every argument before calling these; the launchers only enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Tokens per routing block; also the granularity of the per-block expert
// histograms that the permutation scans.
constexpr int kRouteTile = 32;
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 32;
constexpr int kMaxGroups = 64;

struct RouteParams {
  int T, D, E, k;
  int score_func, renormalize, n_groups, topk_groups, group_rule;
  float route_scale;
  int act_bf16, router_bf16;
  const void* x;
  const void* w_router;
  const float* logit_bias;
  const float* select_bias;
  const uint8_t* token_mask;  // [T] or null: 0 = padding token (not routed)
  int32_t* ids;       // [T*k]
  float* gate_w;      // [T*k]
  float* logits_part; // [ksplit*T*E] split-K partial logits
  int ksplit;
  int32_t* hist;      // [E*nblk]  per-tile expert histogram (expert-major)
  float* pe_part;     // [E*nblk]  per-tile sums of P_e terms
  float* z_part;      // [nblk]    per-block sums of lse^2
  int32_t* valid_part;  // [nblk]  unmasked tokens per block
};

struct FinalizeParams {
  int T, E, k, nblk;
  int capacity;              // <= 0: dropless
  const int32_t* hist;       // [E*nblk] (expert-major)
  const float* pe_part;      // [E*nblk] or null (no aux)
  const float* z_part;       // [nblk] or null
  const int32_t* valid_part; // [nblk] unmasked tokens per block, or null (all T)
  int32_t* counts_ws;        // [E] scratch: counts before the capacity clip
  float* pe_ws;              // [E] scratch: P_e
  int32_t* counts;           // [E] or null
  float* aux;                // [2] or null
  float* mean_prob;          // [E] or null
  int32_t* block_base;       // [E*nblk] or null (no permutation scan)
  int32_t* expert_offsets;   // [E+1] or null
  int32_t* n_kept;           // [1] or null
};

struct ScatterParams {
  int T, E, k, capacity;
  const int32_t* ids;
  const int32_t* block_base;
  const int32_t* expert_offsets;
  int32_t* row_to_assign;
  int32_t* assign_to_row;
};

struct GemmParams {
  int T, D, k;               // tokens, d_model, top_k of the assignment index
  int n_groups;              // experts in this call
  int hidden;                // H of this call
  int max_rows;
  const void* x;             // [T, D]
  const int32_t* row_to_assign;   // null: identity rows
  const int32_t* expert_offsets;  // null: one group of T rows
  const float* gate_w;       // null: weight 1
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  void* hbuf;                // [max_rows, hidden]
  void* y;                   // [max_rows, D]
  float swiglu_limit;        // > 0: clamp gate and up to [-limit, limit]
  // Split-K tail of the large-tile kernel (null: no split).  Per XCD: the
  // fp32 partial tiles [kTailSlots], the (tail tiles, pieces) pair and the
  // tile descriptors (expert, first row, row end, column tile).
  float* tail_part;
  int32_t* tail_meta;        // [kXcds * 2]
  int32_t* tail_desc;        // [kXcds * kTailSlots * 4]
};

// Split-K tail bookkeeping of the large-tile grouped GEMM.
constexpr int kXcds = 8;
constexpr int kTailSlots = 64;                       // partial tiles per XCD
constexpr size_t kTailSlotBytes = (size_t)256 * 256 * 4;  // one fp32 256x256 tile
inline size_t tail_workspace_bytes() {
  return (size_t)kXcds * kTailSlots * kTailSlotBytes + 256 + (size_t)kXcds * kTailSlots * 16;
}

struct CombineParams {
  int T, D, k;
  const void* y_rows;
  const int32_t* assign_to_row;
  const void* shared_rows;
  const void* x;             // [T, D], read only with shared_gate
  const void* shared_gate;   // [D] or null: shared rows scaled by sigmoid(x . g)
  const void* residual;      // [T, D] or null: added to the output
  void* out;
};

hipError_t launch_route(const RouteParams& p, hipStream_t s);
hipError_t launch_hist(int T, int E, int k, const int32_t* ids, int32_t* hist, hipStream_t s);
hipError_t launch_finalize(const FinalizeParams& p, hipStream_t s);
hipError_t launch_scatter(const ScatterParams& p, hipStream_t s);
hipError_t launch_grouped_swiglu(const GemmParams& p, bool bf16, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, bool bf16, hipStream_t s);
hipError_t launch_update_bias(int E, const int32_t* counts, float gamma, float* bias,
                              hipStream_t s);
hipError_t launch_rmsnorm(int T, int D, bool bf16, const void* x, const float* w, float eps,
                          void* y, hipStream_t s);

inline int route_blocks(int T) { return (T + kRouteTile - 1) / kRouteTile; }

// The LDS-tiled router GEMM (64 tokens x 256 experts per block) serves bf16
// routers with many experts and tokens; the others use the per-wave kernel.
inline bool route_tiled(int T, int E, bool bf16_mfma) { return bf16_mfma && E >= 128 && T >= 1024; }
constexpr int kRouteTiledM = 64, kRouteTiledN = 256;

// K-split of the router GEMM: enough blocks to fill the GPU while every split
// keeps at least four k-steps (32 elements each for bf16, 16 for fp32); the
// tiled kernel keeps at least eight.
inline int route_ksplit(int T, int D, int E, bool bf16_mfma) {
  const int nsteps = D / (bf16_mfma ? 32 : 16);
  if (route_tiled(T, E, bf16_mfma)) {
    const long long blocks =
        (long long)((T + kRouteTiledM - 1) / kRouteTiledM) * ((E + kRouteTiledN - 1) / kRouteTiledN);
    int ks = 1;
    while (blocks * ks < 512 && ks * 2 * 8 <= nsteps && ks < 16) ks *= 2;
    return ks;
  }
  const int NT = (E + 15) / 16;
  const int NTB = NT >= 4 ? 4 : (NT >= 2 ? 2 : 1);
  const long long blocks = (long long)route_blocks(T) * ((NT + NTB - 1) / NTB);
  int ks = 1;
  while (blocks * ks < 1024 && ks * 2 * 4 <= nsteps && ks < 16) ks *= 2;
  return ks;
}

}  // namespace moe
