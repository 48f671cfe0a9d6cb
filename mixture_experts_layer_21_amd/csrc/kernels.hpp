// Internal launchers of the gfx950 kernels.  Host code in moe_api.hip checks
// every argument before calling these; the launchers only enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Tokens per routing block; also the granularity of the per-block expert
// histograms that the permutation scans (route_tile below: batches of up to
// kSmallRouteMaxT tokens use 8-token blocks, one token per wave of the
// selection kernel, so that more tokens are in flight per CU).
constexpr int kRouteTile = 32;
constexpr int kSmallRouteTile = 8;
#ifndef MOE_SMALL_ROUTE_MAX_T
#define MOE_SMALL_ROUTE_MAX_T 1024
#endif
constexpr int kSmallRouteMaxT = MOE_SMALL_ROUTE_MAX_T;
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
  int tile;           // tokens per selection block: route_tile(T)
  int32_t* ids;       // [T*k]
  float* gate_w;      // [T*k]
  float* logits_part; // [ksplit*T*E] split-K partial logits
  int ksplit;
  int32_t* hist;      // [E*nblk]  per-tile expert histogram (expert-major)
  float* pe_part;     // [E*nblk]  per-tile sums of P_e terms
  float* z_part;      // [nblk]    per-block sums of lse^2
  int32_t* valid_part;  // [nblk]  unmasked tokens per block
  float* logits_out;    // [T*E] or null: the logits (bias included) of unmasked tokens
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
  int tile;                  // tokens per block: route_tile(T)
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
  // bf16 gate/up only, or null: the two SwiGLU factors d act/d g and
  // d act/d u (clamp included) of every Hb element, [max_rows, hidden] like
  // hbuf, kept for the backward
  uint16_t* save_p1;
  uint16_t* save_p2;
  // Split-K tail of the large-tile kernel (null: no split).  Per XCD: the
  // fp32 partial tiles [kTailSlots], the (tail tiles, pieces) pair and the
  // tile descriptors (expert, first row, row end, column tile).
  float* tail_part;
  int32_t* tail_meta;        // [kXcds * 2]
  int32_t* tail_desc;        // [kXcds * kTailSlots * 4]
  // Floats per partial-tile slot of tail_part.  A kernel whose fp32 partial
  // tile is larger than a slot runs its last round unsplit.
  size_t tail_slot_floats;
  // Nonzero: weight slices that one block reads alone stream through with
  // non-temporal loads (set by the launcher when the experts' weights are
  // larger than the last-level cache, so nothing is kept across calls).
  int stream_weights;
};

// Split-K tail bookkeeping of the large-tile grouped GEMM.
constexpr int kXcds = 8;
constexpr int kTailSlots = 64;                       // partial tiles per XCD
#ifndef MOE_TAIL_SLOT_ROWS
#define MOE_TAIL_SLOT_ROWS 256
#endif
// one fp32 tile of the largest grouped-GEMM tile (MOE_TAIL_SLOT_ROWS x 256)
constexpr size_t kTailSlotBytes = (size_t)MOE_TAIL_SLOT_ROWS * 256 * 4;
// Slots of kTailSlotBytes hold the partial tiles of every kernel; slots of
// 32 KB those of the 32-row (decode-sized) kernels only.
constexpr size_t kSmallTailSlotBytes = (size_t)32 * 256 * 4;
inline size_t tail_workspace_bytes(size_t slot_bytes = kTailSlotBytes) {
  return (size_t)kXcds * kTailSlots * slot_bytes + 256 + (size_t)kXcds * kTailSlots * 16;
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

// ------------------------------------------------------------ backward --

// Grouped bf16 GEMM of the backward pass, both operands K-contiguous:
//   C[g](m, n) = sum_k A[g](m, k) * B[g](n, k), fp32 accumulation.
enum BwdGrouping { BWD_DENSE = 0, BWD_MROWS = 1, BWD_KRAGGED = 2 };
enum BwdEpilogue { BWD_EPI_F32 = 0, BWD_EPI_GATEUP_SAVE = 1 };

struct BwdGemmParams {
  int grouping, epilogue;
  int M, N, K;               // DENSE: all three; MROWS: N and K; KRAGGED: M and N
  int G;                     // groups (experts)
  const int32_t* offsets;    // MROWS: [G+1] row offsets; KRAGGED: [G+1] k offsets (multiples of 64)
  int max_rows;              // MROWS: host bound on offsets[G] (grid size)
  // A: MROWS/DENSE row r at A + src(r)*lda, src(r) = gather ? gather[r] / gdiv : r;
  //    KRAGGED row m at A + m*lda + offsets[g]
  const uint16_t* A;
  long long lda;
  const int32_t* gather;
  int gdiv;
  // B: MROWS/DENSE row n at B + g*b_gstride + n*ldb; KRAGGED row n at B + n*ldb + offsets[g].
  // GATEUP_SAVE: a column tile is 64 rows of B (gate) and the same 64 rows of B2 (up).
  const uint16_t* B;
  const uint16_t* B2;
  long long ldb, b_gstride;
  // b_kmajor (EPI_F32): B is stored k-major instead, row k of group g at
  // B + g*b_gstride + k*ldb holding the N columns (KRAGGED: row krows[g] + k
  // of B); rows k >= k_split are row k - k_split of B2 (k_split a multiple of
  // 64; INT_MAX: no B2).  a_kmajor (EPI_F32, DENSE or KRAGGED): A likewise,
  // row k at A + k*lda (KRAGGED: row krows[g] + k) holding the M columns.
  // A k-major operand reads zeros past its rows: past krows[g+1] (KRAGGED)
  // or past a_bytes / b_bytes.
  int b_kmajor, k_split, a_kmajor;
  const int32_t* krows;      // KRAGGED with a k-major operand: [G+1] row offsets
  // EPI_F32: C row m of group g (KRAGGED) / row r (MROWS, DENSE) at
  // C + g*c_gstride + m*ldc; rows m >= c_split go to C2 + g*c_gstride + (m-c_split)*ldc.
  // With Cb (bf16) instead of C the rows are rounded once into Cb (no split).
  float* C;
  float* C2;
  uint16_t* Cb;
  long long ldc, c_gstride;
  int c_split;
  // GATEUP_SAVE: act = silu(g)*u and the two factors p1 = d act/d g, p2 = d act/d u
  // (clamp included) at [r][h], row stride ldh; limit = swiglu_limit.
  uint16_t* act;
  uint16_t* p1;
  uint16_t* p2;
  long long ldh;
  float limit;
  // Byte extents of A and of one group's B (the whole B when KRAGGED): the
  // 256x256 direct-to-LDS path addresses them with 32-bit buffer offsets.
  long long a_bytes, b_bytes;
};

// SwiGLU backward of the rows r < rows (rows = offsets[G] when offsets is
// given, else n): from dact = dL/d act for unit gate weight (bf16 [r][H]) and
// the saved act, p1, p2 ([r][H]): dgu[r][h] = w*dact*p1, dgu[r][H+h] =
// w*dact*p2 (w = gate_w[r2a[r]], 1 without gate_w) and, with dw, dw[r] = sum
// over h of act*dact (dL/dw of the row's slot) in a fixed order.
struct SwigluBwdParams {
  int n, H;
  const int32_t* offsets;
  int G;
  const uint16_t* dact;
  const uint16_t* act;
  const uint16_t* p1;
  const uint16_t* p2;
  const float* gate_w;
  const int32_t* r2a;
  uint16_t* dgu;
  float* dw;
};

// dst[c][col(j)] = scale(j) * src[row(j)][c]: a tiled transpose.  Row
// strides, column offsets and the column counts are multiples of 8 elements.  col(j) = j,
// or, with offsets/padoff (ragged groups), group g's rows offsets[g].. go to
// columns padoff[g].. and the columns up to padoff[g+1] are zero.
struct TransposeParams {
  int rows, cols;            // source rows j (before padding) and columns c
  const void* src;
  int src_f32;               // source element type: fp32 (1) or bf16 (0)
  long long ld_src, src_bstride;
  const int32_t* gather;     // source row of j: gather[j] / gdiv (null: j)
  int gdiv;
  const float* scale;        // per-j factor scale[scale_idx[j]] (null: 1)
  const int32_t* scale_idx;
  const int32_t* offsets;    // [G+1] or null (col = j)
  const int32_t* padoff;     // [G+1] padded column offsets (multiples of 64)
  int G;
  int out_cols;              // columns of dst to fill (padded total bound)
  uint16_t* dst;
  long long ld_dst, dst_bstride;
  int dst_col0;              // first destination column
  int batch;
  const int32_t* skip_rows;  // [batch+1] offsets or null: batches with no rows are skipped
};

struct RouterBwdParams {
  int T, E, Epad, k, score_func, renormalize;
  float route_scale, alpha, beta;
  const float* logits;       // [T, E] (logit bias included)
  const int32_t* ids;        // [T, k]
  const int32_t* a2r;        // [T*k]
  const float* dw;           // [rows]: dL/dw of each kept row
  const int32_t* counts;     // [E] pre-drop
  uint16_t* dh;              // [T, Epad] bf16 out
  float* dgw;                // [T, k] or null
};

struct DxParams {
  int T, D, k;
  const float* dz;           // [rows, D] per kept row
  const int32_t* a2r;
  const float* dzs;          // [T, D] or null (shared expert)
  const float* dxr;          // [T, D] (router)
  void* dx;                  // [T, D] act dtype, or null with dx_f32
  float* dx_f32;             // [T, D] fp32 out instead of dx (the pre-norm backward's input)
  // gated shared expert (or null): adds g_t (1 - g_t) sdw[t] * wsg[d], the
  // gate logit's gradient times the gate vector (bf16 [D])
  const float* sg;
  const float* sdw;
  const uint16_t* wsg;
};

hipError_t launch_bwd_gemm(const BwdGemmParams& p, hipStream_t s);
hipError_t launch_swiglu_bwd(const SwigluBwdParams& p, hipStream_t s);
hipError_t launch_transpose(const TransposeParams& p, hipStream_t s);
hipError_t launch_pad_offsets(int G, const int32_t* offsets, int32_t* padoff, hipStream_t s);
hipError_t launch_router_bwd(const RouterBwdParams& p, hipStream_t s);
// Gated shared expert: g[t] = sigmoid(x[t] . wsg) (bf16 x [T, D], wsg [D]);
// and dwsg[d] = sum_t g_t (1 - g_t) sdw[t] x[t][d] in a fixed order through
// part (f32 [gate_dw_chunks(T), D]).
hipError_t launch_shared_gate(int T, int D, const uint16_t* x, const uint16_t* wsg, float* g,
                              hipStream_t s);
int gate_dw_chunks(int T);
hipError_t launch_gate_dw(int T, int D, const uint16_t* x, const float* g, const float* sdw,
                          float* part, float* dwsg, hipStream_t s);
hipError_t launch_dx(const DxParams& p, bool bf16, hipStream_t s);

hipError_t launch_route(const RouteParams& p, hipStream_t s);
hipError_t launch_hist(int T, int E, int k, const int32_t* ids, int32_t* hist, hipStream_t s);
// Finalize and scatter in one single-workgroup kernel, for small batches
// (permute_fits_one_block); sp.ids == nullptr: finalize only.
bool permute_fits_one_block(int T, int E, int k);
hipError_t launch_permute_small(const FinalizeParams& fp, const ScatterParams& sp, hipStream_t s);
hipError_t launch_finalize(const FinalizeParams& p, hipStream_t s);
// launch_finalize and the scatter of the assignments into expert-major rows,
// in two launches (the scatter blocks compute the expert offsets themselves).
hipError_t launch_finalize_scatter(const FinalizeParams& fp, const ScatterParams& sp,
                                   hipStream_t s);
hipError_t launch_grouped_swiglu(const GemmParams& p, bool bf16, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, bool bf16, hipStream_t s);
hipError_t launch_update_bias(int E, const int32_t* counts, float gamma, float* bias,
                              hipStream_t s);
hipError_t launch_rmsnorm(int T, int D, bool bf16, const void* x, const float* w, float eps,
                          void* y, hipStream_t s);
// Backward of launch_rmsnorm: dx from dy (fp32 [T, D]); with dw (f32 [D]) also
// the weight gradient through dw_part (f32 [rmsnorm_dw_chunks(T), D]).
int rmsnorm_dw_chunks(int T);
hipError_t launch_rmsnorm_bwd(int T, int D, bool bf16, const void* x, const float* w, float eps,
                              const float* dy, void* dx, float* inv_s, float* dw_part,
                              float* dw, hipStream_t s);

__host__ __device__ inline int route_tile(int T) {
  return T <= kSmallRouteMaxT ? kSmallRouteTile : kRouteTile;
}
inline int route_blocks(int T) { return (T + route_tile(T) - 1) / route_tile(T); }
// Token tiles of the per-wave router GEMM (32 tokens: two 16-row MFMA tiles).
inline int logits_blocks(int T) { return (T + kRouteTile - 1) / kRouteTile; }

// The LDS-tiled router GEMM (64 tokens x 256 experts per block) serves bf16
// routers with many experts and tokens; the others use the per-wave kernel.
inline bool route_tiled(int T, int E, bool bf16_mfma) { return bf16_mfma && E >= 128 && T >= 1024; }

// Routers of at most kFusedMaxE experts and MOE_ROUTE_FUSED_MAX_BYTES of
// weights run as one fused kernel (logits over all of K and selection in one
// block per token tile); larger ones as the split-K logits kernel and the
// selection kernel.  Each fused block reads the whole router, so the bound
// keeps that read short next to the block's x rows.
constexpr int kFusedMaxE = 64;
#ifndef MOE_ROUTE_FUSED_MAX_BYTES
#define MOE_ROUTE_FUSED_MAX_BYTES (512 << 10)
#endif
inline bool route_fused(int D, int E, bool router_bf16) {
  return E <= kFusedMaxE &&
         (long long)E * D * (router_bf16 ? 2 : 4) <= (long long)MOE_ROUTE_FUSED_MAX_BYTES;
}
// Tokens per block of the LDS-tiled router GEMM (64 or 128: 4 threads a
// token), experts per block.  On the DeepSeek-shaped router (8192 tokens,
// 256 experts, K = 7168) 128 tokens and 64-deep k-steps take 50 us, 64
// tokens and 32-deep k-steps 66 us.
#ifndef MOE_ROUTE_TILED_M
#define MOE_ROUTE_TILED_M 128
#endif
// k-step depth (32 or 64).
#ifndef MOE_ROUTE_TILED_K
#define MOE_ROUTE_TILED_K 64
#endif
constexpr int kRouteTiledM = MOE_ROUTE_TILED_M, kRouteTiledN = 256, kRouteTiledK = MOE_ROUTE_TILED_K;
static_assert(kRouteTiledM == 64 || kRouteTiledM == 128, "tiled router rows");
static_assert(kRouteTiledK == 32 || kRouteTiledK == 64, "tiled router k-step");

#ifndef MOE_ROUTE_KSPLIT_MAX
#define MOE_ROUTE_KSPLIT_MAX 16
#endif
// The selection kernel adds the splits with a compile-time count: 1 to 16.
static_assert(MOE_ROUTE_KSPLIT_MAX >= 1 && MOE_ROUTE_KSPLIT_MAX <= 16 &&
                  (MOE_ROUTE_KSPLIT_MAX & (MOE_ROUTE_KSPLIT_MAX - 1)) == 0,
              "MOE_ROUTE_KSPLIT_MAX must be a power of two of at most 16");
// K-split of the router GEMM: enough blocks to fill the GPU while every split
// keeps at least four k-steps (32 elements each for bf16, 16 for fp32); the
// tiled kernel keeps at least eight.
inline int route_ksplit(int T, int D, int E, bool bf16_mfma) {
  const int nsteps = D / (bf16_mfma ? 32 : 16);
  if (route_tiled(T, E, bf16_mfma)) {
    const long long blocks =
        (long long)((T + kRouteTiledM - 1) / kRouteTiledM) * ((E + kRouteTiledN - 1) / kRouteTiledN);
    int ks = 1;
    // about 512 x 64 tokens' worth of blocks in flight
    while (blocks * ks * kRouteTiledM < 512 * 64 && ks * 2 * 8 <= nsteps && ks < 16) ks *= 2;
    return ks;
  }
  const int NT = (E + 15) / 16;
  const int NTB = NT >= 4 ? 4 : (NT >= 2 ? 2 : 1);
  const long long blocks = (long long)logits_blocks(T) * ((NT + NTB - 1) / NTB);
  int ks = 1;
  while (blocks * ks < 1024 && ks * 2 * 4 <= nsteps && ks < MOE_ROUTE_KSPLIT_MAX) ks *= 2;
  return ks;
}

}  // namespace moe
