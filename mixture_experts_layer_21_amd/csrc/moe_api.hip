// C ABI of the MoE-layer forward: argument checks, workspace layout and the
// stream-ordered launch sequence.  Declarations and semantics: include/moe.h.
#include <math.h>
#include <stdarg.h>
#include <string.h>

#include <algorithm>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t esize(int dt) { return dt == MOE_BF16 ? 2 : 4; }

bool is_dtype(int d) { return d == MOE_F32 || d == MOE_BF16; }

moe_status check_config(const moe_config* c) {
  if (!c) return fail(MOE_ERR_NULL_PTR, "config is NULL");
  if (c->T < 1) return fail(MOE_ERR_INVALID_ARG, "T must be >= 1 (got %d)", c->T);
  if (c->D < 1 || c->H < 1) return fail(MOE_ERR_INVALID_ARG, "D and H must be >= 1");
  if (c->E < 1 || c->E > moe::kMaxExperts)
    return fail(MOE_ERR_INVALID_ARG, "E must be in [1, %d] (got %d)", moe::kMaxExperts, c->E);
  if (c->top_k < 1 || c->top_k > c->E)
    return fail(MOE_ERR_INVALID_ARG, "top_k must be in [1, n_experts] (got %d, E=%d)", c->top_k,
                c->E);
  if (c->top_k > moe::kMaxTopK)
    return fail(MOE_ERR_UNSUPPORTED, "top_k > %d is not supported", moe::kMaxTopK);
  if (c->H_shared < 0) return fail(MOE_ERR_INVALID_ARG, "H_shared must be >= 0");
  if (!is_dtype(c->act_dtype) || !is_dtype(c->router_dtype))
    return fail(MOE_ERR_INVALID_ARG, "unknown dtype");
  if (c->score_func != MOE_SCORE_SOFTMAX && c->score_func != MOE_SCORE_SIGMOID &&
      c->score_func != MOE_SCORE_SQRTSOFTPLUS)
    return fail(MOE_ERR_INVALID_ARG, "unknown score function %d", c->score_func);
  if (!(isfinite(c->swiglu_limit) && c->swiglu_limit >= 0.f))
    return fail(MOE_ERR_INVALID_ARG, "swiglu_limit must be finite and >= 0 (0 = off)");
  if (c->pre_norm != 0 && c->pre_norm != 1)
    return fail(MOE_ERR_INVALID_ARG, "pre_norm must be 0 or 1");
  if (!(isfinite(c->norm_eps) && c->norm_eps >= 0.f))
    return fail(MOE_ERR_INVALID_ARG, "norm_eps must be finite and >= 0");
  if (c->renormalize != 0 && c->renormalize != 1)
    return fail(MOE_ERR_INVALID_ARG, "renormalize must be 0 or 1");
  if (!(isfinite(c->route_scale) && c->route_scale > 0.f))
    return fail(MOE_ERR_INVALID_ARG, "route_scale must be finite and > 0");
  if (c->n_groups < 1) return fail(MOE_ERR_INVALID_ARG, "n_groups must be >= 1");
  if (c->n_groups > 1) {
    if (c->n_groups > moe::kMaxGroups)
      return fail(MOE_ERR_UNSUPPORTED, "n_groups > %d is not supported", moe::kMaxGroups);
    if (c->E % c->n_groups)
      return fail(MOE_ERR_INVALID_ARG, "n_groups (%d) must divide E (%d)", c->n_groups, c->E);
    if (c->topk_groups < 1 || c->topk_groups > c->n_groups)
      return fail(MOE_ERR_INVALID_ARG, "topk_groups must be in [1, n_groups]");
    if (c->group_rule != MOE_GROUP_TOP2SUM && c->group_rule != MOE_GROUP_MAX)
      return fail(MOE_ERR_INVALID_ARG, "unknown group rule %d", c->group_rule);
    const int gsz = c->E / c->n_groups;
    if (c->group_rule == MOE_GROUP_TOP2SUM && gsz < 2)
      return fail(MOE_ERR_INVALID_ARG, "the top-2-sum group rule needs >= 2 experts per group");
    if (c->top_k > c->topk_groups * gsz)
      return fail(MOE_ERR_INVALID_ARG, "top_k exceeds the experts of the allowed groups");
  }
  if (!isfinite(c->capacity_factor))
    return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be finite");
  if ((long long)c->T * c->top_k > 0x7fffffffLL)
    return fail(MOE_ERR_UNSUPPORTED, "T*top_k exceeds int32");
  if (c->act_dtype == MOE_BF16) {
    if (c->D % 64 || c->H % 64 || c->H_shared % 64)
      return fail(MOE_ERR_UNSUPPORTED, "bf16 path needs D, H, H_shared multiples of 64");
  } else if (c->D % 16) {
    return fail(MOE_ERR_UNSUPPORTED, "fp32 path needs D a multiple of 16");
  }
  if (c->router_dtype == MOE_F32 && c->D % 16)
    return fail(MOE_ERR_UNSUPPORTED, "an fp32 router needs D a multiple of 16");
  return MOE_OK;
}

long long capacity_of(const moe_config* c) {
  const long long tk = (long long)c->T * c->top_k;
  if (!(c->capacity_factor > 0.0)) return tk;
  const double v = ceil(c->capacity_factor * (double)tk / (double)c->E);
  long long cap = v < 1.0 ? 1 : (v > (double)tk ? tk : (long long)v);
  return cap;
}

long long max_rows_of(const moe_config* c) {
  const long long tk = (long long)c->T * c->top_k;
  if (!(c->capacity_factor > 0.0)) return tk;
  return std::min(tk, (long long)c->E * capacity_of(c));
}

struct Layout {
  size_t ids, gate_w, counts, aux, logits, hist, pe_part, z_part, valid_part, block_base,
      counts_ws, pe_ws,
      offsets, n_kept, r2a, a2r, hbuf, y, shared_y, tail, x_norm, total;
};

// tail_slot_bytes: slot size of the grouped GEMMs' split-K partial tiles.
Layout layout_of(const moe_config* c, size_t tail_slot_bytes = moe::kTailSlotBytes) {
  Layout L{};
  const size_t T = c->T, k = c->top_k, E = c->E, D = c->D;
  const size_t nblk = moe::route_blocks(c->T);
  const size_t rows = (size_t)max_rows_of(c);
  const size_t es = esize(c->act_dtype);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.ids = take(T * k * 4);
  L.gate_w = take(T * k * 4);
  L.counts = take(E * 4);
  L.aux = take(2 * 4);
  const bool mfma16 = c->act_dtype == MOE_BF16 && c->router_dtype == MOE_BF16;
  L.logits = take(moe::route_fused(c->D, c->E, c->router_dtype == MOE_BF16)
                      ? 0
                      : (size_t)moe::route_ksplit(c->T, c->D, c->E, mfma16) * T * E * 4);
  L.hist = take(nblk * E * 4);
  L.pe_part = take(nblk * E * 4);
  L.z_part = take(nblk * 4);
  L.valid_part = take(nblk * 4);
  L.block_base = take(nblk * E * 4);
  L.counts_ws = take(E * 4);
  L.pe_ws = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.n_kept = take(4);
  L.r2a = take(std::max<size_t>(rows, 1) * 4);
  L.a2r = take(T * k * 4);
  L.hbuf = take(std::max(rows * (size_t)c->H, T * (size_t)c->H_shared) * es);
  L.y = take(rows * D * es);
  L.shared_y = take(c->H_shared ? T * D * es : 0);
  L.tail = take(c->act_dtype == MOE_BF16 ? moe::tail_workspace_bytes(tail_slot_bytes) : 0);
  L.x_norm = take(c->pre_norm ? T * D * es : 0);
  L.total = off;
  return L;
}

// Backward workspace: the forward layout (route and permutation scratch),
// then the backward's own buffers.
struct BwdLayout {
  size_t logits, padoff, wrT, act, p1, p2, dact, dgu, dw, dh, dz, dxr, dFT, XT, sact, sp1,
      sp2, sdact, sdgu, sdz, doutT, sgv, sdw, sgp, ninv,
      ndwp, total;
  int Epad, Tpad, Kpad;
};

BwdLayout bwd_layout_of(const moe_config* c) {
  BwdLayout B{};
  const Layout L = layout_of(c);
  size_t off = L.total;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const size_t T = c->T, D = c->D, H = c->H, E = c->E, Hs = c->H_shared;
  const size_t R = (size_t)std::max<long long>(max_rows_of(c), 1);
  B.Epad = (int)((E + 63) / 64 * 64);
  B.Tpad = (int)((T + 63) / 64 * 64);
  B.Kpad = (int)((R + 64 * E + 63) / 64 * 64);
  const size_t Kp = B.Kpad, Tp = B.Tpad, Ep = B.Epad;
  B.logits = take(T * E * 4);
  B.padoff = take((E + 1) * 4);
  B.wrT = take(D * Ep * 2);
  B.act = take(R * H * 2);
  B.p1 = take(R * H * 2);
  B.p2 = take(R * H * 2);
  B.dact = take(R * H * 2);
  B.dgu = take(R * 2 * H * 2);
  B.dw = take(R * 4);
  B.dh = take(T * Ep * 2);
  B.dz = take(R * D * 4);
  B.dxr = take(T * D * 4);
  B.dFT = take(D * Kp * 2);
  B.XT = take(D * Kp * 2);
  if (Hs) {
    B.sact = take(T * Hs * 2);
    B.sp1 = take(T * Hs * 2);
    B.sp2 = take(T * Hs * 2);
    B.sdact = take(T * Hs * 2);
    B.sdgu = take(T * 2 * Hs * 2);
    B.sdz = take(T * D * 4);
    B.doutT = take(D * Tp * 2);
    // the shared expert's gate: g per token, <dout, S> per token, dL/dw_sg partials
    B.sgv = take(T * 4);
    B.sdw = take(T * 4);
    B.sgp = take((size_t)moe::gate_dw_chunks((int)T) * D * 4);
  }
  if (c->pre_norm) {  // the norm's backward: 1/s per row, weight-gradient partials
    B.ninv = take(T * 4);
    B.ndwp = take((size_t)moe::rmsnorm_dw_chunks((int)T) * D * 4);
  }
  B.total = off;
  return B;
}

moe_status check_ws(const moe_config* c, void* ws, size_t bytes) {
  const size_t need = layout_of(c).total;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(MOE_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  if (bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", bytes, need);
  return MOE_OK;
}

// The norm kernels move 16-byte chunks.
moe_status check_align16(const void* p, const char* name) {
  if (reinterpret_cast<uintptr_t>(p) % 16)
    return fail(MOE_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  return MOE_OK;
}

// The pointer must be device (or managed) memory of the current device.
moe_status check_dev(const void* p, const char* name, bool required) {
  if (!p) {
    if (required) return fail(MOE_ERR_NULL_PTR, "%s is NULL", name);
    return MOE_OK;
  }
  hipPointerAttribute_t a;
  memset(&a, 0, sizeof a);
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(MOE_ERR_DEVICE, "%s is not a HIP allocation", name);
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed");
  if (a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged)
    return fail(MOE_ERR_DEVICE, "%s is not device memory", name);
  if (a.device != dev)
    return fail(MOE_ERR_DEVICE, "%s lives on device %d, current device is %d", name, a.device,
                dev);
  return MOE_OK;
}

#define MOE_TRY(expr)                   \
  do {                                  \
    const moe_status _s = (expr);       \
    if (_s != MOE_OK) return _s;        \
  } while (0)

moe_status hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Scratch of moe_forward_noalloc: a static device array, one copy on every
// GPU the library runs on, held until the process ends.  Host code never
// uses the array's own name as a device address (on the host it names a
// stand-in); the address of the current device's copy comes from
// hipGetSymbolAddress on that device's first call and is kept per device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

moe_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_HIP, "moe_forward_noalloc: no usable current device");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "moe_forward_noalloc: hipGetSymbolAddress of the scratch "
                  "array failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

moe::RouteParams route_params(const moe_config* c, const void* x, const void* w_router,
                              const float* lb, const float* sb, const uint8_t* mask,
                              int32_t* ids, float* gw, void* ws, const Layout& L) {
  moe::RouteParams p{};
  p.T = c->T;
  p.D = c->D;
  p.E = c->E;
  p.k = c->top_k;
  p.score_func = c->score_func;
  p.renormalize = c->renormalize;
  p.n_groups = c->n_groups;
  p.topk_groups = c->topk_groups;
  p.group_rule = c->group_rule;
  p.route_scale = c->route_scale;
  p.act_bf16 = c->act_dtype == MOE_BF16;
  p.router_bf16 = c->router_dtype == MOE_BF16;
  p.x = x;
  p.w_router = w_router;
  p.logit_bias = lb;
  p.select_bias = sb;
  p.token_mask = mask;
  p.ids = ids;
  p.gate_w = gw;
  p.logits_part = at<float>(ws, L.logits);
  p.ksplit = moe::route_ksplit(c->T, c->D, c->E, p.act_bf16 && p.router_bf16);
  p.tile = moe::route_tile(c->T);
  p.hist = at<int32_t>(ws, L.hist);
  p.pe_part = at<float>(ws, L.pe_part);
  p.z_part = at<float>(ws, L.z_part);
  p.valid_part = at<int32_t>(ws, L.valid_part);
  return p;
}

// Finalize (counts, P_e, aux, expert offsets) and, when sp.ids is set, the
// scatter, from the per-tile histograms in place: one workgroup for small
// batches, else the per-expert scans and the per-tile scatter.
moe_status launch_permutation(const moe::FinalizeParams& fp, const moe::ScatterParams& sp,
                              hipStream_t stream) {
  if (moe::permute_fits_one_block(fp.T, fp.E, fp.k))
    return hip_ok(moe::launch_permute_small(fp, sp, stream), "permute kernel");
  if (sp.ids) return hip_ok(moe::launch_finalize_scatter(fp, sp, stream), "permute kernels");
  return hip_ok(moe::launch_finalize(fp, stream), "finalize kernel");
}

moe::GemmParams gemm_params(const moe_config* c, int n_groups, int hidden, const void* x,
                            const int32_t* r2a, const int32_t* offsets, int max_rows,
                            const float* gw, const void* wg, const void* wu, const void* wd,
                            void* hbuf, void* y, void* tail,
                            size_t tail_slot_bytes = moe::kTailSlotBytes) {
  moe::GemmParams p{};
  if (tail) {
    char* t = static_cast<char*>(tail);
    const size_t parts = (size_t)moe::kXcds * moe::kTailSlots * tail_slot_bytes;
    p.tail_part = reinterpret_cast<float*>(t);
    p.tail_meta = reinterpret_cast<int32_t*>(t + parts);
    p.tail_desc = reinterpret_cast<int32_t*>(t + parts + 256);
    p.tail_slot_floats = tail_slot_bytes / 4;
  }
  p.T = c->T;
  p.D = c->D;
  p.k = c->top_k;
  p.n_groups = n_groups;
  p.hidden = hidden;
  p.max_rows = max_rows;
  p.x = x;
  p.row_to_assign = r2a;
  p.expert_offsets = offsets;
  p.gate_w = gw;
  p.w_gate = wg;
  p.w_up = wu;
  p.w_down = wd;
  p.hbuf = hbuf;
  p.y = y;
  p.swiglu_limit = c->swiglu_limit;
  return p;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_NULL_PTR: return "MOE_ERR_NULL_PTR";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_check_config(const moe_config* cfg) {
  MOE_TRY(check_config(cfg));
  return ok();
}

int32_t moe_capacity(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return -1;
  return (int32_t)capacity_of(cfg);
}

int32_t moe_max_rows(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return -1;
  return (int32_t)max_rows_of(cfg);
}

size_t moe_workspace_bytes(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return layout_of(cfg).total;
}

// Saved SwiGLU state: act, p1, p2 of every routed row [rows, H], then the
// same of the shared expert [T, Hs], bf16.
struct SavedLayout {
  size_t act, p1, p2, sact, sp1, sp2, total;
};

SavedLayout saved_layout_of(const moe_config* c) {
  SavedLayout S{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const size_t R = (size_t)max_rows_of(c), H = c->H, T = c->T, Hs = c->H_shared;
  S.act = take(R * H * 2);
  S.p1 = take(R * H * 2);
  S.p2 = take(R * H * 2);
  S.sact = take(T * Hs * 2);
  S.sp1 = take(T * Hs * 2);
  S.sp2 = take(T * Hs * 2);
  S.total = off;
  return S;
}

size_t moe_saved_bytes(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK || cfg->act_dtype != MOE_BF16) return 0;
  return saved_layout_of(cfg).total;
}

moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* logit_bias, const float* select_bias,
                     const uint8_t* token_mask, int32_t* expert_ids, float* gate_w,
                     int32_t* counts, float* aux, float* mean_prob, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_config(cfg));
  if (!x || !w_router || !expert_ids || !gate_w || !counts)
    return fail(MOE_ERR_NULL_PTR, "moe_route: x, w_router, expert_ids, gate_w, counts required");
  MOE_TRY(check_ws(cfg, workspace, workspace_bytes));
  MOE_TRY(check_dev(x, "x", true));
  MOE_TRY(check_dev(w_router, "w_router", true));
  MOE_TRY(check_dev(logit_bias, "logit_bias", false));
  MOE_TRY(check_dev(select_bias, "select_bias", false));
  MOE_TRY(check_dev(token_mask, "token_mask", false));
  MOE_TRY(check_dev(expert_ids, "expert_ids", true));
  MOE_TRY(check_dev(gate_w, "gate_w", true));
  MOE_TRY(check_dev(counts, "counts", true));
  MOE_TRY(check_dev(aux, "aux", false));
  MOE_TRY(check_dev(mean_prob, "mean_prob", false));
  MOE_TRY(check_dev(workspace, "workspace", true));
  const Layout L = layout_of(cfg);
  const moe::RouteParams rp = route_params(cfg, x, w_router, logit_bias, select_bias, token_mask,
                                          expert_ids, gate_w, workspace, L);
  MOE_TRY(hip_ok(moe::launch_route(rp, stream), "route kernel"));
  moe::FinalizeParams fp{};
  fp.T = cfg->T;
  fp.E = cfg->E;
  fp.k = cfg->top_k;
  fp.nblk = moe::route_blocks(cfg->T);
  fp.capacity = 0;
  fp.hist = rp.hist;
  fp.counts_ws = at<int32_t>(workspace, L.counts_ws);
  fp.pe_ws = at<float>(workspace, L.pe_ws);
  fp.pe_part = rp.pe_part;
  fp.z_part = rp.z_part;
  fp.valid_part = rp.valid_part;
  fp.counts = counts;
  fp.aux = aux;
  fp.mean_prob = mean_prob;
  MOE_TRY(launch_permutation(fp, moe::ScatterParams{}, stream));
  return ok();
}

moe_status moe_permute(const moe_config* cfg, const int32_t* expert_ids, int32_t capacity,
                       int32_t* expert_offsets, int32_t* row_to_assign, int32_t* assign_to_row,
                       int32_t* n_kept, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  MOE_TRY(check_config(cfg));
  if (!expert_ids || !expert_offsets || !row_to_assign || !assign_to_row || !n_kept)
    return fail(MOE_ERR_NULL_PTR, "moe_permute: every array argument is required");
  MOE_TRY(check_ws(cfg, workspace, workspace_bytes));
  MOE_TRY(check_dev(expert_ids, "expert_ids", true));
  MOE_TRY(check_dev(expert_offsets, "expert_offsets", true));
  MOE_TRY(check_dev(row_to_assign, "row_to_assign", true));
  MOE_TRY(check_dev(assign_to_row, "assign_to_row", true));
  MOE_TRY(check_dev(n_kept, "n_kept", true));
  MOE_TRY(check_dev(workspace, "workspace", true));
  const Layout L = layout_of(cfg);
  int32_t* hist = at<int32_t>(workspace, L.hist);
  int32_t* base = at<int32_t>(workspace, L.block_base);
  MOE_TRY(hip_ok(moe::launch_hist(cfg->T, cfg->E, cfg->top_k, expert_ids, hist, stream),
                 "hist kernel"));
  moe::FinalizeParams fp{};
  fp.T = cfg->T;
  fp.E = cfg->E;
  fp.k = cfg->top_k;
  fp.nblk = moe::route_blocks(cfg->T);
  fp.capacity = capacity > 0 ? capacity : 0;
  fp.hist = hist;
  fp.counts_ws = at<int32_t>(workspace, L.counts_ws);
  fp.pe_ws = at<float>(workspace, L.pe_ws);
  fp.block_base = base;
  fp.expert_offsets = expert_offsets;
  fp.n_kept = n_kept;
  moe::ScatterParams sp{cfg->T, cfg->E, cfg->top_k, fp.capacity, moe::route_tile(cfg->T),
                        expert_ids, base, expert_offsets, row_to_assign, assign_to_row};
  MOE_TRY(launch_permutation(fp, sp, stream));
  return ok();
}

moe_status moe_grouped_swiglu(const moe_config* cfg, int32_t n_experts, int32_t hidden,
                              const void* x, const int32_t* row_to_assign,
                              const int32_t* expert_offsets, int32_t max_rows,
                              const float* gate_w, const void* w_gate, const void* w_up,
                              const void* w_down, void* y_rows, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_config(cfg));
  if (!x || !w_gate || !w_up || !w_down || !y_rows)
    return fail(MOE_ERR_NULL_PTR, "moe_grouped_swiglu: x, weights and y_rows are required");
  const bool identity = row_to_assign == nullptr;
  if (identity) {
    if (expert_offsets || n_experts != 1 || max_rows != cfg->T)
      return fail(MOE_ERR_INVALID_ARG,
                  "identity rows need expert_offsets=NULL, n_experts=1, max_rows=T");
  } else {
    if (!expert_offsets) return fail(MOE_ERR_NULL_PTR, "expert_offsets is NULL");
    if (n_experts < 1 || n_experts > moe::kMaxExperts)
      return fail(MOE_ERR_INVALID_ARG, "n_experts must be in [1, %d]", moe::kMaxExperts);
    if (max_rows < 0 || (long long)max_rows > (long long)cfg->T * cfg->top_k)
      return fail(MOE_ERR_INVALID_ARG, "max_rows must be in [0, T*top_k]");
  }
  if (hidden < 1) return fail(MOE_ERR_INVALID_ARG, "hidden must be >= 1");
  if (cfg->act_dtype == MOE_BF16 && hidden % 64)
    return fail(MOE_ERR_UNSUPPORTED, "bf16 path needs hidden a multiple of 64");
  const size_t hb_need = (size_t)std::max(max_rows, 0) * hidden * esize(cfg->act_dtype);
  if (!workspace) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(MOE_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  if (workspace_bytes < hb_need)
    return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes,
                hb_need);
  MOE_TRY(check_dev(x, "x", true));
  MOE_TRY(check_dev(row_to_assign, "row_to_assign", false));
  MOE_TRY(check_dev(expert_offsets, "expert_offsets", false));
  MOE_TRY(check_dev(gate_w, "gate_w", false));
  MOE_TRY(check_dev(w_gate, "w_gate", true));
  MOE_TRY(check_dev(w_up, "w_up", true));
  MOE_TRY(check_dev(w_down, "w_down", true));
  MOE_TRY(check_dev(y_rows, "y_rows", true));
  MOE_TRY(check_dev(workspace, "workspace", true));
  if (max_rows == 0) return ok();
  // Room after the Hb rows holds the split-K tail of the large-tile kernel
  // (a workspace of moe_workspace_bytes(cfg) always has it).
  void* tail = nullptr;
  if (cfg->act_dtype == MOE_BF16 && workspace_bytes >= align_up(hb_need) + moe::tail_workspace_bytes())
    tail = static_cast<char*>(workspace) + align_up(hb_need);
  const moe::GemmParams gp =
      gemm_params(cfg, n_experts, hidden, x, row_to_assign, expert_offsets, max_rows, gate_w,
                  w_gate, w_up, w_down, workspace, y_rows, tail);
  MOE_TRY(hip_ok(moe::launch_grouped_swiglu(gp, cfg->act_dtype == MOE_BF16, stream),
                 "grouped swiglu kernels"));
  return ok();
}

moe_status moe_combine(const moe_config* cfg, const void* y_rows, const int32_t* assign_to_row,
                       const void* shared_rows, const void* x, const void* shared_expert_gate,
                       const void* residual, void* out, hipStream_t stream) {
  MOE_TRY(check_config(cfg));
  if (!y_rows || !assign_to_row || !out)
    return fail(MOE_ERR_NULL_PTR, "moe_combine: y_rows, assign_to_row and out are required");
  if (shared_expert_gate && (!shared_rows || !x))
    return fail(MOE_ERR_INVALID_ARG,
                "moe_combine: shared_expert_gate needs shared_rows and x");
  MOE_TRY(check_dev(y_rows, "y_rows", true));
  MOE_TRY(check_dev(assign_to_row, "assign_to_row", true));
  MOE_TRY(check_dev(shared_rows, "shared_rows", false));
  MOE_TRY(check_dev(x, "x", false));
  MOE_TRY(check_dev(shared_expert_gate, "shared_expert_gate", false));
  MOE_TRY(check_dev(residual, "residual", false));
  MOE_TRY(check_dev(out, "out", true));
  moe::CombineParams p{cfg->T, cfg->D, cfg->top_k,        y_rows,   assign_to_row,
                       shared_rows, x, shared_expert_gate, residual, out};
  MOE_TRY(hip_ok(moe::launch_combine(p, cfg->act_dtype == MOE_BF16, stream), "combine kernel"));
  return ok();
}

moe_status moe_rmsnorm(const moe_config* cfg, const void* x, const float* norm_weight,
                       void* x_norm, hipStream_t stream) {
  MOE_TRY(check_config(cfg));
  if (!x || !x_norm) return fail(MOE_ERR_NULL_PTR, "moe_rmsnorm: x and x_norm are required");
  MOE_TRY(check_dev(x, "x", true));
  MOE_TRY(check_dev(norm_weight, "norm_weight", false));
  MOE_TRY(check_dev(x_norm, "x_norm", true));
  MOE_TRY(check_align16(x, "x"));
  MOE_TRY(check_align16(norm_weight, "norm_weight"));
  MOE_TRY(check_align16(x_norm, "x_norm"));
  MOE_TRY(hip_ok(moe::launch_rmsnorm(cfg->T, cfg->D, cfg->act_dtype == MOE_BF16, x, norm_weight,
                                     cfg->norm_eps, x_norm, stream),
                 "rmsnorm kernel"));
  return ok();
}

// Argument checks of the forward entry points (all but the workspace); `who`
// names the entry point in error messages.
static moe_status forward_checks(const char* who, const moe_config* cfg, const void* x,
                                 const float* norm_weight, const void* w_router,
                                 const float* logit_bias, const float* select_bias,
                                 const uint8_t* token_mask, const void* w_gate, const void* w_up,
                                 const void* w_down, const void* w_shared_gate,
                                 const void* w_shared_up, const void* w_shared_down,
                                 const void* shared_expert_gate, const void* residual, void* out,
                                 int32_t* expert_ids, float* gate_w, int32_t* counts, float* aux,
                                 void* saved) {
  if (saved && cfg->act_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "%s: saved needs bf16 activations", who);
  if (!x || !w_router || !w_gate || !w_up || !w_down || !out)
    return fail(MOE_ERR_NULL_PTR, "%s: x, w_router, expert weights and out required", who);
  if (cfg->H_shared > 0 && (!w_shared_gate || !w_shared_up || !w_shared_down))
    return fail(MOE_ERR_NULL_PTR, "%s: H_shared > 0 needs the shared-expert weights", who);
  if (shared_expert_gate && cfg->H_shared == 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: shared_expert_gate needs a shared expert", who);
  if (norm_weight && !cfg->pre_norm)
    return fail(MOE_ERR_INVALID_ARG, "%s: norm_weight needs cfg->pre_norm = 1", who);
  MOE_TRY(check_dev(x, "x", true));
  MOE_TRY(check_dev(norm_weight, "norm_weight", false));
  MOE_TRY(check_dev(w_router, "w_router", true));
  MOE_TRY(check_dev(logit_bias, "logit_bias", false));
  MOE_TRY(check_dev(select_bias, "select_bias", false));
  MOE_TRY(check_dev(token_mask, "token_mask", false));
  MOE_TRY(check_dev(shared_expert_gate, "shared_expert_gate", false));
  MOE_TRY(check_dev(residual, "residual", false));
  MOE_TRY(check_dev(w_gate, "w_gate", true));
  MOE_TRY(check_dev(w_up, "w_up", true));
  MOE_TRY(check_dev(w_down, "w_down", true));
  if (cfg->H_shared > 0) {
    MOE_TRY(check_dev(w_shared_gate, "w_shared_gate", true));
    MOE_TRY(check_dev(w_shared_up, "w_shared_up", true));
    MOE_TRY(check_dev(w_shared_down, "w_shared_down", true));
  }
  MOE_TRY(check_dev(out, "out", true));
  MOE_TRY(check_dev(expert_ids, "expert_ids", false));
  MOE_TRY(check_dev(gate_w, "gate_w", false));
  MOE_TRY(check_dev(counts, "counts", false));
  MOE_TRY(check_dev(aux, "aux", false));
  MOE_TRY(check_dev(saved, "saved", false));
  if (reinterpret_cast<uintptr_t>(saved) % kAlign)
    return fail(MOE_ERR_INVALID_ARG, "saved must be %zu-byte aligned", kAlign);
  if (cfg->pre_norm) {
    MOE_TRY(check_align16(x, "x"));
    MOE_TRY(check_align16(norm_weight, "norm_weight"));
  }
  return MOE_OK;
}

// The stream-ordered launches of the forward on a checked workspace laid out
// as L (split-K tail slots of tail_slot_bytes).
static moe_status forward_launch(const moe_config* cfg, const void* x, const float* norm_weight,
                                 const void* w_router, const float* logit_bias,
                                 const float* select_bias, const uint8_t* token_mask,
                                 const void* w_gate, const void* w_up, const void* w_down,
                                 const void* w_shared_gate, const void* w_shared_up,
                                 const void* w_shared_down, const void* shared_expert_gate,
                                 const void* residual, void* out, int32_t* expert_ids,
                                 float* gate_w, int32_t* counts, float* aux, void* saved,
                                 void* workspace, const Layout& L, size_t tail_slot_bytes,
                                 hipStream_t stream) {
  int32_t* ids = expert_ids ? expert_ids : at<int32_t>(workspace, L.ids);
  float* gw = gate_w ? gate_w : at<float>(workspace, L.gate_w);
  int32_t* cnt = counts ? counts : at<int32_t>(workspace, L.counts);
  float* ax = aux ? aux : at<float>(workspace, L.aux);
  int32_t* offsets = at<int32_t>(workspace, L.offsets);
  int32_t* r2a = at<int32_t>(workspace, L.r2a);
  int32_t* a2r = at<int32_t>(workspace, L.a2r);
  const int cap = (int)capacity_of(cfg);
  const bool dropless = !(cfg->capacity_factor > 0.0);
  const int rows = (int)max_rows_of(cfg);

  if (cfg->pre_norm) {  // the layer takes the normalised rows from here on
    void* xn = at<void>(workspace, L.x_norm);
    MOE_TRY(hip_ok(moe::launch_rmsnorm(cfg->T, cfg->D, cfg->act_dtype == MOE_BF16, x,
                                       norm_weight, cfg->norm_eps, xn, stream),
                   "rmsnorm kernel"));
    x = xn;
  }
  const moe::RouteParams rp =
      route_params(cfg, x, w_router, logit_bias, select_bias, token_mask, ids, gw, workspace, L);
  MOE_TRY(hip_ok(moe::launch_route(rp, stream), "route kernel"));
  moe::FinalizeParams fp{};
  fp.T = cfg->T;
  fp.E = cfg->E;
  fp.k = cfg->top_k;
  fp.nblk = moe::route_blocks(cfg->T);
  fp.capacity = dropless ? 0 : cap;
  fp.hist = rp.hist;
  fp.counts_ws = at<int32_t>(workspace, L.counts_ws);
  fp.pe_ws = at<float>(workspace, L.pe_ws);
  fp.pe_part = rp.pe_part;
  fp.z_part = rp.z_part;
  fp.valid_part = rp.valid_part;
  fp.counts = cnt;
  fp.aux = ax;
  fp.block_base = at<int32_t>(workspace, L.block_base);
  fp.expert_offsets = offsets;
  fp.n_kept = at<int32_t>(workspace, L.n_kept);
  moe::ScatterParams sp{cfg->T, cfg->E, cfg->top_k, fp.capacity, moe::route_tile(cfg->T), ids,
                        fp.block_base, offsets, r2a, a2r};
  MOE_TRY(launch_permutation(fp, sp, stream));

  void* hbuf = at<void>(workspace, L.hbuf);
  void* y = at<void>(workspace, L.y);
  const bool bf16 = cfg->act_dtype == MOE_BF16;
  void* tail = bf16 ? at<void>(workspace, L.tail) : nullptr;
  // With `saved`, Hb of the routed rows and of the shared expert lives there
  // (act), next to the SwiGLU factors the gate/up epilogues add.
  const SavedLayout SV = saved_layout_of(cfg);
  auto sv = [&](size_t off) { return reinterpret_cast<uint16_t*>(static_cast<char*>(saved) + off); };
  moe::GemmParams gp = gemm_params(cfg, cfg->E, cfg->H, x, r2a, offsets, rows, gw, w_gate, w_up,
                                   w_down, saved ? sv(SV.act) : hbuf, y, tail, tail_slot_bytes);
  if (saved) {
    gp.save_p1 = sv(SV.p1);
    gp.save_p2 = sv(SV.p2);
  }
  MOE_TRY(hip_ok(moe::launch_grouped_swiglu(gp, bf16, stream), "grouped swiglu kernels"));
  void* sy = nullptr;
  if (cfg->H_shared > 0) {
    sy = at<void>(workspace, L.shared_y);
    moe::GemmParams sp2 =
        gemm_params(cfg, 1, cfg->H_shared, x, nullptr, nullptr, cfg->T, nullptr, w_shared_gate,
                    w_shared_up, w_shared_down, saved ? sv(SV.sact) : hbuf, sy, tail,
                    tail_slot_bytes);
    if (saved) {
      sp2.save_p1 = sv(SV.sp1);
      sp2.save_p2 = sv(SV.sp2);
    }
    MOE_TRY(hip_ok(moe::launch_grouped_swiglu(sp2, bf16, stream), "shared expert kernels"));
  }
  moe::CombineParams cp{cfg->T, cfg->D, cfg->top_k, y,        a2r,
                        sy,     x,      shared_expert_gate,      residual, out};
  MOE_TRY(hip_ok(moe::launch_combine(cp, bf16, stream), "combine kernel"));
  return ok();
}


moe_status moe_forward(const moe_config* cfg, const void* x, const float* norm_weight,
                       const void* w_router,
                       const float* logit_bias, const float* select_bias,
                       const uint8_t* token_mask, const void* w_gate, const void* w_up,
                       const void* w_down, const void* w_shared_gate, const void* w_shared_up,
                       const void* w_shared_down, const void* shared_expert_gate,
                       const void* residual, void* out, int32_t* expert_ids, float* gate_w,
                       int32_t* counts, float* aux, void* saved,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  MOE_TRY(check_config(cfg));
  MOE_TRY(forward_checks("moe_forward", cfg, x, norm_weight, w_router, logit_bias, select_bias,
                        token_mask, w_gate, w_up, w_down, w_shared_gate, w_shared_up,
                        w_shared_down, shared_expert_gate, residual, out, expert_ids, gate_w,
                        counts, aux, saved));
  MOE_TRY(check_ws(cfg, workspace, workspace_bytes));
  MOE_TRY(check_dev(workspace, "workspace", true));
  return forward_launch(cfg, x, norm_weight, w_router, logit_bias, select_bias,
                        token_mask, w_gate, w_up, w_down, w_shared_gate, w_shared_up,
                        w_shared_down, shared_expert_gate, residual, out, expert_ids, gate_w,
                        counts, aux, saved, workspace,
                        layout_of(cfg), moe::kTailSlotBytes, stream);
}

moe_status moe_forward_noalloc(const moe_config* cfg, const void* x, const float* norm_weight,
                               const void* w_router, const float* logit_bias,
                               const float* select_bias, const uint8_t* token_mask,
                               const void* w_gate, const void* w_up, const void* w_down,
                               const void* w_shared_gate, const void* w_shared_up,
                               const void* w_shared_down, const void* shared_expert_gate,
                               const void* residual, void* out, int32_t* expert_ids,
                               float* gate_w, int32_t* counts, float* aux, void* saved,
                               hipStream_t stream) {
  MOE_TRY(check_config(cfg));
  // Compact split-K tail slots: the decode-sized 32-row GEMMs split their
  // last round as in moe_forward; larger tiles run it unsplit.
  const Layout L = layout_of(cfg, moe::kSmallTailSlotBytes);
  if (L.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_forward_noalloc: this configuration needs %zu bytes of scratch, more than "
                "the library's static %zu bytes; use moe_forward with a workspace",
                L.total, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  MOE_TRY(forward_checks("moe_forward_noalloc", cfg, x, norm_weight, w_router, logit_bias, select_bias,
                        token_mask, w_gate, w_up, w_down, w_shared_gate, w_shared_up,
                        w_shared_down, shared_expert_gate, residual, out, expert_ids, gate_w,
                        counts, aux, saved));
  void* ws = nullptr;
  MOE_TRY(noalloc_scratch(&ws));
  return forward_launch(cfg, x, norm_weight, w_router, logit_bias, select_bias,
                        token_mask, w_gate, w_up, w_down, w_shared_gate, w_shared_up,
                        w_shared_down, shared_expert_gate, residual, out, expert_ids, gate_w,
                        counts, aux, saved, ws, L,
                        moe::kSmallTailSlotBytes, stream);
}

size_t moe_backward_workspace_bytes(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK || cfg->act_dtype != MOE_BF16) return 0;
  return bwd_layout_of(cfg).total;
}

moe_status moe_backward(const moe_config* cfg, const void* x, const float* norm_weight,
                        const void* w_router, const float* logit_bias, const void* w_gate,
                        const void* w_up, const void* w_down, const void* w_shared_gate,
                        const void* w_shared_up, const void* w_shared_down,
                        const void* shared_expert_gate, const int32_t* expert_ids,
                        const float* gate_w, const void* dout, float balance_coef, float z_coef,
                        void* dx, float* dw_router, float* dw_gate, float* dw_up,
                        float* dw_down, float* dws_gate, float* dws_up, float* dws_down,
                        float* d_shared_gate, float* d_gate_w, float* d_norm_weight,
                        const void* saved, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  MOE_TRY(check_config(cfg));
  if (cfg->act_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "moe_backward: bf16 activations only");
  if ((norm_weight || d_norm_weight) && !cfg->pre_norm)
    return fail(MOE_ERR_INVALID_ARG,
                "moe_backward: norm_weight and d_norm_weight need cfg->pre_norm = 1");
  if ((shared_expert_gate || d_shared_gate) && cfg->H_shared == 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_backward: shared_expert_gate needs a shared expert");
  if (d_shared_gate && !shared_expert_gate)
    return fail(MOE_ERR_INVALID_ARG, "moe_backward: d_shared_gate needs shared_expert_gate");
  if (!x || !w_router || !w_gate || !w_up || !w_down || !expert_ids || !gate_w || !dout ||
      !dx || !dw_router || !dw_gate || !dw_up || !dw_down)
    return fail(MOE_ERR_NULL_PTR, "moe_backward: inputs, routing and gradient outputs required");
  const bool sh = cfg->H_shared > 0;
  if (sh && (!w_shared_gate || !w_shared_up || !w_shared_down || !dws_gate || !dws_up ||
             !dws_down))
    return fail(MOE_ERR_NULL_PTR, "moe_backward: H_shared > 0 needs the shared weights and grads");
  if (!isfinite(balance_coef) || !isfinite(z_coef))
    return fail(MOE_ERR_INVALID_ARG, "moe_backward: loss coefficients must be finite");
  const BwdLayout B = bwd_layout_of(cfg);
  if (!workspace) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(MOE_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  if (workspace_bytes < B.total)
    return fail(MOE_ERR_WORKSPACE, "backward workspace too small: %zu < %zu bytes",
                workspace_bytes, B.total);
  const void* dev_in[] = {x, w_router, w_gate, w_up, w_down, expert_ids, gate_w, dout, dx,
                          dw_router, dw_gate, dw_up, dw_down, workspace};
  const char* names[] = {"x", "w_router", "w_gate", "w_up", "w_down", "expert_ids", "gate_w",
                         "dout", "dx", "dw_router", "dw_gate", "dw_up", "dw_down", "workspace"};
  for (int i = 0; i < 14; ++i) MOE_TRY(check_dev(dev_in[i], names[i], true));
  MOE_TRY(check_dev(logit_bias, "logit_bias", false));
  MOE_TRY(check_dev(d_gate_w, "d_gate_w", false));
  MOE_TRY(check_dev(norm_weight, "norm_weight", false));
  MOE_TRY(check_dev(d_norm_weight, "d_norm_weight", false));
  MOE_TRY(check_dev(shared_expert_gate, "shared_expert_gate", false));
  MOE_TRY(check_dev(d_shared_gate, "d_shared_gate", false));
  MOE_TRY(check_dev(saved, "saved", false));
  MOE_TRY(check_align16(shared_expert_gate, "shared_expert_gate"));
  if (cfg->pre_norm) {
    MOE_TRY(check_align16(x, "x"));
    MOE_TRY(check_align16(norm_weight, "norm_weight"));
    MOE_TRY(check_align16(dx, "dx"));
  }
  if (sh) {
    MOE_TRY(check_dev(w_shared_gate, "w_shared_gate", true));
    MOE_TRY(check_dev(w_shared_up, "w_shared_up", true));
    MOE_TRY(check_dev(w_shared_down, "w_shared_down", true));
    MOE_TRY(check_dev(dws_gate, "dws_gate", true));
    MOE_TRY(check_dev(dws_up, "dws_up", true));
    MOE_TRY(check_dev(dws_down, "dws_down", true));
  }

  const Layout L = layout_of(cfg);
  const int T = cfg->T, D = cfg->D, H = cfg->H, E = cfg->E, k = cfg->top_k, Hs = cfg->H_shared;
  const int R = (int)max_rows_of(cfg);
  const int cap = (int)capacity_of(cfg);
  const bool dropless = !(cfg->capacity_factor > 0.0);
  auto ws = [&](size_t off) { return static_cast<char*>(workspace) + off; };
  auto u16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws(off)); };
  auto f32 = [&](size_t off) { return reinterpret_cast<float*>(ws(off)); };
  int32_t* offsets = at<int32_t>(workspace, L.offsets);
  int32_t* r2a = at<int32_t>(workspace, L.r2a);
  int32_t* a2r = at<int32_t>(workspace, L.a2r);
  int32_t* counts = at<int32_t>(workspace, L.counts_ws);
  int32_t* padoff = at<int32_t>(workspace, B.padoff);

  // 0. with the pre-norm, the layer's input is the normalised rows, recomputed
  // by the forward's own kernel (bit-identical)
  const void* x_raw = x;
  if (cfg->pre_norm) {
    void* xn = ws(L.x_norm);
    MOE_TRY(hip_ok(moe::launch_rmsnorm(T, D, true, x, norm_weight, cfg->norm_eps, xn, stream),
                   "rmsnorm kernel"));
    x = xn;
  }

  // 1. the forward's permutation, from the given routes
  MOE_TRY(hip_ok(moe::launch_hist(T, E, k, expert_ids, at<int32_t>(workspace, L.hist), stream),
                 "hist kernel"));
  moe::FinalizeParams fp{};
  fp.T = T;
  fp.E = E;
  fp.k = k;
  fp.nblk = moe::route_blocks(T);
  fp.capacity = dropless ? 0 : cap;
  fp.hist = at<int32_t>(workspace, L.hist);
  fp.counts_ws = counts;
  fp.pe_ws = at<float>(workspace, L.pe_ws);
  fp.block_base = at<int32_t>(workspace, L.block_base);
  fp.expert_offsets = offsets;
  fp.n_kept = at<int32_t>(workspace, L.n_kept);
  moe::ScatterParams sp{T, E, k, fp.capacity, moe::route_tile(T), expert_ids, fp.block_base,
                        offsets, r2a, a2r};
  MOE_TRY(launch_permutation(fp, sp, stream));
  MOE_TRY(hip_ok(moe::launch_pad_offsets(E, offsets, padoff, stream), "pad offsets kernel"));

  // 2. the logits (the routing kernels rerun; their own routes are not used)
  moe::RouteParams rp = route_params(cfg, x, w_router, logit_bias, nullptr, nullptr,
                                     at<int32_t>(workspace, L.ids),
                                     at<float>(workspace, L.gate_w), workspace, L);
  rp.logits_out = f32(B.logits);
  MOE_TRY(hip_ok(moe::launch_route(rp, stream), "route kernel"));

  // 3. K-contiguous copy of the router weights (the expert weights are read
  // k-major by the dgrad GEMMs)
  auto transpose = [&](int rows, int cols, const void* src, bool src_f32, long long ld_src,
                       long long src_b, int out_cols, uint16_t* dst, long long ld_dst,
                       long long dst_b, int col0, int batch, const int32_t* gather,
                       const float* scale, const int32_t* scale_idx, bool ragged,
                       const int32_t* skip_rows = nullptr) {
    moe::TransposeParams t{};
    t.rows = rows;
    t.cols = cols;
    t.src = src;
    t.src_f32 = src_f32;
    t.ld_src = ld_src;
    t.src_bstride = src_b;
    t.gather = gather;
    t.gdiv = k;
    t.scale = scale;
    t.scale_idx = scale_idx;
    t.offsets = ragged ? offsets : nullptr;
    t.padoff = ragged ? padoff : nullptr;
    t.G = E;
    t.out_cols = out_cols;
    t.dst = dst;
    t.ld_dst = ld_dst;
    t.dst_bstride = dst_b;
    t.dst_col0 = col0;
    t.batch = batch;
    t.skip_rows = skip_rows;
    return hip_ok(moe::launch_transpose(t, stream), "transpose kernel");
  };
  MOE_TRY(transpose(E, D, w_router, cfg->router_dtype == MOE_F32, D, 0, B.Epad, u16(B.wrT),
                    B.Epad, 0, 0, 1, nullptr, nullptr, nullptr, false));

  auto gemm = [&](moe::BwdGemmParams g, const char* what) {
    return hip_ok(moe::launch_bwd_gemm(g, stream), what);
  };
  const int kNoSplit = 0x7fffffff;
  // The SwiGLU state (act, p1, p2 per row): the forward's `saved`, else
  // recomputed into the workspace.
  const SavedLayout SV = saved_layout_of(cfg);
  auto state = [&](size_t saved_off, size_t ws_off) {
    return saved ? reinterpret_cast<uint16_t*>(const_cast<char*>(static_cast<const char*>(saved)) +
                                               saved_off)
                 : u16(ws_off);
  };
  uint16_t* const act_p = state(SV.act, B.act);
  uint16_t* const p1_p = state(SV.p1, B.p1);
  uint16_t* const p2_p = state(SV.p2, B.p2);
  uint16_t* const sact_p = state(SV.sact, B.sact);
  uint16_t* const sp1_p = state(SV.sp1, B.sp1);
  uint16_t* const sp2_p = state(SV.sp2, B.sp2);
  // 4. recompute gate/up: act, p1, p2 of every kept row
  {
    moe::BwdGemmParams g{};
    g.grouping = moe::BWD_MROWS;
    g.epilogue = moe::BWD_EPI_GATEUP_SAVE;
    g.N = H;
    g.K = D;
    g.G = E;
    g.offsets = offsets;
    g.max_rows = R;
    g.A = static_cast<const uint16_t*>(x);
    g.lda = D;
    g.gather = r2a;
    g.gdiv = k;
    g.B = static_cast<const uint16_t*>(w_gate);
    g.B2 = static_cast<const uint16_t*>(w_up);
    g.ldb = D;
    g.b_gstride = (long long)H * D;
    g.act = act_p;
    g.p1 = p1_p;
    g.p2 = p2_p;
    g.ldh = H;
    g.limit = cfg->swiglu_limit;
    g.a_bytes = 2ll * T * D;
    g.b_bytes = 2ll * H * D;
    if (!saved) MOE_TRY(gemm(g, "recompute gate/up"));
    // 5. down dgrad: dL/d act for unit gate weight (bf16), then the SwiGLU
    // backward with the gate weights: dg, du and dL/dw of every kept row
    moe::BwdGemmParams d{};
    d.grouping = moe::BWD_MROWS;
    d.epilogue = moe::BWD_EPI_F32;
    d.N = H;
    d.K = D;
    d.G = E;
    d.offsets = offsets;
    d.max_rows = R;
    d.A = static_cast<const uint16_t*>(dout);
    d.lda = D;
    d.gather = r2a;
    d.gdiv = k;
    d.B = static_cast<const uint16_t*>(w_down);  // [D][H]: k-major
    d.b_kmajor = 1;
    d.k_split = kNoSplit;
    d.ldb = H;
    d.b_gstride = (long long)D * H;
    d.Cb = u16(B.dact);
    d.ldc = H;
    d.c_split = kNoSplit;
    d.a_bytes = 2ll * T * D;
    d.b_bytes = 2ll * H * D;
    MOE_TRY(gemm(d, "down dgrad"));
    moe::SwigluBwdParams q{R, H, offsets, E, u16(B.dact), act_p, p1_p, p2_p,
                           gate_w, r2a, u16(B.dgu), f32(B.dw)};
    MOE_TRY(hip_ok(moe::launch_swiglu_bwd(q, stream), "swiglu backward kernel"));
  }
  // 6. router: dL/dh
  {
    moe::RouterBwdParams r{};
    r.T = T;
    r.E = E;
    r.Epad = B.Epad;
    r.k = k;
    r.score_func = cfg->score_func;
    r.renormalize = cfg->renormalize;
    r.route_scale = cfg->route_scale;
    r.alpha = balance_coef;
    r.beta = z_coef;
    r.logits = f32(B.logits);
    r.ids = expert_ids;
    r.a2r = a2r;
    r.dw = f32(B.dw);
    r.counts = counts;
    r.dh = u16(B.dh);
    r.dgw = d_gate_w;
    MOE_TRY(hip_ok(moe::launch_router_bwd(r, stream), "router backward kernel"));
  }
  // 7. input gradients: dz of every kept row, dx of the router, shared expert
  {
    moe::BwdGemmParams g{};
    g.grouping = moe::BWD_MROWS;
    g.epilogue = moe::BWD_EPI_F32;
    g.N = D;
    g.K = 2 * H;
    g.G = E;
    g.offsets = offsets;
    g.max_rows = R;
    g.A = u16(B.dgu);
    g.lda = 2 * H;
    g.B = static_cast<const uint16_t*>(w_gate);  // [H][D] then [H][D] of w_up: k-major
    g.B2 = static_cast<const uint16_t*>(w_up);
    g.b_kmajor = 1;
    g.k_split = H;
    g.ldb = D;
    g.b_gstride = (long long)H * D;
    g.C = f32(B.dz);
    g.ldc = D;
    g.c_split = kNoSplit;
    g.a_bytes = 2ll * R * 2 * H;
    g.b_bytes = 2ll * H * D;
    MOE_TRY(gemm(g, "gate/up dgrad"));
    moe::BwdGemmParams r{};
    r.grouping = moe::BWD_DENSE;
    r.epilogue = moe::BWD_EPI_F32;
    r.M = T;
    r.N = D;
    r.K = B.Epad;
    r.G = 1;
    r.A = u16(B.dh);
    r.lda = B.Epad;
    r.B = u16(B.wrT);
    r.ldb = B.Epad;
    r.C = f32(B.dxr);
    r.ldc = D;
    r.c_split = kNoSplit;
    r.a_bytes = 2ll * T * B.Epad;
    r.b_bytes = 2ll * D * B.Epad;
    MOE_TRY(gemm(r, "router dgrad"));
  }
  const uint16_t* sgate = static_cast<const uint16_t*>(shared_expert_gate);
  if (sh) {
    if (sgate)  // the shared expert's per-token gate on the layer's input rows
      MOE_TRY(hip_ok(moe::launch_shared_gate(T, D, static_cast<const uint16_t*>(x), sgate,
                                             f32(B.sgv), stream),
                     "shared gate kernel"));
    moe::BwdGemmParams g{};
    g.grouping = moe::BWD_DENSE;
    g.epilogue = moe::BWD_EPI_GATEUP_SAVE;
    g.M = T;
    g.N = Hs;
    g.K = D;
    g.G = 1;
    g.A = static_cast<const uint16_t*>(x);
    g.lda = D;
    g.B = static_cast<const uint16_t*>(w_shared_gate);
    g.B2 = static_cast<const uint16_t*>(w_shared_up);
    g.ldb = D;
    g.act = sact_p;
    g.p1 = sp1_p;
    g.p2 = sp2_p;
    g.ldh = Hs;
    g.limit = cfg->swiglu_limit;
    g.a_bytes = 2ll * T * D;
    g.b_bytes = 2ll * Hs * D;
    if (!saved) MOE_TRY(gemm(g, "shared recompute"));
    moe::BwdGemmParams d{};
    d.grouping = moe::BWD_DENSE;
    d.epilogue = moe::BWD_EPI_F32;
    d.M = T;
    d.N = Hs;
    d.K = D;
    d.G = 1;
    d.A = static_cast<const uint16_t*>(dout);
    d.lda = D;
    d.B = static_cast<const uint16_t*>(w_shared_down);  // [D][Hs]: k-major
    d.b_kmajor = 1;
    d.k_split = kNoSplit;
    d.ldb = Hs;
    d.Cb = u16(B.sdact);
    d.ldc = Hs;
    d.c_split = kNoSplit;
    d.a_bytes = 2ll * T * D;
    d.b_bytes = 2ll * Hs * D;
    MOE_TRY(gemm(d, "shared down dgrad"));
    // with the gate: the branch sees g_t dout_t, and <dout_t, S_t> (for the
    // gate's own gradient) is sum_h act * dact, as dL/dw of a routed row
    moe::SwigluBwdParams q{T, Hs, nullptr, 1, u16(B.sdact), sact_p, sp1_p, sp2_p,
                           sgate ? f32(B.sgv) : nullptr, nullptr, u16(B.sdgu),
                           sgate ? f32(B.sdw) : nullptr};
    MOE_TRY(hip_ok(moe::launch_swiglu_bwd(q, stream), "shared swiglu backward kernel"));
    moe::BwdGemmParams z{};
    z.grouping = moe::BWD_DENSE;
    z.epilogue = moe::BWD_EPI_F32;
    z.M = T;
    z.N = D;
    z.K = 2 * Hs;
    z.G = 1;
    z.A = u16(B.sdgu);
    z.lda = 2 * Hs;
    z.B = static_cast<const uint16_t*>(w_shared_gate);  // k-major, then w_shared_up
    z.B2 = static_cast<const uint16_t*>(w_shared_up);
    z.b_kmajor = 1;
    z.k_split = Hs;
    z.ldb = D;
    z.C = f32(B.sdz);
    z.ldc = D;
    z.c_split = kNoSplit;
    z.a_bytes = 2ll * T * 2 * Hs;
    z.b_bytes = 2ll * Hs * D;
    MOE_TRY(gemm(z, "shared gate/up dgrad"));
  }
  {
    // with the pre-norm, dL/d(normalised rows) stays fp32, in place over the
    // router's dx (each element is read before it is written, by one thread)
    moe::DxParams p{T, D, k, f32(B.dz), a2r, sh ? f32(B.sdz) : nullptr, f32(B.dxr),
                    cfg->pre_norm ? nullptr : dx, cfg->pre_norm ? f32(B.dxr) : nullptr,
                    sgate ? f32(B.sgv) : nullptr, sgate ? f32(B.sdw) : nullptr, sgate};
    MOE_TRY(hip_ok(moe::launch_dx(p, true, stream), "dx kernel"));
    if (cfg->pre_norm)
      MOE_TRY(hip_ok(moe::launch_rmsnorm_bwd(T, D, true, x_raw, norm_weight, cfg->norm_eps,
                                             f32(B.dxr), dx, f32(B.ninv), f32(B.ndwp),
                                             d_norm_weight, stream),
                     "rmsnorm backward kernel"));
  }

  // 8. weight gradients.  Row-major per-row operands (act, [dg du], dh, x)
  // are read k-major as they are; the gathered ones (w * dout rows, x rows
  // of the kept slots) are transposed with each expert's rows padded to 64.
  MOE_TRY(transpose(R, D, dout, false, D, 0, B.Kpad, u16(B.dFT), B.Kpad, 0, 0, 1, r2a, gate_w,
                    r2a, true));
  MOE_TRY(transpose(R, D, x, false, D, 0, B.Kpad, u16(B.XT), B.Kpad, 0, 0, 1, r2a, nullptr,
                    nullptr, true));
  {
    moe::BwdGemmParams g{};
    g.grouping = moe::BWD_KRAGGED;
    g.epilogue = moe::BWD_EPI_F32;
    g.M = D;
    g.N = H;
    g.G = E;
    g.offsets = padoff;
    g.A = u16(B.dFT);
    g.lda = B.Kpad;
    g.B = act_p;  // [rows, H]: k-major, the expert's rows from krows
    g.b_kmajor = 1;
    g.k_split = kNoSplit;
    g.krows = offsets;
    g.ldb = H;
    g.C = dw_down;
    g.ldc = H;
    g.c_gstride = (long long)D * H;
    g.c_split = kNoSplit;
    g.a_bytes = 2ll * D * B.Kpad;
    g.b_bytes = 2ll * R * H;
    MOE_TRY(gemm(g, "down wgrad"));
    moe::BwdGemmParams u{};
    u.grouping = moe::BWD_KRAGGED;
    u.epilogue = moe::BWD_EPI_F32;
    u.M = 2 * H;
    u.N = D;
    u.G = E;
    u.offsets = padoff;
    u.A = u16(B.dgu);  // [rows, 2H]: k-major
    u.a_kmajor = 1;
    u.krows = offsets;
    u.lda = 2 * H;
    u.B = u16(B.XT);
    u.ldb = B.Kpad;
    u.C = dw_gate;
    u.C2 = dw_up;
    u.ldc = D;
    u.c_gstride = (long long)H * D;
    u.c_split = H;
    u.a_bytes = 2ll * R * 2 * H;
    u.b_bytes = 2ll * D * B.Kpad;
    MOE_TRY(gemm(u, "gate/up wgrad"));
    moe::BwdGemmParams r{};
    r.grouping = moe::BWD_DENSE;
    r.epilogue = moe::BWD_EPI_F32;
    r.M = E;
    r.N = D;
    r.K = B.Tpad;
    r.G = 1;
    r.A = u16(B.dh);  // [T, Epad] and x [T, D]: both k-major, rows past T zero
    r.a_kmajor = 1;
    r.lda = B.Epad;
    r.B = static_cast<const uint16_t*>(x);
    r.b_kmajor = 1;
    r.k_split = kNoSplit;
    r.ldb = D;
    r.C = dw_router;
    r.ldc = D;
    r.c_split = kNoSplit;
    r.a_bytes = 2ll * T * B.Epad;
    r.b_bytes = 2ll * T * D;
    MOE_TRY(gemm(r, "router wgrad"));
  }
  if (sh) {
    MOE_TRY(transpose(T, D, dout, false, D, 0, B.Tpad, u16(B.doutT), B.Tpad, 0, 0, 1, nullptr,
                      sgate ? f32(B.sgv) : nullptr, nullptr, false));
    moe::BwdGemmParams g{};
    g.grouping = moe::BWD_DENSE;
    g.epilogue = moe::BWD_EPI_F32;
    g.M = D;
    g.N = Hs;
    g.K = B.Tpad;
    g.G = 1;
    g.A = u16(B.doutT);
    g.lda = B.Tpad;
    g.B = sact_p;  // [T, Hs]: k-major
    g.b_kmajor = 1;
    g.k_split = kNoSplit;
    g.ldb = Hs;
    g.C = dws_down;
    g.ldc = Hs;
    g.c_split = kNoSplit;
    g.a_bytes = 2ll * D * B.Tpad;
    g.b_bytes = 2ll * T * Hs;
    MOE_TRY(gemm(g, "shared down wgrad"));
    moe::BwdGemmParams u{};
    u.grouping = moe::BWD_DENSE;
    u.epilogue = moe::BWD_EPI_F32;
    u.M = 2 * Hs;
    u.N = D;
    u.K = B.Tpad;
    u.G = 1;
    u.A = u16(B.sdgu);  // [T, 2Hs] and x [T, D]: both k-major
    u.a_kmajor = 1;
    u.lda = 2 * Hs;
    u.B = static_cast<const uint16_t*>(x);
    u.b_kmajor = 1;
    u.k_split = kNoSplit;
    u.ldb = D;
    u.C = dws_gate;
    u.C2 = dws_up;
    u.ldc = D;
    u.c_split = Hs;
    u.a_bytes = 2ll * T * 2 * Hs;
    u.b_bytes = 2ll * T * D;
    MOE_TRY(gemm(u, "shared gate/up wgrad"));
    if (d_shared_gate)
      MOE_TRY(hip_ok(moe::launch_gate_dw(T, D, static_cast<const uint16_t*>(x), f32(B.sgv),
                                         f32(B.sdw), f32(B.sgp), d_shared_gate, stream),
                     "shared gate weight-gradient kernels"));
  }
  return ok();
}

moe_status moe_update_bias(const moe_config* cfg, const int32_t* counts, float gamma,
                           float* select_bias, hipStream_t stream) {
  MOE_TRY(check_config(cfg));
  if (!counts || !select_bias)
    return fail(MOE_ERR_NULL_PTR, "moe_update_bias: counts and select_bias are required");
  if (!isfinite(gamma)) return fail(MOE_ERR_INVALID_ARG, "gamma must be finite");
  MOE_TRY(check_dev(counts, "counts", true));
  MOE_TRY(check_dev(select_bias, "select_bias", true));
  MOE_TRY(hip_ok(moe::launch_update_bias(cfg->E, counts, gamma, select_bias, stream),
                 "update bias kernel"));
  return ok();
}

}  // extern "C"
