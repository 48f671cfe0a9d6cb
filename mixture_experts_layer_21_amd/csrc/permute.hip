// Expert histogram, scan and stable scatter: the dispatch bookkeeping of the
// layer, integer-only and bit-exact.
//
// Semantics follow "Lab: build a tiny MoE in PyTorch", "Add a capacity limit"
// (each expert keeps its first C assignments, tokens in order, slots in order
// inside a token; counts are taken before drops) and the sorted expert-major
// token list of "2.9 Mixture-of-Experts (MoE) Architectures", "MoE in
// Practice".  Rows are ordered by (expert, assignment index a = t*k + s).
//
// Tokens are cut into tiles of kRouteTile.  hist[e][b] counts tile b's
// assignments to expert e (written by the routing kernel, or by hist_kernel
// when the caller supplies the IDs).  column_scan_kernel (one block per
// expert) turns each column into per-tile running bases, the expert's count
// and its P_e sum; expert_scan_kernel clips the counts to the capacity, scans
// them into expert offsets and finishes the aux losses.  When the
// permutation is wanted, scatter_offsets_kernel does that scan in every block
// and then ranks each tile's assignments in order with wave ballots and
// writes both directions of the permutation.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void hist_kernel(int T, int E, int k, const int32_t* ids,
                                                   int32_t* hist) {
  __shared__ int h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
  __syncthreads();
  const int b = blockIdx.x;
  const int tile = route_tile(T);
  const int a0 = b * tile * k;
  const int a1 = min(T, (b + 1) * tile) * k;
  for (int a = a0 + threadIdx.x; a < a1; a += blockDim.x) {
    const int e = ids[a];
    if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);  // out-of-range IDs are ignored
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)e * gridDim.x + b] = h[e];
}

// Block-wide inclusive scan of one int per thread (256 threads); also
// returns the block total.  Fixed shape, so the result is deterministic.
__device__ __forceinline__ int block_scan_incl(int v, int* s_w, int& total) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) s_w[w] = v;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < w) before += s_w[i];
    total += s_w[i];
  }
  __syncthreads();
  return v + before;
}

__device__ __forceinline__ float block_sum(float v, float* s_w) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  if (lane_id() == 0) s_w[threadIdx.x >> 6] = v;
  __syncthreads();
  const float t = (s_w[0] + s_w[1]) + (s_w[2] + s_w[3]);
  __syncthreads();
  return t;
}

// Unmasked tokens: the sum of the per-block counts (fixed order), or T.
__device__ __forceinline__ int valid_tokens(const FinalizeParams& p, int* s_i) {
  if (!p.valid_part) return p.T;
  int n = 0;
  for (int b0 = 0; b0 < p.nblk; b0 += 256) {
    const int b = b0 + threadIdx.x;
    int tot;
    block_scan_incl(b < p.nblk ? p.valid_part[b] : 0, s_i, tot);
    n += tot;
  }
  return n;
}

// One block (256 threads) per expert: scan its column of tile counts.
__global__ __launch_bounds__(256) void column_scan_kernel(FinalizeParams p) {
  __shared__ int s_i[4];
  __shared__ float s_f[4];
  const int e = blockIdx.x;
  const int32_t* h = p.hist + (size_t)e * p.nblk;
  int run = 0;
  float ps = 0.f;
  for (int b0 = 0; b0 < p.nblk; b0 += 256) {
    const int b = b0 + threadIdx.x;
    const int v = b < p.nblk ? h[b] : 0;
    int tot;
    const int incl = block_scan_incl(v, s_i, tot);
    if (p.block_base && b < p.nblk) p.block_base[(size_t)e * p.nblk + b] = run + incl - v;
    run += tot;
    if (p.pe_part) ps += block_sum(b < p.nblk ? p.pe_part[(size_t)e * p.nblk + b] : 0.f, s_f);
  }
  const int nv = p.pe_part ? valid_tokens(p, s_i) : p.T;
  if (threadIdx.x == 0) {
    p.counts_ws[e] = run;
    if (p.counts) p.counts[e] = run;
    if (p.pe_part) {
      const float pe = nv > 0 ? ps / (float)nv : 0.f;
      p.pe_ws[e] = pe;
      if (p.mean_prob) p.mean_prob[e] = pe;
    }
  }
}

// Capacity clip, expert offsets, n_kept and the aux losses, by one block of
// 256 threads (expert_scan_kernel, and the first block of
// scatter_offsets_kernel).
__device__ __forceinline__ void expert_scan_block(const FinalizeParams& p, int* s_i, float* s_f) {
  int base = 0;
  float bal = 0.f;
  const int nv = p.aux ? valid_tokens(p, s_i) : p.T;
  const float inv = nv > 0 ? 1.0f / ((float)nv * (float)p.k) : 0.f;
  for (int e0 = 0; e0 < p.E; e0 += 256) {
    const int e = e0 + threadIdx.x;
    const int c = e < p.E ? p.counts_ws[e] : 0;
    const int kept = p.capacity > 0 ? min(c, p.capacity) : c;
    int tot;
    const int incl = block_scan_incl(kept, s_i, tot);
    if (p.expert_offsets && e < p.E) p.expert_offsets[e] = base + incl - kept;
    base += tot;
    if (p.aux) bal += block_sum(e < p.E ? ((float)c * inv) * p.pe_ws[e] : 0.f, s_f);
  }
  float z = 0.f;
  if (p.aux) {
    for (int b0 = 0; b0 < p.nblk; b0 += 256) {
      const int b = b0 + threadIdx.x;
      z += block_sum(b < p.nblk ? p.z_part[b] : 0.f, s_f);
    }
  }
  if (threadIdx.x == 0) {
    if (p.expert_offsets) p.expert_offsets[p.E] = base;
    if (p.n_kept) *p.n_kept = base;
    if (p.aux) {
      p.aux[0] = (float)p.E * bal;
      p.aux[1] = nv > 0 ? z / (float)nv : 0.f;
    }
  }
}

// One block: capacity clip, expert offsets, n_kept and the aux losses.
__global__ __launch_bounds__(256) void expert_scan_kernel(FinalizeParams p) {
  __shared__ int s_i[4];
  __shared__ float s_f[4];
  expert_scan_block(p, s_i, s_f);
}

// The expert scan and the scatter in one launch.  Every block scans the
// clipped per-expert counts into LDS itself (the same scan as
// expert_scan_block, so the offsets are the same) and the first block also
// writes the finalize outputs.  Then each of the four waves takes one token
// tile: its assignments are ranked 64 at a time in index order; lanes
// holding the same expert find each other with one ballot per bit of the
// expert ID, so a lane's rank is the number of lower lanes with its expert
// plus the running count of that expert in the wave's own LDS array (a
// wave's LDS accesses execute in order, so no barrier is needed between its
// reads of run[] and its leaders' updates).
constexpr int kScatterTiles = 4;
__global__ __launch_bounds__(256) void scatter_offsets_kernel(FinalizeParams fp, ScatterParams p) {
  __shared__ int s_i[4];
  __shared__ float s_f[4];
  __shared__ int off[kMaxExperts];
  __shared__ int run_all[kScatterTiles][kMaxExperts];
  if (blockIdx.x == 0) expert_scan_block(fp, s_i, s_f);
  {
    int base = 0;
    for (int e0 = 0; e0 < p.E; e0 += 256) {
      const int e = e0 + threadIdx.x;
      const int c = e < p.E ? fp.counts_ws[e] : 0;
      const int kept = p.capacity > 0 ? min(c, p.capacity) : c;
      int tot;
      const int incl = block_scan_incl(kept, s_i, tot);
      if (e < p.E) off[e] = base + incl - kept;
      base += tot;
    }
  }
  __syncthreads();  // off[] complete; no block barrier follows
  const int wv = threadIdx.x >> 6, lane = lane_id();
  const int nblk = (p.T + p.tile - 1) / p.tile;
  const int b = blockIdx.x * kScatterTiles + wv;
  if (b >= nblk) return;
  int* run = run_all[wv];
  for (int e = lane; e < p.E; e += 64) run[e] = p.block_base[(size_t)e * nblk + b];
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  int nbits = 1;
  while ((1 << nbits) < p.E) ++nbits;
  const int a0 = b * p.tile * p.k;
  const int a1 = min(p.T, (b + 1) * p.tile) * p.k;
  const uint64_t below = lanemask_lt();
  for (int c = a0; c < a1; c += 64) {
    const int a = c + lane;
    const int e_in = a < a1 ? p.ids[a] : -1;
    const bool in_range = (unsigned)e_in < (unsigned)p.E;
    const bool valid = a < a1 && in_range;
    const int e = valid ? e_in : 0;
    if (a < a1 && !in_range) p.assign_to_row[a] = -1;  // out-of-range IDs are dropped
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t bb = __ballot(set);
      peers &= set ? bb : ~bb;
    }
    const int rank = valid ? run[e] + __popcll(peers & below) : 0;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (valid && (peers & below) == 0) run[e] += __popcll(peers);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (valid) {
      const bool keep = p.capacity <= 0 || rank < p.capacity;
      if (keep) {
        const int row = off[e] + rank;
        p.assign_to_row[a] = row;
        p.row_to_assign[row] = a;
      } else {
        p.assign_to_row[a] = -1;
      }
    }
  }
}

// Small batches: column_scan_kernel and scatter_offsets_kernel in one
// workgroup of 16 waves (one launch instead of two).  Each expert's
// tile bases are kept in LDS; the sums of P_e, z and the valid tokens run
// sequentially in tile order and the balance sum in expert order, so the
// results are deterministic (they may differ from the multi-block kernels'
// tree order in the last bits of the float aux values only; counts,
// offsets and the permutation are identical).
constexpr int kSmallThreads = 1024, kSmallWaves = kSmallThreads / 64;
constexpr int kSmallBaseInts = 8192;  // nblk * E entries of the tile bases

__global__ __launch_bounds__(kSmallThreads) void permute_small_kernel(FinalizeParams p,
                                                                      ScatterParams sp) {
  __shared__ int base[kSmallBaseInts];
  __shared__ int offs[kMaxExperts + 1];
  __shared__ int cnt_lds[kMaxExperts];
  __shared__ float pe_lds[kMaxExperts];
  __shared__ int run[kSmallWaves][kMaxExperts];
  __shared__ float s_nv, s_z;
  const int tid = threadIdx.x, E = p.E, nblk = p.nblk;
  const int wave = tid >> 6, lane = tid & 63;
  // 1. thread e: expert e's tile bases, count and P_e sum, in tile order;
  // the last thread: valid tokens and the z sum.  Loads go 16 at a time so
  // that their latencies overlap.
  constexpr int U = 16;
  if (tid < E) {
    int total = 0;
    float ps = 0.f;
    for (int b0 = 0; b0 < nblk; b0 += U) {
      int v[U];
      float q[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool in = b0 + u < nblk;
        v[u] = in ? p.hist[(size_t)tid * nblk + b0 + u] : 0;
        q[u] = (in && p.pe_part) ? p.pe_part[(size_t)tid * nblk + b0 + u] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b0 + u >= nblk) break;
        base[tid * nblk + b0 + u] = total;
        total += v[u];
        ps += q[u];
      }
    }
    cnt_lds[tid] = total;
    pe_lds[tid] = ps;
  }
  if (tid == kSmallThreads - 1) {
    int nv = 0;
    float z = 0.f;
    for (int b0 = 0; b0 < nblk; b0 += U) {
      int v[U];
      float q[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool in = b0 + u < nblk;
        v[u] = (in && p.valid_part) ? p.valid_part[b0 + u] : 0;
        q[u] = (in && p.z_part) ? p.z_part[b0 + u] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b0 + u >= nblk) break;
        nv += v[u];
        z += q[u];
      }
    }
    s_nv = (float)(p.valid_part ? nv : p.T);
    s_z = z;
  }
  __syncthreads();
  const float nv = s_nv;
  if (tid < E) {
    const int cnt = cnt_lds[tid];
    p.counts_ws[tid] = cnt;
    if (p.counts) p.counts[tid] = cnt;
    if (p.pe_part) {
      const float pe = nv > 0.f ? pe_lds[tid] / nv : 0.f;
      pe_lds[tid] = pe;
      p.pe_ws[tid] = pe;
      if (p.mean_prob) p.mean_prob[tid] = pe;
    }
  }
  // 2. wave 0: capacity clip and the exclusive scan of the kept counts
  // (lane l holds experts 4l .. 4l+3), expert offsets, n_kept, aux losses
  if (tid < 64) {
    int v[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * tid + j;
      const int c = e < E ? cnt_lds[e] : 0;
      v[j] = p.capacity > 0 ? min(c, p.capacity) : c;
      sum += v[j];
    }
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (tid >= d) incl += o;
    }
    int at = incl - sum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * tid + j;
      if (e < E) offs[e] = at;
      at += v[j];
    }
    if (tid == 63) offs[E] = incl;
  }
  __syncthreads();
  if (p.expert_offsets && tid <= E) p.expert_offsets[tid] = offs[tid];
  if (p.n_kept && tid == 0) *p.n_kept = offs[E];
  if (p.aux && tid == 0) {
    const float inv = nv > 0.f ? 1.0f / (nv * (float)p.k) : 0.f;
    float bal = 0.f;
    for (int e = 0; e < E; ++e) bal += ((float)cnt_lds[e] * inv) * pe_lds[e];
    p.aux[0] = (float)E * bal;
    p.aux[1] = nv > 0.f ? s_z / nv : 0.f;
  }
  if (!sp.ids) return;
  // 3. scatter: wave w ranks the assignments of tiles w, w + 16, ... in
  // order (as scatter_offsets_kernel does, its running counts in LDS row w)
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t below = lanemask_lt();
  int* r = run[wave];
  for (int b = wave; b < nblk; b += kSmallWaves) {
    for (int e = lane; e < E; e += 64) r[e] = base[e * nblk + b];
    __builtin_amdgcn_wave_barrier();
    const int a0 = b * sp.tile * sp.k;
    const int a1 = min(sp.T, (b + 1) * sp.tile) * sp.k;
    for (int c = a0; c < a1; c += 64) {
      const int a = c + lane;
      const int e_in = a < a1 ? sp.ids[a] : -1;
      const bool in_range = (unsigned)e_in < (unsigned)E;
      const bool valid = a < a1 && in_range;
      const int e = valid ? e_in : 0;
      if (a < a1 && !in_range) sp.assign_to_row[a] = -1;  // out-of-range IDs are dropped
      uint64_t peers = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (e >> bit) & 1;
        const uint64_t bb = __ballot(set);
        peers &= set ? bb : ~bb;
      }
      const int rank = valid ? r[e] + __popcll(peers & below) : 0;
      __builtin_amdgcn_wave_barrier();  // all of the wave's reads of r[] precede the writes
      if (valid && (peers & below) == 0) r[e] += __popcll(peers);
      __builtin_amdgcn_wave_barrier();
      if (valid) {
        const bool keep = p.capacity <= 0 || rank < p.capacity;
        if (keep) {
          const int row = offs[e] + rank;
          sp.assign_to_row[a] = row;
          sp.row_to_assign[row] = a;
        } else {
          sp.assign_to_row[a] = -1;
        }
      }
    }
  }
}

// Auxiliary-loss-free balancer step ("DeepSeek-MoE and the fine-grained +
// shared-expert idea" and "Exercises" 6 on the book page; NeMo
// Gate.update_bias): bias[e] moves by +gamma when expert e is below the mean
// load and by -gamma when above; the comparison is exact on integers
// (E * counts[e] against the total).
__global__ __launch_bounds__(256) void update_bias_kernel(int E, const int32_t* counts,
                                                          float gamma, float* bias) {
  __shared__ int s_i[4];
  long long total = 0;
  for (int e0 = 0; e0 < E; e0 += 256) {
    const int e = e0 + threadIdx.x;
    int tot;
    block_scan_incl(e < E ? counts[e] : 0, s_i, tot);
    total += tot;
  }
  for (int e = threadIdx.x; e < E; e += 256) {
    const long long d = total - (long long)E * counts[e];
    const float step = d > 0 ? 1.f : (d < 0 ? -1.f : 0.f);
    bias[e] = bias[e] + gamma * step;
  }
}

}  // namespace

hipError_t launch_update_bias(int E, const int32_t* counts, float gamma, float* bias,
                              hipStream_t s) {
  hipLaunchKernelGGL(update_bias_kernel, dim3(1), dim3(256), 0, s, E, counts, gamma, bias);
  return hipGetLastError();
}

hipError_t launch_hist(int T, int E, int k, const int32_t* ids, int32_t* hist, hipStream_t s) {
  hipLaunchKernelGGL(hist_kernel, dim3(route_blocks(T)), dim3(256), 0, s, T, E, k, ids, hist);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(column_scan_kernel, dim3(p.E), dim3(256), 0, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(expert_scan_kernel, dim3(1), dim3(256), 0, s, p);
  return hipGetLastError();
}

bool permute_fits_one_block(int T, int E, int k) {
  return (long long)route_blocks(T) * E <= kSmallBaseInts && (long long)T * k <= 4096;
}

hipError_t launch_permute_small(const FinalizeParams& fp, const ScatterParams& sp,
                                hipStream_t s) {
  hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kSmallThreads), 0, s, fp, sp);
  return hipGetLastError();
}

hipError_t launch_finalize_scatter(const FinalizeParams& fp, const ScatterParams& sp,
                                   hipStream_t s) {
  hipLaunchKernelGGL(column_scan_kernel, dim3(fp.E), dim3(256), 0, s, fp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int nblk = route_blocks(sp.T);
  hipLaunchKernelGGL(scatter_offsets_kernel, dim3((nblk + kScatterTiles - 1) / kScatterTiles),
                     dim3(256), 0, s, fp, sp);
  return hipGetLastError();
}

}  // namespace moe
