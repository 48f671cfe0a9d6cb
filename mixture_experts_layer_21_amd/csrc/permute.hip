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
// them into expert offsets and finishes the aux losses.  scatter_kernel ranks
// each tile's assignments in order with wave ballots and writes both
// directions of the permutation.
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
  const int a0 = b * kRouteTile * k;
  const int a1 = min(T, (b + 1) * kRouteTile) * k;
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

// One block: capacity clip, expert offsets, n_kept and the aux losses.
__global__ __launch_bounds__(256) void expert_scan_kernel(FinalizeParams p) {
  __shared__ int s_i[4];
  __shared__ float s_f[4];
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

// One wave per token tile.  Assignments are taken 64 at a time in index
// order; lanes holding the same expert find each other with one ballot per
// bit of the expert ID, so a lane's rank is the number of lower lanes with
// its expert plus the running count of that expert in LDS.
__global__ __launch_bounds__(64) void scatter_kernel(ScatterParams p) {
  __shared__ int run[kMaxExperts];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < p.E; e += 64) run[e] = p.block_base[(size_t)e * gridDim.x + b];
  __syncthreads();
  int nbits = 1;
  while ((1 << nbits) < p.E) ++nbits;
  const int a0 = b * kRouteTile * p.k;
  const int a1 = min(p.T, (b + 1) * kRouteTile) * p.k;
  const uint64_t below = lanemask_lt();
  for (int c = a0; c < a1; c += 64) {
    const int a = c + (int)threadIdx.x;
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
    __syncthreads();  // every lane has read run[] before the leaders advance it
    if (valid && (peers & below) == 0) run[e] += __popcll(peers);
    __syncthreads();
    if (valid) {
      const bool keep = p.capacity <= 0 || rank < p.capacity;
      if (keep) {
        const int row = p.expert_offsets[e] + rank;
        p.assign_to_row[a] = row;
        p.row_to_assign[row] = a;
      } else {
        p.assign_to_row[a] = -1;
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

hipError_t launch_scatter(const ScatterParams& p, hipStream_t s) {
  hipLaunchKernelGGL(scatter_kernel, dim3(route_blocks(p.T)), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
