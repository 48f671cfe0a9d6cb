// Expert histogram, scan and stable scatter: the dispatch bookkeeping of the
// layer, integer-only and bit-exact.
//
// Semantics follow "Lab: build a tiny MoE in PyTorch", "Add a capacity limit"
// (each expert keeps its first C assignments, tokens in order, slots in order
// inside a token; counts are taken before drops) and the sorted expert-major
// token list of "2.9 Mixture-of-Experts (MoE) Architectures", "MoE in
// Practice".  Rows are ordered by (expert, assignment index a = t*k + s).
//
// Tokens are cut into tiles of kRouteTile.  hist[b][e] counts tile b's
// assignments to expert e (written by the routing kernel, or by hist_kernel
// when the caller supplies the IDs).  finalize_kernel turns the histograms
// into per-tile running bases, capacity-clipped expert offsets and the aux
// losses.  scatter_kernel ranks each tile's assignments in order with wave
// ballots and writes both directions of the permutation.
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
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)b * E + e] = h[e];
}

// One block.  Thread e walks the tiles in order for expert e; thread 0 then
// scans the experts.  Every sum has a fixed order.
__global__ __launch_bounds__(256) void finalize_kernel(FinalizeParams p) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int kept[kMaxExperts];
  __shared__ float pe[kMaxExperts];
  for (int e = threadIdx.x; e < p.E; e += blockDim.x) {
    int run = 0;
    float ps = 0.f;
    for (int b = 0; b < p.nblk; ++b) {
      const size_t i = (size_t)b * p.E + e;
      if (p.block_base) p.block_base[i] = run;
      run += p.hist[i];
      if (p.pe_part) ps += p.pe_part[i];
    }
    cnt[e] = run;
    kept[e] = p.capacity > 0 ? min(run, p.capacity) : run;
    pe[e] = ps / (float)p.T;
    if (p.counts) p.counts[e] = run;
    if (p.mean_prob) p.mean_prob[e] = pe[e];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (p.expert_offsets) {
      int off = 0;
      for (int e = 0; e < p.E; ++e) {
        p.expert_offsets[e] = off;
        off += kept[e];
      }
      p.expert_offsets[p.E] = off;
      if (p.n_kept) *p.n_kept = off;
    }
    if (p.aux) {
      const float inv = 1.0f / ((float)p.T * (float)p.k);
      float bal = 0.f;
      for (int e = 0; e < p.E; ++e) bal += ((float)cnt[e] * inv) * pe[e];
      float z = 0.f;
      for (int b = 0; b < p.nblk; ++b) z += p.z_part[b];
      p.aux[0] = (float)p.E * bal;
      p.aux[1] = z / (float)p.T;
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
  for (int e = threadIdx.x; e < p.E; e += 64) run[e] = p.block_base[(size_t)b * p.E + e];
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

}  // namespace

hipError_t launch_hist(int T, int E, int k, const int32_t* ids, int32_t* hist, hipStream_t s) {
  hipLaunchKernelGGL(hist_kernel, dim3(route_blocks(T)), dim3(256), 0, s, T, E, k, ids, hist);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_scatter(const ScatterParams& p, hipStream_t s) {
  hipLaunchKernelGGL(scatter_kernel, dim3(route_blocks(p.T)), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
