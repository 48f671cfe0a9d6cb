// Combine: out[t] = sum over kept slots (slot order) of the weighted expert
// rows, plus the shared-expert row (optionally scaled by its per-token gate),
// plus the residual stream when given; fp32 accumulation, one rounding.
//
// This is the index_add_ step of "Lab: build a tiny MoE in PyTorch" ("Full
// implementation") written as a gather: each output row is owned by one
// thread group, so there are no atomics and the sum order is fixed.  The
// shared expert joins as in "Add a shared expert" on the same page.
// HBM-bound: each thread moves 16-byte chunks along d_model.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int NTHREADS = 256;

template <typename T>
struct Vec16;  // 16 bytes of T
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
};

template <typename T>
__device__ __forceinline__ void unpack16(const uint4 q, float (&v)[Vec16<T>::N]) {
  if constexpr (Vec16<T>::N == 8) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    v[0] = __uint_as_float(q.x);
    v[1] = __uint_as_float(q.y);
    v[2] = __uint_as_float(q.z);
    v[3] = __uint_as_float(q.w);
  }
}

template <typename T>
__device__ __forceinline__ void load16(const T* p, float (&v)[Vec16<T>::N]) {
  unpack16<T>(*reinterpret_cast<const uint4*>(p), v);
}

template <typename T>
__device__ __forceinline__ void store16(T* p, const float (&v)[Vec16<T>::N]) {
  uint4 q;
  if constexpr (Vec16<T>::N == 8) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16_bits(v[2 * i]) | ((uint32_t)f32_to_bf16_bits(v[2 * i + 1]) << 16);
    q = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    q = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                   __float_as_uint(v[3]));
  }
  *reinterpret_cast<uint4*>(p) = q;
}

// Block = TPB tokens x (NTHREADS / TPB) threads per token.  With a shared
// expert gate, the token's threads first form x[t] . g in fp32 (each thread
// over its chunks, then the token's partials added in thread order), and
// the shared row is scaled by sigmoid of it.
template <typename T>
__global__ __launch_bounds__(NTHREADS) void combine_kernel(CombineParams p, int tpb) {
  constexpr int N = Vec16<T>::N;
  const T* y = static_cast<const T*>(p.y_rows);
  const T* sh = static_cast<const T*>(p.shared_rows);
  const T* res = static_cast<const T*>(p.residual);
  T* out = static_cast<T*>(p.out);
  __shared__ int rows_lds[64 * kMaxTopK];
  __shared__ float red[NTHREADS];
  __shared__ float gate_lds[64];
  const int per_tok = NTHREADS / tpb;
  const int tl = threadIdx.x / per_tok;
  const int t = blockIdx.x * tpb + tl;
  const int sub = threadIdx.x % per_tok;
  const int nchunk = p.D / N;
  for (int i = threadIdx.x; i < tpb * p.k; i += NTHREADS) {
    const int tt = blockIdx.x * tpb + i / p.k;
    rows_lds[i] = tt < p.T ? p.assign_to_row[(size_t)blockIdx.x * tpb * p.k + i] : -1;
  }
  const bool gated = sh && p.shared_gate;  // uniform
  if (gated) {
    const T* xr = static_cast<const T*>(p.x) + (size_t)min(t, p.T - 1) * p.D;
    const T* g = static_cast<const T*>(p.shared_gate);
    float dot = 0.f;
    for (int c = sub; c < nchunk; c += per_tok) {
      float a[N], b[N];
      load16<T>(xr + (size_t)c * N, a);
      load16<T>(g + (size_t)c * N, b);
#pragma unroll
      for (int i = 0; i < N; ++i) dot += a[i] * b[i];
    }
    red[threadIdx.x] = dot;
    __syncthreads();
    if (sub == 0) {
      float s = red[tl * per_tok];
      for (int i = 1; i < per_tok; ++i) s += red[tl * per_tok + i];
      gate_lds[tl] = 1.0f / (1.0f + expf(-s));
    }
  }
  __syncthreads();
  if (t >= p.T) return;
  const float gs = gated ? gate_lds[tl] : 1.f;
  const int* rows = rows_lds + tl * p.k;
  for (int c = sub; c < nchunk; c += per_tok) {
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.f;
    for (int s = 0; s < p.k; ++s) {
      if (rows[s] < 0) continue;
      float v[N];
      load16<T>(y + (size_t)rows[s] * p.D + (size_t)c * N, v);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += v[i];
    }
    if (sh) {
      float v[N];
      load16<T>(sh + (size_t)t * p.D + (size_t)c * N, v);
      if (gated) {
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] += gs * v[i];
      } else {
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] += v[i];
      }
    }
    if (res) {  // the residual stream joins last, before the one rounding
      float v[N];
      load16<T>(res + (size_t)t * p.D + (size_t)c * N, v);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[i] += v[i];
    }
    store16<T>(out + (size_t)t * p.D + (size_t)c * N, acc);
  }
}

// Without the shared-expert gate every 16-byte chunk of an output row is
// independent.  A row's chunks are cut into CPT segments; thread i of a row
// takes chunk i of every segment (consecutive threads on consecutive chunks,
// so each load instruction covers contiguous bytes).  A thread issues the
// loads of up to eight slots' rows (and the shared and residual rows) for
// all its chunks before it adds them in slot order, so the loads of a token
// overlap instead of following one another; the sum order is that of
// combine_kernel, so the bits agree.
template <typename T, int CPT>
__global__ __launch_bounds__(NTHREADS) void combine_rows_kernel(CombineParams p) {
  constexpr int N = Vec16<T>::N;
  constexpr int G = 8 / CPT;  // slots loaded together
  const int nseg = p.D / N / CPT;
  const long long gid = (long long)blockIdx.x * NTHREADS + threadIdx.x;
  if (gid >= (long long)p.T * nseg) return;
  const int t = (int)(gid / nseg), c = (int)(gid % nseg);
  const T* y = static_cast<const T*>(p.y_rows) + (size_t)c * N;
  const int32_t* a2r = p.assign_to_row + (size_t)t * p.k;
  const size_t at = (size_t)t * p.D + (size_t)c * N;
  const size_t seg = (size_t)nseg * N;  // elements between a thread's chunks
  uint4 qs[CPT], qr[CPT];
#pragma unroll
  for (int h = 0; h < CPT; ++h) {
    qs[h] = qr[h] = make_uint4(0u, 0u, 0u, 0u);
    if (p.shared_rows)
      qs[h] = *reinterpret_cast<const uint4*>(static_cast<const T*>(p.shared_rows) + at + h * seg);
    if (p.residual)
      qr[h] = *reinterpret_cast<const uint4*>(static_cast<const T*>(p.residual) + at + h * seg);
  }
  float acc[CPT][N];
#pragma unroll
  for (int h = 0; h < CPT; ++h)
#pragma unroll
    for (int i = 0; i < N; ++i) acc[h][i] = 0.f;
  for (int s0 = 0; s0 < p.k; s0 += G) {
    int row[G];
    uint4 q[G][CPT];
#pragma unroll
    for (int u = 0; u < G; ++u) row[u] = s0 + u < p.k ? a2r[s0 + u] : -1;
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (row[u] >= 0)
#pragma unroll
        for (int h = 0; h < CPT; ++h)
          q[u][h] = *reinterpret_cast<const uint4*>(y + (size_t)row[u] * p.D + h * seg);
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (row[u] < 0) continue;
#pragma unroll
      for (int h = 0; h < CPT; ++h) {
        float v[N];
        unpack16<T>(q[u][h], v);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[h][i] += v[i];
      }
    }
  }
#pragma unroll
  for (int h = 0; h < CPT; ++h) {
    float v[N];
    if (p.shared_rows) {
      unpack16<T>(qs[h], v);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[h][i] += v[i];
    }
    if (p.residual) {  // the residual stream joins last, before the one rounding
      unpack16<T>(qr[h], v);
#pragma unroll
      for (int i = 0; i < N; ++i) acc[h][i] += v[i];
    }
    store16<T>(static_cast<T*>(p.out) + at + h * seg, acc[h]);
  }
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, bool bf16, hipStream_t s) {
  const int n = bf16 ? 8 : 4;
  const int nchunk = p.D / n;
  if (!(p.shared_rows && p.shared_gate)) {
    // Chunks per thread: four once there are at least 256K chunks (the
    // capacity-limited Switch-shaped combine 6.95 -> 5.77 us, Mixtral-shaped
    // 20.2 -> 18.5 us), one for small batches, which need the threads (the
    // decode-shaped combine 4.3 us with one, 6.2 with four).
    int cpt = (long long)p.T * nchunk >= (1 << 18) ? 4 : 1;
    while (cpt > 1 && nchunk % cpt) cpt >>= 1;
    const long long threads = (long long)p.T * (nchunk / cpt);
    const dim3 grid((unsigned)((threads + NTHREADS - 1) / NTHREADS)), block(NTHREADS);
#define MOE_COMBINE_LAUNCH(C)                                                              \
  do {                                                                                     \
    if (bf16)                                                                              \
      hipLaunchKernelGGL((combine_rows_kernel<uint16_t, C>), grid, block, 0, s, p);        \
    else                                                                                   \
      hipLaunchKernelGGL((combine_rows_kernel<float, C>), grid, block, 0, s, p);           \
  } while (0)
    if (cpt >= 4)
      MOE_COMBINE_LAUNCH(4);
    else if (cpt == 2)
      MOE_COMBINE_LAUNCH(2);
    else
      MOE_COMBINE_LAUNCH(1);
#undef MOE_COMBINE_LAUNCH
    return hipGetLastError();
  }
  int tpb = 1;  // tokens per block: keep at least ~nchunk threads per token
  while (tpb < 64 && NTHREADS / (tpb * 2) >= nchunk) tpb *= 2;
  const dim3 grid((p.T + tpb - 1) / tpb), block(NTHREADS);
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<uint16_t>, grid, block, 0, s, p, tpb);
  else
    hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, s, p, tpb);
  return hipGetLastError();
}

}  // namespace moe
