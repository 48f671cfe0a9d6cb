// RMSNorm of the residual stream ahead of the MoE branch:
//   y[t, d] = x[t, d] / sqrt(mean_d' x[t, d']^2 + eps) * w[d]
// The decoder block of "Lab: build a tiny MoE in PyTorch" ("Put the MoE into
// a decoder block") normalises the stream before the layer and adds the
// layer's output back to it; st-moe-pytorch ("rms-norm") puts the same norm
// ahead of the MoE inside SparseMoEBlock.
//
// One wave per token row, 16-byte chunks along d_model; HBM-bound (one read
// of x, one write).  The mean square and the formula run in fp64 and each
// output is rounded once from fp64 to the activation dtype, so the rows are
// the correctly rounded values of the formula up to fp64 rounding.  The wave sum is a fixed butterfly, so
// every lane holds the same bits and repeated calls agree bit for bit.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int NTHREADS = 256;
constexpr int ROWS_PER_BLOCK = NTHREADS / 64;

// Nearest bf16 of a finite fp64 value (ties to even), taken on the fp64 bit
// pattern: the low 45 of its 52 fraction bits go, leaving bf16's 8
// significant bits; the rounded value then converts to fp32 exactly (bf16
// has fp32's exponent range), and its upper half is the bf16.  Values below
// fp32's normal range are outside this kernel's use.
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double v) {
  uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
  b += ((1ull << 44) - 1) + ((b >> 45) & 1ull);
  b &= ~((1ull << 45) - 1);
  const float f = static_cast<float>(__longlong_as_double(static_cast<long long>(b)));
  return static_cast<uint16_t>(__float_as_uint(f) >> 16);
}

template <bool BF16>
struct Chunk {
  static constexpr int N = BF16 ? 8 : 4;  // elements per 16 bytes
  static __device__ __forceinline__ void unpack(const uint4& q, double (&v)[N]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = static_cast<double>(__uint_as_float(w[i] << 16));
        v[2 * i + 1] = static_cast<double>(__uint_as_float(w[i] & 0xffff0000u));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = static_cast<double>(__uint_as_float(w[i]));
    }
  }
  static __device__ __forceinline__ uint4 pack(const double (&v)[N]) {
    uint32_t w[4];
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = static_cast<uint32_t>(f64_to_bf16_bits(v[2 * i])) |
               (static_cast<uint32_t>(f64_to_bf16_bits(v[2 * i + 1])) << 16);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(static_cast<float>(v[i]));
    }
    return uint4{w[0], w[1], w[2], w[3]};
  }
};

// Rows of up to 64 * CPL chunks stay in registers between the two passes
// (one read from memory); longer rows are read again from cache.
constexpr int CPL = 16;

template <bool BF16>
__global__ __launch_bounds__(NTHREADS) void rmsnorm_kernel(int T, int D, const void* x,
                                                           const float* w, double eps,
                                                           void* y) {
  using C = Chunk<BF16>;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  const int nch = D / C::N;
  const size_t row_bytes = (size_t)D * (BF16 ? 2 : 4);
  const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(x) + t * row_bytes);
  uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(y) + t * row_bytes);
  const bool cached = nch <= 64 * CPL;

  uint4 q[CPL];
  double ss = 0.0;
  if (cached) {
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      if (lane + 64 * i < nch) q[i] = src[lane + 64 * i];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      if (lane + 64 * i < nch) {
        double v[C::N];
        C::unpack(q[i], v);
#pragma unroll
        for (int e = 0; e < C::N; ++e) ss = fma(v[e], v[e], ss);
      }
    }
  } else {
    for (int c = lane; c < nch; c += 64) {
      double v[C::N];
      C::unpack(src[c], v);
#pragma unroll
      for (int e = 0; e < C::N; ++e) ss = fma(v[e], v[e], ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  // One reciprocal per row: x * (1/s) differs from x / s by at most an fp64
  // rounding, far below the output's rounding.
  const double inv = 1.0 / sqrt(ss / (double)D + eps);

  // Each lane rewrites only the chunks it has read, so y may alias x.
  auto emit = [&](int c, const uint4& qq) {
    double v[C::N];
    C::unpack(qq, v);
#pragma unroll
    for (int e = 0; e < C::N; ++e) v[e] = v[e] * inv;
    if (w) {  // the chunk's weights in 16-byte loads (w is 16-byte aligned)
      const f32x4* w4 = reinterpret_cast<const f32x4*>(w) + c * (C::N / 4);
#pragma unroll
      for (int q4 = 0; q4 < C::N / 4; ++q4) {
        const f32x4 wv = w4[q4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * q4 + e] *= static_cast<double>(wv[e]);
      }
    }
    dst[c] = C::pack(v);
  };
  if (cached) {
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      if (lane + 64 * i < nch) emit(lane + 64 * i, q[i]);
  } else {
    for (int c = lane; c < nch; c += 64) emit(c, src[c]);
  }
}

// Backward of the norm, one wave per row: with g = w * dy,
//   dx = g / s - x * sum_d(g x) / (D s^3)
// (s as in the forward, fp64), rounded once to the activation dtype; 1/s of
// every row goes to inv_s for the weight gradient.
template <bool BF16>
__global__ __launch_bounds__(NTHREADS) void rmsnorm_bwd_kernel(int T, int D, const void* x,
                                                               const float* w, double eps,
                                                               const float* dy, void* dx,
                                                               float* inv_s) {
  using C = Chunk<BF16>;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  const int nch = D / C::N;
  const size_t row_bytes = (size_t)D * (BF16 ? 2 : 4);
  const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(x) + t * row_bytes);
  const float* dyr = dy + (size_t)t * D;
  double ss = 0.0, gx = 0.0;
  for (int c = lane; c < nch; c += 64) {
    double v[C::N];
    C::unpack(src[c], v);
#pragma unroll
    for (int e = 0; e < C::N; ++e) {
      const double g = (double)dyr[c * C::N + e] * (w ? (double)w[c * C::N + e] : 1.0);
      ss = fma(v[e], v[e], ss);
      gx = fma(g, v[e], gx);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ss += __shfl_xor(ss, off);
    gx += __shfl_xor(gx, off);
  }
  const double s = sqrt(ss / (double)D + eps);
  const double inv = 1.0 / s, k = gx / ((double)D * s * s * s);
  if (lane == 0 && inv_s) inv_s[t] = (float)inv;
  uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(dx) + t * row_bytes);
  for (int c = lane; c < nch; c += 64) {
    double v[C::N];
    C::unpack(src[c], v);
#pragma unroll
    for (int e = 0; e < C::N; ++e) {
      const double g = (double)dyr[c * C::N + e] * (w ? (double)w[c * C::N + e] : 1.0);
      v[e] = g * inv - v[e] * k;
    }
    dst[c] = C::pack(v);
  }
}

// Weight gradient of the norm, sum_t dy_td x_td / s_t: each block sums a chunk
// of rows (256, more past 2^24 rows to keep the grid's y extent within 65535)
// for 256 columns in row order; a second pass adds the chunks in order.
constexpr int kNormRowsPerChunk = 256;
constexpr int kMaxChunks = 65535;

int rows_per_chunk(int T) {
  const int per = (T + kMaxChunks - 1) / kMaxChunks;
  return per > kNormRowsPerChunk ? per : kNormRowsPerChunk;
}

template <bool BF16>
__global__ __launch_bounds__(256) void rmsnorm_dw_part_kernel(int T, int D, const void* x,
                                                              const float* dy,
                                                              const float* inv_s, int per,
                                                              float* part) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  if (d >= D) return;
  const long long t0 = (long long)blockIdx.y * per;
  const long long t1 = min((long long)T, t0 + per);
  float acc = 0.f;
  for (long long t = t0; t < t1; ++t) {
    const float xv = BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(x)[(size_t)t * D + d])
                          : static_cast<const float*>(x)[(size_t)t * D + d];
    acc += dy[(size_t)t * D + d] * xv * inv_s[t];
  }
  part[(size_t)blockIdx.y * D + d] = acc;
}

__global__ __launch_bounds__(256) void rmsnorm_dw_final_kernel(int D, int nchunk,
                                                               const float* part, float* dw) {
  const int d = blockIdx.x * 256 + threadIdx.x;
  if (d >= D) return;
  float acc = part[d];
  for (int c = 1; c < nchunk; ++c) acc += part[(size_t)c * D + d];
  dw[d] = acc;
}

}  // namespace

int rmsnorm_dw_chunks(int T) { return (T + rows_per_chunk(T) - 1) / rows_per_chunk(T); }

hipError_t launch_rmsnorm_bwd(int T, int D, bool bf16, const void* x, const float* w, float eps,
                              const float* dy, void* dx, float* inv_s, float* dw_part,
                              float* dw, hipStream_t s) {
  const int blocks = (T + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  if (bf16)
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<true>, dim3(blocks), dim3(NTHREADS), 0, s, T, D, x, w,
                       (double)eps, dy, dx, inv_s);
  else
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<false>, dim3(blocks), dim3(NTHREADS), 0, s, T, D, x, w,
                       (double)eps, dy, dx, inv_s);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !dw) return err;
  const dim3 grid((D + 255) / 256, rmsnorm_dw_chunks(T));
  if (bf16)
    hipLaunchKernelGGL(rmsnorm_dw_part_kernel<true>, grid, dim3(256), 0, s, T, D, x, dy, inv_s,
                       rows_per_chunk(T), dw_part);
  else
    hipLaunchKernelGGL(rmsnorm_dw_part_kernel<false>, grid, dim3(256), 0, s, T, D, x, dy, inv_s,
                       rows_per_chunk(T), dw_part);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(rmsnorm_dw_final_kernel, dim3((D + 255) / 256), dim3(256), 0, s, D,
                     rmsnorm_dw_chunks(T), dw_part, dw);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int T, int D, bool bf16, const void* x, const float* w, float eps,
                          void* y, hipStream_t s) {
  const int blocks = (T + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  if (bf16)
    hipLaunchKernelGGL(rmsnorm_kernel<true>, dim3(blocks), dim3(NTHREADS), 0, s, T, D, x, w,
                       (double)eps, y);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<false>, dim3(blocks), dim3(NTHREADS), 0, s, T, D, x, w,
                       (double)eps, y);
  return hipGetLastError();
}

}  // namespace moe
