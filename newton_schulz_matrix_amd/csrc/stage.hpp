// stage.hpp - HBM-bound passes before the products: the Frobenius norm and
// the fused scale / cast / orient-to-wide / zero-pad pass.
//
// The iteration wants X with no more rows than columns (the Gram-NS
// article's X in R^{n x m}, aspect alpha = m/n) and unit Frobenius norm.
// Both passes read the caller's matrix in place (row-major, leading
// dimension ld, batch stride bstride) and never write it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "products.hpp"

namespace nsk {

constexpr int kStageThreads = 256;

// Deterministic block sum of one double per thread (fixed order).
__device__ __forceinline__ double block_sum(double v, double* sh) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_down(v, off, 64);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) sh[w] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) {
    for (int i = 0; i < kStageThreads / 64; ++i) t += sh[i];
    sh[0] = t;
  }
  __syncthreads();
  t = sh[0];
  __syncthreads();
  return t;
}

// partial[b * P + blockIdx.x] = sum of squares over rows blockIdx.x,
// blockIdx.x + P, ... of matrix b (accumulated in fp64).  The vector path
// keeps four independent 16-byte loads in flight per thread.
template <typename IO>
__global__ void __launch_bounds__(kStageThreads) k_sumsq(const IO* M, int64_t rows, int64_t cols, int64_t ld,
                                                        int64_t bstride, int vec_ok, double* partial, int P) {
  __shared__ double sh[kStageThreads / 64];
  const IO* A = M + (int64_t)blockIdx.y * bstride;
  double s0 = 0.0, s1 = 0.0;
  constexpr int V = 16 / sizeof(IO);
  if (vec_ok) {
    const int64_t cv = cols / V;
    for (int64_t r = blockIdx.x; r < rows; r += P) {
      const uint4* row = reinterpret_cast<const uint4*>(A + r * ld);
      int64_t c = threadIdx.x;
      for (; c + 3 * kStageThreads < cv; c += 4 * kStageThreads) {
        uint4 q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) q[u] = row[c + u * kStageThreads];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const IO* e = reinterpret_cast<const IO*>(&q[u]);
          float f = 0.f;
#pragma unroll
          for (int k = 0; k < V; ++k) {
            const float x = to_f32<IO>(e[k]);
            f = fmaf(x, x, f);
          }
          if (u & 1) s1 += (double)f; else s0 += (double)f;
        }
      }
      for (; c < cv; c += kStageThreads) {
        const uint4 q = row[c];
        const IO* e = reinterpret_cast<const IO*>(&q);
#pragma unroll
        for (int k = 0; k < V; ++k) {
          const double x = (double)to_f32<IO>(e[k]);
          s0 += x * x;
        }
      }
    }
  } else {
    for (int64_t r = blockIdx.x; r < rows; r += P) {
      const IO* row = A + r * ld;
      for (int64_t c = threadIdx.x; c < cols; c += kStageThreads) {
        const double x = (double)to_f32<IO>(row[c]);
        s0 += x * x;
      }
    }
  }
  const double t = block_sum(s0 + s1, sh);
  if (threadIdx.x == 0) partial[(int64_t)blockIdx.y * P + blockIdx.x] = t;
}

// scale[b] = prescale / (sqrt(sum of the P partials of matrix b) + eps),
// summed in a fixed order.  One block per matrix.
__global__ void __launch_bounds__(kStageThreads) k_scale(const double* partial, int P, float prescale, float eps,
                                                        float* scale) {
  __shared__ double sh[kStageThreads / 64];
  const double* pp = partial + (int64_t)blockIdx.x * P;
  double v = 0.0;
  for (int i = threadIdx.x; i < P; i += kStageThreads) v += pp[i];
  v = block_sum(v, sh);
  if (threadIdx.x == 0) scale[blockIdx.x] = (float)((double)prescale / (sqrt(v) + (double)eps));
}

// Wide orientation, no transpose: X[i][j] = scale * M[i][j] for i < rows,
// j < cols, zero elsewhere in the n_pad x m_pad buffer.  One block per
// output row; each thread writes 16-byte groups.
template <typename IO, typename T>
__global__ void __launch_bounds__(kStageThreads) k_stage_rows(const IO* M, int64_t rows, int64_t cols, int64_t ld,
                                                             int64_t bstride, const float* scales, T* X,
                                                             int64_t m_pad, int64_t xstride) {
  const int b = blockIdx.y;
  const float scale = scales[b];
  const int64_t i = blockIdx.x;
  const IO* src = M + (int64_t)b * bstride + i * ld;
  T* dst = X + (int64_t)b * xstride + i * m_pad;
  constexpr int V = 16 / sizeof(T);
  for (int64_t c0 = (int64_t)threadIdx.x * V; c0 < m_pad; c0 += (int64_t)kStageThreads * V) {
    T out[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
      const int64_t c = c0 + k;
      const float x = (i < rows && c < cols) ? to_f32<IO>(src[c]) : 0.f;
      out[k] = from_f32<T>(x * scale);
    }
    *reinterpret_cast<uint4*>(dst + c0) = *reinterpret_cast<const uint4*>(out);
  }
}

// Tall input: X[i][j] = scale * M[j][i] (i < cols, j < rows), via a 64 x 64
// LDS tile so both the read of M and the write of X are coalesced.
template <typename IO, typename T>
__global__ void __launch_bounds__(kStageThreads) k_stage_transpose(const IO* M, int64_t rows, int64_t cols, int64_t ld,
                                                                  int64_t bstride, const float* scales, T* X,
                                                                  int64_t m_pad, int64_t xstride, int tiles_j) {
  __shared__ float tile[64][65];
  const int b = blockIdx.y;
  const float scale = scales[b];
  const int64_t i0 = (int64_t)(blockIdx.x / tiles_j) * 64;  // X rows  = M cols
  const int64_t j0 = (int64_t)(blockIdx.x % tiles_j) * 64;  // X cols  = M rows
  const IO* src = M + (int64_t)b * bstride;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int64_t mr = j0 + r, mc = i0 + tx;
    tile[r][tx] = (mr < rows && mc < cols) ? to_f32<IO>(src[mr * ld + mc]) : 0.f;
  }
  __syncthreads();
  T* dst = X + (int64_t)b * xstride;
  for (int r = ty; r < 64; r += 4) {
    dst[(i0 + r) * m_pad + j0 + tx] = from_f32<T>(tile[tx][r] * scale);
  }
}

// Fill n x n (ld) blocks of a batch with zero (used to clear buffers
// without memset nodes, so that the sequence can be captured in a graph).
template <typename T>
__global__ void k_fill_zero(T* p, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = T(0);
}

}  // namespace nsk
