// stage.hpp - the small kernels around the products: the Frobenius norm
// and the fused scale / cast / orient-to-wide / zero-pad pass (both
// HBM-bound), the non-finite scan of a result (status word), the guarded
// Gram iteration's flag kernels and restart detector, and the Muon step's
// momentum pass.
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
// A grouped call's member b (members not null) replaces the batch layout: it
// starts at members[b].data with leading dimension members[b].ld and holds
// the rows x cols matrix transposed when members[b].transposed; 16-byte
// loads where its rows allow them.
template <typename IO>
__device__ __forceinline__ void member_layout(const ns_matrix* members, int b, const IO*& A, int64_t& rows,
                                              int64_t& cols, int64_t& ld, int& vec_ok, int& transposed) {
  const ns_matrix mb = members[b];
  A = reinterpret_cast<const IO*>(mb.data);
  ld = mb.ld;
  transposed = mb.transposed;
  if (transposed) {
    const int64_t t = rows;
    rows = cols;
    cols = t;
  }
  constexpr int V = 16 / sizeof(IO);
  vec_ok = cols % V == 0 && ld % V == 0 && (reinterpret_cast<uintptr_t>(A) & 15) == 0;
}

template <typename IO>
__global__ void __launch_bounds__(kStageThreads) k_sumsq(const IO* M, int64_t rows, int64_t cols, int64_t ld,
                                                        int64_t bstride, int vec_ok, double* partial, int P,
                                                        const ns_matrix* members) {
  __shared__ double sh[kStageThreads / 64];
  const IO* A = M + (int64_t)blockIdx.y * bstride;
  if (members) {
    int transposed;
    member_layout(members, blockIdx.y, A, rows, cols, ld, vec_ok, transposed);
  }
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
// summed in a fixed order.  One block per matrix.  A non-finite sum (NaN or
// Inf in the input) ORs status_bits into the optional status word.
static __global__ void __launch_bounds__(kStageThreads) k_scale(const double* partial, int P, float prescale, float eps,
                                                        float* scale, int32_t* d_status, int32_t status_bits) {
  __shared__ double sh[kStageThreads / 64];
  const double* pp = partial + (int64_t)blockIdx.x * P;
  double v = 0.0;
  for (int i = threadIdx.x; i < P; i += kStageThreads) v += pp[i];
  v = block_sum(v, sh);
  if (threadIdx.x == 0) {
    scale[blockIdx.x] = (float)((double)prescale / (sqrt(v) + (double)eps));
    if (d_status && !(v < __builtin_huge_val())) atomicOr(d_status, status_bits);
  }
}

// Both layouts of the scaled, oriented, zero-padded matrix: X (n_pad x
// m_pad, row-major) and X^T (m_pad x n_pad, row-major), one 64 x 64 block of
// X per work-group.  The block of the caller's matrix that holds it (the X
// block itself for a wide input, the X^T block for a tall one) is read with
// 8-element row chunks into LDS; the same-orientation output is written from
// rows of the LDS block and the other one from its columns, 16 bytes per
// thread.  Elements outside the caller's matrix are zero.
template <typename IO, typename T>
__global__ void __launch_bounds__(kStageThreads) k_stage_pair(const IO* M, int64_t rows, int64_t cols, int64_t ld,
                                                             int64_t bstride, int vec_ok, const float* scales, T* X,
                                                             T* XT, int64_t n_pad, int64_t m_pad, int64_t xstride,
                                                             int transposed, int blocks_j,
                                                             const ns_matrix* members) {
  constexpr int kB = 64, kV = 8;
  __shared__ float tile[kB][kB + 1];
  const int b = blockIdx.y;
  const float scale = scales[b];
  const IO* src = M + (int64_t)b * bstride;
  if (members) member_layout(members, b, src, rows, cols, ld, vec_ok, transposed);
  const int64_t i0 = (int64_t)(blockIdx.x / blocks_j) * kB;  // X rows
  const int64_t j0 = (int64_t)(blockIdx.x % blocks_j) * kB;  // X columns
  // The caller's block: rows r0.., columns c0.. of M.
  const int64_t r0 = transposed ? j0 : i0, c0 = transposed ? i0 : j0;
  for (int q = threadIdx.x; q < kB * (kB / kV); q += kStageThreads) {
    const int r = q / (kB / kV), c = (q % (kB / kV)) * kV;
    const int64_t mr = r0 + r, mc = c0 + c;
    float v[kV];
    if (vec_ok && mr < rows && mc + kV <= cols) {
      const IO* p = src + mr * ld + mc;
      IO e[kV];
      if constexpr (sizeof(IO) == 2) {
        *reinterpret_cast<uint4*>(e) = *reinterpret_cast<const uint4*>(p);
      } else {
        reinterpret_cast<uint4*>(e)[0] = reinterpret_cast<const uint4*>(p)[0];
        reinterpret_cast<uint4*>(e)[1] = reinterpret_cast<const uint4*>(p)[1];
      }
#pragma unroll
      for (int k = 0; k < kV; ++k) v[k] = to_f32<IO>(e[k]);
    } else {
#pragma unroll
      for (int k = 0; k < kV; ++k) v[k] = (mr < rows && mc + k < cols) ? to_f32<IO>(src[mr * ld + mc + k]) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kV; ++k) tile[r][c + k] = v[k] * scale;
  }
  __syncthreads();
  // Same orientation as the block read: X for a wide input, X^T for a tall one.
  T* direct = transposed ? XT + (int64_t)b * xstride + j0 * n_pad + i0 : X + (int64_t)b * xstride + i0 * m_pad + j0;
  T* across = transposed ? X + (int64_t)b * xstride + i0 * m_pad + j0 : XT + (int64_t)b * xstride + j0 * n_pad + i0;
  const int64_t ld_direct = transposed ? n_pad : m_pad, ld_across = transposed ? m_pad : n_pad;
  constexpr int kE = 16 / sizeof(T);
  for (int q = threadIdx.x; q < kB * (kB / kE); q += kStageThreads) {
    const int r = q / (kB / kE), c = (q % (kB / kE)) * kE;
    T out[kE];
#pragma unroll
    for (int k = 0; k < kE; ++k) out[k] = from_f32<T>(tile[r][c + k]);
    *reinterpret_cast<uint4*>(direct + r * ld_direct + c) = *reinterpret_cast<const uint4*>(out);
#pragma unroll
    for (int k = 0; k < kE; ++k) out[k] = from_f32<T>(tile[c + k][r]);
    *reinterpret_cast<uint4*>(across + r * ld_across + c) = *reinterpret_cast<const uint4*>(out);
  }
}

// Scan of `count` contiguous elements of each of `batch` buffers (batch
// stride bstride elements) for NaN and Inf: status_bits are ORed into the
// status word when one is found.  16-byte loads when count, bstride and
// the base are multiples of 16 bytes.
template <typename T>
__global__ void __launch_bounds__(kStageThreads) k_check_finite(const T* p, int64_t count, int64_t bstride,
                                                               int vec_ok, int32_t* d_status, int32_t status_bits) {
  const T* a = p + (int64_t)blockIdx.y * bstride;
  const int64_t tid = (int64_t)blockIdx.x * kStageThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kStageThreads;
  bool bad = false;
  int64_t done = 0;
  if (vec_ok) {
    constexpr int V = 16 / sizeof(T);
    const int64_t nv = count / V;
    const uint4* av = reinterpret_cast<const uint4*>(a);
    for (int64_t i = tid; i < nv; i += stride) {
      const uint4 q = av[i];
      const T* e = reinterpret_cast<const T*>(&q);
#pragma unroll
      for (int k = 0; k < V; ++k) bad |= !(fabsf(to_f32<T>(e[k])) < __builtin_inff());
    }
    done = nv * V;
  }
  for (int64_t i = done + tid; i < count; i += stride) bad |= !(fabsf(to_f32<T>(a[i])) < __builtin_inff());
  report_status(d_status, status_bits, bad);
}

// ---------------------------------------------------------------------------
// Guarded Gram iteration: per-matrix device flags, `stride` ints per matrix.
// Index 0 selects the X buffer (0: the first pair, 1: the second); index k
// (2 <= k <= steps) is set when a restart happens before step k.
// ---------------------------------------------------------------------------

// flags[b][0] = 0, flags[b][k] = bit k of the fixed restart mask.
static __global__ void k_guard_init(int32_t* flags, int batch, int stride, uint32_t mask) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < batch * stride) {
    const int k = i % stride;
    flags[i] = (k >= 2 && k < 32) ? (int32_t)((mask >> k) & 1u) : 0;
  }
}

// After a restart before step k: matrices that restarted now hold their X
// in the other buffer.
static __global__ void k_guard_flip(int32_t* flags, int batch, int stride, int k) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch && flags[(int64_t)b * stride + k]) flags[(int64_t)b * stride] ^= 1;
}

// The restart detector, after step k formed Q (one block per matrix).  The
// accumulated Q has an eigenvalue near the product of the a_j since the
// last restart in the directions of X's smallest singular values, and
// stored in fp16 its rounding error grows with that eigenvalue; the largest
// diagonal entry tracks it.  A restart before step k + 1 is scheduled when
// max_i |Q_ii| * |a_{k+1}| exceeds theta, or when a diagonal entry of R (a
// Gram matrix: never negative in exact arithmetic) is negative or not
// finite (a restart recomputes R from X).  Restarting is then reported through the status
// word (guard_bits).
template <typename T>
__global__ void __launch_bounds__(kStageThreads) k_guard_detect(const T* Q, const T* R, int64_t ld, int64_t nstride,
                                                               int n_real, float a_next, float theta, int32_t* flags,
                                                               int stride, int k_next, int32_t* d_status,
                                                               int32_t guard_bits) {
  __shared__ float sh_max[kStageThreads / 64];
  __shared__ int sh_bad[kStageThreads / 64];
  const int b = blockIdx.x;
  const T* q = Q + (int64_t)b * nstride;
  const T* r = R + (int64_t)b * nstride;
  float m = 0.f;
  int bad = 0;
  for (int i = threadIdx.x; i < n_real; i += kStageThreads) {
    const float qi = to_f32<T>(q[(int64_t)i * (ld + 1)]), ri = to_f32<T>(r[(int64_t)i * (ld + 1)]);
    if (ri < 0.f || !(fabsf(ri) < __builtin_inff())) bad = 1;
    m = fmaxf(m, fabsf(qi));  // fmaxf drops a NaN; an Inf schedules a restart
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    m = fmaxf(m, __shfl_down(m, off, 64));
    bad |= __shfl_down(bad, off, 64);
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    sh_max[w] = m;
    sh_bad[w] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kStageThreads / 64; ++i) {
      m = fmaxf(m, sh_max[i]);
      bad |= sh_bad[i];
    }
    int32_t* f = flags + (int64_t)b * stride + k_next;
    if ((bad || m * fabsf(a_next) > theta) && !*f) {
      *f = 1;
      if (d_status) atomicOr(d_status, guard_bits);
    }
  }
}

// Muon momentum: M <- mu M + G (fp32), U = G + mu M (Nesterov) or M, U
// rounded to IO and stored contiguously (rows x cols per matrix).  One
// block per row; 8 consecutive elements per thread, vectorized when rows
// are 16-byte aligned.
template <typename IO>
__global__ void __launch_bounds__(kStageThreads) k_momentum(const IO* G, float* M, IO* U, int64_t cols, int64_t ld,
                                                           int64_t bstride, int vec_ok, float mu, int nesterov) {
  constexpr int kV = 8;
  const int64_t b = blockIdx.y, i = blockIdx.x;
  const IO* g = G + b * bstride + i * ld;
  float* m = M + b * bstride + i * ld;
  IO* u = U + (b * (int64_t)gridDim.x + i) * cols;
  for (int64_t c0 = (int64_t)threadIdx.x * kV; c0 < cols; c0 += (int64_t)kStageThreads * kV) {
    float gv[kV], mv[kV];
    const bool full = vec_ok && c0 + kV <= cols;
    if (full) {
      IO e[kV];
      if constexpr (sizeof(IO) == 2) {
        *reinterpret_cast<uint4*>(e) = *reinterpret_cast<const uint4*>(g + c0);
      } else {
        reinterpret_cast<uint4*>(e)[0] = reinterpret_cast<const uint4*>(g + c0)[0];
        reinterpret_cast<uint4*>(e)[1] = reinterpret_cast<const uint4*>(g + c0)[1];
      }
#pragma unroll
      for (int k = 0; k < kV; ++k) gv[k] = to_f32<IO>(e[k]);
      *reinterpret_cast<float4*>(mv) = reinterpret_cast<const float4*>(m + c0)[0];
      *reinterpret_cast<float4*>(mv + 4) = reinterpret_cast<const float4*>(m + c0)[1];
    } else {
#pragma unroll
      for (int k = 0; k < kV; ++k) {
        gv[k] = c0 + k < cols ? to_f32<IO>(g[c0 + k]) : 0.f;
        mv[k] = c0 + k < cols ? m[c0 + k] : 0.f;
      }
    }
    IO uo[kV];
#pragma unroll
    for (int k = 0; k < kV; ++k) {
      mv[k] = fmaf(mu, mv[k], gv[k]);
      uo[k] = from_f32<IO>(nesterov ? fmaf(mu, mv[k], gv[k]) : mv[k]);
    }
    if (full) {
      reinterpret_cast<float4*>(m + c0)[0] = *reinterpret_cast<const float4*>(mv);
      reinterpret_cast<float4*>(m + c0)[1] = *reinterpret_cast<const float4*>(mv + 4);
    } else {
      for (int k = 0; k < kV && c0 + k < cols; ++k) m[c0 + k] = mv[k];
    }
    // U rows are contiguous: 16-byte stores when the row start is aligned.
    if (full && ((cols * (int64_t)sizeof(IO)) % 16 == 0)) {
      if constexpr (sizeof(IO) == 2) {
        *reinterpret_cast<uint4*>(u + c0) = *reinterpret_cast<const uint4*>(uo);
      } else {
        reinterpret_cast<uint4*>(u + c0)[0] = reinterpret_cast<const uint4*>(uo)[0];
        reinterpret_cast<uint4*>(u + c0)[1] = reinterpret_cast<const uint4*>(uo)[1];
      }
    } else {
      for (int k = 0; k < kV && c0 + k < cols; ++k) u[c0 + k] = uo[k];
    }
  }
}

}  // namespace nsk
