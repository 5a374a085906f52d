// threshold.hpp - ROOT soft-threshold split M = B + O on the device.
//
// ROOT (reportify.cn summary, "technical innovations of ROOT") splits the
// gradient into a robust part B and an outlier part O = soft-threshold(M)
// with an l1 penalty and orthogonalizes only B.  The threshold is
// lambda = mult * median|M| (mult = 3 in the heavy-tailed workload).
//
// The median is found exactly by a radix select on the bit patterns of |M|:
// for IEEE formats, |x| compares like its bit pattern with the sign bit
// cleared read as an unsigned integer.  Digits of up to 11 bits are taken
// from the top; each pass histograms the digit of the keys that match the
// prefix chosen so far (LDS histogram, merged with global atomics) and a
// one-block kernel picks the bucket holding the wanted rank.  16-bit keys
// (15 bits) take two passes, fp32 keys (31 bits) three.  No host sync.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "products.hpp"

namespace nsk {

constexpr int kHistBins = 2048;
constexpr int kHistThreads = 256;

// Select state in device memory.
struct SelectState {
  uint32_t prefix;     // key bits chosen so far
  uint32_t mask;       // which key bits are chosen
  uint64_t rank;       // 1-based rank still wanted inside the current prefix
  float lambda;        // final threshold
  uint32_t pad;
};

template <typename IO> struct KeyOf;
template <> struct KeyOf<__bf16> {
  static constexpr int kBits = 15;
  static __device__ __forceinline__ uint32_t key(__bf16 x) { return __builtin_bit_cast(uint16_t, x) & 0x7fffu; }
  static __device__ __forceinline__ float value(uint32_t k) { return (float)__builtin_bit_cast(__bf16, (uint16_t)k); }
};
template <> struct KeyOf<_Float16> {
  static constexpr int kBits = 15;
  static __device__ __forceinline__ uint32_t key(_Float16 x) { return __builtin_bit_cast(uint16_t, x) & 0x7fffu; }
  static __device__ __forceinline__ float value(uint32_t k) { return (float)__builtin_bit_cast(_Float16, (uint16_t)k); }
};
template <> struct KeyOf<float> {
  static constexpr int kBits = 31;
  static __device__ __forceinline__ uint32_t key(float x) { return __float_as_uint(x) & 0x7fffffffu; }
  static __device__ __forceinline__ float value(uint32_t k) { return __uint_as_float(k); }
};

__global__ void k_select_init(SelectState* st, uint32_t* hist, int nhist, uint64_t rank) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nhist) hist[i] = 0u;
  if (i == 0) {
    st->prefix = 0u;
    st->mask = 0u;
    st->rank = rank;
    st->lambda = 0.f;
    st->pad = 0u;
  }
}

// Histogram of digit (key >> shift) & (2^bits - 1) over keys matching the
// current prefix.
template <typename IO>
__global__ void __launch_bounds__(kHistThreads) k_radix_hist(const IO* M, int64_t numel, const SelectState* st,
                                                            int shift, int bits, uint32_t* hist) {
  __shared__ uint32_t h[kHistBins];
  const int nb = 1 << bits;
  for (int i = threadIdx.x; i < nb; i += kHistThreads) h[i] = 0u;
  __syncthreads();
  const uint32_t prefix = st->prefix, mask = st->mask;
  const uint32_t dmask = (uint32_t)nb - 1u;
  const int64_t stride = (int64_t)gridDim.x * kHistThreads;
  for (int64_t i = (int64_t)blockIdx.x * kHistThreads + threadIdx.x; i < numel; i += stride) {
    const uint32_t k = KeyOf<IO>::key(M[i]);
    if ((k & mask) == prefix) atomicAdd(&h[(k >> shift) & dmask], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += kHistThreads) {
    const uint32_t c = h[i];
    if (c) atomicAdd(&hist[i], c);
  }
}

// One block: find the bucket holding rank st->rank, extend the prefix, and
// after the last pass turn the key into lambda = mult * value (or take the
// caller's lambda when it is >= 0).
template <typename IO>
__global__ void __launch_bounds__(kHistThreads) k_radix_pick(SelectState* st, const uint32_t* hist, int shift,
                                                            int bits, int last, float mult, float user_lambda,
                                                            float* d_lambda_out) {
  __shared__ uint64_t part[kHistThreads];
  const int nb = 1 << bits;
  const int per = (nb + kHistThreads - 1) / kHistThreads;
  const int lo = threadIdx.x * per;
  uint64_t s = 0;
  for (int i = lo; i < lo + per && i < nb; ++i) s += hist[i];
  part[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    // Serial scan over 256 partial sums, then over one thread's bins.
    const uint64_t want = st->rank;
    uint64_t acc = 0;
    int t = 0;
    while (t < kHistThreads - 1 && acc + part[t] < want) acc += part[t++];
    int bin = t * per;
    const int end = min(nb, bin + per);
    while (bin < end - 1 && acc + hist[bin] < want) acc += hist[bin++];
    st->rank = want - acc;
    st->prefix |= (uint32_t)bin << shift;
    st->mask |= ((uint32_t)nb - 1u) << shift;
    if (last) {
      const float lam = user_lambda >= 0.f ? user_lambda : mult * KeyOf<IO>::value(st->prefix);
      st->lambda = lam;
      if (d_lambda_out) *d_lambda_out = lam;
    }
  }
}

// Explicit lambda: only record it.
__global__ void k_set_lambda(SelectState* st, float lam, float* d_lambda_out) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    st->lambda = lam;
    if (d_lambda_out) *d_lambda_out = lam;
  }
}

// B = clip(M, -lambda, lambda); O = M - B (fp32, then rounded).
template <typename IO>
__global__ void __launch_bounds__(256) k_clip_split(const IO* M, IO* B, IO* O, int64_t numel, const SelectState* st) {
  const float lam = st->lambda;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < numel; i += stride) {
    const float x = to_f32<IO>(M[i]);
    // fminf/fmaxf would turn NaN into lambda; keep NaN.
    const float c = (x > lam) ? lam : ((x < -lam) ? -lam : x);
    const IO bq = from_f32<IO>(c);
    B[i] = bq;
    if (O) O[i] = from_f32<IO>(x - to_f32<IO>(bq));
  }
}

}  // namespace nsk
