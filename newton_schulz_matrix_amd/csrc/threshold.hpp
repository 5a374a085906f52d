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
// Copies of each pass's global histogram: block b adds its counts to copy
// b % kHistCopies, so that fewer blocks' atomics meet on one hot bin; the
// pick kernel adds the copies.
constexpr int kHistCopies = 4;

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
  static __device__ __forceinline__ uint32_t key_bits(uint32_t raw) { return raw & 0x7fffu; }
  static __device__ __forceinline__ uint32_t key(__bf16 x) { return __builtin_bit_cast(uint16_t, x) & 0x7fffu; }
  static __device__ __forceinline__ float value(uint32_t k) { return (float)__builtin_bit_cast(__bf16, (uint16_t)k); }
};
template <> struct KeyOf<_Float16> {
  static constexpr int kBits = 15;
  static __device__ __forceinline__ uint32_t key_bits(uint32_t raw) { return raw & 0x7fffu; }
  static __device__ __forceinline__ uint32_t key(_Float16 x) { return __builtin_bit_cast(uint16_t, x) & 0x7fffu; }
  static __device__ __forceinline__ float value(uint32_t k) { return (float)__builtin_bit_cast(_Float16, (uint16_t)k); }
};
template <> struct KeyOf<float> {
  static constexpr int kBits = 31;
  static __device__ __forceinline__ uint32_t key_bits(uint32_t raw) { return raw & 0x7fffffffu; }
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

// Raw bits of element j of a 16-byte chunk of IO elements.
template <typename IO>
__device__ __forceinline__ uint32_t chunk_bits(const uint4& v, int j) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (sizeof(IO) == 2)
    return (w[j >> 1] >> (16 * (j & 1))) & 0xffffu;
  else
    return w[j];
}

// Histogram of digit (key >> shift) & (2^bits - 1) over keys matching the
// current prefix.  Each wave counts into its own LDS copy (hot bins are
// shared by many keys; separate copies keep the waves from contending), and
// the copies are summed into one of the kHistCopies global copies at the end
// (hist: kHistCopies x kHistBins).  With vec_ok
// (16-byte aligned M) the elements are read as 16-byte chunks, four chunks
// in flight per thread, the last numel % (16 / sizeof(IO)) one by one.
template <typename IO>
__global__ void __launch_bounds__(kHistThreads) k_radix_hist(const IO* M, int64_t numel, const SelectState* st,
                                                            int shift, int bits, uint32_t* hist, int vec_ok) {
  constexpr int kWaves = kHistThreads / 64;
  __shared__ uint32_t h[kWaves][kHistBins];
  const int nb = 1 << bits;
  for (int i = threadIdx.x; i < kWaves * kHistBins; i += kHistThreads) (&h[0][0])[i] = 0u;
  __syncthreads();
  uint32_t* hw = h[threadIdx.x >> 6];
  const uint32_t prefix = st->prefix, mask = st->mask;
  const uint32_t dmask = (uint32_t)nb - 1u;
  auto count = [&](uint32_t raw) {
    const uint32_t k = KeyOf<IO>::key_bits(raw);
    if ((k & mask) == prefix) atomicAdd(&hw[(k >> shift) & dmask], 1u);
  };
  constexpr int V = 16 / (int)sizeof(IO);
  auto count_chunk = [&](const uint4& v) {
#pragma unroll
    for (int j = 0; j < V; ++j) count(chunk_bits<IO>(v, j));
  };
  const int64_t tid = (int64_t)blockIdx.x * kHistThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kHistThreads;
  int64_t done = 0;
  if (vec_ok) {
    const int64_t nvec = numel / V;
    const uint4* Mv = reinterpret_cast<const uint4*>(M);
    int64_t i = tid;
    for (; i + 3 * stride < nvec; i += 4 * stride) {
      const uint4 v0 = Mv[i], v1 = Mv[i + stride], v2 = Mv[i + 2 * stride], v3 = Mv[i + 3 * stride];
      count_chunk(v0);
      count_chunk(v1);
      count_chunk(v2);
      count_chunk(v3);
    }
    for (; i < nvec; i += stride) count_chunk(Mv[i]);
    done = nvec * V;
  }
  for (int64_t i = done + tid; i < numel; i += stride) {
    if constexpr (sizeof(IO) == 2)
      count((uint32_t)__builtin_bit_cast(uint16_t, M[i]));
    else
      count(__builtin_bit_cast(uint32_t, M[i]));
  }
  __syncthreads();
  uint32_t* hg = hist + (blockIdx.x % kHistCopies) * kHistBins;
  for (int i = threadIdx.x; i < nb; i += kHistThreads) {
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) c += h[w][i];
    if (c) atomicAdd(&hg[i], c);
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
  __shared__ uint32_t tot[kHistBins];  // per-bin totals over the copies
  // Read before the barriers below: one thread rewrites the state at the end.
  const uint64_t want = st->rank;
  const int nb = 1 << bits;
  const int per = (nb + kHistThreads - 1) / kHistThreads;
  const int lo = threadIdx.x * per;
  uint64_t s = 0;
  for (int i = lo; i < lo + per && i < nb; ++i) {
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < kHistCopies; ++k) c += hist[k * kHistBins + i];
    tot[i] = c;
    s += c;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  // Inclusive prefix sums of the per-thread totals (log-step scan).
  for (int off = 1; off < kHistThreads; off <<= 1) {
    const uint64_t v = (int)threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  const uint64_t incl = part[threadIdx.x], excl = incl - s;
  // The thread whose bins hold rank `want` (the last one if the rank were
  // past the total) scans them.
  if ((excl < want && want <= incl) || (threadIdx.x == kHistThreads - 1 && want > incl)) {
    uint64_t acc = excl;
    int bin = lo;
    const int end = min(nb, lo + per);
    while (bin < end - 1 && acc + tot[bin] < want) acc += tot[bin++];
    if (bin > nb - 1) bin = nb - 1;
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

// B = clip(M, -lambda, lambda); O = M - B (fp32, then rounded).  With
// vec_ok (M, B and O 16-byte aligned) 16-byte chunks, the tail one by one.
template <typename IO>
__device__ __forceinline__ void clip_one(float x, float lam, IO& b, IO& o) {
  // fminf/fmaxf would turn NaN into lambda; keep NaN.
  const float c = (x > lam) ? lam : ((x < -lam) ? -lam : x);
  b = from_f32<IO>(c);
  o = from_f32<IO>(x - to_f32<IO>(b));
}

template <typename IO>
__global__ void __launch_bounds__(256) k_clip_split(const IO* M, IO* B, IO* O, int64_t numel, const SelectState* st,
                                                   int vec_ok) {
  const float lam = st->lambda;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t done = 0;
  if (vec_ok) {
    constexpr int V = 16 / (int)sizeof(IO);
    typedef IO vec_t __attribute__((ext_vector_type(V)));
    const int64_t nvec = numel / V;
    for (int64_t i = tid; i < nvec; i += stride) {
      const vec_t m = reinterpret_cast<const vec_t*>(M)[i];
      vec_t b, o;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        IO bj, oj;
        clip_one<IO>(to_f32<IO>(m[j]), lam, bj, oj);
        b[j] = bj;
        o[j] = oj;
      }
      reinterpret_cast<vec_t*>(B)[i] = b;
      if (O) reinterpret_cast<vec_t*>(O)[i] = o;
    }
    done = nvec * V;
  }
  for (int64_t i = done + tid; i < numel; i += stride) {
    IO b, o;
    clip_one<IO>(to_f32<IO>(M[i]), lam, b, o);
    B[i] = b;
    if (O) O[i] = o;
  }
}

}  // namespace nsk
