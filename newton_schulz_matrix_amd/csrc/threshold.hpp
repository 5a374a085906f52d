// threshold.hpp - ROOT soft-threshold split M = B + O on the device.
//
// ROOT (reportify.cn summary, "technical innovations of ROOT") splits the
// gradient into a robust part B and an outlier part O = soft-threshold(M)
// with an l1 penalty and orthogonalizes only B.  The threshold is
// lambda = mult * median|M| (mult = 3 in the heavy-tailed workload).
//
// The median is found exactly by a select on the bit patterns of |M|: for
// IEEE formats, |x| compares like its bit pattern with the sign bit cleared
// read as an unsigned integer.  16-bit keys (15 bits) take one histogram
// pass over all 2^15 keys (k_hist16, k_pick16).  fp32 keys (31 bits) take a
// radix select: digits of up to 11 bits from the top, each pass
// histogramming the digit of the keys that match the prefix chosen so far
// (LDS histogram, merged with global atomics), a one-block kernel picking
// the bucket that holds the wanted rank; three passes.  No host sync.
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

static __global__ void k_select_init(SelectState* st, uint32_t* hist, int nhist, uint64_t rank) {
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

// Inclusive prefix sum of v over a block of kPickThreads threads (four
// waves): a shuffle scan within each wave plus the totals of the waves
// before it, two barriers in all.  wsum: kPickThreads / 64 words of LDS.
constexpr int kPickThreads = 256;
__device__ __forceinline__ uint64_t pick_scan(uint64_t v, uint64_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t u = __shfl_up((unsigned long long)v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  uint64_t before = 0;
  for (int i = 0; i < w; ++i) before += wsum[i];
  __syncthreads();  // wsum is reused by the next scan
  return v + before;
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
  static_assert(kHistThreads == kPickThreads, "pick_scan's block size");
  __shared__ uint64_t wsum[kPickThreads / 64];
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
  // Inclusive prefix sums of the per-thread totals (its barriers also make
  // every thread's tot[] visible to the scanning thread below).
  const uint64_t incl = pick_scan(s, wsum), excl = incl - s;
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

// ---------------------------------------------------------------------------
// One-pass select for 16-bit keys.  |x| of a bf16 or fp16 value is a 15-bit
// key, so one histogram of all 2^15 keys finds the median exactly.  Every
// work-group counts its share of the elements into a 128 KiB LDS histogram
// and adds its nonzero bins into one of kSelCopies global copies (block b
// into copy b % 8, the XCD it runs on, so a copy's atomics stay in that
// XCD's L2), and the sums of each group of kSelGroup consecutive keys into
// a small coarse histogram (copies likewise).  One block then scans the
// coarse sums to find the group that holds the wanted rank and the group's
// bins to find the key: it reads 2 K coarse sums and one group's bins
// instead of all 8 x 32 K.
// ---------------------------------------------------------------------------
constexpr int kKeyBins16 = 1 << 15;
constexpr int kSelCopies = 8;
constexpr int kSelThreads = 1024;
constexpr int kSelGroup = 128;                          // keys per coarse group
constexpr int kSelGroups = kKeyBins16 / kSelGroup;      // 256
constexpr int kSelFineWords = kSelCopies * kKeyBins16;  // fine histogram words, then the coarse ones
constexpr int kSelWords = kSelFineWords + kSelCopies * kSelGroups;

template <typename IO>
__global__ void __launch_bounds__(kSelThreads) k_hist16(const IO* M, int64_t numel, uint32_t* hist, int vec_ok) {
  __shared__ __attribute__((aligned(16))) uint32_t h[kKeyBins16];
  // The histogram is cleared after this thread's first load is issued, so
  // the clearing overlaps that load's latency; the barrier waits for the LDS
  // stores only (a fenced barrier would also wait for the load).
  auto clear = [&]() {
    for (int i = threadIdx.x; i < kKeyBins16 / 4; i += kSelThreads) reinterpret_cast<uint4*>(h)[i] = uint4{0, 0, 0, 0};
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(63));  // LDS stores only
    lds_barrier();
  };
  auto count = [&](uint32_t raw) { atomicAdd(&h[raw & 0x7fffu], 1u); };
  auto count_chunk = [&](const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      count(w[j] & 0xffffu);
      count(w[j] >> 16);
    }
  };
  const int64_t tid = (int64_t)blockIdx.x * kSelThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kSelThreads;
  int64_t done = 0;
  if (vec_ok) {  // uniform: a kernel argument
    const int64_t nvec = numel / 8;
    const uint4* Mv = reinterpret_cast<const uint4*>(M);
    // Software-pipelined: each 16-byte load is issued before the previous
    // one is counted, so the LDS atomics overlap the memory latency.
    int64_t i = tid;
    const bool any = i < nvec;
    uint4 cur = uint4{0, 0, 0, 0};
    if (any) cur = Mv[i];
    clear();  // every thread of the block
    if (any) {
      for (i += stride; i < nvec; i += stride) {
        const uint4 nxt = Mv[i];
        count_chunk(cur);
        cur = nxt;
      }
      count_chunk(cur);
    }
    done = nvec * 8;
  } else {
    clear();
  }
  for (int64_t i = done + tid; i < numel; i += stride) count((uint32_t)__builtin_bit_cast(uint16_t, M[i]));
  __syncthreads();
  // Flush: key k * kSelThreads + t for thread t (neighbouring lanes read
  // neighbouring words, no LDS bank conflicts); nonzero bins only.  All 32
  // reads are issued before the first atomic, so their latencies overlap.
  const int copy = blockIdx.x % kSelCopies;
  uint32_t* hg = hist + (int64_t)copy * kKeyBins16;
  constexpr int kPerThread = kKeyBins16 / kSelThreads;
  uint32_t c[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) c[k] = h[k * kSelThreads + threadIdx.x];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k)
    if (c[k]) atomicAdd(&hg[k * kSelThreads + threadIdx.x], c[k]);
  // Group totals: four neighbouring threads share a group, each adding 32
  // of its keys (8 16-byte reads, rotated by the lane so that neighbouring
  // threads, 128 bytes apart, meet fewer banks at once); two quad moves sum
  // the four, and one thread adds the total into the coarse histogram.
  static_assert(kSelGroups * 4 == kSelThreads && kSelGroup == 4 * 32, "four threads of 32 keys per group");
  {
    const int t = threadIdx.x;
    const uint4* hv = reinterpret_cast<const uint4*>(h) + t * 8;
    uint32_t part = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 v = hv[(j + t) & 7];
      part += v.x + v.y + v.z + v.w;
    }
    // quad_perm [1,0,3,2] then [2,3,0,1]: every lane of a quad ends with the sum.
    part += (uint32_t)__builtin_amdgcn_mov_dpp((int)part, 0xB1, 0xF, 0xF, false);
    part += (uint32_t)__builtin_amdgcn_mov_dpp((int)part, 0x4E, 0xF, 0xF, false);
    if ((t & 3) == 0 && part) atomicAdd(&hist[kSelFineWords + copy * kSelGroups + (t >> 2)], part);
  }
}

// One block: the key holding rank st->rank; lambda = mult * its value.
// 256 threads: thread t holds coarse group t, then key g*128 + t of the
// chosen group g; both prefix sums are wave scans (pick_scan).
static_assert(kSelGroups == kPickThreads && kSelGroup <= kPickThreads, "one thread per group and per key");

template <typename IO>
__global__ void __launch_bounds__(kPickThreads) k_pick16(SelectState* st, const uint32_t* hist, float mult,
                                                        float* d_lambda_out) {
  __shared__ uint64_t wsum[kPickThreads / 64];
  __shared__ int sh_group;
  __shared__ uint64_t sh_before;
  const uint64_t want = st->rank;
  const int t = threadIdx.x;
  // Coarse pass: group t's total over the copies.
  uint64_t s = 0;
#pragma unroll
  for (int k = 0; k < kSelCopies; ++k) s += hist[kSelFineWords + k * kSelGroups + t];
  {
    const uint64_t incl = pick_scan(s, wsum), excl = incl - s;
    if ((excl < want && want <= incl) || (t == kSelGroups - 1 && want > incl)) {
      sh_group = t;
      sh_before = excl;
    }
  }
  __syncthreads();
  const int g = sh_group;
  const uint64_t before = sh_before;
  // Fine pass over the group's keys: thread t < 128 holds key g*128 + t.
  uint64_t c = 0;
  if (t < kSelGroup) {
#pragma unroll
    for (int k = 0; k < kSelCopies; ++k) c += hist[(int64_t)k * kKeyBins16 + g * kSelGroup + t];
  }
  const uint64_t incl = before + pick_scan(c, wsum), excl = incl - c;
  if (t < kSelGroup && ((excl < want && want <= incl) || (t == kSelGroup - 1 && want > incl))) {
    const uint32_t key = (uint32_t)(g * kSelGroup + t);
    st->rank = want - excl;
    st->prefix = key;
    st->mask = 0x7fffu;
    const float lam = mult * KeyOf<IO>::value(key);
    st->lambda = lam;
    if (d_lambda_out) *d_lambda_out = lam;
  }
}

// Explicit lambda: only record it.
static __global__ void k_set_lambda(SelectState* st, float lam, float* d_lambda_out) {
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

// With a status word, a non-finite lambda, B or O ORs status_bits into it
// (NaN inputs pass through to B, so they are reported too).
template <typename IO>
__global__ void __launch_bounds__(256) k_clip_split(const IO* M, IO* B, IO* O, int64_t numel, const SelectState* st,
                                                   int vec_ok, int32_t* d_status, int32_t status_bits) {
  const float lam = st->lambda;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t done = 0;
  bool bad = false;
  auto check = [&](IO b, IO o) {
    if (d_status) bad |= !(fabsf(to_f32<IO>(b)) < __builtin_inff()) || !(fabsf(to_f32<IO>(o)) < __builtin_inff());
  };
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
        check(bj, oj);
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
    check(b, o);
    B[i] = b;
    if (O) O[i] = o;
  }
  if (d_status) {
    bad |= !(fabsf(lam) < __builtin_inff());
    report_status(d_status, status_bits, bad);
  }
}

}  // namespace nsk
