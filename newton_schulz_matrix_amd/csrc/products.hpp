// products.hpp - MFMA tile engine for the matrix products of Newton-Schulz.
//
// Every product in both Newton-Schulz forms is one of two shapes:
//
//   sym  : C = beta*E + gamma * L R^T   (L, R: n x K row-major, C, E: n x n)
//          with a symmetric result, so only tiles (tm <= tn) are computed and
//          each is also stored mirrored.  X X^T, A A (A symmetric), Z' Q,
//          Z' R and Z' V are all of this shape (Q, R, V, Z' are polynomials
//          in the same Gram matrix, so they are symmetric and commute).
//   nn   : C = alpha*E + gamma * B X   (B: n x n, X: n x m row-major)
//          the update X <- a X + B X and the Gram form's Q X.
//
// Tile engine (gfx950, CDNA4):
//   * 256 threads = 4 wave64s in a 2 x 2 grid; block tile TILE x TILE
//     (TILE = 256 or 128); each wave owns a (TILE/2)^2 sub-tile made of
//     32 x 32 MFMA tiles (v_mfma_f32_32x32x16_{f16,bf16}; for fp32 operands
//     four v_mfma_f32_32x32x2_f32 per 16-byte chunk).
//   * K is consumed in k-tiles of 128 bytes per operand row (64 16-bit or
//     32 fp32 elements), staged through LDS with two buffers; global loads
//     of k-tile t+1 are in flight while k-tile t feeds the MFMAs.
//   * LDS rows are 128 bytes made of eight 16-byte chunks; chunk c of row r
//     lives at slot c ^ ((r ^ (r >> 3)) & 7), so the 32 rows an MFMA operand
//     read touches, and the transposed writes of the nn loader, spread over
//     the banks.
//   * Both operands are read from LDS the same way (row r, 8 consecutive k),
//     so a K-contiguous operand is copied straight through, and the X
//     operand of nn (k is its row index) is transposed in registers on its
//     way from global memory to LDS (8 x 8 blocks of 16-bit elements).
//   * The MFMA's first operand is the right-hand matrix, so each lane ends
//     up holding four consecutive columns of one output row, which makes the
//     fp32 epilogue (alpha*E + gamma*acc, casts) work on 8- or 16-byte
//     vectors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace nsk {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;  // bytes of one operand row in one k-tile

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}

// ---------------------------------------------------------------------------
// Element conversions.
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<_Float16>(_Float16 x) { return (float)x; }
template <> __device__ __forceinline__ float to_f32<__bf16>(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// Four consecutive elements <-> four floats.
template <typename T> struct Quad;
template <> struct Quad<float> {
  static __device__ __forceinline__ f32x4 load(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
  }
  static __device__ __forceinline__ void store(float* p, f32x4 v) {
    *reinterpret_cast<f32x4*>(p) = v;
  }
};
template <typename H> struct Quad16 {
  typedef H h4 __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ f32x4 load(const H* p) {
    h4 v = *reinterpret_cast<const h4*>(p);
    return f32x4{to_f32<H>(v[0]), to_f32<H>(v[1]), to_f32<H>(v[2]), to_f32<H>(v[3])};
  }
  static __device__ __forceinline__ void store(H* p, f32x4 v) {
    h4 o;
    o[0] = from_f32<H>(v[0]);
    o[1] = from_f32<H>(v[1]);
    o[2] = from_f32<H>(v[2]);
    o[3] = from_f32<H>(v[3]);
    *reinterpret_cast<h4*>(p) = o;
  }
};
template <> struct Quad<_Float16> : Quad16<_Float16> {};
template <> struct Quad<__bf16> : Quad16<__bf16> {};

// ---------------------------------------------------------------------------
// One 16-byte chunk of each operand into the 32 x 32 accumulator.
// a: right-hand operand (becomes the MFMA's rows), b: left-hand operand.
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ void mma_chunk(const uint4& a, const uint4& b, f32x16& acc);

template <> __device__ __forceinline__ void mma_chunk<_Float16>(const uint4& a, const uint4& b, f32x16& acc) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mma_chunk<__bf16>(const uint4& a, const uint4& b, f32x16& acc) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
template <> __device__ __forceinline__ void mma_chunk<float>(const uint4& a, const uint4& b, f32x16& acc) {
  // Lane half h holds k = 4h..4h+3 of this 8-wide k group in both operands;
  // the e-th instruction pairs element e of the two halves.
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Global -> LDS loaders.
// ---------------------------------------------------------------------------

// K-contiguous operand: TILE rows of 128 bytes per k-tile.
template <int TILE>
struct RowLoader {
  static constexpr int kPer = TILE * 8 / kThreads;  // 16-byte chunks per thread
  uint4 r[kPer];
  __device__ __forceinline__ void load(const char* g, int64_t ld_bytes, int kt) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = threadIdx.x + i * kThreads;
      const int row = q >> 3, ch = q & 7;
      r[i] = *reinterpret_cast<const uint4*>(g + (int64_t)row * ld_bytes + (int64_t)kt * kRowBytes + ch * 16);
    }
  }
  __device__ __forceinline__ void store(char* s) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = threadIdx.x + i * kThreads;
      const int row = q >> 3, ch = q & 7;
      *reinterpret_cast<uint4*>(s + lds_off(row, ch)) = r[i];
    }
  }
};

// X operand of nn: k runs along X's rows.  A k-tile is BK rows x TILE
// columns of X; it is stored in LDS as TILE rows (one per column of X) of
// BK k-values, by transposing E x E blocks in registers.
template <typename T, int TILE>
struct ColLoader {
  static constexpr int E = 16 / sizeof(T);        // elements per chunk
  static constexpr int BK = 8 * E;                // k values per k-tile
  static constexpr int JB = TILE / E;             // column blocks
  static constexpr int NBLK = (BK / E) * JB;
  static constexpr int kPer = (NBLK + kThreads - 1) / kThreads;
  uint4 r[kPer][E];
  __device__ __forceinline__ void load(const char* g, int64_t ld_bytes, int kt) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = threadIdx.x + i * kThreads;
      if (NBLK % kThreads == 0 || b < NBLK) {
        const int jb = b % JB, kb = b / JB;
        const char* p = g + ((int64_t)kt * BK + kb * E) * ld_bytes + jb * 16;
#pragma unroll
        for (int rr = 0; rr < E; ++rr) r[i][rr] = *reinterpret_cast<const uint4*>(p + rr * ld_bytes);
      }
    }
  }
  __device__ __forceinline__ void store(char* s) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = threadIdx.x + i * kThreads;
      if (NBLK % kThreads == 0 || b < NBLK) {
        const int jb = b % JB, kb = b / JB;
        if constexpr (E == 8) {
          // 8 x 8 block of 16-bit values: in[rr].dword[d] = (col 2d, col 2d+1)
          // of k-row rr; out[jj].dword[e] = (k 2e, k 2e+1) of column jj.
          const uint32_t* in = reinterpret_cast<const uint32_t*>(&r[i][0]);
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t lo = in[(2 * e) * 4 + (jj >> 1)];
              const uint32_t hi = in[(2 * e + 1) * 4 + (jj >> 1)];
              o[e] = (jj & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            *reinterpret_cast<uint4*>(s + lds_off(jb * 8 + jj, kb)) = uint4{o[0], o[1], o[2], o[3]};
          }
        } else {
          // 4 x 4 block of fp32 values.
          const uint32_t* in = reinterpret_cast<const uint32_t*>(&r[i][0]);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            *reinterpret_cast<uint4*>(s + lds_off(jb * 4 + jj, kb)) =
                uint4{in[0 * 4 + jj], in[1 * 4 + jj], in[2 * 4 + jj], in[3 * 4 + jj]};
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Main loop: acc[fm][fn] += L-tile * R-tile^T over `ktiles` k-tiles.
// sL/sR layout per stage: TILE rows x 128 bytes each.
// ---------------------------------------------------------------------------
template <typename T, int TILE>
struct Acc {
  static constexpr int FM = TILE / 64;  // 32x32 MFMA tiles per wave per dim
  f32x16 v[FM][FM];
};

template <typename T, int TILE>
__device__ __forceinline__ void compute_ktile(const char* sL, const char* sR, int wr, int wc, Acc<T, TILE>& acc) {
  constexpr int FM = Acc<T, TILE>::FM;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, h = lane >> 5;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 a[FM], b[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) a[f] = *reinterpret_cast<const uint4*>(sR + lds_off(wc + f * 32 + lr, 2 * s + h));
#pragma unroll
    for (int f = 0; f < FM; ++f) b[f] = *reinterpret_cast<const uint4*>(sL + lds_off(wr + f * 32 + lr, 2 * s + h));
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FM; ++fn) mma_chunk<T>(a[fn], b[fm], acc.v[fm][fn]);
  }
}

template <typename T, int TILE, bool COL_RIGHT>
__device__ __forceinline__ void mainloop(const char* Lg, int64_t ldl_bytes, const char* Rg, int64_t ldr_bytes,
                                         int ktiles, char* smem, Acc<T, TILE>& acc) {
  constexpr int FM = Acc<T, TILE>::FM;
  constexpr int kOpBytes = TILE * kRowBytes;
  // Stage s: L operand at smem + 2*s*kOpBytes, R operand right after it.
  const int w = threadIdx.x >> 6;
  const int wr = (w >> 1) * (TILE / 2), wc = (w & 1) * (TILE / 2);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FM; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.v[fm][fn][v] = 0.f;

  using RightLoader = typename std::conditional<COL_RIGHT, ColLoader<T, TILE>, RowLoader<TILE>>::type;
  {
    RowLoader<TILE> la;
    RightLoader lb;
    la.load(Lg, ldl_bytes, 0);
    lb.load(Rg, ldr_bytes, 0);
    la.store(smem);
    lb.store(smem + kOpBytes);
  }
  __syncthreads();
  // The loaders live inside one iteration so their registers are never
  // carried around the loop; the last k-tile is peeled.
  for (int kt = 0; kt + 1 < ktiles; ++kt) {
    const int cur = kt & 1;
    RowLoader<TILE> la;
    RightLoader lb;
    la.load(Lg, ldl_bytes, kt + 1);
    lb.load(Rg, ldr_bytes, kt + 1);
    const char* sc = smem + cur * 2 * kOpBytes;
    compute_ktile<T, TILE>(sc, sc + kOpBytes, wr, wc, acc);
    char* sn = smem + (cur ^ 1) * 2 * kOpBytes;
    la.store(sn);
    lb.store(sn + kOpBytes);
    __syncthreads();
  }
  {
    const char* sc = smem + ((ktiles - 1) & 1) * 2 * kOpBytes;
    compute_ktile<T, TILE>(sc, sc + kOpBytes, wr, wc, acc);
  }
}

// ---------------------------------------------------------------------------
// Kernel arguments.
// ---------------------------------------------------------------------------
template <typename T>
struct SymArgs {
  const T* L;        // n x K, row stride ldk
  const T* R;        // n x K, row stride ldk
  const T* E;        // n x n (ldn) or null when beta == 0
  T* C;              // n x n (ldn)
  T* C2;             // optional second output: C + delta * I on rows < n_real
  int64_t sL, sR, sE, sC, sC2;  // batch strides in elements
  int ldk, ldn;      // row strides in elements
  int K;             // multiple of the k-tile
  int tiles;         // n / TILE
  int n_real;
  float alpha_unused;
  float beta, gamma, delta;
};

template <typename T, typename OutT>
struct NNArgs {
  const T* B;        // n x n (ldb)
  const T* X;        // n x m (ldx)
  const T* E;        // n x m (ldx) or null when alpha == 0
  OutT* Y;           // output
  int64_t sB, sX, sE, sY;
  int ldb, ldx;
  int64_t ldy;       // output leading dimension
  int K;             // = n padded
  int tiles_m, tiles_n;
  int n_real, m_real;  // valid output rows/cols (wide orientation)
  int transpose_out;   // final output: write element (i, j) to Y[j * ldy + i]
  int final_out;       // 1: bounds-checked store in OutT with out_scale
  float alpha, gamma, out_scale;
  int32_t* d_status;
};

// Upper-triangle tile index -> (tm, tn), tm <= tn, row-major over the
// upper triangle: row tm holds tiles - tm entries.
__device__ __forceinline__ void tri_tile(int idx, int tiles, int& tm, int& tn) {
  int r = 0;
  int left = idx;
  while (left >= tiles - r) {
    left -= tiles - r;
    ++r;
  }
  tm = r;
  tn = r + left;
}

// GRAM_INPUT only separates the X X^T launches (inner dimension m) from the
// n x n products into their own kernel symbol, so profiles list them apart.
template <typename T, int TILE, bool GRAM_INPUT>
__global__ void __launch_bounds__(kThreads, 1) k_sym(SymArgs<T> p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int FM = Acc<T, TILE>::FM;
  int tm, tn;
  tri_tile(blockIdx.x, p.tiles, tm, tn);
  const int bz = blockIdx.y;
  const int64_t ldk_bytes = (int64_t)p.ldk * sizeof(T);
  const char* Lg = reinterpret_cast<const char*>(p.L + bz * p.sL) + (int64_t)tm * TILE * ldk_bytes;
  const char* Rg = reinterpret_cast<const char*>(p.R + bz * p.sR) + (int64_t)tn * TILE * ldk_bytes;
  constexpr int BK = kRowBytes / sizeof(T);
  Acc<T, TILE> acc;
  mainloop<T, TILE, false>(Lg, ldk_bytes, Rg, ldk_bytes, p.K / BK, smem, acc);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 31, h = lane >> 5;
  const int wr = (w >> 1) * (TILE / 2), wc = (w & 1) * (TILE / 2);
  const T* E = p.E ? p.E + bz * p.sE : nullptr;
  T* C = p.C + bz * p.sC;
  T* C2 = p.C2 ? p.C2 + bz * p.sC2 : nullptr;
  const bool diag_tile = (tm == tn);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int i = tm * TILE + wr + fm * 32 + lr;
#pragma unroll
    for (int fn = 0; fn < FM; ++fn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = tn * TILE + wc + fn * 32 + 8 * g + 4 * h;
        f32x4 v;
        v[0] = p.gamma * acc.v[fm][fn][4 * g + 0];
        v[1] = p.gamma * acc.v[fm][fn][4 * g + 1];
        v[2] = p.gamma * acc.v[fm][fn][4 * g + 2];
        v[3] = p.gamma * acc.v[fm][fn][4 * g + 3];
        if (E) {
          const f32x4 e = Quad<T>::load(E + (int64_t)i * p.ldn + j0);
          v += p.beta * e;
        }
        f32x4 v2 = v;
        if (C2) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (i == j0 + e && i < p.n_real) v2[e] += p.delta;
        }
        if (!diag_tile) {
          Quad<T>::store(C + (int64_t)i * p.ldn + j0, v);
#pragma unroll
          for (int e = 0; e < 4; ++e) C[(int64_t)(j0 + e) * p.ldn + i] = from_f32<T>(v[e]);
          if (C2) {
            Quad<T>::store(C2 + (int64_t)i * p.ldn + j0, v2);
#pragma unroll
            for (int e = 0; e < 4; ++e) C2[(int64_t)(j0 + e) * p.ldn + i] = from_f32<T>(v2[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = j0 + e;
            if (i <= j) {
              const T x = from_f32<T>(v[e]);
              C[(int64_t)i * p.ldn + j] = x;
              C[(int64_t)j * p.ldn + i] = x;
              if (C2) {
                const T x2 = from_f32<T>(v2[e]);
                C2[(int64_t)i * p.ldn + j] = x2;
                C2[(int64_t)j * p.ldn + i] = x2;
              }
            }
          }
        }
      }
    }
  }
}

template <typename T, typename OutT, int TILE>
__global__ void __launch_bounds__(kThreads, 1) k_nn(NNArgs<T, OutT> p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int FM = Acc<T, TILE>::FM;
  const int tm = blockIdx.x / p.tiles_n;
  const int tn = blockIdx.x % p.tiles_n;
  const int bz = blockIdx.y;
  const int64_t ldb_bytes = (int64_t)p.ldb * sizeof(T);
  const int64_t ldx_bytes = (int64_t)p.ldx * sizeof(T);
  const char* Lg = reinterpret_cast<const char*>(p.B + bz * p.sB) + (int64_t)tm * TILE * ldb_bytes;
  const char* Rg = reinterpret_cast<const char*>(p.X + bz * p.sX) + (int64_t)tn * TILE * sizeof(T);
  constexpr int BK = kRowBytes / sizeof(T);
  Acc<T, TILE> acc;
  mainloop<T, TILE, true>(Lg, ldb_bytes, Rg, ldx_bytes, p.K / BK, smem, acc);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 31, h = lane >> 5;
  const int wr = (w >> 1) * (TILE / 2), wc = (w & 1) * (TILE / 2);
  const T* E = p.E ? p.E + bz * p.sE : nullptr;
  OutT* Y = p.Y + bz * p.sY;
  bool bad = false;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int i = tm * TILE + wr + fm * 32 + lr;
#pragma unroll
    for (int fn = 0; fn < FM; ++fn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = tn * TILE + wc + fn * 32 + 8 * g + 4 * h;
        f32x4 v;
        v[0] = p.gamma * acc.v[fm][fn][4 * g + 0];
        v[1] = p.gamma * acc.v[fm][fn][4 * g + 1];
        v[2] = p.gamma * acc.v[fm][fn][4 * g + 2];
        v[3] = p.gamma * acc.v[fm][fn][4 * g + 3];
        if (E) {
          const f32x4 e = Quad<T>::load(E + (int64_t)i * p.ldx + j0);
          v += p.alpha * e;
        }
        if (!p.final_out) {
          Quad<OutT>::store(Y + (int64_t)i * p.ldy + j0, v);
        } else {
          v *= p.out_scale;
          if (i < p.n_real) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int j = j0 + e;
              if (j < p.m_real) {
                const OutT x = from_f32<OutT>(v[e]);
                bad |= !__builtin_isfinite(to_f32<OutT>(x));
                if (p.transpose_out)
                  Y[(int64_t)j * p.ldy + i] = x;
                else
                  Y[(int64_t)i * p.ldy + j] = x;
              }
            }
          }
        }
      }
    }
  }
  if (p.d_status) {
    const unsigned long long any_bad = __ballot(bad);
    if (any_bad && lane == __ffsll(any_bad) - 1) atomicOr(p.d_status, 1);
  }
}

}  // namespace nsk
