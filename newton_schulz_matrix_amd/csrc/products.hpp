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
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

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

// K-contiguous operand: TILE rows of 128 bytes per k-tile, copied straight
// from global memory into LDS (global_load_lds_dwordx4: lane L of a wave
// writes its 16 bytes at M0 + 16 L).  One instruction fills 8 LDS rows; lane
// L fetches the chunk that belongs at slot L & 7 of row L >> 3, so the LDS
// swizzle is applied on the global side.  Row r = 8 q + (L >> 3) of the wave
// has swz(r) = (L >> 3) ^ (q & 7).
template <int TILE>
struct DmaLoader {
  static constexpr int kRowsPerWave = TILE / 4;
  static constexpr int kIters = kRowsPerWave / 8;
  uint32_t lane_off;   // (L >> 3) * ld + 16 * ((L & 7) ^ (L >> 3))
  uint32_t ld8;        // 8 * ld (bytes), uniform
  int wave_row0;       // first LDS row this wave fills (uniform)
  __device__ __forceinline__ void init(int64_t ld_bytes) {
    const int lane = threadIdx.x & 63;
    wave_row0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * kRowsPerWave;
    lane_off = (uint32_t)((lane >> 3) * ld_bytes) + (uint32_t)((((lane & 7) ^ (lane >> 3))) << 4);
    ld8 = (uint32_t)(8 * ld_bytes);
  }
  // g: operand tile base (rows of this tile), kt: k-tile, lds_op: LDS base
  // of the operand in the stage being filled.
  __device__ __forceinline__ void issue(const char* g, int kt, char* lds_op) const {
    const char* gw = g + (int64_t)wave_row0 * (ld8 >> 3) + (int64_t)kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int q = (wave_row0 >> 3) + i;  // LDS row group, uniform
      const uint32_t off = lane_off + (uint32_t)i * ld8;
      // The chunk XOR for this row group: (q & 7) applied to the low bits.
      const uint32_t sw = (uint32_t)((q & 7) << 4);
      __builtin_amdgcn_global_load_lds((glb_void_t*)(gw + (off ^ sw)),
                                       (lds_void_t*)(lds_op + q * 8 * kRowBytes), 16, 0, 0);
    }
  }
};

// X operand of nn: k runs along X's rows.  A k-tile is BK rows x TILE
// columns of X; it is stored in LDS as TILE rows (one per column of X) of
// BK k-values, by transposing E x E blocks in registers.  Thread t owns
// column block jb = t % JB and k block kb = t / JB.
template <typename T, int TILE>
struct ColLoader {
  static constexpr int E = 16 / sizeof(T);        // elements per chunk
  static constexpr int BK = 8 * E;                // k values per k-tile
  static constexpr int JB = TILE / E;             // column blocks
  static constexpr int NBLK = (BK / E) * JB;
  static constexpr int kPer = (NBLK + kThreads - 1) / kThreads;
  uint4 r[kPer][E];
  __device__ __forceinline__ void load(const char* g, int64_t ld_bytes, int kt) {
    const char* gk = g + (int64_t)kt * BK * ld_bytes;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = threadIdx.x + i * kThreads;
      if (NBLK % kThreads == 0 || b < NBLK) {
        const int jb = b % JB, kb = b / JB;
        const uint32_t off = (uint32_t)(kb * E * ld_bytes) + (uint32_t)(jb * 16);
#pragma unroll
        for (int rr = 0; rr < E; ++rr)
          r[i][rr] = *reinterpret_cast<const uint4*>(gk + (off + (uint32_t)(rr * ld_bytes)));
      }
    }
  }
  __device__ __forceinline__ void store(char* s) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = threadIdx.x + i * kThreads;
      if (NBLK % kThreads == 0 || b < NBLK) {
        const int jb = b % JB, kb = b / JB;
        // Row j = jb*E + jj; for E == 8, swz(j) = jj ^ (jb & 7).
        const uint32_t* in = reinterpret_cast<const uint32_t*>(&r[i][0]);
        if constexpr (E == 8) {
          // 8 x 8 block of 16-bit values: in[rr].dword[d] = (col 2d, col 2d+1)
          // of k-row rr; out[jj].dword[e] = (k 2e, k 2e+1) of column jj.
          char* base = s + jb * 8 * kRowBytes;
          const int x = kb ^ (jb & 7);
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t lo = in[(2 * e) * 4 + (jj >> 1)];
              const uint32_t hi = in[(2 * e + 1) * 4 + (jj >> 1)];
              o[e] = (jj & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            *reinterpret_cast<uint4*>(base + jj * kRowBytes + ((x ^ jj) << 4)) = uint4{o[0], o[1], o[2], o[3]};
          }
        } else {
          // 4 x 4 block of fp32 values.
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
// Main loop: acc[fm][fn] += L-tile * R-tile^T over a range of k-tiles.
// ---------------------------------------------------------------------------
template <int FM>
struct Frags {
  uint4 a[FM], b[FM];
};

// Per-lane LDS byte offsets of this wave's fragment rows.  Fragment i of a
// wave covers rows w0 + 32 i + (L & 31) with w0 a multiple of 64, so
// swz(row) = (L & 7) ^ (4 (i & 1) + ((L & 31) >> 3)) only depends on the
// parity of i; the offset of (i, chunk c) is row0 + 4096 i + 16 (c ^ swz).
struct FragAddr {
  uint32_t row0L, row0R;  // (w0 + (L & 31)) * 128 for the L and R operands
  int sw0, sw1;           // swz for even and odd i
  __device__ __forceinline__ void init(int wr, int wc) {
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31;
    row0L = (uint32_t)((wr + lr) * kRowBytes);
    row0R = (uint32_t)((wc + lr) * kRowBytes);
    sw0 = (lr & 7) ^ (lr >> 3);
    sw1 = (lr & 7) ^ (4 + (lr >> 3));
  }
};

// Fragments of substep s (16-byte chunk pair 2s, 2s+1) for this wave.
template <int FM>
__device__ __forceinline__ void load_frags(const char* sL, const char* sR, const FragAddr& fa, int s,
                                           Frags<FM>& f) {
  const int h = (threadIdx.x & 63) >> 5;
  const uint32_t c0 = (uint32_t)(((2 * s + h) ^ fa.sw0) << 4);
  const uint32_t c1 = (uint32_t)(((2 * s + h) ^ fa.sw1) << 4);
#pragma unroll
  for (int i = 0; i < FM; ++i)
    f.a[i] = *reinterpret_cast<const uint4*>(sR + (fa.row0R + ((i & 1) ? c1 : c0)) + i * 32 * kRowBytes);
#pragma unroll
  for (int i = 0; i < FM; ++i)
    f.b[i] = *reinterpret_cast<const uint4*>(sL + (fa.row0L + ((i & 1) ? c1 : c0)) + i * 32 * kRowBytes);
}

template <typename T, int FM>
__device__ __forceinline__ void mma_frags(const Frags<FM>& f, f32x16 (&acc)[FM][FM]) {
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FM; ++fn) mma_chunk<T>(f.a[fn], f.b[fm], acc[fm][fn]);
}

// All four substeps of one k-tile, with the fragments of substep s+1 read
// from LDS while the MFMAs of substep s run.  `mid` runs between substeps 1
// and 2 (the nn kernel stores its transposed operand there).
template <typename T, int TILE, class Mid>
__device__ __forceinline__ void compute_ktile(const char* sL, const char* sR, const FragAddr& fa,
                                              f32x16 (&acc)[TILE / 64][TILE / 64], Mid&& mid) {
  constexpr int FM = TILE / 64;
  Frags<FM> f0, f1;
  load_frags<FM>(sL, sR, fa, 0, f0);
  load_frags<FM>(sL, sR, fa, 1, f1);
  mma_frags<T, FM>(f0, acc);
  load_frags<FM>(sL, sR, fa, 2, f0);
  mma_frags<T, FM>(f1, acc);
  mid();
  load_frags<FM>(sL, sR, fa, 3, f1);
  mma_frags<T, FM>(f0, acc);
  mma_frags<T, FM>(f1, acc);
}

// Instruction order for a k-tile of the DMA path (one basic block): the
// global->LDS copies of the next k-tile first, the fragment reads of
// substeps 0 and 1, then the reads of substeps 2 and 3 spread between the
// MFMAs of substeps 0 and 1, then the MFMAs of substeps 2 and 3.  The MFMA
// count per 16-byte chunk is 1 (16-bit) or 4 (fp32).
template <typename T, int TILE>
__device__ __forceinline__ void schedule_dma_ktile() {
  constexpr int FM = TILE / 64;
  constexpr int NR = 2 * FM;                                   // reads per substep
  constexpr int NM = FM * FM * (sizeof(T) == 4 ? 4 : 1);       // MFMAs per substep
  __builtin_amdgcn_sched_group_barrier(0x020, 2 * (TILE / 32), 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * NR, 0);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, NM / NR, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * NM, 0);
}

template <typename T, int TILE>
struct Acc {
  static constexpr int FM = TILE / 64;  // 32x32 MFMA tiles per wave per dim
  f32x16 v[FM][FM];
};

// The two LDS stages are distinct __shared__ objects (per tile size), so the
// compiler can tell the DMA writes into one stage from the fragment reads of
// the other and does not wait for the loads in flight before every read.
// Each stage holds the L operand (TILE rows x 128 bytes) followed by the R
// operand.
__shared__ __attribute__((aligned(1024))) char g_stage0_256[2 * 256 * kRowBytes];
__shared__ __attribute__((aligned(1024))) char g_stage1_256[2 * 256 * kRowBytes];
__shared__ __attribute__((aligned(1024))) char g_stage0_128[2 * 128 * kRowBytes];
__shared__ __attribute__((aligned(1024))) char g_stage1_128[2 * 128 * kRowBytes];

template <int TILE> struct Stages;
template <> struct Stages<256> {
  static __device__ __forceinline__ char* s0() { return g_stage0_256; }
  static __device__ __forceinline__ char* s1() { return g_stage1_256; }
};
template <> struct Stages<128> {
  static __device__ __forceinline__ char* s0() { return g_stage0_128; }
  static __device__ __forceinline__ char* s1() { return g_stage1_128; }
};

// One k-tile: start the loads of k-tile kt+1 into `nxt` (when there is one),
// run the MFMAs on `cur`, then wait for the loads and synchronize.
template <typename T, int TILE, bool COL_RIGHT>
__device__ __forceinline__ void ktile_step(const char* Lg, const char* Rg, int64_t ldr_bytes,
                                           const DmaLoader<TILE>& la, const DmaLoader<TILE>& lb, int kt,
                                           bool more, const char* __restrict__ cur, char* __restrict__ nxt,
                                           const FragAddr& fa,
                                           f32x16 (&acc)[TILE / 64][TILE / 64]) {
  constexpr int kOpBytes = TILE * kRowBytes;
  if constexpr (COL_RIGHT) {
    ColLoader<T, TILE> cb;
    if (more) {
      la.issue(Lg, kt + 1, nxt);
      cb.load(Rg, ldr_bytes, kt + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute_ktile<T, TILE>(cur, cur + kOpBytes, fa, acc, [&] {
      if (more) cb.store(nxt + kOpBytes);
    });
  } else {
    // Always copy: the last k-tile reloads itself into the idle stage, so
    // the step is one basic block the schedule below can order.
    const int ktn = more ? kt + 1 : kt;
    la.issue(Lg, ktn, nxt);
    lb.issue(Rg, ktn, nxt + kOpBytes);
    compute_ktile<T, TILE>(cur, cur + kOpBytes, fa, acc, [] {});
    schedule_dma_ktile<T, TILE>();
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// acc += L-tile * R-tile^T over k-tiles [kt0, kt1) (acc is initialized by the
// caller).
template <typename T, int TILE, bool COL_RIGHT>
__device__ __forceinline__ void mainloop(const char* Lg, int64_t ldl_bytes, const char* Rg, int64_t ldr_bytes,
                                         int kt0, int kt1, Acc<T, TILE>& acc) {
  constexpr int kOpBytes = TILE * kRowBytes;
  const int w = threadIdx.x >> 6;
  const int wr = (w >> 1) * (TILE / 2), wc = (w & 1) * (TILE / 2);
  if (kt1 <= kt0) return;

  char* s0 = Stages<TILE>::s0();
  char* s1 = Stages<TILE>::s1();
  FragAddr fa;
  fa.init(wr, wc);
  DmaLoader<TILE> la, lb;
  la.init(ldl_bytes);
  if constexpr (!COL_RIGHT) lb.init(ldr_bytes);

  la.issue(Lg, kt0, s0);
  if constexpr (COL_RIGHT) {
    ColLoader<T, TILE> cb;
    cb.load(Rg, ldr_bytes, kt0);
    cb.store(s0 + kOpBytes);
  } else {
    lb.issue(Rg, kt0, s0 + kOpBytes);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = kt0; kt < kt1; ++kt) {
    const bool odd = (kt - kt0) & 1;
    ktile_step<T, TILE, COL_RIGHT>(Lg, Rg, ldr_bytes, la, lb, kt, kt + 1 < kt1, odd ? s1 : s0, odd ? s0 : s1, fa,
                                   acc.v);
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

// Work-groups are dealt to the 8 XCDs round-robin (work-group b runs on XCD
// b % 8), and each XCD has its own L2.  xcd_order(b, count) returns the
// position of work-group b in a list of `count` tiles cut into 8 contiguous
// pieces, piece x for XCD x, so tiles that are neighbours in the list (and
// share operand panels) run on the same XCD.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_order(int b, int count) {
  const int x = b % kXcds, j = b / kXcds;
  const int per = count / kXcds, extra = count % kXcds;  // XCD x runs per + (x < extra) work-groups
  return x * per + (x < extra ? x : extra) + j;
}

// Upper-triangle tiles listed row pair by row pair: rows p and nt-1-p hold
// nt - p and p + 1 tiles, nt + 1 together, so a piece of the list covers few
// row panels (the L operand) and the column panels right of them.
__device__ __forceinline__ void tri_tile(int idx, int nt, int& tm, int& tn) {
  const int p = idx / (nt + 1), rem = idx % (nt + 1);
  if (rem < nt - p) {
    tm = p;
    tn = p + rem;
  } else {
    tm = nt - 1 - p;
    tn = tm + rem - (nt - p);
  }
}

// Output tile staged in LDS (the stage buffers are free after the main
// loop): TILE rows of TILE * sizeof(T) bytes, 16-byte chunk q of row r at
// slot q ^ tswz(r).  The swizzle keeps both the row-quad writes from the
// accumulators (32 consecutive rows) and the column reads of the mirrored
// store (rows 8 apart) on distinct chunks.
// The tile spans the two stage buffers: rows [0, kRowsPerStage) in the
// first, the rest in the second.
template <typename T, int TILE>
struct TileLds {
  static constexpr int kRowB = TILE * (int)sizeof(T);
  static constexpr int kCPR = kRowB / 16;          // chunks per row
  static constexpr int kEC = 16 / (int)sizeof(T);  // elements per chunk
  static constexpr int kS = kCPR == 32 ? 5 : 4;
  static constexpr int kStageB = 2 * TILE * kRowBytes;
  static constexpr int kRowsPerStage = kStageB / kRowB;
  static_assert(kCPR == 32 || kCPR == 16, "tile row must be 256 or 512 bytes");
  static_assert(TILE <= 2 * kRowsPerStage, "tile must fit in the two stage buffers");
  static __device__ __forceinline__ int tswz(int r) { return (r ^ (r >> kS)) & (kCPR - 1); }
  static __device__ __forceinline__ char* row_base(int r) {
    return r < kRowsPerStage ? Stages<TILE>::s0() + r * kRowB : Stages<TILE>::s1() + (r - kRowsPerStage) * kRowB;
  }
  static __device__ __forceinline__ char* at(int r, int col) {
    return row_base(r) + (((col / kEC) ^ tswz(r)) << 4) + (col % kEC) * (int)sizeof(T);
  }
  static __device__ __forceinline__ char* chunk(int r, int c) { return row_base(r) + ((c ^ tswz(r)) << 4); }
};

template <typename T, int TILE>
__device__ __forceinline__ void acc_zero(Acc<T, TILE>& acc) {
  constexpr int FM = Acc<T, TILE>::FM;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FM; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.v[fm][fn][v] = 0.f;
}

// GRAM_INPUT only separates the X X^T launches (inner dimension m) from the
// n x n products into their own kernel symbol, so profiles list them apart.
template <typename T, int TILE, bool GRAM_INPUT>
__global__ void __launch_bounds__(kThreads, 1) k_sym(SymArgs<T> p) {
  constexpr int FM = Acc<T, TILE>::FM;
  using TL = TileLds<T, TILE>;
  int tm, tn;
  const int ntri = p.tiles * (p.tiles + 1) / 2;
  tri_tile(gridDim.y == 1 ? xcd_order(blockIdx.x, ntri) : blockIdx.x, p.tiles, tm, tn);
  const int bz = blockIdx.y;
  const int64_t ldk_bytes = (int64_t)p.ldk * sizeof(T);
  const char* Lg = reinterpret_cast<const char*>(p.L + bz * p.sL) + (int64_t)tm * TILE * ldk_bytes;
  const char* Rg = reinterpret_cast<const char*>(p.R + bz * p.sR) + (int64_t)tn * TILE * ldk_bytes;
  constexpr int BK = kRowBytes / sizeof(T);
  const T* E = p.E ? p.E + bz * p.sE : nullptr;
  T* C = p.C + bz * p.sC;
  T* C2 = p.C2 ? p.C2 + bz * p.sC2 : nullptr;
  const bool diag_tile = (tm == tn);
  const int64_t row0 = (int64_t)tm * TILE, col0 = (int64_t)tn * TILE;
  Acc<T, TILE> acc;
  acc_zero<T, TILE>(acc);
  mainloop<T, TILE, false>(Lg, ldk_bytes, Rg, ldk_bytes, 0, p.K / BK, acc);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 31, h = lane >> 5;
  const int wr = (w >> 1) * (TILE / 2), wc = (w & 1) * (TILE / 2);

  // Phase A: beta*E + gamma*acc, rounded to T, into the LDS tile.  The
  // diagonal of C2 (= C + delta I on real rows) is written here, rounded
  // once from fp32.
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int il = wr + fm * 32 + lr;
#pragma unroll
    for (int fn = 0; fn < FM; ++fn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int jl = wc + fn * 32 + 8 * g + 4 * h;
        f32x4 v;
        v[0] = p.gamma * acc.v[fm][fn][4 * g + 0];
        v[1] = p.gamma * acc.v[fm][fn][4 * g + 1];
        v[2] = p.gamma * acc.v[fm][fn][4 * g + 2];
        v[3] = p.gamma * acc.v[fm][fn][4 * g + 3];
        if (E) v += p.beta * Quad<T>::load(E + (row0 + il) * p.ldn + col0 + jl);
        Quad<T>::store(reinterpret_cast<T*>(TL::at(il, jl)), v);
        if (C2 && diag_tile) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (il == jl + e && row0 + il < p.n_real)
              C2[(row0 + il) * p.ldn + col0 + il] = from_f32<T>(v[e] + p.delta);
        }
      }
    }
  }
  __syncthreads();

  // Phase B: rows of the tile.  On a diagonal tile each element (r, j) is
  // taken from the upper triangle, tile[min(r, j)][max(r, j)], so the result
  // is exactly symmetric; C2's diagonal was written in phase A.
  constexpr int kChunks = TILE * TL::kCPR;
  constexpr int EC = TL::kEC;
  for (int q = threadIdx.x; q < kChunks; q += kThreads) {
    const int r = q / TL::kCPR, c = q % TL::kCPR;
    T* dst = C + (row0 + r) * p.ldn + col0 + c * EC;
    T* dst2 = C2 ? C2 + (row0 + r) * p.ldn + col0 + c * EC : nullptr;
    if (!diag_tile) {
      const uint4 val = *reinterpret_cast<const uint4*>(TL::chunk(r, c));
      *reinterpret_cast<uint4*>(dst) = val;
      if (dst2) *reinterpret_cast<uint4*>(dst2) = val;
    } else {
      T vals[EC];
#pragma unroll
      for (int e = 0; e < EC; ++e) {
        const int j = c * EC + e;
        vals[e] = *reinterpret_cast<const T*>(j >= r ? TL::at(r, j) : TL::at(j, r));
      }
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(vals);
      if (dst2) {
        const int jd = r - c * EC;  // position of the diagonal inside this chunk
        if (jd >= 0 && jd < EC && row0 + r < p.n_real) {
#pragma unroll
          for (int e = 0; e < EC; ++e)
            if (e != jd) dst2[e] = vals[e];
        } else {
          *reinterpret_cast<uint4*>(dst2) = *reinterpret_cast<const uint4*>(vals);
        }
      }
    }
  }
  if (diag_tile) return;

  // Phase C: the mirrored tile, C[col0 + jj][row0 + i] = tile[i][jj]; row jj
  // of the mirror is column jj of the LDS tile.
  for (int q = threadIdx.x; q < kChunks; q += kThreads) {
    const int jj = q / TL::kCPR, c = q % TL::kCPR;
    T vals[EC];
#pragma unroll
    for (int e = 0; e < EC; ++e) vals[e] = *reinterpret_cast<const T*>(TL::at(c * EC + e, jj));
    const uint4 val = *reinterpret_cast<const uint4*>(vals);
    *reinterpret_cast<uint4*>(C + (col0 + jj) * p.ldn + row0 + c * EC) = val;
    if (C2) *reinterpret_cast<uint4*>(C2 + (col0 + jj) * p.ldn + row0 + c * EC) = val;
  }
}

template <typename T, typename OutT, int TILE>
__global__ void __launch_bounds__(kThreads, 1) k_nn(NNArgs<T, OutT> p) {
  constexpr int FM = Acc<T, TILE>::FM;
  using TL = TileLds<OutT, TILE>;
  const int tm = blockIdx.x / p.tiles_n;
  const int tn = blockIdx.x % p.tiles_n;
  const int bz = blockIdx.y;
  const int64_t ldb_bytes = (int64_t)p.ldb * sizeof(T);
  const int64_t ldx_bytes = (int64_t)p.ldx * sizeof(T);
  const char* Lg = reinterpret_cast<const char*>(p.B + bz * p.sB) + (int64_t)tm * TILE * ldb_bytes;
  const char* Rg = reinterpret_cast<const char*>(p.X + bz * p.sX) + (int64_t)tn * TILE * sizeof(T);
  constexpr int BK = kRowBytes / sizeof(T);
  const T* E = p.E ? p.E + bz * p.sE : nullptr;
  OutT* Y = p.Y + bz * p.sY;
  const int64_t row0 = (int64_t)tm * TILE, col0 = (int64_t)tn * TILE;
  Acc<T, TILE> acc;
  acc_zero<T, TILE>(acc);
  mainloop<T, TILE, true>(Lg, ldb_bytes, Rg, ldx_bytes, 0, p.K / BK, acc);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 31, h = lane >> 5;
  const int wr = (w >> 1) * (TILE / 2), wc = (w & 1) * (TILE / 2);
  const float scale = p.final_out ? p.out_scale : 1.f;
  bool bad = false;

  // Phase A: alpha*E + gamma*acc (times the output scale), rounded to OutT,
  // into the LDS tile.
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int il = wr + fm * 32 + lr;
#pragma unroll
    for (int fn = 0; fn < FM; ++fn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int jl = wc + fn * 32 + 8 * g + 4 * h;
        f32x4 v;
        v[0] = p.gamma * acc.v[fm][fn][4 * g + 0];
        v[1] = p.gamma * acc.v[fm][fn][4 * g + 1];
        v[2] = p.gamma * acc.v[fm][fn][4 * g + 2];
        v[3] = p.gamma * acc.v[fm][fn][4 * g + 3];
        if (E) v += p.alpha * Quad<T>::load(E + (row0 + il) * p.ldx + col0 + jl);
        v *= scale;
        if (p.final_out) {
#pragma unroll
          for (int e = 0; e < 4; ++e) bad |= !__builtin_isfinite(to_f32<OutT>(from_f32<OutT>(v[e])));
        }
        Quad<OutT>::store(reinterpret_cast<OutT*>(TL::at(il, jl)), v);
      }
    }
  }
  __syncthreads();

  constexpr int kChunks = TILE * TL::kCPR;
  if (!p.final_out) {
    // Internal buffer: whole padded tile, rows of 16-byte chunks.
    for (int q = threadIdx.x; q < kChunks; q += kThreads) {
      const int r = q / TL::kCPR, c = q % TL::kCPR;
      *reinterpret_cast<uint4*>(Y + (row0 + r) * p.ldy + col0 + c * TL::kEC) =
          *reinterpret_cast<const uint4*>(TL::chunk(r, c));
    }
  } else if (!p.transpose_out) {
    // Caller's matrix, same orientation: rows i < n_real, columns j < m_real.
    const bool vec = (p.ldy % TL::kEC) == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0;
    for (int q = threadIdx.x; q < kChunks; q += kThreads) {
      const int r = q / TL::kCPR, c = q % TL::kCPR;
      const int64_t i = row0 + r, j0 = col0 + c * TL::kEC;
      if (i >= p.n_real || j0 >= p.m_real) continue;
      const uint4 val = *reinterpret_cast<const uint4*>(TL::chunk(r, c));
      OutT* dst = Y + i * p.ldy + j0;
      if (vec && j0 + TL::kEC <= p.m_real) {
        *reinterpret_cast<uint4*>(dst) = val;
      } else {
        const OutT* vals = reinterpret_cast<const OutT*>(&val);
        for (int e = 0; e < TL::kEC && j0 + e < p.m_real; ++e) dst[e] = vals[e];
      }
    }
  } else {
    // Caller's matrix is the transpose: its row j holds tile column j.
    const bool vec = (p.ldy % TL::kEC) == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0;
    for (int q = threadIdx.x; q < kChunks; q += kThreads) {
      const int jj = q / TL::kCPR, c = q % TL::kCPR;
      const int64_t j = col0 + jj, i0 = row0 + c * TL::kEC;
      if (j >= p.m_real || i0 >= p.n_real) continue;
      OutT vals[TL::kEC];
#pragma unroll
      for (int e = 0; e < TL::kEC; ++e) vals[e] = *reinterpret_cast<const OutT*>(TL::at(c * TL::kEC + e, jj));
      OutT* dst = Y + j * p.ldy + i0;
      if (vec && i0 + TL::kEC <= p.n_real) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(vals);
      } else {
        for (int e = 0; e < TL::kEC && i0 + e < p.n_real; ++e) dst[e] = vals[e];
      }
    }
  }
  if (p.d_status) {
    const unsigned long long any_bad = __ballot(bad);
    if (any_bad && lane == __ffsll(any_bad) - 1) atomicOr(p.d_status, 1);
  }
}

}  // namespace nsk
