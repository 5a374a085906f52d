// products.hpp - MFMA tile engine for the matrix products of Newton-Schulz.
//
// Every product in both Newton-Schulz forms is one of two shapes, both of
// the form L R^T with L and R stored row-major with K contiguous:
//
//   sym  : C = beta*E + gamma * L R^T   (L, R: n x K, C, E: n x n)
//          with a symmetric result, so only tiles (tm <= tn) are computed and
//          each is also stored mirrored.  X X^T, A A (A symmetric), Q Z',
//          R Z' and V Z' are all of this shape (Q, R, V, Z' are polynomials
//          in the same Gram matrix, so they are symmetric and commute).
//   nt   : Y = alpha*E + gamma * B X = alpha*E + gamma * B (X^T)^T
//          (B: n x n, X^T: m x n), the update X <- a X + B X and the Gram
//          form's Q X.  X is kept in both layouts, X (n x m, for X X^T and
//          the a X term) and X^T (m x n, for this product), and an update
//          whose result feeds another update writes both.
//
// Tile engine (gfx950, CDNA4):
//   * 256 threads = 4 wave64s in a 2 x 2 grid; square block tiles of 128,
//     192 or 256 for 16-bit operands, 64 or 128 for fp32 (the same edge for
//     every product of a call); each wave owns
//     a (TM/2) x (TN/2) sub-tile made of 32 x 32 MFMA tiles
//     (v_mfma_f32_32x32x16_f16; for fp32 operands four
//     v_mfma_f32_32x32x2_f32 per 16-byte chunk).  16-bit input of either
//     type (bf16 or fp16) is multiplied on fp16 operands.  The 192 edge exists for
//     occupancy: a 4096 x 4096 symmetric product has 136 upper-triangle
//     tiles of 256 but 253 of 192, for 256 compute units.
//   * K is consumed in k-tiles of 128 bytes per operand row (64 16-bit or
//     32 fp32 elements), copied straight from global memory into LDS stages
//     (two or three; see Stages) and read back as MFMA fragments while the
//     copies of later k-tiles are in flight.
//   * LDS rows are 128 bytes made of eight 16-byte chunks; chunk c of row r
//     lives at slot c ^ ((r ^ (r >> 3)) & 7), so the 32 rows an MFMA operand
//     read touches spread over the banks.
//   * Both operands are read from LDS the same way (row r, 8 consecutive k).
//   * The MFMA's first operand is the right-hand matrix, so each lane ends
//     up holding four consecutive columns of one output row, which makes the
//     fp32 epilogue (alpha*E + gamma*acc, casts) work on 8- or 16-byte
//     vectors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nsortho.h"

namespace nsk {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
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

// The smallest magnitude that rounds to infinity (round to nearest even):
// a value is finite after rounding to T exactly when its magnitude is below
// this (NaN compares false).
template <typename T> inline constexpr float kRoundsToInf = __builtin_inff();
template <> inline constexpr float kRoundsToInf<_Float16> = 65520.0f;            // 65504 + half an ulp
template <> inline constexpr float kRoundsToInf<__bf16> = 0x1.ffp127f;          // bf16 max + half an ulp

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

// K-contiguous operand: ROWS rows of 128 bytes per k-tile, copied straight
// from global memory into LDS (buffer_load_dwordx4 ... lds: lane L of a wave
// writes its 16 bytes at M0 + 16 L).  One instruction fills 8 LDS rows; lane
// L fetches the chunk that belongs at slot L & 7 of row L >> 3, so the LDS
// swizzle is applied on the global side.  Row r = 8 q + (L >> 3) of the wave
// has swz(r) = (L >> 3) ^ (q & 7).
//
// Each wave addresses its rows through a buffer resource whose base is its
// first row, a per-lane 32-bit offset per row group (fixed for the whole
// loop) and the k-tile's byte offset as the scalar offset, so a copy costs
// no vector address arithmetic.  The offsets stay below 2^32: a wave covers
// at most 64 rows of at most 2^25 bytes (the plan's limit on a row).
template <int ROWS>
struct DmaLoader {
  static_assert(ROWS % 32 == 0, "each wave fills whole groups of 8 rows");
  static constexpr int kRowsPerWave = ROWS / 4;
  static constexpr int kIters = kRowsPerWave / 8;
  static_assert(kRowsPerWave <= 64, "per-lane offsets fit 32 bits for rows of up to 2^25 bytes");
  // The 256 tile has no registers to spare for eight offsets; it forms each
  // one at issue time (two 32-bit operations).
  static constexpr bool kKeep = kIters <= 6;
  __amdgpu_buffer_rsrc_t rsrc;       // this wave's rows of the operand tile (uniform)
  uint32_t voff[kKeep ? kIters : 1]; // lane offset of row group i, chunk swizzle applied
  uint32_t lane_off, ld8;            // for kKeep == false
  int wave_row0;                     // first LDS row this wave fills (uniform)
  __device__ __forceinline__ uint32_t offset(int i) const {
    const int q = (wave_row0 >> 3) + i;  // LDS row group
    // The chunk XOR for this row group: (q & 7) on bits 4-6 (the row part of
    // the offset is a multiple of 256 bytes).
    return (lane_off + (uint32_t)i * ld8) ^ (uint32_t)((q & 7) << 4);
  }
  // g: operand tile base (its first row), ld_bytes: row stride.
  __device__ __forceinline__ void init(const char* g, int64_t ld_bytes) {
    const int lane = threadIdx.x & 63;
    wave_row0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * kRowsPerWave;
    // Word 3 of the resource: the raw (untyped) buffer format; no bounds
    // limit below 2^32 bytes.
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(g) + (int64_t)wave_row0 * ld_bytes, (short)0, -1,
                                             0x00020000);
    lane_off = (uint32_t)((lane >> 3) * ld_bytes) + (uint32_t)((((lane & 7) ^ (lane >> 3))) << 4);
    ld8 = (uint32_t)(8 * ld_bytes);
    if constexpr (kKeep) {
#pragma unroll
      for (int i = 0; i < kIters; ++i) voff[i] = offset(i);
    }
  }
  // kt: k-tile, lds_op: LDS base of the operand in the stage being filled.
  __device__ __forceinline__ void issue(int kt, char* lds_op) const {
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int q = (wave_row0 >> 3) + i;  // LDS row group, uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(lds_op + q * 8 * kRowBytes), 16,
                                               (int)(kKeep ? voff[i] : offset(i)), kt * kRowBytes, 0, 0);
    }
  }
};

// ---------------------------------------------------------------------------
// Main loop: acc[fm][fn] += L-tile * R-tile^T over a range of k-tiles.
// ---------------------------------------------------------------------------
// Fragments of one substep: FN 32-row pieces of R, FM of L.
template <int FM, int FN>
struct Frags {
  uint4 a[FN], b[FM];
};

// Per-lane LDS byte offsets of this wave's fragment rows.  Fragment i of a
// wave covers rows w0 + 32 i + (L & 31) with w0 a multiple of 32, so
// swz(row) = (L & 7) ^ (((w0 >> 3) + 4 i + ((L & 31) >> 3)) & 7) only
// depends on the parity of i; the offset of (i, chunk c) is
// row0 + 4096 i + 16 (c ^ swz).
struct FragAddr {
  uint32_t row0L, row0R;  // (w0 + (L & 31)) * 128 for the L and R operands
  int swL0, swL1, swR0, swR1;  // swz for even and odd i
  __device__ __forceinline__ void init(int wr, int wc) {
    // The lane index goes through an opaque move so that a persistent kernel
    // recomputes these offsets per tile: hoisted out of its tile loop they
    // stay live across the main loop and are spilled at two work-groups per
    // compute unit.
    int lr;
    asm volatile("v_and_b32 %0, 31, %1" : "=v"(lr) : "v"((int)threadIdx.x));
    row0L = (uint32_t)((wr + lr) * kRowBytes);
    row0R = (uint32_t)((wc + lr) * kRowBytes);
    swL0 = swz(wr + lr);
    swL1 = swz(wr + 32 + lr);
    swR0 = swz(wc + lr);
    swR1 = swz(wc + 32 + lr);
  }
};

// Fragments of substep s (16-byte chunk pair 2s, 2s+1) for this wave.
template <int FM, int FN>
__device__ __forceinline__ void load_frags(const char* sL, const char* sR, const FragAddr& fa, int s,
                                           Frags<FM, FN>& f) {
  const int c = 2 * s + ((threadIdx.x & 63) >> 5);
  const uint32_t r0 = (uint32_t)((c ^ fa.swR0) << 4), r1 = (uint32_t)((c ^ fa.swR1) << 4);
  const uint32_t l0 = (uint32_t)((c ^ fa.swL0) << 4), l1 = (uint32_t)((c ^ fa.swL1) << 4);
#pragma unroll
  for (int i = 0; i < FN; ++i)
    f.a[i] = *reinterpret_cast<const uint4*>(sR + (fa.row0R + ((i & 1) ? r1 : r0)) + i * 32 * kRowBytes);
#pragma unroll
  for (int i = 0; i < FM; ++i)
    f.b[i] = *reinterpret_cast<const uint4*>(sL + (fa.row0L + ((i & 1) ? l1 : l0)) + i * 32 * kRowBytes);
}

template <typename T, int FM, int FN>
__device__ __forceinline__ void mma_frags(const Frags<FM, FN>& f, f32x16 (&acc)[FM][FN]) {
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) mma_chunk<T>(f.a[fn], f.b[fm], acc[fm][fn]);
}

// s_waitcnt immediates (gfx9 layout: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8); a field at its maximum does not wait.
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70; }

template <typename T, int TM, int TN>
struct Acc {
  static constexpr int FM = TM / 64;  // 32x32 MFMA tiles per wave, rows
  static constexpr int FN = TN / 64;  // and columns
  f32x16 v[FM][FN];
};

// LDS stages are distinct __shared__ objects, so the compiler can tell the
// DMA writes into one stage from the fragment reads of another and does not
// wait for the copies in flight before every read.  A stage holds the L
// operand (TM rows x 128 bytes) followed by the R operand (TN rows).  Three
// families: 64 KiB stages (two; tiles of 256 + 256 or 192 + 256 rows), 48 KiB
// (three; 192 + 192) and 32 KiB (three, or two in the kernels built for two
// work-groups per compute unit; 128 + 128).  Three stages, where they fit in
// LDS, give every copy two pipeline steps to land.
__shared__ __attribute__((aligned(1024))) char g_stage0_big[65536];
__shared__ __attribute__((aligned(1024))) char g_stage1_big[65536];
__shared__ __attribute__((aligned(1024))) char g_stage0_mid[49152];
__shared__ __attribute__((aligned(1024))) char g_stage1_mid[49152];
__shared__ __attribute__((aligned(1024))) char g_stage2_mid[49152];
__shared__ __attribute__((aligned(1024))) char g_stage0_small[32768];
__shared__ __attribute__((aligned(1024))) char g_stage1_small[32768];
__shared__ __attribute__((aligned(1024))) char g_stage2_small[32768];

template <int BYTES> struct StageMem;
template <> struct StageMem<65536> {
  static __device__ __forceinline__ char* s0() { return g_stage0_big; }
  static __device__ __forceinline__ char* s1() { return g_stage1_big; }
  static __device__ __forceinline__ char* s2() { return nullptr; }
};
template <> struct StageMem<49152> {
  static __device__ __forceinline__ char* s0() { return g_stage0_mid; }
  static __device__ __forceinline__ char* s1() { return g_stage1_mid; }
  static __device__ __forceinline__ char* s2() { return g_stage2_mid; }
};
template <> struct StageMem<32768> {
  static __device__ __forceinline__ char* s0() { return g_stage0_small; }
  static __device__ __forceinline__ char* s1() { return g_stage1_small; }
  static __device__ __forceinline__ char* s2() { return g_stage2_small; }
};

constexpr int kLdsBytes = 160 * 1024;

// C2's diagonal of a diagonal tile (up to 256 elements of up to 4 bytes),
// rounded once from fp32 in phase A and merged into the row stores.
__shared__ __attribute__((aligned(16))) char g_c2_diag[1024];

// G is the number of work-groups a kernel is built to share a compute unit
// with: G = 2 takes two stages (two 128-tile work-groups then fit in LDS
// together, and one's start-up and epilogue overlap the other's main loop).
template <int TM, int TN, int G = 1>
struct Stages {
  static constexpr int kNeed = (TM + TN) * kRowBytes;
  static constexpr int kBytes = kNeed > 49152 ? 65536 : kNeed > 32768 ? 49152 : 32768;
  static constexpr int kCount = G == 1 && 3 * kBytes <= kLdsBytes ? 3 : 2;
  static_assert(G == 1 || G * kCount * kBytes <= kLdsBytes, "G work-groups must fit in LDS");
  using M = StageMem<kBytes>;
  static __device__ __forceinline__ char* s0() { return M::s0(); }
  static __device__ __forceinline__ char* s1() { return M::s1(); }
  static __device__ __forceinline__ char* s2() { return M::s2(); }
};

// Software pipeline over k-tiles.  With k-tile t in stage P and the stage D
// free, one step
//   1. starts the copies of k-tile t + (number of stages) into D,
//   2. runs the MFMAs of substeps 2 and 3 of k-tile t (fragments already in
//      registers) while reading substeps 0 and 1 of k-tile t+1 from P,
//   3. runs the MFMAs of substeps 0 and 1 of k-tile t+1 while reading its
//      substeps 2 and 3,
//   4. waits for its reads and for the copies of k-tile t+2 and meets the
//      other waves at the barrier.
// The one barrier per k-tile thus sits between substeps 1 and 2, and the
// fragment reads of one k-tile overlap the MFMAs of the previous one, so the
// LDS and the matrix cores stay busy across the k-tile boundary.  Four
// fragment sets (two substeps being consumed, two being read) live in
// registers.
template <int FM, int FN>
struct FragSets {
  Frags<FM, FN> f0, f1, f2, f3;
};

// Instruction order of one pipeline step (one basic block).  Each half
// (two substeps of MFMAs) has NR read slots; slot i holds a few MFMAs, one
// fragment read for the next two substeps and V_i copy instructions.  The
// copies are spread out because the vector memory path takes about 16
// cycles per 1 KiB copy instruction per compute unit: issued in one burst,
// they would hold up the wave, and with it the MFMAs, for hundreds of
// cycles.  With three stages the copies spread over the whole step (they
// have two steps to land), with two over the first half.
template <int NM, int NR, int NV, int I>
__device__ __forceinline__ void schedule_half() {
  if constexpr (I < NR) {
    __builtin_amdgcn_sched_group_barrier(0x008, (I + 1) * NM / NR - I * NM / NR, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    constexpr int v = (I + 1) * NV / NR - I * NV / NR;
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);
    schedule_half<NM, NR, NV, I + 1>();
  }
}

template <typename T, int TM, int TN, int G>
__device__ __forceinline__ void schedule_step() {
  constexpr int FM = TM / 64, FN = TN / 64;
  constexpr int NR = 2 * (FM + FN);                               // reads per half
  constexpr int NM = 2 * FM * FN * (sizeof(T) == 4 ? 4 : 1);      // MFMAs per half
  constexpr int NV = TM / 32 + TN / 32;                           // copies per step
  constexpr int NV1 = Stages<TM, TN, G>::kCount == 3 ? (NV + 1) / 2 : NV;
  static_assert(NM >= NR, "at least one MFMA per read");
  schedule_half<NM, NR, NV1, 0>();
  schedule_half<NM, NR, NV - NV1, 0>();
}

// Work-group barrier without the memory fence of __syncthreads(): that
// fence waits for every load in flight, including the copies meant to stay
// in flight across the barrier.  Every wait the LDS needs is explicit before
// each call.  S_BARRIER has side effects, so the scheduler keeps memory
// operations on their side of it; the empty asm does the same for the IR.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <typename T, int TM, int TN, int G, class Capture>
__device__ __forceinline__ void pipe_step(const char* Lg, const char* Rg, const DmaLoader<TM>& la,
                                          const DmaLoader<TN>& lb, int kt_copy, int kt_read, char* __restrict__ D,
                                          const char* __restrict__ P, const FragAddr& fa,
                                          FragSets<TM / 64, TN / 64>& fs, f32x16 (&acc)[TM / 64][TN / 64],
                                          Capture&& capture) {
  constexpr int FM = TM / 64, FN = TN / 64;
  constexpr int kOffR = TM * kRowBytes;
  la.issue(kt_copy, D);
  lb.issue(kt_copy, D + kOffR);
  load_frags<FM, FN>(P, P + kOffR, fa, 0, fs.f0);
  load_frags<FM, FN>(P, P + kOffR, fa, 1, fs.f1);
  mma_frags<T, FM, FN>(fs.f2, acc);
  mma_frags<T, FM, FN>(fs.f3, acc);
  load_frags<FM, FN>(P, P + kOffR, fa, 2, fs.f2);
  load_frags<FM, FN>(P, P + kOffR, fa, 3, fs.f3);
  mma_frags<T, FM, FN>(fs.f0, acc);
  mma_frags<T, FM, FN>(fs.f1, acc);
  schedule_step<T, TM, TN, G>();
  // Extra LDS reads of k-tile kt_read (stage P) for the caller; the wait
  // below completes them before the next step's copies overwrite P.
  capture(kt_read, P, fa);
  // With three stages the copy just issued may stay in flight (it lands in
  // a stage read two steps later); the one issued a step ago must be
  // complete.
  if constexpr (Stages<TM, TN, G>::kCount == 3)
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(TM / 32 + TN / 32));
  else
    __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
}

// acc += L-tile * R-tile^T over k-tiles [kt0, kt1) (acc is initialized by the
// caller).  On return every copy has landed and all waves have passed a
// barrier after their last LDS read, so the stage buffers may be reused.
// `after_copies` runs right after the prologue's copies are issued and
// issues `extra_loads` more vector-memory loads per thread (the epilogue
// operand's prefetch, 0 when there is none); the first wait counts them, so
// they do not delay the first k-tile.  capture(kt, sL, fa) runs once per
// k-tile while k-tile kt is in LDS, with sL the L operand's base in its
// stage and fa the wave's fragment-row offsets; its LDS reads complete
// before the stage is reused.
template <typename T, int TM, int TN, int kExtraLoads, int G, class AfterCopies, class Capture>
__device__ __forceinline__ void mainloop(const char* Lg, int64_t ldl_bytes, const char* Rg, int64_t ldr_bytes,
                                         int kt0, int kt1, Acc<T, TM, TN>& acc, bool extra_loads,
                                         AfterCopies&& after_copies, Capture&& capture) {
  constexpr int FM = TM / 64, FN = TN / 64;
  constexpr int kOffR = TM * kRowBytes;
  constexpr int kDma = TM / 32 + TN / 32;  // copy instructions per k-tile per wave
  using S = Stages<TM, TN, G>;
  constexpr int NS = S::kCount;
  static_assert((TM + TN) * kRowBytes <= S::kBytes, "stage too small");
  const int w = threadIdx.x >> 6;
  const int wr = (w >> 1) * (TM / 2), wc = (w & 1) * (TN / 2);
  if (kt1 <= kt0) {
    after_copies();
    return;
  }
  const int klast = kt1 - 1;
  auto clamp = [klast](int k) { return k < klast ? k : klast; };

  FragAddr fa;
  fa.init(wr, wc);
  DmaLoader<TM> la;
  DmaLoader<TN> lb;
  la.init(Lg, ldl_bytes);
  lb.init(Rg, ldr_bytes);

  // Prologue: k-tiles kt0, kt0+1 (and kt0+2 with three stages), clamped,
  // into stages 0, 1 (and 2), then the MFMAs of substeps 0 and 1 of kt0.
  la.issue(kt0, S::s0());
  lb.issue(kt0, S::s0() + kOffR);
  la.issue(clamp(kt0 + 1), S::s1());
  lb.issue(clamp(kt0 + 1), S::s1() + kOffR);
  if constexpr (NS == 3) {
    la.issue(clamp(kt0 + 2), S::s2());
    lb.issue(clamp(kt0 + 2), S::s2() + kOffR);
  }
  after_copies();
  // Loads complete in order: wait for the first k-tile only.
  static_assert((NS - 1) * kDma + kExtraLoads <= 63, "vmcnt has 6 bits");
  if (extra_loads)
    __builtin_amdgcn_s_waitcnt(wait_vm((NS - 1) * kDma + kExtraLoads));
  else
    __builtin_amdgcn_s_waitcnt(wait_vm((NS - 1) * kDma));
  lds_barrier();
  FragSets<FM, FN> fs;
  {
    const char* s0 = S::s0();
    load_frags<FM, FN>(s0, s0 + kOffR, fa, 0, fs.f0);
    load_frags<FM, FN>(s0, s0 + kOffR, fa, 1, fs.f1);
    load_frags<FM, FN>(s0, s0 + kOffR, fa, 2, fs.f2);
    load_frags<FM, FN>(s0, s0 + kOffR, fa, 3, fs.f3);
  }
  mma_frags<T, FM, FN>(fs.f0, acc.v);
  mma_frags<T, FM, FN>(fs.f1, acc.v);
  capture(kt0, S::s0(), fa);
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((NS - 2) * kDma));
  lds_barrier();

  // Step t copies k-tile t + NS into the stage of k-tile t and reads k-tile
  // t + 1 from the next stage.  With three stages the loop is unrolled by
  // three so that every step names its stages directly (the compiler then
  // sees that a step's reads and its copies touch different objects).
  auto step = [&](int t, char* D, const char* P) {
    pipe_step<T, TM, TN, G>(Lg, Rg, la, lb, clamp(t + NS), t + 1, D, P, fa, fs, acc.v, capture);
  };
  if constexpr (NS == 3) {
    int t = kt0;
    for (; t + 3 <= klast; t += 3) {
      step(t, S::s0(), S::s1());
      step(t + 1, S::s1(), S::s2());
      step(t + 2, S::s2(), S::s0());
    }
    if (t < klast) step(t++, S::s0(), S::s1());
    if (t < klast) step(t, S::s1(), S::s2());
  } else {
    for (int t = kt0; t < klast; ++t) {
      const bool odd = (t - kt0) & 1;
      step(t, odd ? S::s1() : S::s0(), odd ? S::s0() : S::s1());
    }
  }
  mma_frags<T, FM, FN>(fs.f2, acc.v);
  mma_frags<T, FM, FN>(fs.f3, acc.v);
  // The last copies (clamped repeats) must land before the caller reuses
  // LDS.
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
}

// ---------------------------------------------------------------------------
// Kernel arguments.
// ---------------------------------------------------------------------------
template <typename T>
struct SymArgs {
  const T* L;        // n x K, row stride ldk
  const T* R;        // n x K, row stride ldk
  const T* E;        // null when beta == 0, else L itself (ldn == ldk)
  T* C;              // n x n (ldn)
  T* C2;             // optional second output: C + delta * I on rows < n_real
  int64_t sL, sR, sE, sC, sC2;  // batch strides in elements
  int ldk, ldn;      // row strides in elements
  int K;             // multiple of the k-tile
  int tiles;         // n / tile edge
  int n_real;
  int batch;         // matrices (read by the persistent kernel)
  float alpha_unused;
  float beta, gamma, delta;
  // Per-matrix device flags of the guarded Gram iteration (null otherwise),
  // each read at index bz * flag_stride.  gate: the tile is computed only
  // when (gate != 0) == gate_want.  c2_gate: C2 is written only when it is
  // set.  xsel: when set, L and R are taken x_alt elements further on (the
  // other X buffer).
  const int32_t* gate;
  const int32_t* c2_gate;
  const int32_t* xsel;
  int64_t x_alt;
  int32_t gate_want, flag_stride;
  int stream_out;  // 1: the launcher takes the build with non-temporal stores (see store16)
};

// A guarded launch computes matrix bz's tiles only when its flag matches.
__device__ __forceinline__ bool gated_off(const int32_t* gate, int32_t want, int32_t stride, int bz) {
  return gate && ((gate[(int64_t)bz * stride] != 0) != (want != 0));
}
__device__ __forceinline__ bool flag_set(const int32_t* f, int32_t stride, int bz) {
  return f && f[(int64_t)bz * stride] != 0;
}

template <typename T, typename OutT>
struct NTArgs {
  const T* B;        // n x n (ldb), left operand
  const T* XT;       // X^T: m x n (ldxt), right operand
  const T* E;        // X: n x m (lde), or null when alpha == 0
  OutT* Y;           // output (internal: n x m, ld ldy; final: the caller's matrix)
  T* YT;             // optional second internal output Y^T: m x n (ldyt)
  int64_t sB, sXT, sE, sY, sYT;  // batch strides in elements
  int ldb, ldxt, lde, ldyt;
  int64_t ldy;
  int K;             // = n padded
  int tiles_m, tiles_n;
  int batch;         // matrices (read by the persistent kernel)
  int n_real, m_real;  // valid output rows/cols (wide orientation)
  int transpose_out;   // final output: write element (i, j) to Y[j * ldy + i]
  int final_out;       // 1: bounds-checked store in OutT with out_scale
  float alpha, gamma, out_scale;
  int accumulate;      // final output only: 0 stores the result; 1: Y <- Y + apply_scale * result
  float apply_scale;
  int32_t* d_status;    // optional status word: status_bits ORed in on NaN / Inf
  int32_t status_bits;
  // Guarded Gram iteration (see SymArgs): gate as there; when xsel is set,
  // X^T is read xt_alt elements further on and Y / Y^T are written y_alt /
  // yt_alt elements before (the two X buffers swap roles).
  const int32_t* gate;
  const int32_t* xsel;
  int64_t xt_alt, y_alt, yt_alt;
  int32_t gate_want, flag_stride;
  // Grouped call (final output only): matrix bz of the batch is written to
  // members[bz].data with leading dimension members[bz].ld, transposed when
  // members[bz].transposed; Y, sY, ldy and transpose_out are then unused.
  const ns_matrix* members;
  int stream_out;  // 1: the launcher takes the build with non-temporal stores (see store16)
};

// Ors `bits` into the status word once per wave in which some lane saw a
// bad value.
__device__ __forceinline__ void report_status(int32_t* d_status, int32_t bits, bool bad) {
  const unsigned long long any_bad = __ballot(bad);
  if (any_bad && (int)(threadIdx.x & 63) == __ffsll(any_bad) - 1) atomicOr(d_status, bits);
}

// One 16-byte store of an epilogue, non-temporal in the STREAM builds.  The
// launcher takes those when one launch writes more than the MALL holds: the
// output would not stay cached for the next kernel anyway and only displaces
// operands still in use.  Same-box A/B: the 128-expert MoE batch 3.0 %
// (Gram form) and 2.4 % (standard) faster per call; non-temporal stores in
// every launch made a 2048 x 8192 call, whose 8 MB state does stay cached,
// 17 % slower, and 48 matrices of 768 x 768 7 % slower.
// The choice is a template argument of the kernel build (STREAM): behind a
// run-time test of each store the compiler merged the two stores into one
// plain store, and an epilogue instantiated for both kinds in one build
// spilled in the two-work-groups-per-CU kernels.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
template <bool STREAM>
__device__ __forceinline__ void store16(void* dst, const uint4& v) {
  if constexpr (STREAM) {
    const u32x4_t t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(dst));
  } else {
    *reinterpret_cast<uint4*>(dst) = v;
  }
}


// The caller's 16-byte chunk `dst` gets `val` (kEC rounded results), or
// with `acc`, dst + s * val computed in fp32 and rounded once more.
template <bool STREAM, typename OutT>
__device__ __forceinline__ void final_chunk(OutT* dst, uint4 val, int acc, float s) {
  if (acc) {
    constexpr int kEC = 16 / (int)sizeof(OutT);
    const uint4 old = *reinterpret_cast<const uint4*>(dst);
    const OutT* o = reinterpret_cast<const OutT*>(&old);
    OutT* v = reinterpret_cast<OutT*>(&val);
#pragma unroll
    for (int e = 0; e < kEC; ++e) v[e] = from_f32<OutT>(fmaf(s, to_f32<OutT>(v[e]), to_f32<OutT>(o[e])));
  }
  store16<STREAM>(dst, val);
}
template <typename OutT>
__device__ __forceinline__ void final_elem(OutT* dst, OutT val, int acc, float s) {
  *dst = acc ? from_f32<OutT>(fmaf(s, to_f32<OutT>(val), to_f32<OutT>(*dst))) : val;
}

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

// Upper-triangle tiles in bands of kTriBand tile rows; within a band the
// list runs along the columns, the band's rows fastest, so a contiguous piece
// of the list (an XCD's share) covers the band's few row panels and a run of
// column panels: at 22 x 22 tiles at most 14 distinct panels per XCD, against
// up to 22 when the rows are listed one after another.
constexpr int kTriBand = 4;
__device__ __forceinline__ void tri_tile(int idx, int nt, int& tm, int& tn) {
  int r0 = 0;
  for (;;) {
    const int h = nt - r0 < kTriBand ? nt - r0 : kTriBand;
    const int tri = h * (h + 1) / 2;               // columns r0 .. r0+h-1 hold 1 .. h tiles
    const int band = tri + h * (nt - r0 - h);      // the columns right of them h each
    if (idx < band) {
      if (idx < tri) {
        int j = 0;
        while ((j + 1) * (j + 2) / 2 <= idx) ++j;  // column r0 + j
        tn = r0 + j;
        tm = r0 + idx - j * (j + 1) / 2;
      } else {
        const int q = idx - tri;
        tn = r0 + h + q / h;
        tm = r0 + q % h;
      }
      return;
    }
    idx -= band;
    r0 += h;
  }
}

// Full tile grids (the update) in groups of kGroupRows tile rows: within a
// group the list runs down the columns, tile row fastest, so the 32 or so
// work-groups an XCD runs at a time cover a 4 x 8 block of tiles and share
// 4 row panels of B and 8 row panels of X^T in its L2.
constexpr int kGroupRows = 4;
__device__ __forceinline__ void grouped_tile(int idx, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kGroupRows * tiles_n;
  const int g = idx / per_group, within = idx % per_group;
  const int rows = tiles_m - g * kGroupRows < kGroupRows ? tiles_m - g * kGroupRows : kGroupRows;
  tn = within / rows;
  tm = g * kGroupRows + within % rows;
}

// Output tile staged in LDS (the stage buffers are free after the main
// loop): TM rows of TN elements, each row at a power-of-two stride of
// kRowB bytes (kSlots 16-byte slots, the first kCPR of them used), 16-byte
// chunk q of row r at slot q ^ tswz(r).  The swizzle keeps both the
// row-quad writes from the accumulators (32 consecutive rows) and the
// block reads of the transposed stores (the same chunk of rows 8 apart) on
// distinct chunks.
// The tile spans the first two stage buffers: rows [0, kRowsPerStage) in
// the first, the rest in the second.
template <typename T, int TM, int TN, int G>
struct TileLds {
  using S = Stages<TM, TN, G>;
  static constexpr int kRowData = TN * (int)sizeof(T);
  static constexpr int kRowB = kRowData <= 256 ? 256 : 512;
  static constexpr int kSlots = kRowB / 16;
  static constexpr int kCPR = kRowData / 16;       // chunks per row
  static constexpr int kEC = 16 / (int)sizeof(T);  // elements per chunk
  static constexpr int kS = kSlots == 32 ? 5 : 4;
  static constexpr int kRowsPerStage = S::kBytes / kRowB;
  static_assert(kRowData <= 512, "tile row must fit in 512 bytes");
  static_assert(TM <= 2 * kRowsPerStage, "tile must fit in the two stage buffers");
  static __device__ __forceinline__ int tswz(int r) { return (r ^ (r >> kS)) & (kSlots - 1); }
  static __device__ __forceinline__ char* row_base(int r) {
    return r < kRowsPerStage ? S::s0() + r * kRowB : S::s1() + (r - kRowsPerStage) * kRowB;
  }
  static __device__ __forceinline__ char* at(int r, int col) {
    return row_base(r) + (((col / kEC) ^ tswz(r)) << 4) + (col % kEC) * (int)sizeof(T);
  }
  static __device__ __forceinline__ char* chunk(int r, int c) { return row_base(r) + ((c ^ tswz(r)) << 4); }
  // The kEC x kEC block of tile rows rb*kEC.. and columns cb*kEC.., read as
  // kEC row chunks and transposed in registers: out[e] is column cb*kEC + e
  // of the block, kEC consecutive tile rows in one 16-byte chunk (chunk rb
  // of row cb*kEC + e of the transposed tile).
  static __device__ __forceinline__ void block_t(int rb, int cb, uint4 (&out)[kEC]) {
    uint32_t in[kEC][4];
#pragma unroll
    for (int i = 0; i < kEC; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(chunk(rb * kEC + i, cb));
      in[i][0] = v.x;
      in[i][1] = v.y;
      in[i][2] = v.z;
      in[i][3] = v.w;
    }
#pragma unroll
    for (int c = 0; c < kEC; ++c) {
      uint32_t d[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (sizeof(T) == 2) {
          // Word k of the column holds rows 2k and 2k+1: the low or high
          // halves of word c/2 of those two rows.
          const uint32_t a = in[2 * k][c >> 1], b = in[2 * k + 1][c >> 1];
          d[k] = (c & 1) ? (a >> 16) | (b & 0xffff0000u) : (a & 0xffffu) | (b << 16);
        } else {
          d[k] = in[k][c];
        }
      }
      out[c] = uint4{d[0], d[1], d[2], d[3]};
    }
  }
};

template <typename T, int TM, int TN>
__device__ __forceinline__ void acc_zero(Acc<T, TM, TN>& acc) {
#pragma unroll
  for (int fm = 0; fm < Acc<T, TM, TN>::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < Acc<T, TM, TN>::FN; ++fn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.v[fm][fn][v] = 0.f;
}

// The epilogue's E operand (the "alpha E +" / "beta E +" term) in the
// accumulator layout: lane (lr, h) of wave (wr, wc) needs E[il][jl..jl+3]
// for il = wr + 32 fm + lr, jl = wc + 32 fn + 8 g + 4 h.  Tiles up to 192
// have the registers to hold it (8 bytes per (fm, fn, g)) through the main
// loop, so it never sits between the last MFMA and the stores; the 256 tile
// loads it in the epilogue.  E is always one of the operands in LDS: the
// symmetric products take it from L's k-tiles col0 / 64 .. (col0 + TN) / 64
// (capture), the update, where E = X and R = X^T, from R's k-tiles row0 / 64
// .. (row0 + TM) / 64, transposed (capture_t).  So it costs no HBM reads and
// does not hold up the first k-tile.  The update kernels built without the
// capture load E from global memory before the main loop instead (load).
template <typename T, int TM, int TN>
struct EPrefetch {
  static constexpr int FM = TM / 64, FN = TN / 64;
  static constexpr bool kEnabled = FM * FN <= 9 && sizeof(T) == 2;
  static constexpr int kLoads = kEnabled ? FM * FN * 4 : 0;  // vector loads per thread
  uint2 v[kEnabled ? FM : 1][kEnabled ? FN : 1][4];
  __device__ __forceinline__ void load(const T* E, int64_t ld, int64_t row0, int64_t col0) {
    if constexpr (kEnabled) {
      if (!E) return;
      const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
      const int lr = lane & 31, h = lane >> 5;
      const int wr = (w >> 1) * (TM / 2), wc = (w & 1) * (TN / 2);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            v[fm][fn][g] = *reinterpret_cast<const uint2*>(E + (row0 + wr + fm * 32 + lr) * ld + col0 + wc +
                                                           fn * 32 + 8 * g + 4 * h);
    }
  }
  // Before capture: columns in k-tiles past the contraction are never
  // captured and stay zero (they are the zero padding of E).
  __device__ __forceinline__ void zero() {
    if constexpr (kEnabled) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int g = 0; g < 4; ++g) v[fm][fn][g] = uint2{0u, 0u};
    }
  }
  // E = L: this thread's values from the L operand's k-tile kt in LDS (base
  // sL, rows of the tile at kRowBytes each), if kt holds some of its
  // columns; kb is the first k-tile of the tile's column block (col0 / 64
  // for 16-bit T).  Row il = wr + 32 fm + lr sits at fa.row0L + 32 fm
  // kRowBytes with the chunk swizzle fa.swL0 / fa.swL1 (even / odd fm), as
  // for the fragment reads.
  __device__ __forceinline__ void capture(int kt, const char* sL, int kb, const FragAddr& fa) {
    if constexpr (kEnabled) {
      const int d = kt - kb;
      if (d < 0 || d >= TN / 64) return;
      const int w = threadIdx.x >> 6, h = (threadIdx.x & 63) >> 5;
      const int wc = (w & 1) * (TN / 2);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int jd = wc + fn * 32 + 8 * g - 64 * d;  // column inside k-tile kt (uniform per wave)
          if (jd < 0 || jd >= 64) continue;
          const int c = jd >> 3;
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) {
            const int sw = (fm & 1) ? fa.swL1 : fa.swL0;
            v[fm][fn][g] = *reinterpret_cast<const uint2*>(sL + fa.row0L + fm * 32 * kRowBytes + ((c ^ sw) << 4) +
                                                           8 * h);
          }
        }
    }
  }
  // E = R^T (the update: E = X, R = X^T): this thread's values from the R
  // operand's k-tile kt in LDS (base sR, rows of the tile's R panel at
  // kRowBytes each), if kt holds some of its rows; kb is the first k-tile
  // of the tile's row block (row0 / 64).  E[il][jl + e] = R[jl + e][il]:
  // one 2-byte read per element, from R rows jl .. jl + 3 at k-column
  // il - 64 (kt - kb).  A 32-row group of il lies in one k-tile, so the
  // test is uniform per wave.  Row r = wc + 32 fn + 8 g + 4 h + e has
  // swz(r) = (4 h + e) ^ ((wc / 8 + 4 fn + g) & 7) with wc / 8 = 0 or 4
  // (mod 8), so a chunk index xor swz(r) is a per-thread part xor the
  // constant e ^ ((4 fn + g) & 7): eight address registers, recomputed from
  // d at each capture rather than held through the main loop.
  __device__ __forceinline__ void capture_t(int kt, const char* sR, int kb) {
    if constexpr (kEnabled) {
      static_assert(TN % 64 == 0, "wc / 8 must be 0 or 4 mod 8");
      const int d = kt - kb;
      if (d < 0 || d >= TM / 64) return;
      const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
      const int lr = lane & 31, h = lane >> 5;
      const int wr = (w >> 1) * (TM / 2), wc = (w & 1) * (TN / 2);
      const char* rb = sR + (wc + 4 * h) * kRowBytes + (lr & 7) * 2;
      const int sx = (4 * h) ^ ((wc >> 3) & 7);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int i0 = wr + fm * 32 - 64 * d;  // k-column of lane group's row il = wr + 32 fm (uniform)
        if (i0 < 0 || i0 >= 64) continue;
        const int cx = ((i0 + lr) >> 3) ^ sx;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint32_t q[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int k = e ^ ((4 * fn + g) & 7);
              q[e] = *reinterpret_cast<const uint16_t*>(rb + (32 * fn + 8 * g + e) * kRowBytes + ((cx ^ k) << 4));
            }
            v[fm][fn][g] = uint2{q[0] | (q[1] << 16), q[2] | (q[3] << 16)};
          }
      }
    }
  }
  // E[il][jl..jl+3] as floats: from the registers, or loaded now.
  __device__ __forceinline__ f32x4 get(const T* E, int64_t ld, int64_t row0, int64_t col0, int il, int jl, int fm,
                                       int fn, int g) const {
    if constexpr (kEnabled) {
      const T* e = reinterpret_cast<const T*>(&v[fm][fn][g]);
      return f32x4{to_f32<T>(e[0]), to_f32<T>(e[1]), to_f32<T>(e[2]), to_f32<T>(e[3])};
    } else {
      return Quad<T>::load(E + (row0 + il) * ld + col0 + jl);
    }
  }
};

// A 16-byte chunk of T elements with elements k < e taken from `lo` and the
// others from `up` (word masks, so the chunks stay in registers).
template <typename T>
__device__ __forceinline__ uint4 merge_below(uint4 lo, uint4 up, int e) {
  const uint32_t l[4] = {lo.x, lo.y, lo.z, lo.w}, u[4] = {up.x, up.y, up.z, up.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t m;
    if constexpr (sizeof(T) == 2)
      m = (2 * i < e ? 0x0000ffffu : 0u) | (2 * i + 1 < e ? 0xffff0000u : 0u);
    else
      m = i < e ? 0xffffffffu : 0u;
    o[i] = (l[i] & m) | (u[i] & ~m);
  }
  return uint4{o[0], o[1], o[2], o[3]};
}

// The chunk v with element k replaced by d.
template <typename T>
__device__ __forceinline__ uint4 with_elem(uint4 v, int k, T d) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t bits = __builtin_bit_cast(uint16_t, d);
      const uint32_t lo = 2 * i == k ? bits : (w[i] & 0xffffu);
      const uint32_t hi = 2 * i + 1 == k ? bits : (w[i] >> 16);
      w[i] = lo | (hi << 16);
    } else {
      if (i == k) w[i] = __builtin_bit_cast(uint32_t, d);
    }
  }
  return uint4{w[0], w[1], w[2], w[3]};
}

// One upper-triangle tile (tm <= tn) of matrix bz of a symmetric product.
// EXT: the build that reads the extended arguments (the guarded Gram
// iteration's device flags; for updates also the member table of a grouped
// call); other launches take the build without that code (it changed the
// schedule of the products enough to cost 6 % of a call).
template <typename T, int TILE, int G, bool EXT, bool STREAM>
__device__ __forceinline__ void sym_tile(const SymArgs<T>& p, int tm, int tn, int bz) {
  using A = Acc<T, TILE, TILE>;
  constexpr int FM = A::FM, FN = A::FN;
  using TL = TileLds<T, TILE, TILE, G>;
  const int64_t ldk_bytes = (int64_t)p.ldk * sizeof(T);
  int64_t xo = 0;
  if constexpr (EXT) {
    if (gated_off(p.gate, p.gate_want, p.flag_stride, bz)) return;
    xo = flag_set(p.xsel, p.flag_stride, bz) ? p.x_alt : 0;
  }
  const char* Lg = reinterpret_cast<const char*>(p.L + bz * p.sL + xo) + (int64_t)tm * TILE * ldk_bytes;
  const char* Rg = reinterpret_cast<const char*>(p.R + bz * p.sR + xo) + (int64_t)tn * TILE * ldk_bytes;
  constexpr int BK = kRowBytes / sizeof(T);
  const T* E = p.E ? p.E + bz * p.sE : nullptr;
  T* C = p.C + bz * p.sC;
  T* C2 = p.C2 ? p.C2 + bz * p.sC2 : nullptr;
  if constexpr (EXT) {
    if (p.c2_gate && !flag_set(p.c2_gate, p.flag_stride, bz)) C2 = nullptr;
  }
  const bool diag_tile = (tm == tn);
  static_assert(TILE * sizeof(T) <= sizeof(g_c2_diag), "C2 diagonal buffer");
  T* c2d = reinterpret_cast<T*>(g_c2_diag);
  const int64_t row0 = (int64_t)tm * TILE, col0 = (int64_t)tn * TILE;
  // E is null or the L operand (SymArgs), so its tile rows are L's tile
  // rows and its columns col0.. are L's k-tiles from col0 / BK on.
  using EP = EPrefetch<T, TILE, TILE>;
  EP ep;
  ep.zero();
  A acc;
  acc_zero(acc);
  const int kb = (int)(col0 / BK);
  mainloop<T, TILE, TILE, 0, G>(Lg, ldk_bytes, Rg, ldk_bytes, 0, p.K / BK, acc, false, [] {},
                                [&](int kt, const char* sL, const FragAddr& fa) {
                                  if (E) ep.capture(kt, sL, kb, fa);
                                });

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 31, h = lane >> 5;
  const int wr = (w >> 1) * (TILE / 2), wc = (w & 1) * (TILE / 2);

  // Phase A: beta*E + gamma*acc, rounded to T, into the LDS tile.  The
  // diagonal of C2 (= C + delta I on real rows) is written here, rounded
  // once from fp32.  (Non-finite results are found by a separate scan of
  // the output when the caller asks for it: a check here slowed the
  // products down by 7 %, status word or not.)
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int il = wr + fm * 32 + lr;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int jl = wc + fn * 32 + 8 * g + 4 * h;
        f32x4 v;
        v[0] = p.gamma * acc.v[fm][fn][4 * g + 0];
        v[1] = p.gamma * acc.v[fm][fn][4 * g + 1];
        v[2] = p.gamma * acc.v[fm][fn][4 * g + 2];
        v[3] = p.gamma * acc.v[fm][fn][4 * g + 3];
        if (E) v += p.beta * ep.get(E, p.ldn, row0, col0, il, jl, fm, fn, g);
        Quad<T>::store(reinterpret_cast<T*>(TL::at(il, jl)), v);
        if (C2 && diag_tile) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (il == jl + e) c2d[il] = from_f32<T>(v[e] + p.delta);
        }
      }
    }
  }
  __syncthreads();

  constexpr int kChunks = TILE * TL::kCPR;
  constexpr int EC = TL::kEC;
  constexpr int kB = TL::kCPR;  // EC x EC blocks along a tile edge
  constexpr int kBlocks = kB * kB;
  static_assert(kChunks % kThreads == 0, "whole chunks per thread");
  // Phase B: rows of the tile.  Every thread handles the same number of
  // chunks, so the loop is unrolled and its LDS reads overlap.  A diagonal
  // tile takes every element from its upper triangle, so the stored matrix
  // is exactly symmetric: here it writes only the chunks right of its
  // diagonal blocks, and phase C the rest.
  constexpr bool S = STREAM;
#pragma unroll 6
  for (int it = 0; it < kChunks / kThreads; ++it) {
    const int q = it * kThreads + threadIdx.x;
    const int r = q / TL::kCPR, c = q % TL::kCPR;
    if (!diag_tile || c > r / EC) {
      const uint4 val = *reinterpret_cast<const uint4*>(TL::chunk(r, c));
      store16<S>(C + (row0 + r) * p.ldn + col0 + c * EC, val);
      if (C2) store16<S>(C2 + (row0 + r) * p.ldn + col0 + c * EC, val);
    }
  }

  // Phase C: the mirrored tile, C[col0 + j][row0 + i] = tile[i][j], from
  // EC x EC blocks transposed in registers.  Block (rb, cb) gives chunk rb of
  // mirrored rows cb*EC .. cb*EC + EC - 1; consecutive threads take
  // consecutive rb, so each mirrored row is written as adjacent chunks.  On
  // a diagonal tile the mirror of each upper block (rb < cb) is the lower
  // block (cb, rb); a diagonal block (rb == cb) is written once, its row e
  // taking the elements left of the diagonal from its transpose and the
  // rest as staged, and C2's copy takes the diagonal element from phase A
  // (real rows).  Blocks below the diagonal are not read.
#pragma unroll 1
  for (int it = 0; it < (kBlocks + kThreads - 1) / kThreads; ++it) {
    const int q = it * kThreads + threadIdx.x;
    const int rb = q % kB, cb = q / kB;
    if ((kBlocks % kThreads == 0 || q < kBlocks) && !(diag_tile && rb > cb)) {
      uint4 cols[EC];
      TL::block_t(rb, cb, cols);
      const bool on_diag = diag_tile && rb == cb;
      if (on_diag) {
#pragma unroll
        for (int e = 0; e < EC; ++e)
          cols[e] = merge_below<T>(cols[e], *reinterpret_cast<const uint4*>(TL::chunk(rb * EC + e, cb)), e);
      }
#pragma unroll
      for (int e = 0; e < EC; ++e) {
        const int64_t off = (col0 + cb * EC + e) * p.ldn + row0 + rb * EC;
        store16<S>(C + off, cols[e]);
        if (C2) {
          const int rr = rb * EC + e;
          store16<S>(C2 + off, on_diag && row0 + rr < p.n_real ? with_elem<T>(cols[e], e, c2d[rr]) : cols[e]);
        }
      }
    }
  }
}

// Position of work-group b in a persistent grid of G work-groups (G a
// multiple of 8): XCD x = b % 8 takes the contiguous piece
// [x G/8, (x+1) G/8) of every G consecutive list positions.
__device__ __forceinline__ int persistent_piece(int b, int G) { return (b % kXcds) * (G / kXcds) + b / kXcds; }

// GRAM_INPUT only separates the X X^T launches (inner dimension m) from the
// n x n products into their own kernel symbol, so profiles list them apart.
// One work-group per upper-triangle tile.
template <typename T, int TILE, bool GRAM_INPUT, int G = 1, bool EXT = false, bool STREAM = false>
__global__ void __launch_bounds__(kThreads, G) k_sym(SymArgs<T> p) {
  const int ntri = p.tiles * (p.tiles + 1) / 2;
  int tm, tn;
  tri_tile(gridDim.y == 1 ? xcd_order(blockIdx.x, ntri) : blockIdx.x, p.tiles, tm, tn);
  sym_tile<T, TILE, G, EXT, STREAM>(p, tm, tn, blockIdx.y);
}

// Persistent form: a grid of work-groups looping over the tiles of all
// matrices in list order, so one tile's stores drain while the next one
// starts.  A kernel of its own: the loop's live state would push the 256
// tile past the register file.
template <typename T, int TILE, bool GRAM_INPUT, int G = 1, bool EXT = false, bool STREAM = false>
__global__ void __launch_bounds__(kThreads, G) k_sym_loop(SymArgs<T> p) {
  const int ntri = p.tiles * (p.tiles + 1) / 2;
  const int total = ntri * p.batch, groups = gridDim.x, piece = persistent_piece(blockIdx.x, groups);
  for (int base = 0; base + piece < total; base += groups) {
    const int pos = base + piece, bz = pos / ntri;
    int tm, tn;
    tri_tile(pos % ntri, p.tiles, tm, tn);
    sym_tile<T, TILE, G, EXT, STREAM>(p, tm, tn, bz);
    lds_barrier();  // the next tile's copies reuse the LDS the epilogue read
  }
}

// Y = alpha E + gamma B (X^T)^T on TM x TN tiles: the update of both forms.
// CAP: E is taken from the X^T panel in LDS during the main loop; otherwise
// it is loaded from global memory before the main loop (or absent).
template <typename T, typename OutT, int TM, int TN, int G, bool CAP, bool EXT, bool STREAM>
__device__ __forceinline__ void nt_tile(const NTArgs<T, OutT>& p, int tm, int tn, int bz) {
  using A = Acc<T, TM, TN>;
  constexpr int FM = A::FM, FN = A::FN;
  using TL = TileLds<OutT, TM, TN, G>;
  const int64_t ldb_bytes = (int64_t)p.ldb * sizeof(T);
  const int64_t ldxt_bytes = (int64_t)p.ldxt * sizeof(T);
  bool swap = false;
  if constexpr (EXT) {
    if (gated_off(p.gate, p.gate_want, p.flag_stride, bz)) return;
    swap = flag_set(p.xsel, p.flag_stride, bz);
  }
  const char* Lg = reinterpret_cast<const char*>(p.B + bz * p.sB) + (int64_t)tm * TM * ldb_bytes;
  const char* Rg =
      reinterpret_cast<const char*>(p.XT + bz * p.sXT + (swap ? p.xt_alt : 0)) + (int64_t)tn * TN * ldxt_bytes;
  constexpr int BK = kRowBytes / sizeof(T);
  const T* E = p.E ? p.E + bz * p.sE : nullptr;
  OutT* Y = p.Y + bz * p.sY - (swap ? p.y_alt : 0);
  T* YT = p.YT ? p.YT + bz * p.sYT - (swap ? p.yt_alt : 0) : nullptr;
  int64_t ldy = p.ldy;
  int transpose_out = p.transpose_out;
  if constexpr (EXT) {
    if (p.members) {
      const ns_matrix mb = p.members[bz];
      Y = reinterpret_cast<OutT*>(mb.data);
      ldy = mb.ld;
      transpose_out = mb.transposed;
    }
  }
  const int64_t row0 = (int64_t)tm * TM, col0 = (int64_t)tn * TN;
  using EP = EPrefetch<T, TM, TN>;
  EP ep;
  A acc;
  acc_zero(acc);
  if constexpr (CAP) {
    // E is X and the R operand X^T, so E's tile is the transpose of the R
    // panel's k-tiles row0 / BK .. (row0 + TM) / BK, taken from LDS as they
    // pass (rows past the contraction are X's zero padding).
    ep.zero();
    const int kb = (int)(row0 / BK);
    mainloop<T, TM, TN, 0, G>(Lg, ldb_bytes, Rg, ldxt_bytes, 0, p.K / BK, acc, false, [] {},
                              [&](int kt, const char* sL, const FragAddr&) {
                                if constexpr (EP::kEnabled) {
                                  // E is set whenever CAP is; without the test the
                                  // 192 tile's schedule spills registers.
                                  if (E) ep.capture_t(kt, sL + TM * kRowBytes, kb);
                                }
                              });
  } else {
    // E-free updates (the Gram form) take this path.  Its schedule is the
    // one measured fastest for them; built without these E registers the
    // 192 tile ran 40 % slower.
    mainloop<T, TM, TN, EP::kLoads, G>(Lg, ldb_bytes, Rg, ldxt_bytes, 0, p.K / BK, acc, EP::kLoads > 0 && E,
                                       [&] { ep.load(E, p.lde, row0, col0); },
                                       [](int, const char*, const FragAddr&) {});
  }

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 31, h = lane >> 5;
  const int wr = (w >> 1) * (TM / 2), wc = (w & 1) * (TN / 2);
  const float scale = p.final_out ? p.out_scale : 1.f;
  bool bad = false;

  // Phase A: alpha*E + gamma*acc (times the output scale), rounded to OutT,
  // into the LDS tile.
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int il = wr + fm * 32 + lr;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int jl = wc + fn * 32 + 8 * g + 4 * h;
        f32x4 v;
        v[0] = p.gamma * acc.v[fm][fn][4 * g + 0];
        v[1] = p.gamma * acc.v[fm][fn][4 * g + 1];
        v[2] = p.gamma * acc.v[fm][fn][4 * g + 2];
        v[3] = p.gamma * acc.v[fm][fn][4 * g + 3];
        if (E) v += p.alpha * ep.get(E, p.lde, row0, col0, il, jl, fm, fn, g);
        v *= scale;
        if (p.d_status) {
#pragma unroll
          for (int e = 0; e < 4; ++e) bad |= !(fabsf(v[e]) < kRoundsToInf<OutT>);
        }
        Quad<OutT>::store(reinterpret_cast<OutT*>(TL::at(il, jl)), v);
      }
    }
  }
  __syncthreads();

  constexpr int kEC = TL::kEC;
  constexpr int kChunks = TM * TL::kCPR;  // row chunks of the tile
  static_assert(kChunks % kThreads == 0, "whole chunks per thread");
  // EC x EC blocks for the transposed stores (see TileLds::block_t): block
  // q covers tile rows rb*kEC.. and columns cb*kEC.., consecutive threads
  // take consecutive rb, so a transposed row is written as adjacent chunks.
  constexpr int kRB = TM / kEC, kBlocks = kRB * TL::kCPR;
  constexpr int kBIters = (kBlocks + kThreads - 1) / kThreads;
  constexpr bool S = STREAM;
  if (!p.final_out) {
    // Internal buffers: the whole padded tile, rows of Y and, when asked,
    // rows of Y^T (columns of the tile).
#pragma unroll 6
    for (int it = 0; it < kChunks / kThreads; ++it) {
      const int q = it * kThreads + threadIdx.x;
      const int r = q / TL::kCPR, c = q % TL::kCPR;
      store16<S>(Y + (row0 + r) * ldy + col0 + c * kEC, *reinterpret_cast<const uint4*>(TL::chunk(r, c)));
    }
    if (YT) {
#pragma unroll 1
      for (int it = 0; it < kBIters; ++it) {
        const int q = it * kThreads + threadIdx.x;
        if (kBlocks % kThreads == 0 || q < kBlocks) {
          const int rb = q % kRB, cb = q / kRB;
          uint4 cols[kEC];
          TL::block_t(rb, cb, cols);
#pragma unroll
          for (int e = 0; e < kEC; ++e)
            store16<S>(YT + (col0 + cb * kEC + e) * p.ldyt + row0 + rb * kEC, cols[e]);
        }
      }
    }
  } else if (!transpose_out) {
    // Caller's matrix, same orientation: rows i < n_real, columns j < m_real.
    const bool vec = (ldy % kEC) == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0;
#pragma unroll 6
    for (int it = 0; it < kChunks / kThreads; ++it) {
      const int q = it * kThreads + threadIdx.x;
      const int r = q / TL::kCPR, c = q % TL::kCPR;
      const int64_t i = row0 + r, j0 = col0 + c * kEC;
      if (i >= p.n_real || j0 >= p.m_real) continue;
      const uint4 val = *reinterpret_cast<const uint4*>(TL::chunk(r, c));
      OutT* dst = Y + i * ldy + j0;
      if (vec && j0 + kEC <= p.m_real) {
        final_chunk<S>(dst, val, p.accumulate, p.apply_scale);
      } else {
        const OutT* vals = reinterpret_cast<const OutT*>(&val);
        for (int e = 0; e < kEC && j0 + e < p.m_real; ++e) final_elem(dst + e, vals[e], p.accumulate, p.apply_scale);
      }
    }
  } else {
    // Caller's matrix is the transpose: its row j holds tile column j, in
    // TM / kEC chunks of kEC tile rows.
    const bool vec = (ldy % kEC) == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0;
#pragma unroll 1
    for (int it = 0; it < kBIters; ++it) {
      const int q = it * kThreads + threadIdx.x;
      if (kBlocks % kThreads != 0 && q >= kBlocks) continue;
      const int rb = q % kRB, cb = q / kRB;
      const int64_t i0 = row0 + rb * kEC;
      if (i0 >= p.n_real) continue;
      uint4 cols[kEC];
      TL::block_t(rb, cb, cols);
#pragma unroll
      for (int e = 0; e < kEC; ++e) {
        const int64_t j = col0 + cb * kEC + e;
        if (j >= p.m_real) continue;
        OutT* dst = Y + j * ldy + i0;
        if (vec && i0 + kEC <= p.n_real) {
          final_chunk<S>(dst, cols[e], p.accumulate, p.apply_scale);
        } else {
          const OutT* vals = reinterpret_cast<const OutT*>(&cols[e]);
          for (int k = 0; k < kEC && i0 + k < p.n_real; ++k) final_elem(dst + k, vals[k], p.accumulate, p.apply_scale);
        }
      }
    }
  }
  if (p.d_status) report_status(p.d_status, p.status_bits, bad);
}

// One work-group per tile on a one-dimensional grid over the tiles of all
// matrices: the list (matrix by matrix, each in grouped_tile order) is cut
// into one contiguous piece per XCD.
template <typename T, typename OutT, int TM, int TN, int G = 1, bool CAP = false, bool EXT = false,
          bool STREAM = false>
__global__ void __launch_bounds__(kThreads, G) k_nt(NTArgs<T, OutT> p) {
  const int per = p.tiles_m * p.tiles_n;
  const int pos = xcd_order(blockIdx.x, per * p.batch);
  int tm, tn;
  grouped_tile(pos % per, p.tiles_m, p.tiles_n, tm, tn);
  nt_tile<T, OutT, TM, TN, G, CAP, EXT, STREAM>(p, tm, tn, pos / per);
}

// Persistent form of k_nt (see k_sym_loop).
template <typename T, typename OutT, int TM, int TN, int G = 1, bool CAP = false, bool EXT = false,
          bool STREAM = false>
__global__ void __launch_bounds__(kThreads, G) k_nt_loop(NTArgs<T, OutT> p) {
  const int per = p.tiles_m * p.tiles_n;
  const int total = per * p.batch, groups = gridDim.x, piece = persistent_piece(blockIdx.x, groups);
  for (int base = 0; base + piece < total; base += groups) {
    const int pos = base + piece, bz = pos / per;
    int tm, tn;
    grouped_tile(pos % per, p.tiles_m, p.tiles_n, tm, tn);
    nt_tile<T, OutT, TM, TN, G, CAP, EXT, STREAM>(p, tm, tn, bz);
    lds_barrier();  // the next tile's copies reuse the LDS the epilogue read
  }
}

}  // namespace nsk
