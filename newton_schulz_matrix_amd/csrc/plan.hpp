// plan.hpp - host side of libnsortho shared by its translation units: the
// plan of a call (shapes, tile edge, workspace layout), the kernel
// launchers and the launch sequence of both Newton-Schulz forms.  api.hip
// holds the C entry points; the product launchers (and with them the
// kernel builds) are instantiated in kern_*.hip.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <math.h>

#include <algorithm>
#include <string>
#include <vector>
#include <stdint.h>
#include <string.h>

#include "../../include/nsortho.h"
#include "products.hpp"
#include "stage.hpp"

namespace nsr {

using namespace nsk;

constexpr size_t kAlign = 256;
// Per-matrix flags of the guarded Gram iteration: X buffer selector and one
// restart flag per step.
constexpr int kFlagStride = NS_MAX_STEPS + 2;
constexpr int kPrescaleExp16 = 10;  // X is held as 2^10 * X in 16-bit storage
constexpr int kMaxPartials = 1024;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

inline int elem_size(ns_dtype d) { return d == NS_FP32 ? 4 : 2; }

// A launch of the two-work-groups-per-CU kernels (the large batches) that
// writes more than this many bytes takes their build with non-temporal
// stores (the MI355X MALL holds 256 MiB; see store16).
constexpr double kStreamOutBytes = 256.0 * 1024 * 1024;
inline int stream_out(double written_bytes) { return written_bytes > kStreamOutBytes ? 1 : 0; }

// Shapes and workspace layout of one call.
struct Plan {
  int64_t rows = 0, cols = 0, n = 0, m = 0, n_pad = 0, m_pad = 0;
  int64_t batch = 1;
  bool transposed = false;
  int tile = 256;    // edge of the square tiles of the products
  int tile_n = 256;  // columns of the update tiles (the padding of m)
  ns_dtype io = NS_BF16, internal = NS_FP16;
  ns_mode mode = NS_STANDARD;
  int esz = 2;
  int partials = 1;
  int nn_count = 2;
  int64_t x_elems = 0, nn_elems = 0;
  size_t off_partial = 0, off_scale = 0, off_flags = 0, off_x[2] = {0, 0}, off_xt[2] = {0, 0}, off_nn[4] = {0, 0, 0, 0};
  size_t total = 0;
};

// Columns of the update tiles that go with a square tile edge: square tiles
// (192 x 256 update tiles were measured slower than 192 x 192 at 4096 x 14336).
constexpr int nn_tile_n(int edge) { return edge; }

// Products run on fp16 operands for 16-bit input and on fp32 operands for
// fp32 input.  bf16 operands are refused: with 8 mantissa bits in every
// stored intermediate the iteration misses the 1e-2 relative error bar of
// 16-bit input on ordinary shapes (the Gram-NS article's stabilized
// iteration keeps float16 in its key steps for this reason).
inline bool resolve_internal(ns_dtype io, const ns_options* opt, ns_dtype* out) {
  const int req = opt ? opt->internal : -1;
  if (io == NS_FP32) {
    if (req != -1 && req != NS_FP32) return false;
    *out = NS_FP32;
    return true;
  }
  if (io != NS_BF16 && io != NS_FP16) return false;
  if (req == -1 || req == NS_FP16) {
    *out = NS_FP16;
    return true;
  }
  return false;
}

// Tile edge.  fp32 products use 128 (a larger fp32 tile does not fit in
// LDS).  For 16-bit products the edge (128, 192 or 256) minimizes a cost
// estimate of one call: work-group waves over the 256 compute units times
// the time of one work-group, in units of one 256-edge k-tile, with the
// per-k-tile and fixed (prologue and epilogue) costs measured on MI355X with
// random operands.
// Smaller tiles lose MFMA efficiency (more LDS reads per MFMA) but fill the
// chip when a product has few tiles.
struct TileCost {
  int edge;
  double sym_ktile, sym_fixed, nn_ktile, nn_fixed;
};
// The 256 tile has room for only two LDS stages (64 KiB each), so its
// copies run one k-tile ahead instead of two; measured on 4096 x 14336,
// 5120 x 17920, 8192 x 8192 and 8192 x 28672 it takes 2.0-2.1 us per k-tile
// against 0.95 us for the 192 tile (1.78 times the work), and the automatic
// choice never takes it where the 192 tile fits.
constexpr TileCost kTileCosts[] = {
    {128, 0.45, 8.0, 0.45, 9.0},
    {192, 0.67, 13.0, 0.67, 14.0},
    {256, 1.41, 18.0, 1.48, 20.0},
};
constexpr double kComputeUnits = 256.0;
// Launches of short contractions with more tiles than CUs run persistent
// (see launch_sym); measured, that cuts their per-tile fixed cost to about
// this fraction.
constexpr double kPersistentFixed = 0.6;

// True when a product with `tiles` tiles (all matrices) and `ktiles` k-tiles
// per tile runs as a persistent grid.
constexpr int kPersistentGroups = 256;
constexpr int kPersistentMaxKtiles = 48;
inline bool use_persistent(int edge, int64_t tiles, int64_t ktiles) {
  return edge <= 192 && tiles > kPersistentGroups && ktiles <= kPersistentMaxKtiles;
}

// Launches that take the two-work-groups-per-CU kernels (16-bit, 128 tiles,
// at least 512 tiles; see use_pair): per pair of tiles on a CU, measured on
// MI355X against the table above on the 128 x 1408 x 2048 expert batch.
constexpr double kPairKtile = 0.79, kPairSymFixed = 4.9, kPairNnFixed = 5.7;

inline bool use_pair(int edge, int esz, int64_t tiles);

inline double product_estimate(int edge, double tiles, double ktiles, double per_ktile, double fixed,
                        double pair_fixed) {
  if (use_pair(edge, 2, (int64_t)tiles)) return ceil(tiles / (2 * kComputeUnits)) * (ktiles * kPairKtile + pair_fixed);
  const double waves = ceil(tiles / kComputeUnits);
  if (use_persistent(edge, (int64_t)tiles, (int64_t)ktiles)) fixed *= kPersistentFixed;
  return waves * (ktiles * per_ktile + fixed);
}

inline double tile_estimate(const TileCost& c, int64_t n, int64_t m, int64_t batch, ns_mode mode) {
  const int64_t n_pad = round_up(n, c.edge), tn = nn_tile_n(c.edge), m_pad = round_up(m, tn);
  const double nt = (double)(n_pad / c.edge), b = (double)batch;
  const double sym_tiles = nt * (nt + 1) / 2 * b, nn_tiles = nt * (double)(m_pad / tn) * b;
  const double kn = ceil((double)n / 64), km = ceil((double)m / 64);  // contractions stop at the real size
  const double sym = product_estimate(c.edge, sym_tiles, kn, c.sym_ktile, c.sym_fixed, kPairSymFixed);
  const double gram = product_estimate(c.edge, sym_tiles, km, c.sym_ktile, c.sym_fixed, kPairSymFixed);
  const double nn = product_estimate(c.edge, nn_tiles, kn, c.nn_ktile, c.nn_fixed, kPairNnFixed);
  // Launch counts of five steps: standard 5 X X^T, 5 n x n, 5 updates; Gram
  // (one restart) 2 X X^T, about 14 n x n products and 2 updates.
  return mode == NS_GRAM ? 2 * gram + 14 * sym + 2 * nn : 5 * (gram + sym + nn);
}

// Index math: tile counts and leading dimensions are 32-bit, and a copy
// instruction's per-lane offset within a k-tile panel (at most 64 rows of a
// row of m_pad elements) must fit in 32 bits.
inline bool padding_fits(int64_t n_pad, int64_t m_pad, int esz) {
  return n_pad <= 65536 && m_pad * esz <= (int64_t(1) << 25);
}

// fp32 products: 128 tiles, or 64 when the n x n products would not fill
// the chip with one wave of 128 tiles (small matrices, where a launch
// otherwise keeps a handful of compute units busy).
inline int pick_tile_fp32(int64_t n, int64_t batch) {
  const int64_t t = (n + 127) / 128, ntri = t * (t + 1) / 2;
  return ntri * batch < (int64_t)kComputeUnits ? 64 : 128;
}

inline int pick_tile(int64_t n, int64_t m, int64_t batch, ns_dtype internal, ns_mode mode) {
  if (internal == NS_FP32) return pick_tile_fp32(n, batch);
  int best = 128;
  double best_t = 0.0;
  for (const TileCost& c : kTileCosts) {
    if (c.edge != 128 && !padding_fits(round_up(n, c.edge), round_up(m, nn_tile_n(c.edge)), elem_size(internal)))
      continue;
    const double t = tile_estimate(c, n, m, batch, mode);
    if (c.edge == 128 || t < best_t) {
      best = c.edge;
      best_t = t;
    }
  }
  return best;
}

inline ns_status make_plan(int64_t rows, int64_t cols, int64_t batch, ns_dtype io, ns_mode mode, const ns_options* opt,
                    Plan* p) {
  if (rows < 1 || cols < 1 || batch < 1 || batch > 65535) return NS_ERR_INVALID_ARG;
  if (mode != NS_STANDARD && mode != NS_GRAM) return NS_ERR_INVALID_ARG;
  if (io != NS_BF16 && io != NS_FP16 && io != NS_FP32) return NS_ERR_UNSUPPORTED_DTYPE;
  ns_dtype internal;
  if (!resolve_internal(io, opt, &internal)) return NS_ERR_UNSUPPORTED_DTYPE;
  p->rows = rows;
  p->cols = cols;
  p->batch = batch;
  p->io = io;
  p->internal = internal;
  p->mode = mode;
  p->transposed = rows > cols;
  p->n = p->transposed ? cols : rows;
  p->m = p->transposed ? rows : cols;
  const int req_tile = opt ? opt->tile : 0;
  if (req_tile != 0 && !(req_tile == 128 || (internal != NS_FP32 && (req_tile == 192 || req_tile == 256)) ||
                         (internal == NS_FP32 && req_tile == 64)))
    return NS_ERR_INVALID_ARG;
  p->tile = req_tile ? req_tile : pick_tile(p->n, p->m, batch, internal, mode);
  p->tile_n = nn_tile_n(p->tile);
  p->n_pad = round_up(p->n, p->tile);
  p->m_pad = round_up(p->m, p->tile_n);
  p->esz = elem_size(internal);
  p->x_elems = p->n_pad * p->m_pad;
  p->nn_elems = p->n_pad * p->n_pad;
  if (!padding_fits(p->n_pad, p->m_pad, p->esz)) return NS_ERR_INVALID_ARG;
  // The update's grid is one-dimensional over the tiles of all matrices (the
  // bound is taken at the smallest tile edge, so it holds for every plan).
  if (batch * ((p->n + 127) / 128) * ((p->m + 127) / 128) > INT32_MAX) return NS_ERR_INVALID_ARG;
  // About 2048 norm blocks in total, at most one per input row.
  const int64_t want = (2048 + batch - 1) / batch;
  p->partials = (int)std::min<int64_t>(std::min<int64_t>(want, rows), kMaxPartials);
  p->nn_count = mode == NS_GRAM ? 4 : 2;
  size_t off = 0;
  p->off_partial = off;
  off = align_up(off + (size_t)batch * p->partials * sizeof(double));
  p->off_scale = off;
  off = align_up(off + (size_t)batch * sizeof(float));
  p->off_flags = off;
  off = align_up(off + (size_t)batch * kFlagStride * sizeof(int32_t));
  for (int i = 0; i < 2; ++i) {
    p->off_x[i] = off;
    off = align_up(off + (size_t)batch * p->x_elems * p->esz);
    p->off_xt[i] = off;
    off = align_up(off + (size_t)batch * p->x_elems * p->esz);
  }
  for (int i = 0; i < p->nn_count; ++i) {
    p->off_nn[i] = off;
    off = align_up(off + (size_t)batch * p->nn_elems * p->esz);
  }
  p->total = off;
  return NS_OK;
}

inline ns_status hip_status(hipError_t e) { return e == hipSuccess ? NS_OK : NS_ERR_HIP; }

// Brackets launches with the caller's events when a trace is attached.
// Start and stop events of one traced launch.  They are handed to
// hipExtLaunchKernel, which binds them to the kernel's own dispatch: no
// marker packets of their own go into the stream between kernels (two
// hipEventRecord calls around a launch cost about 5 us of idle GPU each).
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, LaunchEvents ev,
                         Args... args) {
  hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
  return hipGetLastError();
}

// Runs launch(LaunchEvents) for one kernel launch and records it in the
// caller's trace when its kind is selected.
struct Tracer {
  ns_trace* t;
  hipStream_t st;
  template <class F>
  hipError_t run(ns_kernel_kind kind, double flops, double bytes, F&& launch) const {
    const bool rec = t && t->events && ((t->kind_mask >> (int)kind) & 1u) && t->count >= 0 &&
                     t->count < t->capacity;
    const int i = rec ? t->count : -1;
    LaunchEvents ev;
    if (rec) {
      ev.start = reinterpret_cast<hipEvent_t>(t->events[2 * i]);
      ev.stop = reinterpret_cast<hipEvent_t>(t->events[2 * i + 1]);
    }
    hipError_t e;
    if ((e = launch(ev)) != hipSuccess) return e;
    if (rec) {
      if (t->kinds) t->kinds[i] = (int32_t)kind;
      if (t->flops) t->flops[i] = flops;
      if (t->bytes) t->bytes[i] = bytes;
      t->count = i + 1;
    }
    return hipSuccess;
  }
};

// ---------------------------------------------------------------------------
// Kernel launchers.
// ---------------------------------------------------------------------------
// A launch with more tiles than compute units and a short contraction (at
// most kPersistentMaxKtiles k-tiles, where start-up and epilogue weigh most)
// runs as a persistent grid of kPersistentGroups work-groups (one per CU of
// MI355X) that loop over the tiles, so one tile's stores drain while the
// next one starts; other launches get one work-group per tile.  The 256 tile
// has no persistent kernel (its registers are full).  16-bit products on 128
// tiles with at least two work-groups' worth of tiles per CU use the kernels
// built for two work-groups per CU (two LDS stages), where one work-group's
// start-up and epilogue overlap the other's main loop; the update's loop
// kernel does not fit that register budget, so it runs one work-group per
// tile.  Correctness does not depend on the CU count.
template <typename T, int TILE>
constexpr bool kHasPairKernels = TILE == 128 && sizeof(T) == 2;

inline bool use_pair(int edge, int esz, int64_t tiles) {
  return edge == 128 && esz == 2 && tiles >= 2 * (int64_t)kPersistentGroups;
}

// The kernel build a product launch takes: one work-group per tile or a
// persistent grid, for one or two work-groups per compute unit.
enum class Form { kTile, kLoop, kPairTile, kPairLoop };

inline Form sym_form(int edge, int esz, int64_t tiles, int64_t ktiles) {
  if (use_pair(edge, esz, tiles)) return use_persistent(edge, tiles, ktiles) ? Form::kPairLoop : Form::kPairTile;
  if (edge <= 192 && use_persistent(edge, tiles, ktiles)) return Form::kLoop;
  return Form::kTile;
}

inline Form nt_form(int edge, int esz, int64_t tiles, int64_t ktiles) {
  if (use_pair(edge, esz, tiles)) return Form::kPairTile;
  if (edge <= 192 && use_persistent(edge, tiles, ktiles)) return Form::kLoop;
  return Form::kTile;
}

template <typename T, int TILE, bool GRAM_INPUT, bool EXT>
hipError_t launch_sym_g(SymArgs<T> a, int64_t batch, hipStream_t s, LaunchEvents ev) {
  const int64_t ntri = (int64_t)a.tiles * (a.tiles + 1) / 2;
  const int ktiles = a.K / (kRowBytes / (int)sizeof(T));
  const dim3 tiles_grid((unsigned)ntri, (unsigned)batch);
  a.batch = (int)batch;
  switch (sym_form(TILE, (int)sizeof(T), ntri * batch, ktiles)) {
    case Form::kPairLoop:
      if constexpr (kHasPairKernels<T, TILE>) {
        if constexpr (!EXT)
          if (a.stream_out)
            return launch_kernel(k_sym_loop<T, TILE, GRAM_INPUT, 2, false, true>, dim3(2 * kPersistentGroups),
                                 dim3(kThreads), s, ev, a);
        return launch_kernel(k_sym_loop<T, TILE, GRAM_INPUT, 2, EXT>, dim3(2 * kPersistentGroups), dim3(kThreads), s,
                             ev, a);
      }
      break;
    case Form::kPairTile:
      if constexpr (kHasPairKernels<T, TILE>) {
        if constexpr (!EXT)
          if (a.stream_out)
            return launch_kernel(k_sym<T, TILE, GRAM_INPUT, 2, false, true>, tiles_grid, dim3(kThreads), s, ev, a);
        return launch_kernel(k_sym<T, TILE, GRAM_INPUT, 2, EXT>, tiles_grid, dim3(kThreads), s, ev, a);
      }
      break;
    case Form::kLoop:
      if constexpr (TILE <= 192)
        return launch_kernel(k_sym_loop<T, TILE, GRAM_INPUT, 1, EXT>, dim3(kPersistentGroups), dim3(kThreads), s, ev,
                             a);
      break;
    case Form::kTile:
      return launch_kernel(k_sym<T, TILE, GRAM_INPUT, 1, EXT>, tiles_grid, dim3(kThreads), s, ev, a);
  }
  return hipErrorInvalidConfiguration;
}

// Launches that read the guard's device flags take the kernels built for
// them.
template <typename T, int TILE, bool GRAM_INPUT>
hipError_t launch_sym(SymArgs<T> a, int64_t batch, hipStream_t s, LaunchEvents ev) {
  if (a.gate || a.c2_gate || a.xsel) return launch_sym_g<T, TILE, GRAM_INPUT, true>(a, batch, s, ev);
  return launch_sym_g<T, TILE, GRAM_INPUT, false>(a, batch, s, ev);
}

template <typename T, typename OutT, int TILE, bool CAP, bool EXT>
hipError_t launch_nt_g(NTArgs<T, OutT> a, int64_t batch, hipStream_t s, LaunchEvents ev) {
  constexpr int TN = nn_tile_n(TILE);
  const int64_t per = (int64_t)a.tiles_m * a.tiles_n;
  const dim3 flat((unsigned)(per * batch));
  a.batch = (int)batch;
  switch (nt_form(TILE, (int)sizeof(T), per * batch, a.K / (kRowBytes / (int)sizeof(T)))) {
    case Form::kPairTile:
      if constexpr (kHasPairKernels<T, TILE>) {
        if constexpr (!EXT)
          if (a.stream_out)
            return launch_kernel(k_nt<T, OutT, TILE, TN, 2, CAP, false, true>, flat, dim3(kThreads), s, ev, a);
        return launch_kernel(k_nt<T, OutT, TILE, TN, 2, CAP, EXT>, flat, dim3(kThreads), s, ev, a);
      }
      break;
    case Form::kLoop:
      if constexpr (TILE <= 192)
        return launch_kernel(k_nt_loop<T, OutT, TILE, TN, 1, CAP, EXT>, dim3(kPersistentGroups), dim3(kThreads), s,
                             ev, a);
      break;
    case Form::kTile:
      return launch_kernel(k_nt<T, OutT, TILE, TN, 1, CAP, EXT>, flat, dim3(kThreads), s, ev, a);
    case Form::kPairLoop:
      break;
  }
  return hipErrorInvalidConfiguration;
}

template <typename T, typename OutT, int TILE, bool CAP>
hipError_t launch_nt_cap(NTArgs<T, OutT> a, int64_t batch, hipStream_t s, LaunchEvents ev) {
  return launch_nt_g<T, OutT, TILE, CAP, false>(a, batch, s, ev);
}

// Updates with an E term (the standard form) take the kernels that capture
// E from LDS, where the tile has the registers for it; E-free updates (the
// Gram form) and the other tiles take the kernels without the capture.
template <typename T, typename OutT, int TILE>
hipError_t launch_nt(NTArgs<T, OutT> a, int64_t batch, hipStream_t s, LaunchEvents ev) {
  // Launches with extended arguments (guard flags, a grouped call's member
  // table) take the kernels built to read them.
  const bool ext = a.gate || a.xsel || a.members;
  if constexpr (EPrefetch<T, TILE, nn_tile_n(TILE)>::kEnabled) {
    if (a.E)
      return ext ? launch_nt_g<T, OutT, TILE, true, true>(a, batch, s, ev)
                 : launch_nt_cap<T, OutT, TILE, true>(a, batch, s, ev);
  }
  return ext ? launch_nt_g<T, OutT, TILE, false, true>(a, batch, s, ev)
             : launch_nt_cap<T, OutT, TILE, false>(a, batch, s, ev);
}

// Device flags a launch of the guarded Gram iteration reads (see SymArgs):
// compute only where the flag at `gate` equals `want`, write C2 only where
// the flag at `c2` is set, and take the X buffers through the selector.
struct Gate {
  const int32_t* gate = nullptr;
  int32_t want = 0;
  const int32_t* c2 = nullptr;
  bool xsel = false;
};

// One Newton-Schulz run over a batch, for internal type T and I/O type IO.
template <typename T, typename IO>
struct Runner {
  const Plan& p;
  char* ws;
  hipStream_t st;
  IO* user;                  // input, read by the norm and staging passes
  int64_t ld, bstride;
  IO* out;                   // written by the final epilogue
  int64_t out_ld, out_bstride;
  const ns_matrix* members;  // grouped call: the members' layouts (device), else null
  bool accumulate;           // false: out = result; true: out += apply * result
  float apply;
  const ns_options* opt;
  Tracer tr;

  T* xbuf(int i) const { return reinterpret_cast<T*>(ws + p.off_x[i]); }
  int32_t* status() const { return opt ? opt->d_status : nullptr; }
  int32_t* flags() const { return reinterpret_cast<int32_t*>(ws + p.off_flags); }
  // Length of a contraction over `real` rows or columns: a whole number of
  // k-tiles (64 16-bit or 32 fp32 elements).
  static int64_t k_extent(int64_t real) { return round_up(real, kRowBytes / (int64_t)sizeof(T)); }
  T* xtbuf(int i) const { return reinterpret_cast<T*>(ws + p.off_xt[i]); }
  T* nnbuf(int i) const { return reinterpret_cast<T*>(ws + p.off_nn[i]); }

  // C = beta*E + gamma * L R^T on upper tiles, mirrored.  L and R are the
  // X buffers (K = m_pad) or n x n buffers (K = n_pad).  E is null or L
  // (the kernels take E's tile from L's k-tiles).
  template <int TILE>
  hipError_t sym(const T* L, const T* R, int K, int ldk, const T* E, float beta, float gamma, T* C, T* C2,
                 float delta, const Gate& g = Gate{}) const {
    if (E && E != L) return hipErrorInvalidValue;
    SymArgs<T> a{};
    a.L = L;
    a.R = R;
    a.E = E;
    a.C = C;
    a.C2 = C2;
    // X X^T reads an X buffer (stride n_pad * m_pad); the others read n x n
    // buffers.
    const bool gram = (L == xbuf(0) || L == xbuf(1));
    const int64_t xs = gram ? p.x_elems : p.nn_elems;
    a.sL = xs;
    a.sR = xs;
    a.sE = p.nn_elems;
    a.sC = p.nn_elems;
    a.sC2 = p.nn_elems;
    a.ldk = ldk;
    a.ldn = (int)p.n_pad;
    a.K = K;
    a.tiles = (int)(p.n_pad / TILE);
    a.n_real = (int)p.n;
    a.alpha_unused = 0.f;
    a.beta = beta;
    a.gamma = gamma;
    a.delta = delta;
    a.gate = g.gate;
    a.gate_want = g.want;
    a.c2_gate = g.c2;
    a.xsel = g.xsel ? flags() : nullptr;
    a.x_alt = xbuf(1) - xbuf(0);
    a.flag_stride = kFlagStride;
    a.stream_out = stream_out((double)p.batch * (double)p.nn_elems * sizeof(T) * (C2 ? 2.0 : 1.0));
    const double n = (double)p.n, bt = (double)p.batch, es = sizeof(T);
    const double inner = gram ? (double)p.m : n;
    const double flops = n * n * inner * bt;
    double bytes = (L == R ? 1.0 : 2.0) * n * inner * es + n * n * es * (1.0 + (E ? 1.0 : 0.0) + (C2 ? 1.0 : 0.0));
    bytes *= bt;
    hipError_t e =
        gram ? tr.run(NS_KERNEL_GRAM, flops, bytes, [&](LaunchEvents ev) { return launch_sym<T, TILE, true>(a, p.batch, st, ev); })
             : tr.run(NS_KERNEL_SYM, flops, bytes, [&](LaunchEvents ev) { return launch_sym<T, TILE, false>(a, p.batch, st, ev); });
    if (e != hipSuccess) return e;
    if ((e = check_state(C)) != hipSuccess) return e;
    return C2 ? check_state(C2) : hipSuccess;
  }

  // With a status word, scans a freshly written n x n buffer (all matrices
  // of the batch, padding included: it is zero) for NaN and Inf.
  hipError_t check_state(const T* C) const {
    if (!status()) return hipSuccess;
    const int64_t count = p.nn_elems;
    const bool vec = (count * (int64_t)sizeof(T)) % 16 == 0;
    const int64_t want = (count * p.batch + 4095) / 4096;  // about 16 elements per thread
    const unsigned gx = (unsigned)std::max<int64_t>(1, std::min<int64_t>((want + p.batch - 1) / p.batch, 1024));
    hipLaunchKernelGGL(k_check_finite<T>, dim3(gx, (unsigned)p.batch), dim3(kStageThreads), 0, st, C, count,
                       p.nn_elems, vec ? 1 : 0, status(), (int32_t)(NS_ERR_NONFINITE | NS_STATUS_AT_STATE));
    return hipGetLastError();
  }

  // Y = alpha * X_in + B X_in into X_out and X_out^T (E omitted when alpha
  // is 0).
  template <int TILE>
  hipError_t nn_internal(const T* B, int xin, bool with_e, float alpha, int xout, const Gate& g = Gate{}) const {
    NTArgs<T, T> a{};
    a.B = B;
    a.XT = xtbuf(xin);
    a.E = with_e ? xbuf(xin) : nullptr;
    a.Y = xbuf(xout);
    a.YT = xtbuf(xout);
    a.sB = p.nn_elems;
    a.sXT = p.x_elems;
    a.sE = p.x_elems;
    a.sY = p.x_elems;
    a.sYT = p.x_elems;
    a.ldb = (int)p.n_pad;
    a.ldxt = (int)p.n_pad;
    a.lde = (int)p.m_pad;
    a.ldyt = (int)p.n_pad;
    a.ldy = p.m_pad;
    a.K = (int)k_extent(p.n);
    a.tiles_m = (int)(p.n_pad / TILE);
    a.tiles_n = (int)(p.m_pad / nn_tile_n(TILE));
    a.n_real = (int)p.n;
    a.m_real = (int)p.m;
    a.transpose_out = 0;
    a.final_out = 0;
    a.accumulate = 0;
    a.apply_scale = 0.f;
    a.alpha = alpha;
    a.gamma = 1.f;
    a.out_scale = 1.f;
    a.d_status = status();
    a.status_bits = NS_ERR_NONFINITE | NS_STATUS_AT_ITERATE;
    a.gate = g.gate;
    a.gate_want = g.want;
    a.xsel = g.xsel ? flags() : nullptr;
    a.xt_alt = xtbuf(1) - xtbuf(0);
    a.y_alt = xbuf(1) - xbuf(0);
    a.yt_alt = xtbuf(1) - xtbuf(0);
    a.flag_stride = kFlagStride;
    a.stream_out = stream_out(2.0 * (double)p.batch * (double)p.x_elems * sizeof(T));
    const double n = (double)p.n, m = (double)p.m, bt = (double)p.batch, es = sizeof(T);
    const double bytes = bt * (n * n * es + n * m * es * (3.0 + (with_e ? 1.0 : 0.0)));
    return tr.run(NS_KERNEL_UPDATE, 2.0 * n * n * m * bt, bytes,
                  [&](LaunchEvents ev) { return launch_nt<T, T, TILE>(a, p.batch, st, ev); });
  }

  // The caller's matrix = out_scale * (alpha * X_in + B X_in), oriented back.
  template <int TILE>
  hipError_t nn_final(const T* B, int xin, bool with_e, float alpha, float out_scale, const Gate& g = Gate{}) const {
    NTArgs<T, IO> a{};
    a.B = B;
    a.XT = xtbuf(xin);
    a.E = with_e ? xbuf(xin) : nullptr;
    a.Y = out;
    a.YT = nullptr;
    a.sB = p.nn_elems;
    a.sXT = p.x_elems;
    a.sE = p.x_elems;
    a.sY = out_bstride;
    a.sYT = 0;
    a.ldb = (int)p.n_pad;
    a.ldxt = (int)p.n_pad;
    a.lde = (int)p.m_pad;
    a.ldyt = 0;
    a.ldy = out_ld;
    a.accumulate = accumulate ? 1 : 0;
    a.apply_scale = apply;
    a.K = (int)k_extent(p.n);
    a.tiles_m = (int)(p.n_pad / TILE);
    a.tiles_n = (int)(p.m_pad / nn_tile_n(TILE));
    a.n_real = (int)p.n;
    a.m_real = (int)p.m;
    a.transpose_out = p.transposed ? 1 : 0;
    a.final_out = 1;
    a.alpha = alpha;
    a.gamma = 1.f;
    a.out_scale = out_scale;
    a.d_status = status();
    a.status_bits = NS_ERR_NONFINITE | NS_STATUS_AT_OUTPUT;
    a.gate = g.gate;
    a.gate_want = g.want;
    a.xsel = g.xsel ? flags() : nullptr;
    a.xt_alt = xtbuf(1) - xtbuf(0);
    a.y_alt = 0;
    a.yt_alt = 0;
    a.flag_stride = kFlagStride;
    a.members = members;
    a.stream_out = stream_out((double)p.batch * (double)p.rows * (double)p.cols * sizeof(IO));
    const double n = (double)p.n, m = (double)p.m, bt = (double)p.batch, es = sizeof(T);
    const double bytes = bt * (n * n * es + n * m * es * (1.0 + (with_e ? 1.0 : 0.0)) + n * m * sizeof(IO));
    return tr.run(NS_KERNEL_UPDATE, 2.0 * n * n * m * bt, bytes,
                  [&](LaunchEvents ev) { return launch_nt<T, IO, TILE>(a, p.batch, st, ev); });
  }

  hipError_t stage(float prescale, float eps) const {
    double* partial = reinterpret_cast<double*>(ws + p.off_partial);
    const bool vec_ok = (p.cols % (16 / sizeof(IO)) == 0) && (ld % (16 / sizeof(IO)) == 0) &&
                        ((reinterpret_cast<uintptr_t>(user) & 15) == 0) &&
                        (p.batch == 1 || bstride % (16 / sizeof(IO)) == 0);
    const double elems = (double)p.rows * (double)p.cols * (double)p.batch;
    hipError_t e = tr.run(NS_KERNEL_NORM, 0.0, elems * sizeof(IO), [&](LaunchEvents ev) {
      return launch_kernel((k_sumsq<IO>), dim3(p.partials, (unsigned)p.batch), dim3(kStageThreads), st, ev,
                           (const IO*)user, p.rows, p.cols, ld, bstride, vec_ok ? 1 : 0, partial, p.partials,
                           members);
    });
    if (e != hipSuccess) return e;
    float* scales = reinterpret_cast<float*>(ws + p.off_scale);
    hipLaunchKernelGGL(k_scale, dim3((unsigned)p.batch), dim3(kStageThreads), 0, st, partial, p.partials, prescale,
                       eps, scales, status(), (int32_t)(NS_ERR_NONFINITE | NS_STATUS_AT_INPUT));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return tr.run(NS_KERNEL_STAGE, 0.0, elems * (sizeof(IO) + 2 * sizeof(T)), [&](LaunchEvents ev) {
      const int bi = (int)(p.n_pad / 64), bj = (int)(p.m_pad / 64);
      return launch_kernel(k_stage_pair<IO, T>, dim3((unsigned)(bi * bj), (unsigned)p.batch), dim3(kStageThreads), st,
                           ev, (const IO*)user, p.rows, p.cols, ld, bstride, vec_ok ? 1 : 0, (const float*)scales,
                           xbuf(0), xtbuf(0), p.n_pad, p.m_pad, p.x_elems, p.transposed ? 1 : 0, bj, members);
    });
  }

  template <int TILE>
  hipError_t run(int steps, const float* a, const float* b, const float* c, float eps) const {
    const int pe = (sizeof(T) == 2) ? kPrescaleExp16 : 0;
    const float prescale = ldexpf(1.f, pe);
    const float unscale = ldexpf(1.f, -pe);
    const float gram_scale = ldexpf(1.f, -2 * pe);
    const int mp = (int)p.m_pad, np = (int)p.n_pad;
    // Contractions stop at the real size rounded up to the k-tile: the padded
    // rows and columns of X and of every n x n matrix are exactly zero.
    const int km = (int)k_extent(p.m), kn = (int)k_extent(p.n);
    hipError_t e = stage(prescale, eps);
    if (e != hipSuccess) return e;
    int xi = 0;
    if (p.mode == NS_STANDARD) {
      T* A = nnbuf(0);
      T* B = nnbuf(1);
      for (int k = 0; k < steps; ++k) {
        T* X = xbuf(xi);
        if ((e = sym<TILE>(X, X, km, mp, nullptr, 0.f, gram_scale, A, nullptr, 0.f)) != hipSuccess) return e;
        if ((e = sym<TILE>(A, A, kn, np, A, b[k], c[k], B, nullptr, 0.f)) != hipSuccess) return e;
        if (k + 1 < steps) {
          if ((e = nn_internal<TILE>(B, xi, true, a[k], xi ^ 1)) != hipSuccess) return e;
          xi ^= 1;
        } else {
          if ((e = nn_final<TILE>(B, xi, true, a[k], unscale)) != hipSuccess) return e;
        }
      }
      return hipSuccess;
    }
    if (opt && opt->guard_threshold > 0.f) return run_guarded<TILE>(steps, a, b, c, km, kn, mp, np, gram_scale, unscale);
    // Gram form.
    const uint32_t mask = opt ? opt->restart_mask : (1u << 4);
    T* R = nnbuf(0);
    T* Z = nnbuf(1);
    T* Qb[2] = {nnbuf(2), nnbuf(3)};
    int qi = 0;
    if ((e = sym<TILE>(xbuf(0), xbuf(0), km, mp, nullptr, 0.f, gram_scale, R, nullptr, 0.f)) != hipSuccess) return e;
    bool fresh = true;
    for (int k = 1; k <= steps; ++k) {
      if (k > 1 && ((mask >> k) & 1u)) {
        if ((e = nn_internal<TILE>(Qb[qi], xi, false, 0.f, xi ^ 1)) != hipSuccess) return e;
        xi ^= 1;
        if ((e = sym<TILE>(xbuf(xi), xbuf(xi), km, mp, nullptr, 0.f, gram_scale, R, nullptr, 0.f)) != hipSuccess)
          return e;
        fresh = true;
      }
      const float ak = a[k - 1], bk = b[k - 1], ck = c[k - 1];
      // Z' = b R + c R^2; at a fresh start Q = a I + Z' comes out of the same
      // epilogue.
      if ((e = sym<TILE>(R, R, kn, np, R, bk, ck, Z, fresh ? Qb[qi] : nullptr, ak)) != hipSuccess) return e;
      // The products below are taken as Q Z', R Z' and V Z' (equal to Z' Q,
      // Z' R and Z' V: all are polynomials in the same Gram matrix), so that
      // the epilogue's E operand is the left operand.
      if (!fresh) {
        if ((e = sym<TILE>(Qb[qi], Z, kn, np, Qb[qi], ak, 1.f, Qb[qi ^ 1], nullptr, 0.f)) != hipSuccess) return e;
        qi ^= 1;
      }
      fresh = false;
      const bool need_r = k < steps && !((mask >> (k + 1)) & 1u);
      if (need_r) {
        T* V = Qb[qi ^ 1];
        if ((e = sym<TILE>(R, Z, kn, np, R, ak, 1.f, V, nullptr, 0.f)) != hipSuccess) return e;
        if ((e = sym<TILE>(V, Z, kn, np, V, ak, 1.f, R, nullptr, 0.f)) != hipSuccess) return e;
      }
    }
    return nn_final<TILE>(Qb[qi], xi, false, 0.f, unscale);
  }

  // The Gram form with restarts on demand (ns_options.guard_threshold).
  // Every step k >= 2 has a possible restart; its kernels are always
  // enqueued and compute, matrix by matrix, only where the flag "restart
  // before step k" is set: by the fixed restart mask, or by the detector
  // after step k - 1.  The kernels on either side of a possible restart are
  // gated the other way (Q's product, R's update), and the fresh
  // Q = a I + Z' is written where the restart happened.  A restart writes X
  // into the other buffer pair; the per-matrix selector tells later
  // launches which pair holds X.  No host synchronization.
  template <int TILE>
  hipError_t run_guarded(int steps, const float* a, const float* b, const float* c, int km, int kn, int mp, int np,
                         float gram_scale, float unscale) const {
    const uint32_t mask = opt->restart_mask;
    const float theta = opt->guard_threshold;
    int32_t* f = flags();
    const int nf = (int)p.batch * kFlagStride;
    hipLaunchKernelGGL(k_guard_init, dim3((nf + 255) / 256), dim3(256), 0, st, f, (int)p.batch, kFlagStride, mask);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    T* R = nnbuf(0);
    T* Z = nnbuf(1);
    T* Qb[2] = {nnbuf(2), nnbuf(3)};
    int qi = 0;  // Qb[qi] holds Q after each step
    Gate sel;
    sel.xsel = true;
    if ((e = sym<TILE>(xbuf(0), xbuf(0), km, mp, nullptr, 0.f, gram_scale, R, nullptr, 0.f, sel)) != hipSuccess)
      return e;
    for (int k = 1; k <= steps; ++k) {
      const int32_t* fk = f + k;
      const float ak = a[k - 1], bk = b[k - 1], ck = c[k - 1];
      if (k > 1) {
        Gate rs;
        rs.gate = fk;
        rs.want = 1;
        rs.xsel = true;
        if ((e = nn_internal<TILE>(Qb[qi], 0, false, 0.f, 1, rs)) != hipSuccess) return e;
        hipLaunchKernelGGL(k_guard_flip, dim3(((unsigned)p.batch + 255) / 256), dim3(256), 0, st, f, (int)p.batch,
                           kFlagStride, k);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = sym<TILE>(xbuf(0), xbuf(0), km, mp, nullptr, 0.f, gram_scale, R, nullptr, 0.f, rs)) != hipSuccess)
          return e;
      }
      // Z' = b R + c R^2, with the fresh Q = a I + Z' where step k starts
      // from I (always at k = 1).
      Gate zg;
      zg.c2 = k > 1 ? fk : nullptr;
      if ((e = sym<TILE>(R, R, kn, np, R, bk, ck, Z, Qb[qi ^ 1], ak, zg)) != hipSuccess) return e;
      if (k > 1) {
        Gate qg;
        qg.gate = fk;
        qg.want = 0;
        if ((e = sym<TILE>(Qb[qi], Z, kn, np, Qb[qi], ak, 1.f, Qb[qi ^ 1], nullptr, 0.f, qg)) != hipSuccess) return e;
      }
      qi ^= 1;
      if (k < steps) {
        hipLaunchKernelGGL(k_guard_detect<T>, dim3((unsigned)p.batch), dim3(kStageThreads), 0, st, Qb[qi], R,
                           p.n_pad, p.nn_elems, (int)p.n, a[k], theta, f, kFlagStride, k + 1, status(),
                           (int32_t)(NS_STATUS_GUARD_RESTART | NS_STATUS_GUARD_STEP(k + 1)));
        if ((e = hipGetLastError()) != hipSuccess) return e;
        Gate rg;
        rg.gate = f + k + 1;
        rg.want = 0;
        T* V = Qb[qi ^ 1];
        if ((e = sym<TILE>(R, Z, kn, np, R, ak, 1.f, V, nullptr, 0.f, rg)) != hipSuccess) return e;
        if ((e = sym<TILE>(V, Z, kn, np, V, ak, 1.f, R, nullptr, 0.f, rg)) != hipSuccess) return e;
      }
    }
    return nn_final<TILE>(Qb[qi], 0, false, 0.f, unscale, sel);
  }
};

// The kernel builds a call launches, as text (see ns_plan_kernels): one
// entry per distinct build, in launch order.
inline const char* form_name(Form f) {
  switch (f) {
    case Form::kTile: return "tile";
    case Form::kLoop: return "loop";
    case Form::kPairTile: return "pair";
    case Form::kPairLoop: return "pairloop";
  }
  return "?";
}
inline const char* dtype_name(ns_dtype d) { return d == NS_FP32 ? "f32" : d == NS_FP16 ? "f16" : "bf16"; }

inline std::string describe_plan(const Plan& p, int steps, uint32_t mask, bool guard, bool grouped) {
  const int esz = p.esz;
  const int64_t per_k = kRowBytes / esz;
  const int64_t km = round_up(p.m, per_k) / per_k, kn = round_up(p.n, per_k) / per_k;
  const int64_t nt = p.n_pad / p.tile, ntri = nt * (nt + 1) / 2 * p.batch;
  const int64_t nt_tiles = nt * (p.m_pad / p.tile_n) * p.batch;
  const std::string T = dtype_name(p.internal), IO = dtype_name(p.io), E = std::to_string(p.tile);
  // Updates with an E term capture it from LDS where the tile has the
  // registers (16-bit, edges up to 192), else read it from global memory.
  const std::string e_term = esz == 2 && p.tile <= 192 ? ",E" : ",Eg";
  const Form fx = sym_form(p.tile, esz, ntri, km), fn = sym_form(p.tile, esz, ntri, kn),
             fu = nt_form(p.tile, esz, nt_tiles, kn);
  // ",nt": the build with non-temporal stores, which a launch of a
  // two-work-groups-per-CU kernel without extended arguments takes when it
  // writes more than kStreamOutBytes (see launch_sym_g, launch_nt_g).
  const double bt = (double)p.batch, nn_bytes = bt * (double)p.nn_elems * esz;
  const double x2_bytes = 2.0 * bt * (double)p.x_elems * esz;
  const double out_bytes = bt * (double)p.rows * (double)p.cols * elem_size(p.io);
  auto ntag = [](Form f, bool ext, double bytes) {
    return (f == Form::kPairLoop || f == Form::kPairTile) && !ext && stream_out(bytes) ? std::string(",nt")
                                                                                       : std::string();
  };
  // ",x": the build that reads extended arguments (the guard's device flags,
  // a grouped call's member table); see launch_sym and launch_nt.
  auto xtag = [](bool ext) { return ext ? std::string(",x") : std::string(); };
  auto xxt = [&](bool ext) {
    return "xxt<" + T + "," + E + "," + form_name(fx) + xtag(ext) + ntag(fx, ext, nn_bytes) + ">";
  };
  auto nn = [&](bool ext, bool c2) {
    return "nn<" + T + "," + E + "," + form_name(fn) + xtag(ext) + ntag(fn, ext, nn_bytes * (c2 ? 2.0 : 1.0)) + ">";
  };
  auto upd = [&](bool ext, const std::string& et) {
    return "upd<" + T + "," + T + "," + E + "," + form_name(fu) + et + xtag(ext) + ntag(fu, ext, x2_bytes) + ">";
  };
  // A grouped call's final product reads the member table.
  auto fin = [&](bool ext, const std::string& et) {
    ext = ext || grouped;
    return "out<" + T + "," + IO + "," + E + "," + form_name(fu) + et + xtag(ext) + ntag(fu, ext, out_bytes) + ">";
  };
  // The launches of one call, in the order of the runner (Runner::run and
  // Runner::run_guarded), by kind.
  std::vector<std::string> xs, ns, us;
  std::string fo;
  if (p.mode == NS_STANDARD) {
    xs.push_back(xxt(false));
    ns.push_back(nn(false, false));
    if (steps > 1) us.push_back(upd(false, e_term));
    fo = fin(false, e_term);
  } else if (guard) {
    // Every launch reads the guard's flags except the first step's Z'
    // product, which writes the fresh Q.
    xs.push_back(xxt(true));
    ns.push_back(nn(false, true));
    if (steps > 1) {
      us.push_back(upd(true, ",noE"));
      ns.push_back(nn(true, false));
    }
    fo = fin(true, ",noE");
  } else {
    xs.push_back(xxt(false));
    bool fresh = true;
    for (int k = 1; k <= steps; ++k) {
      if (k > 1 && ((mask >> k) & 1u)) {
        us.push_back(upd(false, ",noE"));
        fresh = true;
      }
      ns.push_back(nn(false, fresh));
      if (!fresh || (k < steps && !((mask >> (k + 1)) & 1u))) ns.push_back(nn(false, false));
      fresh = false;
    }
    fo = fin(false, ",noE");
  }
  std::vector<std::string> seen;
  std::string out;
  auto add = [&](const std::string& v) {
    if (std::find(seen.begin(), seen.end(), v) != seen.end()) return;
    seen.push_back(v);
    out += (out.empty() ? "" : " ") + v;
  };
  add("sumsq<" + IO + ">");
  add("stage<" + IO + "," + T + ">");
  for (const auto& v : xs) add(v);
  for (const auto& v : ns) add(v);
  for (const auto& v : us) add(v);
  add(fo);
  return out;
}

// Where a call reads its input and writes its result.
struct IoSpec {
  void* in;
  int64_t ld, bstride;
  void* out;
  int64_t out_ld, out_bstride;
  bool accumulate;  // false: out = result; true: out += apply * result
  float apply;
  const ns_matrix* members = nullptr;  // grouped call (device table), else null
};

template <typename T, typename IO>
ns_status run_typed(const Plan& p, const IoSpec& io, int steps, const float* a, const float* b, const float* c,
                    const ns_options* opt, void* ws, hipStream_t st) {
  Runner<T, IO> r{p,
                  reinterpret_cast<char*>(ws),
                  st,
                  reinterpret_cast<IO*>(io.in),
                  io.ld,
                  io.bstride,
                  reinterpret_cast<IO*>(io.out),
                  io.out_ld,
                  io.out_bstride,
                  io.members,
                  io.accumulate,
                  io.apply,
                  opt,
                  Tracer{opt ? opt->trace : nullptr, st}};
  const float eps = opt ? opt->eps : 1e-7f;
  hipError_t e;
  if constexpr (sizeof(T) == 4) {
    e = p.tile == 64 ? r.template run<64>(steps, a, b, c, eps) : r.template run<128>(steps, a, b, c, eps);
  } else {
    switch (p.tile) {
      case 256: e = r.template run<256>(steps, a, b, c, eps); break;
      case 192: e = r.template run<192>(steps, a, b, c, eps); break;
      default: e = r.template run<128>(steps, a, b, c, eps); break;
    }
  }
  return hip_status(e);
}


// The product launchers are instantiated in the kern_*.hip translation
// units, one per kernel family and tile edge, so the kernel builds compile
// in parallel and once each.
#define NS_SYM_LAUNCHERS(T, TILE)                                                            \
  template hipError_t launch_sym<T, TILE, true>(SymArgs<T>, int64_t, hipStream_t, LaunchEvents); \
  template hipError_t launch_sym<T, TILE, false>(SymArgs<T>, int64_t, hipStream_t, LaunchEvents);
#define NS_NT_LAUNCHER(T, OUT, TILE) \
  template hipError_t launch_nt<T, OUT, TILE>(NTArgs<T, OUT>, int64_t, hipStream_t, LaunchEvents);
#define NS_EXTERN_SYM(T, TILE) \
  extern template hipError_t launch_sym<T, TILE, true>(SymArgs<T>, int64_t, hipStream_t, LaunchEvents); \
  extern template hipError_t launch_sym<T, TILE, false>(SymArgs<T>, int64_t, hipStream_t, LaunchEvents);
#define NS_EXTERN_NT(T, OUT, TILE) \
  extern template hipError_t launch_nt<T, OUT, TILE>(NTArgs<T, OUT>, int64_t, hipStream_t, LaunchEvents);
#ifndef NS_KERNEL_UNIT
NS_EXTERN_SYM(_Float16, 128)
NS_EXTERN_SYM(_Float16, 192)
NS_EXTERN_SYM(_Float16, 256)
NS_EXTERN_SYM(float, 128)
NS_EXTERN_SYM(float, 64)
NS_EXTERN_NT(_Float16, _Float16, 128)
NS_EXTERN_NT(_Float16, __bf16, 128)
NS_EXTERN_NT(_Float16, _Float16, 192)
NS_EXTERN_NT(_Float16, __bf16, 192)
NS_EXTERN_NT(_Float16, _Float16, 256)
NS_EXTERN_NT(_Float16, __bf16, 256)
NS_EXTERN_NT(float, float, 128)
NS_EXTERN_NT(float, float, 64)
#endif

}  // namespace nsr
