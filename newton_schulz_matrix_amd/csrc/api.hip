// api.hip - host side of libnsortho: argument checks, workspace layout and
// the launch sequence of both Newton-Schulz forms on the caller's stream.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <math.h>

#include <algorithm>
#include <stdint.h>
#include <string.h>

#include "../../include/nsortho.h"
#include "products.hpp"
#include "stage.hpp"
#include "threshold.hpp"

using namespace nsk;

namespace {

constexpr size_t kAlign = 256;
constexpr int kPrescaleExp16 = 10;  // X is held as 2^10 * X in 16-bit storage
constexpr int kMaxPartials = 1024;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int elem_size(ns_dtype d) { return d == NS_FP32 ? 4 : 2; }

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
  size_t off_partial = 0, off_scale = 0, off_x[2] = {0, 0}, off_xt[2] = {0, 0}, off_nn[4] = {0, 0, 0, 0};
  size_t total = 0;
};

// Columns of the update tiles that go with a square tile edge: square tiles
// (192 x 256 update tiles were measured slower than 192 x 192 at 4096 x 14336).
constexpr int nn_tile_n(int edge) { return edge; }

bool resolve_internal(ns_dtype io, const ns_options* opt, ns_dtype* out) {
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
  if (req == NS_BF16) {
    *out = NS_BF16;
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
bool use_persistent(int edge, int64_t tiles, int64_t ktiles) {
  return edge <= 192 && tiles > kPersistentGroups && ktiles <= kPersistentMaxKtiles;
}

// Launches that take the two-work-groups-per-CU kernels (16-bit, 128 tiles,
// at least 512 tiles; see use_pair): per pair of tiles on a CU, measured on
// MI355X against the table above on the 128 x 1408 x 2048 expert batch.
constexpr double kPairKtile = 0.79, kPairSymFixed = 4.9, kPairNnFixed = 5.7;

bool use_pair(int edge, int esz, int64_t tiles);

double product_estimate(int edge, double tiles, double ktiles, double per_ktile, double fixed,
                        double pair_fixed) {
  if (use_pair(edge, 2, (int64_t)tiles)) return ceil(tiles / (2 * kComputeUnits)) * (ktiles * kPairKtile + pair_fixed);
  const double waves = ceil(tiles / kComputeUnits);
  if (use_persistent(edge, (int64_t)tiles, (int64_t)ktiles)) fixed *= kPersistentFixed;
  return waves * (ktiles * per_ktile + fixed);
}

double tile_estimate(const TileCost& c, int64_t n, int64_t m, int64_t batch, ns_mode mode) {
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
bool padding_fits(int64_t n_pad, int64_t m_pad, int esz) {
  return n_pad <= 65536 && m_pad * esz <= (int64_t(1) << 25);
}

int pick_tile(int64_t n, int64_t m, int64_t batch, ns_dtype internal, ns_mode mode) {
  if (internal == NS_FP32) return 128;
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

ns_status make_plan(int64_t rows, int64_t cols, int64_t batch, ns_dtype io, ns_mode mode, const ns_options* opt,
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
  if (req_tile != 0 && !(req_tile == 128 || (internal != NS_FP32 && (req_tile == 192 || req_tile == 256))))
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

ns_status hip_status(hipError_t e) { return e == hipSuccess ? NS_OK : NS_ERR_HIP; }

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

bool use_pair(int edge, int esz, int64_t tiles) {
  return edge == 128 && esz == 2 && tiles >= 2 * (int64_t)kPersistentGroups;
}

template <typename T, int TILE, bool GRAM_INPUT>
hipError_t launch_sym(SymArgs<T> a, int64_t batch, hipStream_t s, LaunchEvents ev) {
  const int64_t ntri = (int64_t)a.tiles * (a.tiles + 1) / 2;
  const int ktiles = a.K / (kRowBytes / (int)sizeof(T));
  const dim3 tiles_grid((unsigned)ntri, (unsigned)batch);
  a.batch = (int)batch;
  if constexpr (kHasPairKernels<T, TILE>) {
    if (use_pair(TILE, (int)sizeof(T), ntri * batch)) {
      if (use_persistent(TILE, ntri * batch, ktiles))
        return launch_kernel(k_sym_loop<T, TILE, GRAM_INPUT, 2>, dim3(2 * kPersistentGroups), dim3(kThreads), s, ev, a);
      return launch_kernel(k_sym<T, TILE, GRAM_INPUT, 2>, tiles_grid, dim3(kThreads), s, ev, a);
    }
  }
  if constexpr (TILE <= 192) {
    if (use_persistent(TILE, ntri * batch, ktiles))
      return launch_kernel(k_sym_loop<T, TILE, GRAM_INPUT>, dim3(kPersistentGroups), dim3(kThreads), s, ev, a);
  }
  return launch_kernel(k_sym<T, TILE, GRAM_INPUT>, tiles_grid, dim3(kThreads), s, ev, a);
}

template <typename T, typename OutT, int TILE, bool CAP>
hipError_t launch_nt_cap(NTArgs<T, OutT> a, int64_t batch, hipStream_t s, LaunchEvents ev) {
  constexpr int TN = nn_tile_n(TILE);
  const int64_t per = (int64_t)a.tiles_m * a.tiles_n;
  const dim3 flat((unsigned)(per * batch));
  a.batch = (int)batch;
  if constexpr (kHasPairKernels<T, TILE>) {
    if (use_pair(TILE, (int)sizeof(T), per * batch))
      return launch_kernel(k_nt<T, OutT, TILE, TN, 2, CAP>, flat, dim3(kThreads), s, ev, a);
  }
  if constexpr (TILE <= 192) {
    if (use_persistent(TILE, per * batch, a.K / (kRowBytes / (int)sizeof(T))))
      return launch_kernel(k_nt_loop<T, OutT, TILE, TN, 1, CAP>, dim3(kPersistentGroups), dim3(kThreads), s, ev, a);
  }
  return launch_kernel(k_nt<T, OutT, TILE, TN, 1, CAP>, flat, dim3(kThreads), s, ev, a);
}

// Updates with an E term (the standard form) take the kernels that capture
// E from LDS, where the tile has the registers for it; E-free updates (the
// Gram form) and the other tiles take the kernels without the capture.
template <typename T, typename OutT, int TILE>
hipError_t launch_nt(NTArgs<T, OutT> a, int64_t batch, hipStream_t s, LaunchEvents ev) {
  if constexpr (EPrefetch<T, TILE, nn_tile_n(TILE)>::kEnabled) {
    if (a.E) return launch_nt_cap<T, OutT, TILE, true>(a, batch, s, ev);
  }
  return launch_nt_cap<T, OutT, TILE, false>(a, batch, s, ev);
}

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
  bool accumulate;           // false: out = result; true: out += apply * result
  float apply;
  const ns_options* opt;
  Tracer tr;

  T* xbuf(int i) const { return reinterpret_cast<T*>(ws + p.off_x[i]); }
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
                 float delta) const {
    if (E && E != L) return hipErrorInvalidValue;
    SymArgs<T> a;
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
    const double n = (double)p.n, bt = (double)p.batch, es = sizeof(T);
    const double inner = gram ? (double)p.m : n;
    const double flops = n * n * inner * bt;
    double bytes = (L == R ? 1.0 : 2.0) * n * inner * es + n * n * es * (1.0 + (E ? 1.0 : 0.0) + (C2 ? 1.0 : 0.0));
    bytes *= bt;
    if (gram)
      return tr.run(NS_KERNEL_GRAM, flops, bytes, [&](LaunchEvents ev) { return launch_sym<T, TILE, true>(a, p.batch, st, ev); });
    return tr.run(NS_KERNEL_SYM, flops, bytes, [&](LaunchEvents ev) { return launch_sym<T, TILE, false>(a, p.batch, st, ev); });
  }

  // Y = alpha * X_in + B X_in into X_out and X_out^T (E omitted when alpha
  // is 0).
  template <int TILE>
  hipError_t nn_internal(const T* B, int xin, bool with_e, float alpha, int xout) const {
    NTArgs<T, T> a;
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
    a.d_status = nullptr;
    const double n = (double)p.n, m = (double)p.m, bt = (double)p.batch, es = sizeof(T);
    const double bytes = bt * (n * n * es + n * m * es * (3.0 + (with_e ? 1.0 : 0.0)));
    return tr.run(NS_KERNEL_UPDATE, 2.0 * n * n * m * bt, bytes,
                  [&](LaunchEvents ev) { return launch_nt<T, T, TILE>(a, p.batch, st, ev); });
  }

  // The caller's matrix = out_scale * (alpha * X_in + B X_in), oriented back.
  template <int TILE>
  hipError_t nn_final(const T* B, int xin, bool with_e, float alpha, float out_scale) const {
    NTArgs<T, IO> a;
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
    a.d_status = opt ? opt->d_status : nullptr;
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
                           (const IO*)user, p.rows, p.cols, ld, bstride, vec_ok ? 1 : 0, partial, p.partials);
    });
    if (e != hipSuccess) return e;
    float* scales = reinterpret_cast<float*>(ws + p.off_scale);
    hipLaunchKernelGGL(k_scale, dim3((unsigned)p.batch), dim3(kStageThreads), 0, st, partial, p.partials, prescale,
                       eps, scales);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return tr.run(NS_KERNEL_STAGE, 0.0, elems * (sizeof(IO) + 2 * sizeof(T)), [&](LaunchEvents ev) {
      const int bi = (int)(p.n_pad / 64), bj = (int)(p.m_pad / 64);
      return launch_kernel(k_stage_pair<IO, T>, dim3((unsigned)(bi * bj), (unsigned)p.batch), dim3(kStageThreads), st,
                           ev, (const IO*)user, p.rows, p.cols, ld, bstride, vec_ok ? 1 : 0, (const float*)scales,
                           xbuf(0), xtbuf(0), p.n_pad, p.m_pad, p.x_elems, p.transposed ? 1 : 0, bj);
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
};

// Where a call reads its input and writes its result.
struct IoSpec {
  void* in;
  int64_t ld, bstride;
  void* out;
  int64_t out_ld, out_bstride;
  bool accumulate;  // false: out = result; true: out += apply * result
  float apply;
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
                  io.accumulate,
                  io.apply,
                  opt,
                  Tracer{opt ? opt->trace : nullptr, st}};
  const float eps = opt ? opt->eps : 1e-7f;
  hipError_t e;
  if constexpr (sizeof(T) == 4) {
    e = r.template run<128>(steps, a, b, c, eps);
  } else {
    switch (p.tile) {
      case 256: e = r.template run<256>(steps, a, b, c, eps); break;
      case 192: e = r.template run<192>(steps, a, b, c, eps); break;
      default: e = r.template run<128>(steps, a, b, c, eps); break;
    }
  }
  return hip_status(e);
}

// Calls f.template run<T, IO>() for the (internal, I/O) type pair of a plan.
template <class F>
ns_status dispatch_types(const Plan& p, F&& f) {
  if (p.io == NS_FP32) return f.template run<float, float>();
  if (p.io == NS_BF16) {
    if (p.internal == NS_FP16) return f.template run<_Float16, __bf16>();
    return f.template run<__bf16, __bf16>();
  }
  if (p.internal == NS_FP16) return f.template run<_Float16, _Float16>();
  return f.template run<__bf16, _Float16>();
}

struct OrthCall {
  const Plan& p;
  IoSpec io;
  int32_t steps;
  const float *a, *b, *c;
  const ns_options* opt;
  void* ws;
  hipStream_t st;
  template <typename T, typename IO>
  ns_status run() const {
    return run_typed<T, IO>(p, io, steps, a, b, c, opt, ws, st);
  }
};

ns_status check_coefficients(int32_t steps, const float* a, const float* b, const float* c, ns_mode mode,
                             uint32_t mask, ns_dtype internal) {
  if (steps < 1 || steps > NS_MAX_STEPS || !a || !b || !c) return NS_ERR_INVALID_ARG;
  for (int k = 0; k < steps; ++k)
    if (!isfinite(a[k]) || !isfinite(b[k]) || !isfinite(c[k])) return NS_ERR_INVALID_ARG;
  if (mode == NS_GRAM && internal != NS_FP32) {
    // The accumulated Q is a product of factors a_k I + ... whose largest
    // eigenvalue can reach |a_k| per step; keep it inside fp16 range.
    double run = 1.0;
    for (int k = 1; k <= steps; ++k) {
      if (k > 1 && ((mask >> k) & 1u)) run = 1.0;
      run *= fabs((double)a[k - 1]);
      if (run >= 32768.0) return NS_ERR_INVALID_ARG;
    }
  }
  return NS_OK;
}

ns_status orthogonalize_impl(void* X, int64_t batch, int64_t rows, int64_t cols, int64_t ld, int64_t bstride,
                             ns_dtype dtype, int32_t steps, const float* a, const float* b, const float* c,
                             ns_mode mode, const ns_options* opt, void* ws, size_t ws_bytes, ns_stream_t stream) {
  if (!X) return NS_ERR_INVALID_ARG;
  if (ld < cols) return NS_ERR_INVALID_ARG;
  if (batch > 1 && bstride < rows * ld) return NS_ERR_INVALID_ARG;
  Plan p;
  ns_status s = make_plan(rows, cols, batch, dtype, mode, opt, &p);
  if (s != NS_OK) return s;
  if (opt && !(opt->eps >= 0.f && isfinite(opt->eps))) return NS_ERR_INVALID_ARG;
  const uint32_t mask = opt ? opt->restart_mask : (1u << 4);
  if ((s = check_coefficients(steps, a, b, c, mode, mask, p.internal)) != NS_OK) return s;
  if (!ws || ws_bytes < p.total || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0) return NS_ERR_WORKSPACE;
  return dispatch_types(p, OrthCall{p, IoSpec{X, ld, bstride, X, ld, bstride, false, 0.f}, steps, a, b, c, opt, ws,
                                    reinterpret_cast<hipStream_t>(stream)});
}

// Muon step: the momentum pass writes U into the workspace after the
// orthogonalization's own buffers; the orthogonalization then reads U and
// its final epilogue applies W <- W - lr * NS(U).
size_t muon_u_offset(const Plan& p) { return align_up(p.total); }
size_t muon_total(const Plan& p) {
  return muon_u_offset(p) + align_up((size_t)p.batch * p.rows * p.cols * elem_size(p.io));
}

// The Muon step for one (internal, I/O) type pair: momentum pass, then the
// orthogonalization of U with W <- W - lr * result in its final epilogue.
struct MuonCall {
  const Plan& p;
  void *W, *U;
  const void* G;
  float* M;
  int64_t ld, bstride;
  float lr, mu;
  int32_t nesterov, steps;
  const float *a, *b, *c;
  const ns_options* opt;
  void* ws;
  hipStream_t st;
  template <typename T, typename IO>
  ns_status run() const {
    const int v = 16 / (int)sizeof(IO);
    const bool vec_ok = ld % v == 0 && (p.batch == 1 || bstride % v == 0) &&
                        (reinterpret_cast<uintptr_t>(G) & 15) == 0 && (reinterpret_cast<uintptr_t>(M) & 15) == 0;
    const double elems = (double)p.rows * (double)p.cols * (double)p.batch;
    Tracer tr{opt ? opt->trace : nullptr, st};
    hipError_t e = tr.run(NS_KERNEL_MOMENTUM, 0.0, elems * (2.0 * sizeof(IO) + 8.0), [&](LaunchEvents ev) {
      return launch_kernel(k_momentum<IO>, dim3((unsigned)p.rows, (unsigned)p.batch), dim3(kStageThreads), st, ev,
                           reinterpret_cast<const IO*>(G), M, reinterpret_cast<IO*>(U), p.cols, ld, bstride,
                           vec_ok ? 1 : 0, mu, nesterov ? 1 : 0);
    });
    if (e != hipSuccess) return NS_ERR_HIP;
    return run_typed<T, IO>(p, IoSpec{U, p.cols, p.rows * p.cols, W, ld, bstride, true, -lr}, steps, a, b, c, opt, ws,
                            st);
  }
};

ns_status muon_impl(void* W, const void* G, float* M, int64_t batch, int64_t rows, int64_t cols, int64_t ld,
                    int64_t bstride, ns_dtype dtype, float lr, float mu, int32_t nesterov, int32_t steps,
                    const float* a, const float* b, const float* c, ns_mode mode, const ns_options* opt, void* ws,
                    size_t ws_bytes, ns_stream_t stream) {
  if (!W || !G || !M) return NS_ERR_INVALID_ARG;
  if (ld < cols) return NS_ERR_INVALID_ARG;
  if (batch > 1 && bstride < rows * ld) return NS_ERR_INVALID_ARG;
  if (!isfinite(lr) || !(mu >= 0.f && mu < 1.f)) return NS_ERR_INVALID_ARG;
  Plan p;
  ns_status s = make_plan(rows, cols, batch, dtype, mode, opt, &p);
  if (s != NS_OK) return s;
  if (opt && !(opt->eps >= 0.f && isfinite(opt->eps))) return NS_ERR_INVALID_ARG;
  const uint32_t mask = opt ? opt->restart_mask : (1u << 4);
  if ((s = check_coefficients(steps, a, b, c, mode, mask, p.internal)) != NS_OK) return s;
  if (!ws || ws_bytes < muon_total(p) || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0) return NS_ERR_WORKSPACE;
  void* U = reinterpret_cast<char*>(ws) + muon_u_offset(p);
  return dispatch_types(p, MuonCall{p, W, U, G, M, ld, bstride, lr, mu, nesterov, steps, a, b, c, opt, ws,
                                    reinterpret_cast<hipStream_t>(stream)});
}

// Soft-threshold workspace: select state + three histograms (kHistCopies copies each).
size_t threshold_ws_bytes() {
  return align_up(sizeof(SelectState)) + align_up(3 * kHistCopies * kHistBins * sizeof(uint32_t));
}

template <typename IO>
ns_status threshold_typed(const void* M, void* B, void* O, int64_t numel, float lambda, float mult,
                          float* d_lambda_out, void* ws, hipStream_t st) {
  char* w = reinterpret_cast<char*>(ws);
  SelectState* state = reinterpret_cast<SelectState*>(w);
  uint32_t* hist = reinterpret_cast<uint32_t*>(w + align_up(sizeof(SelectState)));
  const IO* m = reinterpret_cast<const IO*>(M);
  const int64_t blocks64 = (numel + 255) / 256;
  const unsigned grid = (unsigned)(blocks64 < 2048 ? blocks64 : 2048);
  // Histogram passes: about 64 elements per thread, so that fewer blocks
  // merge their LDS histograms into the global one.
  const int64_t hblocks = (numel + (int64_t)kHistThreads * 64 - 1) / ((int64_t)kHistThreads * 64);
  const unsigned hgrid = (unsigned)(hblocks < 512 ? hblocks : 512);
  const int vec_hist = (reinterpret_cast<uintptr_t>(M) & 15) == 0 ? 1 : 0;
  const int vec_clip = vec_hist && (reinterpret_cast<uintptr_t>(B) & 15) == 0 &&
                       (!O || (reinterpret_cast<uintptr_t>(O) & 15) == 0) ? 1 : 0;
  const uint64_t rank = (uint64_t)((numel + 1) / 2);
  hipLaunchKernelGGL(k_select_init, dim3((3 * kHistCopies * kHistBins + 255) / 256), dim3(256), 0, st, state, hist,
                     3 * kHistCopies * kHistBins,
                     rank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return NS_ERR_HIP;
  if (lambda >= 0.f) {
    hipLaunchKernelGGL(k_set_lambda, dim3(1), dim3(64), 0, st, state, lambda, d_lambda_out);
  } else {
    constexpr int kb = KeyOf<IO>::kBits;
    // Digits from the top, at most 11 bits each.
    int shifts[3], bits[3], npass = 0;
    int hi = kb;
    while (hi > 0) {
      const int nbits = hi >= 11 ? 11 : hi;
      shifts[npass] = hi - nbits;
      bits[npass] = nbits;
      hi -= nbits;
      ++npass;
    }
    for (int ps = 0; ps < npass; ++ps) {
      uint32_t* h = hist + ps * kHistCopies * kHistBins;
      hipLaunchKernelGGL((k_radix_hist<IO>), dim3(hgrid), dim3(kHistThreads), 0, st, m, numel, state, shifts[ps],
                         bits[ps], h, vec_hist);
      hipLaunchKernelGGL((k_radix_pick<IO>), dim3(1), dim3(kHistThreads), 0, st, state, h, shifts[ps], bits[ps],
                         ps == npass - 1 ? 1 : 0, mult, -1.f, d_lambda_out);
    }
  }
  hipLaunchKernelGGL((k_clip_split<IO>), dim3(grid), dim3(256), 0, st, m, reinterpret_cast<IO*>(B),
                     reinterpret_cast<IO*>(O), numel, state, vec_clip);
  return hip_status(hipGetLastError());
}

}  // namespace

extern "C" {

void ns_options_default(ns_options* opt) {
  if (!opt) return;
  opt->restart_mask = 1u << 4;
  opt->eps = 1e-7f;
  opt->internal = -1;
  opt->d_status = nullptr;
  opt->trace = nullptr;
  opt->tile = 0;
}

size_t ns_workspace_size(int64_t rows, int64_t cols, int64_t batch, ns_dtype dtype, ns_mode mode,
                         const ns_options* opt) {
  Plan p;
  if (make_plan(rows, cols, batch, dtype, mode, opt, &p) != NS_OK) return 0;
  return p.total;
}

ns_status ns_orthogonalize(void* X, int64_t rows, int64_t cols, int64_t ld, ns_dtype dtype, int32_t steps,
                           const float* a, const float* b, const float* c, ns_mode mode, const ns_options* opt,
                           void* workspace, size_t workspace_bytes, ns_stream_t stream) {
  return orthogonalize_impl(X, 1, rows, cols, ld, rows * ld, dtype, steps, a, b, c, mode, opt, workspace,
                            workspace_bytes, stream);
}

ns_status ns_orthogonalize_batched(void* X, int64_t batch, int64_t rows, int64_t cols, int64_t ld,
                                   int64_t batch_stride, ns_dtype dtype, int32_t steps, const float* a,
                                   const float* b, const float* c, ns_mode mode, const ns_options* opt,
                                   void* workspace, size_t workspace_bytes, ns_stream_t stream) {
  return orthogonalize_impl(X, batch, rows, cols, ld, batch_stride, dtype, steps, a, b, c, mode, opt, workspace,
                            workspace_bytes, stream);
}

size_t ns_muon_workspace_size(int64_t rows, int64_t cols, int64_t batch, ns_dtype dtype, ns_mode mode,
                              const ns_options* opt) {
  Plan p;
  if (make_plan(rows, cols, batch, dtype, mode, opt, &p) != NS_OK) return 0;
  return muon_total(p);
}

ns_status ns_muon_step(void* W, const void* G, float* M, int64_t batch, int64_t rows, int64_t cols, int64_t ld,
                       int64_t batch_stride, ns_dtype dtype, float lr, float momentum, int32_t nesterov,
                       int32_t steps, const float* a, const float* b, const float* c, ns_mode mode,
                       const ns_options* opt, void* workspace, size_t workspace_bytes, ns_stream_t stream) {
  return muon_impl(W, G, M, batch, rows, cols, ld, batch == 1 ? rows * ld : batch_stride, dtype, lr, momentum,
                   nesterov, steps, a, b, c, mode, opt, workspace, workspace_bytes, stream);
}

// Bin counts are 32-bit: at most 2^32 - 1 elements.
constexpr int64_t kMaxThresholdNumel = (int64_t(1) << 32) - 1;

size_t ns_soft_threshold_workspace_size(int64_t numel, ns_dtype dtype) {
  if (numel < 1 || numel > kMaxThresholdNumel) return 0;
  if (dtype != NS_BF16 && dtype != NS_FP16 && dtype != NS_FP32) return 0;
  return threshold_ws_bytes();
}

ns_status ns_soft_threshold_split(const void* M, void* B, void* O, int64_t numel, ns_dtype dtype, float lambda,
                                  float mult, float* d_lambda_out, void* workspace, size_t workspace_bytes,
                                  ns_stream_t stream) {
  if (!M || !B || numel < 1 || numel > kMaxThresholdNumel) return NS_ERR_INVALID_ARG;
  if (isnan(lambda) || (lambda < 0.f && !(isfinite(mult) && mult >= 0.f))) return NS_ERR_INVALID_ARG;
  if (dtype != NS_BF16 && dtype != NS_FP16 && dtype != NS_FP32) return NS_ERR_UNSUPPORTED_DTYPE;
  if (!workspace || workspace_bytes < threshold_ws_bytes() || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return NS_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == NS_BF16) return threshold_typed<__bf16>(M, B, O, numel, lambda, mult, d_lambda_out, workspace, st);
  if (dtype == NS_FP16) return threshold_typed<_Float16>(M, B, O, numel, lambda, mult, d_lambda_out, workspace, st);
  return threshold_typed<float>(M, B, O, numel, lambda, mult, d_lambda_out, workspace, st);
}

const char* ns_status_string(ns_status s) {
  switch (s) {
    case NS_OK: return "ok";
    case NS_ERR_INVALID_ARG: return "invalid argument";
    case NS_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case NS_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case NS_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t ns_version(void) { return 200; }

}  // extern "C"
