// api.hip - the C entry points of libnsortho: argument checks, the
// workspace query, dispatch to the launch sequence of the call's type pair
// (plan.hpp, instantiated in run_*.hip), the Muon step, the soft-threshold
// split and the allocation-free variant.
#include <mutex>

#include "plan.hpp"
#include "threshold.hpp"

using namespace nsr;

namespace {

// Calls f.template run<T, IO>() for the (internal, I/O) type pair of a plan.
template <class F>
ns_status dispatch_types(const Plan& p, F&& f) {
  if (p.io == NS_FP32) return f.template run<float, float>();
  if (p.io == NS_BF16) return f.template run<_Float16, __bf16>();
  return f.template run<_Float16, _Float16>();
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

// Largest magnitude each stored quantity of the iteration reaches in exact
// arithmetic.  Every matrix of both forms is a function of the singular
// values of X0 (which lie in [0, 1] after the Frobenius scaling), with its
// entries bounded by its spectral norm, so tracking one singular value s
// through the steps bounds them all:
//   standard: A = s^2, b A + c A^2, the new X = p(s) (held as 2^10 X in
//     16-bit storage);
//   Gram: from a start or restart with singular value s, R = lambda = s^2,
//     Z' = b lambda + c lambda^2, Q's eigenvalue (a + Z') Q, V = lambda z,
//     R <- lambda z^2, and at a restart X <- Q X.
// The maxima are taken over a grid of s (linear on [0, 1] and logarithmic
// down to 1e-9, where Q's eigenvalue reaches the product of the a_k); the
// limits keep a factor of two below each type's largest value for the
// maxima between grid points (a value that still overflows on the device is
// reported through the status word).
struct RangeBound {
  double x = 0, nn = 0, out = 0;  // X iterates (unscaled), n x n state, result
};

RangeBound scalar_bounds(int steps, const float* a, const float* b, const float* c, ns_mode mode, uint32_t mask) {
  RangeBound r;
  auto upd = [](double& m, double v) { m = std::max(m, fabs(v)); };
  auto one = [&](double sigma) {
    if (mode == NS_STANDARD) {
      double s = sigma;
      for (int k = 0; k < steps; ++k) {
        const double A = s * s, B = b[k] * A + c[k] * A * A;
        upd(r.nn, A);
        upd(r.nn, B);
        s = a[k] * s + B * s;
        if (k + 1 < steps) upd(r.x, s);
      }
      upd(r.out, s);
      return;
    }
    double s = sigma, lam = s * s, q = 1.0;
    bool fresh = true;
    upd(r.nn, lam);
    for (int k = 1; k <= steps; ++k) {
      if (k > 1 && ((mask >> k) & 1u)) {
        s *= q;
        upd(r.x, s);
        lam = s * s;
        upd(r.nn, lam);
        q = 1.0;
        fresh = true;
      }
      const double zp = b[k - 1] * lam + c[k - 1] * lam * lam, z = a[k - 1] + zp;
      upd(r.nn, zp);
      q = fresh ? z : q * z;
      upd(r.nn, q);
      fresh = false;
      if (k < steps && !((mask >> (k + 1)) & 1u)) {
        upd(r.nn, lam * z);
        lam *= z * z;
        upd(r.nn, lam);
      }
    }
    upd(r.out, q * s);
  };
  for (int i = 0; i <= 512; ++i) one(i / 512.0);
  const double step = 1.1220184543019633;  // 10^(1/20)
  double sigma = 1e-9;
  for (int i = 0; i < 180; ++i, sigma *= step) one(sigma);
  return r;
}

ns_status check_coefficients(int32_t steps, const float* a, const float* b, const float* c, ns_mode mode,
                             uint32_t mask, ns_dtype internal, ns_dtype io) {
  if (steps < 1 || steps > NS_MAX_STEPS || !a || !b || !c) return NS_ERR_INVALID_ARG;
  for (int k = 0; k < steps; ++k)
    if (!isfinite(a[k]) || !isfinite(b[k]) || !isfinite(c[k])) return NS_ERR_INVALID_ARG;
  // Stored values stay below half of the storage type's largest finite
  // value: 2^15 for fp16 (X is held as 2^10 X), 2^127 for fp32; the result
  // below half of the I/O type's (bf16 shares fp32's range).
  const RangeBound r = scalar_bounds(steps, a, b, c, mode, mask);
  const double lim = internal == NS_FP32 ? 0x1p127 : 32768.0;
  const double xlim = internal == NS_FP32 ? 0x1p127 : 32768.0 / (double)(1 << kPrescaleExp16);
  const double olim = io == NS_FP16 ? 32768.0 : 0x1p127;
  if (!(r.nn < lim) || !(r.x < xlim) || !(r.out < olim)) return NS_ERR_INVALID_ARG;
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
  if (opt && !(opt->guard_threshold >= 0.f && isfinite(opt->guard_threshold))) return NS_ERR_INVALID_ARG;
  const uint32_t mask = opt ? opt->restart_mask : (1u << 4);
  if ((s = check_coefficients(steps, a, b, c, mode, mask, p.internal, p.io)) != NS_OK) return s;
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
  if (opt && !(opt->guard_threshold >= 0.f && isfinite(opt->guard_threshold))) return NS_ERR_INVALID_ARG;
  const uint32_t mask = opt ? opt->restart_mask : (1u << 4);
  if ((s = check_coefficients(steps, a, b, c, mode, mask, p.internal, p.io)) != NS_OK) return s;
  if (!ws || ws_bytes < muon_total(p) || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0) return NS_ERR_WORKSPACE;
  void* U = reinterpret_cast<char*>(ws) + muon_u_offset(p);
  return dispatch_types(p, MuonCall{p, W, U, G, M, ld, bstride, lr, mu, nesterov, steps, a, b, c, opt, ws,
                                    reinterpret_cast<hipStream_t>(stream)});
}

// Soft-threshold workspace: select state + the histograms (three radix
// passes of kHistCopies copies for fp32 keys, kSelCopies copies of all 2^15
// keys for 16-bit ones).
size_t threshold_ws_bytes() {
  return align_up(sizeof(SelectState)) +
         align_up(std::max<size_t>(3 * kHistCopies * kHistBins, (size_t)kSelWords) * sizeof(uint32_t));
}

template <typename IO>
ns_status threshold_typed(const void* M, void* B, void* O, int64_t numel, float lambda, float mult,
                          float* d_lambda_out, int32_t* d_status, void* ws, hipStream_t st) {
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
  constexpr bool one_pass = sizeof(IO) == 2;
  const int nhist = lambda >= 0.f ? 0 : one_pass ? kSelWords : 3 * kHistCopies * kHistBins;
  hipLaunchKernelGGL(k_select_init, dim3((std::max(nhist, 1) + 255) / 256), dim3(256), 0, st, state, hist, nhist, rank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return NS_ERR_HIP;
  if (lambda >= 0.f) {
    hipLaunchKernelGGL(k_set_lambda, dim3(1), dim3(64), 0, st, state, lambda, d_lambda_out);
  } else if constexpr (one_pass) {
    // One block per compute unit (the LDS histogram takes 128 KiB).
    const int64_t want = (numel + (int64_t)kSelThreads * 64 - 1) / ((int64_t)kSelThreads * 64);
    const unsigned g = (unsigned)std::max<int64_t>(1, std::min<int64_t>(want, 256));
    hipLaunchKernelGGL((k_hist16<IO>), dim3(g), dim3(kSelThreads), 0, st, m, numel, hist, vec_hist);
    hipLaunchKernelGGL((k_pick16<IO>), dim3(1), dim3(kPickThreads), 0, st, state, hist, mult, d_lambda_out);
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
                     reinterpret_cast<IO*>(O), numel, state, vec_clip, d_status,
                     (int32_t)(NS_ERR_NONFINITE | NS_STATUS_AT_SPLIT));
  return hip_status(hipGetLastError());
}

// Scratch of ns_orthogonalize_static: one array per device, allocated when
// the code object is loaded and held until the process ends.  Host code
// never uses its name as an address: scratch_ptr() asks the runtime for the
// current device's copy once and keeps it.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch, or nullptr when the runtime cannot give it.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
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
  opt->guard_threshold = 0.f;
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

}  // extern "C"

namespace {

int64_t plan_string(int64_t rows, int64_t cols, int64_t batch, ns_dtype dtype, ns_mode mode, int32_t steps,
                    const ns_options* opt, bool grouped, char* buf, size_t len) {
  Plan p;
  if (make_plan(rows, cols, batch, dtype, mode, opt, &p) != NS_OK || steps < 1 || steps > NS_MAX_STEPS) return -1;
  const std::string d =
      describe_plan(p, steps, opt ? opt->restart_mask : (1u << 4), opt && opt->guard_threshold > 0.f, grouped);
  if (buf && len > 0) {
    const size_t n = std::min(len - 1, d.size());
    memcpy(buf, d.data(), n);
    buf[n] = 0;
  }
  return (int64_t)d.size() + 1;
}

}  // namespace

extern "C" {

int64_t ns_plan_kernels(int64_t rows, int64_t cols, int64_t batch, ns_dtype dtype, ns_mode mode, int32_t steps,
                        const ns_options* opt, char* buf, size_t len) {
  return plan_string(rows, cols, batch, dtype, mode, steps, opt, false, buf, len);
}

int64_t ns_plan_kernels_grouped(int64_t n, int64_t m, int64_t count, ns_dtype dtype, ns_mode mode, int32_t steps,
                                const ns_options* opt, char* buf, size_t len) {
  if (n > m) return -1;
  return plan_string(n, m, count, dtype, mode, steps, opt, true, buf, len);
}

// A grouped call's member table reaches the device through kernel
// arguments, up to kTableChunk entries per launch (3 KiB of arguments), so
// the call needs neither a copy from pageable host memory (which can make
// the host wait for the stream) nor a host synchronization.
constexpr int kTableChunk = 128;
struct TableChunk {
  ns_matrix m[kTableChunk];
  int32_t count;
};

static __global__ void k_write_table(TableChunk c, ns_matrix* dst) {
  const int i = threadIdx.x;
  if (i < c.count) dst[i] = c.m[i];
}

// Grouped call: the workspace of a batch of `count` n x m matrices, then the
// members' table.
size_t grouped_table_offset(const Plan& p) { return align_up(p.total); }
size_t grouped_total(const Plan& p) { return grouped_table_offset(p) + align_up((size_t)p.batch * sizeof(ns_matrix)); }

size_t ns_grouped_workspace_size(int64_t n, int64_t m, int64_t count, ns_dtype dtype, ns_mode mode,
                                 const ns_options* opt) {
  Plan p;
  if (n > m || make_plan(n, m, count, dtype, mode, opt, &p) != NS_OK) return 0;
  return grouped_total(p);
}

ns_status ns_orthogonalize_grouped(const ns_matrix* members, int64_t count, int64_t n, int64_t m, ns_dtype dtype,
                                   int32_t steps, const float* a, const float* b, const float* c, ns_mode mode,
                                   const ns_options* opt, void* workspace, size_t workspace_bytes,
                                   ns_stream_t stream) {
  if (!members || n < 1 || n > m) return NS_ERR_INVALID_ARG;
  Plan p;
  ns_status s = make_plan(n, m, count, dtype, mode, opt, &p);
  if (s != NS_OK) return s;
  for (int64_t i = 0; i < count; ++i) {
    const ns_matrix& mb = members[i];
    if (!mb.data || (mb.transposed != 0 && mb.transposed != 1) || mb.reserved != 0) return NS_ERR_INVALID_ARG;
    if (mb.ld < (mb.transposed ? n : m)) return NS_ERR_INVALID_ARG;
  }
  if (opt && !(opt->eps >= 0.f && isfinite(opt->eps))) return NS_ERR_INVALID_ARG;
  if (opt && !(opt->guard_threshold >= 0.f && isfinite(opt->guard_threshold))) return NS_ERR_INVALID_ARG;
  const uint32_t mask = opt ? opt->restart_mask : (1u << 4);
  if ((s = check_coefficients(steps, a, b, c, mode, mask, p.internal, p.io)) != NS_OK) return s;
  if (!workspace || workspace_bytes < grouped_total(p) || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return NS_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  ns_matrix* table = reinterpret_cast<ns_matrix*>(reinterpret_cast<char*>(workspace) + grouped_table_offset(p));
  for (int64_t i0 = 0; i0 < count; i0 += kTableChunk) {
    TableChunk chunk;
    chunk.count = (int32_t)std::min<int64_t>(kTableChunk, count - i0);
    memcpy(chunk.m, members + i0, (size_t)chunk.count * sizeof(ns_matrix));
    hipLaunchKernelGGL(k_write_table, dim3(1), dim3(kTableChunk), 0, st, chunk, table + i0);
    if (hipGetLastError() != hipSuccess) return NS_ERR_HIP;
  }
  IoSpec io{nullptr, m, 0, nullptr, m, 0, false, 0.f, table};
  return dispatch_types(p, OrthCall{p, io, steps, a, b, c, opt, workspace, st});
}

size_t ns_static_scratch_bytes(void) { return kStaticScratchBytes; }

ns_status ns_orthogonalize_static(void* X, int64_t batch, int64_t rows, int64_t cols, int64_t ld, int64_t batch_stride,
                                  ns_dtype dtype, int32_t steps, const float* a, const float* b, const float* c,
                                  ns_mode mode, const ns_options* opt, ns_stream_t stream) {
  Plan p;
  ns_status s = make_plan(rows, cols, batch, dtype, mode, opt, &p);
  if (s != NS_OK) return s;
  if (p.total > kStaticScratchBytes) return NS_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return NS_ERR_HIP;
  return orthogonalize_impl(X, batch, rows, cols, ld, batch_stride, dtype, steps, a, b, c, mode, opt, ws,
                            kStaticScratchBytes, stream);
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
                                  float mult, float* d_lambda_out, int32_t* d_status, void* workspace,
                                  size_t workspace_bytes, ns_stream_t stream) {
  if (!M || !B || numel < 1 || numel > kMaxThresholdNumel) return NS_ERR_INVALID_ARG;
  if (isnan(lambda) || (lambda < 0.f && !(isfinite(mult) && mult >= 0.f))) return NS_ERR_INVALID_ARG;
  if (dtype != NS_BF16 && dtype != NS_FP16 && dtype != NS_FP32) return NS_ERR_UNSUPPORTED_DTYPE;
  if (!workspace || workspace_bytes < threshold_ws_bytes() || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return NS_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (dtype == NS_BF16) return threshold_typed<__bf16>(M, B, O, numel, lambda, mult, d_lambda_out, d_status, workspace, st);
  if (dtype == NS_FP16) return threshold_typed<_Float16>(M, B, O, numel, lambda, mult, d_lambda_out, d_status, workspace, st);
  return threshold_typed<float>(M, B, O, numel, lambda, mult, d_lambda_out, d_status, workspace, st);
}

const char* ns_status_string(ns_status s) {
  switch (s) {
    case NS_OK: return "ok";
    case NS_ERR_INVALID_ARG: return "invalid argument";
    case NS_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case NS_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case NS_ERR_HIP: return "HIP runtime error";
    case NS_ERR_NONFINITE: return "non-finite value produced on the device";
  }
  return "unknown status";
}

int32_t ns_version(void) { return 300; }

}  // extern "C"
