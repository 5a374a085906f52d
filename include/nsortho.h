/*
 * nsortho.h - Newton-Schulz orthogonalization on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libnsortho.so.  Every entry point takes plain pointers and sizes;
 * device pointers are HIP device memory, host pointers are ordinary memory.
 * All device work is enqueued on the caller's HIP stream; no entry point
 * synchronizes, allocates device memory, or keeps state between calls.
 *
 * What is computed.  Muon replaces an update matrix G = U S V^T by its polar
 * factor U V^T and approximates it by a few steps of a quintic Newton-Schulz
 * iteration (Muon / NanoGPT article on blog.hotdry.top, sections "From SGD to
 * Muon" and "Coefficient tuning of the Newton-Schulz iteration and FLOP
 * overhead"; Gram Newton-Schulz article on itsolotime.com, section
 * "Algorithm advantages: from standard Newton-Schulz to Gram Newton-Schulz").
 * With X the input oriented so that it has no more rows than columns
 * (n = min(rows, cols), m = max(rows, cols)) and scaled to unit Frobenius
 * norm, X <- X / (||X||_F + eps), each step k = 1..steps applies
 *
 *     A = X X^T,   X <- a_k X + (b_k A + c_k A^2) X          (standard form)
 *
 * The Gram form (same article, "Algorithm advantages ..." and "Stability
 * challenges and solutions") iterates in the n x n space instead:
 * R = X X^T, Q = I; per step Z = a_k I + b_k R + c_k R^2, Q <- Z Q,
 * R <- Z R Z; a restart before step k sets X <- Q X, R <- X X^T, Q <- I; the
 * result is Q X.  In exact arithmetic both forms give the same matrix.
 *
 * Error behaviour.  Arguments are checked on the host before anything is
 * enqueued; a bad argument returns an error code and enqueues nothing.
 * A HIP launch failure returns NS_ERR_HIP (the stream may then hold part of
 * the work).  Non-finite results are reported asynchronously through the
 * optional device status word (ns_options.d_status).
 */
#ifndef NSORTHO_H
#define NSORTHO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A HIP stream (hipStream_t); NULL is the default stream. */
typedef void* ns_stream_t;

typedef enum {
  NS_OK = 0,
  NS_ERR_INVALID_ARG = 1,       /* a size, pointer, step count or option is out of range */
  NS_ERR_UNSUPPORTED_DTYPE = 2, /* dtype or internal dtype combination not supported */
  NS_ERR_WORKSPACE = 3,         /* workspace missing, misaligned or smaller than required */
  NS_ERR_HIP = 4                /* a HIP runtime call or kernel launch failed */
} ns_status;

typedef enum { NS_BF16 = 0, NS_FP16 = 1, NS_FP32 = 2 } ns_dtype;

typedef enum { NS_STANDARD = 0, NS_GRAM = 1 } ns_mode;

#define NS_MAX_STEPS 16

/* Kinds of kernel launches, for ns_trace. */
typedef enum {
  NS_KERNEL_NORM = 0,      /* sum of squares of the input (HBM read) */
  NS_KERNEL_STAGE = 1,     /* scale, cast, orient to wide, zero-pad (HBM read + write) */
  NS_KERNEL_GRAM = 2,      /* X X^T, inner dimension m (symmetric result) */
  NS_KERNEL_SYM = 3,       /* n x n symmetric products: b A + c A^2, Z' Q, Z' R, Z' V */
  NS_KERNEL_UPDATE = 4,    /* (n x n) X products: a X + B X, Q X */
  NS_KERNEL_THRESHOLD = 5, /* soft-threshold select and split */
  NS_KERNEL_MOMENTUM = 6   /* Muon momentum update (HBM read + write) */
} ns_kernel_kind;

/* Optional launch trace, for measuring kernels on the caller's stream.
 * Host memory owned by the caller.  When ns_options.trace is not NULL, each
 * launch whose kind bit is set in kind_mask is given events[2*i] and
 * events[2*i+1] (i = count before the launch; the caller creates the events
 * with timing enabled) as the start and stop events of hipExtLaunchKernel,
 * so hipEventElapsedTime on the pair gives that kernel's run time.  Tracing
 * leaves the GPU idle for a few microseconds around each recorded launch;
 * kinds[i], flops[i] and bytes[i]
 * receive its kind, its algorithmic FLOPs (symmetric results counted at
 * half the dense cost; all matrices of a batch) and its algorithmic HBM
 * bytes (one read of each input and one write of each output).  count is
 * incremented per recorded launch; launches past capacity are not recorded.
 * flops and bytes may be NULL. */
typedef struct ns_trace {
  void** events;
  int32_t* kinds;
  double* flops;
  double* bytes;
  int32_t capacity;
  int32_t count;
  uint32_t kind_mask;
} ns_trace;

typedef struct ns_options {
  /* Gram form only.  Bit k (1 <= k <= steps) set: restart before step k
   * (X <- Q X, R <- X X^T, Q <- I).  0 is the naive Gram iteration.
   * Default (1u << 4): one restart, before step 4. */
  uint32_t restart_mask;
  /* Added to ||X||_F before dividing.  Default 1e-7.  A zero matrix gives a
   * zero result. */
  float eps;
  /* Operand type of the matrix products: -1 = automatic (NS_FP16 for bf16
   * and fp16 input, NS_FP32 for fp32 input), NS_FP16 or NS_BF16 for 16-bit
   * input, NS_FP32 for fp32 input.  Products always accumulate in fp32. */
  int32_t internal;
  /* Optional device int32.  When not NULL, kernels set it to 1 if any output
   * element is NaN or Inf.  The caller clears it; it is never cleared here. */
  int32_t* d_status;
  /* Optional launch trace (see ns_trace); NULL for none. */
  ns_trace* trace;
  /* Tile edge of the matrix products: 0 = automatic (a cost estimate for
   * MI355X picks it from the shape and batch), or 128, 192 or 256 (192 and
   * 256 for 16-bit products only).  Results do not depend on it beyond
   * fp32 accumulation order; it changes the workspace size. */
  int32_t tile;
} ns_options;

/* Fill *opt with the defaults above. */
void ns_options_default(ns_options* opt);

/* Bytes of device workspace ns_orthogonalize_batched needs for `batch`
 * matrices of rows x cols (ns_orthogonalize: batch = 1).  Returns 0 for
 * invalid arguments.  Host only; touches no device. */
size_t ns_workspace_size(int64_t rows, int64_t cols, int64_t batch,
                         ns_dtype dtype, ns_mode mode, const ns_options* opt);

/*
 * Orthogonalize one rows x cols matrix in place.
 *
 *   X        device pointer, row-major, element (i, j) at X[i * ld + j],
 *            dtype `dtype`; read as input, overwritten with the result.
 *   rows, cols  >= 1.  The pages' n x m matrix is min x max of these;
 *            n <= 65536 and m <= 2^24 (fp32 input: 2^23), else
 *            NS_ERR_INVALID_ARG.
 *   ld       leading dimension in elements, >= cols.
 *   steps    1..NS_MAX_STEPS Newton-Schulz steps (the pages use 5).
 *   a, b, c  host arrays of `steps` floats: step k uses (a[k-1], b[k-1],
 *            c[k-1]).  Muon's tuned triple is (3.4445, -4.7750, 2.0315).
 *   mode     NS_STANDARD or NS_GRAM.
 *   opt      NULL for the defaults.
 *   workspace, workspace_bytes   device memory of at least
 *            ns_workspace_size(...) bytes, 256-byte aligned, owned by the
 *            caller; its contents on entry do not matter.
 *   stream   the HIP stream all work is enqueued on.
 *
 * Gram form with 16-bit internal operands: the product of |a_k| over any run
 * of steps without a restart must stay below 2^15 (the accumulated Q is held
 * in 16 bits); otherwise NS_ERR_INVALID_ARG.
 */
ns_status ns_orthogonalize(void* X, int64_t rows, int64_t cols, int64_t ld,
                           ns_dtype dtype, int32_t steps, const float* a,
                           const float* b, const float* c, ns_mode mode,
                           const ns_options* opt, void* workspace,
                           size_t workspace_bytes, ns_stream_t stream);

/*
 * Orthogonalize `batch` independent rows x cols matrices in place, each
 * stage launched once for all of them (MoE experts; Gram-NS essay on
 * showapi.com, section on many experts in one kernel, and the Kimi K2 expert
 * shapes in the Gram-NS article's "Performance comparison" section).
 * Matrix e starts at X + e * batch_stride elements; other arguments as for
 * ns_orthogonalize.  batch_stride >= rows * ld; 1 <= batch <= 65535, and
 * batch * ceil(n / 128) * ceil(m / 128) < 2^31 (the update's tile count),
 * else NS_ERR_INVALID_ARG.
 */
ns_status ns_orthogonalize_batched(void* X, int64_t batch, int64_t rows,
                                   int64_t cols, int64_t ld,
                                   int64_t batch_stride, ns_dtype dtype,
                                   int32_t steps, const float* a,
                                   const float* b, const float* c,
                                   ns_mode mode, const ns_options* opt,
                                   void* workspace, size_t workspace_bytes,
                                   ns_stream_t stream);

/*
 * ROOT soft-threshold split (ROOT optimizer summary on reportify.cn,
 * "technical innovations of ROOT"): M = B + O with
 *
 *     O = sign(M) max(|M| - lambda, 0),   B = clip(M, -lambda, lambda).
 *
 *   M        device pointer to numel contiguous elements of `dtype` (read).
 *   B        device pointer to numel elements (written; may equal M).
 *   O        device pointer to numel elements, or NULL to skip it.
 *   lambda   >= 0: use it.  < 0: lambda = mult * median|M|, with the median
 *            the ceil(numel/2)-th smallest |M| (1-based), found exactly
 *            on the device by a radix select over the bit patterns.
 *   d_lambda_out  optional device float receiving lambda (fp32).
 *   workspace   device memory of ns_soft_threshold_workspace_size(...)
 *            bytes, 256-byte aligned.
 * B is rounded to `dtype` (clipped entries become lambda rounded to nearest
 * even); O is computed as M - B in fp32 and rounded.  NaN inputs pass
 * through to B.  1 <= numel <= 2^32 - 1 (the select's bin counts are
 * 32-bit); otherwise NS_ERR_INVALID_ARG, and the workspace query returns 0.
 */
size_t ns_soft_threshold_workspace_size(int64_t numel, ns_dtype dtype);

ns_status ns_soft_threshold_split(const void* M, void* B, void* O,
                                  int64_t numel, ns_dtype dtype, float lambda,
                                  float mult, float* d_lambda_out,
                                  void* workspace, size_t workspace_bytes,
                                  ns_stream_t stream);

/*
 * One Muon optimizer step on `batch` equal-shape weight matrices (batch = 1
 * for one matrix):
 *
 *     M <- momentum * M + G
 *     U  = G + momentum * M        (nesterov != 0)   or   U = M
 *     W <- W - lr * NS(U)
 *
 * (Gram Newton-Schulz article on itsolotime.com, "Algorithm advantages
 * ...": Muon's update takes the polar factor of the momentum, with a
 * momentum coefficient and a learning rate; Muon / NanoGPT article,
 * "Engineering reproduction checklist": momentum 0.95 with Nesterov, five
 * Newton-Schulz steps.)  NS(U) is exactly what ns_orthogonalize_batched
 * computes for U with the same steps, coefficients, mode and options; no
 * shape-dependent factor is applied to lr.
 *
 *   W        device, dtype `dtype`; matrix e at W + e * batch_stride,
 *            row-major with leading dimension ld; updated in place.
 *   G        device, same dtype and layout as W; read only.
 *   M        device fp32 momentum, same layout as W (ld and batch_stride in
 *            elements); updated in place.
 *   lr       finite learning rate; momentum in [0, 1).
 *   workspace   ns_muon_workspace_size(...) bytes, 256-byte aligned.
 * U is formed in fp32 and rounded to `dtype` before the orthogonalization;
 * the new W is W + (-lr) * O in fp32 from O rounded to `dtype`, rounded
 * once more to `dtype`.  d_status (if set) flags non-finite entries of O.
 * Other arguments and errors as for ns_orthogonalize_batched.
 */
size_t ns_muon_workspace_size(int64_t rows, int64_t cols, int64_t batch,
                              ns_dtype dtype, ns_mode mode,
                              const ns_options* opt);

ns_status ns_muon_step(void* W, const void* G, float* M, int64_t batch,
                       int64_t rows, int64_t cols, int64_t ld,
                       int64_t batch_stride, ns_dtype dtype, float lr,
                       float momentum, int32_t nesterov, int32_t steps,
                       const float* a, const float* b, const float* c,
                       ns_mode mode, const ns_options* opt, void* workspace,
                       size_t workspace_bytes, ns_stream_t stream);

/* Static description of a status code. */
const char* ns_status_string(ns_status s);

/* Library version as 10000 * major + 100 * minor + patch. */
int32_t ns_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NSORTHO_H */
