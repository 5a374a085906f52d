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
 * the work).  Non-finite values are reported asynchronously through the
 * optional device status word (see "Status word" below).
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
  NS_ERR_HIP = 4,               /* a HIP runtime call or kernel launch failed */
  NS_ERR_NONFINITE = 5          /* a NaN or Inf was produced on the device; reported only
                                   through the device status word, never returned */
} ns_status;

/*
 * Status word.  An optional device int32 owned by the caller, who clears it
 * before the call; kernels only OR bits into it, so one word may collect
 * several calls.  When any kernel of the call produces a NaN or Inf (or,
 * for stored 16-bit values, a value that rounds to Inf) it ORs in
 * NS_ERR_NONFINITE together with one NS_STATUS_AT_* bit naming where:
 * NS_STATUS_CODE(word) is then NS_ERR_NONFINITE, and NS_OK while the word
 * is clear of it.  The Gram-NS article ("Stability challenges and
 * solutions") names this failure: in half precision the Gram matrix of the
 * naive iteration can develop negative eigenvalues and the iteration
 * diverges to Inf.  NS_STATUS_GUARD_RESTART reports an on-demand restart of
 * the guarded Gram iteration (ns_options.guard); it is not an error.
 */
#define NS_STATUS_CODE(word) ((ns_status)((word) & 0xff))
#define NS_STATUS_AT_INPUT (1 << 8)    /* the input's Frobenius norm is not finite */
#define NS_STATUS_AT_STATE (1 << 9)    /* an n x n intermediate: A, b A + c A^2 (standard form);
                                          R, Z', Q, V (Gram form) */
#define NS_STATUS_AT_ITERATE (1 << 10) /* an intermediate X (between steps, or at a restart) */
#define NS_STATUS_AT_OUTPUT (1 << 11)  /* the result written to the caller's matrix */
#define NS_STATUS_AT_SPLIT (1 << 12)   /* soft-threshold split: lambda, B or O */
#define NS_STATUS_GUARD_RESTART (1 << 16)
/* With NS_STATUS_GUARD_RESTART: the guard restarted before step k, 2 <= k <= 16. */
#define NS_STATUS_GUARD_STEP(k) ((int32_t)(1u << (15 + (k))))

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
  /* Operand type of the matrix products: -1 = automatic, NS_FP16 for bf16
   * and fp16 input, NS_FP32 for fp32 input; any other value (NS_BF16
   * included) gives NS_ERR_UNSUPPORTED_DTYPE.  Products always accumulate in
   * fp32.  bf16 operands are not offered: with 8 mantissa bits in every
   * stored intermediate the iteration misses the 1e-2 relative error bar
   * for 16-bit input (the Gram-NS article keeps float16 in the key steps). */
  int32_t internal;
  /* Optional device status word (see "Status word").  Kernels check their
   * results for NaN and Inf only when it is set. */
  int32_t* d_status;
  /* Optional launch trace (see ns_trace); NULL for none. */
  ns_trace* trace;
  /* Tile edge of the matrix products: 0 = automatic (a cost estimate for
   * MI355X picks it from the shape and batch), or 128, 192 or 256 (192 and
   * 256 for 16-bit products only).  Results do not depend on it beyond
   * fp32 accumulation order; it changes the workspace size. */
  int32_t tile;
  /* Gram form only: restarts on demand (the Gram-NS article's restart,
   * "Stability challenges and solutions", triggered by the state instead of
   * a fixed step).  0 (default) = off.  theta > 0: after step k forms Q, a
   * restart before step k + 1 is scheduled, matrix by matrix and on the
   * device, when max_i |Q_ii| * |a_{k+1}| > theta, or when a diagonal entry
   * of R is negative or not finite.  Q's eigenvalue in the directions of
   * the smallest singular values grows like the product of the a_j since
   * the last restart, and its fp16 rounding error with it; 100 restarts an
   * ill-conditioned input where the fixed schedule does and lets a
   * well-conditioned one run without a restart.  Restarts of restart_mask
   * still happen.  Each on-demand restart ORs NS_STATUS_GUARD_RESTART |
   * NS_STATUS_GUARD_STEP(k) into the status word.  Must be finite. */
  float guard_threshold;
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
 * Coefficient range: every stored intermediate must stay below half of its
 * storage type's largest value in exact arithmetic, or the call returns
 * NS_ERR_INVALID_ARG.  The check follows one singular value s in [0, 1]
 * of the scaled input through the steps (every matrix of both forms is a
 * function of the singular values, and its entries are bounded by its
 * spectral norm): X (held as 2^10 X in fp16), A = s^2 and b A + c A^2
 * (standard form); R, Z' = b R + c R^2, Q, V = R Z and X at a restart
 * (Gram form); and the result in the caller's dtype.  The 16-bit limit is
 * 2^15.  For the Gram form the accumulated Q reaches the product of the
 * a_k between restarts, so a naive run of nine tuned steps is refused.
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
 * Grouped call: `count` matrices that share one shape up to orientation,
 * each with its own storage, every stage launched once for all of them (the
 * Gram-NS essay on showapi.com, sections 2.3 and 4.1: experts launched
 * together and advancing in step).  With n <= m the oriented shape, member i
 * is the matrix at members[i].data (device memory), n x m with leading
 * dimension ld when transposed == 0, or m x n (stored transposed, like a
 * tall weight) with leading dimension ld when transposed == 1; it is
 * orthogonalized in place in its own layout.  So the 768 x 3072 and
 * 3072 x 768 matrices of a transformer's MLP go in one group.
 *
 *   members  host array of `count` entries, written into the workspace on
 *            the stream by the call (through kernel arguments, no host
 *            copy or synchronization), so it may be reused once the call
 *            returns; data not NULL,
 *            transposed 0 or 1, reserved 0, ld >= m (transposed == 0) or
 *            >= n (transposed == 1), else NS_ERR_INVALID_ARG.
 *   count    1..65535 and n, m as for ns_orthogonalize_batched's shape.
 *   workspace   ns_grouped_workspace_size(n, m, count, ...) bytes.
 * Every member's result equals ns_orthogonalize's on that matrix bit for
 * bit.  Members must not overlap.  Other arguments and errors as for
 * ns_orthogonalize_batched.
 */
typedef struct ns_matrix {
  void* data;
  int64_t ld;
  int32_t transposed;
  int32_t reserved;
} ns_matrix;

size_t ns_grouped_workspace_size(int64_t n, int64_t m, int64_t count,
                                 ns_dtype dtype, ns_mode mode,
                                 const ns_options* opt);

ns_status ns_orthogonalize_grouped(const ns_matrix* members, int64_t count,
                                   int64_t n, int64_t m, ns_dtype dtype,
                                   int32_t steps, const float* a,
                                   const float* b, const float* c,
                                   ns_mode mode, const ns_options* opt,
                                   void* workspace, size_t workspace_bytes,
                                   ns_stream_t stream);

/*
 * ns_orthogonalize_batched without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * and harnesses that forbid hipMalloc).  It calls no allocating routine: its
 * buffers live in a device array of ns_static_scratch_bytes() bytes (64 MiB)
 * that the library holds on every device it runs on until the process
 * ends.  A call whose ns_workspace_size(...) exceeds that returns
 * NS_ERR_WORKSPACE and enqueues nothing; it fits matrices up to about
 * 1024 x 4096 (16-bit input), or batches of the same total size.  Results
 * equal ns_orthogonalize_batched's bit for bit (same kernels).  Nothing in
 * the array needs to start at zero; every call overwrites what it reads.
 * All calls on one device share the one array: calls that overlap on one
 * device (different streams, or threads) race and must be ordered by the
 * caller.  batch = 1 with batch_stride = rows * ld is a single matrix.
 * NS_ERR_HIP if the runtime cannot give the array's device address.
 */
size_t ns_static_scratch_bytes(void);

ns_status ns_orthogonalize_static(void* X, int64_t batch, int64_t rows,
                                  int64_t cols, int64_t ld,
                                  int64_t batch_stride, ns_dtype dtype,
                                  int32_t steps, const float* a,
                                  const float* b, const float* c,
                                  ns_mode mode, const ns_options* opt,
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
 *   d_lambda_out  optional device float receiving lambda.  lambda is
 *            formed in fp32: mult * median rounded once to fp32 (the
 *            median of 16-bit or fp32 input is exact in fp32), and every
 *            clip decision compares |M| with that fp32 value.
 *   d_status optional device status word (see "Status word"): a NaN or Inf
 *            in lambda, B or O ORs in NS_ERR_NONFINITE | NS_STATUS_AT_SPLIT.
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
                                  int32_t* d_status, void* workspace,
                                  size_t workspace_bytes, ns_stream_t stream);

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

/*
 * The kernel builds one call would launch, for inspection (host only;
 * touches no device).  Arguments as for ns_workspace_size, plus the step
 * count.  Writes a NUL-terminated, space-separated list of the distinct
 * builds (see below for the order) into buf (truncated to len bytes; buf may be NULL)
 * and returns the length the whole list needs including the NUL, or -1 for
 * invalid arguments.  Entries: sumsq<io>, stage<io,op>; xxt<op,tile,form>
 * (X X^T) and nn<op,tile,form> (n x n products); upd<op,op,tile,form,e>
 * (intermediate X updates) and out<op,io,tile,form,e> (the final product);
 * op is the product operand type, form one of tile (a work-group per tile),
 * loop (a persistent grid), pair and pairloop (the same, built for two
 * work-groups per compute unit), e is E when the a X term is taken from
 * LDS, Eg when it is read from global memory and noE when there is none.
 * A trailing ",nt" marks the pair/pairloop builds whose output stores are
 * non-temporal, taken by a launch that writes more than 256 MiB (the
 * MI355X MALL's size) and reads no guard flags or member table.  A ",x"
 * before it marks the builds that read such extended arguments: every
 * launch of a guarded Gram call (opt->guard_threshold > 0) except the
 * first step's n x n product, and a grouped call's final product.  The list
 * follows the call's launches by kind: the norm and staging passes, the
 * X X^T builds, the n x n builds, the intermediate updates, the final
 * product.
 */
int64_t ns_plan_kernels(int64_t rows, int64_t cols, int64_t batch,
                        ns_dtype dtype, ns_mode mode, int32_t steps,
                        const ns_options* opt, char* buf, size_t len);

/*
 * The same list for a grouped call (ns_orthogonalize_grouped) of `count`
 * matrices of shape n x m up to orientation (n <= m; -1 otherwise).  For
 * inspection only, like ns_plan_kernels.
 */
int64_t ns_plan_kernels_grouped(int64_t n, int64_t m, int64_t count,
                                ns_dtype dtype, ns_mode mode, int32_t steps,
                                const ns_options* opt, char* buf, size_t len);

/* Static description of a status code. */
const char* ns_status_string(ns_status s);

/* Library version as 10000 * major + 100 * minor + patch. */
int32_t ns_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NSORTHO_H */
