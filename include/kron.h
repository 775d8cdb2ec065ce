/*
 * libkron -- Kronecker-factored linear layers and Kronecker-sparse matmuls on AMD
 * Instinct MI355X (gfx950).  Plain C ABI: device pointers, sizes, a HIP stream.
 *
 * Notation (Kronecker layer tutorial, intro and "Build W, then multiply"):
 *   S      p x q                sparsity mask (l1-penalised); NULL means S == 1
 *   A      r x p x q            A_i, i = 0..r-1
 *   B      r x m x n            B_i
 *   C_i    = S o A_i            (elementwise product)
 *   W      = sum_i kron(C_i, B_i), (p*m) x (q*n), oriented in x out
 *   y      = x W + bias         x is N x (p*m), y is N x (q*n), bias has q*n entries
 * The library never forms W.  Each row x_n is read as a p x m row-major matrix X_n
 * and the row of y is vec_row(sum_i C_i^T X_n B_i) + bias (tutorial, "The vec trick"
 * and "The vec trick without the loop"): the X_n B_i products stay on chip.
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers to dense row-major fp32 (or bf16 where
 *     stated) arrays, base address aligned to 16 bytes.  The caller owns all memory,
 *     including any workspace; no entry point allocates or frees device memory.
 *   - Calls are asynchronous on `stream` (0 = the null stream).  No host sync.
 *   - Arguments are validated on the host before any HIP call.  On error nothing is
 *     launched, nothing is written, and a kron_status_t other than KRON_OK is
 *     returned; kron_last_error() then holds a detail string for the calling thread.
 *     A failed kernel launch returns KRON_E_HIP.  Nothing aborts, prints or throws.
 *   - Gradient outputs are overwritten, not accumulated.
 *   - Results are deterministic: the same inputs on the same device give bitwise
 *     identical outputs (fixed-order reductions, no floating-point atomics).
 *   - Calls are thread-safe; the only global state is the per-thread error string.
 */
#ifndef LIBKRON_KRON_H
#define LIBKRON_KRON_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KRON_ABI_VERSION 1

typedef enum {
  KRON_OK = 0,
  KRON_E_NULL = 1,        /* a required pointer is NULL (or an optional pair is inconsistent) */
  KRON_E_SHAPE = 2,       /* a size is out of range or sizes disagree                       */
  KRON_E_ALIGN = 3,       /* a pointer is not 16-byte aligned                                */
  KRON_E_ALIAS = 4,       /* an output overlaps an input or another output                   */
  KRON_E_DTYPE = 5,       /* unknown dtype                                                   */
  KRON_E_WORKSPACE = 6,   /* workspace missing or smaller than required                      */
  KRON_E_UNSUPPORTED = 7, /* valid, but beyond what this build supports (see limits below)   */
  KRON_E_HIP = 8,         /* a HIP call failed; kron_last_error() has hipGetErrorString      */
  KRON_E_ARG = 9          /* another invalid argument (step < 1, negative count, bad flag)   */
} kron_status_t;

typedef enum { KRON_F32 = 0, KRON_BF16 = 1 } kron_dtype_t;

/* kron_shape_t.flags */
#define KRON_RELU_OUT     1u  /* fwd: y = max(x W + bias, 0)                              */
#define KRON_DX_RELU_MASK 2u  /* bwd: dX = (dY W^T) o [x > 0]  (x is the output of a ReLU) */
/* hint, for S with whole rows zero (e.g. after l1 pruning): the forward's 32- and 64-row
 * block layouts and the 32x32-block, r = 4 backward build the sparsity map of C = S o A_i
 * (its rows with a nonzero entry in any rank, compacted to the front) and run only the
 * 16-row tiles that hold such rows (tutorial, intro: zeros of S give zero blocks of W): in
 * the forward both products, in the backward G = C dY, dX and dB (Z and dC stay dense:
 * dS needs dC everywhere).  The forward also skips the stage-2 steps over every 16 x 16
 * block of S (rows in map order) that is entirely zero, e.g. a block-diagonal mask.
 * Results equal the dense path's up to the order of the sums.  Costs a little on an S
 * with no empty row tile or block; other kernels ignore it. */
#define KRON_SPARSE_ROWS  4u

typedef struct {
  int64_t N;                 /* rows, >= 0                              */
  int32_t p, q, m, n, r;     /* in = p*m, out = q*n; each >= 1          */
  uint32_t flags;            /* KRON_RELU_OUT | KRON_DX_RELU_MASK | KRON_SPARSE_ROWS */
} kron_shape_t;

/* Limits of this build: 1 <= p,q,m,n <= 4096, 1 <= r <= 64, p*m and q*n <= 65536,
 * N <= 2^31 - 1; r*p*q and r*m*n <= 2^24.  Small square blocks (m = n in {2, 4, 8},
 * p and q multiples of 16, r <= 16) always run; other shapes whose per-row working set
 * does not fit in one workgroup's LDS return KRON_E_UNSUPPORTED. */

int32_t kron_abi_version(void);
const char* kron_status_str(kron_status_t status);
/* Detail string of the last failed call on this thread ("" if none).  Valid until the
 * next call on the same thread. */
const char* kron_last_error(void);

/* Host-only shape validation (no HIP call); returns KRON_OK or the error. */
kron_status_t kron_linear_check(const kron_shape_t* shape);

/* Bytes of workspace kron_linear_bwd needs for this shape (0 on an invalid shape).
 * Depends only on the shape. */
size_t kron_linear_bwd_workspace_bytes(const kron_shape_t* shape);

/*
 * Forward: y = x W + bias (tutorial, "The vec trick without the loop": the rank is
 * fused into one pass, the X_n B_i products never leave the chip).  Terms with
 * S[j,k] == 0 contribute nothing (zero blocks of W, tutorial intro).
 *   x    [N, p*m]   S [p, q] or NULL   A [r, p, q]   B [r, m, n]
 *   bias [q*n] or NULL                  y [N, q*n]  (must not overlap any input)
 */
kron_status_t kron_linear_fwd(const kron_shape_t* shape, const float* x, const float* S,
                              const float* A, const float* B, const float* bias, float* y,
                              hipStream_t stream);

/*
 * Backward of y = x W + bias for the upstream gradient dy [N, q*n]:
 *   dx    = dy W^T                      [N, p*m]   (NULL: not computed)
 *   dS    = sum_i A_i o dC_i            [p, q]     (must be NULL iff S is NULL)
 *   dA_i  = S o dC_i                    [r, p, q]  (dC_i when S is NULL)
 *   dB_i  = sum_n X_n^T G_{n,i}         [r, m, n]  with G_{n,i} = C_i dY_n
 *   dbias = sum_n dy_n                  [q*n]      (NULL: not computed)
 * where dC_i = sum_n (X_n B_i) dY_n^T.  X_n B_i is recomputed on chip rather than
 * stored by the forward.  With KRON_DX_RELU_MASK, dx is multiplied by [x > 0].
 * N == 0 is valid: the parameter gradients are set to zero.
 * workspace: device buffer of at least kron_linear_bwd_workspace_bytes(shape) bytes,
 * 256-byte aligned; its contents on entry are ignored.  Outputs must not overlap each
 * other, the inputs or the workspace.
 */
kron_status_t kron_linear_bwd(const kron_shape_t* shape, const float* x, const float* S,
                              const float* A, const float* B, const float* dy,
                              float* dx, float* dS, float* dA, float* dB, float* dbias,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kron_linear_bwd without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same operation, arguments, checks and results as kron_linear_bwd; the
 * partial-row workspace is a fixed scratch array inside the library instead, one copy
 * per GPU, KRON_NOALLOC_SCRATCH_BYTES long, held until the process ends.  The call
 * itself allocates and frees nothing.
 *   - A shape whose kron_linear_bwd_workspace_bytes exceeds KRON_NOALLOC_SCRATCH_BYTES
 *     is refused with KRON_E_UNSUPPORTED before anything runs.
 *   - The first call made with a device current looks up that device's scratch address
 *     (hipGetSymbolAddress); a failure there returns KRON_E_HIP.
 *   - Every call on one GPU uses that GPU's one scratch array: calls that may overlap on
 *     one GPU (different streams, different host threads) race on it and must be
 *     serialised by the caller.  Calls ordered on one stream are safe.  Nothing in the
 *     scratch needs to start at zero: each call writes the part it reads.
 */
#define KRON_NOALLOC_SCRATCH_BYTES (32u << 20)
kron_status_t kron_linear_bwd_noalloc(const kron_shape_t* shape, const float* x, const float* S,
                                      const float* A, const float* B, const float* dy,
                                      float* dx, float* dS, float* dA, float* dB, float* dbias,
                                      hipStream_t stream);

/*
 * Saved-intermediate variant of the layer: the forward also stores Z_{n,i} = X_n B_i (the
 * first contraction of the tutorial's "The vec trick without the loop", which the
 * tutorial's "Takeaways" recompute in the backward) for the first ranks, and the backward
 * reads those back instead of recomputing them.  That trades HBM traffic (8 KB per row,
 * written once and read once, for the 1024 x 1024 layer at m = 32, r = 4: Z of ranks 0
 * and 1) for a tenth of the backward's products; saving more ranks makes the forward
 * HBM-bound and the pair slower.
 *
 * kron_linear_zcache_bytes: bytes of the cache for shape->N rows; 0 when the shape has no
 *   saved-intermediate path (then use kron_linear_fwd / kron_linear_bwd) or N == 0.
 *   Available for p = q = m = n = 32 with r = 4.
 *
 * kron_linear_fwd_save: kron_linear_fwd (same arguments, checks and y, bit for bit) that
 *   also fills zcache [zcache_bytes >= kron_linear_zcache_bytes(shape)], 16-byte aligned,
 *   disjoint from every input and from y.  The cache's layout is private to the library.
 *
 * kron_linear_bwd_saved: kron_linear_bwd (same arguments, checks and results up to
 *   rounding) that reads the saved Z from zcache.  zcache must hold what
 *   kron_linear_fwd_save wrote for the same shape, x and B (A, S and bias may have changed
 *   since: Z depends on x and B only); nothing checks this, and a stale cache gives wrong
 *   dS and dA.
 *
 * Both return KRON_E_UNSUPPORTED for a shape without the path, KRON_E_ARG with
 * KRON_SPARSE_ROWS, KRON_E_WORKSPACE for a short cache and KRON_E_NULL for a missing one
 * (N > 0).
 */
size_t kron_linear_zcache_bytes(const kron_shape_t* shape);
kron_status_t kron_linear_fwd_save(const kron_shape_t* shape, const float* x, const float* S,
                                   const float* A, const float* B, const float* bias, float* y,
                                   float* zcache, size_t zcache_bytes, hipStream_t stream);
kron_status_t kron_linear_bwd_saved(const kron_shape_t* shape, const float* x, const float* S,
                                    const float* A, const float* B, const float* dy,
                                    const float* zcache, size_t zcache_bytes,
                                    float* dx, float* dS, float* dA, float* dB, float* dbias,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * bf16 layer (mixed precision; the tutorial's "Takeaways" name a mixed-precision rerun as
 * the next step).  Same operation as kron_linear_fwd / kron_linear_bwd with bf16 storage
 * (bfloat16 bit patterns) for x, S, A, B, bias, dy and the outputs y and dx; products
 * run on bf16 matrix instructions with fp32 accumulation.  C_i = S o A_i is formed in
 * fp32 and rounded to bf16, and X_n B_i and G_{n,i} are rounded to bf16 before their
 * second product (round to nearest even); y and dx are rounded once at the end.  The
 * parameter gradients dS, dA, dB and dbias are fp32.
 * Shapes: (p, q, m, n, r) in {(32,32,32,32,1), (32,32,32,32,2), (32,32,32,32,4),
 * (16,16,64,64,2)} and the GPT-2 small FFN pair (32,64,24,48,r) and (64,32,48,24,r) with
 * r in {1, 2, 4, 8} (a side of 24 runs padded to 32 inside the kernels' tiles); other shapes
 * return KRON_E_UNSUPPORTED.  Pointers as for the fp32 calls (16-byte aligned); workspace
 * from kron_linear_bwd_bf16_workspace_bytes.
 */
size_t kron_linear_bwd_bf16_workspace_bytes(const kron_shape_t* shape);
kron_status_t kron_linear_fwd_bf16(const kron_shape_t* shape, const void* x, const void* S,
                                   const void* A, const void* B, const void* bias, void* y,
                                   hipStream_t stream);
kron_status_t kron_linear_bwd_bf16(const kron_shape_t* shape, const void* x, const void* S,
                                   const void* A, const void* B, const void* dy, void* dx,
                                   float* dS, float* dA, float* dB, float* dbias,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Kronecker-sparse matmul ("Fast Inference with Kronecker-Sparse Matrices", abstract):
 * Y = X K with K of support I_a (x) 1_{b x c} (x) I_d, (a*b*d) x (a*c*d):
 *   Y[n, (al*c + ga)*d + de] = sum_be X[n, (al*b + be)*d + de] * vals[al][de][be][ga]
 *   x    [N, a*b*d]  fp32 or bf16 (in_dtype)
 *   vals [a, d, b, c] same dtype as x
 *   y    [N, a*c*d]  fp32, accumulated in fp32
 * Limits: a*b*d and a*c*d <= 65536.
 */
kron_status_t ks_matmul(int64_t N, int32_t a, int32_t b, int32_t c, int32_t d, int32_t in_dtype,
                        const void* x, const void* vals, float* y, hipStream_t stream);

/*
 * ks_matmul with the output dtype chosen (the same product; "Fast Inference with
 * Kronecker-Sparse Matrices", abstract): out_dtype KRON_F32 gives ks_matmul exactly;
 * KRON_BF16 stores each fp32-accumulated value of y rounded once to bf16 (nearest even),
 * y being [N, a*c*d] bf16 (2-byte elements).  Same limits, alignment and errors as
 * ks_matmul, plus KRON_E_DTYPE for an out_dtype other than KRON_F32 / KRON_BF16.
 */
kron_status_t ks_matmul_out(int64_t N, int32_t a, int32_t b, int32_t c, int32_t d, int32_t in_dtype,
                            int32_t out_dtype, const void* x, const void* vals, void* y,
                            hipStream_t stream);

/*
 * Backward of ks_matmul (by calculus from Y = X K with the KS matrix K of "Fast Inference
 * with Kronecker-Sparse Matrices", abstract):
 *   dx    [N, a*b*d]     fp32:  dx = dy K^T, itself a KS product with the pattern
 *                               (a, c, b, d) and each (alpha, delta) block transposed
 *   dvals [a, d, b, c]   fp32:  dvals[al][de][be][ga] =
 *                               sum_n x[n, (al*b + be)*d + de] * dy[n, (al*c + ga)*d + de]
 * x, vals and dy are in in_dtype (KRON_F32 or KRON_BF16); accumulation is fp32.  dx or
 * dvals may be NULL (not computed); with N = 0, dvals is written as zeros.  Outputs are
 * overwritten.  dvals is summed over rows in a fixed order (bitwise repeatable).
 * workspace: device memory of ks_matmul_bwd_workspace_bytes(...) bytes, 256-byte aligned,
 * owned by the caller; its contents need no initialisation.  Limits: those of ks_matmul for
 * both (a,b,c,d) and (a,c,b,d), and a*b*c*d <= 2^28.  Errors: KRON_E_SHAPE, KRON_E_DTYPE,
 * KRON_E_UNSUPPORTED, KRON_E_NULL, KRON_E_ALIGN, KRON_E_ALIAS, KRON_E_WORKSPACE,
 * KRON_E_HIP.  ks_matmul_bwd_workspace_bytes returns 0 for arguments ks_matmul_bwd rejects.
 */
/*
 * Van Loan rank-r Kronecker projection of a dense W ("Replicating & Extending Krony-PT on
 * GPT-2 Small", section "Core Algorithm - Van Loan Kronecker Decomposition"): factors with
 * sum_i kron(C_i, B_i) the best rank-r Kronecker sum to W in the Frobenius norm, from the
 * leading singular triplets of the rearrangement R[(j*q + k), (a*n + b)] = W[j*m + a, k*n + b]:
 * C_i = sqrt(sigma_i) reshape(u_i, p x q), B_i = sqrt(sigma_i) reshape(v_i, m x n).  The
 * triplets come from block subspace iteration of width s (r <= s <= 32) started from the
 * caller's random block omega and run for iters power iterations; accuracy grows with
 * s - r and iters (the error factor is (sigma_{s+1} / sigma_r)^(2 iters + 1)).  Sign of each
 * pair: the entry of C_i largest in magnitude (first in row-major order) is positive.
 *   W      [p*m, q*n]  fp32 (the layer's in x out orientation)
 *   omega  [m*n, s]    fp32 starting block (e.g. standard normal draws)
 *   C [r, p, q], B [r, m, n], sigma [r]: fp32 outputs (sigma decreasing)
 * workspace: kron_van_loan_workspace_bytes(p, q, m, n, s) bytes, 256-byte aligned, caller
 * owned.  Limits: p*q and m*n <= 8192, p*m and q*n <= 65536, 0 <= iters <= 100.  Errors:
 * KRON_E_SHAPE, KRON_E_ARG, KRON_E_UNSUPPORTED, KRON_E_NULL, KRON_E_ALIGN, KRON_E_ALIAS,
 * KRON_E_WORKSPACE, KRON_E_HIP.  The workspace query returns 0 for rejected shapes.
 */
size_t kron_van_loan_workspace_bytes(int32_t p, int32_t q, int32_t m, int32_t n, int32_t s);
kron_status_t kron_van_loan(int32_t p, int32_t q, int32_t m, int32_t n, int32_t r, int32_t s,
                            int32_t iters, const float* W, const float* omega, float* C, float* B,
                            float* sigma, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One Kronecker-sparse factor of a chain: support I_a (x) 1_{b x c} (x) I_d, values
 * vals[a][d][b][c] (device pointer, dtype of the chain's input).
 */
typedef struct {
  int32_t a, b, c, d;
  const void* vals;
} ks_factor_t;

/*
 * Fused chain y = x K_1 K_2 ... K_n of Kronecker-sparse factors ("Fast Inference with
 * Kronecker-Sparse Matrices", abstract: products of KS factors such as butterfly and
 * Monarch factors; the triple Kronecker product A (x) B (x) C is a three-factor chain by the
 * mixed-product rule).  Each factor maps a*b*d values per row to a*c*d with the index map
 * of ks_matmul; factor f+1 takes what factor f gives.  Intermediate rows stay on chip
 * (fp32); only y is written.
 *   factors  HOST array of nfactors (1..8) ks_factor_t
 *   x        [N, a1*b1*d1]  fp32 or bf16 (in_dtype; every factor's vals in the same dtype)
 *   y        [N, an*cn*dn]  fp32
 * Limits: every row width <= 16384.  Errors: KRON_E_SHAPE (widths that do not chain),
 * KRON_E_ARG (nfactors), KRON_E_NULL, KRON_E_DTYPE, KRON_E_UNSUPPORTED, KRON_E_ALIGN,
 * KRON_E_ALIAS (y over x or any vals), KRON_E_HIP.
 */
kron_status_t ks_chain(int64_t N, int32_t nfactors, const ks_factor_t* factors, int32_t in_dtype,
                       const void* x, float* y, hipStream_t stream);

size_t ks_matmul_bwd_workspace_bytes(int64_t N, int32_t a, int32_t b, int32_t c, int32_t d,
                                     int32_t in_dtype);
kron_status_t ks_matmul_bwd(int64_t N, int32_t a, int32_t b, int32_t c, int32_t d, int32_t in_dtype,
                            const void* x, const void* vals, const void* dy, float* dx, float* dvals,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Fused multi-tensor Adam with an l1 penalty (tutorial, "Setup": Adam update of the
 * training step; intro: l1 penalty on S).  For tensor t and element e:
 *   g  = grads[t][e] + l1[t] * sign(params[t][e])       (sign(0) = 0)
 *   m  = beta1*m + (1-beta1)*g,   v = beta2*v + (1-beta2)*g*g
 *   params -= lr * (m / (1 - beta1^step)) / (sqrt(v / (1 - beta2^step)) + eps)
 * params, grads, m, v, numel and l1 are HOST arrays of length ntensors; the first four
 * hold device pointers.  l1 may be NULL (no penalty).  step >= 1.  Tensors with
 * numel 0 are skipped.  Up to 4096 tensors per call.  The hyper-parameters are taken in
 * double: 1 - beta and the bias corrections are formed on the host in double and
 * rounded once to fp32 (1 - 0.999f in fp32 would be off by 1.3e-5 relative).
 */
kron_status_t kron_adam_l1_step(int32_t ntensors, float* const* params, const float* const* grads,
                                float* const* m, float* const* v, const int64_t* numel,
                                const float* l1, int64_t step, double lr, double beta1, double beta2,
                                double eps, hipStream_t stream);

/*
 * Dense classification head with mean softmax cross-entropy, forward and backward in
 * one call (tutorial, "Setup": the 10-class output layer stays dense; the loss is the
 * cross-entropy):
 *   z = h Wh + bh,  loss = mean_n (logsumexp(z_n) - z_n[label_n])
 *   dz = (softmax(z) - onehot(label)) / N
 *   dWh = h^T dz [K, C],  dbh = sum_n dz [C],  dh = dz Wh^T [N, K]
 * With KRON_DX_RELU_MASK in flags, dh is multiplied by [h > 0].
 *   h [N, K]  Wh [K, C]  bh [C]  labels [N] int64 in [0, C)
 *   loss: one device float.  dh may be NULL.
 * Labels outside [0, C) make the loss NaN (no out-of-bounds access).
 * Limits: 1 <= C <= 64, 1 <= K <= 8192.  workspace as for kron_linear_bwd.
 */
size_t kron_head_ce_workspace_bytes(int64_t N, int32_t K, int32_t C);
kron_status_t kron_head_ce(int64_t N, int32_t K, int32_t C, const float* h, const float* Wh,
                           const float* bh, const int64_t* labels, float* loss, float* dh,
                           float* dWh, float* dbh, uint32_t flags, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * The gradient through a ReLU output (tutorial, "Setup": the hidden layers end in a
 * ReLU): out = dy o [y > 0] for y = max(z, 0), n elements.  out may be dy itself (in
 * place); otherwise out must not overlap y or dy.  Used for a layer whose forward ran
 * with KRON_RELU_OUT, before its kron_linear_bwd.
 */
kron_status_t kron_relu_bwd(int64_t n, const float* y, const float* dy, float* out, hipStream_t stream);

/* kron_l1_penalty flags */
#define KRON_ACCUMULATE 1u    /* add to *loss instead of overwriting it */

/*
 * The l1 penalty on S (tutorial, intro: S is l1-penalised; "Setup": the loss is the
 * cross-entropy plus the model's penalty):
 *   loss[0] = (flags & KRON_ACCUMULATE ? loss[0] : 0) + lam * sum_t sum_e |tensors[t][e]|
 * tensors and numel are HOST arrays of length ntensors (<= 64); tensors holds device
 * pointers.  loss is one device float and must not overlap a tensor.  The sum is taken in
 * fp64 in a fixed order by a single workgroup (meant for S-sized tensors), then rounded
 * once to fp32: bitwise reproducible.  ntensors = 0 sets (or keeps) loss[0].
 */
kron_status_t kron_l1_penalty(int32_t ntensors, const float* const* tensors, const int64_t* numel,
                              float lam, float* loss, uint32_t flags, hipStream_t stream);

/*
 * Subgradient of lam * sum|S| scaled by an upstream scalar gradient g (one device float):
 *   dS = lam * g[0] * sign(S),  sign(0) = 0,  n elements.
 * dS must not overlap S or g.  (kron_adam_l1_step applies the same subgradient inside the
 * update; this call serves autograd-style callers.)
 */
kron_status_t kron_l1_penalty_grad(int64_t n, const float* S, float lam, const float* g, float* dS,
                                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBKRON_KRON_H */
