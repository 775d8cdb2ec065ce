// Internal declarations of libkron: launchers implemented in the .hip files and
// called by the C-ABI layer (kron_api.cpp).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "kron.h"

namespace kron {

// ---------------------------------------------------------------------------------
// Column reduction of per-workgroup partial sums: G partial rows of PW fp32 columns
// (row g holds workgroup g's partial sums); column c is summed over g in a fixed order
// in fp64 and written, scaled, to the segment that covers c.
//
// Storage is blocked by columns: the G values of a block of kRedCols columns are
// contiguous (G x kRedCols floats, block after block), so a producer writes its row as
// whole 128-byte lines and the reduction of a block reads one contiguous range.
// ---------------------------------------------------------------------------------
constexpr int kRedCols = 32;
__host__ __device__ inline int64_t part_floats(int64_t G, int64_t PW) {
  return G * ((PW + kRedCols - 1) / kRedCols) * kRedCols;
}
__host__ __device__ inline int64_t part_index(int64_t G, int64_t g, int64_t col) {
  return (col / kRedCols) * G * kRedCols + g * kRedCols + col % kRedCols;
}
// Row g of the partial sums, from column `off` on.
struct PartRow {
  float* part;
  int64_t G, g, off;
  __device__ float& operator[](int64_t col) const { return part[part_index(G, g, off + col)]; }
  __device__ PartRow operator+(int64_t d) const { return PartRow{part, G, g, off + d}; }
};
struct RedSeg {
  float* dst;          // NULL: skip this segment
  int32_t count;       // columns in this segment
  float scale;
  int32_t accumulate;  // 0: dst = scale * sum;  1: dst += scale * sum
};
constexpr int kMaxRedSeg = 4;
struct RedPlan {
  RedSeg seg[kMaxRedSeg];
  int32_t nseg;
};
hipError_t launch_column_reduce(const float* part, int32_t G, int32_t PW, const RedPlan& plan,
                                hipStream_t stream);

// ---------------------------------------------------------------------------------
// Kronecker layer.
// ---------------------------------------------------------------------------------
struct LayerArgs {
  int64_t N;
  int32_t p, q, m, n, r;
  uint32_t flags;
  const float* x;
  const float* S;
  const float* A;
  const float* B;
  const float* bias;
  const float* dy;
  float* y;
  float* dx;
  float* dS;
  float* dA;
  float* dB;
  float* dbias;
  float* part;   // workspace: G partial rows of PW columns (column-blocked)
  int32_t dx_accumulate;   // backward: dx += this call's dX (before the optional mask)
  float* zc;     // saved Z_i = X B_i: written by the forward, read by the backward (NULL: none)
};

// Partial sums of one backward workgroup, in this order:
//   dB (r*m*n) | dA (r*p*q) | dS (p*q) | dbias (q*n)
// A workgroup accumulates dC_i over its rows and turns it into its share of
// dA_i = S o dC_i and dS = sum_i A_i o dC_i before writing (both are linear in dC), so
// one fixed-order column reduction yields every parameter gradient.  The dS slot is
// present (and zero) when S is absent, so the width depends on the shape only.
__host__ __device__ inline int64_t partial_width(int64_t p, int64_t q, int64_t m, int64_t n, int64_t r) {
  return r * m * n + r * p * q + p * q + q * n;
}

// Generic path: any shape whose per-tile working set fits in LDS.
int generic_fwd_rows_per_tile(int p, int q, int m, int n);        // 0: unsupported
int generic_bwd_rows_per_tile(int p, int q, int m, int n, bool want_dx);
int generic_bwd_groups(int64_t N, int T);
hipError_t launch_fwd_generic(const LayerArgs& a, hipStream_t s);
hipError_t launch_bwd_generic(const LayerArgs& a, int G, hipStream_t s);

// Matrix-core path for the shapes in its table (see kron_mfma.hip).
bool mfma_fwd_supported(int p, int q, int m, int n, int r);
bool mfma_bwd_supported(int p, int q, int m, int n, int r);
// Floats per row of the saved Z_i = X B_i that the forward writes and the backward reads
// back (0: the shape has no saved path).
int mfma_zcache_row_floats(int p, int q, int m, int n, int r);
int mfma_bwd_groups(int64_t N, int p, int q, int m, int n, int r);
// bf16 layer (kron_bf16.hip): bf16 tensors as 16-bit patterns, fp32 parameter gradients.
struct LayerArgsBf16 {
  int64_t N;
  int32_t p, q, m, n, r;
  uint32_t flags;
  const uint16_t* x;
  const uint16_t* S;
  const uint16_t* A;
  const uint16_t* B;
  const uint16_t* bias;
  const uint16_t* dy;
  uint16_t* y;
  uint16_t* dx;
  float* part;   // workspace: G partial rows of PW columns (column-blocked)
};
bool bf16_supported(int p, int q, int m, int n, int r);
int bf16_bwd_groups(int64_t N, int p, int q, int m, int n, int r);
hipError_t launch_fwd_bf16(const LayerArgsBf16& a, hipStream_t s);
hipError_t launch_bwd_bf16(const LayerArgsBf16& a, int G, hipStream_t s);

// Small-block matrix-core path (kron_small.hip): m = n in {2, 4, 8}, p and q multiples
// of 16, r <= 16.  The backward writes two partial arrays into the workspace: dB rows
// (G1 x r*m*n) at float offset 0 and [dC | dbias] rows (G2 x (r*p*q + q*n)) at off2.
struct SmallBwdPlan {
  int G1, G2;
  int64_t rpg;          // rows per row group of the dC kernel
  int64_t PW1, PW2;     // partial widths
  int64_t off2;         // float offset of the second partial array
  int64_t ws_floats;    // workspace floats
};
bool small_supported(int p, int q, int m, int n, int r);
SmallBwdPlan small_bwd_plan(int64_t N, int p, int q, int m, int n, int r);
hipError_t launch_fwd_small(const LayerArgs& a, hipStream_t s);
// Runs the whole backward: kernels, both column reductions and the dA / dS epilogue.
hipError_t launch_bwd_small(const LayerArgs& a, const SmallBwdPlan& pl, hipStream_t s);

// Ranks per chunk when a backward with r ranks runs as r / chunk passes of the
// chunk-rank MFMA kernel (dX accumulated over the passes), else 0.
int mfma_bwd_chunk(int p, int q, int m, int n, int r);
hipError_t launch_fwd_mfma(const LayerArgs& a, hipStream_t s);
hipError_t launch_bwd_mfma(const LayerArgs& a, int G, hipStream_t s);



// ---------------------------------------------------------------------------------
// Kronecker-sparse matmul.
// ---------------------------------------------------------------------------------
struct KSArgs {
  int64_t N;
  int32_t a, b, c, d;
  int32_t dtype;       // of x and vals: KRON_F32 / KRON_BF16
  int32_t out_dtype;   // of y: KRON_F32 / KRON_BF16 (rounded to nearest even)
  const void* x;
  const void* vals;
  void* y;
};
bool ks_supported(int a, int b, int c, int d);
hipError_t launch_ks(const KSArgs& k, hipStream_t s);
// Matrix-core path for the (b, c, d) in its table (see ks_mfma.hip).
bool ks_mfma_supported(int a, int b, int c, int d);
hipError_t launch_ks_mfma(const KSArgs& k, hipStream_t s);
// Backward of the KS matmul (ks_bwd.hip): dx = dy K^T (NULL: skipped), dvals (NULL: skipped).
struct KSBwdArgs {
  int64_t N;
  int32_t a, b, c, d;
  int32_t dtype;   // of x, vals and dy
  const void* x;
  const void* vals;
  const void* dy;
  float* dx;
  float* dvals;
};
// Fused chain of KS factors (ks_chain.hip): y = x K_1 ... K_nf, rows of at most maxw values.
constexpr int kChainMaxFactors = 8;
constexpr int kChainMaxWidth = 16384;
struct ChainFactor {
  int32_t a, b, c, d;
  const void* vals;
};
struct ChainArgs {
  int64_t N;
  int32_t nf, dtype, maxw, wl;   // wl: width of the output rows
  ChainFactor f[kChainMaxFactors];
  const void* x;
  float* y;
};
int chain_rows_per_tile(int maxw);
hipError_t launch_ks_chain(const ChainArgs& a, hipStream_t s);
// Van Loan rank-r projection (vanloan.hip).
struct VanLoanArgs {
  int32_t p, q, m, n, r, s, iters;
  const float* W;       // [p*m, q*n]
  const float* omega;   // [m*n, s] starting block
  float* C;             // [r, p, q]
  float* B;             // [r, m, n]
  float* sigma;         // [r]
};
size_t van_loan_workspace_bytes(int p, int q, int m, int n, int s);
hipError_t launch_van_loan(const VanLoanArgs& a, void* workspace, hipStream_t s);
bool ks_bwd_supported(int a, int b, int c, int d);
size_t ks_bwd_workspace_bytes(int64_t N, int a, int b, int c, int d, int dtype);
hipError_t launch_ks_bwd(const KSBwdArgs& k, void* workspace, hipStream_t s);

// ---------------------------------------------------------------------------------
// Adam + l1.
// ---------------------------------------------------------------------------------
struct AdamTensor {
  float* p;
  const float* g;
  float* m;
  float* v;
  int64_t numel;
  float l1;
  float pad_;
};
constexpr int kAdamMaxPerLaunch = 64;
struct AdamBatch {
  AdamTensor t[kAdamMaxPerLaunch];
  int32_t count;
  int32_t pad_;
};
// Hyper-parameters rounded once to fp32 from host doubles.
struct AdamHyper {
  float lr, beta1, one_minus_beta1, beta2, one_minus_beta2, eps, inv_bc1, inv_bc2;
};
hipError_t launch_adam(const AdamBatch& b, int64_t max_numel, const AdamHyper& h, hipStream_t s);

// ---------------------------------------------------------------------------------
// ReLU gradient and the l1 penalty on S.
// ---------------------------------------------------------------------------------
constexpr int kL1MaxTensors = 64;
struct L1Batch {
  const float* t[kL1MaxTensors];
  int64_t numel[kL1MaxTensors];
  int32_t count;
  int32_t pad_;
};
hipError_t launch_relu_bwd(int64_t n, const float* y, const float* dy, float* out, hipStream_t s);
hipError_t launch_l1_penalty(const L1Batch& b, float lam, float* loss, bool accumulate, hipStream_t s);
hipError_t launch_l1_grad(int64_t n, const float* S, float lam, const float* g, float* dS, hipStream_t s);

// ---------------------------------------------------------------------------------
// Dense head + softmax cross-entropy.
// ---------------------------------------------------------------------------------
struct HeadArgs {
  int64_t N;
  int32_t K, C;
  uint32_t flags;
  const float* h;
  const float* W;
  const float* b;
  const int64_t* labels;
  float* loss;
  float* dh;
  float* dW;
  float* db;
  float* dz;     // workspace: N x C
  float* part;   // workspace: G partial rows of K*C + C + 1 columns (column-blocked)
};
int head_groups(int64_t N);
int head_mfma_groups(int64_t N);
bool head_mfma_ok(int K, int C);
int64_t head_rows_per_group(int64_t N);
hipError_t launch_head(const HeadArgs& a, int G, hipStream_t s);

}  // namespace kron
