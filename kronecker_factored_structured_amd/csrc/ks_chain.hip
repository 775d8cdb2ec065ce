// Fused chain of Kronecker-sparse factors: Y = X K_1 K_2 ... K_F, each K_f with support
// I_a (x) 1_{b x c} (x) I_d ("Fast Inference with Kronecker-Sparse Matrices", abstract: KS
// matrices and products of them, such as butterfly and Monarch factors; the triple
// Kronecker product A (x) B (x) C is the three-factor case by the mixed-product rule).
// A workgroup takes a tile of rows, holds them in LDS in fp32 through every factor
// (two row buffers, alternating), and writes only the last factor's output to HBM.
#include "kron_internal.h"

namespace kron {
namespace {

constexpr int kChainThreads = 1024;
constexpr int kChainMaxRows = 16;
constexpr size_t kChainLds = 160 * 1024;

__device__ __forceinline__ float load_in(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_in(const uint16_t* p, int64_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}

template <typename TIn>
__global__ __launch_bounds__(kChainThreads) void ks_chain_kernel(ChainArgs A, int T) {
  extern __shared__ float s[];
  float* in = s;
  float* out = s + (size_t)T * A.maxw;
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.x * T;
  const int rows = (int)(A.N - row0 < T ? A.N - row0 : T);
  const int w0 = A.f[0].a * A.f[0].b * A.f[0].d;
  const TIn* x = static_cast<const TIn*>(A.x);
  for (int i = tid; i < rows * w0; i += kChainThreads) {
    const int t = i / w0, col = i - t * w0;
    in[t * A.maxw + col] = load_in(x, (row0 + t) * w0 + col);
  }
  __syncthreads();
  for (int fi = 0; fi < A.nf; ++fi) {
    const int a = A.f[fi].a, b = A.f[fi].b, c = A.f[fi].c, d = A.f[fi].d;
    const int wout = a * c * d;
    const TIn* V = static_cast<const TIn*>(A.f[fi].vals);
    const bool last = fi == A.nf - 1;
    // a thread owns output columns; each value is loaded once per tile and applied to
    // every row of the tile from LDS
    for (int col = tid; col < wout; col += kChainThreads) {
      const int de = col % d, rest = col / d, ga = rest % c, al = rest / c;
      const float* ir = in + (al * b) * d + de;
      const TIn* v = V + ((int64_t)(al * d + de) * b) * c + ga;
      float acc[kChainMaxRows];
#pragma unroll
      for (int t = 0; t < kChainMaxRows; ++t) acc[t] = 0.f;
#pragma unroll 8
      for (int be = 0; be < b; ++be) {
        const float vv = load_in(v, (int64_t)be * c);
        const float* ib = ir + be * d;
#pragma unroll
        for (int t = 0; t < kChainMaxRows; ++t)
          if (t < rows) acc[t] = fmaf(ib[t * A.maxw], vv, acc[t]);
      }
#pragma unroll
      for (int t = 0; t < kChainMaxRows; ++t) {
        if (t < rows) {
          if (last)
            A.y[(row0 + t) * wout + col] = acc[t];
          else
            out[t * A.maxw + col] = acc[t];
        }
      }
    }
    __syncthreads();
    float* tmp = in;
    in = out;
    out = tmp;
  }
}

}  // namespace

int chain_rows_per_tile(int maxw) {
  int64_t T = (int64_t)(kChainLds / (2 * (size_t)maxw * sizeof(float)));
  if (T > kChainMaxRows) T = kChainMaxRows;
  return (int)T;
}

hipError_t launch_ks_chain(const ChainArgs& A, hipStream_t s) {
  const int T = chain_rows_per_tile(A.maxw);
  if (T < 1) return hipErrorInvalidValue;
  const int64_t grid = (A.N + T - 1) / T;
  if (grid == 0) return hipSuccess;
  const size_t lds = 2 * (size_t)T * A.maxw * sizeof(float);
  static const bool attr = [] {
    const bool a1 = hipFuncSetAttribute((const void*)ks_chain_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                        (int)kChainLds) == hipSuccess;
    const bool a2 = hipFuncSetAttribute((const void*)ks_chain_kernel<uint16_t>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kChainLds) == hipSuccess;
    return a1 && a2;
  }();
  (void)attr;
  if (A.dtype == KRON_F32)
    hipLaunchKernelGGL(ks_chain_kernel<float>, dim3((unsigned)grid), dim3(kChainThreads), lds, s, A, T);
  else
    hipLaunchKernelGGL(ks_chain_kernel<uint16_t>, dim3((unsigned)grid), dim3(kChainThreads), lds, s, A, T);
  return hipGetLastError();
}

}  // namespace kron
