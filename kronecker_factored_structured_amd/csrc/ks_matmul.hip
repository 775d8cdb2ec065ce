// Kronecker-sparse matmul Y = X K, K with support I_a (x) 1_{b x c} (x) I_d
// ("Fast Inference with Kronecker-Sparse Matrices", abstract: supports that are
// Kronecker products of identity and all-ones blocks).
//
// Index map (row-major Kronecker indices): input column (al*b + be)*d + de, output
// column (al*c + ga)*d + de, value vals[al][de][be][ga].  For a fixed alpha the input
// columns form one contiguous slab of b*d floats per row and the output columns one
// contiguous slab of c*d floats, so the kernel is output-stationary without any
// permutation pass: a workgroup stages T rows of one alpha-slab in LDS, de-interleaves
// delta on chip by indexing, and writes its c*d outputs per row straight to y.
#include "kron_internal.h"

namespace kron {
namespace {

constexpr int kThreads = 256;
constexpr size_t kKsLds = 160 * 1024;   // a CU's LDS

__device__ __forceinline__ float load_in(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_in(const uint16_t* p, int64_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}
__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t* p, float v) { *p = __builtin_bit_cast(uint16_t, (__bf16)v); }

template <typename TIn, typename TOut>
__global__ __launch_bounds__(kThreads) void ks_generic_kernel(int64_t N, int a, int b, int c, int d,
                                                              int T, const TIn* __restrict__ x,
                                                              const TIn* __restrict__ vals,
                                                              TOut* __restrict__ y) {
  extern __shared__ float Xs[];   // T x (b*d)
  const int al = blockIdx.y;
  const int bd = b * d, cd = c * d;
  const int64_t in = (int64_t)a * bd, outw = (int64_t)a * cd;
  const int64_t row0 = (int64_t)blockIdx.x * T;
  const int rows = (int)((N - row0) < T ? (N - row0) : T);
  for (int e = threadIdx.x; e < rows * bd; e += kThreads) {
    const int t = e / bd, k = e - t * bd;
    Xs[e] = load_in(x, (row0 + t) * in + (int64_t)al * bd + k);
  }
  __syncthreads();
  const TIn* V = vals + (int64_t)al * d * b * c;
  for (int o = threadIdx.x; o < rows * cd; o += kThreads) {
    const int t = o / cd, rem = o - t * cd, ga = rem / d, de = rem - ga * d;
    const TIn* v = V + (int64_t)de * b * c + ga;
    const float* xr = Xs + t * bd + de;
    float acc = 0.f;
    for (int be = 0; be < b; ++be) acc = fmaf(xr[be * d], load_in(v, (int64_t)be * c), acc);
    store_out(y + (row0 + t) * outw + (int64_t)al * cd + rem, acc);
  }
}

int ks_rows_per_tile(int b, int d) {
  const int64_t bd = (int64_t)b * d;
  for (int T = 64; T >= 1; T /= 2)
    if ((int64_t)T * bd * (int64_t)sizeof(float) <= (int64_t)kKsLds) return T;
  return 0;
}

}  // namespace

bool ks_supported(int a, int b, int c, int d) {
  (void)a;
  (void)c;
  return ks_rows_per_tile(b, d) > 0;
}

hipError_t launch_ks(const KSArgs& k, hipStream_t s) {
  if (ks_mfma_supported(k.a, k.b, k.c, k.d)) return launch_ks_mfma(k, s);
  const int T = ks_rows_per_tile(k.b, k.d);
  if (T == 0) return hipErrorInvalidValue;
  const int64_t gx = (k.N + T - 1) / T;
  if (gx == 0) return hipSuccess;
  const size_t lds = (size_t)T * k.b * k.d * sizeof(float);
  dim3 grid((unsigned)gx, (unsigned)k.a);
  static const bool attr = [] {
    const void* fns[4] = {(const void*)ks_generic_kernel<float, float>, (const void*)ks_generic_kernel<float, uint16_t>,
                          (const void*)ks_generic_kernel<uint16_t, float>,
                          (const void*)ks_generic_kernel<uint16_t, uint16_t>};
    bool ok = true;
    for (const void* f : fns)
      ok = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kKsLds) == hipSuccess && ok;
    return ok;
  }();
  (void)attr;
  const bool fin = k.dtype == KRON_F32, fout = k.out_dtype == KRON_F32;
  if (fin && fout)
    hipLaunchKernelGGL((ks_generic_kernel<float, float>), grid, dim3(kThreads), lds, s, k.N, k.a, k.b, k.c, k.d, T,
                       (const float*)k.x, (const float*)k.vals, (float*)k.y);
  else if (fin)
    hipLaunchKernelGGL((ks_generic_kernel<float, uint16_t>), grid, dim3(kThreads), lds, s, k.N, k.a, k.b, k.c, k.d,
                       T, (const float*)k.x, (const float*)k.vals, (uint16_t*)k.y);
  else if (fout)
    hipLaunchKernelGGL((ks_generic_kernel<uint16_t, float>), grid, dim3(kThreads), lds, s, k.N, k.a, k.b, k.c, k.d,
                       T, (const uint16_t*)k.x, (const uint16_t*)k.vals, (float*)k.y);
  else
    hipLaunchKernelGGL((ks_generic_kernel<uint16_t, uint16_t>), grid, dim3(kThreads), lds, s, k.N, k.a, k.b, k.c,
                       k.d, T, (const uint16_t*)k.x, (const uint16_t*)k.vals, (uint16_t*)k.y);
  return hipGetLastError();
}

}  // namespace kron
