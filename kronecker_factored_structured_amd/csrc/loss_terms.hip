// The training step's pieces around the layers that are not products: the gradient
// through a ReLU output, and the l1 penalty on S with its subgradient.
//
// Kronecker layer tutorial, "Setup": the MLP's hidden layers end in a ReLU and the loss
// is the cross-entropy plus the model's penalty; intro: that penalty is lam * sum|S|,
// the l1 norm that drives entries of S to zero.
//   relu_bwd:       out = dy o [y > 0]        (y = max(z, 0), so [y > 0] = [z > 0])
//   l1_penalty:     loss = (loss or 0) + lam * sum_t sum_e |T_t[e]|
//   l1_penalty_grad dS = lam * g * sign(S),   sign(0) = 0, g the upstream scalar gradient
// The sum is taken in fp64 in a fixed order (one workgroup, each thread a fixed strided
// subset, then a fixed tree), so it is bitwise reproducible.
#include "kron_internal.h"

namespace kron {
namespace {

constexpr int kThreads = 256;
typedef float f4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void relu_bwd_kernel(int64_t n, const float* __restrict__ y,
                                                            const float* dy, float* out) {
  const int64_t n4 = n >> 2;
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n4; e += (int64_t)gridDim.x * kThreads) {
    const f4 yv = reinterpret_cast<const f4*>(y)[e];
    f4 g = reinterpret_cast<const f4*>(dy)[e];
#pragma unroll
    for (int v = 0; v < 4; ++v) g[v] = yv[v] > 0.f ? g[v] : 0.f;
    reinterpret_cast<f4*>(out)[e] = g;
  }
  // the last n % 4 elements
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t e = 4 * n4 + threadIdx.x;
    out[e] = y[e] > 0.f ? dy[e] : 0.f;
  }
}

__global__ __launch_bounds__(kThreads) void l1_penalty_kernel(L1Batch b, float lam, float* loss, int accumulate) {
  __shared__ double red[kThreads];
  double s = 0.0;
  for (int t = 0; t < b.count; ++t) {
    const float* p = b.t[t];
    const int64_t n = b.numel[t];
    double st = 0.0;
    for (int64_t e = threadIdx.x; e < n; e += kThreads) st += fabs((double)p[e]);
    s += st;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double base = accumulate ? (double)loss[0] : 0.0;
    loss[0] = (float)(base + (double)lam * red[0]);
  }
}

__global__ __launch_bounds__(kThreads) void l1_grad_kernel(int64_t n, const float* __restrict__ S, float lam,
                                                           const float* __restrict__ g, float* __restrict__ dS) {
  const float k = lam * g[0];
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n; e += (int64_t)gridDim.x * kThreads) {
    const float s = S[e];
    dS[e] = s > 0.f ? k : (s < 0.f ? -k : 0.f);
  }
}

int64_t grid_for(int64_t work) {
  int64_t g = (work + kThreads - 1) / kThreads;
  if (g > 2048) g = 2048;
  return g < 1 ? 1 : g;
}

}  // namespace

hipError_t launch_relu_bwd(int64_t n, const float* y, const float* dy, float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(relu_bwd_kernel, dim3((unsigned)grid_for(n >> 2)), dim3(kThreads), 0, s, n, y, dy, out);
  return hipGetLastError();
}

hipError_t launch_l1_penalty(const L1Batch& b, float lam, float* loss, bool accumulate, hipStream_t s) {
  hipLaunchKernelGGL(l1_penalty_kernel, dim3(1), dim3(kThreads), 0, s, b, lam, loss, accumulate ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_l1_grad(int64_t n, const float* S, float lam, const float* g, float* dS, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(l1_grad_kernel, dim3((unsigned)grid_for(n)), dim3(kThreads), 0, s, n, S, lam, g, dS);
  return hipGetLastError();
}

}  // namespace kron
