// Fused multi-tensor Adam with an l1 penalty: one launch updates every parameter
// tensor of the training step (Kronecker layer tutorial, "Setup": an Adam update per
// step; intro: an l1 penalty on S).  Per element, in fp32:
//   g = grad + l1*sign(theta);  m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*g*g
//   theta -= lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
// 1 - beta and the bias-correction reciprocals are formed on the host in double.
#include "kron_internal.h"

namespace kron {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void adam_l1_kernel(AdamBatch batch, AdamHyper h) {
  const AdamTensor T = batch.t[blockIdx.y];
  for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < T.numel;
       e += (int64_t)gridDim.x * kThreads) {
    const float th = T.p[e];
    float g = T.g[e];
    if (T.l1 != 0.f) g = fmaf(T.l1, (th > 0.f) ? 1.f : ((th < 0.f) ? -1.f : 0.f), g);
    const float m = fmaf(h.beta1, T.m[e], h.one_minus_beta1 * g);
    const float v = fmaf(h.beta2, T.v[e], h.one_minus_beta2 * g * g);
    T.m[e] = m;
    T.v[e] = v;
    T.p[e] = th - h.lr * (m * h.inv_bc1) / (sqrtf(v * h.inv_bc2) + h.eps);
  }
}

}  // namespace

hipError_t launch_adam(const AdamBatch& b, int64_t max_numel, const AdamHyper& h, hipStream_t s) {
  if (b.count == 0 || max_numel == 0) return hipSuccess;
  int64_t gx = (max_numel + kThreads * 4 - 1) / (kThreads * 4);
  if (gx > 1024) gx = 1024;
  hipLaunchKernelGGL(adam_l1_kernel, dim3((unsigned)gx, (unsigned)b.count), dim3(kThreads), 0, s, b, h);
  return hipGetLastError();
}

}  // namespace kron
