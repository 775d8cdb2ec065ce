// Dense classification head with mean softmax cross-entropy, forward and backward
// (Kronecker layer tutorial, "Setup": the 10-class output layer stays dense; the step's
// loss is the cross-entropy).
//   z = h W + b;  loss = mean_n (logsumexp(z_n) - z_n[label_n])
//   dz = (softmax(z) - onehot) / N;  dh = dz W^T (o [h > 0]);  dW = h^T dz;  db = sum dz
// Pass 1: one wavefront per row computes z with a butterfly all-reduce across the
// 64 lanes, the softmax, dz, the row's loss and dh.  Pass 2: each thread owns one row
// k of dW (all C classes in registers) over a chunk of rows; the chunks' partial sums
// go through the shared fixed-order column reduction.
#include "kron_internal.h"

namespace kron {
namespace {

constexpr int kThreads = 256;
constexpr int kWave = 64;
constexpr int kPass1Blocks = 512;

template <int CMAX>
__global__ __launch_bounds__(kThreads) void head_rows_kernel(
    int64_t N, int K, int C, uint32_t flags, const float* __restrict__ h, const float* __restrict__ W,
    const float* __restrict__ b, const int64_t* __restrict__ labels, float* __restrict__ dh,
    float* __restrict__ dz, float* __restrict__ lossrow) {
  extern __shared__ float Wt[];   // C x K (transposed head weight)
  for (int e = threadIdx.x; e < K * C; e += kThreads) {
    const int k = e / C, c = e - k * C;
    Wt[c * K + k] = W[e];
  }
  __syncthreads();
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / kWave);
  const float invN = 1.f / (float)N;
  for (int64_t row = (int64_t)blockIdx.x * (kThreads / kWave) + wave; row < N; row += nwaves) {
    const float* hr = h + row * K;
    float z[CMAX];
#pragma unroll
    for (int c = 0; c < CMAX; ++c) z[c] = 0.f;
    for (int k = lane; k < K; k += kWave) {
      const float hk = hr[k];
#pragma unroll
      for (int c = 0; c < CMAX; ++c)
        if (c < C) z[c] = fmaf(hk, Wt[c * K + k], z[c]);
    }
#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
      if (c < C) {
        float v = z[c];
#pragma unroll
        for (int off = kWave / 2; off >= 1; off /= 2) v += __shfl_xor(v, off, kWave);
        z[c] = v + b[c];
      }
    }
    float zmax = -INFINITY;
#pragma unroll
    for (int c = 0; c < CMAX; ++c)
      if (c < C) zmax = fmaxf(zmax, z[c]);
    const int64_t lab = labels[row];
    const bool ok = lab >= 0 && lab < C;
    float zlm = 0.f;   // z[label] - max
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CMAX; ++c)
      if (c < C) {
        const float d = z[c] - zmax;
        if (ok && c == lab) zlm = d;
        z[c] = expf(d);   // z now holds exp(z - max)
        s += z[c];
      }
    const float inv_s = 1.f / s;
    float mydz = 0.f;
#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
      if (c < C) {
        const float pc = z[c] * inv_s;
        const float d = (pc - ((ok && c == lab) ? 1.f : 0.f)) * invN;
        z[c] = d;                  // z now holds dz
        if (lane == c) mydz = d;
      }
    }
    if (lane < C) dz[row * C + lane] = mydz;
    if (lane == 0) lossrow[row] = ok ? (logf(s) - zlm) : __builtin_nanf("");
    float* dhr = dh ? dh + row * K : nullptr;
    if (dhr) {
      for (int k = lane; k < K; k += kWave) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CMAX; ++c)
          if (c < C) acc = fmaf(z[c], Wt[c * K + k], acc);
        if ((flags & KRON_DX_RELU_MASK) && !(hr[k] > 0.f)) acc = 0.f;
        dhr[k] = acc;
      }
    }
  }
}

// grid (ceil((K+1)/256), G): thread k < K owns dW[k][:] over rows [g*R, (g+1)*R);
// thread k == K owns db[:] and the loss sum of the same rows.
template <int CMAX>
__global__ __launch_bounds__(kThreads) void head_dw_kernel(int64_t N, int K, int C, int64_t R,
                                                           const float* __restrict__ h,
                                                           const float* __restrict__ dz,
                                                           const float* __restrict__ lossrow,
                                                           float* __restrict__ part) {
  const int k = blockIdx.x * kThreads + threadIdx.x;
  if (k > K) return;
  const int64_t r0 = (int64_t)blockIdx.y * R;
  const int64_t r1 = (r0 + R) < N ? (r0 + R) : N;
  const int64_t PW = (int64_t)K * C + C + 1;
  const PartRow out{part, (int64_t)gridDim.y, (int64_t)blockIdx.y, 0};
  (void)PW;
  float acc[CMAX];
#pragma unroll
  for (int c = 0; c < CMAX; ++c) acc[c] = 0.f;
  if (k < K) {
    for (int64_t n = r0; n < r1; ++n) {
      const float hv = h[n * K + k];
#pragma unroll
      for (int c = 0; c < CMAX; ++c)
        if (c < C) acc[c] = fmaf(hv, dz[n * C + c], acc[c]);
    }
#pragma unroll
    for (int c = 0; c < CMAX; ++c)
      if (c < C) out[(int64_t)k * C + c] = acc[c];
  } else {
    float ls = 0.f;
    for (int64_t n = r0; n < r1; ++n) {
#pragma unroll
      for (int c = 0; c < CMAX; ++c)
        if (c < C) acc[c] += dz[n * C + c];
      ls += lossrow[n];
    }
#pragma unroll
    for (int c = 0; c < CMAX; ++c)
      if (c < C) out[(int64_t)K * C + c] = acc[c];
    out[(int64_t)K * C + C] = ls;
  }
}

}  // namespace

int head_groups(int64_t N) {
  const int64_t g = (N + 127) / 128;
  return (int)(g < 256 ? g : 256);
}

int64_t head_rows_per_group(int64_t N) {
  const int G = head_groups(N);
  return G == 0 ? 0 : (N + G - 1) / G;
}

hipError_t launch_head(const HeadArgs& a, int G, hipStream_t s) {
  float* lossrow = a.dz + a.N * a.C;
  if (a.N > 0) {
    int64_t blocks = (a.N + 3) / 4;
    if (blocks > kPass1Blocks) blocks = kPass1Blocks;
    const size_t lds = (size_t)a.K * a.C * sizeof(float);
    if (a.C <= 16)
      hipLaunchKernelGGL(head_rows_kernel<16>, dim3((unsigned)blocks), dim3(kThreads), lds, s, a.N, a.K,
                         a.C, a.flags, a.h, a.W, a.b, a.labels, a.dh, a.dz, lossrow);
    else
      hipLaunchKernelGGL(head_rows_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), lds, s, a.N, a.K,
                         a.C, a.flags, a.h, a.W, a.b, a.labels, a.dh, a.dz, lossrow);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t R = head_rows_per_group(a.N);
    dim3 grid((unsigned)((a.K + 1 + kThreads - 1) / kThreads), (unsigned)G);
    if (a.C <= 16)
      hipLaunchKernelGGL(head_dw_kernel<16>, grid, dim3(kThreads), 0, s, a.N, a.K, a.C, R, a.h, a.dz,
                         lossrow, a.part);
    else
      hipLaunchKernelGGL(head_dw_kernel<64>, grid, dim3(kThreads), 0, s, a.N, a.K, a.C, R, a.h, a.dz,
                         lossrow, a.part);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  RedPlan plan{};
  plan.nseg = 3;
  plan.seg[0] = RedSeg{a.dW, a.K * a.C, 1.f, 0};
  plan.seg[1] = RedSeg{a.db, a.C, 1.f, 0};
  plan.seg[2] = RedSeg{a.loss, 1, a.N > 0 ? (float)(1.0 / (double)a.N) : 0.f, 0};
  return launch_column_reduce(a.part, G, a.K * a.C + a.C + 1, plan, s);
}

}  // namespace kron
