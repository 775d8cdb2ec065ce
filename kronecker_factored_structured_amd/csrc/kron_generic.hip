// Generic (any-shape) kernels of the Kronecker-factored layer and the fixed-order
// column reduction shared by every backward.
//
// Math (Kronecker layer tutorial, "The vec trick" and "The vec trick without the
// loop"): with X_n the p x m row-major view of row x_n and C_i = S o A_i,
//   Z_{n,i} = X_n B_i               (p x n, kept in LDS, never written to HBM)
//   Y_n     = sum_i C_i^T Z_{n,i}   (q x n), y_n = vec_row(Y_n) + bias
// Backward, from the calculus of the same expression:
//   G_{n,i} = C_i dY_n,  dX_n = sum_i G_{n,i} B_i^T,
//   dB_i = sum_n X_n^T G_{n,i},  dC_i = sum_n Z_{n,i} dY_n^T,  dbias = sum_n dy_n.
// Terms with S[j,k] == 0 are skipped (zero blocks of W).
//
// These kernels are LDS-tiled VALU code: one workgroup owns T rows at a time and
// loops over the rank.  They cover every valid shape; the MFMA kernels cover the
// shapes whose tiles map onto matrix-core instructions.
#include "kron_internal.h"

namespace kron {
namespace {

constexpr int kThreads = 256;
constexpr size_t kGenericLds = 160 * 1024;   // bytes of LDS the generic kernels may use (a CU's LDS)
constexpr int kMaxTileRows = 32;

__global__ __launch_bounds__(kThreads) void fwd_generic_kernel(
    int64_t N, int p, int q, int m, int n, int r, int T, uint32_t flags,
    const float* __restrict__ x, const float* __restrict__ S, const float* __restrict__ A,
    const float* __restrict__ B, const float* __restrict__ bias, float* __restrict__ y) {
  extern __shared__ float lds[];
  const int in = p * m, out = q * n, pn = p * n, pq = p * q, mn = m * n;
  float* Xs = lds;            // T x in
  float* Zs = Xs + T * in;    // T x p x n
  float* Ys = Zs + T * pn;    // T x out
  float* Bs = Ys + T * out;   // m x n
  float* Cs = Bs + mn;        // p x q
  float* Ss = Cs + pq;        // p x q
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.x * T;
  const int rows = (int)((N - row0) < T ? (N - row0) : T);

  const float* xt = x + row0 * in;
  for (int e = tid; e < rows * in; e += kThreads) Xs[e] = xt[e];
  for (int e = tid; e < rows * out; e += kThreads) Ys[e] = 0.f;
  if (S)
    for (int e = tid; e < pq; e += kThreads) Ss[e] = S[e];

  for (int i = 0; i < r; ++i) {
    __syncthreads();
    for (int e = tid; e < mn; e += kThreads) Bs[e] = B[(int64_t)i * mn + e];
    for (int e = tid; e < pq; e += kThreads) {
      const float a = A[(int64_t)i * pq + e];
      Cs[e] = S ? S[e] * a : a;
    }
    __syncthreads();
    // Z = X B_i
    for (int e = tid; e < rows * pn; e += kThreads) {
      const int t = e / pn, rem = e - t * pn, j = rem / n, b = rem - j * n;
      const float* xr = Xs + t * in + j * m;
      float acc = 0.f;
      for (int a = 0; a < m; ++a) acc = fmaf(xr[a], Bs[a * n + b], acc);
      Zs[e] = acc;
    }
    __syncthreads();
    // Y += C_i^T Z
    for (int e = tid; e < rows * out; e += kThreads) {
      const int t = e / out, rem = e - t * out, k = rem / n, b = rem - k * n;
      const float* zr = Zs + t * pn + b;
      float acc = 0.f;
      for (int j = 0; j < p; ++j) {
        if (S && Ss[j * q + k] == 0.f) continue;
        acc = fmaf(Cs[j * q + k], zr[j * n], acc);
      }
      Ys[e] += acc;
    }
  }
  float* yt = y + row0 * out;
  for (int e = tid; e < rows * out; e += kThreads) {
    float v = Ys[e];
    if (bias) v += bias[e % out];
    if (flags & KRON_RELU_OUT) v = v > 0.f ? v : 0.f;
    yt[e] = v;
  }
}

__global__ __launch_bounds__(kThreads) void bwd_generic_kernel(
    int64_t N, int p, int q, int m, int n, int r, int T, uint32_t flags,
    const float* __restrict__ x, const float* __restrict__ S, const float* __restrict__ A,
    const float* __restrict__ B, const float* __restrict__ dy, float* __restrict__ dx,
    float* __restrict__ part) {
  extern __shared__ float lds[];
  const int in = p * m, out = q * n, pn = p * n, pq = p * q, mn = m * n;
  const bool want_dx = dx != nullptr;
  float* Xs = lds;               // T x in
  float* dYs = Xs + T * in;      // T x out
  float* Zs = dYs + T * out;     // T x p x n
  float* Gs = Zs + T * pn;       // T x p x n
  float* Bs = Gs + T * pn;       // m x n
  float* Cs = Bs + mn;           // p x q
  float* Ss = Cs + pq;           // p x q
  float* dXs = Ss + pq;          // T x in (only with dx)
  const int tid = threadIdx.x;
  const int PW = (int)partial_width(p, q, m, n, r);
  const PartRow pdB{part, (int64_t)gridDim.x, (int64_t)blockIdx.x, 0};
  const PartRow pdC = pdB + r * mn;   // dC_i during the loop, dA_i at the end
  const PartRow pdS = pdC + r * pq;
  const PartRow pdb = pdS + pq;
  for (int e = tid; e < PW; e += kThreads) pdB[e] = 0.f;
  if (S)
    for (int e = tid; e < pq; e += kThreads) Ss[e] = S[e];

  const int64_t ntiles = (N + T - 1) / T;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t row0 = tile * T;
    const int rows = (int)((N - row0) < T ? (N - row0) : T);
    __syncthreads();
    const float* xt = x + row0 * in;
    const float* dyt = dy + row0 * out;
    for (int e = tid; e < rows * in; e += kThreads) Xs[e] = xt[e];
    for (int e = tid; e < rows * out; e += kThreads) dYs[e] = dyt[e];
    if (want_dx)
      for (int e = tid; e < rows * in; e += kThreads) dXs[e] = 0.f;
    __syncthreads();
    for (int e = tid; e < out; e += kThreads) {
      float s = 0.f;
      for (int t = 0; t < rows; ++t) s += dYs[t * out + e];
      pdb[e] += s;
    }
    for (int i = 0; i < r; ++i) {
      __syncthreads();
      for (int e = tid; e < mn; e += kThreads) Bs[e] = B[(int64_t)i * mn + e];
      for (int e = tid; e < pq; e += kThreads) {
        const float a = A[(int64_t)i * pq + e];
        Cs[e] = S ? S[e] * a : a;
      }
      __syncthreads();
      for (int e = tid; e < rows * pn; e += kThreads) {
        const int t = e / pn, rem = e - t * pn, j = rem / n, b = rem - j * n;
        const float* xr = Xs + t * in + j * m;
        float z = 0.f;
        for (int a = 0; a < m; ++a) z = fmaf(xr[a], Bs[a * n + b], z);
        Zs[e] = z;
        const float* dyr = dYs + t * out + b;
        float g = 0.f;
        for (int k = 0; k < q; ++k) {
          if (S && Ss[j * q + k] == 0.f) continue;
          g = fmaf(Cs[j * q + k], dyr[k * n], g);
        }
        Gs[e] = g;
      }
      __syncthreads();
      if (want_dx) {
        for (int e = tid; e < rows * in; e += kThreads) {
          const int t = e / in, rem = e - t * in, j = rem / m, a = rem - j * m;
          const float* gr = Gs + t * pn + j * n;
          const float* br = Bs + a * n;
          float acc = 0.f;
          for (int b = 0; b < n; ++b) acc = fmaf(gr[b], br[b], acc);
          dXs[e] += acc;
        }
      }
      for (int e = tid; e < mn; e += kThreads) {
        const int a = e / n, b = e - a * n;
        float acc = 0.f;
        for (int t = 0; t < rows; ++t)
          for (int j = 0; j < p; ++j) acc = fmaf(Xs[t * in + j * m + a], Gs[t * pn + j * n + b], acc);
        pdB[i * mn + e] += acc;
      }
      for (int e = tid; e < pq; e += kThreads) {
        const int j = e / q, k = e - j * q;
        float acc = 0.f;
        for (int t = 0; t < rows; ++t)
          for (int b = 0; b < n; ++b) acc = fmaf(Zs[t * pn + j * n + b], dYs[t * out + k * n + b], acc);
        pdC[i * pq + e] += acc;
      }
    }
    if (want_dx) {
      float* dxt = dx + row0 * in;
      for (int e = tid; e < rows * in; e += kThreads) {
        float v = dXs[e];
        if ((flags & KRON_DX_RELU_MASK) && !(Xs[e] > 0.f)) v = 0.f;
        dxt[e] = v;
      }
    }
  }
  // this workgroup's dC_i -> its shares of dA_i = S o dC_i and dS = sum_i A_i o dC_i
  __syncthreads();
  for (int e = tid; e < pq; e += kThreads) {
    const float sv = S ? S[e] : 1.f;
    float ds = 0.f;
    for (int i = 0; i < r; ++i) {
      const float dc = pdC[i * pq + e];
      ds = fmaf(A[(int64_t)i * pq + e], dc, ds);
      pdC[i * pq + e] = sv * dc;
    }
    pdS[e] = S ? ds : 0.f;
  }
}

// A workgroup of CX * RY threads reduces one block of CX * VEC = kRedCols columns: thread
// (tx, ty) reads VEC columns as one vector from partial rows g = ty (mod RY), U loads in
// flight at a time (all of them at once for G <= U * RY), and sums them in fp64 in row
// order; the RY per-thread sums are then combined in a fixed tree, so the result does not
// depend on timing.
template <int VEC, int CX, int RY, int U>
__global__ __launch_bounds__(CX * RY) void column_reduce_kernel(const float* __restrict__ part, int G, int PW,
                                                                RedPlan plan) {
  static_assert(CX * VEC == kRedCols, "one workgroup per column block");
  typedef float fv __attribute__((ext_vector_type(VEC)));
  __shared__ double red[RY][CX * VEC];
  const int tx = threadIdx.x % CX, ty = threadIdx.x / CX;
  const int col0 = blockIdx.x * kRedCols + tx * VEC;
  double s[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) s[v] = 0.0;
  {
    const float* p = part + (int64_t)blockIdx.x * G * kRedCols + tx * VEC;
    for (int g0 = ty; g0 < G; g0 += U * RY) {
      fv a[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int g = g0 + u * RY;
        if (g < G) {
          a[u] = *reinterpret_cast<const fv*>(p + (int64_t)g * kRedCols);
        } else {
#pragma unroll
          for (int v = 0; v < VEC; ++v) a[u][v] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int v = 0; v < VEC; ++v) s[v] += (double)a[u][v];
    }
  }
#pragma unroll
  for (int v = 0; v < VEC; ++v) red[ty][tx * VEC + v] = s[v];
  __syncthreads();
#pragma unroll
  for (int h = RY / 2; h >= 1; h /= 2) {
    if (ty < h)
#pragma unroll
      for (int v = 0; v < VEC; ++v) red[ty][tx * VEC + v] += red[ty + h][tx * VEC + v];
    __syncthreads();
  }
  if (ty == 0) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      int c = col0 + v;
      if (c >= PW) break;
      const double tot = red[0][tx * VEC + v];
      for (int k = 0; k < plan.nseg; ++k) {
        if (c < plan.seg[k].count) {
          if (plan.seg[k].dst) {
            double v = tot * (double)plan.seg[k].scale;
            if (plan.seg[k].accumulate) v += (double)plan.seg[k].dst[c];
            plan.seg[k].dst[c] = (float)v;
          }
          break;
        }
        c -= plan.seg[k].count;
      }
    }
  }
}

size_t fwd_lds_floats(int T, int p, int q, int m, int n) {
  return (size_t)T * ((size_t)p * m + (size_t)p * n + (size_t)q * n) + (size_t)m * n + 2 * (size_t)p * q;
}
size_t bwd_lds_floats(int T, int p, int q, int m, int n, bool want_dx) {
  return (size_t)T * ((size_t)p * m + (size_t)q * n + 2 * (size_t)p * n + (want_dx ? (size_t)p * m : 0)) +
         (size_t)m * n + 2 * (size_t)p * q;
}

}  // namespace

int generic_fwd_rows_per_tile(int p, int q, int m, int n) {
  for (int T = kMaxTileRows; T >= 1; T /= 2)
    if (fwd_lds_floats(T, p, q, m, n) * sizeof(float) <= kGenericLds) return T;
  return 0;
}

int generic_bwd_rows_per_tile(int p, int q, int m, int n, bool want_dx) {
  for (int T = kMaxTileRows; T >= 1; T /= 2)
    if (bwd_lds_floats(T, p, q, m, n, want_dx) * sizeof(float) <= kGenericLds) return T;
  return 0;
}

int generic_bwd_groups(int64_t N, int T) {
  const int64_t ntiles = (N + T - 1) / T;
  return (int)(ntiles < 1024 ? ntiles : 1024);
}

hipError_t launch_fwd_generic(const LayerArgs& a, hipStream_t s) {
  const int T = generic_fwd_rows_per_tile(a.p, a.q, a.m, a.n);
  if (T == 0) return hipErrorInvalidValue;
  const int64_t grid = (a.N + T - 1) / T;
  if (grid == 0) return hipSuccess;
  const size_t lds = fwd_lds_floats(T, a.p, a.q, a.m, a.n) * sizeof(float);
  static const bool attr =
      hipFuncSetAttribute((const void*)fwd_generic_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)kGenericLds) == hipSuccess;
  (void)attr;
  hipLaunchKernelGGL(fwd_generic_kernel, dim3((unsigned)grid), dim3(kThreads), lds, s, a.N, a.p, a.q,
                     a.m, a.n, a.r, T, a.flags, a.x, a.S, a.A, a.B, a.bias, a.y);
  return hipGetLastError();
}

hipError_t launch_bwd_generic(const LayerArgs& a, int G, hipStream_t s) {
  const bool want_dx = a.dx != nullptr;
  const int T = generic_bwd_rows_per_tile(a.p, a.q, a.m, a.n, want_dx);
  if (T == 0) return hipErrorInvalidValue;
  if (G == 0) return hipSuccess;
  const size_t lds = bwd_lds_floats(T, a.p, a.q, a.m, a.n, want_dx) * sizeof(float);
  static const bool attr =
      hipFuncSetAttribute((const void*)bwd_generic_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)kGenericLds) == hipSuccess;
  (void)attr;
  hipLaunchKernelGGL(bwd_generic_kernel, dim3(G), dim3(kThreads), lds, s, a.N, a.p, a.q, a.m, a.n,
                     a.r, T, a.flags, a.x, a.S, a.A, a.B, a.dy, a.dx, a.part);
  return hipGetLastError();
}

hipError_t launch_column_reduce(const float* part, int32_t G, int32_t PW, const RedPlan& plan,
                                hipStream_t stream) {
  if (PW == 0) return hipSuccess;
  // 16-byte vector loads need the partial sums 16-byte aligned (workspaces are 256-byte aligned)
  const unsigned blocks = (unsigned)((PW + kRedCols - 1) / kRedCols);
  if (((uintptr_t)part & 15) == 0)
    hipLaunchKernelGGL((column_reduce_kernel<4, 8, 32, 8>), dim3(blocks), dim3(256), 0, stream, part, G, PW, plan);
  else
    hipLaunchKernelGGL((column_reduce_kernel<1, 32, 8, 16>), dim3(blocks), dim3(256), 0, stream, part, G, PW, plan);
  return hipGetLastError();
}

}  // namespace kron
