// Van Loan rank-r Kronecker projection of a dense W ("Replicating & Extending Krony-PT on
// GPT-2 Small", section "Core Algorithm - Van Loan Kronecker Decomposition"): rearrange W
// into R with R[(j*q + k), (a*n + b)] = W[j*m + a, k*n + b] (W is in x out, in = p*m,
// out = q*n), take the leading r singular triplets of R, and return C_i = sqrt(sigma_i) *
// reshape(u_i, p x q), B_i = sqrt(sigma_i) * reshape(v_i, m x n), so that
// sum_i kron(C_i, B_i) is the best rank-r sum of Kronecker products to W.
//
// The singular triplets come from block subspace iteration (the standard randomized
// range finder with power iterations) started from a caller-supplied random K x s block:
//   Q <- orth(Omega); repeat iters times: Z <- orth(R Q), Q <- orth(R^T Z);
//   Z <- orth(R Q); Bt <- R^T Z (= (Z^T R)^T); G = Bt^T Bt = E diag(lambda) E^T (Jacobi);
//   u_i = Z E e_i, sigma_i = sqrt(lambda_i), v_i = Bt E e_i / sigma_i.
// R is never materialised: the products read W through the index map above.  All sums
// run in a fixed order (bitwise repeatable).  Sign of each pair: the entry of u_i largest
// in magnitude (the first such) is made positive; C_i (x) B_i does not depend on it.
#include <cmath>

#include "kron_internal.h"

namespace kron {
namespace {

constexpr int kVlMaxS = 32;

// Y (Lout x s) = R X (MODE 0: Lout = p*q, Lin = m*n) or R^T X (MODE 1: Lout = m*n, Lin = p*q)
template <int MODE>
__global__ __launch_bounds__(256) void vl_apply_kernel(int p, int q, int m, int n, int s, const float* __restrict__ W,
                                                       const float* __restrict__ X, float* __restrict__ Y) {
  __shared__ float Xs[64][kVlMaxS + 1];
  __shared__ float Rs[16][65];
  const int tid = threadIdx.x;
  const int M = p * q, K = m * n, out = q * n;
  const int Lout = MODE == 0 ? M : K, Lin = MODE == 0 ? K : M;
  const int o0 = blockIdx.x * 16;
  const int rl = tid / 16, cg = tid % 16;
  float acc0 = 0.f, acc1 = 0.f;
  for (int c0 = 0; c0 < Lin; c0 += 64) {
    __syncthreads();
    for (int e = tid; e < 64 * s; e += 256) {
      const int rr = e / s, t = e - rr * s;
      Xs[rr][t] = c0 + rr < Lin ? X[(int64_t)(c0 + rr) * s + t] : 0.f;
    }
    for (int e = tid; e < 16 * 64; e += 256) {
      const int ol = e / 64, cl = e - ol * 64;
      const int o = o0 + ol, ci = c0 + cl;
      float v = 0.f;
      if (o < Lout && ci < Lin) {
        const int i = MODE == 0 ? o : ci, col = MODE == 0 ? ci : o;   // R[i][col]
        const int j = i / q, k = i - j * q, a = col / n, b = col - a * n;
        v = W[(int64_t)(j * m + a) * out + k * n + b];
      }
      Rs[ol][cl] = v;
    }
    __syncthreads();
#pragma unroll 8
    for (int cl = 0; cl < 64; ++cl) {
      const float rv = Rs[rl][cl];
      acc0 = fmaf(rv, Xs[cl][cg], acc0);
      acc1 = fmaf(rv, Xs[cl][cg + 16], acc1);
    }
  }
  const int o = o0 + rl;
  if (o < Lout) {
    if (cg < s) Y[(int64_t)o * s + cg] = acc0;
    if (cg + 16 < s) Y[(int64_t)o * s + cg + 16] = acc1;
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Columns of X (L x s, row-major) made orthonormal in place: classical Gram-Schmidt with
// one re-orthogonalisation per column; a zero column stays zero.  One workgroup.
__global__ __launch_bounds__(1024) void vl_orth_kernel(int L, int s, float* __restrict__ X) {
  __shared__ float part[16][kVlMaxS + 1];
  __shared__ float dots[kVlMaxS + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int t = 0; t < s; ++t) {
    for (int pass = 0; pass < 2 && t > 0; ++pass) {
      float pd[kVlMaxS];
#pragma unroll
      for (int u = 0; u < kVlMaxS; ++u) pd[u] = 0.f;
      for (int l = tid; l < L; l += 1024) {
        const float xt = X[(int64_t)l * s + t];
#pragma unroll
        for (int u = 0; u < kVlMaxS; ++u)
          if (u < t) pd[u] = fmaf(xt, X[(int64_t)l * s + u], pd[u]);
      }
#pragma unroll
      for (int u = 0; u < kVlMaxS; ++u) {
        if (u < t) {
          const float w = wave_sum(pd[u]);
          if (lane == 0) part[wave][u] = w;
        }
      }
      __syncthreads();
      if (tid < t) {
        float d = 0.f;
        for (int w = 0; w < 16; ++w) d += part[w][tid];
        dots[tid] = d;
      }
      __syncthreads();
      for (int l = tid; l < L; l += 1024) {
        float xt = X[(int64_t)l * s + t];
        for (int u = 0; u < t; ++u) xt = fmaf(-dots[u], X[(int64_t)l * s + u], xt);
        X[(int64_t)l * s + t] = xt;
      }
      __syncthreads();
    }
    float ps = 0.f;
    for (int l = tid; l < L; l += 1024) {
      const float xt = X[(int64_t)l * s + t];
      ps = fmaf(xt, xt, ps);
    }
    ps = wave_sum(ps);
    if (lane == 0) part[wave][0] = ps;
    __syncthreads();
    if (tid == 0) {
      float d = 0.f;
      for (int w = 0; w < 16; ++w) d += part[w][0];
      dots[kVlMaxS] = d > 0.f ? 1.f / sqrtf(d) : 0.f;
    }
    __syncthreads();
    const float inv = dots[kVlMaxS];
    for (int l = tid; l < L; l += 1024) X[(int64_t)l * s + t] *= inv;
    __syncthreads();
  }
}

// G = Bt^T Bt (s x s, Bt is K x s), then its eigenvectors E (columns, by cyclic Jacobi on
// one wavefront) and eigenvalues lam, sorted by decreasing eigenvalue.
__global__ __launch_bounds__(256) void vl_eig_kernel(int K, int s, const float* __restrict__ Bt, float* __restrict__ E,
                                                     float* __restrict__ lam) {
  __shared__ float G[kVlMaxS][kVlMaxS + 1];
  __shared__ float V[kVlMaxS][kVlMaxS + 1];
  __shared__ int order[kVlMaxS];
  const int tid = threadIdx.x;
  for (int e = tid; e < s * s; e += 256) {
    const int u = e / s, v = e - u * s;
    float acc = 0.f;
    for (int l = 0; l < K; ++l) acc = fmaf(Bt[(int64_t)l * s + u], Bt[(int64_t)l * s + v], acc);
    G[u][v] = acc;
    V[u][v] = u == v ? 1.f : 0.f;
  }
  __syncthreads();
  if (tid < 64) {
    const int l = tid;
    for (int sweep = 0; sweep < 40; ++sweep) {
      float off = 0.f, dia = 0.f;
      for (int u = 0; u < s; ++u) {
        dia += G[u][u] * G[u][u];
        for (int v = u + 1; v < s; ++v) off += G[u][v] * G[u][v];
      }
      if (off <= 1e-14f * dia) break;
      for (int u = 0; u < s - 1; ++u) {
        for (int v = u + 1; v < s; ++v) {
          const float guv = G[u][v];
          if (guv == 0.f) continue;
          const float tau = (G[v][v] - G[u][u]) / (2.f * guv);
          const float tt = tau >= 0.f ? 1.f / (tau + sqrtf(1.f + tau * tau)) : -1.f / (-tau + sqrtf(1.f + tau * tau));
          const float cc = 1.f / sqrtf(1.f + tt * tt), ss = tt * cc;
          __builtin_amdgcn_wave_barrier();
          if (l < s) {   // columns u, v of G and of V
            const float a = G[l][u], b = G[l][v];
            G[l][u] = cc * a - ss * b;
            G[l][v] = ss * a + cc * b;
            const float va = V[l][u], vb = V[l][v];
            V[l][u] = cc * va - ss * vb;
            V[l][v] = ss * va + cc * vb;
          }
          __builtin_amdgcn_wave_barrier();
          if (l < s) {   // rows u, v of G
            const float a = G[u][l], b = G[v][l];
            G[u][l] = cc * a - ss * b;
            G[v][l] = ss * a + cc * b;
          }
          __builtin_amdgcn_wave_barrier();
        }
      }
    }
    if (l == 0) {   // order by decreasing eigenvalue (stable selection)
      for (int i = 0; i < s; ++i) order[i] = i;
      for (int i = 0; i < s; ++i) {
        int best = i;
        for (int j = i + 1; j < s; ++j)
          if (G[order[j]][order[j]] > G[order[best]][order[best]]) best = j;
        const int tmp = order[i];
        order[i] = order[best];
        order[best] = tmp;
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < s * s; e += 256) {
    const int u = e / s, i = e - u * s;
    E[u * s + i] = V[u][order[i]];
  }
  if (tid < s) lam[tid] = G[order[tid]][order[tid]];
}

// Term i = blockIdx.x: u = Z E e_i (M), v = Bt E e_i / sigma (K), sign, scaled factors.
__global__ __launch_bounds__(1024) void vl_assemble_kernel(int M, int K, int s, const float* __restrict__ Z,
                                                           const float* __restrict__ Bt, const float* __restrict__ E,
                                                           const float* __restrict__ lam, float* __restrict__ C,
                                                           float* __restrict__ B, float* __restrict__ sigma) {
  extern __shared__ float u[];   // M
  __shared__ float bv[16];
  __shared__ int bi[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, i = blockIdx.x;
  const float lm = lam[i];
  const float sg = lm > 0.f ? sqrtf(lm) : 0.f;
  float best = -1.f;
  int bidx = 0x7fffffff;
  for (int l = tid; l < M; l += 1024) {
    float acc = 0.f;
    for (int t = 0; t < s; ++t) acc = fmaf(Z[(int64_t)l * s + t], E[t * s + i], acc);
    u[l] = acc;
    const float a = fabsf(acc);
    if (a > best) {   // l increases within a thread, so the first index wins ties
      best = a;
      bidx = l;
    }
  }
  // the largest |u| and its first index: per wavefront, then across wavefronts in order
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ob = __shfl_xor(best, off, 64);
    const int oi = __shfl_xor(bidx, off, 64);
    if (ob > best || (ob == best && oi < bidx)) {
      best = ob;
      bidx = oi;
    }
  }
  if (lane == 0) {
    bv[wave] = best;
    bi[wave] = bidx;
  }
  __syncthreads();
  float gb = bv[0];
  int gi = bi[0];
  for (int w = 1; w < 16; ++w)
    if (bv[w] > gb || (bv[w] == gb && bi[w] < gi)) {
      gb = bv[w];
      gi = bi[w];
    }
  const float sgn = u[gi] >= 0.f ? 1.f : -1.f;
  const float root = sqrtf(sg);
  for (int l = tid; l < M; l += 1024) C[(int64_t)i * M + l] = sgn * root * u[l];
  const float scale = sg > 0.f ? sgn / root : 0.f;   // sqrt(sigma) * v with v = Bt E e_i / sigma
  for (int l = tid; l < K; l += 1024) {
    float acc = 0.f;
    for (int t = 0; t < s; ++t) acc = fmaf(Bt[(int64_t)l * s + t], E[t * s + i], acc);
    B[(int64_t)i * K + l] = scale * acc;
  }
  if (tid == 0) sigma[i] = sg;
}

size_t align256v(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

size_t van_loan_workspace_bytes(int p, int q, int m, int n, int s) {
  const size_t M = (size_t)p * q, K = (size_t)m * n;
  return align256v(M * s * 4) + align256v(K * s * 4) + align256v((size_t)s * s * 4) + align256v((size_t)s * 4);
}

hipError_t launch_van_loan(const VanLoanArgs& A, void* ws, hipStream_t st) {
  const int M = A.p * A.q, K = A.m * A.n, s = A.s;
  unsigned char* w = static_cast<unsigned char*>(ws);
  float* Z = reinterpret_cast<float*>(w);
  float* Q = reinterpret_cast<float*>(w + align256v((size_t)M * s * 4));
  float* E = reinterpret_cast<float*>(w + align256v((size_t)M * s * 4) + align256v((size_t)K * s * 4));
  float* lam = E + align256v((size_t)s * s * 4) / 4;
  hipError_t e = hipMemcpyAsync(Q, A.omega, (size_t)K * s * 4, hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return e;
  const dim3 gM((unsigned)((M + 15) / 16)), gK((unsigned)((K + 15) / 16));
  hipLaunchKernelGGL(vl_orth_kernel, dim3(1), dim3(1024), 0, st, K, s, Q);
  for (int it = 0; it < A.iters; ++it) {
    hipLaunchKernelGGL(vl_apply_kernel<0>, gM, dim3(256), 0, st, A.p, A.q, A.m, A.n, s, A.W, Q, Z);
    hipLaunchKernelGGL(vl_orth_kernel, dim3(1), dim3(1024), 0, st, M, s, Z);
    hipLaunchKernelGGL(vl_apply_kernel<1>, gK, dim3(256), 0, st, A.p, A.q, A.m, A.n, s, A.W, Z, Q);
    hipLaunchKernelGGL(vl_orth_kernel, dim3(1), dim3(1024), 0, st, K, s, Q);
  }
  hipLaunchKernelGGL(vl_apply_kernel<0>, gM, dim3(256), 0, st, A.p, A.q, A.m, A.n, s, A.W, Q, Z);
  hipLaunchKernelGGL(vl_orth_kernel, dim3(1), dim3(1024), 0, st, M, s, Z);
  hipLaunchKernelGGL(vl_apply_kernel<1>, gK, dim3(256), 0, st, A.p, A.q, A.m, A.n, s, A.W, Z, Q);   // Bt
  hipLaunchKernelGGL(vl_eig_kernel, dim3(1), dim3(256), 0, st, K, s, Q, E, lam);
  hipLaunchKernelGGL(vl_assemble_kernel, dim3((unsigned)A.r), dim3(1024), (size_t)M * 4, st, M, K, s, Z, Q, E, lam,
                     A.C, A.B, A.sigma);
  return hipGetLastError();
}

}  // namespace kron
