// Van Loan rank-r Kronecker projection of a dense W ("Replicating & Extending Krony-PT on
// GPT-2 Small", section "Core Algorithm - Van Loan Kronecker Decomposition"): rearrange W
// into R with R[(j*q + k), (a*n + b)] = W[j*m + a, k*n + b] (W is in x out, in = p*m,
// out = q*n), take the leading r singular triplets of R, and return C_i = sqrt(sigma_i) *
// reshape(u_i, p x q), B_i = sqrt(sigma_i) * reshape(v_i, m x n), so that
// sum_i kron(C_i, B_i) is the best rank-r sum of Kronecker products to W.
//
// The singular triplets come from block subspace iteration (the standard randomized
// range finder with power iterations) started from a caller-supplied random K x s block:
//   Q <- orth(Omega); repeat iters times: Q <- orth(R^T (R Q)) (orthogonal iteration on
//   R^T R; the span of R^T R Q does not depend on orthonormalising R Q first; inside the
//   loop orth is a shifted Cholesky-QR re-basing, which keeps the span);
//   Z <- orth(R Q); Bt <- R^T Z (= (Z^T R)^T); G = Bt^T Bt = E diag(lambda) E^T (Jacobi);
//   u_i = Z E e_i, sigma_i = sqrt(lambda_i), v_i = Bt E e_i / sigma_i.
// R is never materialised: the products read W through the index map above.  The s-column
// panels (Q, Z, Bt) live in the workspace column by column ([s][L]), so every column is
// contiguous.  All sums run in a fixed order (bitwise repeatable).  Sign of each pair: the
// entry of u_i largest in magnitude (the first such) is made positive; C_i (x) B_i does not
// depend on it.
#include <cmath>

#include "kron_internal.h"

namespace kron {
namespace {

constexpr int kVlMaxS = 32;
constexpr int kVlApplyThreads = 256;
constexpr size_t kVlApplyLds = 128 * 1024;
constexpr int kVlOrthThreads = 1024;
constexpr int kVlOrthWaves = kVlOrthThreads / 64;
constexpr int kVlBatch = 16;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Orders one wavefront's LDS accesses: what its lanes wrote before is seen by its lanes after.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// x = quo * d + rem for 0 <= x < 2^24, d >= 1: the float quotient is off by at most one,
// which one correction step fixes.
__device__ __forceinline__ void divmod(int x, int d, float invd, int& quo, int& rem) {
  int qq = __float2int_rz((float)x * invd);
  int rr = x - qq * d;
  if (rr < 0) {
    --qq;
    rr += d;
  } else if (rr >= d) {
    ++qq;
    rr -= d;
  }
  quo = qq;
  rem = rr;
}

// Yt (s x Lout, column panel) = R Xt^T (MODE 0: Lout = p*q, Lin = m*n) or R^T Xt^T (MODE 1:
// Lout = m*n, Lin = p*q).  A workgroup owns O consecutive outputs rows o and takes the
// contraction in chunks of CH: the chunk of the input panel (s x CH) and of the O rows of R
// (O x CH, gathered from W through the index map) are staged in LDS, then every output
// (o, t) is split over G contiguous slices of the chunk and the G partial sums are added in
// slice order.  For MODE 0, O consecutive rows (j, k) read O runs of n contiguous W values
// per W row; for MODE 1 the O rows (a, b) are O consecutive W columns of one W row.
template <int MODE, int O>
__global__ __launch_bounds__(kVlApplyThreads) void vl_apply_kernel(int p, int q, int m, int n, int s, int CH,
                                                                   const float* __restrict__ W,
                                                                   const float* __restrict__ Xt,
                                                                   float* __restrict__ Yt) {
  extern __shared__ float sm[];
  const int LD = CH + 4;
  float* xs = sm;               // [s][LD]
  float* ts = sm + s * LD;      // [O][LD]
  float* red = ts + O * LD;     // [kVlApplyThreads]
  const int tid = threadIdx.x;
  const int M = p * q, K = m * n, out = q * n;
  const int Lout = MODE == 0 ? M : K, Lin = MODE == 0 ? K : M;
  const int o0 = blockIdx.x * O;
  const float inv_q = 1.f / (float)q, inv_n = 1.f / (float)n;
  const int nout = O * s;
  const int G = kVlApplyThreads / nout;
  const int t = tid % s, r2 = tid / s, ol = r2 % O, g = r2 / O;
  const bool active = tid < nout * G;
  float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
  for (int c0 = 0; c0 < Lin; c0 += CH) {
    const int len = min(CH, Lin - c0);
    const int lenp = (len + 3) & ~3;
    const float inv_lenp = 1.f / (float)lenp;
    __syncthreads();
    // every load of a batch is issued before its LDS stores, so a batch costs one trip
    if ((Lin & 3) == 0) {
      const int q4 = lenp / 4, nx = s * q4;
      const float inv_q4 = 1.f / (float)q4;
      for (int base = 0; base < nx; base += kVlBatch * kVlApplyThreads) {
        float4 r[kVlBatch];
#pragma unroll
        for (int u = 0; u < kVlBatch; ++u) {
          const int it = base + u * kVlApplyThreads + tid;
          r[u] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (it < nx) {
            int tt, c4;
            divmod(it, q4, inv_q4, tt, c4);
            r[u] = *reinterpret_cast<const float4*>(Xt + (int64_t)tt * Lin + c0 + 4 * c4);
          }
        }
#pragma unroll
        for (int u = 0; u < kVlBatch; ++u) {
          const int it = base + u * kVlApplyThreads + tid;
          if (it < nx) {
            int tt, c4;
            divmod(it, q4, inv_q4, tt, c4);
            *reinterpret_cast<float4*>(xs + tt * LD + 4 * c4) = r[u];
          }
        }
      }
    } else {
      const int nx = s * lenp;
      for (int base = 0; base < nx; base += kVlBatch * kVlApplyThreads) {
        float r[kVlBatch];
#pragma unroll
        for (int u = 0; u < kVlBatch; ++u) {
          const int it = base + u * kVlApplyThreads + tid;
          r[u] = 0.f;
          if (it < nx) {
            int tt, cl;
            divmod(it, lenp, inv_lenp, tt, cl);
            if (cl < len) r[u] = Xt[(int64_t)tt * Lin + c0 + cl];
          }
        }
#pragma unroll
        for (int u = 0; u < kVlBatch; ++u) {
          const int it = base + u * kVlApplyThreads + tid;
          if (it < nx) {
            int tt, cl;
            divmod(it, lenp, inv_lenp, tt, cl);
            xs[tt * LD + cl] = r[u];
          }
        }
      }
    }
    {
      const int nt = O * lenp;
      for (int base = 0; base < nt; base += kVlBatch * kVlApplyThreads) {
        float r[kVlBatch];
#pragma unroll
        for (int u = 0; u < kVlBatch; ++u) {
          const int it = base + u * kVlApplyThreads + tid;
          r[u] = 0.f;
          if (it < nt) {
            // MODE 0: consecutive items walk a row of R (runs of n contiguous W values);
            // MODE 1: consecutive items walk the O rows (O consecutive W columns)
            int rr, cl;
            if (MODE == 0)
              divmod(it, lenp, inv_lenp, rr, cl);
            else
              rr = it % O, cl = it / O;
            const int o = o0 + rr, c = c0 + cl;
            if (o < Lout && cl < len) {
              int j, k, a, b;
              divmod(MODE == 0 ? o : c, q, inv_q, j, k);
              divmod(MODE == 0 ? c : o, n, inv_n, a, b);
              r[u] = W[(int64_t)(j * m + a) * out + k * n + b];
            }
          }
        }
#pragma unroll
        for (int u = 0; u < kVlBatch; ++u) {
          const int it = base + u * kVlApplyThreads + tid;
          if (it < nt) {
            int rr, cl;
            if (MODE == 0)
              divmod(it, lenp, inv_lenp, rr, cl);
            else
              rr = it % O, cl = it / O;
            ts[rr * LD + cl] = r[u];
          }
        }
      }
    }
    __syncthreads();
    if (active) {
      const int per = ((lenp / 4 + G - 1) / G) * 4;
      const int cb = g * per, ce = min(lenp, cb + per);
      const float4* xr = reinterpret_cast<const float4*>(xs + t * LD);
      const float4* tr = reinterpret_cast<const float4*>(ts + ol * LD);
#pragma unroll 4
      for (int c4 = cb / 4; c4 < ce / 4; ++c4) {
        const float4 xv = xr[c4], tv = tr[c4];
        acc0 = fmaf(tv.x, xv.x, acc0);
        acc1 = fmaf(tv.y, xv.y, acc1);
        acc2 = fmaf(tv.z, xv.z, acc2);
        acc3 = fmaf(tv.w, xv.w, acc3);
      }
    }
  }
  if (active) red[tid] = (acc0 + acc1) + (acc2 + acc3);
  __syncthreads();
  if (tid < nout) {   // the slice-0 thread of output (ol, t) adds the G slices in order
    float sum = 0.f;
    for (int gg = 0; gg < G; ++gg) sum += red[gg * nout + tid];
    const int o = o0 + ol;
    if (o < Lout) Yt[(int64_t)t * Lout + o] = sum;
  }
}

// Workgroup-wide sums of v[u], u < cnt (cnt is a compile-time constant after unrolling):
// per wavefront, then over wavefronts in order.  Results land in dots[u].
__device__ __forceinline__ void block_sums(const float* v, int cnt, float (*part)[kVlMaxS + 1], float* dots) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int u = 0; u < kVlMaxS; ++u) {
    if (u < cnt) {
      const float w = wave_sum(v[u]);
      if (lane == 0) part[wave][u] = w;
    }
  }
  __syncthreads();
  if (tid < cnt) {
    float d = 0.f;
#pragma unroll
    for (int w = 0; w < kVlOrthWaves; ++w) d += part[w][tid];
    dots[tid] = d;
  }
  __syncthreads();
}

// Sum over a wavefront through DPP: two quad permutations and two row rotations leave each
// 16-lane row's total in all of its lanes, then the four row totals are read out and added
// in a fixed order.  Needs every lane active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// the four 16-lane row totals (each row already holds its total in every lane), added in order
__device__ __forceinline__ float row_total(float v) {
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_mov<0x124>(v);   // row_ror 4
  v += dpp_mov<0x128>(v);   // row_ror 8
  return row_total(v);
}

// Columns of an L x s panel (L <= 1024) made orthonormal: classical Gram-Schmidt with one
// re-orthogonalisation per column, a zero column stays zero.  One workgroup of four
// wavefronts; thread tid holds rows tid + 256 i (i < 4) of every column in registers.  Each
// workgroup-wide sum is one barrier: the wavefront totals go to one of two alternating LDS
// slots and every thread adds the four in order.  The input is read row-major (L x s,
// ROWIN) or as a column panel; the output is a column panel (may alias a column-panel input).
constexpr int kVlOrthRegThreads = 256;
constexpr int kVlOrthRegRows = 4;

template <int SM, bool ROWIN>
__global__ __launch_bounds__(kVlOrthRegThreads) void vl_orth_reg_kernel(int L, int s, const float* in, float* X) {
  constexpr int NW = kVlOrthRegThreads / 64;
  __shared__ float part[2][NW][kVlMaxS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float x[kVlOrthRegRows][SM];
#pragma unroll
  for (int i = 0; i < kVlOrthRegRows; ++i) {
    const int l = tid + i * kVlOrthRegThreads;
#pragma unroll
    for (int u = 0; u < SM; ++u)
      x[i][u] = (l < L && u < s) ? (ROWIN ? in[(int64_t)l * s + u] : in[(int64_t)u * L + l]) : 0.f;
  }
  int buf = 0;
#pragma unroll
  for (int t = 0; t < SM; ++t) {
    if (t < s) {
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        if (t > 0) {
          // the t sums advance together, one DPP step for all of them at a time
          float pd[SM];
#pragma unroll
          for (int u = 0; u < t; ++u) {
            pd[u] = 0.f;
#pragma unroll
            for (int i = 0; i < kVlOrthRegRows; ++i) pd[u] = fmaf(x[i][t], x[i][u], pd[u]);
          }
#pragma unroll
          for (int u = 0; u < t; ++u) pd[u] += dpp_mov<0xB1>(pd[u]);
#pragma unroll
          for (int u = 0; u < t; ++u) pd[u] += dpp_mov<0x4E>(pd[u]);
#pragma unroll
          for (int u = 0; u < t; ++u) pd[u] += dpp_mov<0x124>(pd[u]);
#pragma unroll
          for (int u = 0; u < t; ++u) pd[u] += dpp_mov<0x128>(pd[u]);
#pragma unroll
          for (int u = 0; u < t; ++u) pd[u] = row_total(pd[u]);
          if (lane == 0) {
#pragma unroll
            for (int u = 0; u < t; ++u) part[buf][wave][u] = pd[u];
          }
          __syncthreads();
#pragma unroll
          for (int u = 0; u < t; ++u) {
            const float d = (part[buf][0][u] + part[buf][1][u]) + (part[buf][2][u] + part[buf][3][u]);
#pragma unroll
            for (int i = 0; i < kVlOrthRegRows; ++i) x[i][t] = fmaf(-d, x[i][u], x[i][t]);
          }
          buf ^= 1;
        }
      }
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < kVlOrthRegRows; ++i) ps = fmaf(x[i][t], x[i][t], ps);
      const float w = wave_sum_dpp(ps);
      if (lane == 0) part[buf][wave][0] = w;
      __syncthreads();
      const float nn = (part[buf][0][0] + part[buf][1][0]) + (part[buf][2][0] + part[buf][3][0]);
      buf ^= 1;
      const float inv = nn > 0.f ? 1.f / sqrtf(nn) : 0.f;
#pragma unroll
      for (int i = 0; i < kVlOrthRegRows; ++i) x[i][t] *= inv;
    }
  }
  __syncthreads();   // an aliased input has been read by every thread before any write
#pragma unroll
  for (int i = 0; i < kVlOrthRegRows; ++i) {
    const int l = tid + i * kVlOrthRegThreads;
    if (l < L) {
#pragma unroll
      for (int u = 0; u < SM; ++u)
        if (u < s) X[(int64_t)u * L + l] = x[i][u];
    }
  }
}

// Inside the power iteration only the span of Q matters, so its L x s panel (L <= 1024) is
// re-based with one round of shifted Cholesky-QR instead of Gram-Schmidt: the Gram matrix
// G = X^T X (all s(s+1)/2 sums at once: per wavefront by DPP, then over wavefronts in fp64),
// G + shift * I = R^T R by Cholesky in fp64 on one wavefront (the shift, 1e-6 of G's mean
// diagonal, keeps a rank-deficient panel factorisable), then X <- X R^{-1} row by row by
// forward substitution.  Columns that carry the dominant directions come out orthonormal to
// about the shift; the last orthonormalisation (of Z) is the Gram-Schmidt kernel above.
constexpr int kVlPairs = kVlMaxS * (kVlMaxS + 1) / 2;

template <int SM, bool ROWIN>
__global__ __launch_bounds__(kVlOrthRegThreads) void vl_cholqr_kernel(int L, int s, const float* in, float* X) {
  constexpr int NW = kVlOrthRegThreads / 64;
  __shared__ float part[NW][kVlPairs];
  __shared__ double G[kVlMaxS][kVlMaxS + 1];
  __shared__ float R[kVlMaxS][kVlMaxS + 1];   // upper triangle of R; R[t][t] holds 1 / R_tt
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float x[kVlOrthRegRows][SM];
#pragma unroll
  for (int i = 0; i < kVlOrthRegRows; ++i) {
    const int l = tid + i * kVlOrthRegThreads;
#pragma unroll
    for (int u = 0; u < SM; ++u)
      x[i][u] = (l < L && u < s) ? (ROWIN ? in[(int64_t)l * s + u] : in[(int64_t)u * L + l]) : 0.f;
  }
  // Gram row u: pairs (u, v), v >= u, at pair index u*s - u(u-1)/2 + (v - u)
#pragma unroll
  for (int u = 0; u < SM; ++u) {
    if (u < s) {
      float pd[SM];
#pragma unroll
      for (int v = u; v < SM; ++v) {
        pd[v] = 0.f;
#pragma unroll
        for (int i = 0; i < kVlOrthRegRows; ++i) pd[v] = fmaf(x[i][u], x[i][v], pd[v]);
      }
#pragma unroll
      for (int v = u; v < SM; ++v) pd[v] += dpp_mov<0xB1>(pd[v]);
#pragma unroll
      for (int v = u; v < SM; ++v) pd[v] += dpp_mov<0x4E>(pd[v]);
#pragma unroll
      for (int v = u; v < SM; ++v) pd[v] += dpp_mov<0x124>(pd[v]);
#pragma unroll
      for (int v = u; v < SM; ++v) pd[v] += dpp_mov<0x128>(pd[v]);
#pragma unroll
      for (int v = u; v < SM; ++v) pd[v] = row_total(pd[v]);
      if (lane == 0) {
        const int base = u * s - u * (u - 1) / 2 - u;
#pragma unroll
        for (int v = u; v < SM; ++v)
          if (v < s) part[wave][base + v] = pd[v];
      }
    }
  }
  __syncthreads();
  const int npairs = s * (s + 1) / 2;
  for (int pi = tid; pi < npairs; pi += kVlOrthRegThreads) {
    int u = 0, rem = pi;
    while (rem >= s - u) {
      rem -= s - u;
      ++u;
    }
    const int v = u + rem;
    double g = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) g += (double)part[w][pi];
    G[u][v] = g;
    G[v][u] = g;
  }
  __syncthreads();
  if (tid < 64) {   // Cholesky of G + shift * I, right-looking, lanes over the trailing columns
    const int l = tid;
    double tr = 0.0;
    if (l < s) tr = G[l][l];
    tr = wave_sum(tr);
    const double shift = 1e-6 * tr / s + 1e-300;
    if (l < s) G[l][l] += shift;
    wave_sync();
    for (int t = 0; t < s; ++t) {
      const double d = sqrt(G[t][t] > 0.0 ? G[t][t] : shift);
      const double inv = 1.0 / d;
      if (l >= t && l < s) R[t][l] = l == t ? (float)inv : (float)(G[t][l] * inv);
      wave_sync();
      for (int e = l; e < (s - t - 1) * (s - t - 1); e += 64) {   // trailing update
        const int a = t + 1 + e / (s - t - 1), b = t + 1 + e % (s - t - 1);
        G[a][b] -= (G[t][a] * inv) * (G[t][b] * inv);
      }
      wave_sync();
    }
  }
  __syncthreads();
  // X <- X R^{-1}: x_t = (x_t - sum_{u<t} R[u][t] x_u) / R_tt, row by row
#pragma unroll
  for (int t = 0; t < SM; ++t) {
    if (t < s) {
#pragma unroll
      for (int u = 0; u < t; ++u) {
        const float ru = R[u][t];
#pragma unroll
        for (int i = 0; i < kVlOrthRegRows; ++i) x[i][t] = fmaf(-ru, x[i][u], x[i][t]);
      }
      const float inv = R[t][t];
#pragma unroll
      for (int i = 0; i < kVlOrthRegRows; ++i) x[i][t] *= inv;
    }
  }
  __syncthreads();   // an aliased input has been read by every thread before any write
#pragma unroll
  for (int i = 0; i < kVlOrthRegRows; ++i) {
    const int l = tid + i * kVlOrthRegThreads;
    if (l < L) {
#pragma unroll
      for (int u = 0; u < SM; ++u)
        if (u < s) X[(int64_t)u * L + l] = x[i][u];
    }
  }
}

// The same orthonormalisation for panels too tall for registers (L > 1024): the panel is
// worked on in place in global memory.  Every thread reads and writes only its own rows.
template <bool ROWIN>
__global__ __launch_bounds__(kVlOrthThreads) void vl_orth_mem_kernel(int L, int s, const float* in, float* X) {
  __shared__ float part[kVlOrthWaves][kVlMaxS + 1];
  __shared__ float dots[kVlMaxS + 1];
  const int tid = threadIdx.x;
  if (ROWIN) {
    for (int l = tid; l < L; l += kVlOrthThreads)
      for (int u = 0; u < s; ++u) X[(int64_t)u * L + l] = in[(int64_t)l * s + u];
  }
  for (int t = 0; t < s; ++t) {
    float* xt = X + (int64_t)t * L;
    for (int pass = 0; pass < 2 && t > 0; ++pass) {
      float pd[kVlMaxS];
#pragma unroll
      for (int u = 0; u < kVlMaxS; ++u) pd[u] = 0.f;
      for (int l = tid; l < L; l += kVlOrthThreads) {
        const float v = xt[l];
#pragma unroll
        for (int u = 0; u < kVlMaxS; ++u)
          if (u < t) pd[u] = fmaf(v, X[(int64_t)u * L + l], pd[u]);
      }
      block_sums(pd, t, part, dots);
      for (int l = tid; l < L; l += kVlOrthThreads) {
        float v = xt[l];
        for (int u = 0; u < t; ++u) v = fmaf(-dots[u], X[(int64_t)u * L + l], v);
        xt[l] = v;
      }
    }
    float ps[1] = {0.f};
    for (int l = tid; l < L; l += kVlOrthThreads) ps[0] = fmaf(xt[l], xt[l], ps[0]);
    block_sums(ps, 1, part, dots);
    const float nn = dots[0];
    const float inv = nn > 0.f ? 1.f / sqrtf(nn) : 0.f;
    for (int l = tid; l < L; l += kVlOrthThreads) xt[l] *= inv;
  }
}

// G = Bt^T Bt (s x s; Bt is a K x s column panel) accumulated in fp64 (the fp32 products
// are exact there), then its eigenvectors E (columns) and eigenvalues lam by cyclic Jacobi
// in fp64 on one wavefront (round-robin ordering), sorted by decreasing eigenvalue.
constexpr int kVlEigThreads = 1024;
constexpr int kVlEigChunk = 256;
constexpr int kVlJacItems = (kVlMaxS * kVlMaxS / 2 + 63) / 64;   // (pair, row) items per lane
constexpr int kVlJacBatch = 2;
static_assert(kVlMaxS * kVlEigChunk <= 8 * kVlEigThreads, "a chunk of the panel is staged 8 values per thread");

__global__ __launch_bounds__(kVlEigThreads) void vl_eig_kernel(int K, int s, const float* __restrict__ Bt,
                                                               float* __restrict__ E, float* __restrict__ lam) {
  __shared__ float bs[kVlMaxS][kVlEigChunk + 1];
  __shared__ double part[kVlEigThreads];
  __shared__ double G[kVlMaxS][kVlMaxS + 1];
  __shared__ double V[kVlMaxS][kVlMaxS + 1];
  __shared__ int order[kVlMaxS];
  __shared__ unsigned char pair_u[kVlMaxS - 1][kVlMaxS / 2], pair_v[kVlMaxS - 1][kVlMaxS / 2];
  __shared__ double rot_c[kVlMaxS / 2], rot_s[kVlMaxS / 2];
  const int tid = threadIdx.x;
  const int npairs = s * (s + 1) / 2;
  const int ngroups = kVlEigThreads / npairs;
  const int pr = tid % npairs, grp = tid / npairs;
  int pu = 0, pv = 0;   // pair pr -> (pu <= pv), row-major over the upper triangle
  {
    int rem = pr;
    while (rem >= s - pu) {
      rem -= s - pu;
      ++pu;
    }
    pv = pu + rem;
  }
  double acc = 0.0;
  for (int c0 = 0; c0 < K; c0 += kVlEigChunk) {
    const int len = min(kVlEigChunk, K - c0);
    __syncthreads();
    {   // the chunk is at most 32 x 256 values, 8 per thread: all loads before the stores
      const int nel = s * len;
      const float invl = 1.f / (float)len;
      float r[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int e = tid + w * kVlEigThreads;
        r[w] = 0.f;
        if (e < nel) {
          int u, c;
          divmod(e, len, invl, u, c);
          r[w] = Bt[(int64_t)u * K + c0 + c];
        }
      }
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int e = tid + w * kVlEigThreads;
        if (e < nel) {
          int u, c;
          divmod(e, len, invl, u, c);
          bs[u][c] = r[w];
        }
      }
    }
    __syncthreads();
    if (grp < ngroups)
      for (int c = grp; c < len; c += ngroups) acc = fma((double)bs[pu][c], (double)bs[pv][c], acc);
  }
  part[tid] = acc;
  __syncthreads();
  if (tid < npairs) {
    double sum = 0.0;
    for (int gg = 0; gg < ngroups; ++gg) sum += part[gg * npairs + tid];
    G[pu][pv] = sum;
    G[pv][pu] = sum;
  }
  for (int e = tid; e < s * s; e += kVlEigThreads) {
    const int u = e / s, v = e - u * s;
    V[u][v] = u == v ? 1.0 : 0.0;
  }
  {   // round k of the circle pairing: position 0 fixed, positions 1.. rotate by k; pair i
      // joins positions i and se - 1 - i; a pair with the padding index se - 1 = s (s odd)
      // is stored as (u, u), the identity
    const int se = s + (s & 1), np = se / 2;
    for (int e = tid; e < (se - 1) * np; e += kVlEigThreads) {
      const int k = e / np, i = e - k * np;
      const int pa = i == 0 ? 0 : ((i - 1 + k) % (se - 1)) + 1;
      const int pb = ((se - 2 - i + k) % (se - 1)) + 1;
      const int u = min(pa, pb), v = max(pa, pb);
      pair_u[k][i] = (unsigned char)u;
      pair_v[k][i] = (unsigned char)(v < s ? v : u);
    }
  }
  __syncthreads();
  if (tid < 64) {
    // Parallel cyclic Jacobi: a sweep is se - 1 rounds of the round-robin (circle) pairing
    // of se = s rounded up to even indices, index 0 fixed and the others rotating; every
    // unordered pair meets once per sweep, and the rotations of one round act on disjoint
    // index pairs, so they are computed together from the same G and applied together
    // (columns, i.e. G J and V J, then rows, J^T (G J)).
    const int l = tid;
    const int se = s + (s & 1), np = se / 2, nitems = s * np;
    // this lane's (pair, row) items of the column and row phases, fixed for every round
    int ipair[kVlJacItems], irow[kVlJacItems];
#pragma unroll
    for (int w = 0; w < kVlJacItems; ++w) {
      const int it = l + 64 * w;
      ipair[w] = it < nitems ? it / s : -1;
      irow[w] = it < nitems ? it - ipair[w] * s : 0;
    }
    for (int sweep = 0; sweep < 40; ++sweep) {
      double off = 0.0, dia = 0.0;
      if (l < s) {
        dia = G[l][l] * G[l][l];
        for (int v = l + 1; v < s; ++v) off += G[l][v] * G[l][v];
      }
      off = wave_sum(off);
      dia = wave_sum(dia);
      if (off <= 1e-26 * dia) break;
      for (int k = 0; k < se - 1; ++k) {
        if (l < np) {
          const int u = pair_u[k][l], v = pair_v[k][l];
          double cc = 1.0, ss = 0.0;
          if (v != u) {
            const double guv = G[u][v];
            if (guv != 0.0) {
              const double tau = (G[v][v] - G[u][u]) / (2.0 * guv);
              const double tt = tau >= 0.0 ? 1.0 / (tau + sqrt(1.0 + tau * tau)) : -1.0 / (-tau + sqrt(1.0 + tau * tau));
              cc = 1.0 / sqrt(1.0 + tt * tt);
              ss = tt * cc;
            }
          }
          rot_c[l] = cc;
          rot_s[l] = ss;
        }
        wave_sync();
        // columns u, v of G and of V, then rows u, v of G; within a batch of items every
        // read comes first, then the writes
        for (int w0 = 0; w0 < kVlJacItems && l + 64 * w0 < nitems; w0 += kVlJacBatch) {
          double ga[kVlJacBatch], gb[kVlJacBatch], va[kVlJacBatch], vb[kVlJacBatch];
          double rc[kVlJacBatch], rs[kVlJacBatch];
          int uu[kVlJacBatch], vv[kVlJacBatch];
#pragma unroll
          for (int w = 0; w < kVlJacBatch; ++w) {
            uu[w] = vv[w] = 0;
            ga[w] = gb[w] = va[w] = vb[w] = rc[w] = rs[w] = 0.0;
            if (ipair[w0 + w] >= 0) {
              const int i = ipair[w0 + w], r = irow[w0 + w];
              uu[w] = pair_u[k][i];
              vv[w] = pair_v[k][i];
              rc[w] = rot_c[i];
              rs[w] = rot_s[i];
              ga[w] = G[r][uu[w]];
              gb[w] = G[r][vv[w]];
              va[w] = V[r][uu[w]];
              vb[w] = V[r][vv[w]];
            }
          }
#pragma unroll
          for (int w = 0; w < kVlJacBatch; ++w) {
            if (ipair[w0 + w] >= 0 && uu[w] != vv[w]) {
              const int r = irow[w0 + w];
              G[r][uu[w]] = rc[w] * ga[w] - rs[w] * gb[w];
              G[r][vv[w]] = rs[w] * ga[w] + rc[w] * gb[w];
              V[r][uu[w]] = rc[w] * va[w] - rs[w] * vb[w];
              V[r][vv[w]] = rs[w] * va[w] + rc[w] * vb[w];
            }
          }
        }
        wave_sync();
        for (int w0 = 0; w0 < kVlJacItems && l + 64 * w0 < nitems; w0 += kVlJacBatch) {
          double ga[kVlJacBatch], gb[kVlJacBatch], rc[kVlJacBatch], rs[kVlJacBatch];
          int uu[kVlJacBatch], vv[kVlJacBatch];
#pragma unroll
          for (int w = 0; w < kVlJacBatch; ++w) {
            uu[w] = vv[w] = 0;
            ga[w] = gb[w] = rc[w] = rs[w] = 0.0;
            if (ipair[w0 + w] >= 0) {
              const int i = ipair[w0 + w], c = irow[w0 + w];
              uu[w] = pair_u[k][i];
              vv[w] = pair_v[k][i];
              rc[w] = rot_c[i];
              rs[w] = rot_s[i];
              ga[w] = G[uu[w]][c];
              gb[w] = G[vv[w]][c];
            }
          }
#pragma unroll
          for (int w = 0; w < kVlJacBatch; ++w) {
            if (ipair[w0 + w] >= 0 && uu[w] != vv[w]) {
              const int c = irow[w0 + w];
              G[uu[w]][c] = rc[w] * ga[w] - rs[w] * gb[w];
              G[vv[w]][c] = rs[w] * ga[w] + rc[w] * gb[w];
            }
          }
        }
        wave_sync();
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
  for (int e = tid; e < s * s; e += kVlEigThreads) {
    const int u = e / s, i = e - u * s;
    E[u * s + i] = (float)V[u][order[i]];
  }
  if (tid < s) lam[tid] = (float)G[order[tid]][order[tid]];
}

// Term i = blockIdx.x: u = Z E e_i (M), v = Bt E e_i / sigma (K), sign, scaled factors.
__global__ __launch_bounds__(1024) void vl_assemble_kernel(int M, int K, int s, const float* __restrict__ Z,
                                                           const float* __restrict__ Bt, const float* __restrict__ E,
                                                           const float* __restrict__ lam, float* __restrict__ C,
                                                           float* __restrict__ B, float* __restrict__ sigma) {
  extern __shared__ float u[];   // M
  __shared__ float bv[16];
  __shared__ int bi[16];
  __shared__ float ev[kVlMaxS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, i = blockIdx.x;
  if (tid < s) ev[tid] = E[tid * s + i];
  __syncthreads();
  const float lm = lam[i];
  const float sg = lm > 0.f ? sqrtf(lm) : 0.f;
  float best = -1.f;
  int bidx = 0x7fffffff;
  for (int l = tid; l < M; l += 1024) {
    float acc = 0.f;
    for (int t = 0; t < s; ++t) acc = fmaf(Z[(int64_t)t * M + l], ev[t], acc);
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
    for (int t = 0; t < s; ++t) acc = fmaf(Bt[(int64_t)t * K + l], ev[t], acc);
    B[(int64_t)i * K + l] = scale * acc;
  }
  if (tid == 0) sigma[i] = sg;
}

size_t align256v(size_t v) { return (v + 255) / 256 * 256; }

constexpr int kVlO0 = 4;   // output rows per workgroup, R X
constexpr int kVlO1 = 8;   // output rows per workgroup, R^T X

// Chunk of the contraction staged per step: as long as the LDS budget allows, a multiple of 4.
int apply_chunk(int Lin, int s, int O) {
  const int64_t fit = (int64_t)(kVlApplyLds / 4 - kVlApplyThreads) / (s + O) - 4;
  int64_t ch = ((int64_t)Lin + 3) / 4 * 4;
  if (ch > fit) ch = fit / 4 * 4;
  return (int)ch;
}

template <int MODE, int O>
void launch_apply(const VanLoanArgs& A, const float* Xt, float* Yt, hipStream_t st) {
  static const bool attr = hipFuncSetAttribute((const void*)vl_apply_kernel<MODE, O>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)kVlApplyLds) == hipSuccess;
  (void)attr;
  const int M = A.p * A.q, K = A.m * A.n;
  const int Lout = MODE == 0 ? M : K, Lin = MODE == 0 ? K : M;
  const int CH = apply_chunk(Lin, A.s, O);
  const size_t lds = ((size_t)(A.s + O) * (CH + 4) + kVlApplyThreads) * 4;
  hipLaunchKernelGGL((vl_apply_kernel<MODE, O>), dim3((unsigned)((Lout + O - 1) / O)), dim3(kVlApplyThreads), lds,
                     st, A.p, A.q, A.m, A.n, A.s, CH, A.W, Xt, Yt);
}

// Re-basing inside the power iteration (the span is what matters): Cholesky-QR when the
// panel fits the register kernels, else Gram-Schmidt in memory.
template <bool ROWIN>
void launch_rebase(int L, int s, const float* in, float* X, hipStream_t st) {
  const dim3 g(1), b(kVlOrthRegThreads);
  if (L <= kVlOrthRegThreads * kVlOrthRegRows && s <= 8)
    hipLaunchKernelGGL((vl_cholqr_kernel<8, ROWIN>), g, b, 0, st, L, s, in, X);
  else if (L <= kVlOrthRegThreads * kVlOrthRegRows && s <= 16)
    hipLaunchKernelGGL((vl_cholqr_kernel<16, ROWIN>), g, b, 0, st, L, s, in, X);
  else if (L <= kVlOrthRegThreads * kVlOrthRegRows)
    hipLaunchKernelGGL((vl_cholqr_kernel<32, ROWIN>), g, b, 0, st, L, s, in, X);
  else
    hipLaunchKernelGGL((vl_orth_mem_kernel<ROWIN>), dim3(1), dim3(kVlOrthThreads), 0, st, L, s, in, X);
}

template <bool ROWIN>
void launch_orth(int L, int s, const float* in, float* X, hipStream_t st) {
  const dim3 g(1), b(kVlOrthRegThreads);
  if (L <= kVlOrthRegThreads * kVlOrthRegRows && s <= 8)
    hipLaunchKernelGGL((vl_orth_reg_kernel<8, ROWIN>), g, b, 0, st, L, s, in, X);
  else if (L <= kVlOrthRegThreads * kVlOrthRegRows && s <= 16)
    hipLaunchKernelGGL((vl_orth_reg_kernel<16, ROWIN>), g, b, 0, st, L, s, in, X);
  else if (L <= kVlOrthRegThreads * kVlOrthRegRows)
    hipLaunchKernelGGL((vl_orth_reg_kernel<32, ROWIN>), g, b, 0, st, L, s, in, X);
  else
    hipLaunchKernelGGL((vl_orth_mem_kernel<ROWIN>), dim3(1), dim3(kVlOrthThreads), 0, st, L, s, in, X);
}

}  // namespace

size_t van_loan_workspace_bytes(int p, int q, int m, int n, int s) {
  const size_t M = (size_t)p * q, K = (size_t)m * n;
  return align256v(M * s * 4) + align256v(K * s * 4) + align256v((size_t)s * s * 4) + align256v((size_t)s * 4);
}

hipError_t launch_van_loan(const VanLoanArgs& A, void* ws, hipStream_t st) {
  const int M = A.p * A.q, K = A.m * A.n, s = A.s;
  unsigned char* w = static_cast<unsigned char*>(ws);
  float* Z = reinterpret_cast<float*>(w);                                   // s x M panel
  float* Q = reinterpret_cast<float*>(w + align256v((size_t)M * s * 4));   // s x K panel
  float* E = reinterpret_cast<float*>(w + align256v((size_t)M * s * 4) + align256v((size_t)K * s * 4));
  float* lam = E + align256v((size_t)s * s * 4) / 4;
  launch_rebase<true>(K, s, A.omega, Q, st);
  for (int it = 0; it < A.iters; ++it) {   // orthogonal iteration on R^T R
    launch_apply<0, kVlO0>(A, Q, Z, st);
    launch_apply<1, kVlO1>(A, Z, Q, st);
    launch_rebase<false>(K, s, Q, Q, st);
  }
  launch_apply<0, kVlO0>(A, Q, Z, st);
  launch_orth<false>(M, s, Z, Z, st);
  launch_apply<1, kVlO1>(A, Z, Q, st);   // Bt
  hipLaunchKernelGGL(vl_eig_kernel, dim3(1), dim3(kVlEigThreads), 0, st, K, s, Q, E, lam);
  hipLaunchKernelGGL(vl_assemble_kernel, dim3((unsigned)A.r), dim3(1024), (size_t)M * 4, st, M, K, s, Z, Q, E, lam,
                     A.C, A.B, A.sigma);
  return hipGetLastError();
}

}  // namespace kron
