// Matrix-core (MFMA) kernels of the Kronecker-factored layer for gfx950.
//
// Math (Kronecker layer tutorial, "The vec trick" / "The vec trick without the loop"):
// per row n, X = x_n viewed p x m, C_i = S o A_i,
//   forward   Z_i = X B_i (p x n),  Y = sum_i C_i^T Z_i (q x n),  y_n = vec_row(Y) + bias
//   backward  Z_i^T = B_i^T X^T,    dC_i += Z_i dY^T,  G_i^T = dY^T C_i^T,
//             dX^T += sum_i B_i G_i^T,                 dB_i += X^T G_i,  dbias += dY.
//
// Every product is a 16x16x4 fp32 MFMA (v_mfma_f32_16x16x4_f32).  Lane l = 16*g + c
// (g = l / 16, c = l % 16) supplies A[row c][k(g)] and B[k(g)][col c] and receives
// D[4*g + v][c] in accumulator register v.  Because the D tile has its row index in
// (g, v) -- the same place an operand keeps its contraction index -- the output of one
// product feeds the next product straight from registers when the next contraction runs
// over that row index:
//   forward: Z_i (rows j) is the A operand of Y^T = Z_i^T C_i (contraction over j), so Z
//            never leaves the registers of the wavefront that made it;
//   backward: Z_i^T (rows b) feeds dC_i (contraction over b), G_i^T (rows b) feeds dX^T
//            (contraction over b); dB_i contracts G_i over j, so G_i^T takes one trip
//            through a per-wavefront LDS tile to swap its indices.
// Contraction orders inside a K step are free as long as both operands agree; the
// kernels use a(s,g) = g*SA + s for the a index (so a lane's X values are contiguous in
// memory) and 4*s + g for the j and k indices read from LDS or memory.
//
// One wavefront processes one row at a time and all r ranks of it; workgroups are
// persistent and stride over rows.  The factor operands (B_i and C_i in the exact lane
// layouts the products need) are built once per workgroup in LDS.  Dimensions that are
// not multiples of 16 (4 for contraction steps) are padded with zeros inside the tiles.
// The backward keeps dC_i and dB_i accumulators in registers over all of a wavefront's
// rows, combines the four wavefronts of a workgroup in LDS in a fixed order and writes one
// partial sum per workgroup; the shared fixed-order column reduction finishes the sums.
#include "kron_internal.h"

namespace kron {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // four wavefronts
constexpr int kWaves = kThreads / 64;
constexpr int kBwdGroups = 256; // workgroups of the backward (fixed: the workspace depends on it)
constexpr size_t kMaxLds = 160 * 1024;

__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int L>
__device__ __forceinline__ void lds_load(float (&dst)[L], const float* src) {
  if constexpr (L % 4 == 0) {
#pragma unroll
    for (int t = 0; t < L / 4; ++t) {
      const f4 v = reinterpret_cast<const f4*>(src)[t];
      dst[4 * t] = v[0]; dst[4 * t + 1] = v[1]; dst[4 * t + 2] = v[2]; dst[4 * t + 3] = v[3];
    }
  } else if constexpr (L % 2 == 0) {
#pragma unroll
    for (int t = 0; t < L / 2; ++t) {
      const float2 v = reinterpret_cast<const float2*>(src)[t];
      dst[2 * t] = v.x; dst[2 * t + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int t = 0; t < L; ++t) dst[t] = src[t];
  }
}

template <int P_, int Q_, int M_, int N_, int R_>
struct Dims {
  static constexpr int P = P_, Q = Q_, M = M_, N = N_, R = R_;
  static constexpr int TJ = (P + 15) / 16;  // 16-tiles over j (p)
  static constexpr int TK = (Q + 15) / 16;  // over k (q)
  static constexpr int TA = (M + 15) / 16;  // over a (m)
  static constexpr int TB = (N + 15) / 16;  // over b (n)
  static constexpr int SA = (M + 3) / 4;    // K steps over a:  a = g*SA + s
  static constexpr int SK = (Q + 3) / 4;    // K steps over k:  k = 4*s + g
  static constexpr int SJ = TJ * 4;         // K steps over j:  j = 4*s + g (padded p)
  static constexpr int IN = P * M, OUT = Q * N;
  // LDS operand tables (floats)
  static constexpr int BOP = R * TB * 64 * SA;       // B_i[g*SA+s][16tb+c]
  static constexpr int COPF = R * TK * 64 * SJ;      // C_i[16tj+4g+v][16tk+c]
  static constexpr int COPG = R * TJ * 64 * SK;      // C_i[16tj+c][4s+g]
  static constexpr int BOPX = R * TA * 64 * TB * 4;  // B_i[16ta+c][16tb+4g+v]
  // per-wavefront G tile, row stride chosen so the four lane groups of a read hit
  // different LDS bank halves
  static constexpr int LDG = 16 * TB + ((TB % 2 == 0) ? 16 : 0);
  static constexpr int GS = 16 * TJ * LDG;
  static constexpr int PW = R * M * N + R * P * Q + Q * N;
  static constexpr size_t FWD_LDS = (size_t)(BOP + COPF) * 4;
  static constexpr size_t BWD_LDS_MAIN = (size_t)(BOP + COPG + BOPX + kWaves * GS) * 4;
  static constexpr size_t BWD_LDS = BWD_LDS_MAIN > (size_t)PW * 4 ? BWD_LDS_MAIN : (size_t)PW * 4;
  // registers held across a backward row (accumulators and per-row operands), in floats
  static constexpr int BWD_REGS = R * TJ * TK * 4 + R * TA * TB * 4 + TK * TB * 4 + TJ * SA + TA * SJ +
                                  TK * TB * 4 + TB * SK + TA * TJ * 4 + TB * TJ * 8;
  static_assert(M % 4 == 0 && N % 4 == 0, "rows are moved as 4-float vectors");
  static constexpr bool FWD_OK = FWD_LDS <= kMaxLds;
  static constexpr bool BWD_OK = BWD_LDS <= kMaxLds && BWD_REGS <= 400;
};

__device__ __forceinline__ float cval(const float* S, const float* A, int i, int j, int k, int P, int Q) {
  const float a = A[(i * P + j) * Q + k];
  return S ? S[j * Q + k] * a : a;
}

// Fill the B-operand table of the forward's first product (also the A operand of the
// backward's Z^T product): bop[i][tb][lane][s] = B_i[a = g*SA+s][b = 16tb+c].
template <class D>
__device__ void fill_bop(float* bop, const float* B) {
  for (int e = threadIdx.x; e < D::BOP; e += kThreads) {
    int t = e;
    const int s = t % D::SA; t /= D::SA;
    const int l = t % 64; t /= 64;
    const int tb = t % D::TB; const int i = t / D::TB;
    const int g = l >> 4, c = l & 15;
    const int a = g * D::SA + s, b = 16 * tb + c;
    bop[e] = (a < D::M && b < D::N) ? B[(i * D::M + a) * D::N + b] : 0.f;
  }
}

template <class D>
__global__ __launch_bounds__(kThreads) void fwd_mfma_kernel(int64_t N, uint32_t flags,
                                                            const float* __restrict__ x,
                                                            const float* __restrict__ Sm,
                                                            const float* __restrict__ A,
                                                            const float* __restrict__ B,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ y) {
  extern __shared__ float lds[];
  float* bop = lds;
  float* cop = bop + D::BOP;
  fill_bop<D>(bop, B);
  // cop[i][tk][lane][tj*4+v] = C_i[j = 16tj+4g+v][k = 16tk+c]
  for (int e = threadIdx.x; e < D::COPF; e += kThreads) {
    int t = e;
    const int sv = t % D::SJ; t /= D::SJ;
    const int l = t % 64; t /= 64;
    const int tk = t % D::TK; const int i = t / D::TK;
    const int g = l >> 4, c = l & 15;
    const int j = 16 * (sv / 4) + 4 * g + (sv % 4), k = 16 * tk + c;
    cop[e] = (j < D::P && k < D::Q) ? cval(Sm, A, i, j, k, D::P, D::Q) : 0.f;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int wave = threadIdx.x >> 6;
  f4 bb[D::TB][D::TK];
#pragma unroll
  for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk) {
      const int k = 16 * tk + c, b0 = 16 * tb + 4 * g;
      bb[tb][tk] = (bias && k < D::Q && b0 < D::N) ? *reinterpret_cast<const f4*>(bias + k * D::N + b0)
                                                  : f4{0.f, 0.f, 0.f, 0.f};
    }
  const bool relu = flags & KRON_RELU_OUT;

  for (int64_t row = (int64_t)blockIdx.x * kWaves + wave; row < N; row += (int64_t)gridDim.x * kWaves) {
    const float* xr = x + row * D::IN;
    float xa[D::TJ][D::SA];   // X[j = 16tj+c][a = g*SA+s]
#pragma unroll
    for (int tj = 0; tj < D::TJ; ++tj) {
      const int j = 16 * tj + c;
      if (j < D::P && g * D::SA < D::M) {
        lds_load<D::SA>(xa[tj], xr + j * D::M + g * D::SA);   // global load, same vector widths
#pragma unroll
        for (int s = 0; s < D::SA; ++s)
          if (g * D::SA + s >= D::M) xa[tj][s] = 0.f;
      } else {
#pragma unroll
        for (int s = 0; s < D::SA; ++s) xa[tj][s] = 0.f;
      }
    }
    f4 acc[D::TB][D::TK];
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int tk = 0; tk < D::TK; ++tk) acc[tb][tk] = f4{0.f, 0.f, 0.f, 0.f};

    // (ranks beyond four are not unrolled: the operand loads hoisted across an unrolled
    // rank loop would not fit the register file)
#pragma unroll(D::R <= 4 ? D::R : 2)
    for (int i = 0; i < D::R; ++i) {
      f4 z[D::TJ][D::TB];
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb) {
        float bo[D::SA];
        lds_load<D::SA>(bo, bop + ((i * D::TB + tb) * 64 + lane) * D::SA);
#pragma unroll
        for (int tj = 0; tj < D::TJ; ++tj) {
          f4 t = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < D::SA; ++s) t = mfma(xa[tj][s], bo[s], t);
          z[tj][tb] = t;   // Z[j = 16tj+4g+v][b = 16tb+c]
        }
      }
#pragma unroll
      for (int tk = 0; tk < D::TK; ++tk) {
        float co[D::SJ];
        lds_load<D::SJ>(co, cop + ((i * D::TK + tk) * 64 + lane) * D::SJ);
#pragma unroll
        for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
          for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[tb][tk] = mfma(z[tj][tb][v], co[tj * 4 + v], acc[tb][tk]);
      }
    }
    // acc[tb][tk] register v = Y^T[b = 16tb+4g+v][k = 16tk+c] -> y[k*N + b]
    float* yr = y + row * D::OUT;
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int tk = 0; tk < D::TK; ++tk) {
        const int k = 16 * tk + c, b0 = 16 * tb + 4 * g;
        if (k < D::Q && b0 < D::N) {
          f4 o = acc[tb][tk] + bb[tb][tk];
          if (relu) {
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v] = o[v] > 0.f ? o[v] : 0.f;
          }
          *reinterpret_cast<f4*>(yr + k * D::N + b0) = o;
        }
      }
  }
}

template <class D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_mfma_kernel(int64_t N, uint32_t flags, const float* __restrict__ x, const float* __restrict__ Sm,
                     const float* __restrict__ A, const float* __restrict__ B, const float* __restrict__ dy,
                     float* __restrict__ dx, float* __restrict__ part) {
  extern __shared__ float lds[];
  float* bop = lds;                 // B_i[g*SA+s][16tb+c]        (A operand of Z^T)
  float* copg = bop + D::BOP;       // C_i[16tj+c][4s+g]          (B operand of G^T)
  float* bopx = copg + D::COPG;     // B_i[16ta+c][16tb+4g+v]     (A operand of dX^T)
  float* gsall = bopx + D::BOPX;    // per-wavefront G tiles
  fill_bop<D>(bop, B);
  for (int e = threadIdx.x; e < D::COPG; e += kThreads) {
    int t = e;
    const int s = t % D::SK; t /= D::SK;
    const int l = t % 64; t /= 64;
    const int tj = t % D::TJ; const int i = t / D::TJ;
    const int g = l >> 4, c = l & 15;
    const int j = 16 * tj + c, k = 4 * s + g;
    copg[e] = (j < D::P && k < D::Q) ? cval(Sm, A, i, j, k, D::P, D::Q) : 0.f;
  }
  for (int e = threadIdx.x; e < D::BOPX; e += kThreads) {
    int t = e;
    const int sv = t % (D::TB * 4); t /= D::TB * 4;
    const int l = t % 64; t /= 64;
    const int ta = t % D::TA; const int i = t / D::TA;
    const int g = l >> 4, c = l & 15;
    const int a = 16 * ta + c, b = 16 * (sv / 4) + 4 * g + (sv % 4);
    bopx[e] = (a < D::M && b < D::N) ? B[(i * D::M + a) * D::N + b] : 0.f;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int wave = threadIdx.x >> 6;
  float* gs = gsall + wave * D::GS;
  const bool want_dx = dx != nullptr;
  const bool mask = flags & KRON_DX_RELU_MASK;

  f4 dC[D::R][D::TJ][D::TK];   // dC_i[j = 16tj+4g+v][k = 16tk+c]
  f4 dB[D::R][D::TA][D::TB];   // dB_i[a = 16ta+4g+v][b = 16tb+c]
  f4 db[D::TK][D::TB];         // dbias[k = 16tk+c][b = 16tb+4g+v]
#pragma unroll
  for (int i = 0; i < D::R; ++i) {
#pragma unroll
    for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
      for (int tk = 0; tk < D::TK; ++tk) dC[i][tj][tk] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb) dB[i][ta][tb] = f4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb) db[tk][tb] = f4{0.f, 0.f, 0.f, 0.f};

  for (int64_t row = (int64_t)blockIdx.x * kWaves + wave; row < N; row += (int64_t)gridDim.x * kWaves) {
    const float* xr = x + row * D::IN;
    const float* dyr = dy + row * D::OUT;
    float xa[D::TJ][D::SA];    // X[j = 16tj+c][a = g*SA+s]       B operand of Z^T
    float xaj[D::TA][D::SJ];   // X[j = 4s+g][a = 16ta+c]         A operand of dB
    f4 dyk[D::TK][D::TB];      // dY[k = 16tk+c][b = 16tb+4g+v]   B operand of dC
    float dyb[D::TB][D::SK];   // dY[k = 4s+g][b = 16tb+c]        A operand of G^T
#pragma unroll
    for (int tj = 0; tj < D::TJ; ++tj) {
      const int j = 16 * tj + c;
      if (j < D::P && g * D::SA < D::M) {
        lds_load<D::SA>(xa[tj], xr + j * D::M + g * D::SA);
#pragma unroll
        for (int s = 0; s < D::SA; ++s)
          if (g * D::SA + s >= D::M) xa[tj][s] = 0.f;
      } else {
#pragma unroll
        for (int s = 0; s < D::SA; ++s) xa[tj][s] = 0.f;
      }
    }
#pragma unroll
    for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
      for (int s = 0; s < D::SJ; ++s) {
        const int j = 4 * s + g, a = 16 * ta + c;
        xaj[ta][s] = (j < D::P && a < D::M) ? xr[j * D::M + a] : 0.f;
      }
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb) {
        const int k = 16 * tk + c, b0 = 16 * tb + 4 * g;
        dyk[tk][tb] = (k < D::Q && b0 < D::N) ? *reinterpret_cast<const f4*>(dyr + k * D::N + b0)
                                             : f4{0.f, 0.f, 0.f, 0.f};
        db[tk][tb] += dyk[tk][tb];
      }
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int s = 0; s < D::SK; ++s) {
        const int k = 4 * s + g, b = 16 * tb + c;
        dyb[tb][s] = (k < D::Q && b < D::N) ? dyr[k * D::N + b] : 0.f;
      }

    f4 dxt[D::TA][D::TJ];       // dX^T[a = 16ta+4g+v][j = 16tj+c]
#pragma unroll
    for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj) dxt[ta][tj] = f4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int i = 0; i < D::R; ++i) {
      // Z^T[b][j] = sum_a B_i[a][b] X[j][a]
      f4 zt[D::TB][D::TJ];
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb) {
        float bo[D::SA];
        lds_load<D::SA>(bo, bop + ((i * D::TB + tb) * 64 + lane) * D::SA);
#pragma unroll
        for (int tj = 0; tj < D::TJ; ++tj) {
          f4 t = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < D::SA; ++s) t = mfma(bo[s], xa[tj][s], t);
          zt[tb][tj] = t;
        }
      }
      // dC_i[j][k] += sum_b Z^T[b][j] dY[k][b]
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
        for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
          for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
            for (int v = 0; v < 4; ++v) dC[i][tj][tk] = mfma(zt[tb][tj][v], dyk[tk][tb][v], dC[i][tj][tk]);
      // G^T[b][j] = sum_k dY[k][b] C_i[j][k]
      f4 gt[D::TB][D::TJ];
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj) {
        float co[D::SK];
        lds_load<D::SK>(co, copg + ((i * D::TJ + tj) * 64 + lane) * D::SK);
#pragma unroll
        for (int tb = 0; tb < D::TB; ++tb) {
          f4 t = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < D::SK; ++s) t = mfma(dyb[tb][s], co[s], t);
          gt[tb][tj] = t;
        }
      }
      // dX^T[a][j] += sum_b B_i[a][b] G^T[b][j]
      if (want_dx) {
#pragma unroll
        for (int ta = 0; ta < D::TA; ++ta) {
          float bx[D::TB * 4];
          lds_load<D::TB * 4>(bx, bopx + ((i * D::TA + ta) * 64 + lane) * (D::TB * 4));
#pragma unroll
          for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
            for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
              for (int v = 0; v < 4; ++v) dxt[ta][tj] = mfma(bx[tb * 4 + v], gt[tb][tj][v], dxt[ta][tj]);
        }
      }
      // G^T -> LDS as G[j][b]; dB_i[a][b] += sum_j X[j][a] G[j][b]
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
        for (int tj = 0; tj < D::TJ; ++tj)
          *reinterpret_cast<f4*>(gs + (16 * tj + c) * D::LDG + 16 * tb + 4 * g) = gt[tb][tj];
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
        for (int s = 0; s < D::SJ; ++s) {
          const float gv = gs[(4 * s + g) * D::LDG + 16 * tb + c];
#pragma unroll
          for (int ta = 0; ta < D::TA; ++ta) dB[i][ta][tb] = mfma(xaj[ta][s], gv, dB[i][ta][tb]);
        }
      __builtin_amdgcn_wave_barrier();
    }
    if (want_dx) {
      float* dxr = dx + row * D::IN;
#pragma unroll
      for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
        for (int tj = 0; tj < D::TJ; ++tj) {
          const int j = 16 * tj + c, a0 = 16 * ta + 4 * g;
          if (j < D::P && a0 < D::M) {
            f4 o = dxt[ta][tj];
            if (mask) {
              const f4 xv = *reinterpret_cast<const f4*>(xr + j * D::M + a0);
#pragma unroll
              for (int v = 0; v < 4; ++v) o[v] = xv[v] > 0.f ? o[v] : 0.f;
            }
            *reinterpret_cast<f4*>(dxr + j * D::M + a0) = o;
          }
        }
    }
  }

  // Combine the wavefronts' partial sums in LDS in wave order, then write this
  // workgroup's partial row: [dB (R*M*N) | dC (R*P*Q) | dbias (Q*N)].
  __syncthreads();
  float* red = lds;
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int i = 0; i < D::R; ++i) {
#pragma unroll
        for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
          for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int a = 16 * ta + 4 * g + v, b = 16 * tb + c;
              if (a < D::M && b < D::N) {
                float* p = red + (i * D::M + a) * D::N + b;
                *p = (w == 0) ? dB[i][ta][tb][v] : *p + dB[i][ta][tb][v];
              }
            }
#pragma unroll
        for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
          for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int j = 16 * tj + 4 * g + v, k = 16 * tk + c;
              if (j < D::P && k < D::Q) {
                float* p = red + D::R * D::M * D::N + (i * D::P + j) * D::Q + k;
                *p = (w == 0) ? dC[i][tj][tk][v] : *p + dC[i][tj][tk][v];
              }
            }
      }
#pragma unroll
      for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
        for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int k = 16 * tk + c, b = 16 * tb + 4 * g + v;
            if (k < D::Q && b < D::N) {
              float* p = red + D::R * (D::M * D::N + D::P * D::Q) + k * D::N + b;
              *p = (w == 0) ? db[tk][tb][v] : *p + db[tk][tb][v];
            }
          }
    }
    __syncthreads();
  }
  float* out = part + (int64_t)blockIdx.x * D::PW;
  for (int e = threadIdx.x; e < D::PW; e += kThreads) out[e] = red[e];
}

// ---------------------------------------------------------------------------------
// Shape table.
// ---------------------------------------------------------------------------------
struct Entry {
  int p, q, m, n, r;
  bool fwd_ok, bwd_ok;
  size_t fwd_lds, bwd_lds;
  void (*fwd)(const LayerArgs&, int, hipStream_t);
  void (*bwd)(const LayerArgs&, int, hipStream_t);
};

template <class D>
void run_fwd(const LayerArgs& a, int grid, hipStream_t s) {
  if constexpr (D::FWD_OK) {
    (void)hipFuncSetAttribute((const void*)fwd_mfma_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)D::FWD_LDS);
    hipLaunchKernelGGL(fwd_mfma_kernel<D>, dim3(grid), dim3(kThreads), D::FWD_LDS, s, a.N, a.flags, a.x, a.S,
                       a.A, a.B, a.bias, a.y);
  }
}

template <class D>
void run_bwd(const LayerArgs& a, int grid, hipStream_t s) {
  if constexpr (D::BWD_OK) {
    (void)hipFuncSetAttribute((const void*)bwd_mfma_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)D::BWD_LDS);
    hipLaunchKernelGGL(bwd_mfma_kernel<D>, dim3(grid), dim3(kThreads), D::BWD_LDS, s, a.N, a.flags, a.x, a.S,
                       a.A, a.B, a.dy, a.dx, a.part);
  }
}

#define KRON_ENTRY(P, Q, M, N, R)                                                                      \
  Entry{P, Q, M, N, R, Dims<P, Q, M, N, R>::FWD_OK, Dims<P, Q, M, N, R>::BWD_OK,                        \
        Dims<P, Q, M, N, R>::FWD_LDS, Dims<P, Q, M, N, R>::BWD_LDS, &run_fwd<Dims<P, Q, M, N, R>>,       \
        &run_bwd<Dims<P, Q, M, N, R>>}

// The shapes of the workloads: the 64x64 tiny layer (m = 8), the 1024x1024 layers with
// m = 32 and m = 64, and the GPT-2 FFN pair 768 <-> 3072.
const Entry kTable[] = {
    KRON_ENTRY(8, 8, 8, 8, 1),      KRON_ENTRY(8, 8, 8, 8, 2),      KRON_ENTRY(32, 32, 32, 32, 1),
    KRON_ENTRY(32, 32, 32, 32, 2),  KRON_ENTRY(32, 32, 32, 32, 4),  KRON_ENTRY(16, 16, 64, 64, 1),
    KRON_ENTRY(16, 16, 64, 64, 2),  KRON_ENTRY(32, 64, 24, 48, 1),  KRON_ENTRY(32, 64, 24, 48, 2),
    KRON_ENTRY(32, 64, 24, 48, 4),  KRON_ENTRY(32, 64, 24, 48, 8),  KRON_ENTRY(64, 32, 48, 24, 1),
    KRON_ENTRY(64, 32, 48, 24, 2),  KRON_ENTRY(64, 32, 48, 24, 4),  KRON_ENTRY(64, 32, 48, 24, 8),
};

const Entry* find(int p, int q, int m, int n, int r) {
  for (const Entry& e : kTable)
    if (e.p == p && e.q == q && e.m == m && e.n == n && e.r == r) return &e;
  return nullptr;
}

}  // namespace

bool mfma_fwd_supported(int p, int q, int m, int n, int r) {
  const Entry* e = find(p, q, m, n, r);
  return e && e->fwd_ok;
}

bool mfma_bwd_supported(int p, int q, int m, int n, int r) {
  const Entry* e = find(p, q, m, n, r);
  return e && e->bwd_ok;
}

int mfma_bwd_groups(int64_t N) {
  const int64_t g = (N + kWaves - 1) / kWaves;
  return (int)(g < kBwdGroups ? g : kBwdGroups);
}

hipError_t launch_fwd_mfma(const LayerArgs& a, hipStream_t s) {
  const Entry* e = find(a.p, a.q, a.m, a.n, a.r);
  if (!e || !e->fwd_ok) return hipErrorInvalidValue;
  if (a.N == 0) return hipSuccess;
  // enough workgroups to fill every CU several times; each wavefront strides over rows
  int64_t grid = (a.N + kWaves - 1) / kWaves;
  const int64_t cap = 256 * 4;
  if (grid > cap) grid = cap;
  e->fwd(a, (int)grid, s);
  return hipGetLastError();
}

hipError_t launch_bwd_mfma(const LayerArgs& a, int G, hipStream_t s) {
  const Entry* e = find(a.p, a.q, a.m, a.n, a.r);
  if (!e || !e->bwd_ok) return hipErrorInvalidValue;
  if (G == 0) return hipSuccess;
  e->bwd(a, G, s);
  return hipGetLastError();
}

}  // namespace kron
