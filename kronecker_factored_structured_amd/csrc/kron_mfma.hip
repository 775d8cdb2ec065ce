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
// kernels pick them so that each lane's values are contiguous where they are read.
//
// One wavefront processes one row at a time and all r ranks of it; workgroups are
// persistent and stride over rows.  Each workgroup first stages B and S o A in LDS with
// coalesced vector loads and then lays out operand tables: for every product, the exact
// values each lane needs, chunk-interleaved ([chunk][lane][4 floats]) so that one
// ds_read_b128 per chunk is contiguous across the wavefront (no bank conflicts).
// Dimensions that are not multiples of 16 (4 for contraction steps) are padded with zeros
// inside the tiles.  The backward keeps dC_i and dB_i accumulators in registers over all
// of a wavefront's rows, combines the four wavefronts of a workgroup in LDS in a fixed
// order, turns dC into its shares of dA and dS, and writes one partial row per workgroup;
// the shared fixed-order column reduction finishes the sums.
#include <atomic>
#include <type_traits>

#include "kron_internal.h"

// The file is compiled twice: pass 1 holds the forward kernels (built with the
// instruction-level-parallelism scheduler, measured faster for them), pass 2 everything
// else.  KRON_MFMA_PASS 0 compiles the whole file at once.
#ifndef KRON_MFMA_PASS
#define KRON_MFMA_PASS 0
#endif

// The shapes with matrix-core kernels, (p, q, m, n, r, prefer the rank-parallel backward):
// the 64x64 tiny layer (m = 8), the 1024x1024 layers with m = 32 and m = 64, and the
// GPT-2 FFN pair 768 <-> 3072.
#define KRON_MFMA_SHAPES(X)                                                                             \
  X(8, 8, 8, 8, 1, true) X(8, 8, 8, 8, 2, true) X(32, 32, 32, 32, 1, true) X(32, 32, 32, 32, 2, true)   \
  X(32, 32, 32, 32, 4, true) X(16, 16, 64, 64, 1, false) X(16, 16, 64, 64, 2, false)                    \
  X(32, 64, 24, 48, 1, true) X(32, 64, 24, 48, 2, false) X(32, 64, 24, 48, 4, true)                     \
  X(32, 64, 24, 48, 8, true) X(64, 32, 48, 24, 1, false) X(64, 32, 48, 24, 2, true)                     \
  X(64, 32, 48, 24, 4, true) X(64, 32, 48, 24, 8, true)

namespace kron {

// The forward of one shape (defined with the forward kernels).
template <int P, int Q, int M, int N, int R>
void run_fwd_shape(const LayerArgs& a, int max_grid, hipStream_t s);

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;   // four wavefronts
constexpr int kWaves = kThreads / 64;
[[maybe_unused]] constexpr int kBwdGroups = 256; // backward workgroups per 256 CUs (fixed: the workspace depends on it)
constexpr size_t kMaxLds = 160 * 1024;

__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// L contiguous floats with the widest aligned vector loads.
template <int L>
__device__ __forceinline__ void vload(float (&dst)[L], const float* src) {
  if constexpr (L % 4 == 0) {
#pragma unroll
    for (int t = 0; t < L / 4; ++t) {
      const f4 v = reinterpret_cast<const f4*>(src)[t];
      dst[4 * t] = v[0]; dst[4 * t + 1] = v[1]; dst[4 * t + 2] = v[2]; dst[4 * t + 3] = v[3];
    }
  } else if constexpr (L % 2 == 0) {
#pragma unroll
    for (int t = 0; t < L / 2; ++t) {
      const f2 v = reinterpret_cast<const f2*>(src)[t];
      dst[2 * t] = v[0]; dst[2 * t + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int t = 0; t < L; ++t) dst[t] = src[t];
  }
}

// Operand tables: a lane's L values are stored as L/W chunks of W floats,
// [chunk][lane][W], so that a chunk read is contiguous across the wavefront.
template <int L>
constexpr int chunk_width() { return L % 4 == 0 ? 4 : (L % 2 == 0 ? 2 : 1); }

template <int L>
__device__ __forceinline__ void table_read(float (&dst)[L], const float* blk, int lane) {
  constexpr int W = chunk_width<L>();
#pragma unroll
  for (int t = 0; t < L / W; ++t) {
    if constexpr (W == 4) {
      const f4 v = reinterpret_cast<const f4*>(blk)[t * 64 + lane];
      dst[4 * t] = v[0]; dst[4 * t + 1] = v[1]; dst[4 * t + 2] = v[2]; dst[4 * t + 3] = v[3];
    } else if constexpr (W == 2) {
      const f2 v = reinterpret_cast<const f2*>(blk)[t * 64 + lane];
      dst[2 * t] = v[0]; dst[2 * t + 1] = v[1];
    } else {
      dst[t] = blk[t * 64 + lane];
    }
  }
}

// Lay out table[i][tile][chunk][lane][w] (i < R, tile < T, L values per lane) from
// val(i, tile, g, c, s) with s = chunk * W + w.
// (fully unrolled, so that a thread's reads of the source values are all in flight at once)
template <int R, int T, int L, class F>
__device__ __forceinline__ void build_table(float* tab, F val) {
  constexpr int W = chunk_width<L>();
  constexpr int total = R * T * 64 * L;
  constexpr int iters = (total + kThreads - 1) / kThreads;
#pragma unroll
  for (int it = 0; it < iters; ++it) {
    const int e = threadIdx.x + it * kThreads;
    if (total % kThreads != 0 && e >= total) break;
    int r = e;
    const int w = r % W; r /= W;
    const int l = r % 64; r /= 64;
    const int ch = r % (L / W); r /= (L / W);
    const int tile = r % T;
    const int i = r / T;
    tab[e] = val(i, tile, l >> 4, l & 15, ch * W + w);
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
  static constexpr int SJ = TJ * 4;         // K steps over j:  j = g*SJ + s (padded p)
  static constexpr int IN = P * M, OUT = Q * N;
  // operand tables (floats): per rank and tile, 64 lanes x L values
  static constexpr int BOP = R * TB * 64 * SA;       // B_i[g*SA+s][16tb+c]       L = SA
  static constexpr int COPF = R * TK * 64 * SJ;      // C_i[16tj+4g+v][16tk+c]    L = SJ (s = 4tj+v)
  static constexpr int COPG = R * TJ * 64 * SK;      // C_i[16tj+c][4s+g]         L = SK
  static constexpr int BOPX = R * TA * 64 * TB * 4;  // B_i[16ta+c][16tb+4g+v]    L = 4TB (s = 4tb+v)
  // raw staging of B (R*M*N) and C = S o A (R*P*Q)
  static constexpr int RAWB = R * M * N;
  static constexpr int RAWC = (R * P * Q + 3) / 4 * 4;
  static constexpr int RAW = RAWB + RAWC;
  // per-wavefront G^T -> G tile: gs[b][j], row stride LDGT = 16*TJ + 4 (conflict-free
  // b32 writes of a D tile and b128 reads of a lane's j run)
  static constexpr int LDGT = 16 * TJ + 4;
  static constexpr int GS = 16 * TB * LDGT;
  static constexpr int PW = R * M * N + R * P * Q + P * Q + Q * N;   // see partial_width()
  static constexpr int PWW = R * M * N + R * P * Q + Q * N;           // one wavefront's sums
  // the forward stages the raw factors next to its tables when they fit, else builds the
  // tables straight from global memory
  static constexpr bool FWD_RAW = (size_t)(BOP + COPF + RAW) * 4 <= kMaxLds;
  static constexpr int FWD_FLOATS = BOP + COPF + (FWD_RAW ? RAW : 0);
  static constexpr int BWD_TABLES = BOP + COPG + BOPX;
  static constexpr int BWD_SCRATCH = (kWaves * GS > RAW) ? kWaves * GS : RAW;
  static constexpr int BWD_MAIN = BWD_TABLES + BWD_SCRATCH;
  static constexpr size_t FWD_LDS = (size_t)FWD_FLOATS * 4;
  static constexpr size_t BWD_LDS = (size_t)(BWD_MAIN > kWaves * PWW ? BWD_MAIN : kWaves * PWW) * 4;
  // registers held across a backward row (accumulators and per-row operands), in floats
  static constexpr int ROW_REGS = TJ * SA + TA * SJ + TK * TB * 4 + TB * SK;
  static constexpr int BWD_REGS =
      R * TJ * TK * 4 + R * TA * TB * 4 + TK * TB * 4 + ROW_REGS + TA * TJ * 4 + TB * TJ * 8;
  static_assert(M % 4 == 0 && N % 4 == 0, "rows are moved as 4-float vectors");
  static constexpr bool FWD_OK = FWD_LDS <= kMaxLds;
  // thresholds measured against the compiler's allocation (no scratch below them)
  static constexpr bool BWD_OK = BWD_LDS <= kMaxLds && BWD_REGS <= 360;
  static constexpr bool BWD_PREFETCH = BWD_REGS + ROW_REGS <= 420;   // double-buffer the row operands
};

// Stage B (as is) and C = S o A in LDS with coalesced 16-byte loads.
template <class D>
__device__ __forceinline__ void stage_raw(float* rB, float* rC, const float* __restrict__ B,
                                          const float* __restrict__ S, const float* __restrict__ A) {
  constexpr int PQ = D::P * D::Q;
#pragma unroll 4
  for (int e = threadIdx.x; e < D::RAWB / 4; e += kThreads)
    reinterpret_cast<f4*>(rB)[e] = reinterpret_cast<const f4*>(B)[e];
  if constexpr (PQ % 4 == 0) {
#pragma unroll 4
    for (int e = threadIdx.x; e < D::R * PQ / 4; e += kThreads) {
      f4 a = reinterpret_cast<const f4*>(A)[e];
      if (S) a *= reinterpret_cast<const f4*>(S)[e % (PQ / 4)];
      reinterpret_cast<f4*>(rC)[e] = a;
    }
  } else {
    for (int e = threadIdx.x; e < D::R * PQ; e += kThreads) rC[e] = S ? S[e % PQ] * A[e] : A[e];
  }
}

template <class D>
__device__ __forceinline__ void stage_raw_b(float* rB, const float* __restrict__ B) {
#pragma unroll 4
  for (int e = threadIdx.x; e < D::RAWB / 4; e += kThreads)
    reinterpret_cast<f4*>(rB)[e] = reinterpret_cast<const f4*>(B)[e];
}
template <class D>
__device__ __forceinline__ void stage_raw_c(float* rC, const float* __restrict__ S, const float* __restrict__ A) {
  constexpr int PQ = D::P * D::Q;
  if constexpr (PQ % 4 == 0) {
#pragma unroll 4
    for (int e = threadIdx.x; e < D::R * PQ / 4; e += kThreads) {
      f4 a = reinterpret_cast<const f4*>(A)[e];
      if (S) a *= reinterpret_cast<const f4*>(S)[e % (PQ / 4)];
      reinterpret_cast<f4*>(rC)[e] = a;
    }
  } else {
    for (int e = threadIdx.x; e < D::R * PQ; e += kThreads) rC[e] = S ? S[e % PQ] * A[e] : A[e];
  }
}

template <class D>
__device__ __forceinline__ float rawB(const float* rB, int i, int a, int b) {
  return (a < D::M && b < D::N) ? rB[(i * D::M + a) * D::N + b] : 0.f;
}
template <class D>
__device__ __forceinline__ float rawC(const float* rC, int i, int j, int k) {
  return (j < D::P && k < D::Q) ? rC[(i * D::P + j) * D::Q + k] : 0.f;
}

// Wait, before the row loop, for the first row's prefetched operands.  The loop body
// issues the next row's loads before the current row's stores, so on the loop's back
// edge only stores are outstanding when the operands are consumed; without this wait the
// loop head would merge that state with the preheader's (loads outstanding) and wait for
// every store of the previous row.
template <class T, int A, int B>
__device__ __forceinline__ void settle(const T (&v)[A][B]) {
#pragma unroll
  for (int i = 0; i < A; ++i)
#pragma unroll
    for (int j = 0; j < B; ++j) asm volatile("" ::"v"(v[i][j]));
}

// X[j = 16tj+c][a = g*SA+s] of one row: SA contiguous floats per lane and tile.
template <class D>
__device__ __forceinline__ void load_xa(float (&xa)[D::TJ][D::SA], const float* xr, int g, int c) {
#pragma unroll
  for (int tj = 0; tj < D::TJ; ++tj) {
    const int j = 16 * tj + c;
    if (j < D::P) {
      vload<D::SA>(xa[tj], xr + j * D::M + g * D::SA);
    } else {
#pragma unroll
      for (int s = 0; s < D::SA; ++s) xa[tj][s] = 0.f;
    }
  }
}

#if KRON_MFMA_PASS != 2
template <class D>
__global__ __launch_bounds__(kThreads) void fwd_mfma_kernel(int64_t N, uint32_t flags,
                                                            const float* __restrict__ x,
                                                            const float* __restrict__ Sm,
                                                            const float* __restrict__ A,
                                                            const float* __restrict__ B,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ y) {
  extern __shared__ float lds[];
  float* bop = lds;              // B_i[g*SA+s][16tb+c]
  float* cop = bop + D::BOP;     // C_i[16tj+4g+v][16tk+c]
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int wave = threadIdx.x >> 6;
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  int64_t row = (int64_t)blockIdx.x * kWaves + wave;
  // the first row's X is loaded while the tables are built
  float xa[D::TJ][D::SA];   // X[j = 16tj+c][a = g*SA+s]
  if (row < N) load_xa<D>(xa, x + row * D::IN, g, c);
  if constexpr (D::FWD_RAW) {
    float* rB = cop + D::COPF;
    float* rC = rB + D::RAWB;
    stage_raw<D>(rB, rC, B, Sm, A);
    __syncthreads();
    build_table<D::R, D::TB, D::SA>(bop, [&](int i, int tb, int g, int c, int s) {
      return rawB<D>(rB, i, g * D::SA + s, 16 * tb + c);
    });
    build_table<D::R, D::TK, D::SJ>(cop, [&](int i, int tk, int g, int c, int sv) {
      return rawC<D>(rC, i, 16 * (sv / 4) + 4 * g + (sv % 4), 16 * tk + c);
    });
  } else {
    build_table<D::R, D::TB, D::SA>(bop, [&](int i, int tb, int g, int c, int s) {
      const int a = g * D::SA + s, b = 16 * tb + c;
      return (a < D::M && b < D::N) ? B[(i * D::M + a) * D::N + b] : 0.f;
    });
    build_table<D::R, D::TK, D::SJ>(cop, [&](int i, int tk, int g, int c, int sv) {
      const int j = 16 * (sv / 4) + 4 * g + (sv % 4), k = 16 * tk + c;
      if (j >= D::P || k >= D::Q) return 0.f;
      const float a = A[(i * D::P + j) * D::Q + k];
      return Sm ? Sm[j * D::Q + k] * a : a;
    });
  }
  __syncthreads();

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

  // The next row's X is loaded at the top of each row (the last row reloads itself), and
  // a scheduling barrier keeps the compiler from sinking those loads towards their use.
  float xn[D::TJ][D::SA];
  settle(xa);
  for (; row < N; row += stride) {
    {
      const int64_t nr = row + stride < N ? row + stride : row;
      load_xa<D>(xn, x + nr * D::IN, g, c);
    }
    __builtin_amdgcn_sched_barrier(0);
    f4 acc[D::TB][D::TK];
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int tk = 0; tk < D::TK; ++tk) acc[tb][tk] = f4{0.f, 0.f, 0.f, 0.f};

    // (ranks beyond four are not unrolled: the operand reads hoisted across an unrolled
    // rank loop would not fit the register file)
#pragma unroll(D::R <= 4 ? D::R : 2)
    for (int i = 0; i < D::R; ++i) {
      f4 z[D::TJ][D::TB];
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb) {
        float bo[D::SA];
        table_read<D::SA>(bo, bop + (i * D::TB + tb) * 64 * D::SA, lane);
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
        table_read<D::SJ>(co, cop + (i * D::TK + tk) * 64 * D::SJ, lane);
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
#pragma unroll
    for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
      for (int s = 0; s < D::SA; ++s) xa[tj][s] = xn[tj][s];
  }
}

#endif  // forward kernels

#if KRON_MFMA_PASS != 1
// The backward's per-row operands.
template <class D>
struct BwdRow {
  float xa[D::TJ][D::SA];    // X[j = 16tj+c][a = g*SA+s]       B operand of Z^T
  float xaj[D::TA][D::SJ];   // X[j = g*SJ+s][a = 16ta+c]       A operand of dB
  f4 dyk[D::TK][D::TB];      // dY[k = 16tk+c][b = 16tb+4g+v]   B operand of dC
  float dyb[D::TB][D::SK];   // dY[k = 4s+g][b = 16tb+c]        A operand of G^T
};

template <class D>
__device__ __forceinline__ void load_bwd_row(BwdRow<D>& o, const float* xr, const float* dyr, int g, int c) {
  load_xa<D>(o.xa, xr, g, c);
#pragma unroll
  for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
    for (int s = 0; s < D::SJ; ++s) {
      const int j = g * D::SJ + s, a = 16 * ta + c;
      o.xaj[ta][s] = (j < D::P && a < D::M) ? xr[j * D::M + a] : 0.f;
    }
#pragma unroll
  for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb) {
      const int k = 16 * tk + c, b0 = 16 * tb + 4 * g;
      o.dyk[tk][tb] = (k < D::Q && b0 < D::N) ? *reinterpret_cast<const f4*>(dyr + k * D::N + b0)
                                             : f4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
  for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
    for (int s = 0; s < D::SK; ++s) {
      const int k = 4 * s + g, b = 16 * tb + c;
      o.dyb[tb][s] = (k < D::Q && b < D::N) ? dyr[k * D::N + b] : 0.f;
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
  float* scratch = bopx + D::BOPX;  // raw factors while the tables are built, then G tiles
  float* rB = scratch;
  float* rC = rB + D::RAWB;
  BwdRow<D> nx;   // the next row's operands, loaded while the current row computes; the
                  // first row's loads are issued before the tables are built
  if constexpr (D::BWD_PREFETCH) {
    const int64_t row0 = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row0 < N) load_bwd_row<D>(nx, x + row0 * D::IN, dy + row0 * D::OUT, (threadIdx.x & 63) >> 4, threadIdx.x & 15);
  }
  stage_raw<D>(rB, rC, B, Sm, A);
  __syncthreads();
  build_table<D::R, D::TB, D::SA>(bop, [&](int i, int tb, int g, int c, int s) {
    return rawB<D>(rB, i, g * D::SA + s, 16 * tb + c);
  });
  build_table<D::R, D::TJ, D::SK>(copg, [&](int i, int tj, int g, int c, int s) {
    return rawC<D>(rC, i, 16 * tj + c, 4 * s + g);
  });
  build_table<D::R, D::TA, D::TB * 4>(bopx, [&](int i, int ta, int g, int c, int sv) {
    return rawB<D>(rB, i, 16 * ta + c, 16 * (sv / 4) + 4 * g + (sv % 4));
  });
  __syncthreads();

  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int wave = threadIdx.x >> 6;
  float* gs = scratch + wave * D::GS;   // G[j][b] stored as gs[b * LDGT + j]
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

  const int64_t stride = (int64_t)gridDim.x * kWaves;
  int64_t row = (int64_t)blockIdx.x * kWaves + wave;
  if constexpr (D::BWD_PREFETCH) {
    settle(nx.xa);
    settle(nx.xaj);
    settle(nx.dyk);
    settle(nx.dyb);
  }
  for (; row < N; row += stride) {
    const float* xr = x + row * D::IN;
    BwdRow<D> cur;
    if constexpr (D::BWD_PREFETCH) {
      cur = nx;
      if (row + stride < N) load_bwd_row<D>(nx, x + (row + stride) * D::IN, dy + (row + stride) * D::OUT, g, c);
    } else {
      load_bwd_row<D>(cur, xr, dy + row * D::OUT, g, c);
    }
    const auto& xa = cur.xa;
    const auto& xaj = cur.xaj;
    const auto& dyk = cur.dyk;
    const auto& dyb = cur.dyb;
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb) db[tk][tb] += dyk[tk][tb];

    f4 dxt[D::TA][D::TJ];       // dX^T[a = 16ta+4g+v][j = 16tj+c]
#pragma unroll
    for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj) dxt[ta][tj] = f4{0.f, 0.f, 0.f, 0.f};

    // Operand tables are read one product (or one rank) ahead of their use, so that the
    // LDS latency hides behind the matrix products in flight.
    float bo_next[D::TB][D::SA];
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb) table_read<D::SA>(bo_next[tb], bop + tb * 64 * D::SA, lane);
#pragma unroll
    for (int i = 0; i < D::R; ++i) {
      float bo[D::TB][D::SA];
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
        for (int s = 0; s < D::SA; ++s) bo[tb][s] = bo_next[tb][s];
      float co[D::TJ][D::SK];
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj) table_read<D::SK>(co[tj], copg + (i * D::TJ + tj) * 64 * D::SK, lane);
      float bx[D::TA][D::TB * 4];
      if (want_dx) {
#pragma unroll
        for (int ta = 0; ta < D::TA; ++ta)
          table_read<D::TB * 4>(bx[ta], bopx + (i * D::TA + ta) * 64 * D::TB * 4, lane);
      }
      // Z^T[b][j] = sum_a B_i[a][b] X[j][a]
      f4 zt[D::TB][D::TJ];
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
        for (int tj = 0; tj < D::TJ; ++tj) {
          f4 t = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < D::SA; ++s) t = mfma(bo[tb][s], xa[tj][s], t);
          zt[tb][tj] = t;
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
      for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
        for (int tb = 0; tb < D::TB; ++tb) {
          f4 t = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < D::SK; ++s) t = mfma(dyb[tb][s], co[tj][s], t);
          gt[tb][tj] = t;
        }
      // G^T -> LDS (gs[b][j]) first, so that the dX^T products below cover the round trip
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
        for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
          for (int v = 0; v < 4; ++v) gs[(16 * tb + 4 * g + v) * D::LDGT + 16 * tj + c] = gt[tb][tj][v];
      __builtin_amdgcn_wave_barrier();
      // dX^T[a][j] += sum_b B_i[a][b] G^T[b][j]
      if (want_dx) {
#pragma unroll
        for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
          for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
            for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
              for (int v = 0; v < 4; ++v) dxt[ta][tj] = mfma(bx[ta][tb * 4 + v], gt[tb][tj][v], dxt[ta][tj]);
      }
      if (i + 1 < D::R) {
#pragma unroll
        for (int tb = 0; tb < D::TB; ++tb)
          table_read<D::SA>(bo_next[tb], bop + ((i + 1) * D::TB + tb) * 64 * D::SA, lane);
      }
      // dB_i[a][b] += sum_j X[j][a] G[j][b] with j = g*SJ + s
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb) {
        float gv[D::SJ];
        vload<D::SJ>(gv, gs + (16 * tb + c) * D::LDGT + g * D::SJ);
#pragma unroll
        for (int s = 0; s < D::SJ; ++s)
#pragma unroll
          for (int ta = 0; ta < D::TA; ++ta) dB[i][ta][tb] = mfma(xaj[ta][s], gv[s], dB[i][ta][tb]);
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

  // Every wavefront stores its partial sums in its own LDS block at once, then the
  // workgroup adds the blocks in wave order and writes its partial row
  //   [dB (R*M*N) | dA (R*P*Q) | dS (P*Q) | dbias (Q*N)]
  // turning dC into its shares of dA_i = S o dC_i and dS = sum_i A_i o dC_i on the way.
  __syncthreads();
  constexpr int MN = D::M * D::N, PQ = D::P * D::Q, QN = D::Q * D::N;
  float* red = lds + wave * D::PWW;   // [dB | dC | dbias] of this wavefront
#pragma unroll
  for (int i = 0; i < D::R; ++i) {
#pragma unroll
    for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int a = 16 * ta + 4 * g + v, b = 16 * tb + c;
          if (a < D::M && b < D::N) red[i * MN + a * D::N + b] = dB[i][ta][tb][v];
        }
#pragma unroll
    for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
      for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int j = 16 * tj + 4 * g + v, k = 16 * tk + c;
          if (j < D::P && k < D::Q) red[D::R * MN + i * PQ + j * D::Q + k] = dC[i][tj][tk][v];
        }
  }
#pragma unroll
  for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int k = 16 * tk + c, b = 16 * tb + 4 * g + v;
        if (k < D::Q && b < D::N) red[D::R * (MN + PQ) + k * D::N + b] = db[tk][tb][v];
      }
  __syncthreads();
  const PartRow out{part, (int64_t)gridDim.x, (int64_t)blockIdx.x, 0};
  auto wsum = [&](int e) {
    float t = lds[e];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += lds[w * D::PWW + e];
    return t;
  };
  for (int e = threadIdx.x; e < D::R * MN; e += kThreads) out[e] = wsum(e);
  for (int e = threadIdx.x; e < PQ; e += kThreads) {
    const float sv = Sm ? Sm[e] : 1.f;
    float ds = 0.f;
#pragma unroll
    for (int i = 0; i < D::R; ++i) {
      const float dcv = wsum(D::R * MN + i * PQ + e);
      ds = fmaf(A[i * PQ + e], dcv, ds);
      out[D::R * MN + i * PQ + e] = sv * dcv;
    }
    out[D::R * (MN + PQ) + e] = Sm ? ds : 0.f;
  }
  for (int e = threadIdx.x; e < QN; e += kThreads) out[D::R * (MN + PQ) + PQ + e] = wsum(D::R * (MN + PQ) + e);
}

// ---------------------------------------------------------------------------------
// Rank-parallel backward.  A workgroup of four wavefronts owns RPI = 4 / R rows at a
// time; wavefront w computes rank w % R of row slot w / R.  The rows' X and dY are staged
// once per step in LDS with padded strides, every wavefront reads its operands from there
// and keeps only its own rank's dC_i and dB_i in registers, so two workgroups (two
// wavefronts per SIMD) fit on a compute unit.  dX^T partials of the R ranks of a row
// meet in LDS and are added in rank order.  K-step orders: a = g*SA + s for X B_i,
// j, k = 16*(s/4) + 4*g + s%4 for the j and k contractions (the D-tile row order), so
// that every LDS read and write of the step is free of bank conflicts.
// ---------------------------------------------------------------------------------
template <class D>
struct RP {
  static constexpr int R = D::R;
  static constexpr int RPI = 4 / R;                 // rows per step
  static constexpr int LX = 16 * D::TA + 4;         // X row stride (a padded to 16*TA)
  static constexpr int XR = 16 * D::TJ;             // X rows (j padded)
  static constexpr int LY = 16 * D::TB + 4;         // dY row stride
  static constexpr int YR = 16 * D::TK;             // dY rows (k padded)
  static constexpr int SLOT = XR * LX + YR * LY;    // one row's X and dY
  static constexpr int ROWBUF = RPI * SLOT;
  static constexpr int SKP = 4 * D::TK;             // k steps (padded)
  static constexpr int COPG = R * D::TJ * 64 * SKP; // C_i[16tj+c][kappa(s,g)]
  static constexpr int TABLES = D::BOP + COPG + D::BOPX;
  static constexpr int LDGT = 16 * D::TJ + 4;       // G tile gs[b][j]
  static constexpr int GS = 16 * D::TB * LDGT;
  static constexpr int LDXP = 16 * D::TA + 4;       // dX partial dxp[j][a]
  static constexpr int DXP = 16 * D::TJ * LDXP;
  static constexpr int WREG = GS > DXP ? GS : DXP;  // per wavefront: G tile, then dX partial
  static constexpr int RAWMAX = D::RAWB > D::RAWC ? D::RAWB : D::RAWC;
  static constexpr int WORK = (ROWBUF + 4 * WREG) > RAWMAX ? (ROWBUF + 4 * WREG) : RAWMAX;
  static constexpr int MAIN = TABLES + WORK;
  static constexpr int COMBINE = RPI * D::PWW;
  static constexpr size_t LDS = (size_t)(MAIN > COMBINE ? MAIN : COMBINE) * 4;
  static constexpr int NF4 = ROWBUF / SLOT * (D::IN + D::OUT) / 4;   // float4s staged per step
  static constexpr int NPF = (NF4 + kThreads - 1) / kThreads;
  // workgroups per compute unit: two when their LDS fits twice (two wavefronts per SIMD),
  // else one (one wavefront per SIMD, with the whole register file)
  static constexpr int WPC = LDS * 2 <= kMaxLds ? 2 : 1;
  static constexpr bool OK = (R == 1 || R == 2 || R == 4) && LDS <= kMaxLds && D::IN % 4 == 0 &&
                             D::OUT % 4 == 0;
};

__device__ __forceinline__ int kidx(int s, int g) { return 16 * (s >> 2) + 4 * g + (s & 3); }

// DXM: 0 = no dX, 1 = dX, 2 = dX masked by [x > 0], 3 = dX added to dx, 4 = dX added to
// dx and the sum masked by [x > 0] (modes 3 and 4 serve rank chunks after the first).  With the mode fixed at compile time
// and the one partial row group peeled off the loop, every step issues the same stores,
// so the wait for the next step's prefetched rows does not also wait for them.
template <class D, int DXM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(RP<D>::WPC, RP<D>::WPC)))
void bwd_rp_kernel(int64_t N, uint32_t flags, const float* __restrict__ x, const float* __restrict__ Sm,
                   const float* __restrict__ A, const float* __restrict__ B, const float* __restrict__ dy,
                   float* __restrict__ dx, float* __restrict__ part) {
  using Q = RP<D>;
  extern __shared__ float lds[];
  float* bop = lds;                      // B_i[g*SA+s][16tb+c]
  float* copg = bop + D::BOP;            // C_i[16tj+c][kappa(s,g)]
  float* bopx = copg + Q::COPG;          // B_i[16ta+c][16tb+4g+v]
  float* work = bopx + D::BOPX;
  float* rowbuf = work;                  // RPI slots of [X (XR x LX) | dY (YR x LY)]
  float* wreg = work + Q::ROWBUF;        // per wavefront: G tile / dX partial

  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wave = tid >> 6;
  const int slot = wave / Q::R, rank = wave % Q::R;
  const int64_t ngrp = (N + Q::RPI - 1) / Q::RPI;

  // prefetch of the first step's rows (registers), issued before the tables are built
  f4 pf[Q::NPF];
  auto fetch = [&](int64_t grp) {
#pragma unroll
    for (int t = 0; t < Q::NPF; ++t) {
      const int f = tid + t * kThreads;
      f4 v = f4{0.f, 0.f, 0.f, 0.f};
      if (f < Q::NF4) {
        const int s = f / ((D::IN + D::OUT) / 4), o = 4 * (f % ((D::IN + D::OUT) / 4));
        const int64_t row = grp * Q::RPI + s;
        if (grp < ngrp && row < N)
          v = o < D::IN ? *reinterpret_cast<const f4*>(x + row * D::IN + o)
                        : *reinterpret_cast<const f4*>(dy + row * D::OUT + (o - D::IN));
      }
      pf[t] = v;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int t = 0; t < Q::NPF; ++t) {
      const int f = tid + t * kThreads;
      if (f < Q::NF4) {
        const int s = f / ((D::IN + D::OUT) / 4), o = 4 * (f % ((D::IN + D::OUT) / 4));
        float* sb = rowbuf + s * Q::SLOT;
        float* dst = o < D::IN ? sb + (o / D::M) * Q::LX + o % D::M
                               : sb + Q::XR * Q::LX + ((o - D::IN) / D::N) * Q::LY + (o - D::IN) % D::N;
        *reinterpret_cast<f4*>(dst) = pf[t];
      }
    }
  };
  fetch(blockIdx.x);

  // operand tables, B first and then C through the same staging area
  stage_raw_b<D>(work, B);
  __syncthreads();
  build_table<D::R, D::TB, D::SA>(bop, [&](int i, int tb, int gg, int cc, int s) {
    return rawB<D>(work, i, gg * D::SA + s, 16 * tb + cc);
  });
  build_table<D::R, D::TA, D::TB * 4>(bopx, [&](int i, int ta, int gg, int cc, int sv) {
    return rawB<D>(work, i, 16 * ta + cc, 16 * (sv / 4) + 4 * gg + (sv % 4));
  });
  __syncthreads();
  stage_raw_c<D>(work, Sm, A);
  __syncthreads();
  build_table<D::R, D::TJ, Q::SKP>(copg, [&](int i, int tj, int gg, int cc, int s) {
    return rawC<D>(work, i, 16 * tj + cc, kidx(s, gg));
  });
  __syncthreads();
  for (int e = tid; e < Q::ROWBUF; e += kThreads) rowbuf[e] = 0.f;   // padding stays zero
  __syncthreads();

  const float* bop_i = bop + rank * D::TB * 64 * D::SA;
  const float* copg_i = copg + rank * D::TJ * 64 * Q::SKP;
  const float* bopx_i = bopx + rank * D::TA * 64 * D::TB * 4;
  float* gs = wreg + wave * Q::WREG;      // G[j][b] as gs[b * LDGT + j]; later dX^T partial [j][a]
  const float* Xs = rowbuf + slot * Q::SLOT;
  const float* Ys = Xs + Q::XR * Q::LX;
  (void)flags;

  f4 dC[D::TJ][D::TK];    // dC_rank[j = 16tj+4g+v][k = 16tk+c]
  f4 dB[D::TA][D::TB];    // dB_rank[a = 16ta+4g+v][b = 16tb+c]
  f4 db[D::TK][D::TB];    // dbias[k = 16tk+c][b = 16tb+4g+v] (rank 0 only)
#pragma unroll
  for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk) dC[tj][tk] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb) dB[ta][tb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb) db[tk][tb] = f4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int64_t grp, auto tail_c) {
    constexpr bool kTail = decltype(tail_c)::value;
    stash();
    __syncthreads();
    fetch(grp + gridDim.x);
    // Z^T[b][j] = sum_a B_i[a][b] X[j][a]
    f4 zt[D::TB][D::TJ];
    {
      float xa[D::TJ][D::SA];
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj) vload<D::SA>(xa[tj], Xs + (16 * tj + c) * Q::LX + g * D::SA);
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb) {
        float bo[D::SA];
        table_read<D::SA>(bo, bop_i + tb * 64 * D::SA, lane);
#pragma unroll
        for (int tj = 0; tj < D::TJ; ++tj) {
          f4 t = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < D::SA; ++s) t = mfma(bo[s], xa[tj][s], t);
          zt[tb][tj] = t;
        }
      }
    }
    // dC[j][k] += sum_b Z^T[b][j] dY[k][b]
    {
      f4 dyk[D::TK][D::TB];
#pragma unroll
      for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
        for (int tb = 0; tb < D::TB; ++tb)
          dyk[tk][tb] = *reinterpret_cast<const f4*>(Ys + (16 * tk + c) * Q::LY + 16 * tb + 4 * g);
      if (rank == 0) {
#pragma unroll
        for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
          for (int tb = 0; tb < D::TB; ++tb) db[tk][tb] += dyk[tk][tb];
      }
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
        for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
          for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
            for (int v = 0; v < 4; ++v) dC[tj][tk] = mfma(zt[tb][tj][v], dyk[tk][tb][v], dC[tj][tk]);
    }
    // G^T[b][j] = sum_k dY[k][b] C_i[j][k], k = kappa(s, g)
    f4 gt[D::TB][D::TJ];
    {
      float dyb[D::TB][Q::SKP];
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
        for (int s = 0; s < Q::SKP; ++s) dyb[tb][s] = Ys[kidx(s, g) * Q::LY + 16 * tb + c];
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj) {
        float co[Q::SKP];
        table_read<Q::SKP>(co, copg_i + tj * 64 * Q::SKP, lane);
#pragma unroll
        for (int tb = 0; tb < D::TB; ++tb) {
          f4 t = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < Q::SKP; ++s) t = mfma(dyb[tb][s], co[s], t);
          gt[tb][tj] = t;
        }
      }
    }
    // G^T -> LDS as gs[b][j]
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
        for (int v = 0; v < 4; ++v) gs[(16 * tb + 4 * g + v) * Q::LDGT + 16 * tj + c] = gt[tb][tj][v];
    __builtin_amdgcn_wave_barrier();
    // dX^T[a][j] = sum_b B_i[a][b] G^T[b][j]   (this rank's share)
    f4 dxt[D::TA][D::TJ];
#pragma unroll
    for (int ta = 0; ta < D::TA; ++ta) {
      float bx[D::TB * 4];
      table_read<D::TB * 4>(bx, bopx_i + ta * 64 * D::TB * 4, lane);
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj) {
        f4 t = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
          for (int v = 0; v < 4; ++v) t = mfma(bx[tb * 4 + v], gt[tb][tj][v], t);
        dxt[ta][tj] = t;
      }
    }
    // dB[a][b] += sum_j X[j][a] G[j][b], j = kappa(s, g)
#pragma unroll
    for (int ta = 0; ta < D::TA; ++ta) {
      float xaj[D::SJ];
#pragma unroll
      for (int s = 0; s < D::SJ; ++s) xaj[s] = Xs[kidx(s, g) * Q::LX + 16 * ta + c];
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb) {
        float gv[D::SJ];
#pragma unroll
        for (int tj = 0; tj < D::TJ; ++tj) {
          const f4 q4 = *reinterpret_cast<const f4*>(gs + (16 * tb + c) * Q::LDGT + 16 * tj + 4 * g);
          gv[4 * tj] = q4[0]; gv[4 * tj + 1] = q4[1]; gv[4 * tj + 2] = q4[2]; gv[4 * tj + 3] = q4[3];
        }
#pragma unroll
        for (int s = 0; s < D::SJ; ++s) dB[ta][tb] = mfma(xaj[s], gv[s], dB[ta][tb]);
      }
    }
    __builtin_amdgcn_wave_barrier();
    // this rank's dX^T partial -> LDS as dxp[j][a]
#pragma unroll
    for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj)
        *reinterpret_cast<f4*>(gs + (16 * tj + c) * Q::LDXP + 16 * ta + 4 * g) = dxt[ta][tj];
    __syncthreads();
    // dX of the step's rows: add the R rank partials of each row in rank order (the mask
    // reads x from the row's LDS copy)
    if constexpr (DXM != 0) {
      constexpr int PER_ROW = D::IN / 4;
      constexpr int TOT = Q::RPI * PER_ROW;
#pragma unroll
      for (int t = 0; t < (TOT + kThreads - 1) / kThreads; ++t) {
        const int f = tid + t * kThreads;
        if (TOT % kThreads != 0 && f >= TOT) continue;
        const int s = f / PER_ROW, o = 4 * (f % PER_ROW);
        const int64_t row = grp * Q::RPI + s;
        if (kTail && row >= N) continue;
        const int j = o / D::M, a = o % D::M;
        f4 acc = *reinterpret_cast<const f4*>(wreg + (s * Q::R) * Q::WREG + j * Q::LDXP + a);
#pragma unroll
        for (int i = 1; i < Q::R; ++i)
          acc += *reinterpret_cast<const f4*>(wreg + (s * Q::R + i) * Q::WREG + j * Q::LDXP + a);
        if constexpr (DXM >= 3) acc += *reinterpret_cast<const f4*>(dx + row * D::IN + o);
        if constexpr (DXM == 2 || DXM == 4) {
          const f4 xv = *reinterpret_cast<const f4*>(rowbuf + s * Q::SLOT + j * Q::LX + a);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[v] = xv[v] > 0.f ? acc[v] : 0.f;
        }
        *reinterpret_cast<f4*>(dx + row * D::IN + o) = acc;
      }
    }
  };
  // groups whose rows are all valid, then the one partial group (if N % RPI != 0)
  const int64_t nfull = N / Q::RPI;
  int64_t grp = blockIdx.x;
  for (; grp < nfull; grp += gridDim.x) step(grp, std::false_type{});
  if (grp < ngrp) step(grp, std::true_type{});

  // Partial row of this workgroup: [dB (R*M*N) | dA (R*P*Q) | dS (P*Q) | dbias (Q*N)].
  __syncthreads();
  constexpr int MN = D::M * D::N, PQ = D::P * D::Q, QN = D::Q * D::N;
  float* red = lds + slot * D::PWW;   // [dB | dC | dbias] of this row slot
#pragma unroll
  for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int a = 16 * ta + 4 * g + v, b = 16 * tb + c;
        if (a < D::M && b < D::N) red[rank * MN + a * D::N + b] = dB[ta][tb][v];
      }
#pragma unroll
  for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 16 * tj + 4 * g + v, k = 16 * tk + c;
        if (j < D::P && k < D::Q) red[D::R * MN + rank * PQ + j * D::Q + k] = dC[tj][tk][v];
      }
  if (rank == 0) {
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int k = 16 * tk + c, b = 16 * tb + 4 * g + v;
          if (k < D::Q && b < D::N) red[D::R * (MN + PQ) + k * D::N + b] = db[tk][tb][v];
        }
  }
  __syncthreads();
  const PartRow out{part, (int64_t)gridDim.x, (int64_t)blockIdx.x, 0};
  auto ssum = [&](int e) {
    float t = lds[e];
#pragma unroll
    for (int s = 1; s < Q::RPI; ++s) t += lds[s * D::PWW + e];
    return t;
  };
  for (int e = tid; e < D::R * MN; e += kThreads) out[e] = ssum(e);
  for (int e = tid; e < PQ; e += kThreads) {
    const float sv = Sm ? Sm[e] : 1.f;
    float ds = 0.f;
#pragma unroll
    for (int i = 0; i < D::R; ++i) {
      const float dcv = ssum(D::R * MN + i * PQ + e);
      ds = fmaf(A[i * PQ + e], dcv, ds);
      out[D::R * MN + i * PQ + e] = sv * dcv;
    }
    out[D::R * (MN + PQ) + e] = Sm ? ds : 0.f;
  }
  for (int e = tid; e < QN; e += kThreads) out[D::R * (MN + PQ) + PQ + e] = ssum(D::R * (MN + PQ) + e);
}

#endif  // backward kernels

// ---------------------------------------------------------------------------------
// Shape table.
// ---------------------------------------------------------------------------------
struct Entry {
  int p, q, m, n, r;
  bool fwd_ok, bwd_ok, bwd_rp;
  int rows_per_step;   // of the rank-parallel backward
  int rp_per_cu;       // its workgroups per compute unit
  void (*fwd)(const LayerArgs&, int, hipStream_t);
  void (*bwd)(const LayerArgs&, int, hipStream_t);
};

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

#if KRON_MFMA_PASS != 2
// The forward is persistent: as many workgroups as fit on the device at once (and no
// more than one row per wavefront), each wavefront striding over rows.
template <class D>
void run_fwd(const LayerArgs& a, int max_grid, hipStream_t s) {
  if constexpr (D::FWD_OK) {
    static const int per_cu = [] {
      (void)hipFuncSetAttribute((const void*)fwd_mfma_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)D::FWD_LDS);
      int nb = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fwd_mfma_kernel<D>, kThreads, D::FWD_LDS) !=
              hipSuccess || nb < 1)
        nb = 1;
      return nb;
    }();
    int64_t grid = (int64_t)per_cu * device_cus();
    if (grid > max_grid) grid = max_grid;
    hipLaunchKernelGGL(fwd_mfma_kernel<D>, dim3((unsigned)grid), dim3(kThreads), D::FWD_LDS, s, a.N, a.flags,
                       a.x, a.S, a.A, a.B, a.bias, a.y);
  }
}

#endif

#if KRON_MFMA_PASS != 1
// RPF: prefer the rank-parallel kernel when both backward kernels fit (measured per shape).
template <class D, bool RPF>
void run_bwd(const LayerArgs& a, int grid, hipStream_t s) {
  constexpr bool use_rp = RP<D>::OK && (RPF || !D::BWD_OK);
  if constexpr (use_rp) {
    static const bool attr = [] {
      (void)hipFuncSetAttribute((const void*)bwd_rp_kernel<D, 0>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)RP<D>::LDS);
      (void)hipFuncSetAttribute((const void*)bwd_rp_kernel<D, 1>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)RP<D>::LDS);
      (void)hipFuncSetAttribute((const void*)bwd_rp_kernel<D, 2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)RP<D>::LDS);
      (void)hipFuncSetAttribute((const void*)bwd_rp_kernel<D, 3>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)RP<D>::LDS);
      (void)hipFuncSetAttribute((const void*)bwd_rp_kernel<D, 4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)RP<D>::LDS);
      return true;
    }();
    (void)attr;
    const bool mask = a.flags & KRON_DX_RELU_MASK;
    const int dxm = a.dx == nullptr ? 0 : (a.dx_accumulate ? (mask ? 4 : 3) : (mask ? 2 : 1));
#define KRON_RP_LAUNCH(M)                                                                                \
  hipLaunchKernelGGL((bwd_rp_kernel<D, M>), dim3(grid), dim3(kThreads), RP<D>::LDS, s, a.N, a.flags, a.x, \
                     a.S, a.A, a.B, a.dy, a.dx, a.part)
    switch (dxm) {
      case 0: KRON_RP_LAUNCH(0); break;
      case 1: KRON_RP_LAUNCH(1); break;
      case 2: KRON_RP_LAUNCH(2); break;
      case 3: KRON_RP_LAUNCH(3); break;
      default: KRON_RP_LAUNCH(4); break;
    }
#undef KRON_RP_LAUNCH
  } else if constexpr (D::BWD_OK) {
    static const bool attr = [] {
      (void)hipFuncSetAttribute((const void*)bwd_mfma_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)D::BWD_LDS);
      return true;
    }();
    (void)attr;
    hipLaunchKernelGGL(bwd_mfma_kernel<D>, dim3(grid), dim3(kThreads), D::BWD_LDS, s, a.N, a.flags, a.x, a.S,
                       a.A, a.B, a.dy, a.dx, a.part);
  }
}

#define KRON_ENTRY(P, Q, M, N, R, RPF)                                                                 \
  Entry{P, Q, M, N, R, Dims<P, Q, M, N, R>::FWD_OK,                                                    \
        Dims<P, Q, M, N, R>::BWD_OK || RP<Dims<P, Q, M, N, R>>::OK,                                     \
        RP<Dims<P, Q, M, N, R>>::OK && (RPF || !Dims<P, Q, M, N, R>::BWD_OK),                           \
        RP<Dims<P, Q, M, N, R>>::RPI, RP<Dims<P, Q, M, N, R>>::WPC, &run_fwd_shape<P, Q, M, N, R>,       \
        &run_bwd<Dims<P, Q, M, N, R>, RPF>},

const Entry kTable[] = {KRON_MFMA_SHAPES(KRON_ENTRY)};

const Entry* find(int p, int q, int m, int n, int r) {
  for (const Entry& e : kTable)
    if (e.p == p && e.q == q && e.m == m && e.n == n && e.r == r) return &e;
  return nullptr;
}
#endif  // KRON_MFMA_PASS != 1

}  // namespace

#if KRON_MFMA_PASS != 2
template <int P, int Q, int M, int N, int R>
void run_fwd_shape(const LayerArgs& a, int max_grid, hipStream_t s) {
  run_fwd<Dims<P, Q, M, N, R>>(a, max_grid, s);
}
#define KRON_FWD_INST(P, Q, M, N, R, RPF) template void run_fwd_shape<P, Q, M, N, R>(const LayerArgs&, int, hipStream_t);
KRON_MFMA_SHAPES(KRON_FWD_INST)
#undef KRON_FWD_INST
#endif

#if KRON_MFMA_PASS != 1

bool mfma_fwd_supported(int p, int q, int m, int n, int r) {
  const Entry* e = find(p, q, m, n, r);
  return e && e->fwd_ok;
}

bool mfma_bwd_supported(int p, int q, int m, int n, int r) {
  const Entry* e = find(p, q, m, n, r);
  return e && e->bwd_ok;
}

int mfma_bwd_chunk(int p, int q, int m, int n, int r) {
  if (r <= 4 || r % 4 != 0 || mfma_bwd_supported(p, q, m, n, r)) return 0;
  const Entry* e = find(p, q, m, n, 4);
  return (e && e->bwd_rp) ? 4 : 0;
}

int mfma_bwd_groups(int64_t N, int p, int q, int m, int n, int r) {
  const Entry* e = find(p, q, m, n, r);
  if (e && e->bwd_rp) {
    // rp_per_cu workgroups per compute unit, each stepping over rows_per_step rows at a time
    const int64_t g = (N + e->rows_per_step - 1) / e->rows_per_step;
    const int64_t gmax = (int64_t)e->rp_per_cu * kBwdGroups;
    return (int)(g < gmax ? g : gmax);
  }
  const int64_t g = (N + kWaves - 1) / kWaves;
  return (int)(g < kBwdGroups ? g : kBwdGroups);
}

hipError_t launch_fwd_mfma(const LayerArgs& a, hipStream_t s) {
  const Entry* e = find(a.p, a.q, a.m, a.n, a.r);
  if (!e || !e->fwd_ok) return hipErrorInvalidValue;
  if (a.N == 0) return hipSuccess;
  int64_t grid = (a.N + kWaves - 1) / kWaves;
  if (grid > (1 << 20)) grid = 1 << 20;
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
#endif  // KRON_MFMA_PASS != 1

}  // namespace kron
