// bf16 Kronecker-factored layer on bf16 matrix instructions (mixed precision: bf16
// operands, fp32 accumulation).  Same products as the fp32 kernels (Kronecker layer
// tutorial, "The vec trick" and "The vec trick without the loop"; the backward by
// calculus from them); every product is v_mfma_f32_16x16x16_bf16:
//   lane l = 16*g + c supplies A[c][4g..4g+3] and B[4g..4g+3][c] (four consecutive K
//   values, 8 bytes) and receives D[4g+v][c], v = 0..3.
// A D tile therefore holds, per lane, four consecutive values of its row index -- exactly
// the four K values the lane supplies when the next product contracts over that index --
// so an fp32 accumulator tile, rounded to bf16 (round-to-nearest-even), is the operand of
// the next product without leaving the registers (Z into Y^T = Z^T C in the forward; Z^T
// into dC and G^T into dX^T in the backward).
//
// Storage: x, S, A, B, bias, dy, y and dx are bf16 (bit patterns); dS, dA, dB and dbias
// are fp32.  C_i = S o A_i is formed in fp32 (exact for bf16 factors) and rounded to
// bf16; X B_i and G_i are rounded to bf16 before they enter their second product.
// Dimensions p, q, m, n must be multiples of 16.
#include <type_traits>

#include "kron_internal.h"

namespace kron {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ f4 mfma16(s4 a, s4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float bf2f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
// fp32 -> bf16 by the hardware conversion (v_cvt_pk_bf16_f32, two values per instruction),
// round to nearest even under the default rounding mode
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), b2));
}
__device__ __forceinline__ s4 pack4(f4 v) {
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(s4, (u2{pack2(v[0], v[1]), pack2(v[2], v[3])}));
}
__device__ __forceinline__ s4 load_s4(const uint16_t* p) { return *reinterpret_cast<const s4*>(p); }
__device__ __forceinline__ s4 gather4(const uint16_t* p, int stride) {
  return s4{(short)p[0], (short)p[stride], (short)p[2 * stride], (short)p[3 * stride]};
}

template <int P_, int Q_, int M_, int N_, int R_>
struct BD {
  static constexpr int P = P_, Q = Q_, M = M_, N = N_, R = R_;
  static constexpr int TJ = P / 16, TK = Q / 16, TA = M / 16, TB = N / 16;
  static constexpr int IN = P * M, OUT = Q * N;
  static constexpr int MN = M * N, PQ = P * Q;
  static constexpr int PW = R * MN + R * PQ + PQ + Q * N;   // partial row (partial_width())
  static constexpr int PWW = R * MN + R * PQ + Q * N;       // one row slot's sums
  static constexpr bool SHAPE_OK = P % 16 == 0 && Q % 16 == 0 && M % 16 == 0 && N % 16 == 0;
};

// ---------------------------------------------------------------------------------
// Operands of 16 x 16 x (4W) products.  W = 4: v_mfma_f32_16x16x16_bf16; W = 8:
// v_mfma_f32_16x16x32_bf16 (lane l = 16g + c supplies A[c][8g..8g+7] and B[8g..8g+7][c]).
// A contraction does not depend on the order of its K values as long as both operands use
// the same order, so each product fixes, per lane group g and element u, which K index the
// element carries:
//   k_row: W consecutive K values (an operand read from a row in memory),
//   k_acc: four consecutive K values from each of W/4 accumulator tiles 16 apart (an
//          operand assembled from D tiles of the previous product: a D tile gives lane
//          group g the rows 4g..4g+3 of its 16).
// The factor operand of the same product (a register table) is built in the matching order.
// ---------------------------------------------------------------------------------
typedef short s8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

template <int W>
struct OpT;
template <>
struct OpT<4> {
  typedef s4 T;
};
template <>
struct OpT<8> {
  typedef s8 T;
};
__device__ __forceinline__ f4 mfma(s4 a, s4 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0); }
__device__ __forceinline__ f4 mfma(s8 a, s8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
}
template <int W>
__device__ __forceinline__ int k_row(int s, int g, int u) { return 4 * W * s + W * g + u; }
template <int W>
__device__ __forceinline__ int k_acc(int s, int g, int u) { return 4 * W * s + 16 * (u / 4) + 4 * g + (u % 4); }
// operand of chunk s from accumulator tiles packed to bf16: tiles W/4*s .. W/4*s + W/4 - 1
__device__ __forceinline__ s4 join(s4 a) { return a; }
__device__ __forceinline__ s8 join(s4 a, s4 b) { return s8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }

// ---------------------------------------------------------------------------------
// Forward.  Persistent; one row per wavefront at a time.  Per rank i:
//   Z_i   = X B_i      (TJ x TB tiles, KC1 products each)   A = X[j][k_row], B = B_i[k_row][b]
//   Y^T  += Z_i^T C_i  (TB x TK tiles, KC2 products each)   A = bf16(Z tiles), B = C_i[k_acc][k]
// B_i and C_i = S o A_i (rounded to bf16) are staged once per workgroup in LDS in lane
// order (each lane's operand is one contiguous 8- or 16-byte piece) and then held in
// registers; the bias values of the lane's outputs are held in registers too, so that the
// only global loads in the row loop are the next row's x.
// ---------------------------------------------------------------------------------
template <class D>
struct FB {
  static constexpr int W1 = D::M % 32 == 0 ? 8 : 4, KC1 = D::M / (4 * W1);   // Z = X B_i over a
  static constexpr int W2 = D::P % 32 == 0 ? 8 : 4, KC2 = D::P / (4 * W2);   // Y^T over j
  static constexpr int TAB_B = D::R * D::TB * KC1 * 64;   // lane entries of W1 values
  static constexpr int TAB_C = D::R * D::TK * KC2 * 64;   // lane entries of W2 values
  // registers per lane: factor tables, x (current and next row), accumulators, Z tiles, bias
  static constexpr int REGS = D::R * D::TB * KC1 * W1 / 2 + D::R * D::TK * KC2 * W2 / 2 + D::TJ * KC1 * W1 +
                              D::TB * D::TK * 6 + D::TJ * D::TB * 2 + 16;
  static constexpr int NT = REGS <= 128 ? 1024 : 512;
  static constexpr int NW = NT / 64;
};

template <class D>
__global__ __launch_bounds__((FB<D>::NT)) void fwd_bf16_kernel(int64_t N, uint32_t flags,
                                                               const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ Sm,
                                                               const uint16_t* __restrict__ A,
                                                               const uint16_t* __restrict__ B,
                                                               const uint16_t* __restrict__ bias,
                                                               uint16_t* __restrict__ y) {
  using F = FB<D>;
  constexpr int W1 = F::W1, KC1 = F::KC1, W2 = F::W2, KC2 = F::KC2;
  typedef typename OpT<W1>::T O1;
  typedef typename OpT<W2>::T O2;
  __shared__ __attribute__((aligned(16))) uint16_t tabB[F::TAB_B * W1];
  __shared__ __attribute__((aligned(16))) uint16_t tabC[F::TAB_C * W2];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15, wave = tid >> 6;
  const int64_t stride = (int64_t)gridDim.x * F::NW;
  int64_t row = (int64_t)blockIdx.x * F::NW + wave;

  // X operands of a row: X[j = 16tj + c][k_row(s, g, 0 .. W1-1)], one contiguous piece each
  O1 xn[D::TJ][KC1];
  auto load_x = [&](O1 (&dst)[D::TJ][KC1], int64_t r) {
    const uint16_t* xr = x + r * D::IN;
#pragma unroll
    for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
      for (int s = 0; s < KC1; ++s)
        dst[tj][s] = *reinterpret_cast<const O1*>(xr + (16 * tj + c) * D::M + k_row<W1>(s, g, 0));
  };
  if (row < N) load_x(xn, row);

  for (int e = tid; e < F::TAB_B; e += F::NT) {   // e = ((i*TB + tb)*KC1 + s)*64 + lane
    const int ln = e & 63, rest = e >> 6, s = rest % KC1, tb = (rest / KC1) % D::TB, i = rest / (KC1 * D::TB);
    const uint16_t* Bi = B + i * D::MN + 16 * tb + (ln & 15);
    O1 v;
#pragma unroll
    for (int u = 0; u < W1; ++u) v[u] = (short)Bi[k_row<W1>(s, ln >> 4, u) * D::N];
    *reinterpret_cast<O1*>(tabB + e * W1) = v;
  }
  for (int e = tid; e < F::TAB_C; e += F::NT) {   // e = ((i*TK + tk)*KC2 + s)*64 + lane
    const int ln = e & 63, rest = e >> 6, s = rest % KC2, tk = (rest / KC2) % D::TK, i = rest / (KC2 * D::TK);
    const int k = 16 * tk + (ln & 15);
    O2 v;
#pragma unroll
    for (int u = 0; u < W2; ++u) {
      const int jk = k_acc<W2>(s, ln >> 4, u) * D::Q + k;
      const float av = bf2f(A[i * D::PQ + jk]);
      v[u] = (short)f2bf(Sm ? bf2f(Sm[jk]) * av : av);
    }
    *reinterpret_cast<O2*>(tabC + e * W2) = v;
  }
  // bias of the lane's outputs: Y^T[b = 16tb + 4g + v][k = 16tk + c] -> bias[k*N + b]
  s4 bv[D::TB][D::TK];
#pragma unroll
  for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk)
      bv[tb][tk] = bias ? load_s4(bias + (16 * tk + c) * D::N + 16 * tb + 4 * g) : s4{0, 0, 0, 0};
  __syncthreads();
  O1 bop[D::R][D::TB][KC1];
  O2 cop[D::R][D::TK][KC2];
#pragma unroll
  for (int i = 0; i < D::R; ++i) {
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int s = 0; s < KC1; ++s)
        bop[i][tb][s] = *reinterpret_cast<const O1*>(tabB + (((i * D::TB + tb) * KC1 + s) * 64 + lane) * W1);
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
      for (int s = 0; s < KC2; ++s)
        cop[i][tk][s] = *reinterpret_cast<const O2*>(tabC + (((i * D::TK + tk) * KC2 + s) * 64 + lane) * W2);
  }
  const bool relu = flags & KRON_RELU_OUT;

  for (; row < N; row += stride) {
    O1 xa[D::TJ][KC1];
#pragma unroll
    for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
      for (int s = 0; s < KC1; ++s) xa[tj][s] = xn[tj][s];
    load_x(xn, row + stride < N ? row + stride : row);   // the next row (the last row reloads itself)
    __builtin_amdgcn_sched_barrier(0);
    f4 acc[D::TB][D::TK];
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[tb][tk][v] = bf2f((uint16_t)bv[tb][tk][v]);
#pragma unroll
    for (int i = 0; i < D::R; ++i) {
      s4 zb[D::TJ][D::TB];   // bf16(Z_i)[j = 16tj + 4g + v][b = 16tb + c]
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
        for (int tb = 0; tb < D::TB; ++tb) {
          f4 z = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KC1; ++s) z = mfma(xa[tj][s], bop[i][tb][s], z);
          zb[tj][tb] = pack4(z);
        }
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
        for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
          for (int s = 0; s < KC2; ++s) {
            O2 zo;
            if constexpr (W2 == 8)
              zo = join(zb[2 * s][tb], zb[2 * s + 1][tb]);
            else
              zo = join(zb[s][tb]);
            acc[tb][tk] = mfma(zo, cop[i][tk][s], acc[tb][tk]);
          }
    }
    // acc[tb][tk] register v = Y^T[b = 16tb + 4g + v][k = 16tk + c] -> y[k*N + b]
    uint16_t* yr = y + row * D::OUT;
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int tk = 0; tk < D::TK; ++tk) {
        f4 o = acc[tb][tk];
        if (relu) {
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] = o[v] > 0.f ? o[v] : 0.f;
        }
        *reinterpret_cast<s4*>(yr + (16 * tk + c) * D::N + 16 * tb + 4 * g) = pack4(o);
      }
  }
}

// ---------------------------------------------------------------------------------
// Backward, rank-parallel: a workgroup of four wavefronts owns RPI = 4 / R rows per step,
// wavefront w computes rank w % R of row slot w / R.  The rows are staged in LDS in both
// index orders (X[j][a], X^T[a][j], dY[k][b], dY^T[b][k]) so that every operand is one
// 8-byte read.  Per rank and row:
//   Z^T[b][j]  = sum_a B_i[a][b] X[j][a]        A = B_i^T[b][a..] (registers), B = X[j][a..]
//   dC[j][k]  += sum_b Z^T[b][j] dY[k][b]       A = bf16(Z^T tile),             B = dY[k][b..]
//   G^T[b][j]  = sum_k dY[k][b] C_i[j][k]       A = dY^T[b][k..],               B = C_i[j][k..] (registers)
//   dX^T[a][j] = sum_b B_i[a][b] G^T[b][j]      A = B_i[a][b..] (registers),    B = bf16(G^T tile)
//   dB[a][b]  += sum_j X[j][a] G[j][b]          A = X^T[a][j..],                B = G (G^T tile through LDS)
// dX^T partials of the R ranks of a row meet in LDS and are added in rank order; the
// partial row [dB | dA | dS | dbias] and the fixed-order column reduction are those of the
// fp32 layer.
// ---------------------------------------------------------------------------------
template <class D>
struct RB {
  static constexpr int R = D::R;
  static constexpr int RPI = 4 / R;
  // row strides (bf16 elements), padded by 8 so that rows stay 16-byte aligned and the
  // sixteen rows of a lane group start on different banks
  static constexpr int LXA = D::M + 8;   // X[j][a]
  static constexpr int LXJ = D::P + 8;   // X^T[a][j]
  static constexpr int LYB = D::N + 8;   // dY[k][b]
  static constexpr int LYK = D::Q + 8;   // dY^T[b][k]
  static constexpr int OX = 0, OXT = D::P * LXA, OY = OXT + D::M * LXJ, OYT = OY + D::Q * LYB;
  static constexpr int SLOT = OYT + D::N * LYK;   // bf16 elements per row slot
  static constexpr int ROWBUF = RPI * SLOT;
  static constexpr int LG = D::P + 8;             // G^T tile gs[b][j] (bf16)
  static constexpr int LDX = D::M + 4;            // dX^T partial dxp[j][a] (fp32)
  static constexpr int WREG_BYTES = (D::N * LG * 2 > D::P * LDX * 4 ? D::N * LG * 2 : D::P * LDX * 4);
  static constexpr int WREG = (WREG_BYTES + 15) / 16 * 16;   // bytes per wavefront
  static constexpr size_t MAIN = (size_t)ROWBUF * 2 + (size_t)kWaves * WREG;
  static constexpr size_t COMBINE = (size_t)RPI * D::PWW * 4;
  static constexpr size_t LDS = (MAIN > COMBINE ? MAIN : COMBINE);
  static constexpr int CHUNKS = (D::IN + D::OUT) / 8;   // 16-byte pieces of one row's x and dy
  static constexpr int NPF = (RPI * CHUNKS + kThreads - 1) / kThreads;
  static constexpr bool OK = D::SHAPE_OK && (R == 1 || R == 2 || R == 4) && LDS <= 80 * 1024;
};

template <class D, int DXM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_bf16_kernel(int64_t N, const uint16_t* __restrict__ x, const uint16_t* __restrict__ Sm,
                     const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                     const uint16_t* __restrict__ dy, uint16_t* __restrict__ dx, float* __restrict__ part) {
  using Q = RB<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* rowbuf = reinterpret_cast<uint16_t*>(smem);
  unsigned char* wbase = smem + (size_t)Q::ROWBUF * 2;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15, wave = tid >> 6;
  const int slot = wave / Q::R, rank = wave % Q::R;
  const int64_t ngrp = (N + Q::RPI - 1) / Q::RPI;

  // prefetch: 16-byte pieces of the step's rows (x then dy of each row slot)
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  u4 pf[Q::NPF];
  auto fetch = [&](int64_t grp) {
#pragma unroll
    for (int t = 0; t < Q::NPF; ++t) {
      const int f = tid + t * kThreads;
      u4 v = u4{0u, 0u, 0u, 0u};
      if (f < Q::RPI * Q::CHUNKS) {
        const int s = f / Q::CHUNKS, o = 8 * (f % Q::CHUNKS);
        const int64_t row = grp * Q::RPI + s;
        if (grp < ngrp && row < N)
          v = o < D::IN ? *reinterpret_cast<const u4*>(x + row * D::IN + o)
                        : *reinterpret_cast<const u4*>(dy + row * D::OUT + (o - D::IN));
      }
      pf[t] = v;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int t = 0; t < Q::NPF; ++t) {
      const int f = tid + t * kThreads;
      if (f < Q::RPI * Q::CHUNKS) {
        const int s = f / Q::CHUNKS, o = 8 * (f % Q::CHUNKS);
        uint16_t* sb = rowbuf + s * Q::SLOT;
        const u4 v = pf[t];
        const uint16_t e[8] = {(uint16_t)(v[0] & 0xffffu), (uint16_t)(v[0] >> 16), (uint16_t)(v[1] & 0xffffu),
                               (uint16_t)(v[1] >> 16), (uint16_t)(v[2] & 0xffffu), (uint16_t)(v[2] >> 16),
                               (uint16_t)(v[3] & 0xffffu), (uint16_t)(v[3] >> 16)};
        if (o < D::IN) {   // X[j][a .. a+7] and X^T[a .. a+7][j]
          const int j = o / D::M, a = o % D::M;
          *reinterpret_cast<u4*>(sb + Q::OX + j * Q::LXA + a) = v;
#pragma unroll
          for (int u = 0; u < 8; ++u) sb[Q::OXT + (a + u) * Q::LXJ + j] = e[u];
        } else {           // dY[k][b .. b+7] and dY^T[b .. b+7][k]
          const int o2 = o - D::IN, k = o2 / D::N, b = o2 % D::N;
          *reinterpret_cast<u4*>(sb + Q::OY + k * Q::LYB + b) = v;
#pragma unroll
          for (int u = 0; u < 8; ++u) sb[Q::OYT + (b + u) * Q::LYK + k] = e[u];
        }
      }
    }
  };
  fetch(blockIdx.x);

  // this wavefront's rank operands (bf16), straight from global memory
  const uint16_t* Bi = B + rank * D::MN;
  const uint16_t* Ai = A + rank * D::PQ;
  s4 bt[D::TB][D::TA];   // B_i^T[b = 16tb + c][a = 16t + 4g ..]   (A operand of Z^T)
  s4 ct[D::TJ][D::TK];   // C_i[j = 16tj + c][k = 16t + 4g ..]     (B operand of G^T)
  s4 bx[D::TA][D::TB];   // B_i[a = 16ta + c][b = 16t + 4g ..]     (A operand of dX^T)
#pragma unroll
  for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
    for (int t = 0; t < D::TA; ++t) bt[tb][t] = gather4(Bi + (16 * t + 4 * g) * D::N + 16 * tb + c, D::N);
#pragma unroll
  for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
    for (int t = 0; t < D::TK; ++t) {
      const int j = 16 * tj + c, k0 = 16 * t + 4 * g;
      s4 v;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float a = bf2f(Ai[j * D::Q + k0 + u]);
        v[u] = (short)f2bf(Sm ? bf2f(Sm[j * D::Q + k0 + u]) * a : a);
      }
      ct[tj][t] = v;
    }
#pragma unroll
  for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
    for (int t = 0; t < D::TB; ++t) bx[ta][t] = load_s4(Bi + (16 * ta + c) * D::N + 16 * t + 4 * g);

  for (int e = tid; e < Q::ROWBUF; e += kThreads) rowbuf[e] = 0;   // padding stays zero
  __syncthreads();

  const uint16_t* Xs = rowbuf + slot * Q::SLOT;
  uint16_t* gs = reinterpret_cast<uint16_t*>(wbase + wave * Q::WREG);   // G^T tile [b][j] (bf16)
  float* dxp = reinterpret_cast<float*>(wbase + wave * Q::WREG);        // then the dX^T partial [j][a]

  f4 dC[D::TJ][D::TK];   // dC_rank[j = 16tj + 4g + v][k = 16tk + c]
  f4 dB[D::TA][D::TB];   // dB_rank[a = 16ta + 4g + v][b = 16tb + c]
  f4 db[D::TK][D::TB];   // dbias[k = 16tk + c][b = 16tb + 4g + v]   (rank 0)
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
    const uint16_t* X = Xs + Q::OX;
    const uint16_t* XT = Xs + Q::OXT;
    const uint16_t* Y = Xs + Q::OY;
    const uint16_t* YT = Xs + Q::OYT;
    // Z^T[b][j]
    f4 zt[D::TB][D::TJ];
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj) {
        f4 t4 = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < D::TA; ++t) t4 = mfma16(bt[tb][t], load_s4(X + (16 * tj + c) * Q::LXA + 16 * t + 4 * g), t4);
        zt[tb][tj] = t4;
      }
    // dC[j][k] += sum_b Z^T[b][j] dY[k][b];  dbias += dY (rank 0)
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb) {
        const s4 yk = load_s4(Y + (16 * tk + c) * Q::LYB + 16 * tb + 4 * g);   // dY[k = 16tk + c][b = 16tb + 4g ..]
        if (rank == 0) {
#pragma unroll
          for (int v = 0; v < 4; ++v) db[tk][tb][v] += bf2f((uint16_t)yk[v]);
        }
#pragma unroll
        for (int tj = 0; tj < D::TJ; ++tj) dC[tj][tk] = mfma16(pack4(zt[tb][tj]), yk, dC[tj][tk]);
      }
    // G^T[b][j]
    f4 gt[D::TB][D::TJ];
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj) {
        f4 t4 = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < D::TK; ++t) t4 = mfma16(load_s4(YT + (16 * tb + c) * Q::LYK + 16 * t + 4 * g), ct[tj][t], t4);
        gt[tb][tj] = t4;
      }
    // G^T tile -> LDS as gs[b][j] (bf16)
    s4 gb[D::TB][D::TJ];
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj) {
        gb[tb][tj] = pack4(gt[tb][tj]);
#pragma unroll
        for (int v = 0; v < 4; ++v) gs[(16 * tb + 4 * g + v) * Q::LG + 16 * tj + c] = (uint16_t)gb[tb][tj][v];
      }
    __builtin_amdgcn_wave_barrier();
    // dX^T[a][j] = sum_b B_i[a][b] G^T[b][j]
    f4 dxt[D::TA][D::TJ];
#pragma unroll
    for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj) {
        f4 t4 = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tb = 0; tb < D::TB; ++tb) t4 = mfma16(bx[ta][tb], gb[tb][tj], t4);
        dxt[ta][tj] = t4;
      }
    // dB[a][b] += sum_j X^T[a][j] G[j][b]
#pragma unroll
    for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
        for (int t = 0; t < D::TJ; ++t)
          dB[ta][tb] = mfma16(load_s4(XT + (16 * ta + c) * Q::LXJ + 16 * t + 4 * g),
                              load_s4(gs + (16 * tb + c) * Q::LG + 16 * t + 4 * g), dB[ta][tb]);
    __builtin_amdgcn_wave_barrier();
    // this rank's dX^T partial -> LDS as dxp[j][a] (fp32)
#pragma unroll
    for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj)
        *reinterpret_cast<f4*>(dxp + (16 * tj + c) * Q::LDX + 16 * ta + 4 * g) = dxt[ta][tj];
    __syncthreads();
    // dX of the step's rows: the R rank partials added in rank order, rounded to bf16
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
        const float* w0 = reinterpret_cast<const float*>(wbase + (s * Q::R) * Q::WREG);
        f4 acc = *reinterpret_cast<const f4*>(w0 + j * Q::LDX + a);
#pragma unroll
        for (int i = 1; i < Q::R; ++i)
          acc += *reinterpret_cast<const f4*>(reinterpret_cast<const float*>(wbase + (s * Q::R + i) * Q::WREG) +
                                              j * Q::LDX + a);
        if constexpr (DXM == 2) {
          const uint16_t* xr = rowbuf + s * Q::SLOT + Q::OX + j * Q::LXA + a;
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[v] = bf2f(xr[v]) > 0.f ? acc[v] : 0.f;
        }
        *reinterpret_cast<s4*>(dx + row * D::IN + o) = pack4(acc);
      }
    }
    __syncthreads();   // the next step's stash overwrites the rows and this step's partials
  };
  const int64_t nfull = N / Q::RPI;
  int64_t grp = blockIdx.x;
  for (; grp < nfull; grp += gridDim.x) step(grp, std::false_type{});
  if (grp < ngrp) step(grp, std::true_type{});

  // Partial row of this workgroup: [dB (R*M*N) | dA (R*P*Q) | dS (P*Q) | dbias (Q*N)], fp32.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem) + slot * D::PWW;
#pragma unroll
  for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[rank * D::MN + (16 * ta + 4 * g + v) * D::N + 16 * tb + c] = dB[ta][tb][v];
#pragma unroll
  for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        red[D::R * D::MN + rank * D::PQ + (16 * tj + 4 * g + v) * D::Q + 16 * tk + c] = dC[tj][tk][v];
  if (rank == 0) {
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          red[D::R * (D::MN + D::PQ) + (16 * tk + c) * D::N + 16 * tb + 4 * g + v] = db[tk][tb][v];
  }
  __syncthreads();
  const PartRow out{part, (int64_t)gridDim.x, (int64_t)blockIdx.x, 0};
  const float* L = reinterpret_cast<const float*>(smem);
  auto ssum = [&](int e) {
    float t = L[e];
#pragma unroll
    for (int s = 1; s < Q::RPI; ++s) t += L[s * D::PWW + e];
    return t;
  };
  for (int e = tid; e < D::R * D::MN; e += kThreads) out[e] = ssum(e);
  for (int e = tid; e < D::PQ; e += kThreads) {
    const float sv = Sm ? bf2f(Sm[e]) : 1.f;
    float ds = 0.f;
#pragma unroll
    for (int i = 0; i < D::R; ++i) {
      const float dcv = ssum(D::R * D::MN + i * D::PQ + e);
      ds = fmaf(bf2f(A[i * D::PQ + e]), dcv, ds);
      out[D::R * D::MN + i * D::PQ + e] = sv * dcv;
    }
    out[D::R * (D::MN + D::PQ) + e] = Sm ? ds : 0.f;
  }
  for (int e = tid; e < D::Q * D::N; e += kThreads) out[D::R * (D::MN + D::PQ) + D::PQ + e] = ssum(D::R * (D::MN + D::PQ) + e);
}

int device_cus_bf16() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 256;
  return v;
}

template <class D>
void run_fwd_bf16(const LayerArgsBf16& a, hipStream_t s) {
  using F = FB<D>;
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fwd_bf16_kernel<D>, F::NT, 0) != hipSuccess || nb < 1)
      nb = 1;
    return nb;
  }();
  int64_t grid = (int64_t)per_cu * device_cus_bf16();
  const int64_t need = (a.N + F::NW - 1) / F::NW;
  if (grid > need) grid = need;
  hipLaunchKernelGGL(fwd_bf16_kernel<D>, dim3((unsigned)grid), dim3(F::NT), 0, s, a.N, a.flags, a.x, a.S, a.A,
                     a.B, a.bias, a.y);
}

template <class D>
void run_bwd_bf16(const LayerArgsBf16& a, int grid, hipStream_t s) {
  using Q = RB<D>;
  static const bool attr = [] {
    (void)hipFuncSetAttribute((const void*)bwd_bf16_kernel<D, 0>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Q::LDS);
    (void)hipFuncSetAttribute((const void*)bwd_bf16_kernel<D, 1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Q::LDS);
    (void)hipFuncSetAttribute((const void*)bwd_bf16_kernel<D, 2>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Q::LDS);
    return true;
  }();
  (void)attr;
  const int dxm = a.dx == nullptr ? 0 : ((a.flags & KRON_DX_RELU_MASK) ? 2 : 1);
  if (dxm == 0)
    hipLaunchKernelGGL((bwd_bf16_kernel<D, 0>), dim3(grid), dim3(kThreads), Q::LDS, s, a.N, a.x, a.S, a.A, a.B,
                       a.dy, a.dx, a.part);
  else if (dxm == 1)
    hipLaunchKernelGGL((bwd_bf16_kernel<D, 1>), dim3(grid), dim3(kThreads), Q::LDS, s, a.N, a.x, a.S, a.A, a.B,
                       a.dy, a.dx, a.part);
  else
    hipLaunchKernelGGL((bwd_bf16_kernel<D, 2>), dim3(grid), dim3(kThreads), Q::LDS, s, a.N, a.x, a.S, a.A, a.B,
                       a.dy, a.dx, a.part);
}

struct EntryBf16 {
  int p, q, m, n, r;
  int rows_per_step;
  void (*fwd)(const LayerArgsBf16&, hipStream_t);
  void (*bwd)(const LayerArgsBf16&, int, hipStream_t);
};

#define KRON_BF16_ENTRY(P, Q, M, N, R)                                                             \
  EntryBf16{P, Q, M, N, R, RB<BD<P, Q, M, N, R>>::RPI, &run_fwd_bf16<BD<P, Q, M, N, R>>,            \
            &run_bwd_bf16<BD<P, Q, M, N, R>>}

// The 1024x1024 layers with m = 32 (r = 1, 2, 4) and m = 64 (r = 2).
const EntryBf16 kBf16Table[] = {
    KRON_BF16_ENTRY(32, 32, 32, 32, 1), KRON_BF16_ENTRY(32, 32, 32, 32, 2), KRON_BF16_ENTRY(32, 32, 32, 32, 4),
    KRON_BF16_ENTRY(16, 16, 64, 64, 2),
};
static_assert(RB<BD<32, 32, 32, 32, 4>>::OK && RB<BD<32, 32, 32, 32, 2>>::OK && RB<BD<32, 32, 32, 32, 1>>::OK &&
                  RB<BD<16, 16, 64, 64, 2>>::OK,
              "every bf16 table shape fits its LDS budget");

const EntryBf16* find_bf16(int p, int q, int m, int n, int r) {
  for (const EntryBf16& e : kBf16Table)
    if (e.p == p && e.q == q && e.m == m && e.n == n && e.r == r) return &e;
  return nullptr;
}

}  // namespace

bool bf16_supported(int p, int q, int m, int n, int r) { return find_bf16(p, q, m, n, r) != nullptr; }

int bf16_bwd_groups(int64_t N, int p, int q, int m, int n, int r) {
  const EntryBf16* e = find_bf16(p, q, m, n, r);
  if (!e) return 0;
  const int64_t g = (N + e->rows_per_step - 1) / e->rows_per_step;
  const int64_t gmax = 2 * 256;   // two workgroups per compute unit (fixed: the workspace depends on it)
  return (int)(g < gmax ? g : gmax);
}

hipError_t launch_fwd_bf16(const LayerArgsBf16& a, hipStream_t s) {
  const EntryBf16* e = find_bf16(a.p, a.q, a.m, a.n, a.r);
  if (!e) return hipErrorInvalidValue;
  if (a.N == 0) return hipSuccess;
  e->fwd(a, s);
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(const LayerArgsBf16& a, int G, hipStream_t s) {
  const EntryBf16* e = find_bf16(a.p, a.q, a.m, a.n, a.r);
  if (!e) return hipErrorInvalidValue;
  if (G == 0) return hipSuccess;
  e->bwd(a, G, s);
  return hipGetLastError();
}

}  // namespace kron
