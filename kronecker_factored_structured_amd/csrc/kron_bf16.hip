// bf16 Kronecker-factored layer on bf16 matrix instructions (mixed precision: bf16
// operands, fp32 accumulation).  Same products as the fp32 kernels (Kronecker layer
// tutorial, "The vec trick" and "The vec trick without the loop"; the backward by
// calculus from them), on v_mfma_f32_16x16x32_bf16 where the contracted dimension is a
// multiple of 32 and v_mfma_f32_16x16x16_bf16 otherwise.  Lane l = 16g + c receives
// D[4g+v][c], v = 0..3, so an fp32 accumulator tile, rounded to bf16, supplies four
// consecutive values of its row index: two tiles 16 rows apart are the eight K values of a
// 16x16x32 operand when the next product contracts over that index (see k_acc below).
//
// Storage: x, S, A, B, bias, dy, y and dx are bf16 (bit patterns); dS, dA, dB and dbias
// are fp32.  C_i = S o A_i is formed in fp32 (exact for bf16 factors) and rounded to
// bf16; X B_i and G_i are rounded to bf16 (round to nearest even) before they enter their
// second product.  p and q are multiples of 16, m and n multiples of 8 (padded to 16 inside
// the tiles).
#include <type_traits>

#include "kron_internal.h"

namespace kron {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));


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

// P, Q, M, N are the layer's sizes; MP and NP round m and n up to a whole number of 16-wide
// tiles.  The products run over the padded sizes: the factor operands beyond m or n are
// zero (so is the padding of the row buffers), and nothing beyond m or n is stored.
template <int P_, int Q_, int M_, int N_, int R_>
struct BD {
  static constexpr int P = P_, Q = Q_, M = M_, N = N_, R = R_;
  static constexpr int MP = (M + 15) / 16 * 16, NP = (N + 15) / 16 * 16;
  static constexpr int TJ = P / 16, TK = Q / 16, TA = MP / 16, TB = NP / 16;
  static constexpr int IN = P * M, OUT = Q * N;
  static constexpr int MN = M * N, PQ = P * Q;
  static constexpr int PW = R * MN + R * PQ + PQ + Q * N;   // partial row (partial_width())
  static constexpr int PWW = R * MN + R * PQ + Q * N;       // one row slot's sums
  // (m and n in 8-element pieces: a 16-byte piece of a row never straddles two rows and a
  // padded K chunk starts on a piece boundary)
  static constexpr bool SHAPE_OK = P % 16 == 0 && Q % 16 == 0 && M % 8 == 0 && N % 8 == 0;
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
  static constexpr int W1 = D::MP % 32 == 0 ? 8 : 4, KC1 = D::MP / (4 * W1);  // Z = X B_i over a (padded)
  static constexpr int W2 = D::P % 32 == 0 ? 8 : 4, KC2 = D::P / (4 * W2);   // Y^T over j
  static constexpr int TAB_B = D::R * D::TB * KC1 * 64;   // lane entries of W1 values
  static constexpr int TAB_C = D::R * D::TK * KC2 * 64;   // lane entries of W2 values
  // registers per lane: factor tables, x (current and next row), accumulators, Z tiles, bias
  static constexpr int REGS = D::R * D::TB * KC1 * W1 / 2 + D::R * D::TK * KC2 * W2 / 2 + D::TJ * KC1 * W1 +
                              D::TB * D::TK * 6 + D::TJ * D::TB * 2 + 16;
  static constexpr int NT = REGS <= 128 ? 1024 : (REGS <= 200 ? 512 : 256);
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
      for (int s = 0; s < KC1; ++s) {
        const int a0 = k_row<W1>(s, g, 0);   // (a piece lies wholly below or above m)
        if (D::MP == D::M || a0 < D::M)
          dst[tj][s] = *reinterpret_cast<const O1*>(xr + (16 * tj + c) * D::M + a0);
        else
          dst[tj][s] = O1{};
      }
  };
  static_assert(D::M % W1 == 0, "x pieces of W1 elements");
  if (row < N) load_x(xn, row);

  for (int e = tid; e < F::TAB_B; e += F::NT) {   // e = ((i*TB + tb)*KC1 + s)*64 + lane
    const int ln = e & 63, rest = e >> 6, s = rest % KC1, tb = (rest / KC1) % D::TB, i = rest / (KC1 * D::TB);
    const int b = 16 * tb + (ln & 15);
    const uint16_t* Bi = B + i * D::MN + b;
    O1 v;
#pragma unroll
    for (int u = 0; u < W1; ++u) {
      const int a = k_row<W1>(s, ln >> 4, u);
      v[u] = (a < D::M && b < D::N) ? (short)Bi[a * D::N] : (short)0;
    }
    *reinterpret_cast<O1*>(tabB + e * W1) = v;
  }
  for (int e = tid; e < F::TAB_C; e += F::NT) {   // e = ((i*TK + tk)*KC2 + s)*64 + lane
    const int ln = e & 63, rest = e >> 6, s = rest % KC2, tk = (rest / KC2) % D::TK, i = rest / (KC2 * D::TK);
    const int k = 16 * tk + (ln & 15);
    // every load unconditional (S absent: A stands in, and the factor is 1), so that the
    // loads of all W2 values go out before the first wait
    const uint16_t* Sp = Sm ? Sm : A;
    uint16_t av[W2], sv[W2];
#pragma unroll
    for (int u = 0; u < W2; ++u) {
      const int jk = k_acc<W2>(s, ln >> 4, u) * D::Q + k;
      av[u] = A[i * D::PQ + jk];
      sv[u] = Sp[jk];
    }
    O2 v;
#pragma unroll
    for (int u = 0; u < W2; ++u) v[u] = (short)f2bf((Sm ? bf2f(sv[u]) : 1.f) * bf2f(av[u]));
    *reinterpret_cast<O2*>(tabC + e * W2) = v;
  }
  // bias of the lane's outputs: Y^T[b = 16tb + 4g + v][k = 16tk + c] -> bias[k*N + b]
  s4 bv[D::TB][D::TK];
#pragma unroll
  for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk)
      bv[tb][tk] = (bias && 16 * tb + 4 * g < D::N) ? load_s4(bias + (16 * tk + c) * D::N + 16 * tb + 4 * g)
                                                     : s4{0, 0, 0, 0};
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
        if (D::NP == D::N || 16 * tb + 4 * g < D::N)
          *reinterpret_cast<s4*>(yr + (16 * tk + c) * D::N + 16 * tb + 4 * g) = pack4(o);
      }
  }
}

// ---------------------------------------------------------------------------------
// Backward, rank-parallel: a workgroup of R * RPI wavefronts owns RPI rows per step;
// wavefront w works on row slot w / R and rank i = w % R.  Per rank and row, with the K
// order of each product's operands in brackets:
//   Z^T[b][j]  = sum_a B_i^T[b][a] X[j][a]      A: table          B: X row pieces      [k_row]
//   dC[j][k]  += sum_b Z[j][b] dY[k][b]         A: Z^T tiles      B: dY row pieces     [k_acc]
//   G^T[b][j]  = sum_k dY[k][b] C_i[j][k]       A: dY columns     B: table             [k_acc]
//   G[j][b]    = sum_k C_i[j][k] dY[k][b]       A: table          B: dY columns        [k_acc]
//   dB[a][b]  += sum_j X[j][a] G_i[j][b]        A: X columns      B: G tiles           [k_acc]
// and per row, all ranks in one contraction over (i, b), split by output tile over the
// row's R wavefronts:
//   dX^T[a][j] = sum_(i,b) B_i[a][b] G_i[j][b]  A: table          B: G_i row pieces    [k_row]
// Rows and G_i tiles live in LDS in row-major order (16-byte row writes, 8-byte G_i writes);
// column operands come from the LDS transpose read ds_read_b64_tr_b16, which hands each
// lane four consecutive rows of one column.  Rows are triple-buffered and G tiles
// double-buffered, so one barrier per step suffices: the rows of step t+1 are written
// during step t into the buffer last read in step t-2, and every wavefront has left step
// t-2 once all have reached the barrier of step t-1.
// The partial row [dB | dA | dS | dbias] and the fixed-order column reduction are those of
// the fp32 layer.
// ---------------------------------------------------------------------------------
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

// lane (g, c) receives m[r0 + v][cb + c], v = 0..3, where r0 is the lane group's first row
__device__ __forceinline__ s4 tr16(const uint16_t* m, int ld, int r0, int cb, int lane) {
  const int l = lane & 15;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4*)(m + (r0 + (l >> 2)) * ld + cb + 4 * (l & 3)));
}
// W values of one column (cb + c) over the K rows of chunk s in k_acc order
template <int W>
__device__ __forceinline__ typename OpT<W>::T col_op(const uint16_t* m, int ld, int s, int g, int cb, int lane) {
  if constexpr (W == 8)
    return join(tr16(m, ld, 32 * s + 4 * g, cb, lane), tr16(m, ld, 32 * s + 16 + 4 * g, cb, lane));
  else
    return tr16(m, ld, 16 * s + 4 * g, cb, lane);
}
// W values of one row in k_acc order (two 8-byte pieces for W = 8)
template <int W>
__device__ __forceinline__ typename OpT<W>::T row_acc(const uint16_t* r, int s, int g) {
  if constexpr (W == 8)
    return join(load_s4(r + 32 * s + 4 * g), load_s4(r + 32 * s + 16 + 4 * g));
  else
    return load_s4(r + 16 * s + 4 * g);
}

template <class D, int RPI_>
struct BB {
  static constexpr int R = D::R;
  static constexpr int RPI = RPI_;   // rows per step
  static constexpr int NW = R * RPI, NT = 64 * NW;
  static constexpr int WA = D::MP % 32 == 0 ? 8 : 4, KA = D::MP / (4 * WA);   // over a (padded)
  static constexpr int WB = D::NP % 32 == 0 ? 8 : 4, KB = D::NP / (4 * WB);   // over b (padded)
  static constexpr int WK = D::Q % 32 == 0 ? 8 : 4, KK = D::Q / (4 * WK);   // over k
  static constexpr int WJ = D::P % 32 == 0 ? 8 : 4, KJ = D::P / (4 * WJ);   // over j
  // dX^T tiles per wavefront (the last ranks' wavefronts get fewer when R does not divide
  // the tile count)
  static constexpr int DXT = (D::TA * D::TJ + R - 1) / R;
  // LDS (bf16 elements), row strides chosen by measured bank behaviour: x rows (16-byte row
  // reads and transpose reads) at 16 mod 32 elements, dy rows (pairs of 8-byte row reads and
  // transpose reads) and G rows (8-byte writes, 16-byte reads) at 8 mod 16 elements.
  // A step's rows: x [P][LX], dy [Q][LY]; its G tiles [R][P][LG].
  static constexpr int LX = D::MP + 16, LY = D::NP + 24, LG = D::NP + 24;
  static constexpr int XS = D::P * LX, YS = D::Q * LY, GR = D::P * LG;
  static constexpr int ROWS = RPI * (XS + YS), GBUF = RPI * R * GR;
  // Rows are triple-buffered and G tiles double-buffered so that one barrier per step
  // orders the wavefronts; a workgroup of one wavefront needs neither (its LDS accesses
  // complete in program order), so it keeps two row buffers and one G buffer.
  static constexpr int NRB = NW == 1 ? 2 : 3, NGB = NW == 1 ? 1 : 2;
  static constexpr size_t MAIN = (size_t)(NRB * ROWS + NGB * GBUF) * 2;
  // prologue staging: B_i [a][b] and C_i [j][k] row-major with odd-word row strides
  static constexpr int SB = D::N + 2, SC = D::Q + 2;
  static constexpr size_t STAGE = (size_t)(R * D::M * SB + R * D::P * SC) * 2;
  static constexpr size_t COMBINE = (size_t)RPI * D::PWW * 4;
  static constexpr size_t LDS = MAIN > COMBINE ? (MAIN > STAGE ? MAIN : STAGE) : (COMBINE > STAGE ? COMBINE : STAGE);
  static constexpr int CHUNKS = (D::IN + D::OUT) / 8;   // 16-byte pieces of one row's x and dy
  static constexpr int NPF = (RPI * CHUNKS + NT - 1) / NT;
  static constexpr bool OK = D::SHAPE_OK && (R == 1 || R == 2 || R == 4 || R == 8) && NW <= 16 &&
                             LDS <= 160 * 1024;
};

template <class D, int RPI, int DXM>
__global__ __launch_bounds__((BB<D, RPI>::NT)) void bwd_bf16_kernel(int64_t N, const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ Sm,
                                                               const uint16_t* __restrict__ A,
                                                               const uint16_t* __restrict__ B,
                                                               const uint16_t* __restrict__ dy,
                                                               uint16_t* __restrict__ dx, float* __restrict__ part) {
  using Q = BB<D, RPI>;
  constexpr int R = D::R, NT = Q::NT;
  constexpr int WA = Q::WA, KA = Q::KA, WB = Q::WB, KB = Q::KB, WK = Q::WK, KK = Q::KK, WJ = Q::WJ, KJ = Q::KJ;
  typedef typename OpT<WA>::T OA;
  typedef typename OpT<WB>::T OB;
  typedef typename OpT<WK>::T OQ;
  typedef typename OpT<WJ>::T OJ;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15, wave = tid >> 6;
  const int slot = wave / R, rank = wave % R;
  const int64_t ngrp = (N + Q::RPI - 1) / Q::RPI;

  // one step's rows as 16-byte pieces: x then dy of each row slot (zero past the last row);
  // two register sets alternate so that each step's rows are requested three steps ahead.
  // Every piece is loaded unconditionally (rows past the end read the last row, or the
  // workspace when there are no rows) and a bit per piece says whether it is live; the
  // zeroing waits for the stash.  With no branches around the loads the compiler can count
  // them, so a stash waits only for its own loads, not for the dX stores issued after them.
  u4 pfA[Q::NPF], pfB[Q::NPF];
  uint32_t okA = 0, okB = 0;
  static_assert(Q::NPF <= 32, "one live bit per prefetched piece");
  auto fetch = [&](u4 (&pf)[Q::NPF], uint32_t& ok, int64_t grp) {
    ok = 0;
#pragma unroll
    for (int t = 0; t < Q::NPF; ++t) {
      const int f = tid + t * NT;
      const bool fin = f < Q::RPI * Q::CHUNKS;
      const int fc = fin ? f : Q::RPI * Q::CHUNKS - 1;
      const int s = fc / Q::CHUNKS, o = 8 * (fc % Q::CHUNKS);
      const int64_t row = grp * Q::RPI + s;
      const bool live = fin && grp < ngrp && row < N;
      const int64_t rc = row < N ? row : N - 1;
      const uint16_t* src = o < D::IN ? x + rc * D::IN + o : dy + rc * D::OUT + (o - D::IN);
      if (N == 0) src = reinterpret_cast<const uint16_t*>(part);
      pf[t] = *reinterpret_cast<const u4*>(src);
      ok |= (live ? 1u : 0u) << t;
    }
  };
  auto stash = [&](const u4 (&pf)[Q::NPF], uint32_t ok, int buf) {
#pragma unroll
    for (int t = 0; t < Q::NPF; ++t) {
      const int f = tid + t * NT;
      if (f < Q::RPI * Q::CHUNKS) {
        const int s = f / Q::CHUNKS, o = 8 * (f % Q::CHUNKS);
        uint16_t* rb = lds + buf * Q::ROWS + s * (Q::XS + Q::YS);
        const u4 v = (ok >> t) & 1u ? pf[t] : u4{0u, 0u, 0u, 0u};
        if (o < D::IN)
          *reinterpret_cast<u4*>(rb + (o / D::M) * Q::LX + o % D::M) = v;
        else
          *reinterpret_cast<u4*>(rb + Q::XS + ((o - D::IN) / D::N) * Q::LY + (o - D::IN) % D::N) = v;
      }
    }
  };
  fetch(pfA, okA, blockIdx.x);

  // ---- prologue: B_i and C_i = S o A_i staged row-major, then this wavefront's operands
  uint16_t* sB = lds;                               // [i][a][SB]
  uint16_t* sC = lds + R * D::M * Q::SB;            // [i][j][SC]
  for (int e = tid; e < R * D::MN / 2; e += NT) {   // pairs of B values
    const int i = e / (D::MN / 2), r = 2 * (e % (D::MN / 2)), a = r / D::N, b = r % D::N;
    *reinterpret_cast<uint32_t*>(sB + (i * D::M + a) * Q::SB + b) =
        *reinterpret_cast<const uint32_t*>(B + i * D::MN + r);
  }
  for (int e = tid; e < R * D::PQ / 2; e += NT) {
    const int i = e / (D::PQ / 2), r = 2 * (e % (D::PQ / 2)), j = r / D::Q, k = r % D::Q;
    // (both loads unconditional: S absent, A stands in and the factor is 1)
    const uint32_t av = *reinterpret_cast<const uint32_t*>(A + i * D::PQ + r);
    const uint32_t sv = *reinterpret_cast<const uint32_t*>((Sm ? Sm : A) + r);
    float a0 = bf2f((uint16_t)(av & 0xffffu)), a1 = bf2f((uint16_t)(av >> 16));
    if (Sm) {
      a0 *= bf2f((uint16_t)(sv & 0xffffu));
      a1 *= bf2f((uint16_t)(sv >> 16));
    }
    *reinterpret_cast<uint32_t*>(sC + (i * D::P + j) * Q::SC + k) = pack2(a0, a1);
  }
  __syncthreads();
  OA t1[D::TB][KA];         // B_i^T[b = 16tb + c][a = k_row(s, g, u)]
  OQ t3[D::TJ][KK];         // C_i^T[k = k_acc(s, g, u)][j = 16tj + c]
  OB t4[Q::DXT][R][KB];     // B_i'[a = 16ta + c][b = k_row(s, g, u)] for this wavefront's dX^T tiles
  {
    const uint16_t* Bi = sB + rank * D::M * Q::SB;
    const uint16_t* Ci = sC + rank * D::P * Q::SC;
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int s = 0; s < KA; ++s)
#pragma unroll
        for (int u = 0; u < WA; ++u) {
          const int a = k_row<WA>(s, g, u), b = 16 * tb + c;
          t1[tb][s][u] = (a < D::M && b < D::N) ? (short)Bi[a * Q::SB + b] : (short)0;
        }
#pragma unroll
    for (int tj = 0; tj < D::TJ; ++tj)
#pragma unroll
      for (int s = 0; s < KK; ++s)
#pragma unroll
        for (int u = 0; u < WK; ++u) t3[tj][s][u] = (short)Ci[(16 * tj + c) * Q::SC + k_acc<WK>(s, g, u)];
#pragma unroll
    for (int d = 0; d < Q::DXT; ++d) {
      const int ta = (rank * Q::DXT + d) / D::TJ;
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int s = 0; s < KB; ++s)
#pragma unroll
          for (int u = 0; u < WB; ++u) {
            const int a = 16 * ta + c, b = k_row<WB>(s, g, u);
            t4[d][i][s][u] = (a < D::M && b < D::N) ? (short)sB[(i * D::M + a) * Q::SB + b] : (short)0;
          }
    }
  }
  __syncthreads();   // the staging area becomes row buffers
  if constexpr (D::MP != D::M || D::NP != D::N) {
    // the padding columns of every row buffer (x: a in [m, MP), dy: b in [n, NP)) are read
    // by the products and never written by the row stashes: zero them once
    constexpr int XPAD = D::MP - D::M, YPAD = D::NP - D::N;
    constexpr int XD = XPAD > 0 ? XPAD : 1, YD = YPAD > 0 ? YPAD : 1;
    constexpr int PER = D::P * XPAD + D::Q * YPAD;   // padding elements of one row slot
    for (int e = tid; e < Q::NRB * Q::RPI * PER; e += NT) {
      const int slot_all = e / PER, r = e % PER;
      uint16_t* rb = lds + (slot_all / Q::RPI) * Q::ROWS + (slot_all % Q::RPI) * (Q::XS + Q::YS);
      if (r < D::P * XPAD)
        rb[(r / XD) * Q::LX + D::M + r % XD] = 0;
      else
        rb[Q::XS + ((r - D::P * XPAD) / YD) * Q::LY + D::N + (r - D::P * XPAD) % YD] = 0;
    }
  }
  stash(pfA, okA, 0);
  fetch(pfA, okA, blockIdx.x + (int64_t)gridDim.x);
  fetch(pfB, okB, blockIdx.x + 2 * (int64_t)gridDim.x);
  __syncthreads();

  f4 dC[D::TJ][D::TK];    // dC_i[j = 16tj + 4g + v][k = 16tk + c]
  f4 dB[D::TA][D::TB];    // dB_i[a = 16ta + 4g + v][b = 16tb + c]
  float db[D::TK][KB][WB];  // dbias[k = 16tk + c][b = k_acc(s, g, u)]   (rank 0)
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
    for (int s = 0; s < KB; ++s)
#pragma unroll
      for (int u = 0; u < WB; ++u) db[tk][s][u] = 0.f;

  auto step = [&](int64_t grp, int rbuf, int gbuf, u4 (&pf)[Q::NPF], uint32_t& ok, auto tail_c) {
    constexpr bool kTail = decltype(tail_c)::value;
    const uint16_t* X = lds + rbuf * Q::ROWS + slot * (Q::XS + Q::YS);
    const uint16_t* Y = X + Q::XS;
    uint16_t* Gs = lds + Q::NRB * Q::ROWS + gbuf * Q::GBUF + slot * R * Q::GR;   // G_i: Gs + i * GR
    uint16_t* Gi = Gs + rank * Q::GR;
    // Z^T[b][j] = sum_a B_i^T[b][a] X[j][a]
    s4 zb[D::TB][D::TJ];
#pragma unroll
    for (int tj = 0; tj < D::TJ; ++tj) {
      OA xo[KA];
#pragma unroll
      for (int s = 0; s < KA; ++s) xo[s] = *reinterpret_cast<const OA*>(X + (16 * tj + c) * Q::LX + k_row<WA>(s, g, 0));
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb) {
        f4 z = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KA; ++s) z = mfma(t1[tb][s], xo[s], z);
        zb[tb][tj] = pack4(z);
      }
    }
    // dC[j][k] += sum_b Z[j][b] dY[k][b];  dbias += dY (rank 0)
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
      for (int s = 0; s < KB; ++s) {
        const OB yo = row_acc<WB>(Y + (16 * tk + c) * Q::LY, s, g);
        if (rank == 0) {
#pragma unroll
          for (int u = 0; u < WB; ++u) db[tk][s][u] += bf2f((uint16_t)yo[u]);
        }
#pragma unroll
        for (int tj = 0; tj < D::TJ; ++tj) {
          OB zo;
          if constexpr (WB == 8)
            zo = join(zb[2 * s][tj], zb[2 * s + 1][tj]);
          else
            zo = join(zb[s][tj]);
          dC[tj][tk] = mfma(zo, yo, dC[tj][tk]);
        }
      }
    // G_i in both orientations from the same two operands (the dY columns and the C_i
    // table, which are each other's transpose roles): G^T[b][j] goes to LDS as G_i[j][b] for
    // the dX contraction of all ranks; G[j][b] stays in registers as the B operand of dB.
    s4 gj[D::TJ][D::TB];   // bf16 G[j = 16tj + 4g + v][b = 16tb + c]
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb) {
      OQ yc[KK];
#pragma unroll
      for (int s = 0; s < KK; ++s) yc[s] = col_op<WK>(Y, Q::LY, s, g, 16 * tb, lane);
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj) {
        f4 gtv = f4{0.f, 0.f, 0.f, 0.f}, gv = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KK; ++s) {
          gtv = mfma(yc[s], t3[tj][s], gtv);
          gv = mfma(t3[tj][s], yc[s], gv);
        }
        *reinterpret_cast<s4*>(Gi + (16 * tj + c) * Q::LG + 16 * tb + 4 * g) = pack4(gtv);
        gj[tj][tb] = pack4(gv);
      }
    }
    // the next step's rows into the next row buffer; this register set fetches three steps ahead
    stash(pf, ok, rbuf == Q::NRB - 1 ? 0 : rbuf + 1);
    fetch(pf, ok, grp + 3 * (int64_t)gridDim.x);
    __syncthreads();
    // dX^T[a][j] = sum_(i,b) B_i[a][b] G_i[j][b]: this wavefront's tiles
    const int64_t row = grp * Q::RPI + slot;
#pragma unroll
    for (int d = 0; d < Q::DXT; ++d) {
      const int t = rank * Q::DXT + d, ta = t / D::TJ, tj = t % D::TJ;
      if ((D::TA * D::TJ) % R != 0 && t >= D::TA * D::TJ) break;   // (uniform per wavefront)
      f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int s = 0; s < KB; ++s)
          acc = mfma(t4[d][i][s],
                     *reinterpret_cast<const OB*>(Gs + i * Q::GR + (16 * tj + c) * Q::LG + k_row<WB>(s, g, 0)), acc);
      if constexpr (DXM != 0) {
        if ((!kTail || row < N) && (D::MP == D::M || 16 * ta + 4 * g < D::M)) {
          const int off = (16 * tj + c) * D::M + 16 * ta + 4 * g;   // dX[j][a .. a+3]
          if constexpr (DXM == 2) {
            const s4 xm = load_s4(X + (16 * tj + c) * Q::LX + 16 * ta + 4 * g);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] = bf2f((uint16_t)xm[v]) > 0.f ? acc[v] : 0.f;
          }
          *reinterpret_cast<s4*>(dx + row * D::IN + off) = pack4(acc);
        }
      }
    }
    // dB_i[a][b] += sum_j X[j][a] G_i[j][b]; the G operand (K = j in k_acc order) is the
    // pair of G tiles 2s, 2s + 1 (or tile s) held since the first phase
    OJ gc[D::TB][KJ];
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int s = 0; s < KJ; ++s) {
        if constexpr (WJ == 8)
          gc[tb][s] = join(gj[2 * s][tb], gj[2 * s + 1][tb]);
        else
          gc[tb][s] = join(gj[s][tb]);
      }
#pragma unroll
    for (int ta = 0; ta < D::TA; ++ta) {
      OJ xc[KJ];
#pragma unroll
      for (int s = 0; s < KJ; ++s) xc[s] = col_op<WJ>(X, Q::LX, s, g, 16 * ta, lane);
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
        for (int s = 0; s < KJ; ++s) dB[ta][tb] = mfma(xc[s], gc[tb][s], dB[ta][tb]);
    }
  };
  const int64_t nfull = N / Q::RPI, G = gridDim.x;
  int64_t grp = blockIdx.x;
  int rbuf = 0, gbuf = 0;
  auto advance = [&]() {
    rbuf = rbuf == Q::NRB - 1 ? 0 : rbuf + 1;
    gbuf = Q::NGB == 1 ? 0 : gbuf ^ 1;
    grp += G;
  };
  while (grp + G < nfull) {   // local steps in pairs: register set A, then B
    step(grp, rbuf, gbuf, pfA, okA, std::false_type{});
    advance();
    step(grp, rbuf, gbuf, pfB, okB, std::false_type{});
    advance();
  }
  if (grp < nfull) {
    step(grp, rbuf, gbuf, pfA, okA, std::false_type{});
    advance();
    if (grp < ngrp) step(grp, rbuf, gbuf, pfB, okB, std::true_type{});
  } else if (grp < ngrp) {
    step(grp, rbuf, gbuf, pfA, okA, std::true_type{});
  }

  // Partial row of this workgroup: [dB (R*M*N) | dA (R*P*Q) | dS (P*Q) | dbias (Q*N)], fp32.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem) + slot * D::PWW;
#pragma unroll
  for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int a = 16 * ta + 4 * g + v, b = 16 * tb + c;
        if (a < D::M && b < D::N) red[rank * D::MN + a * D::N + b] = dB[ta][tb][v];
      }
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
      for (int s = 0; s < KB; ++s)
#pragma unroll
        for (int u = 0; u < WB; ++u) {
          const int b = k_acc<WB>(s, g, u);
          if (b < D::N) red[D::R * (D::MN + D::PQ) + (16 * tk + c) * D::N + b] = db[tk][s][u];
        }
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
  for (int e = tid; e < D::R * D::MN; e += NT) out[e] = ssum(e);
  for (int e = tid; e < D::PQ; e += NT) {
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
  for (int e = tid; e < D::Q * D::N; e += NT) out[D::R * (D::MN + D::PQ) + D::PQ + e] = ssum(D::R * (D::MN + D::PQ) + e);
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

template <class D, int RPI>
void run_bwd_bf16(const LayerArgsBf16& a, int grid, hipStream_t s) {
  using Q = BB<D, RPI>;
  static const bool attr = [] {
    (void)hipFuncSetAttribute((const void*)bwd_bf16_kernel<D, RPI, 0>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)Q::LDS);
    (void)hipFuncSetAttribute((const void*)bwd_bf16_kernel<D, RPI, 1>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)Q::LDS);
    (void)hipFuncSetAttribute((const void*)bwd_bf16_kernel<D, RPI, 2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)Q::LDS);
    return true;
  }();
  (void)attr;
  const int dxm = a.dx == nullptr ? 0 : ((a.flags & KRON_DX_RELU_MASK) ? 2 : 1);
  if (dxm == 0)
    hipLaunchKernelGGL((bwd_bf16_kernel<D, RPI, 0>), dim3(grid), dim3(Q::NT), Q::LDS, s, a.N, a.x, a.S, a.A, a.B,
                       a.dy, a.dx, a.part);
  else if (dxm == 1)
    hipLaunchKernelGGL((bwd_bf16_kernel<D, RPI, 1>), dim3(grid), dim3(Q::NT), Q::LDS, s, a.N, a.x, a.S, a.A, a.B,
                       a.dy, a.dx, a.part);
  else
    hipLaunchKernelGGL((bwd_bf16_kernel<D, RPI, 2>), dim3(grid), dim3(Q::NT), Q::LDS, s, a.N, a.x, a.S, a.A, a.B,
                       a.dy, a.dx, a.part);
}

struct EntryBf16 {
  int p, q, m, n, r;
  int rows_per_step, groups_per_cu;
  void (*fwd)(const LayerArgsBf16&, hipStream_t);
  void (*bwd)(const LayerArgsBf16&, int, hipStream_t);
};

// Rows per backward step and backward workgroups per compute unit, chosen per shape so
// that the resident workgroups' rows, G tiles (LDS) and registers fill a compute unit.
#define KRON_BF16_ENTRY(P, Q, M, N, R, RPI, WPC)                                               \
  EntryBf16{P, Q, M, N, R, RPI, WPC, &run_fwd_bf16<BD<P, Q, M, N, R>>, &run_bwd_bf16<BD<P, Q, M, N, R>, RPI>}

// The 1024x1024 layers with m = 32 (r = 1, 2, 4) and m = 64 (r = 2), and the GPT-2 FFN
// pair 768 <-> 3072 (A_i 32 x 64, B_i 24 x 48 and the transposed layer; r = 1, 2, 4, 8).
#define KRON_BF16_SHAPES(X)                                                                       \
  X(32, 32, 32, 32, 1, 4, 1) X(32, 32, 32, 32, 2, 4, 1) X(32, 32, 32, 32, 4, 3, 1)                \
  X(16, 16, 64, 64, 2, 2, 1) X(32, 64, 24, 48, 1, 1, 4) X(32, 64, 24, 48, 2, 1, 2)                \
  X(32, 64, 24, 48, 4, 1, 2) X(32, 64, 24, 48, 8, 1, 1) X(64, 32, 48, 24, 1, 1, 4)                \
  X(64, 32, 48, 24, 2, 1, 2) X(64, 32, 48, 24, 4, 1, 1) X(64, 32, 48, 24, 8, 1, 1)
#define KRON_BF16_ROW(P, Q, M, N, R, RPI, WPC) KRON_BF16_ENTRY(P, Q, M, N, R, RPI, WPC),
const EntryBf16 kBf16Table[] = {KRON_BF16_SHAPES(KRON_BF16_ROW)};
#undef KRON_BF16_ROW
#define KRON_BF16_FITS(P, Q, M, N, R, RPI, WPC)                                                  \
  static_assert(BD<P, Q, M, N, R>::SHAPE_OK && BB<BD<P, Q, M, N, R>, RPI>::OK &&                  \
                    WPC * BB<BD<P, Q, M, N, R>, RPI>::LDS <= 160 * 1024,                            \
                "bf16 table shape within its LDS budget");
KRON_BF16_SHAPES(KRON_BF16_FITS)
#undef KRON_BF16_FITS

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
  const int64_t gmax = (int64_t)e->groups_per_cu * 256;   // fixed per shape: the workspace depends on it
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
