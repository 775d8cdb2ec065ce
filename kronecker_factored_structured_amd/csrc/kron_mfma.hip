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

// The shapes with matrix-core kernels, (p, q, m, n, r, backward kernel): the 64x64 tiny
// layer (m = 8), the 1024x1024 layers with m = 32 and m = 64, and the GPT-2 FFN pair
// 768 <-> 3072.  Backward kernel (measured per shape): 0 = bwd_mfma_kernel, 1 = the
// rank-parallel bwd_rp_kernel, 2 = the whole-row bwd_solo_kernel.
#define KRON_MFMA_SHAPES(X)                                                                             \
  X(8, 8, 8, 8, 1, 1) X(8, 8, 8, 8, 2, 1) X(32, 32, 32, 32, 1, 1) X(32, 32, 32, 32, 2, 1)               \
  X(32, 32, 32, 32, 4, 2) X(16, 16, 64, 64, 1, 0) X(16, 16, 64, 64, 2, 0)                               \
  X(32, 64, 24, 48, 1, 0) X(32, 64, 24, 48, 2, 0) X(32, 64, 24, 48, 4, 1)                               \
  X(32, 64, 24, 48, 8, 1) X(64, 32, 48, 24, 1, 0) X(64, 32, 48, 24, 2, 1)                               \
  X(64, 32, 48, 24, 4, 1) X(64, 32, 48, 24, 8, 1)

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
  // the forward stages the raw factors next to its tables when they fit, else one rank's
  // raw factors at a time (FWD_RAW1), else builds the tables straight from global memory
  static constexpr bool FWD_RAW = (size_t)(BOP + COPF + RAW) * 4 <= kMaxLds;
  static constexpr int RAW1 = M * N + (P * Q + 3) / 4 * 4;
  static constexpr bool FWD_RAW1 = !FWD_RAW && (P * Q) % 4 == 0 && (size_t)(BOP + COPF + RAW1) * 4 <= kMaxLds;
  // the forward's row map (FwdMap): a 64-bit row mask per wavefront and the map (TJ*16 ints)
  static constexpr int FWD_MAP = (2 * kWaves + TJ * 16 + 1 + 3) / 4 * 4;   // + the tile mask
  static constexpr int FWD_FLOATS = BOP + COPF + (FWD_RAW ? RAW + FWD_MAP : (FWD_RAW1 ? RAW1 : 0));
  static constexpr int BWD_TABLES = BOP + COPG + BOPX;
  static constexpr int BWD_SCRATCH = (kWaves * GS > RAW) ? kWaves * GS : RAW;
  static constexpr int BWD_MAIN = BWD_TABLES + BWD_SCRATCH;
  static constexpr size_t FWD_LDS = (size_t)FWD_FLOATS * 4;
  // registers held across a backward row (accumulators and per-row operands), in floats
  static constexpr int ROW_REGS = TJ * SA + TA * SJ + TK * TB * 4 + TB * SK;
  static constexpr int BWD_REGS =
      R * TJ * TK * 4 + R * TA * TB * 4 + TK * TB * 4 + ROW_REGS + TA * TJ * 4 + TB * TJ * 8;
  static_assert(M % 4 == 0 && N % 4 == 0, "rows are moved as 4-float vectors");
  // bwd_mfma_kernel's row tiles: each wavefront stages its next row's x and dY in LDS
  // (16-byte loads, 16-byte writes) and reads the row operands back from there.  Row
  // pitches: x rows at m + 4 floats, dY rows at a pitch of 16 mod 32 words, so that the
  // 4-byte column reads of one half-wavefront fall in distinct banks.
  static constexpr int TLX = M + 4;
  static constexpr int TLY = N + ((16 - N % 32) + 32) % 32;
  static constexpr int TXT = P * TLX, TYT = Q * TLY;                    // one wavefront's tiles
  static constexpr int NXF = (IN / 4 + 63) / 64, NYF = (OUT / 4 + 63) / 64;   // 16-byte loads per lane
  static constexpr bool BWD_TILED = (size_t)(BWD_MAIN + kWaves * (TXT + TYT)) * 4 <= kMaxLds &&
                                    BWD_REGS + 4 * (NXF + NYF) <= 420;
  static constexpr int BWD_USED = BWD_MAIN + (BWD_TILED ? kWaves * (TXT + TYT) : 0);
  static constexpr size_t BWD_LDS = (size_t)(BWD_USED > kWaves * PWW ? BWD_USED : kWaves * PWW) * 4;
  static constexpr bool FWD_OK = FWD_LDS <= kMaxLds;
  // thresholds measured against the compiler's allocation (no scratch below them)
  static constexpr bool BWD_OK = BWD_LDS <= kMaxLds && BWD_REGS <= 360;
  static constexpr bool BWD_PREFETCH = BWD_REGS + ROW_REGS <= 420;   // double-buffer the row operands
};

// The saved intermediate Z_i = X B_i of the 32x32-block layers, for the ranks i < RANKS:
// the forward writes it for every row, and the whole-row backward reads it for those ranks
// instead of recomputing them.  RANKS = 2 of 4 was measured best at 20,000 rows: each
// saved rank takes about 6 us off the backward, while the forward, whose HBM traffic
// doubles with two saved ranks, slows by 3 and 7 us for one and two and by 18 us for
// three, where it reaches the HBM rate a device copy gets.  Per row, rank-major; per
// rank, the four 16x16 tiles (tb, tj) in the forward's lane order: lane 16g + c holds
// Z[16tj + 4g + v][16tb + c] in slot v.  The forward stores a tile as one 16-byte piece
// per lane (whole 128-byte lines); the backward, which needs the tile transposed, gathers
// it with 4-byte loads whose lines L1 serves after the first.
template <class D>
struct ZCache {
  static constexpr bool OK = D::P == 32 && D::Q == 32 && D::M == 32 && D::N == 32 && D::R == 4;
  static constexpr int RANKS = 2;
  static_assert(2 * RANKS <= D::R || !OK, "the next row's requests sit in recomputed ranks");
  static constexpr int ROW = RANKS * 1024;   // floats per row
};

// Stage B (as is) and C = S o A in LDS with coalesced 16-byte loads.  Every global load
// is issued before the first LDS store, so the staging costs one memory round trip.
// With cbits, also set bit j of *cbits for every row j of C (any rank) that holds a
// nonzero value among this thread's entries (Q % 4 == 0: a 4-float vector lies in one row).
template <class D>
__device__ __forceinline__ void stage_raw(float* rB, float* rC, const float* __restrict__ B,
                                          const float* __restrict__ S, const float* __restrict__ A,
                                          unsigned long long* cbits = nullptr) {
  constexpr int PQ = D::P * D::Q;
  if constexpr (PQ % 4 == 0) {
    constexpr int NB = D::RAWB / 4, NC = D::R * PQ / 4;
    constexpr int KB = (NB + kThreads - 1) / kThreads, KC = (NC + kThreads - 1) / kThreads;
    f4 b[KB], a[KC], m[KC];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int e = threadIdx.x + k * kThreads;
      if (NB % kThreads == 0 || e < NB) b[k] = reinterpret_cast<const f4*>(B)[e];
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int e = threadIdx.x + k * kThreads;
      if (NC % kThreads == 0 || e < NC) {
        a[k] = reinterpret_cast<const f4*>(A)[e];
        m[k] = S ? reinterpret_cast<const f4*>(S)[e % (PQ / 4)] : f4{1.f, 1.f, 1.f, 1.f};
      }
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int e = threadIdx.x + k * kThreads;
      if (NB % kThreads == 0 || e < NB) reinterpret_cast<f4*>(rB)[e] = b[k];
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int e = threadIdx.x + k * kThreads;
      if (NC % kThreads == 0 || e < NC) {
        const f4 cv = S ? a[k] * m[k] : a[k];
        reinterpret_cast<f4*>(rC)[e] = cv;
        if constexpr (D::Q % 4 == 0 && D::P <= 64) {
          if (cbits && (cv[0] != 0.f || cv[1] != 0.f || cv[2] != 0.f || cv[3] != 0.f))
            *cbits |= 1ull << ((4 * e / D::Q) % D::P);
        }
      }
    }
  } else {
#pragma unroll 4
    for (int e = threadIdx.x; e < D::RAWB / 4; e += kThreads)
      reinterpret_cast<f4*>(rB)[e] = reinterpret_cast<const f4*>(B)[e];
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
// The row map of the forward (the sparsity map of C = S o A_i, kept per row of C because
// a matrix-core K step needs the same rows j for all 16 columns k of its tile): the rows
// j of C with a nonzero entry in any rank, in order, then the all-zero rows.  Z rows and
// stage-2 K steps are taken in map order over the first TJE 16-row tiles only, TJE =
// ceil(nonzero rows / 16): the tiles beyond hold only zero rows of every C_i, whose
// products add nothing.  With every row nonzero the map is the identity and TJE = TJ.
template <class D, bool MAP>
struct FwdMap {
  static constexpr bool ON = MAP && D::FWD_RAW && D::TJ > 1 && D::P <= 64 && D::Q % 4 == 0 &&
                             (D::P * D::Q) % 4 == 0;   // (one tile: nothing to skip)
};

// X[j = map(16tj+c)][a = g*SA+s] of one row for the first TJE tiles (jr < 0: padding).
template <class D, int TJE>
__device__ __forceinline__ void load_xa_map(float (&xa)[D::TJ][D::SA], const float* xr, const int (&jr)[D::TJ],
                                            int g) {
#pragma unroll
  for (int tj = 0; tj < TJE; ++tj) {
    if (D::P % 16 == 0 || jr[tj] >= 0) {   // (a whole number of tiles has no padding rows)
      vload<D::SA>(xa[tj], xr + jr[tj] * D::M + g * D::SA);
    } else {
#pragma unroll
      for (int s = 0; s < D::SA; ++s) xa[tj][s] = 0.f;
    }
  }
}

// The row loop of the forward over the first TJE tiles of the row map.
// With SKIP, bit tj*TK + tk of tmask says whether the 16 x 16 tile (tj, tk) of C (rows in
// map order) holds a nonzero entry in any rank; stage 2 skips the K steps of the others.
template <class D, int TJE, bool SKIP, bool ZS>
__device__ __forceinline__ void fwd_rows(int64_t row, int64_t N, bool relu, const float* __restrict__ x,
                                         float* __restrict__ y, float* __restrict__ zc, const float* bop,
                                         const float* cop,
                                         float (&xa)[D::TJ][D::SA], const int (&jr)[D::TJ],
                                         const f4 (&bb)[D::TB][D::TK], int lane, int g, int c, unsigned tmask) {
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  // The next row's X is loaded at the top of each row (the last row reloads itself), and
  // a scheduling barrier keeps the compiler from sinking those loads towards their use.
  float xn[D::TJ][D::SA];
#pragma unroll
  for (int tj = 0; tj < TJE; ++tj)
#pragma unroll
    for (int s = 0; s < D::SA; ++s) asm volatile("" ::"v"(xa[tj][s]));
  for (; row < N; row += stride) {
    {
      const int64_t nr = row + stride < N ? row + stride : row;
      load_xa_map<D, TJE>(xn, x + nr * D::IN, jr, g);
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
      f4 z[TJE][D::TB];
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb) {
        float bo[D::SA];
        table_read<D::SA>(bo, bop + (i * D::TB + tb) * 64 * D::SA, lane);
#pragma unroll
        for (int tj = 0; tj < TJE; ++tj) {
          f4 t = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < D::SA; ++s) t = mfma(xa[tj][s], bo[s], t);
          z[tj][tb] = t;   // Z[j = map(16tj+4g+v)][b = 16tb+c]
          // (read back by the backward only, much later: non-temporal stores, measured 4 us
          // faster than ordinary ones at 20,000 rows)
          if (ZS && TJE == D::TJ && i < ZCache<D>::RANKS)
            __builtin_nontemporal_store(
                t, reinterpret_cast<f4*>(zc + row * ZCache<D>::ROW + i * 1024 + (tb * 2 + tj) * 256) + lane);
        }
      }
#pragma unroll
      for (int tk = 0; tk < D::TK; ++tk) {
        float co[D::SJ];
        table_read<D::SJ>(co, cop + (i * D::TK + tk) * 64 * D::SJ, lane);
#pragma unroll
        for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
          for (int tj = 0; tj < TJE; ++tj) {
            if (SKIP && !((tmask >> (tj * D::TK + tk)) & 1u)) continue;   // (uniform) all-zero tile of C
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[tb][tk] = mfma(z[tj][tb][v], co[tj * 4 + v], acc[tb][tk]);
          }
      }
    }
    // acc[tb][tk] register v = Y^T[b = 16tb+4g+v][k = 16tk+c] -> y[k*N + b]
    float* yr = y + row * D::OUT;
    if constexpr (D::N == 32 && D::Q % 16 == 0 && D::R != 1) {
      // Rows of 32 floats: lanes c and c ^ 8 swap one 16-byte piece, so that each store
      // covers eight whole 128-byte rows of y (lanes c < 8 the pieces 0-3 of row c, lanes
      // c >= 8 the pieces 4-7) instead of half of sixteen.
      const bool lo = c < 8;
#pragma unroll
      for (int tk = 0; tk < D::TK; ++tk) {
        f4 o[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          o[tb] = acc[tb][tk] + bb[tb][tk];
          if (relu) {
#pragma unroll
            for (int v = 0; v < 4; ++v) o[tb][v] = o[tb][v] > 0.f ? o[tb][v] : 0.f;
          }
        }
        const f4 send = lo ? o[1] : o[0];
        f4 recv;
#pragma unroll
        for (int v = 0; v < 4; ++v) recv[v] = __shfl_xor(send[v], 8);
        float* yk = yr + (16 * tk + (c & 7)) * 32 + (lo ? 0 : 16) + 4 * g;
        __builtin_nontemporal_store(lo ? o[0] : recv, reinterpret_cast<f4*>(yk));
        __builtin_nontemporal_store(lo ? recv : o[1], reinterpret_cast<f4*>(yk + 8 * 32));
      }
    } else {
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
          // y is not read back: non-temporal stores, except at r = 1, where a row's few
          // products leave the kernel closer to the memory bound and ordinary stores,
          // combined in L2, were measured faster (GPT-2 pair at r = 1: 31.4 -> 28.5 and
          // 29.1 -> 28.5 us; at r = 4 and at the headline shape they were 1% slower)
          if constexpr (D::R == 1)
            *reinterpret_cast<f4*>(yr + k * D::N + b0) = o;
          else
            __builtin_nontemporal_store(o, reinterpret_cast<f4*>(yr + k * D::N + b0));
        }
      }
    }
#pragma unroll
    for (int tj = 0; tj < TJE; ++tj)
#pragma unroll
      for (int s = 0; s < D::SA; ++s) xa[tj][s] = xn[tj][s];
  }
}

template <class D, int T, bool SKIP, bool ZS>
__device__ __forceinline__ void fwd_rows_tje(int tje, int64_t row, int64_t N, bool relu, const float* __restrict__ x,
                                             float* __restrict__ y, float* __restrict__ zc, const float* bop,
                                             const float* cop,
                                             float (&xa)[D::TJ][D::SA], const int (&jr)[D::TJ],
                                             const f4 (&bb)[D::TB][D::TK], int lane, int g, int c, unsigned tmask) {
  if constexpr (T >= 1) {
    if (tje == T) {
      // the tile branches only where a tile of the first T row tiles is empty (uniform)
      constexpr unsigned kFull = (T * D::TK >= 32) ? ~0u : ((1u << (T * D::TK)) - 1u);
      if (SKIP && (tmask & kFull) != kFull)
        fwd_rows<D, T, SKIP, ZS>(row, N, relu, x, y, zc, bop, cop, xa, jr, bb, lane, g, c, tmask);
      else
        fwd_rows<D, T, false, ZS>(row, N, relu, x, y, zc, bop, cop, xa, jr, bb, lane, g, c, tmask);
    } else {
      fwd_rows_tje<D, T - 1, SKIP, ZS>(tje, row, N, relu, x, y, zc, bop, cop, xa, jr, bb, lane, g, c, tmask);
    }
  }
}

// ZS: also write Z_i = X B_i of every row into the cache zc (ZCache layout).
template <class D, bool MAP, bool ZS = false>
__global__ __launch_bounds__(kThreads) void fwd_mfma_kernel(int64_t N, uint32_t flags,
                                                            const float* __restrict__ x,
                                                            const float* __restrict__ Sm,
                                                            const float* __restrict__ A,
                                                            const float* __restrict__ B,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ y, float* __restrict__ zc) {
  static_assert(!ZS || (ZCache<D>::OK && !MAP), "the cache is written by the dense forward of its shapes");
  extern __shared__ float lds[];
  float* bop = lds;              // B_i[g*SA+s][16tb+c]
  float* cop = bop + D::BOP;     // C_i[map(16tj+4g+v)][16tk+c]
  // the row map after the raw staging (kept in the dynamic block: a static LDS variable
  // would shift the dynamic block off its 16-byte alignment)
  unsigned long long* s_wmask = reinterpret_cast<unsigned long long*>(cop + D::COPF + D::RAW);  // per wavefront
  int* s_map = reinterpret_cast<int*>(s_wmask + kWaves);                                    // position -> row
  int* s_tmask = s_map + D::TJ * 16;                                                         // nonzero tiles
  if (FwdMap<D, MAP>::ON && threadIdx.x == 0) *s_tmask = 0;   // (read after the staging barrier)
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int wave = threadIdx.x >> 6;
  int64_t row = (int64_t)blockIdx.x * kWaves + wave;
  // the first row's X (identity map) is loaded while the tables are built
  int jr[D::TJ];
#pragma unroll
  for (int tj = 0; tj < D::TJ; ++tj) jr[tj] = 16 * tj + c < D::P ? 16 * tj + c : -1;
  float xa[D::TJ][D::SA];   // X[j = map(16tj+c)][a = g*SA+s]
  if (row < N) load_xa_map<D, D::TJ>(xa, x + row * D::IN, jr, g);
  // the bias is loaded with the first row, before the tables are built
  f4 bb[D::TB][D::TK];
#pragma unroll
  for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk) {
      const int k = 16 * tk + c, b0 = 16 * tb + 4 * g;
      bb[tb][tk] = (bias && k < D::Q && b0 < D::N) ? *reinterpret_cast<const f4*>(bias + k * D::N + b0)
                                                  : f4{0.f, 0.f, 0.f, 0.f};
    }
  int tje = D::TJ;
  bool remap = false;
  unsigned tmask = ~0u;
  if constexpr (D::FWD_RAW) {
    float* rB = cop + D::COPF;
    float* rC = rB + D::RAWB;
    // the staged C also gives the sparsity map: the rows of C with a nonzero entry in
    // any rank (a bit per row, ORed over each wavefront, then over the wavefronts)
    unsigned long long bits = 0;
    stage_raw<D>(rB, rC, B, Sm, A, FwdMap<D, MAP>::ON ? &bits : nullptr);
    if constexpr (FwdMap<D, MAP>::ON) {
      unsigned long long wbits = 0;   // the wavefront's OR, one ballot per row
#pragma unroll
      for (int j = 0; j < D::P; ++j)
        if (__ballot((bits >> j) & 1)) wbits |= 1ull << j;
      if (lane == 0) s_wmask[wave] = wbits;
    }
    __syncthreads();
    build_table<D::R, D::TB, D::SA>(bop, [&](int i, int tb, int g, int c, int s) {
      return rawB<D>(rB, i, g * D::SA + s, 16 * tb + c);
    });
    if constexpr (FwdMap<D, MAP>::ON) {
      unsigned long long m64 = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) m64 |= s_wmask[w];
      // the same in every lane: made scalar
      const unsigned long long mask =
          (unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)m64) |
          ((unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(m64 >> 32)) << 32);
      const int nnz = __popcll(mask);
      tje = nnz == 0 ? 1 : (nnz + 15) / 16;
      // nonzero rows not a prefix: compact them to the front
      remap = mask != (nnz == 64 ? ~0ull : (1ull << nnz) - 1);
      if (remap) {
        if (threadIdx.x < D::P) {
          const int jj = threadIdx.x;
          const int before = __popcll(mask & ((1ull << jj) - 1));
          s_map[(mask >> jj) & 1 ? before : nnz + (jj - before)] = jj;
        }
        __syncthreads();
      }
      // the tile mask: which 16 x 16 tiles of S, rows in map order, hold a nonzero entry (a
      // zero tile of S is a zero tile of every C_i; per output block-column tk, the row tiles
      // its sum runs over).  Without S nothing is skipped.
      static_assert(D::TJ * D::TK <= 32, "one bit per tile");
      if (Sm) {
        unsigned tm = 0;
        constexpr int QV = D::Q / 4;   // 4-float pieces per row of S
        for (int e = threadIdx.x; e < D::P * QV; e += kThreads) {
          const int p = e / QV, k0 = 4 * (e % QV);
          const f4 sv = *reinterpret_cast<const f4*>(Sm + (remap ? s_map[p] : p) * D::Q + k0);
          if (sv[0] != 0.f || sv[1] != 0.f || sv[2] != 0.f || sv[3] != 0.f) tm |= 1u << ((p >> 4) * D::TK + (k0 >> 4));
        }
        if (tm) atomicOr(s_tmask, (int)tm);
        __syncthreads();
        tmask = (unsigned)__builtin_amdgcn_readfirstlane(*s_tmask);
      }
    }
    if (FwdMap<D, MAP>::ON && remap) {
      build_table<D::R, D::TK, D::SJ>(cop, [&](int i, int tk, int g, int c, int sv) {
        const int jp = 16 * (sv / 4) + 4 * g + (sv % 4);
        return jp < D::P ? rawC<D>(rC, i, s_map[jp], 16 * tk + c) : 0.f;
      });
#pragma unroll
      for (int tj = 0; tj < D::TJ; ++tj) jr[tj] = 16 * tj + c < D::P ? s_map[16 * tj + c] : -1;
      // the first row's X again, through the map
      if (row < N) load_xa_map<D, D::TJ>(xa, x + row * D::IN, jr, g);
    } else {
      build_table<D::R, D::TK, D::SJ>(cop, [&](int i, int tk, int g, int c, int sv) {
        return rawC<D>(rC, i, 16 * (sv / 4) + 4 * g + (sv % 4), 16 * tk + c);
      });
    }
  } else if constexpr (D::FWD_RAW1) {
    // One rank at a time: B_i and C_i = S o A_i staged with 16-byte loads, then that rank's
    // slices of the tables built from LDS (the tables are rank-major).
    float* rB = cop + D::COPF;
    float* rC = rB + D::M * D::N;
    constexpr int NB4 = D::M * D::N / 4, NC4 = D::P * D::Q / 4;
    constexpr int KB = (NB4 + kThreads - 1) / kThreads, KC = (NC4 + kThreads - 1) / kThreads;
    const f4* S4 = reinterpret_cast<const f4*>(Sm ? Sm : A);   // (A stands in without S)
    for (int i = 0; i < D::R; ++i) {
      const f4* B4 = reinterpret_cast<const f4*>(B + i * D::M * D::N);
      const f4* A4 = reinterpret_cast<const f4*>(A + i * D::P * D::Q);
      f4 b[KB], a[KC], m[KC];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int e = threadIdx.x + k * kThreads;
        if (NB4 % kThreads == 0 || e < NB4) b[k] = B4[e];
      }
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const int e = threadIdx.x + k * kThreads;
        if (NC4 % kThreads == 0 || e < NC4) {
          a[k] = A4[e];
          m[k] = S4[e];
        }
      }
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int e = threadIdx.x + k * kThreads;
        if (NB4 % kThreads == 0 || e < NB4) reinterpret_cast<f4*>(rB)[e] = b[k];
      }
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const int e = threadIdx.x + k * kThreads;
        if (NC4 % kThreads == 0 || e < NC4) reinterpret_cast<f4*>(rC)[e] = Sm ? a[k] * m[k] : a[k];
      }
      __syncthreads();
      build_table<1, D::TB, D::SA>(bop + i * D::TB * 64 * D::SA, [&](int, int tb, int g, int c, int s) {
        return rawB<D>(rB, 0, g * D::SA + s, 16 * tb + c);
      });
      build_table<1, D::TK, D::SJ>(cop + i * D::TK * 64 * D::SJ, [&](int, int tk, int g, int c, int sv) {
        return rawC<D>(rC, 0, 16 * (sv / 4) + 4 * g + (sv % 4), 16 * tk + c);
      });
      __syncthreads();   // the staging area is reused by the next rank
    }
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
  fwd_rows_tje<D, D::TJ, FwdMap<D, MAP>::ON, ZS>(tje, row, N, (flags & KRON_RELU_OUT) != 0, x, y, zc, bop, cop, xa,
                                                 jr, bb, lane, g, c, tmask);
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
  // BWD_TILED: the next row's x and dY in registers as 16-byte pieces, staged in this
  // wavefront's LDS tiles at the end of a row and read back as the row operands
  float* xt = lds + D::BWD_MAIN + (threadIdx.x >> 6) * (D::TXT + D::TYT);
  float* yt = xt + D::TXT;
  f4 sx[D::NXF], sy[D::NYF];
  auto fetch_t = [&](int64_t r) {
    const int ln = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < D::NXF; ++t) {
      const int f = 64 * t + ln;
      if (D::IN % 256 == 0 || f < D::IN / 4) sx[t] = *reinterpret_cast<const f4*>(x + r * D::IN + 4 * f);
    }
#pragma unroll
    for (int t = 0; t < D::NYF; ++t) {
      const int f = 64 * t + ln;
      if (D::OUT % 256 == 0 || f < D::OUT / 4) sy[t] = *reinterpret_cast<const f4*>(dy + r * D::OUT + 4 * f);
    }
  };
  auto stage_t = [&]() {
    const int ln = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < D::NXF; ++t) {
      const int f = 64 * t + ln, e = 4 * f;
      if (D::IN % 256 == 0 || f < D::IN / 4) *reinterpret_cast<f4*>(xt + (e / D::M) * D::TLX + e % D::M) = sx[t];
    }
#pragma unroll
    for (int t = 0; t < D::NYF; ++t) {
      const int f = 64 * t + ln, e = 4 * f;
      if (D::OUT % 256 == 0 || f < D::OUT / 4) *reinterpret_cast<f4*>(yt + (e / D::N) * D::TLY + e % D::N) = sy[t];
    }
  };
  auto rd_ops_t = [&](BwdRow<D>& o, int g, int c) {
#pragma unroll
    for (int tj = 0; tj < D::TJ; ++tj) {
      const int j = 16 * tj + c;
      if (j < D::P) {
        vload<D::SA>(o.xa[tj], xt + j * D::TLX + g * D::SA);
      } else {
#pragma unroll
        for (int s = 0; s < D::SA; ++s) o.xa[tj][s] = 0.f;
      }
    }
#pragma unroll
    for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
      for (int s = 0; s < D::SJ; ++s) {
        const int j = g * D::SJ + s, a = 16 * ta + c;
        o.xaj[ta][s] = (j < D::P && a < D::M) ? xt[j * D::TLX + a] : 0.f;
      }
#pragma unroll
    for (int tk = 0; tk < D::TK; ++tk)
#pragma unroll
      for (int tb = 0; tb < D::TB; ++tb) {
        const int k = 16 * tk + c, b0 = 16 * tb + 4 * g;
        o.dyk[tk][tb] = (k < D::Q && b0 < D::N) ? *reinterpret_cast<const f4*>(yt + k * D::TLY + b0)
                                               : f4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int tb = 0; tb < D::TB; ++tb)
#pragma unroll
      for (int s = 0; s < D::SK; ++s) {
        const int k = 4 * s + g, b = 16 * tb + c;
        o.dyb[tb][s] = (k < D::Q && b < D::N) ? yt[k * D::TLY + b] : 0.f;
      }
  };
  if constexpr (D::BWD_TILED) {
    const int64_t row0 = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row0 < N) fetch_t(row0);
  } else if constexpr (D::BWD_PREFETCH) {
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
  BwdRow<D> cur;
  if constexpr (D::BWD_TILED) {
    if (row < N) {
      stage_t();
      rd_ops_t(cur, g, c);
    }
  } else if constexpr (D::BWD_PREFETCH) {
    settle(nx.xa);
    settle(nx.xaj);
    settle(nx.dyk);
    settle(nx.dyb);
  }
  for (; row < N; row += stride) {
    const float* xr = x + row * D::IN;
    if constexpr (D::BWD_TILED) {
      fetch_t(row + stride < N ? row + stride : row);
    } else if constexpr (D::BWD_PREFETCH) {
      cur = nx;
      if (row + stride < N) load_bwd_row<D>(nx, x + (row + stride) * D::IN, dy + (row + stride) * D::OUT, g, c);
    } else {
      load_bwd_row<D>(cur, xr, dy + row * D::OUT, g, c);
    }
    const auto& xa = cur.xa;
    const auto& xaj = cur.xaj;
    const auto& dyk = cur.dyk;
    const auto& dyb = cur.dyb;
    // x under this lane's dX entries for the ReLU mask, requested now so that the row's
    // products cover the load (read at the end, it leaves the load's latency exposed per
    // row), where the registers allow
    constexpr bool EARLY_MASK = D::BWD_REGS + 4 * D::TA * D::TJ <= 300;
    f4 xm[D::TA][D::TJ];
    if (EARLY_MASK && want_dx && mask) {
#pragma unroll
      for (int ta = 0; ta < D::TA; ++ta)
#pragma unroll
        for (int tj = 0; tj < D::TJ; ++tj) {
          const int j = 16 * tj + c, a0 = 16 * ta + 4 * g;
          xm[ta][tj] = (j < D::P && a0 < D::M)
                           ? *reinterpret_cast<const f4*>(D::BWD_TILED ? xt + j * D::TLX + a0 : xr + j * D::M + a0)
                           : f4{0.f, 0.f, 0.f, 0.f};
        }
    }
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
              const f4 xv = EARLY_MASK ? xm[ta][tj]
                                       : *reinterpret_cast<const f4*>(D::BWD_TILED ? xt + j * D::TLX + a0
                                                                                   : xr + j * D::M + a0);
#pragma unroll
              for (int v = 0; v < 4; ++v) o[v] = xv[v] > 0.f ? o[v] : 0.f;
            }
            __builtin_nontemporal_store(o, reinterpret_cast<f4*>(dxr + j * D::M + a0));
          }
        }
    }
    if constexpr (D::BWD_TILED) {
      // the next row into the tiles (this row's reads of them are done) and its operands
      __builtin_amdgcn_wave_barrier();
      stage_t();
      __builtin_amdgcn_wave_barrier();
      rd_ops_t(cur, g, c);
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
  static constexpr int COMBINE = RPI * D::PWW;
  static constexpr int STEPW = ROWBUF + 4 * WREG;
  // the work area stages B and then C (two passes), or both at once when that still
  // leaves room for the same number of workgroups per compute unit
  static constexpr int WORK2 = STEPW > RAWMAX ? STEPW : RAWMAX;
  static constexpr int WORK1 = STEPW > D::RAWB + D::RAWC ? STEPW : D::RAWB + D::RAWC;
  static constexpr size_t lds_of(int work) {
    return (size_t)((TABLES + work) > COMBINE ? (TABLES + work) : COMBINE) * 4;
  }
  // workgroups per compute unit: two when their LDS fits twice (two wavefronts per SIMD),
  // else one (one wavefront per SIMD, with the whole register file)
  static constexpr int WPC = lds_of(WORK2) * 2 <= kMaxLds ? 2 : 1;
  static constexpr bool ONE_PASS = lds_of(WORK1) * WPC <= kMaxLds;
  static constexpr int WORK = ONE_PASS ? WORK1 : WORK2;
  static constexpr int MAIN = TABLES + WORK;
  static constexpr size_t LDS = lds_of(WORK);
  // padded row entries are read (and must stay zero) unless every dimension is a
  // multiple of 16
  static constexpr bool PADDED = D::P % 16 != 0 || D::Q % 16 != 0 || D::M % 16 != 0 || D::N % 16 != 0;
  static constexpr int NF4 = ROWBUF / SLOT * (D::IN + D::OUT) / 4;   // float4s staged per step
  static constexpr int NPF = (NF4 + kThreads - 1) / kThreads;
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

  if constexpr (Q::ONE_PASS) {
    // operand tables from B and C staged together (one memory round trip)
    float* rB = work;
    float* rC = work + D::RAWB;
    stage_raw<D>(rB, rC, B, Sm, A);
    __syncthreads();
    build_table<D::R, D::TB, D::SA>(bop, [&](int i, int tb, int gg, int cc, int s) {
      return rawB<D>(rB, i, gg * D::SA + s, 16 * tb + cc);
    });
    build_table<D::R, D::TA, D::TB * 4>(bopx, [&](int i, int ta, int gg, int cc, int sv) {
      return rawB<D>(rB, i, 16 * ta + cc, 16 * (sv / 4) + 4 * gg + (sv % 4));
    });
    build_table<D::R, D::TJ, Q::SKP>(copg, [&](int i, int tj, int gg, int cc, int s) {
      return rawC<D>(rC, i, 16 * tj + cc, kidx(s, gg));
    });
    __syncthreads();
  } else {
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
  }
  if constexpr (Q::PADDED || !Q::ONE_PASS) {
    for (int e = tid; e < Q::ROWBUF; e += kThreads) rowbuf[e] = 0.f;   // padding stays zero
    __syncthreads();
  }

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
        __builtin_nontemporal_store(acc, reinterpret_cast<f4*>(dx + row * D::IN + o));
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

// ---------------------------------------------------------------------------------
// Whole-row backward ("solo") for the 32 x 32 factor blocks (p = q = m = n = 32, r <= 4).
// One wavefront per SIMD: a workgroup of four wavefronts per compute unit, each
// wavefront owning whole rows and every rank of them, so the row loop has no barrier and
// no exchange between wavefronts.  Per row and rank i:
//   Z^T = B_i^T X^T,  G^T = dY^T C_i^T,  dC_i += Z dY^T,  dX^T += B_i G^T,  dB_i += X^T G,
// with dX accumulated over the ranks in registers and stored once.  The ranks' operand
// tables (B_i in two lane orders, C_i) are in LDS, read one rank ahead and cyclically
// into the next row.  Each wavefront's LDS tiles stage its next row: the row's global
// loads are issued at the top of the row, written to the tiles once the current row's
// operands have been read from them, and the next row's operands (row- and column-order
// reads of X and dY) are read back after the last rank.  G takes one trip through a
// per-wavefront tile to swap its indices for dB.  The row loop keeps the matrix cores
// about 88% busy at the full shader clock.
// ---------------------------------------------------------------------------------
template <class D>
struct Solo {
  static constexpr int R = D::R;
  static constexpr bool OK = D::P == 32 && D::Q == 32 && D::M == 32 && D::N == 32 && R <= 4;
  static constexpr int L = 36;               // pitch of a 32-float row in the tiles
  static constexpr int TILE = 32 * L;
  static constexpr int TAB = R * 1024;       // one table: [rank][tile 2][chunk 2][lane][4]
  static constexpr int WSP = 3 * TILE;       // per wavefront: X tile, dY tile, G tile
  static constexpr int MAIN = 3 * TAB + kWaves * WSP;
  static constexpr int RW = 2 * R * 1024 + 1024;   // per wavefront at the end: dB | dC | dbias
  static constexpr int COMBINE = kWaves * RW;
  // the row map (KRON_SPARSE_ROWS): a word of row bits per wavefront, position -> row and
  // row -> position, after the tables and tiles
  static constexpr int MAPW = kWaves + 64;
  static constexpr size_t LDS = (size_t)(MAIN + MAPW > COMBINE ? MAIN + MAPW : COMBINE) * 4;
  static_assert(!OK || 2 * R * 1024 <= kWaves * WSP, "raw factors are staged in the tile area");
};

__device__ __forceinline__ int kxs(int s, int g) { return 16 * (s >> 2) + 4 * g + (s & 3); }

// DXM as for bwd_rp_kernel: 0 = no dX, 1 = dX, 2 = dX masked by [x > 0], 3 = dX added to
// dx, 4 = dX added to dx and the sum masked.
// MAP (KRON_SPARSE_ROWS): the rows j of C with a nonzero entry in any rank are compacted to
// the front of the tiles (the X tile is staged in that order and the C table built in it),
// and when they fit one 16-row tile the products that run over them -- G = C dY, dX and
// dB -- take that tile only: G, dX and the dB terms of the other rows are zero.  Z and dC
// stay dense (dS needs dC at every entry); dX and dC are written back in row order.
// ZC: Z_i = X B_i of the ranks i < ZR = ZCache<D>::RANKS is read from the forward's cache
// zc instead of being recomputed.  Register slot k holds rank k of the current row; the
// next row's rank k is requested at the top of rank k + R - ZR of this one (a recomputed
// rank: ZR <= R / 2).
template <class D, int DXM, bool MAP = false, bool ZC = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_solo_kernel(int64_t N, const float* __restrict__ x, const float* __restrict__ Sm,
                     const float* __restrict__ A, const float* __restrict__ B, const float* __restrict__ dy,
                     float* __restrict__ dx, float* __restrict__ part, const float* __restrict__ zc) {
  using SL = Solo<D>;
  static_assert(!ZC || (ZCache<D>::OK && !MAP && DXM <= 2), "the cached backward is dense, without dx accumulation");
  constexpr int R = D::R, L = SL::L, TILE = SL::TILE;
  extern __shared__ float lds[];
  float* tabB = lds;                 // B_i[8g+s][16t+c]                 (A operand of Z^T)
  float* tabC = lds + SL::TAB;       // C_i[16t+c][kxs(s,g)]             (B operand of G^T)
  float* tabX = lds + 2 * SL::TAB;   // B_i[16t+c][16(s>>2)+4g+(s&3)]    (A operand of dX^T)
  float* wsp = lds + 3 * SL::TAB;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15, w = tid >> 6;
  float* xt = wsp + w * SL::WSP;
  float* yt = xt + TILE;
  float* gs = yt + TILE;
  int* s_wrows = reinterpret_cast<int*>(lds + SL::MAIN);   // [wavefront] row bits
  int* s_map = s_wrows + kWaves;                            // position -> row
  int* s_inv = s_map + 32;                                  // row -> position
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  int64_t row = (int64_t)blockIdx.x * kWaves + w;

  // this lane's pieces of a row (float4 index 64t + lane), placed so that each 16-lane
  // group writes rows j and j + 8 of a tile (no bank conflicts)
  int soff[4], goff[4], soffx[4];   // (soffx: the X tile's, which follows the row map)
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int f = 64 * t + lane, q = f & 15, g16 = f >> 4;
    const int pj = (g16 & 7) + 16 * (g16 >> 3) + 8 * (q >> 3), pa = 4 * (q & 7);
    soff[t] = pj * L + pa;
    goff[t] = pj * 32 + pa;
    soffx[t] = soff[t];
  }
  f4 sx[4], sy[4];
  auto fetch = [&](int64_t r) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sx[t] = *reinterpret_cast<const f4*>(x + r * D::IN + goff[t]);
      sy[t] = *reinterpret_cast<const f4*>(dy + r * D::OUT + goff[t]);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      *reinterpret_cast<f4*>(xt + (MAP ? soffx[t] : soff[t])) = sx[t];
      *reinterpret_cast<f4*>(yt + soff[t]) = sy[t];
    }
  };
  // the row map: tiles of rows run by G, dX and dB, whether rows moved, and where this
  // lane's dX rows go
  int tje = 2;
  bool remap = false;
  int dxrow[2] = {c, 16 + c};
  if (row < N) fetch(row);
  {
    // tables: B and C = S o A staged raw in the tile area, then laid out per lane
    float* rB = wsp;
    float* rC = wsp + R * 1024;
    f4 b[R], a[R], m[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      b[k] = reinterpret_cast<const f4*>(B)[tid + kThreads * k];
      a[k] = reinterpret_cast<const f4*>(A)[tid + kThreads * k];
      m[k] = Sm ? reinterpret_cast<const f4*>(Sm)[tid] : f4{1.f, 1.f, 1.f, 1.f};
    }
    bool nz = false;   // this thread's C values all lie in row tid / 8 (every rank)
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const f4 cv = a[k] * m[k];
      reinterpret_cast<f4*>(rB)[tid + kThreads * k] = b[k];
      reinterpret_cast<f4*>(rC)[tid + kThreads * k] = cv;
      nz |= cv[0] != 0.f || cv[1] != 0.f || cv[2] != 0.f || cv[3] != 0.f;
    }
    if constexpr (MAP) {
      // rows 8w .. 8w+7: one bit each, from the ballot of the wavefront's 8-lane groups
      const unsigned long long bal = __ballot(nz);
      int bits = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) bits |= ((bal >> (8 * q)) & 0xffull) ? 1 << q : 0;
      if (lane == 0) s_wrows[w] = bits;
    }
    __syncthreads();
    if constexpr (MAP) {
      int m32 = 0;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) m32 |= s_wrows[q] << (8 * q);
      const uint32_t mask = (uint32_t)__builtin_amdgcn_readfirstlane(m32);
      const int nnz = __popc(mask);
      tje = nnz <= 16 ? 1 : 2;
      remap = mask != (nnz == 32 ? 0xffffffffu : (1u << nnz) - 1);
      if (remap) {   // nonzero rows not a prefix: compact them to the front (uniform branch)
        if (tid < 32) {
          const int before = __popc(mask & ((1u << tid) - 1));
          const int pos = (mask >> tid) & 1 ? before : nnz + (tid - before);
          s_map[pos] = tid;
          s_inv[tid] = pos;
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int f = 64 * t + lane, q = f & 15, g16 = f >> 4;
          const int pj = (g16 & 7) + 16 * (g16 >> 3) + 8 * (q >> 3), pa = 4 * (q & 7);
          soffx[t] = s_inv[pj] * L + pa;
        }
#pragma unroll
        for (int tj = 0; tj < 2; ++tj) dxrow[tj] = s_map[16 * tj + c];
      }
    }
#pragma unroll
    for (int it = 0; it < 4 * R; ++it) {
      const int e = tid + kThreads * it;
      const int v = e & 3, l = (e >> 2) & 63, ch = (e >> 8) & 1, tl = (e >> 9) & 1, i = e >> 10;
      const int gg = l >> 4, cc = l & 15, s = 4 * ch + v;
      tabB[e] = rB[(i * 32 + 8 * gg + s) * 32 + 16 * tl + cc];
      const int jc = (MAP && remap) ? s_map[16 * tl + cc] : 16 * tl + cc;
      tabC[e] = rC[(i * 32 + jc) * 32 + kxs(s, gg)];
      tabX[e] = rB[(i * 32 + 16 * tl + cc) * 32 + 16 * (s >> 2) + 4 * gg + (s & 3)];
    }
    __syncthreads();
  }
  auto rd_tab = [&](float (&d)[2][8], const float* t, int i) {
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        const f4 v = reinterpret_cast<const f4*>(t)[((i * 2 + tl) * 2 + ch) * 64 + lane];
        d[tl][4 * ch] = v[0]; d[tl][4 * ch + 1] = v[1]; d[tl][4 * ch + 2] = v[2]; d[tl][4 * ch + 3] = v[3];
      }
  };
  float xa[2][8], xaj[2][8], dyb[2][8];   // X[16t+c][8g+s], X[kxs][16t+c], dY[kxs][16t+c]
  f4 dyk[2][2];                           // dY[16tk+c][16tb+4g..]
  auto rd_ops = [&]() {
    if constexpr (!ZC || ZCache<D>::RANKS < R) {   // (X's row-order operand only feeds the recomputation of Z)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const f4 v = *reinterpret_cast<const f4*>(xt + (16 * tj + c) * L + 8 * g + 4 * t);
          xa[tj][4 * t] = v[0]; xa[tj][4 * t + 1] = v[1]; xa[tj][4 * t + 2] = v[2]; xa[tj][4 * t + 3] = v[3];
        }
    }
#pragma unroll
    for (int tk = 0; tk < 2; ++tk)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) dyk[tk][tb] = *reinterpret_cast<const f4*>(yt + (16 * tk + c) * L + 16 * tb + 4 * g);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        xaj[t][s] = xt[kxs(s, g) * L + 16 * t + c];
        dyb[t][s] = yt[kxs(s, g) * L + 16 * t + c];
      }
  };
  f4 dC[R][2][2], dB[R][2][2], db[2][2];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 2; ++v) { dC[i][u][v] = f4{0.f, 0.f, 0.f, 0.f}; dB[i][u][v] = f4{0.f, 0.f, 0.f, 0.f}; }
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v) db[u][v] = f4{0.f, 0.f, 0.f, 0.f};
  float bo[2][8], co[2][8], bx[2][8];
  if (row < N) {
    stage();
    rd_ops();
  }
  if constexpr (!ZC) rd_tab(bo, tabB, 0);   // (the saved path reads it with its ranks)
  rd_tab(co, tabC, 0);
  if constexpr (DXM != 0) rd_tab(bx, tabX, 0);
  f4 zs[R][2][2];   // the cached Z of the saved ranks
  // Z^T[16tb+4g+v][16tj+c] = Z[16tj+c][16tb+4g+v] is slot c & 3 of the forward's lane
  // 16(c >> 2) + 4g + v
  auto zload = [&](f4 (&d)[2][2], int64_t r, int i) {
    const float* zp = zc + r * ZCache<D>::ROW + i * 1024 + 64 * (c >> 2) + 16 * g + (c & 3);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
#pragma unroll
        for (int v = 0; v < 4; ++v) d[tb][tj][v] = zp[(tb * 2 + tj) * 256 + 4 * v];
  };
  // The row loop, instantiated per count of 16-row tiles that G, dX and dB run over (two
  // without the row map).
  auto rows = [&](auto tiles, auto zranks) {
    constexpr int TJE_ = decltype(tiles)::value;
    constexpr int ZR = decltype(zranks)::value;
    // the first row's saved ranks (a wavefront without rows reads the last row, unused),
    // and rank 0's B table when rank 0 is recomputed
    if constexpr (ZR > 0) {
      // in rank order, as the row loop requests them: the compiler derives the loop's
      // memory waits from both paths into it, and with rank 1 issued first it waited for
      // rank 1 and the last row's dX stores before rank 0's first product
      const int64_t r0 = row < N ? row : N - 1;
  #pragma unroll
      for (int k = 0; k < ZR; ++k) {
        zload(zs[k], r0, k);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (ZC && ZR == 0) rd_tab(bo, tabB, 0);
    for (; row < N; row += stride) {
      const int64_t nrow = row + stride < N ? row + stride : row;
      fetch(nrow);
      f4 xm[2][2], dold[2][2];   // x under this lane's dX entries (mask), dx already there
      if constexpr (DXM == 2 || DXM == 4) {
  #pragma unroll
        for (int ta = 0; ta < 2; ++ta)
  #pragma unroll
          for (int tj = 0; tj < 2; ++tj) xm[ta][tj] = *reinterpret_cast<const f4*>(xt + (16 * tj + c) * L + 16 * ta + 4 * g);
      }
      if constexpr (DXM >= 3) {
  #pragma unroll
        for (int ta = 0; ta < 2; ++ta)
  #pragma unroll
          for (int tj = 0; tj < 2; ++tj)
            dold[ta][tj] = *reinterpret_cast<const f4*>(dx + row * D::IN + dxrow[tj] * 32 + 16 * ta + 4 * g);
      }
  #pragma unroll
      for (int tk = 0; tk < 2; ++tk)
  #pragma unroll
        for (int tb = 0; tb < 2; ++tb) db[tk][tb] += dyk[tk][tb];
      f4 dxt[2][2];   // dX^T[16ta+4g+v][16tj+c]
  #pragma unroll
      for (int u = 0; u < 2; ++u)
  #pragma unroll
        for (int v = 0; v < 2; ++v) dxt[u][v] = f4{0.f, 0.f, 0.f, 0.f};
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int i = 0; i < R; ++i) {
        f4 zt[2][2];   // Z^T[16tb+4g+v][16tj+c]
        if (i < ZR) {
  #pragma unroll
          for (int tb = 0; tb < 2; ++tb)
  #pragma unroll
            for (int tj = 0; tj < 2; ++tj) zt[tb][tj] = zs[i][tb][tj];
        } else {
          // the next row's saved rank i - (R - ZR), into the slot it takes there, requested
          // before this rank's products (measured 0.6 us faster than after its dC products)
          if (ZR > 0 && i >= R - ZR) zload(zs[i - (R - ZR)], nrow, i - (R - ZR));
  #pragma unroll
          for (int tb = 0; tb < 2; ++tb)
  #pragma unroll
            for (int tj = 0; tj < 2; ++tj) {
              f4 t = f4{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
              for (int s = 0; s < 8; ++s) t = mfma(bo[tb][s], xa[tj][s], t);
              zt[tb][tj] = t;
            }
        }
        f4 gt[2][2];   // G^T[16tb+4g+v][16tj+c]
  #pragma unroll
        for (int tj = 0; tj < 2; ++tj)
  #pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            f4 t = f4{0.f, 0.f, 0.f, 0.f};
            if (TJE_ == 2 || tj < TJE_) {
  #pragma unroll
              for (int s = 0; s < 8; ++s) t = mfma(dyb[tb][s], co[tj][s], t);
            }
            gt[tb][tj] = t;
          }
        // the next rank's tables (the last rank reads rank 0 for the next row)
        float bo2[2][8], co2[2][8];
        if ((i + 1) % R >= ZR) rd_tab(bo2, tabB, (i + 1) % R);
        rd_tab(co2, tabC, (i + 1) % R);
        __builtin_amdgcn_sched_barrier(0);
        // dC_i[16tj+4g+v][16tk+c] += sum_b Z[j][b] dY[k][b]
  #pragma unroll
        for (int tj = 0; tj < 2; ++tj)
  #pragma unroll
          for (int tk = 0; tk < 2; ++tk)
  #pragma unroll
            for (int tb = 0; tb < 2; ++tb)
  #pragma unroll
              for (int v = 0; v < 4; ++v) dC[i][tj][tk] = mfma(zt[tb][tj][v], dyk[tk][tb][v], dC[i][tj][tk]);
        // G as gs[j][b], read back in column order for dB
  #pragma unroll
        for (int tb = 0; tb < 2; ++tb)
  #pragma unroll
          for (int tj = 0; tj < 2; ++tj)
            if (TJE_ == 2 || tj < TJE_) *reinterpret_cast<f4*>(gs + (16 * tj + c) * L + 16 * tb + 4 * g) = gt[tb][tj];
        float gcol[2][8];   // G[kxs][16tb+c]
  #pragma unroll
        for (int tb = 0; tb < 2; ++tb)
  #pragma unroll
          for (int s = 0; s < 8; ++s) gcol[tb][s] = (TJE_ == 2 || s < 4 * TJE_) ? gs[kxs(s, g) * L + 16 * tb + c] : 0.f;
        __builtin_amdgcn_sched_barrier(0);
        float bx2[2][8];
        if constexpr (DXM != 0) {
          // dX^T[a][j] += sum_b B_i[a][b] G^T[b][j]
  #pragma unroll
          for (int ta = 0; ta < 2; ++ta)
  #pragma unroll
            for (int tj = 0; tj < 2; ++tj)
              if (TJE_ == 2 || tj < TJE_) {
  #pragma unroll
                for (int tb = 0; tb < 2; ++tb)
  #pragma unroll
                  for (int v = 0; v < 4; ++v) dxt[ta][tj] = mfma(bx[ta][tb * 4 + v], gt[tb][tj][v], dxt[ta][tj]);
              }
          rd_tab(bx2, tabX, (i + 1) % R);
        }
        if (i == 0) stage();   // the next row into the tiles: this row's reads of them are done
        __builtin_amdgcn_sched_barrier(0);
        // dB_i[16ta+4g+v][16tb+c] += sum_j X[j][a] G[j][b]
  #pragma unroll
        for (int ta = 0; ta < 2; ++ta)
  #pragma unroll
          for (int tb = 0; tb < 2; ++tb)
  #pragma unroll
            for (int s = 0; s < 8; ++s)
              if (TJE_ == 2 || s < 4 * TJE_) dB[i][ta][tb] = mfma(xaj[ta][s], gcol[tb][s], dB[i][ta][tb]);
        if (i == R - 1) rd_ops();   // the next row's operands from the tiles
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int u = 0; u < 2; ++u)
  #pragma unroll
          for (int v = 0; v < 8; ++v) {
            if ((i + 1) % R >= ZR) bo[u][v] = bo2[u][v];
            co[u][v] = co2[u][v];
            if constexpr (DXM != 0) bx[u][v] = bx2[u][v];
          }
      }
      if constexpr (DXM != 0) {
        float* dxr = dx + row * D::IN;
        f4 o[2][2];
  #pragma unroll
        for (int ta = 0; ta < 2; ++ta)
  #pragma unroll
          for (int tj = 0; tj < 2; ++tj) {
            o[ta][tj] = dxt[ta][tj];
            if constexpr (DXM >= 3) o[ta][tj] += dold[ta][tj];
            if constexpr (DXM == 2 || DXM == 4) {
  #pragma unroll
              for (int v = 0; v < 4; ++v) o[ta][tj][v] = xm[ta][tj][v] > 0.f ? o[ta][tj][v] : 0.f;
            }
          }
  #pragma unroll
          for (int ta = 0; ta < 2; ++ta)
  #pragma unroll
            for (int tj = 0; tj < 2; ++tj)
              __builtin_nontemporal_store(o[ta][tj], reinterpret_cast<f4*>(dxr + dxrow[tj] * 32 + 16 * ta + 4 * g));
      }
    }
  };
  if constexpr (ZC) {
    rows(std::integral_constant<int, 2>{}, std::integral_constant<int, ZCache<D>::RANKS>{});
  } else if (MAP && tje == 1) {
    rows(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
  } else {
    rows(std::integral_constant<int, 2>{}, std::integral_constant<int, 0>{});
  }
  // Partial row of this workgroup: [dB (R*M*N) | dA (R*P*Q) | dS (P*Q) | dbias (Q*N)],
  // the four wavefronts added in wavefront order.  dC's rows go back to row order (the
  // map is read before the combine area overwrites it).
  int dcrow[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) dcrow[u][v] = (MAP && remap) ? s_map[16 * u + 4 * g + v] : 16 * u + 4 * g + v;
  __syncthreads();
  float* red = lds + w * SL::RW;   // [dB | dC | dbias] of this wavefront
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          red[i * 1024 + (16 * u + 4 * g + v) * 32 + 16 * t + c] = dB[i][u][t][v];
          red[R * 1024 + i * 1024 + dcrow[u][v] * 32 + 16 * t + c] = dC[i][u][t][v];
        }
#pragma unroll
  for (int tk = 0; tk < 2; ++tk)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) *reinterpret_cast<f4*>(red + 2 * R * 1024 + (16 * tk + c) * 32 + 16 * tb + 4 * g) = db[tk][tb];
  __syncthreads();
  auto wsum = [&](int e) {
    f4 t = *reinterpret_cast<const f4*>(lds + e);
#pragma unroll
    for (int v = 1; v < kWaves; ++v) t += *reinterpret_cast<const f4*>(lds + v * SL::RW + e);
    return t;
  };
  const int64_t G = gridDim.x, gb = blockIdx.x;
  auto store = [&](int col, f4 v) { *reinterpret_cast<f4*>(part + part_index(G, gb, col)) = v; };
#pragma unroll
  for (int k = 0; k < R; ++k) store(4 * (tid + kThreads * k), wsum(4 * (tid + kThreads * k)));
  {
    const int e = 4 * tid;
    const f4 sv = Sm ? *reinterpret_cast<const f4*>(Sm + e) : f4{1.f, 1.f, 1.f, 1.f};
    f4 ds = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const f4 d = wsum(R * 1024 + i * 1024 + e);
      store(R * 1024 + i * 1024 + e, sv * d);
      ds += *reinterpret_cast<const f4*>(A + i * 1024 + e) * d;
    }
    store(2 * R * 1024 + e, Sm ? ds : f4{0.f, 0.f, 0.f, 0.f});
    store(2 * R * 1024 + 1024 + e, wsum(2 * R * 1024 + e));
  }
}

#endif  // backward kernels

// ---------------------------------------------------------------------------------
// Shape table.
// ---------------------------------------------------------------------------------
struct Entry {
  int p, q, m, n, r;
  bool fwd_ok, bwd_ok;
  int bwd_kind;        // backward kernel that runs: 0 bwd_mfma, 1 rank-parallel, 2 whole-row
  int rows_per_step;   // rows a workgroup takes per step of its row loop
  int per_cu;          // backward workgroups per compute unit
  int zc_row;          // floats per row of the saved Z (0: no saved path; whole-row kernel only)
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
template <class D, bool MAP, bool ZS = false>
void run_fwd_map(const LayerArgs& a, int max_grid, hipStream_t s) {
  static const int per_cu = [] {
    (void)hipFuncSetAttribute((const void*)fwd_mfma_kernel<D, MAP, ZS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)D::FWD_LDS);
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fwd_mfma_kernel<D, MAP, ZS>, kThreads, D::FWD_LDS) !=
            hipSuccess || nb < 1)
      nb = 1;
    return nb;
  }();
  int64_t grid = (int64_t)per_cu * device_cus();
  if (grid > max_grid) grid = max_grid;
  hipLaunchKernelGGL((fwd_mfma_kernel<D, MAP, ZS>), dim3((unsigned)grid), dim3(kThreads), D::FWD_LDS, s, a.N,
                     a.flags, a.x, a.S, a.A, a.B, a.bias, a.y, ZS ? a.zc : nullptr);
}

template <class D>
void run_fwd(const LayerArgs& a, int max_grid, hipStream_t s) {
  if constexpr (D::FWD_OK) {
    if constexpr (ZCache<D>::OK) {
      if (a.zc) {   // (the host refuses the cache together with the sparse-row hint)
        run_fwd_map<D, false, true>(a, max_grid, s);
        return;
      }
    }
    if constexpr (FwdMap<D, true>::ON) {
      if (a.flags & KRON_SPARSE_ROWS) {
        run_fwd_map<D, true>(a, max_grid, s);
        return;
      }
    }
    run_fwd_map<D, false>(a, max_grid, s);
  }
}

#endif

#if KRON_MFMA_PASS != 1
// The backward kernel of a shape: the preferred one (BK, measured per shape) when it
// supports the shape, else the rank-parallel one, else bwd_mfma_kernel.
template <class D, int BK>
constexpr int bwd_kind() {
  return (BK == 2 && Solo<D>::OK) ? 2 : (RP<D>::OK && (BK >= 1 || !D::BWD_OK)) ? 1 : 0;
}

template <class D, int BK>
void run_bwd(const LayerArgs& a, int grid, hipStream_t s) {
  constexpr int kind = bwd_kind<D, BK>();
  if constexpr (kind == 2) {
    static const bool attr = [] {
      (void)hipFuncSetAttribute((const void*)bwd_solo_kernel<D, 0>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)Solo<D>::LDS);
      (void)hipFuncSetAttribute((const void*)bwd_solo_kernel<D, 1>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)Solo<D>::LDS);
      (void)hipFuncSetAttribute((const void*)bwd_solo_kernel<D, 2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)Solo<D>::LDS);
      (void)hipFuncSetAttribute((const void*)bwd_solo_kernel<D, 3>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)Solo<D>::LDS);
      (void)hipFuncSetAttribute((const void*)bwd_solo_kernel<D, 4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)Solo<D>::LDS);
      return true;
    }();
    (void)attr;
    static const bool attr_map = [] {
      (void)hipFuncSetAttribute((const void*)bwd_solo_kernel<D, 0, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)Solo<D>::LDS);
      (void)hipFuncSetAttribute((const void*)bwd_solo_kernel<D, 1, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)Solo<D>::LDS);
      (void)hipFuncSetAttribute((const void*)bwd_solo_kernel<D, 2, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)Solo<D>::LDS);
      return true;
    }();
    (void)attr_map;
    const bool mask = a.flags & KRON_DX_RELU_MASK;
    const int dxm = a.dx == nullptr ? 0 : (a.dx_accumulate ? (mask ? 4 : 3) : (mask ? 2 : 1));
    const bool map = (a.flags & KRON_SPARSE_ROWS) && dxm <= 2;
#define KRON_SOLO_LAUNCH(M, MP)                                                                                 \
  hipLaunchKernelGGL((bwd_solo_kernel<D, M, MP>), dim3(grid), dim3(kThreads), Solo<D>::LDS, s, a.N, a.x, a.S, a.A, \
                     a.B, a.dy, a.dx, a.part, (const float*)nullptr)
#define KRON_SOLO_ZC_LAUNCH(M)                                                                                  \
  hipLaunchKernelGGL((bwd_solo_kernel<D, M, false, true>), dim3(grid), dim3(kThreads), Solo<D>::LDS, s, a.N, a.x, \
                     a.S, a.A, a.B, a.dy, a.dx, a.part, (const float*)a.zc)
    if constexpr (ZCache<D>::OK) {
      if (a.zc) {   // (the host refuses the cache with the sparse-row hint and with dx accumulation)
        static const bool attr_zc = [] {
          (void)hipFuncSetAttribute((const void*)bwd_solo_kernel<D, 0, false, true>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)Solo<D>::LDS);
          (void)hipFuncSetAttribute((const void*)bwd_solo_kernel<D, 1, false, true>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)Solo<D>::LDS);
          (void)hipFuncSetAttribute((const void*)bwd_solo_kernel<D, 2, false, true>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)Solo<D>::LDS);
          return true;
        }();
        (void)attr_zc;
        switch (dxm) {
          case 0: KRON_SOLO_ZC_LAUNCH(0); break;
          case 1: KRON_SOLO_ZC_LAUNCH(1); break;
          default: KRON_SOLO_ZC_LAUNCH(2); break;
        }
        return;
      }
    }
    if (map) {
      switch (dxm) {
        case 0: KRON_SOLO_LAUNCH(0, true); break;
        case 1: KRON_SOLO_LAUNCH(1, true); break;
        default: KRON_SOLO_LAUNCH(2, true); break;
      }
    } else {
      switch (dxm) {
        case 0: KRON_SOLO_LAUNCH(0, false); break;
        case 1: KRON_SOLO_LAUNCH(1, false); break;
        case 2: KRON_SOLO_LAUNCH(2, false); break;
        case 3: KRON_SOLO_LAUNCH(3, false); break;
        default: KRON_SOLO_LAUNCH(4, false); break;
      }
    }
#undef KRON_SOLO_LAUNCH
#undef KRON_SOLO_ZC_LAUNCH
  } else if constexpr (kind == 1) {
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

#define KRON_ENTRY(P, Q, M, N, R, BK)                                                                  \
  Entry{P, Q, M, N, R, Dims<P, Q, M, N, R>::FWD_OK,                                                    \
        Dims<P, Q, M, N, R>::BWD_OK || RP<Dims<P, Q, M, N, R>>::OK || Solo<Dims<P, Q, M, N, R>>::OK,    \
        bwd_kind<Dims<P, Q, M, N, R>, BK>(),                                                           \
        bwd_kind<Dims<P, Q, M, N, R>, BK>() == 1 ? RP<Dims<P, Q, M, N, R>>::RPI : kWaves,              \
        bwd_kind<Dims<P, Q, M, N, R>, BK>() == 1 ? RP<Dims<P, Q, M, N, R>>::WPC : 1,                   \
        ZCache<Dims<P, Q, M, N, R>>::OK && bwd_kind<Dims<P, Q, M, N, R>, BK>() == 2                     \
            ? ZCache<Dims<P, Q, M, N, R>>::ROW : 0,                                                     \
        &run_fwd_shape<P, Q, M, N, R>, &run_bwd<Dims<P, Q, M, N, R>, BK>},

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
#define KRON_FWD_INST(P, Q, M, N, R, BK) template void run_fwd_shape<P, Q, M, N, R>(const LayerArgs&, int, hipStream_t);
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

int mfma_zcache_row_floats(int p, int q, int m, int n, int r) {
  const Entry* e = find(p, q, m, n, r);
  return (e && e->fwd_ok && e->bwd_ok) ? e->zc_row : 0;
}

int mfma_bwd_chunk(int p, int q, int m, int n, int r) {
  if (r <= 4 || r % 4 != 0 || mfma_bwd_supported(p, q, m, n, r)) return 0;
  const Entry* e = find(p, q, m, n, 4);
  return (e && e->bwd_kind >= 1) ? 4 : 0;
}

int mfma_bwd_groups(int64_t N, int p, int q, int m, int n, int r) {
  const Entry* e = find(p, q, m, n, r);
  if (e && e->bwd_kind >= 1) {
    // per_cu workgroups per compute unit, each stepping over rows_per_step rows at a time
    const int64_t g = (N + e->rows_per_step - 1) / e->rows_per_step;
    const int64_t gmax = (int64_t)e->per_cu * kBwdGroups;
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
