// Matrix-core kernels of the Kronecker-factored layer for small blocks: m = n in {2, 4, 8}
// with p and q multiples of 16 (a 1024-wide layer with 8x8, 4x4 or 2x2 blocks has
// p = q = 128, 256 or 512).  The tutorial's batch sweep (Kronecker layer tutorial,
// "Results") finds low-rank layers with these blocks the only ones that beat a dense
// layer.  Their per-row matrices are too thin for the per-row tiles of the other
// matrix-core kernels, so each contraction with a long inner dimension runs here as an
// LDS-tiled GEMM over many rows, and the m x n mixing by B_i is done on the fly while an
// operand is staged.
//
// With X_n the p x m view of row n, Z_{n,i} = X_n B_i and C_i = S o A_i (Kronecker layer
// tutorial, "The vec trick" and "The vec trick without the loop"), and c < n a column of
// the blocks:
//   forward   Y_c[row][k] = sum_{(i,j)} Z_i[row][j][c] C_i[j][k]        (sb_fwd_kernel)
//             n GEMMs that share the factor operand C'[(i,j)][k] = C_i[j][k]
//   backward  G_{i,c}[row][j] = sum_k dY[row][k n + c] C_i[j][k]        (sb_bwd_g_kernel)
//             dX[row][j m + b] = sum_{i,c} G_{i,c}[row][j] B_i[b][c]
//             dB_i[b][c] = sum_{row,j} X[row][j m + b] G_{i,c}[row][j]
//             dC_i[j][k] = sum_{(row,c)} Z_i[row][j][c] dY[row][k n + c]  (sb_bwd_dc_kernel)
//             dbias = sum_row dY[row];  dA_i = S o dC_i,  dS = sum_i A_i o dC_i  (sb_dcs_kernel)
// The parameter gradients leave the kernels as per-workgroup partial rows and are summed
// by the fixed-order column reduction, so every result is deterministic.
#include "kron_internal.h"

#include <algorithm>

namespace kron {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

constexpr int kSbThreads = 256;   // four wavefronts
constexpr int kSbKC = 16;         // inner-dimension entries per staged chunk: four 16x16x4 steps
constexpr int kSbMaxRank = 16;

__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// v <- its m contiguous floats at p (p aligned to 4 * min(m, 4) bytes)
template <int M>
__device__ __forceinline__ void load_vec(float (&v)[M], const float* p) {
  if constexpr (M == 8) {
    const f4 a = *reinterpret_cast<const f4*>(p), b = *reinterpret_cast<const f4*>(p + 4);
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  } else if constexpr (M == 4) {
    const f4 a = *reinterpret_cast<const f4*>(p);
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  } else {
    static_assert(M == 2, "block side 2, 4 or 8");
    const f2 a = *reinterpret_cast<const f2*>(p);
    v[0] = a[0]; v[1] = a[1];
  }
}
template <int M>
__device__ __forceinline__ void store_vec(float* p, const float (&v)[M]) {
  // (the forward's y: written once and not read back, so streamed past the caches)
  if constexpr (M == 8) {
    __builtin_nontemporal_store(f4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f4*>(p));
    __builtin_nontemporal_store(f4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f4*>(p + 4));
  } else if constexpr (M == 4) {
    __builtin_nontemporal_store(f4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f4*>(p));
  } else {
    __builtin_nontemporal_store(f2{v[0], v[1]}, reinterpret_cast<f2*>(p));
  }
}

// The same with ordinary (cached) stores, for dX, which later ranks read back.
template <int M>
__device__ __forceinline__ void store_vec_cached(float* p, const float (&v)[M]) {
  if constexpr (M == 8) {
    *reinterpret_cast<f4*>(p) = f4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f4*>(p + 4) = f4{v[4], v[5], v[6], v[7]};
  } else if constexpr (M == 4) {
    *reinterpret_cast<f4*>(p) = f4{v[0], v[1], v[2], v[3]};
  } else {
    *reinterpret_cast<f2*>(p) = f2{v[0], v[1]};
  }
}

// Lane stride of an LDS factor table in which each lane's T tile values of one inner index
// are contiguous (one or a few 8/16-byte reads): conflict-free for the 8 or 16 lanes a
// read serves at a time.
constexpr int lane_stride(int T) { return T == 2 ? 2 : T == 4 ? 4 : T + 4; }

template <int T>
__device__ __forceinline__ void read_tiles(float (&v)[T], const float* p) {
  if constexpr (T == 2) {
    const f2 a = *reinterpret_cast<const f2*>(p);
    v[0] = a[0]; v[1] = a[1];
  } else {
    static_assert(T % 4 == 0, "2, 4, 8 or 16 tiles");
#pragma unroll
    for (int u = 0; u < T / 4; ++u) {
      const f4 a = *reinterpret_cast<const f4*>(p + 4 * u);
      v[4 * u] = a[0]; v[4 * u + 1] = a[1]; v[4 * u + 2] = a[2]; v[4 * u + 3] = a[3];
    }
  }
}

// An empty use of registers loaded before a loop: the wait for those loads is placed
// here once, instead of inside the loop on every trip (the wait-count pass merges the
// loop entry's pending loads into the loop header).
template <int A, int B>
__device__ __forceinline__ void settle(float (&v)[A][B]) {
#pragma unroll
  for (int a = 0; a < A; ++a)
#pragma unroll
    for (int b = 0; b < B; ++b) asm volatile("" ::"v"(v[a][b]));
}

template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_add_src(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xF, false));
}
// Sum over the wavefront in a fixed order; the total lands in lane 63.
__device__ __forceinline__ float wave_total_lane63(float v) {
  v += dpp_add_src<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
  v += dpp_add_src<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
  v += dpp_add_src<0x124, 0xF>(v);   // row_ror 4
  v += dpp_add_src<0x128, 0xF>(v);   // row_ror 8: every lane holds its 16-lane row total
  v += dpp_add_src<0x142, 0xA>(v);   // row_bcast 15 into rows 1 and 3
  v += dpp_add_src<0x143, 0xC>(v);   // row_bcast 31 into rows 2 and 3
  return v;
}

// Row block, column block of a tile index such that the tiles of one row block share
// their index modulo 8: consecutive workgroups are dispatched to the eight XCDs in turn,
// so the tiles that read the same rows land on one XCD and share its L2.
__device__ __forceinline__ void xcd_tile(int64_t t, int ninner, int64_t& outer, int& inner) {
  const int64_t rest = t >> 3;
  inner = (int)(rest % ninner);
  outer = (rest / ninner) * 8 + (t & 7);
}

// ---------------------------------------------------------------------------------
// Forward.  A workgroup computes 64 rows (16 per wavefront) x TN output blocks k, for all
// n columns c: n accumulator sets of KT 16x16 tiles.  The inner dimension (i, j) runs in
// chunks of 16: the chunk of C' (16 x TN) is staged in LDS (double-buffered, one barrier
// per chunk), and each lane forms its A operand Z_c[row][(i,j)] = sum_b X[row][j m + b]
// B_i[b][c] for all c from m floats of its row, so one mixing step feeds n * KT products.
// ---------------------------------------------------------------------------------
template <int NB>
struct SbF {
  static constexpr int KT = 32 / NB;        // 16-wide k tiles per workgroup: 4 KT NB = 128 accumulators
  static constexpr int TN = 16 * KT;
  static constexpr int KS = lane_stride(KT);
  static constexpr int LD = 16 * KS;        // one inner index: lane c16's KT values at c16 * KS
  static constexpr int NST = TN / 64;       // float4s of the chunk per thread
};

template <int MB, int NB>
__global__ __launch_bounds__(kSbThreads, 2) void sb_fwd_kernel(int64_t N, int p, int q, int r, uint32_t flags,
                                                             const float* __restrict__ x,
                                                             const float* __restrict__ S,
                                                             const float* __restrict__ A,
                                                             const float* __restrict__ B,
                                                             const float* __restrict__ bias,
                                                             float* __restrict__ y) {
  using F = SbF<NB>;
  constexpr int KT = F::KT, TN = F::TN, KS = F::KS, LD = F::LD, NST = F::NST;
  __shared__ __align__(16) float cs[2][kSbKC * LD];
  const int nkb = (q + TN - 1) / TN;
  int kb;
  int64_t rb;
  xcd_tile(blockIdx.x, nkb, rb, kb);
  if (rb * 64 >= N) return;
  const int k0 = kb * TN;
  const int ktv = min(KT, (q - k0) >> 4);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int64_t in = (int64_t)p * MB, out = (int64_t)q * NB, pq = (int64_t)p * q;
  const int64_t arow = rb * 64 + w * 16 + c16;
  const float* xr = x + (arow < N ? arow : N - 1) * in;
  const int nch = r * (p / kSbKC);

  // A_i and S pieces are loaded raw (S read from A's address when absent, so the loads are
  // unconditional) and multiplied only when stored, so no wait for them precedes the
  // chunk's products
  const bool hs = S != nullptr;
  const float* Sp = hs ? S : A;
  f4 sta[NST], sts[NST];
  auto stage_load = [&](int ch) {
    const int kap0 = ch * kSbKC, i = kap0 / p, j0 = kap0 - i * p;
    const float* Ai = A + (int64_t)i * pq;
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      const int f = tid + u * kSbThreads;
      const int kk = f / (TN / 4), kc = 4 * (f % (TN / 4));
      const int64_t e = (int64_t)(j0 + kk) * q + (k0 + kc < q ? k0 + kc : 0);
      sta[u] = *reinterpret_cast<const f4*>(Ai + e);
      sts[u] = *reinterpret_cast<const f4*>(Sp + e);
    }
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      const int f = tid + u * kSbThreads;
      const int kk = f / (TN / 4), kc = 4 * (f % (TN / 4));
      const f4 a = k0 + kc < q ? (hs ? sta[u] * sts[u] : sta[u]) : f4{0.f, 0.f, 0.f, 0.f};
      const int t = kc >> 4, cl = kc & 15;
#pragma unroll
      for (int h = 0; h < 4; ++h) cs[buf][kk * LD + (cl + h) * KS + t] = a[h];
    }
  };
  float xv[4][MB], xn[4][MB];
  auto x_load = [&](int ch, float (&d)[4][MB]) {
    const int kap0 = ch * kSbKC, i = kap0 / p, j0 = kap0 - i * p;
#pragma unroll
    for (int s = 0; s < 4; ++s) load_vec<MB>(d[s], xr + (int64_t)(j0 + 4 * s + g) * MB);
  };

  f4 acc[KT][NB];
#pragma unroll
  for (int t = 0; t < KT; ++t)
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[t][c] = f4{0.f, 0.f, 0.f, 0.f};

  stage_load(0);
  x_load(0, xv);
  stage_store(0);
  settle(xv);
  __syncthreads();
  // ranks outside, chunks of j inside: B_i goes to scalar registers once per rank
  const int njc = p / kSbKC;
  for (int i = 0, ch = 0; i < r; ++i) {
  const float* Bi = B + (int64_t)i * MB * NB;
  float bm[MB][NB];
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int c = 0; c < NB; ++c) bm[b][c] = Bi[b * NB + c];
  for (int jc = 0; jc < njc; ++jc, ++ch) {
    const int buf = ch & 1;
    const bool more = ch + 1 < nch;
    if (more) {
      stage_load(ch + 1);
      x_load(ch + 1, xn);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the factor values of step s + 1 are read while step s's products run; the
    // scheduling barrier keeps the compiler from hoisting further reads (registers).
    // The A operands of step s + 1 are mixed inside step s, so their VALU work runs
    // while step s's products occupy the matrix core.
    float bo0[KT], bo1[KT];
    float za[NB], zb[NB];
    auto mix = [&](const int s, float (&z)[NB]) {
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        z[c] = 0.f;
#pragma unroll
        for (int b = 0; b < MB; ++b) z[c] = fmaf(xv[s][b], bm[b][c], z[c]);
      }
    };
    auto kstep = [&](const int s, float (&cur)[KT], float (&nxt)[KT], float (&z)[NB], float (&zn)[NB]) {
      if (s < 3) read_tiles<KT>(nxt, &cs[buf][(4 * (s + 1) + g) * LD + c16 * KS]);
#pragma unroll
      for (int c = 0; c < NB; ++c) {
#pragma unroll
        for (int t = 0; t < KT; ++t) acc[t][c] = mfma(z[c], cur[t], acc[t][c]);
        if (s < 3) {
          zn[c] = 0.f;
#pragma unroll
          for (int b = 0; b < MB; ++b) zn[c] = fmaf(xv[s + 1][b], bm[b][c], zn[c]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    read_tiles<KT>(bo0, &cs[buf][g * LD + c16 * KS]);
    mix(0, za);
    kstep(0, bo0, bo1, za, zb);
    kstep(1, bo1, bo0, zb, za);
    kstep(2, bo0, bo1, za, zb);
    kstep(3, bo1, bo0, zb, za);
    if (more) {
      stage_store(buf ^ 1);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int b = 0; b < MB; ++b) xv[s][b] = xn[s][b];
    }
    __syncthreads();
  }
  }

  // lane (g, c16) holds Y_c[row = 4g + v][k = k0 + 16t + c16] in acc[t][c][v]
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    if (t >= ktv) continue;
    const int k = k0 + 16 * t + c16;
    float bb[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) bb[c] = bias ? bias[k * NB + c] : 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = rb * 64 + w * 16 + 4 * g + v;
      if (row >= N) continue;
      float o[NB];
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        o[c] = acc[t][c][v] + bb[c];
        if (flags & KRON_RELU_OUT) o[c] = o[c] > 0.f ? o[c] : 0.f;
      }
      store_vec<NB>(y + row * out + (int64_t)k * NB, o);
    }
  }
}

// ---------------------------------------------------------------------------------
// Backward, part 1: G, dX and dB.  A workgroup tile is 64 rows x TN blocks j; for each
// rank the G_{i,c} tiles (rows x j, one per c) accumulate over k in chunks of 16, whose
// C_i^T chunk (16 x TN) is staged in LDS; dY's n floats at (row, k) are the A operands of
// the n products.  After the rank's last chunk its G is folded into dX (mixing by B_i^T,
// added in place to the rank-sum in dx) and into this lane's share of dB_i, which is
// summed over the wavefront in a fixed order and added to the wavefront's LDS slot.
// Workgroups are persistent over tiles; each writes one partial row of dB (all ranks).
// ---------------------------------------------------------------------------------
template <int NB>
struct SbG {
  static constexpr int JT = 16 / NB;        // 16-wide j tiles: 4 JT NB = 64 accumulators
  static constexpr int TN = 16 * JT;
  static constexpr int KS = lane_stride(JT);
  static constexpr int LD = 16 * KS;        // one k: lane c16's JT values at c16 * KS
  static constexpr int NST = (4 * TN + kSbThreads - 1) / kSbThreads;
};

// DXM: 0 no dX, 1 dX, 2 dX masked by [x > 0]
template <int MB, int NB, int DXM>
__global__ __launch_bounds__(kSbThreads, 2) void sb_bwd_g_kernel(int64_t N, int p, int q, int r, int64_t ntiles8,
                                                               const float* __restrict__ x,
                                                               const float* __restrict__ S,
                                                               const float* __restrict__ A,
                                                               const float* __restrict__ B,
                                                               const float* __restrict__ dy,
                                                               float* __restrict__ dx,
                                                               float* __restrict__ part) {
  using Gd = SbG<NB>;
  constexpr int JT = Gd::JT, TN = Gd::TN, KS = Gd::KS, LD = Gd::LD, NST = Gd::NST, MN = MB * NB;
  __shared__ __align__(16) float cs[2][kSbKC * LD];
  __shared__ float dbs[4][kSbMaxRank * MN];
  __shared__ float bms[kSbMaxRank * MN];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int64_t in = (int64_t)p * MB, out = (int64_t)q * NB, pq = (int64_t)p * q;
  const int njb = (p + TN - 1) / TN;
  const int nkc = q / kSbKC;
  const int nch = r * nkc;
  const bool hs = S != nullptr;
  const float* Sp = hs ? S : A;
  for (int e = tid; e < 4 * kSbMaxRank * MN; e += kSbThreads) (&dbs[0][0])[e] = 0.f;
  for (int e = tid; e < r * MN; e += kSbThreads) bms[e] = B[e];
  __syncthreads();

  for (int64_t tile = blockIdx.x; tile < ntiles8; tile += gridDim.x) {
    int jb;
    int64_t rb;
    xcd_tile(tile, njb, rb, jb);
    if (rb * 64 >= N) continue;
    const int j0 = jb * TN;
    const int64_t arow = rb * 64 + w * 16 + c16;
    const float* yr = dy + (arow < N ? arow : N - 1) * out;

    // raw A_i and S pieces (S read from A's address when absent), multiplied when stored
    f4 sta[NST], sts[NST];
    auto stage_load = [&](int ch) {
      const int i = ch / nkc, kc0 = (ch - i * nkc) * kSbKC;
      const float* Ai = A + (int64_t)i * pq;
#pragma unroll
      for (int u = 0; u < NST; ++u) {
        const int f = tid + u * kSbThreads;
        const int jj = f >> 2, kq = f & 3;
        const bool ok = f < 4 * TN && j0 + jj < p;
        const int64_t e = (int64_t)(ok ? j0 + jj : 0) * q + kc0 + 4 * kq;
        sta[u] = *reinterpret_cast<const f4*>(Ai + e);
        sts[u] = *reinterpret_cast<const f4*>(Sp + e);
      }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
      for (int u = 0; u < NST; ++u) {
        const int f = tid + u * kSbThreads;
        if (4 * TN % kSbThreads != 0 && f >= 4 * TN) continue;
        const int jj = f >> 2, kq = f & 3;
        const f4 a = j0 + jj < p ? (hs ? sta[u] * sts[u] : sta[u]) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < 4; ++h) cs[buf][(4 * kq + h) * LD + (jj & 15) * KS + (jj >> 4)] = a[h];
      }
    };
    float yv[4][NB], yn[4][NB];
    auto y_load = [&](int ch, float (&d)[4][NB]) {
      const int i = ch / nkc, kc0 = (ch - i * nkc) * kSbKC;
#pragma unroll
      for (int s = 0; s < 4; ++s) load_vec<NB>(d[s], yr + (int64_t)(kc0 + 4 * s + g) * NB);
    };

    f4 acc[JT][NB];
#pragma unroll
    for (int t = 0; t < JT; ++t)
#pragma unroll
      for (int c = 0; c < NB; ++c) acc[t][c] = f4{0.f, 0.f, 0.f, 0.f};

    stage_load(0);
    y_load(0, yv);
    stage_store(0);
    settle(yv);
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
      const int buf = ch & 1;
      const bool more = ch + 1 < nch;
      const bool rank_end = (ch % nkc) == nkc - 1;
      if (more && !rank_end) {
        stage_load(ch + 1);
        y_load(ch + 1, yn);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float bo[JT];
        read_tiles<JT>(bo, &cs[buf][(4 * s + g) * LD + c16 * KS]);
#pragma unroll
        for (int t = 0; t < JT; ++t)
#pragma unroll
          for (int c = 0; c < NB; ++c) acc[t][c] = mfma(yv[s][c], bo[t], acc[t][c]);
      }
      if (rank_end) {
        // lane (g, c16) holds G_{i,c}[row = 4g + v][j = j0 + 16t + c16] in acc[t][c][v].
        // dX gets this rank's G B_i^T added in place (written by rank 0, read back and
        // added to by the later ranks: the same thread's earlier store), the ReLU mask
        // applied by the last rank; dB_i's share is summed in passes over ranges of c so
        // that at most 16 sums are live.
        const int i = ch / nkc;
        constexpr int CP = MN > 16 ? MN / 16 : 1, CW = NB / CP;
        // lane offsets laundered here, so the compiler does not hoist the (t, v) addresses
        // of the epilogue out of the chunk loop and hold them in registers
        int lrow = 4 * g, lj = c16;
        asm volatile("" : "+v"(lrow), "+v"(lj));
#pragma unroll
        for (int cp = 0; cp < CP; ++cp) {
          float dbp[MB][CW];
#pragma unroll
          for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int c = 0; c < CW; ++c) dbp[b][c] = 0.f;
#pragma unroll
          for (int t = 0; t < JT; ++t) {
            const int j = j0 + 16 * t + lj;
            const int jc = j < p ? j : p - 1;
            // x of dead rows is zeroed (their G, from a clamped dY row, is not); G of
            // dead j is zero already (zero factor columns were staged)
            float xt[4][MB];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int64_t row = rb * 64 + w * 16 + lrow + v;
              load_vec<MB>(xt[v], x + (row < N ? row : N - 1) * in + (int64_t)jc * MB);
#pragma unroll
              for (int b = 0; b < MB; ++b) xt[v][b] = row < N ? xt[v][b] : 0.f;
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int64_t row = rb * 64 + w * 16 + lrow + v;
              const bool live = j < p && row < N;
              if constexpr (DXM != 0) {
                if (cp == 0 && live) {
                  // B_i re-read per (t, v) from LDS (broadcast), not held in registers
                  int bo = i * MN;
                  asm volatile("" : "+v"(bo));
                  float o[MB];
#pragma unroll
                  for (int b = 0; b < MB; ++b) {
                    o[b] = 0.f;
#pragma unroll
                    for (int c = 0; c < NB; ++c) o[b] = fmaf(acc[t][c][v], bms[bo + b * NB + c], o[b]);
                  }
                  float* dst = dx + row * in + (int64_t)j * MB;
                  if (i > 0) {
                    float prev[MB];
                    load_vec<MB>(prev, dst);
#pragma unroll
                    for (int b = 0; b < MB; ++b) o[b] += prev[b];
                  }
                  if (DXM == 2 && i == r - 1)
#pragma unroll
                    for (int b = 0; b < MB; ++b) o[b] = xt[v][b] > 0.f ? o[b] : 0.f;
                  store_vec_cached<MB>(dst, o);
                }
              }
#pragma unroll
              for (int b = 0; b < MB; ++b)
#pragma unroll
                for (int c = 0; c < CW; ++c)
                  dbp[b][c] = fmaf(xt[v][b], acc[t][cp * CW + c][v], dbp[b][c]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int c = 0; c < CW; ++c) dbp[b][c] = wave_total_lane63(dbp[b][c]);
          if (lane == 63) {
#pragma unroll
            for (int b = 0; b < MB; ++b)
#pragma unroll
              for (int c = 0; c < CW; ++c) dbs[w][i * MN + b * NB + cp * CW + c] += dbp[b][c];
          }
        }
#pragma unroll
        for (int t = 0; t < JT; ++t)
#pragma unroll
          for (int c = 0; c < NB; ++c) acc[t][c] = f4{0.f, 0.f, 0.f, 0.f};
        if (more) {
          stage_load(ch + 1);
          y_load(ch + 1, yn);
        }
      }
      if (more) {
        stage_store(buf ^ 1);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int c = 0; c < NB; ++c) yv[s][c] = yn[s][c];
      }
      __syncthreads();
    }

  }

  // this workgroup's partial row of dB (all ranks): the four wavefront slots in order
  __syncthreads();
  const PartRow pr{part, (int64_t)gridDim.x, (int64_t)blockIdx.x, 0};
  for (int e = tid; e < r * MN; e += kSbThreads) pr[e] = (dbs[0][e] + dbs[1][e]) + (dbs[2][e] + dbs[3][e]);
}

// ---------------------------------------------------------------------------------
// Backward, part 2: dC and dbias.  dC_i (p x q) is a GEMM over the inner dimension
// (row, c); a workgroup owns a 128 x 128 tile (j x k) of one rank for one group of rows
// and writes it to its partial row.  Per chunk of 32 inner entries (32 / n rows), the Z_i
// operand (built from x and B_i) and the dY operand are staged in LDS (double-buffered);
// each wavefront computes a 64 x 64 quarter as 4 x 4 products of 16 x 16.  The k-tile's
// dbias columns are summed by the rank-0, first-j-tile workgroup of each row group from
// the dY values it stages.
// ---------------------------------------------------------------------------------
constexpr int kDcT = 128;
constexpr int kDcLD = kDcT + 16;
constexpr int kDcKC = 32;

template <int MB, int NB>
__global__ __launch_bounds__(kSbThreads, 2) void sb_bwd_dc_kernel(int64_t N, int p, int q, int r, int G2,
                                                                int64_t rpg, const float* __restrict__ x,
                                                                const float* __restrict__ B,
                                                                const float* __restrict__ dy,
                                                                float* __restrict__ part) {
  constexpr int RCH = kDcKC / NB;           // rows per chunk
  constexpr int PZ = kDcT * RCH / kSbThreads;   // (row, j) pairs per thread
  constexpr int PY = kDcT * kDcKC / 4 / kSbThreads;   // dY float4s per thread
  constexpr int YROW4 = kDcT * NB / 4;      // float4s of one row's k-tile segment
  static_assert(PZ * kSbThreads == kDcT * RCH && PY == 4, "staging shape");
  __shared__ __align__(16) float zs[2][kDcKC * kDcLD];
  __shared__ __align__(16) float ys[2][kDcKC * kDcLD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int wj = w & 1, wk = w >> 1;
  const int64_t in = (int64_t)p * MB, out = (int64_t)q * NB, pq = (int64_t)p * q;
  const int njt = (p + kDcT - 1) / kDcT, nkt = (q + kDcT - 1) / kDcT;
  const int T = njt * nkt * r;
  int tl;
  int64_t gg;
  xcd_tile(blockIdx.x, T, gg, tl);
  const int kt = tl % nkt, jt = (tl / nkt) % njt, i = tl / (nkt * njt);
  const int j0 = jt * kDcT, k0 = kt * kDcT;
  const int64_t rbeg = gg * rpg;
  const int64_t rend = std::min<int64_t>(N, rbeg + rpg);
  const int64_t nrows = rend > rbeg ? rend - rbeg : 0;
  const int nch = (int)((nrows + RCH - 1) / RCH);
  const float* Bi = B + (int64_t)i * MB * NB;
  float bm[MB][NB];
#pragma unroll
  for (int b = 0; b < MB; ++b)
#pragma unroll
    for (int c = 0; c < NB; ++c) bm[b][c] = Bi[b * NB + c];

  float xz[PZ][MB];
  f4 yv[PY];
  f4 db4 = f4{0.f, 0.f, 0.f, 0.f};
  auto fetch = [&](int ch) {
    const int64_t r0 = rbeg + (int64_t)ch * RCH;
#pragma unroll
    for (int u = 0; u < PZ; ++u) {
      const int f = tid + u * kSbThreads;
      const int rr = f / kDcT, jj = f % kDcT;
      const int64_t row = r0 + rr;
      const int j = j0 + jj;
      load_vec<MB>(xz[u], x + (row < rend ? row : rend - 1) * in + (int64_t)(j < p ? j : p - 1) * MB);
      if (!(row < rend && j < p))
#pragma unroll
        for (int b = 0; b < MB; ++b) xz[u][b] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < PY; ++u) {
      const int f = tid + u * kSbThreads;
      const int rr = f / YROW4, e = f % YROW4;
      const int64_t row = r0 + rr;
      const bool ok = row < rend && k0 * NB + 4 * e < out;
      const f4 v = *reinterpret_cast<const f4*>(dy + (row < rend ? row : rend - 1) * out +
                                                (ok ? k0 * NB + 4 * e : 0));
      yv[u] = ok ? v : f4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PZ; ++u) {
      const int f = tid + u * kSbThreads;
      const int rr = f / kDcT, jj = f % kDcT;
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        float z = 0.f;
#pragma unroll
        for (int b = 0; b < MB; ++b) z = fmaf(xz[u][b], bm[b][c], z);
        zs[buf][(rr * NB + c) * kDcLD + jj] = z;
      }
    }
#pragma unroll
    for (int u = 0; u < PY; ++u) {
      const int f = tid + u * kSbThreads;
      const int rr = f / YROW4, e = f % YROW4;
      db4 += yv[u];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int idx = 4 * e + h, kk = idx / NB, c = idx % NB;
        ys[buf][(rr * NB + c) * kDcLD + kk] = yv[u][h];
      }
    }
  };

  f4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f4{0.f, 0.f, 0.f, 0.f};

  if (nch > 0) {
    fetch(0);
    stash(0);
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
      const int buf = ch & 1;
      const bool more = ch + 1 < nch;
      if (more) fetch(ch + 1);
#pragma unroll
      for (int s = 0; s < kDcKC / 4; ++s) {
        const float* zr = &zs[buf][(4 * s + g) * kDcLD + 64 * wj + c16];
        const float* yr = &ys[buf][(4 * s + g) * kDcLD + 64 * wk + c16];
        float a[4], bq[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          a[t] = zr[16 * t];
          bq[t] = yr[16 * t];
        }
#pragma unroll
        for (int ta = 0; ta < 4; ++ta)
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) acc[ta][tb] = mfma(a[ta], bq[tb], acc[ta][tb]);
      }
      if (more) stash(buf ^ 1);
      __syncthreads();
    }
  }

  // partial row gg: dC_i[j][k] at column i*p*q + j*q + k; lane (g, c16) holds
  // dC[j = j0 + 64wj + 16ta + 4g + v][k = k0 + 64wk + 16tb + c16]
  const PartRow pr{part, (int64_t)G2, gg, 0};
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int k = k0 + 64 * wk + 16 * tb + c16;
    if (k >= q) continue;
#pragma unroll
    for (int ta = 0; ta < 4; ++ta)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = j0 + 64 * wj + 16 * ta + 4 * g + v;
        if (j < p) pr[(int64_t)i * pq + (int64_t)j * q + k] = acc[ta][tb][v];
      }
  }
  if (i == 0 && jt == 0) {
    // dbias of this k tile: thread tid staged float4 e = tid % YROW4 of every row it
    // loaded; the kSbThreads / YROW4 threads that share e are added in thread order
    __syncthreads();
    f4* red = reinterpret_cast<f4*>(&zs[0][0]);
    red[tid] = db4;
    __syncthreads();
    if (tid < YROW4) {
      f4 sacc = red[tid];
      for (int u = 1; u < kSbThreads / YROW4; ++u) sacc += red[tid + u * YROW4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int col = k0 * NB + 4 * tid + h;
        if (col < out) pr[(int64_t)r * pq + col] = sacc[h];
      }
    }
  }
}

// dC (held in dA) -> dA_i = S o dC_i and dS = sum_i A_i o dC_i, in rank order.
__global__ __launch_bounds__(256) void sb_dcs_kernel(int64_t pq, int r, const float* __restrict__ S,
                                                     const float* __restrict__ A, float* __restrict__ dA,
                                                     float* __restrict__ dS) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= pq) return;
  const float sv = S[e];
  float ds = 0.f;
  for (int i = 0; i < r; ++i) {
    const float dc = dA[(int64_t)i * pq + e];
    ds = fmaf(A[(int64_t)i * pq + e], dc, ds);
    dA[(int64_t)i * pq + e] = sv * dc;
  }
  dS[e] = ds;
}

int64_t round8(int64_t v) { return (v + 7) / 8 * 8; }

// One launch per 2^24 rows at most, so the grid (a workgroup per 64 rows and k block)
// stays far below the 2^31 limit for every valid shape.
template <int MB>
void fwd_small(const LayerArgs& a, hipStream_t s) {
  constexpr int NB = MB;
  constexpr int64_t kRowsPerLaunch = int64_t(1) << 24;
  const int nkb = (a.q + SbF<NB>::TN - 1) / SbF<NB>::TN;
  const int64_t in = (int64_t)a.p * MB, out = (int64_t)a.q * NB;
  for (int64_t r0 = 0; r0 < a.N; r0 += kRowsPerLaunch) {
    const int64_t rows = std::min(kRowsPerLaunch, a.N - r0);
    const int64_t nrb = (rows + 63) / 64;
    const int64_t grid = 8 * nkb * ((nrb + 7) / 8);
    hipLaunchKernelGGL((sb_fwd_kernel<MB, NB>), dim3((unsigned)grid), dim3(kSbThreads), 0, s, rows, a.p, a.q, a.r,
                       a.flags, a.x + r0 * in, a.S, a.A, a.B, a.bias, a.y + r0 * out);
  }
}

template <int MB, int DXM>
void bwd_g_small(const LayerArgs& a, const SmallBwdPlan& pl, hipStream_t s) {
  constexpr int NB = MB;
  const int64_t nrb = (a.N + 63) / 64;
  const int njb = (a.p + SbG<NB>::TN - 1) / SbG<NB>::TN;
  const int64_t ntiles8 = 8 * njb * ((nrb + 7) / 8);
  hipLaunchKernelGGL((sb_bwd_g_kernel<MB, NB, DXM>), dim3((unsigned)pl.G1), dim3(kSbThreads), 0, s, a.N, a.p, a.q,
                     a.r, ntiles8, a.x, a.S, a.A, a.B, a.dy, a.dx, a.part);
}

template <int MB>
void bwd_small(const LayerArgs& a, const SmallBwdPlan& pl, hipStream_t s) {
  constexpr int NB = MB;
  if (!a.dx)
    bwd_g_small<MB, 0>(a, pl, s);
  else if (a.flags & KRON_DX_RELU_MASK)
    bwd_g_small<MB, 2>(a, pl, s);
  else
    bwd_g_small<MB, 1>(a, pl, s);
  const int T = ((a.p + kDcT - 1) / kDcT) * ((a.q + kDcT - 1) / kDcT) * a.r;
  hipLaunchKernelGGL((sb_bwd_dc_kernel<MB, NB>), dim3((unsigned)(pl.G2 * T)), dim3(kSbThreads), 0, s, a.N, a.p,
                     a.q, a.r, pl.G2, pl.rpg, a.x, a.B, a.dy, a.part + pl.off2);
}

}  // namespace

bool small_supported(int p, int q, int m, int n, int r) {
  return m == n && (m == 2 || m == 4 || m == 8) && p % 16 == 0 && q % 16 == 0 && r >= 1 && r <= kSbMaxRank;
}

SmallBwdPlan small_bwd_plan(int64_t N, int p, int q, int m, int n, int r) {
  SmallBwdPlan pl{};
  // part 1: persistent workgroups over (64-row, TN-block) tiles, a multiple of 8
  const int TNG = 256 / n;
  const int64_t tiles = ((N + 63) / 64) * ((p + TNG - 1) / TNG);
  pl.G1 = (int)std::max<int64_t>(8, std::min<int64_t>(round8(tiles), 512));
  // part 2: row groups (a multiple of 8) so that groups x tiles is about 512 workgroups
  const int64_t T = (int64_t)((p + kDcT - 1) / kDcT) * ((q + kDcT - 1) / kDcT) * r;
  int64_t G2 = round8(std::max<int64_t>(1, 512 / T));
  const int64_t rch = kDcKC / n;
  const int64_t maxg = round8(std::max<int64_t>(1, (N + rch - 1) / rch));
  pl.G2 = (int)std::max<int64_t>(8, std::min(G2, maxg));
  pl.rpg = (N + pl.G2 - 1) / pl.G2;
  pl.PW1 = (int64_t)r * m * n;
  pl.PW2 = (int64_t)r * p * q + (int64_t)q * n;
  const int64_t f1 = part_floats(pl.G1, pl.PW1);
  pl.off2 = (f1 + 63) / 64 * 64;
  pl.ws_floats = pl.off2 + part_floats(pl.G2, pl.PW2);
  return pl;
}

hipError_t launch_fwd_small(const LayerArgs& a, hipStream_t s) {
  if (!small_supported(a.p, a.q, a.m, a.n, a.r)) return hipErrorInvalidValue;
  if (a.N == 0) return hipSuccess;
  switch (a.m) {
    case 8: fwd_small<8>(a, s); break;
    case 4: fwd_small<4>(a, s); break;
    default: fwd_small<2>(a, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_small(const LayerArgs& a, const SmallBwdPlan& pl, hipStream_t s) {
  if (!small_supported(a.p, a.q, a.m, a.n, a.r)) return hipErrorInvalidValue;
  switch (a.m) {
    case 8: bwd_small<8>(a, pl, s); break;
    case 4: bwd_small<4>(a, pl, s); break;
    default: bwd_small<2>(a, pl, s); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int32_t pq = a.p * a.q;
  RedPlan r1{};
  r1.nseg = 1;
  r1.seg[0] = RedSeg{a.dB, a.r * a.m * a.n, 1.f, 0};
  e = launch_column_reduce(a.part, pl.G1, (int32_t)pl.PW1, r1, s);
  if (e != hipSuccess) return e;
  RedPlan r2{};
  r2.nseg = 2;
  r2.seg[0] = RedSeg{a.dA, a.r * pq, 1.f, 0};
  r2.seg[1] = RedSeg{a.dbias, a.q * a.n, 1.f, 0};
  e = launch_column_reduce(a.part + pl.off2, pl.G2, (int32_t)pl.PW2, r2, s);
  if (e != hipSuccess) return e;
  if (a.S) {
    hipLaunchKernelGGL(sb_dcs_kernel, dim3((unsigned)((pq + 255) / 256)), dim3(256), 0, s, (int64_t)pq, a.r, a.S,
                       a.A, a.dA, a.dS);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace kron
