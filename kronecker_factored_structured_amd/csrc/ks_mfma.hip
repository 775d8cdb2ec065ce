// Matrix-core kernel of the Kronecker-sparse matmul Y = X K, K of support
// I_a (x) 1_{b x c} (x) I_d ("Fast Inference with Kronecker-Sparse Matrices", abstract).
//
// For one (alpha, delta) the product is an ordinary GEMM over the rows,
//   Y[n, (al*c + ga)*d + de] = sum_be X[n, (al*b + be)*d + de] * V[al][de][be][ga],
// and the d GEMMs of one alpha read and write interleaved columns.  The kernel is output
// stationary: a task is 16 rows x (a group of 16-wide gamma tiles) x all d deltas of one
// alpha, so a lane holds the d values of delta for one (row, beta) -- one vector load of
// X -- and writes the d values of delta for one (row, gamma) -- one vector store of Y.
// No permutation pass exists: the interleave is absorbed by which accumulator a product
// goes to.  Products are 16x16x4 fp32 MFMAs; bf16 inputs are widened to fp32 on load
// (a bf16 x bf16 product is exact in fp32, so only the accumulation order differs from a
// bf16 matrix instruction), except in the d = 4 register kernels, whose bf16 twins run
// 16x16x16 bf16 MFMAs.
//
// Two kernels.  For d = 4 (ks_vreg_kernel, below) each wavefront keeps its slice of V in
// registers and only rows pass through LDS.  For the other shapes of the table
// (ks_mfma_kernel) workgroups (8 wavefronts) are specialised by alpha and keep V[alpha]
// in LDS as chunk-interleaved operand tables: table[de][gamma tile][chunk][lane][4] holds
// V[al][de][be = g*SB + s][ga = 16*tile + c] for K step s, so that one ds_read_b128 per
// chunk is contiguous across the wavefront.  Tasks are dealt round-robin to the
// workgroup's wavefronts; the GQ gamma groups of a row tile go to neighbouring
// wavefronts, which share its X through the L1 cache.
#include "kron_internal.h"

namespace kron {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

// y stores: fp32 as is, or bf16 rounded to nearest even (v_cvt_pk_bf16_f32).  y is
// written once and not read again by the call, so the stores are non-temporal: they
// stream to memory without displacing cached rows (measured: ViT fp32 52.7 -> 40.5 us).
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), b2));
}
typedef uint32_t u2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store4(float* p, f4 v) { __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p)); }
__device__ __forceinline__ void store4(uint16_t* p, f4 v) {
  __builtin_nontemporal_store(u2v{bf16x2(v[0], v[1]), bf16x2(v[2], v[3])}, reinterpret_cast<u2v*>(p));
}
__device__ __forceinline__ void store2(float* p, f2 v) { __builtin_nontemporal_store(v, reinterpret_cast<f2*>(p)); }
__device__ __forceinline__ void store2(uint16_t* p, f2 v) {
  __builtin_nontemporal_store(bf16x2(v[0], v[1]), reinterpret_cast<uint32_t*>(p));
}
__device__ __forceinline__ void store1(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store1(uint16_t* p, float v) {
  __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, (__bf16)v), p);
}

constexpr int kThreads = 512;   // eight wavefronts
constexpr int kWaves = kThreads / 64;
constexpr size_t kMaxLds = 160 * 1024;

__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int B_, int C_, int D_>
struct KS {
  static constexpr int Bv = B_, Cv = C_, Dv = D_;
  static constexpr int SB = B_ / 4;          // K steps per lane group: be = g*SB + s
  static constexpr int TG = C_ / 16;         // gamma tiles
  static constexpr int GQ = TG % 3 == 0 && TG > 3 ? TG / 3 : (TG % 2 == 0 && TG > 2 ? TG / 2 : 1);
  static constexpr int TPQ = TG / GQ;        // gamma tiles per task
  static constexpr int TABLE = D_ * TG * 64 * SB;   // = d*b*c floats
  static constexpr size_t LDS = (size_t)TABLE * 4;
  static constexpr bool OK = B_ % 4 == 0 && C_ % 16 == 0 && (D_ == 1 || D_ == 2 || D_ == 4) && LDS <= kMaxLds &&
                             SB % 4 == 0;
};

template <int L>
__device__ __forceinline__ void table_read4(float (&dst)[L], const float* blk, int lane) {
#pragma unroll
  for (int t = 0; t < L / 4; ++t) {
    const f4 v = reinterpret_cast<const f4*>(blk)[t * 64 + lane];
    dst[4 * t] = v[0]; dst[4 * t + 1] = v[1]; dst[4 * t + 2] = v[2]; dst[4 * t + 3] = v[3];
  }
}

template <int DV>
__device__ __forceinline__ void load_d(float (&dst)[DV], const float* p) {
  if constexpr (DV == 4) {
    const f4 v = *reinterpret_cast<const f4*>(p);
    dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
  } else if constexpr (DV == 2) {
    const f2 v = *reinterpret_cast<const f2*>(p);
    dst[0] = v[0]; dst[1] = v[1];
  } else {
    dst[0] = p[0];
  }
}
template <int DV>
__device__ __forceinline__ void load_d(float (&dst)[DV], const uint16_t* p) {
  if constexpr (DV == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    dst[0] = __uint_as_float(v.x << 16); dst[1] = __uint_as_float(v.x & 0xffff0000u);
    dst[2] = __uint_as_float(v.y << 16); dst[3] = __uint_as_float(v.y & 0xffff0000u);
  } else if constexpr (DV == 2) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
    dst[0] = __uint_as_float(v << 16); dst[1] = __uint_as_float(v & 0xffff0000u);
  } else {
    dst[0] = __uint_as_float(((uint32_t)p[0]) << 16);
  }
}
__device__ __forceinline__ float widen(float v) { return v; }
__device__ __forceinline__ float widen(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

template <class K, class TIn, class TOut>
__global__ __launch_bounds__(kThreads) void ks_mfma_kernel(int64_t N, int a_count, const TIn* __restrict__ x,
                                                           const TIn* __restrict__ vals,
                                                           TOut* __restrict__ y) {
  constexpr int b = K::Bv, c_ = K::Cv, d = K::Dv, SB = K::SB;
  extern __shared__ float tab[];
  const int groups_per_alpha = gridDim.x / a_count;
  const int al = blockIdx.x / groups_per_alpha;
  const int gidx = blockIdx.x % groups_per_alpha;
  // V[al] -> table[de][tile][chunk][lane][4]: each thread gathers the four K steps of one
  // (lane, chunk) and writes them with one 16-byte LDS store (consecutive threads write
  // consecutive 16 bytes); the sixteen lanes of a group read sixteen consecutive gammas
  const TIn* V = vals + (int64_t)al * d * b * c_;
#pragma unroll 4
  for (int e4 = threadIdx.x; e4 < K::TABLE / 4; e4 += kThreads) {
    int r = e4;
    const int l = r % 64; r /= 64;
    const int ch = r % (SB / 4); r /= (SB / 4);
    const int tile = r % K::TG;
    const int de = r / K::TG;
    const int be0 = (l >> 4) * SB + ch * 4, ga = 16 * tile + (l & 15);
    const TIn* src = V + ((int64_t)de * b + be0) * c_ + ga;
    reinterpret_cast<f4*>(tab)[e4] = f4{widen(src[0]), widen(src[c_]), widen(src[2 * c_]), widen(src[3 * c_])};
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int wave = threadIdx.x >> 6;
  const int64_t in_w = (int64_t)a_count * b * d, out_w = (int64_t)a_count * c_ * d;
  const int64_t tiles = (N + 15) / 16;
  const int64_t ntasks = tiles * K::GQ;
  const int64_t stride = (int64_t)groups_per_alpha * kWaves;
  // A operand of a task: X[row][(al*b + be)*d + de] for be = g*SB + s, all de; the next
  // task's is loaded while the current one computes
  auto load_x = [&](float (&xa)[SB][d], int64_t task) {
    const int64_t row = task / K::GQ * 16 + c;
    if (task < ntasks && row < N) {
      const TIn* xr = x + row * in_w + ((int64_t)al * b + g * SB) * d;
#pragma unroll
      for (int s = 0; s < SB; ++s) load_d<d>(xa[s], xr + s * d);
    } else {
#pragma unroll
      for (int s = 0; s < SB; ++s)
#pragma unroll
        for (int de = 0; de < d; ++de) xa[s][de] = 0.f;
    }
  };
  int64_t task = (int64_t)gidx * kWaves + wave;
  float xn[SB][d];
  load_x(xn, task);
  // wait here for the first task's loads, so that the loop head only ever has the
  // previous task's stores outstanding (a merged wait there would drain them)
#pragma unroll
  for (int s = 0; s < SB; ++s)
#pragma unroll
    for (int de = 0; de < d; ++de) asm volatile("" ::"v"(xn[s][de]));
  for (; task < ntasks; task += stride) {
    const int64_t rt = task / K::GQ;
    const int q = (int)(task % K::GQ);
    float xa[SB][d];
#pragma unroll
    for (int s = 0; s < SB; ++s)
#pragma unroll
      for (int de = 0; de < d; ++de) xa[s][de] = xn[s][de];
    load_x(xn, task + stride);
    f4 acc[K::TPQ][d];
#pragma unroll
    for (int t = 0; t < K::TPQ; ++t)
#pragma unroll
      for (int de = 0; de < d; ++de) acc[t][de] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ch = 0; ch < SB / 4; ++ch) {
      float bv[K::TPQ][d][4];
#pragma unroll
      for (int t = 0; t < K::TPQ; ++t)
#pragma unroll
        for (int de = 0; de < d; ++de) {
          const int tile = q * K::TPQ + t;
          const f4 v = reinterpret_cast<const f4*>(tab + ((de * K::TG + tile) * (SB / 4) + ch) * 64 * 4)[lane];
          bv[t][de][0] = v[0]; bv[t][de][1] = v[1]; bv[t][de][2] = v[2]; bv[t][de][3] = v[3];
        }
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4)
#pragma unroll
        for (int t = 0; t < K::TPQ; ++t)
#pragma unroll
          for (int de = 0; de < d; ++de) acc[t][de] = mfma(xa[ch * 4 + w4][de], bv[t][de][w4], acc[t][de]);
    }
    // acc[t][de] register v = Y[row = 16rt + 4g + v][ga = 16*(q*TPQ + t) + c] for delta de
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t orow = rt * 16 + 4 * g + v;
      if (orow >= N) continue;
      TOut* yr = y + orow * out_w + (int64_t)al * c_ * d;
#pragma unroll
      for (int t = 0; t < K::TPQ; ++t) {
        const int ga = 16 * (q * K::TPQ + t) + c;
        if constexpr (d == 4) {
          store4(yr + ga * 4, f4{acc[t][0][v], acc[t][1][v], acc[t][2][v], acc[t][3][v]});
        } else if constexpr (d == 2) {
          store2(yr + ga * 2, f2{acc[t][0][v], acc[t][1][v]});
        } else {
          store1(yr + ga, acc[t][0][v]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// d = 4: V held in registers.  One workgroup per compute unit, alpha fixed per
// workgroup, one wavefront per 16-wide gamma tile (c / 16 wavefronts).  Wavefront w
// keeps v[de][s] = V[al][de][be = g*SB + s][ga = 16*w + c] for all four delta in
// registers for the whole kernel, so the LDS holds only rows: 16-row tiles of the
// alpha slab of X (16 x 4b floats, row stride 4b + 4 so that the sixteen lanes of a
// lane group read disjoint banks), double-buffered with one barrier per tile.  A lane's
// 16-byte LDS read of X[row c][be = g*SB + s][0..3] gives its A operand for all four
// delta, and its four accumulators give one 16-byte store of Y per output row.  Full
// tiles run in the loop (stores unconditional, so waiting for the next tile's rows does
// not wait for the stores); the partial tile, if any, is peeled off.
// ---------------------------------------------------------------------------------
template <int B_, int C_, int GS_ = 1>
struct KV {
  static constexpr int GS = GS_;                 // workgroups sharing one row tile (gamma split)
  static constexpr int NW = C_ / 16 / GS_, NT = 64 * NW;
  static constexpr int SB = B_ / 4;
  static constexpr int ROWF = 4 * B_;            // floats of one row's alpha slab
  static constexpr int LXS = ROWF + 4;
  static constexpr int TILE = 16 * LXS;
  static constexpr int NF4 = 16 * ROWF / 4;      // float4s per row tile
  static constexpr int NPF = (NF4 + NT - 1) / NT;
  static constexpr size_t LDS = (size_t)2 * TILE * 4;
  static constexpr bool OK = B_ % 4 == 0 && C_ % (16 * GS_) == 0 && NW >= 1 && NW <= 16 && LDS <= kMaxLds;
};

// Four consecutive inputs as loaded (raw), widened to fp32 only when staged in LDS, so
// that a prefetch does not wait for its own data.
template <class TIn> struct Raw4;
template <> struct Raw4<float> { typedef f4 type; };
template <> struct Raw4<uint16_t> { typedef uint2 type; };
__device__ __forceinline__ f4 load_raw4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ uint2 load_raw4(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ f4 widen4(f4 v) { return v; }
__device__ __forceinline__ f4 widen4(uint2 v) {
  return f4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
            __uint_as_float(v.y & 0xffff0000u)};
}

// Wait, before a row-tile loop, for the registers loaded ahead of it (V and the first
// prefetch).  The loop issues each prefetch before its tile's stores, so on the back edge a
// prefetch can be waited for while the stores stay in flight; without this wait the loop
// head would merge that state with the preheader's (loads outstanding) and wait for every
// store of the previous tile.
__device__ __forceinline__ void settle1(float v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void settle1(f4 v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void settle1(uint2 v) { asm volatile("" ::"v"(v.x), "v"(v.y)); }
typedef short s4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void settle1(s4 v) { asm volatile("" ::"v"(v)); }
template <class T, int A>
__device__ __forceinline__ void settle(const T (&v)[A]) {
#pragma unroll
  for (int i = 0; i < A; ++i) settle1(v[i]);
}
template <class T, int A, int B>
__device__ __forceinline__ void settle(const T (&v)[A][B]) {
#pragma unroll
  for (int i = 0; i < A; ++i) settle(v[i]);
}

template <int B_, int C_, int GS_, class TIn, class TOut>
__global__ __launch_bounds__((KV<B_, C_, GS_>::NT)) void ks_vreg_kernel(int64_t N, int a_count,
                                                                    const TIn* __restrict__ x,
                                                                    const TIn* __restrict__ vals,
                                                                    TOut* __restrict__ y) {
  using K = KV<B_, C_, GS_>;
  extern __shared__ float lds[];   // 2 x TILE
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int al = blockIdx.x % a_count;
  const int h = (blockIdx.x / a_count) % GS_;    // which gamma share
  const int w = h * K::NW + (tid >> 6);          // this wavefront's gamma tile
  const int64_t step = gridDim.x / (a_count * GS_);   // workgroups per (alpha, share); grid is a multiple
  const int64_t ntile = (N + 15) / 16, nfull = N / 16;
  const int64_t in_w = (int64_t)a_count * K::ROWF, out_w = (int64_t)a_count * C_ * 4;
  const TIn* xa = x + (int64_t)al * K::ROWF;
  TOut* ya = y + ((int64_t)al * C_ + 16 * w + c) * 4;

  typedef typename Raw4<TIn>::type R4;
  R4 pf[K::NPF];
  auto fetch = [&](int64_t tile) {
#pragma unroll
    for (int t = 0; t < K::NPF; ++t) {
      const int f = tid + t * K::NT;
      R4 v = {};
      if (K::NF4 % K::NT == 0 || f < K::NF4) {
        const int r = f / (K::ROWF / 4), o = 4 * (f % (K::ROWF / 4));
        const int64_t row = tile * 16 + r;
        if (tile < ntile && row < N) v = load_raw4(xa + row * in_w + o);
      }
      pf[t] = v;
    }
  };
  auto stash = [&](float* buf) {
#pragma unroll
    for (int t = 0; t < K::NPF; ++t) {
      const int f = tid + t * K::NT;
      if (K::NF4 % K::NT == 0 || f < K::NF4) {
        const int r = f / (K::ROWF / 4), o = 4 * (f % (K::ROWF / 4));
        *reinterpret_cast<f4*>(buf + r * K::LXS + o) = widen4(pf[t]);
      }
    }
  };

  int64_t tile = blockIdx.x / (a_count * GS_);
  fetch(tile);
  float v[4][K::SB];
  const TIn* V = vals + (int64_t)al * 4 * B_ * C_;
#pragma unroll
  for (int de = 0; de < 4; ++de)
#pragma unroll
    for (int s = 0; s < K::SB; ++s) v[de][s] = widen(V[((int64_t)de * B_ + g * K::SB + s) * C_ + 16 * w + c]);
  stash(lds);
  fetch(tile + step);
  settle(v);
  settle(pf);
  __syncthreads();

  auto compute = [&](const float* xs, f4 (&acc)[4]) {
#pragma unroll
    for (int de = 0; de < 4; ++de) acc[de] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < K::SB; ++s) {
      const f4 xv = *reinterpret_cast<const f4*>(xs + c * K::LXS + (g * K::SB + s) * 4);
#pragma unroll
      for (int de = 0; de < 4; ++de) acc[de] = mfma(xv[de], v[de][s], acc[de]);
    }
  };
  // Per tile: products, the next tile's rows into LDS, the loads two tiles ahead, then
  // this tile's stores.  The vector-memory counter retires in issue order, so loads issued
  // before the stores can be waited for (next iteration's stash) without waiting for them.
  int it = 0;
  for (; tile < nfull; tile += step, ++it) {
    f4 acc[4];
    compute(lds + (it & 1) * K::TILE, acc);
    stash(lds + ((it + 1) & 1) * K::TILE);
    fetch(tile + 2 * step);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int vv = 0; vv < 4; ++vv)
      store4(ya + (tile * 16 + 4 * g + vv) * out_w, f4{acc[0][vv], acc[1][vv], acc[2][vv], acc[3][vv]});
    __syncthreads();
  }
  if (tile < ntile) {   // the partial tile
    f4 acc[4];
    compute(lds + (it & 1) * K::TILE, acc);
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) {
      const int64_t row = tile * 16 + 4 * g + vv;
      if (row < N) store4(ya + row * out_w, f4{acc[0][vv], acc[1][vv], acc[2][vv], acc[3][vv]});
    }
  }
}

// ---------------------------------------------------------------------------------
// d = 4 with a long contraction (b large, c small; e.g. the transposed ViT pattern
// (192, 48) of the input gradient): V in registers as above, but each gamma tile's
// contraction over beta is split over four wavefronts (a quarter of the K steps each, so
// 48 registers of V per lane at b = 192).  After a row tile's products the four partial
// 16 x 16 x 4-delta tiles meet in LDS; wavefront quarter q adds the four partials in
// quarter order (fixed, deterministic) for output row 4g + q and stores it.
// ---------------------------------------------------------------------------------
template <int B_, int C_>
struct KVK {
  static constexpr int KSP = 4;                    // contraction split (one output row each)
  static constexpr int NWG = C_ / 16;              // gamma tiles
  static constexpr int NW = NWG * KSP, NT = 64 * NW;
  static constexpr int SB = B_ / 4, SBK = SB / KSP;
  static constexpr int ROWF = 4 * B_;
  static constexpr int LXS = ROWF + 4;
  static constexpr int TILE = 16 * LXS;
  static constexpr int NF4 = 16 * ROWF / 4;
  static constexpr int NPF = (NF4 + NT - 1) / NT;
  static constexpr int RED = NW * 64 * 16;         // floats: every wavefront's 16 accumulators per lane
  static constexpr size_t LDS = ((size_t)2 * TILE + RED) * 4;
  static constexpr bool OK = B_ % (4 * KSP) == 0 && C_ % 16 == 0 && NW <= 16 && LDS <= kMaxLds;
};

template <int B_, int C_, class TIn, class TOut>
__global__ __launch_bounds__((KVK<B_, C_>::NT)) void ks_vregk_kernel(int64_t N, int a_count, const TIn* __restrict__ x,
                                                                 const TIn* __restrict__ vals,
                                                                 TOut* __restrict__ y) {
  using K = KVK<B_, C_>;
  extern __shared__ float lds[];   // 2 x TILE rows, then RED
  f4* red = reinterpret_cast<f4*>(lds + 2 * K::TILE);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15, wv = tid >> 6;
  const int gt = wv % K::NWG, kq = wv / K::NWG;   // gamma tile, contraction quarter
  const int al = blockIdx.x % a_count;
  const int64_t step = gridDim.x / a_count;
  const int64_t ntile = (N + 15) / 16, nfull = N / 16;
  const int64_t in_w = (int64_t)a_count * K::ROWF, out_w = (int64_t)a_count * C_ * 4;
  const TIn* xa = x + (int64_t)al * K::ROWF;
  TOut* ya = y + ((int64_t)al * C_ + 16 * gt + c) * 4;

  typedef typename Raw4<TIn>::type R4;
  R4 pf[K::NPF];
  auto fetch = [&](int64_t tile) {
#pragma unroll
    for (int t = 0; t < K::NPF; ++t) {
      const int f = tid + t * K::NT;
      R4 v = {};
      if (K::NF4 % K::NT == 0 || f < K::NF4) {
        const int r = f / (K::ROWF / 4), o = 4 * (f % (K::ROWF / 4));
        const int64_t row = tile * 16 + r;
        if (tile < ntile && row < N) v = load_raw4(xa + row * in_w + o);
      }
      pf[t] = v;
    }
  };
  auto stash = [&](float* buf) {
#pragma unroll
    for (int t = 0; t < K::NPF; ++t) {
      const int f = tid + t * K::NT;
      if (K::NF4 % K::NT == 0 || f < K::NF4) {
        const int r = f / (K::ROWF / 4), o = 4 * (f % (K::ROWF / 4));
        *reinterpret_cast<f4*>(buf + r * K::LXS + o) = widen4(pf[t]);
      }
    }
  };

  int64_t tile = blockIdx.x / a_count;
  fetch(tile);
  // v[de][s] = V[al][de][be = g*SB + kq*SBK + s][ga = 16*gt + c]
  float v[4][K::SBK];
  const TIn* V = vals + (int64_t)al * 4 * B_ * C_;
#pragma unroll
  for (int de = 0; de < 4; ++de)
#pragma unroll
    for (int s = 0; s < K::SBK; ++s)
      v[de][s] = widen(V[((int64_t)de * B_ + g * K::SB + kq * K::SBK + s) * C_ + 16 * gt + c]);
  stash(lds);
  fetch(tile + step);
  settle(v);
  settle(pf);
  __syncthreads();

  // the quarter's partial tile -> LDS as red[wave][lane][vv] = f4 over delta; then this
  // wavefront's output row vv = kq, summed over the quarters of its gamma tile
  auto compute_and_reduce = [&](const float* xs) {
    f4 acc[4];
#pragma unroll
    for (int de = 0; de < 4; ++de) acc[de] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < K::SBK; ++s) {
      const f4 xv = *reinterpret_cast<const f4*>(xs + c * K::LXS + (g * K::SB + kq * K::SBK + s) * 4);
#pragma unroll
      for (int de = 0; de < 4; ++de) acc[de] = mfma(xv[de], v[de][s], acc[de]);
    }
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) red[(wv * 64 + lane) * 4 + vv] = f4{acc[0][vv], acc[1][vv], acc[2][vv], acc[3][vv]};
    __syncthreads();
    f4 sum = red[((0 * K::NWG + gt) * 64 + lane) * 4 + kq];
#pragma unroll
    for (int q = 1; q < K::KSP; ++q) sum += red[((q * K::NWG + gt) * 64 + lane) * 4 + kq];
    return sum;   // Y[row 4g + kq][ga = 16*gt + c][0..3]
  };
  int it = 0;
  for (; tile < nfull; tile += step, ++it) {   // same order as ks_vreg_kernel
    const f4 o = compute_and_reduce(lds + (it & 1) * K::TILE);
    stash(lds + ((it + 1) & 1) * K::TILE);
    fetch(tile + 2 * step);
    __builtin_amdgcn_sched_barrier(0);
    store4(ya + (tile * 16 + 4 * g + kq) * out_w, o);
    __syncthreads();
  }
  if (tile < ntile) {   // the partial tile
    const f4 o = compute_and_reduce(lds + (it & 1) * K::TILE);
    const int64_t row = tile * 16 + 4 * g + kq;
    if (row < N) store4(ya + row * out_w, o);
  }
}

// ---------------------------------------------------------------------------------
// bf16 inputs, d = 4: the same two kernels on bf16 matrix instructions
// (v_mfma_f32_16x16x16_bf16, fp32 accumulation).  Rows stay bf16 in LDS.  A K step covers
// 16 beta values; lane group g takes beta = 16s + 4g + u (u < 4) in both operands.  A lane
// reads its 4 beta x 4 delta values of a row as 32 contiguous bytes and regroups them into
// one 4-value operand per delta with byte permutes; its V operands (4 beta of one gamma, per
// delta and step) sit in registers as packed bf16.
// ---------------------------------------------------------------------------------
typedef short s4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma16(s4 a, s4 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0); }

// 4 beta x 4 delta bf16 (beta-major, as in a row) -> op[de] = {beta 0..3 of delta de}
__device__ __forceinline__ void split_deltas(u4v lo, u4v hi, s4 (&op)[4]) {
  // words: lo = beta0 (d0d1, d2d3), beta1 (d0d1, d2d3); hi = beta2, beta3
  const unsigned LO = 0x05040100u, HI = 0x07060302u;   // low / high halves of (S1, S0)
  op[0] = __builtin_bit_cast(s4, (u2v{__builtin_amdgcn_perm(lo[2], lo[0], LO), __builtin_amdgcn_perm(hi[2], hi[0], LO)}));
  op[1] = __builtin_bit_cast(s4, (u2v{__builtin_amdgcn_perm(lo[2], lo[0], HI), __builtin_amdgcn_perm(hi[2], hi[0], HI)}));
  op[2] = __builtin_bit_cast(s4, (u2v{__builtin_amdgcn_perm(lo[3], lo[1], LO), __builtin_amdgcn_perm(hi[3], hi[1], LO)}));
  op[3] = __builtin_bit_cast(s4, (u2v{__builtin_amdgcn_perm(lo[3], lo[1], HI), __builtin_amdgcn_perm(hi[3], hi[1], HI)}));
}

__device__ __forceinline__ s4 vals4(const uint16_t* p, int stride) {   // 4 bf16 at p, p + stride, ...
  return s4{(short)p[0], (short)p[stride], (short)p[2 * stride], (short)p[3 * stride]};
}

template <int B_>
struct Row16 {
  static constexpr int ROWE = 4 * B_;                        // bf16 of one row's alpha slab
  static constexpr int LXB = (ROWE * 2 + 127) / 128 * 128 + 64;   // row pitch in bytes: /4 = 16 mod 32
  static constexpr int TILEB = 16 * LXB;
  static constexpr int NU2 = ROWE / 4;                        // 8-byte pieces per row
};

template <int B_, int C_>
struct KV16 {
  static constexpr int NW = C_ / 16, NT = 64 * NW;
  static constexpr int SK = B_ / 16;                          // K steps
  using R = Row16<B_>;
  static constexpr int NP = 16 * R::NU2;                      // pieces per row tile
  static constexpr int NPF = (NP + NT - 1) / NT;
  static constexpr size_t LDS = (size_t)2 * R::TILEB;
  static constexpr bool OK = B_ % 16 == 0 && C_ % 16 == 0 && NW >= 1 && NW <= 16 && LDS <= kMaxLds;
};

template <int B_, int C_, class TOut>
__global__ __launch_bounds__((KV16<B_, C_>::NT)) void ks_vreg16_kernel(int64_t N, int a_count,
                                                                     const uint16_t* __restrict__ x,
                                                                     const uint16_t* __restrict__ vals,
                                                                     TOut* __restrict__ y) {
  using K = KV16<B_, C_>;
  using R = typename K::R;
  extern __shared__ float lds[];
  unsigned char* lb = reinterpret_cast<unsigned char*>(lds);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15, w = tid >> 6;
  const int al = blockIdx.x % a_count;
  const int64_t step = gridDim.x / a_count;
  const int64_t ntile = (N + 15) / 16, nfull = N / 16;
  const int64_t in_w = (int64_t)a_count * R::ROWE, out_w = (int64_t)a_count * C_ * 4;
  const uint16_t* xa = x + (int64_t)al * R::ROWE;
  TOut* ya = y + ((int64_t)al * C_ + 16 * w + c) * 4;

  uint2 pf[K::NPF];
  auto fetch = [&](int64_t tile) {
#pragma unroll
    for (int t = 0; t < K::NPF; ++t) {
      const int f = tid + t * K::NT;
      uint2 v = {0u, 0u};
      if (K::NP % K::NT == 0 || f < K::NP) {
        const int r = f / R::NU2, o = 4 * (f % R::NU2);
        const int64_t row = tile * 16 + r;
        if (tile < ntile && row < N) v = *reinterpret_cast<const uint2*>(xa + row * in_w + o);
      }
      pf[t] = v;
    }
  };
  auto stash = [&](unsigned char* buf) {
#pragma unroll
    for (int t = 0; t < K::NPF; ++t) {
      const int f = tid + t * K::NT;
      if (K::NP % K::NT == 0 || f < K::NP) {
        const int r = f / R::NU2, o = 4 * (f % R::NU2);
        *reinterpret_cast<uint2*>(buf + r * R::LXB + 2 * o) = pf[t];
      }
    }
  };

  int64_t tile = blockIdx.x / a_count;
  fetch(tile);
  s4 v[4][K::SK];   // V[al][de][16s + 4g + u][16w + c], u = 0..3
  const uint16_t* V = vals + (int64_t)al * 4 * B_ * C_;
#pragma unroll
  for (int de = 0; de < 4; ++de)
#pragma unroll
    for (int s = 0; s < K::SK; ++s) v[de][s] = vals4(V + ((int64_t)de * B_ + 16 * s + 4 * g) * C_ + 16 * w + c, C_);
  stash(lb);
  fetch(tile + step);
  settle(v);
  settle(pf);
  __syncthreads();

  auto compute = [&](const unsigned char* xs, f4 (&acc)[4]) {
#pragma unroll
    for (int de = 0; de < 4; ++de) acc[de] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < K::SK; ++s) {
      const unsigned char* p = xs + c * R::LXB + (16 * s + 4 * g) * 8;
      s4 op[4];
      split_deltas(*reinterpret_cast<const u4v*>(p), *reinterpret_cast<const u4v*>(p + 16), op);
#pragma unroll
      for (int de = 0; de < 4; ++de) acc[de] = mfma16(op[de], v[de][s], acc[de]);
    }
  };
  int it = 0;
  for (; tile < nfull; tile += step, ++it) {   // same order as ks_vreg_kernel
    f4 acc[4];
    compute(lb + (it & 1) * R::TILEB, acc);
    stash(lb + ((it + 1) & 1) * R::TILEB);
    fetch(tile + 2 * step);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int vv = 0; vv < 4; ++vv)
      store4(ya + (tile * 16 + 4 * g + vv) * out_w, f4{acc[0][vv], acc[1][vv], acc[2][vv], acc[3][vv]});
    __syncthreads();
  }
  if (tile < ntile) {
    f4 acc[4];
    compute(lb + (it & 1) * R::TILEB, acc);
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) {
      const int64_t row = tile * 16 + 4 * g + vv;
      if (row < N) store4(ya + row * out_w, f4{acc[0][vv], acc[1][vv], acc[2][vv], acc[3][vv]});
    }
  }
}

// The split-contraction kernel on bf16: quarter kq of a gamma tile takes beta in
// [kq*B/4, (kq+1)*B/4), K steps of 16 inside it.
template <int B_, int C_>
struct KVK16 {
  static constexpr int KSP = 4;
  static constexpr int NWG = C_ / 16;
  static constexpr int NW = NWG * KSP, NT = 64 * NW;
  static constexpr int QB = B_ / KSP, SKQ = QB / 16;         // beta per quarter, K steps per quarter
  using R = Row16<B_>;
  static constexpr int NP = 16 * R::NU2;
  static constexpr int NPF = (NP + NT - 1) / NT;
  static constexpr int RED = NW * 64 * 16;                    // floats
  static constexpr size_t LDS = (size_t)2 * R::TILEB + (size_t)RED * 4;
  static constexpr bool OK = B_ % (16 * KSP) == 0 && C_ % 16 == 0 && NW <= 16 && LDS <= kMaxLds;
};

template <int B_, int C_, class TOut>
__global__ __launch_bounds__((KVK16<B_, C_>::NT)) void ks_vregk16_kernel(int64_t N, int a_count,
                                                                       const uint16_t* __restrict__ x,
                                                                       const uint16_t* __restrict__ vals,
                                                                       TOut* __restrict__ y) {
  using K = KVK16<B_, C_>;
  using R = typename K::R;
  extern __shared__ float lds[];
  unsigned char* lb = reinterpret_cast<unsigned char*>(lds);
  f4* red = reinterpret_cast<f4*>(lb + 2 * R::TILEB);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15, wv = tid >> 6;
  const int gt = wv % K::NWG, kq = wv / K::NWG;
  const int al = blockIdx.x % a_count;
  const int64_t step = gridDim.x / a_count;
  const int64_t ntile = (N + 15) / 16, nfull = N / 16;
  const int64_t in_w = (int64_t)a_count * R::ROWE, out_w = (int64_t)a_count * C_ * 4;
  const uint16_t* xa = x + (int64_t)al * R::ROWE;
  TOut* ya = y + ((int64_t)al * C_ + 16 * gt + c) * 4;

  uint2 pf[K::NPF];
  auto fetch = [&](int64_t tile) {
#pragma unroll
    for (int t = 0; t < K::NPF; ++t) {
      const int f = tid + t * K::NT;
      uint2 v = {0u, 0u};
      if (K::NP % K::NT == 0 || f < K::NP) {
        const int r = f / R::NU2, o = 4 * (f % R::NU2);
        const int64_t row = tile * 16 + r;
        if (tile < ntile && row < N) v = *reinterpret_cast<const uint2*>(xa + row * in_w + o);
      }
      pf[t] = v;
    }
  };
  auto stash = [&](unsigned char* buf) {
#pragma unroll
    for (int t = 0; t < K::NPF; ++t) {
      const int f = tid + t * K::NT;
      if (K::NP % K::NT == 0 || f < K::NP) {
        const int r = f / R::NU2, o = 4 * (f % R::NU2);
        *reinterpret_cast<uint2*>(buf + r * R::LXB + 2 * o) = pf[t];
      }
    }
  };

  int64_t tile = blockIdx.x / a_count;
  fetch(tile);
  s4 v[4][K::SKQ];   // V[al][de][kq*QB + 16s + 4g + u][16gt + c]
  const uint16_t* V = vals + (int64_t)al * 4 * B_ * C_;
#pragma unroll
  for (int de = 0; de < 4; ++de)
#pragma unroll
    for (int s = 0; s < K::SKQ; ++s)
      v[de][s] = vals4(V + ((int64_t)de * B_ + kq * K::QB + 16 * s + 4 * g) * C_ + 16 * gt + c, C_);
  stash(lb);
  fetch(tile + step);
  settle(v);
  settle(pf);
  __syncthreads();

  auto compute_and_reduce = [&](const unsigned char* xs) {
    f4 acc[4];
#pragma unroll
    for (int de = 0; de < 4; ++de) acc[de] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < K::SKQ; ++s) {
      const unsigned char* p = xs + c * R::LXB + (kq * K::QB + 16 * s + 4 * g) * 8;
      s4 op[4];
      split_deltas(*reinterpret_cast<const u4v*>(p), *reinterpret_cast<const u4v*>(p + 16), op);
#pragma unroll
      for (int de = 0; de < 4; ++de) acc[de] = mfma16(op[de], v[de][s], acc[de]);
    }
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) red[(wv * 64 + lane) * 4 + vv] = f4{acc[0][vv], acc[1][vv], acc[2][vv], acc[3][vv]};
    __syncthreads();
    f4 sum = red[((0 * K::NWG + gt) * 64 + lane) * 4 + kq];
#pragma unroll
    for (int q = 1; q < K::KSP; ++q) sum += red[((q * K::NWG + gt) * 64 + lane) * 4 + kq];
    return sum;
  };
  int it = 0;
  for (; tile < nfull; tile += step, ++it) {   // same order as ks_vreg_kernel
    const f4 o = compute_and_reduce(lb + (it & 1) * R::TILEB);
    stash(lb + ((it + 1) & 1) * R::TILEB);
    fetch(tile + 2 * step);
    __builtin_amdgcn_sched_barrier(0);
    store4(ya + (tile * 16 + 4 * g + kq) * out_w, o);
    __syncthreads();
  }
  if (tile < ntile) {
    const f4 o = compute_and_reduce(lb + (it & 1) * R::TILEB);
    const int64_t row = tile * 16 + 4 * g + kq;
    if (row < N) store4(ya + row * out_w, o);
  }
}

struct KvkEntry {
  int b, c;
  size_t lds[2];          // [x and vals bf16]
  int nt;
  const void* fn[2][2];   // [x and vals bf16][y bf16]
};
#define KVK_ENTRY(B, C)                                                                                   \
  KvkEntry{B, C, {KVK<B, C>::LDS, KVK16<B, C>::LDS}, KVK<B, C>::NT,                                        \
           {{(const void*)&ks_vregk_kernel<B, C, float, float>, (const void*)&ks_vregk_kernel<B, C, float, uint16_t>}, \
            {(const void*)&ks_vregk16_kernel<B, C, float>, (const void*)&ks_vregk16_kernel<B, C, uint16_t>}}}
// d = 4 shapes with the contraction split: the transposed ViT-S/16 MLP pattern (192, 48).
const KvkEntry kKvkTable[] = {KVK_ENTRY(192, 48)};
static_assert(KVK<192, 48>::OK && KVK16<192, 48>::OK && KVK16<192, 48>::NT == KVK<192, 48>::NT,
              "the split-contraction KS shape fits the LDS");

struct KsEntry {
  int b, c, d;
  bool ok;
  size_t lds;
  const void* fn[2][2];   // [x and vals bf16][y bf16]
};

#define KS_ENTRY(B, C, D)                                                                                      \
  KsEntry{B, C, D, KS<B, C, D>::OK, KS<B, C, D>::LDS,                                                          \
          {{(const void*)&ks_mfma_kernel<KS<B, C, D>, float, float>,                                          \
            (const void*)&ks_mfma_kernel<KS<B, C, D>, float, uint16_t>},                                      \
           {(const void*)&ks_mfma_kernel<KS<B, C, D>, uint16_t, float>,                                       \
            (const void*)&ks_mfma_kernel<KS<B, C, D>, uint16_t, uint16_t>}}}

// The ViT-S/16 MLP pattern (b, c, d) = (48, 192, 4), plus the Kronecker-layer factors
// written as KS matrices with d = 1.
const KsEntry kKsTable[] = {
    KS_ENTRY(48, 192, 4), KS_ENTRY(32, 128, 1), KS_ENTRY(128, 32, 1), KS_ENTRY(64, 64, 1),
};

const KsEntry* ks_find(int b, int c, int d) {
  for (const KsEntry& e : kKsTable)
    if (e.b == b && e.c == c && e.d == d && e.ok) return &e;
  return nullptr;
}

int device_cus_ks() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 256;
  return v;
}

struct KvEntry {
  int b, c, gs;
  size_t lds[2];          // [x and vals bf16]
  int nt;
  const void* fn[2][2];   // [x and vals bf16][y bf16]
};
// bf16 inputs run on bf16 matrix instructions (one workgroup per row tile, GS = 1)
#define KV_ENTRY(B, C)                                                                                            \
  KvEntry{B, C, 1, {KV<B, C, 1>::LDS, KV16<B, C>::LDS}, KV<B, C, 1>::NT,                                          \
          {{(const void*)&ks_vreg_kernel<B, C, 1, float, float>, (const void*)&ks_vreg_kernel<B, C, 1, float, uint16_t>}, \
           {(const void*)&ks_vreg16_kernel<B, C, float>, (const void*)&ks_vreg16_kernel<B, C, uint16_t>}}}
// d = 4 shapes with V in registers: the ViT-S/16 MLP pattern (b, c) = (48, 192), one
// workgroup per row tile (splitting the gamma tiles over two or three workgroups was
// measured no faster).
const KvEntry kKvTable[] = {KV_ENTRY(48, 192)};
static_assert(KV16<48, 192>::OK && KV16<48, 192>::NT == KV<48, 192, 1>::NT, "the bf16 register KS shape fits");

const KvEntry* kv_find(int b, int c, int d) {
  if (d != 4) return nullptr;
  for (const KvEntry& e : kKvTable)
    if (e.b == b && e.c == c) return &e;
  return nullptr;
}

const KvkEntry* kvk_find(int b, int c, int d) {
  if (d != 4) return nullptr;
  for (const KvkEntry& e : kKvkTable)
    if (e.b == b && e.c == c) return &e;
  return nullptr;
}

hipError_t launch_ks_vregk(const KvkEntry* e, const KSArgs& k, hipStream_t s) {
  const void* fn = e->fn[k.dtype == KRON_BF16][k.out_dtype == KRON_BF16];
  const size_t lds = e->lds[k.dtype == KRON_BF16];
  (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  int per_cu = 1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, e->nt, lds) != hipSuccess || per_cu < 1)
    per_cu = 1;
  int64_t per_alpha = (int64_t)per_cu * device_cus_ks() / k.a;
  if (per_alpha < 1) per_alpha = 1;
  const int64_t tiles = (k.N + 15) / 16;
  if (per_alpha > tiles) per_alpha = tiles;
  const int grid = (int)(per_alpha * k.a);
  void* args[] = {(void*)&k.N, (void*)&k.a, (void*)&k.x, (void*)&k.vals, (void*)&k.y};
  return hipLaunchKernel(fn, dim3(grid), dim3(e->nt), args, lds, s);
}

hipError_t launch_ks_vreg(const KvEntry* e, const KSArgs& k, hipStream_t s) {
  const void* fn = e->fn[k.dtype == KRON_BF16][k.out_dtype == KRON_BF16];
  const size_t lds = e->lds[k.dtype == KRON_BF16];
  (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  int per_cu = 1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, e->nt, lds) != hipSuccess || per_cu < 1)
    per_cu = 1;
  // workgroups per (alpha, gamma share): as many as fit, and no more than the row tiles
  int64_t per_share = (int64_t)per_cu * device_cus_ks() / (k.a * e->gs);
  if (per_share < 1) per_share = 1;
  const int64_t tiles = (k.N + 15) / 16;
  if (per_share > tiles) per_share = tiles;
  const int grid = (int)(per_share * k.a * e->gs);
  void* args[] = {(void*)&k.N, (void*)&k.a, (void*)&k.x, (void*)&k.vals, (void*)&k.y};
  return hipLaunchKernel(fn, dim3(grid), dim3(e->nt), args, lds, s);
}

}  // namespace

bool ks_mfma_supported(int a, int b, int c, int d) {
  (void)a;
  return kv_find(b, c, d) != nullptr || kvk_find(b, c, d) != nullptr || ks_find(b, c, d) != nullptr;
}

hipError_t launch_ks_mfma(const KSArgs& k, hipStream_t s) {
  if (k.N == 0) return hipSuccess;
  if (const KvEntry* ev = kv_find(k.b, k.c, k.d)) return launch_ks_vreg(ev, k, s);
  if (const KvkEntry* ek = kvk_find(k.b, k.c, k.d)) return launch_ks_vregk(ek, k, s);
  const KsEntry* e = ks_find(k.b, k.c, k.d);
  if (!e) return hipErrorInvalidValue;
  if (k.N == 0) return hipSuccess;
  const void* fn = e->fn[k.dtype == KRON_BF16][k.out_dtype == KRON_BF16];
  (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)e->lds);
  // one workgroup per compute unit, split evenly between the alphas
  int per_alpha = device_cus_ks() / k.a;
  if (per_alpha < 1) per_alpha = 1;
  const int64_t tasks = (k.N + 15) / 16 * 4;
  const int64_t need = (tasks + kWaves - 1) / kWaves;
  if (per_alpha > need) per_alpha = (int)need;
  const int grid = per_alpha * k.a;
  void* args[] = {(void*)&k.N, (void*)&k.a, (void*)&k.x, (void*)&k.vals, (void*)&k.y};
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, e->lds, s);
}

}  // namespace kron
