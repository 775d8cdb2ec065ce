// Fused chain of Kronecker-sparse factors: Y = X K_1 K_2 ... K_F, each K_f with support
// I_a (x) 1_{b x c} (x) I_d ("Fast Inference with Kronecker-Sparse Matrices", abstract: KS
// matrices and products of them, such as butterfly and Monarch factors; the triple
// Kronecker product A (x) B (x) C is the three-factor case by the mixed-product rule).
// A workgroup takes a tile of rows, holds them in LDS in fp32 through every factor
// (two row buffers, alternating), and writes only the last factor's output to HBM.
#include "kron_internal.h"

namespace kron {
namespace {

constexpr int kChainThreads = 1024;
constexpr int kChainMaxRows = 16;
constexpr size_t kChainLds = 160 * 1024;
constexpr int kCmMaxWidth = 1248;   // two 16-row buffers of (width rounded to 32, + 1) fp32 in 160 KB
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float load_in(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_in(const uint16_t* p, int64_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}

template <typename TIn>
__global__ __launch_bounds__(kChainThreads) void ks_chain_kernel(ChainArgs A, int T) {
  extern __shared__ float s[];
  float* in = s;
  float* out = s + (size_t)T * A.maxw;
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.x * T;
  const int rows = (int)(A.N - row0 < T ? A.N - row0 : T);
  const int w0 = A.f[0].a * A.f[0].b * A.f[0].d;
  const TIn* x = static_cast<const TIn*>(A.x);
  for (int i = tid; i < rows * w0; i += kChainThreads) {
    const int t = i / w0, col = i - t * w0;
    in[t * A.maxw + col] = load_in(x, (row0 + t) * w0 + col);
  }
  __syncthreads();
  for (int fi = 0; fi < A.nf; ++fi) {
    const int a = A.f[fi].a, b = A.f[fi].b, c = A.f[fi].c, d = A.f[fi].d;
    const int wout = a * c * d;
    const TIn* V = static_cast<const TIn*>(A.f[fi].vals);
    const bool last = fi == A.nf - 1;
    // a thread owns output columns; each value is loaded once per tile and applied to
    // every row of the tile from LDS
    for (int col = tid; col < wout; col += kChainThreads) {
      const int de = col % d, rest = col / d, ga = rest % c, al = rest / c;
      const float* ir = in + (al * b) * d + de;
      const TIn* v = V + ((int64_t)(al * d + de) * b) * c + ga;
      float acc[kChainMaxRows];
#pragma unroll
      for (int t = 0; t < kChainMaxRows; ++t) acc[t] = 0.f;
#pragma unroll 8
      for (int be = 0; be < b; ++be) {
        const float vv = load_in(v, (int64_t)be * c);
        const float* ib = ir + be * d;
#pragma unroll
        for (int t = 0; t < kChainMaxRows; ++t)
          if (t < rows) acc[t] = fmaf(ib[t * A.maxw], vv, acc[t]);
      }
#pragma unroll
      for (int t = 0; t < kChainMaxRows; ++t) {
        if (t < rows) {
          if (last)
            A.y[(row0 + t) * wout + col] = acc[t];
          else
            out[t * A.maxw + col] = acc[t];
        }
      }
    }
    __syncthreads();
    float* tmp = in;
    in = out;
    out = tmp;
  }
}

// Matrix-core chain for rows of at most kCmMaxWidth values.  Factor f is a batch of small
// products, one per block (alpha, delta): Y_blk (rows x c) = X_blk (rows x b) V[alpha][delta]
// (b x c), X_blk's columns being the input columns (alpha*b + beta)*d + delta.  A persistent
// workgroup takes 16-row tiles; the tile sits in LDS (fp32) through every factor in two
// buffers that swap roles, and the next tile's rows wait in registers meanwhile.  A
// wavefront (eight per workgroup) takes tasks (alpha, delta, 16-column gamma tile) and runs
// 16x16x4 fp32 products over beta with the factor as the first operand: lane 16g + i
// supplies V[alpha][delta][4s + g][gamma tile + i] (from memory, cached) and row i of the
// tile at beta = 4s + g (from LDS), and receives row i's outputs at gamma tile + 4g + v.
// Every lane thus reads and writes one row, and the row pitch (1 mod 32 floats) keeps the
// LDS accesses of a half-wavefront within two-way bank conflicts for any d.  Zero padding
// covers b and c that are not multiples of 4 and 16.
constexpr int kCmRows = 16;
constexpr int kCmThreads = 512;
constexpr int kCmWaves = kCmThreads / 64;
constexpr int kCmPre = 10;      // float4 of the next tile per thread: 16 rows x 1248 values
constexpr int kCmKChunk = 8;    // beta steps whose loads are issued together
constexpr size_t kCmLds = 160 * 1024;

__device__ __forceinline__ float4 load4_in(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4_in(const uint16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                     __uint_as_float(v.y & 0xffff0000u));
}

// A tile's output rows from LDS to y: a fixed number of unconditional 16-byte stores per
// thread (items past the tile's last row or column store that row's or column's own value
// again).  A fixed count lets the wait for the next tile's prefetch, issued before these
// stores, leave them in flight (the vector-memory counter retires in issue order).
constexpr int kCmStores = (kCmRows * 1248 / 4 + kCmThreads - 1) / kCmThreads;

__device__ __forceinline__ void store_tile(float* __restrict__ y, const float* ob, int LD, int64_t tile, int64_t N,
                                           int wl, int ql) {
  const int rmax = (int)(N - tile * kCmRows < kCmRows ? N - tile * kCmRows : kCmRows) - 1;
#pragma unroll
  for (int u = 0; u < kCmStores; ++u) {
    const int e = threadIdx.x + u * kCmThreads;
    int r = e & (kCmRows - 1), c4 = e / kCmRows;
    r = r < rmax ? r : rmax;
    c4 = c4 < ql - 1 ? c4 : ql - 1;
    const float* p = ob + r * LD + 4 * c4;
    *reinterpret_cast<float4*>(y + (tile * kCmRows + r) * wl + 4 * c4) = make_float4(p[0], p[1], p[2], p[3]);
  }
}

// x = quo * dv + rem for 0 <= x < 2^24, dv >= 1: the float quotient is off by at most one,
// which one correction step fixes.
__device__ __forceinline__ void divmod(int x, int dv, float inv, int& quo, int& rem) {
  int qq = __float2int_rz((float)x * inv);
  int rr = x - qq * dv;
  if (rr < 0) {
    --qq;
    rr += dv;
  } else if (rr >= dv) {
    ++qq;
    rr -= dv;
  }
  quo = qq;
  rem = rr;
}

struct CmFactor {
  int b, c, d, nct, ntask;
  float inv_nct, inv_d;
};

// The wavefront's tasks w, w + 8, ... taken TG at a time with at most SK beta steps each
// (nks <= SK); a group's operand loads are all issued before its products run.
template <int TG, int SK, typename TIn>
__device__ __forceinline__ void run_factor(const CmFactor& F, const TIn* V, const float* in, float* out, int LD) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
  const int b = F.b, c = F.c, d = F.d, bc = b * c;
  for (int t0 = w; t0 < F.ntask; t0 += TG * kCmWaves) {
    float av[TG][SK], bv[TG][SK];
    int obase[TG], gam[TG];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const int task = t0 + tg * kCmWaves;
      const bool tv = task < F.ntask;
      int ad, ct, al, de;
      divmod(task, F.nct, F.inv_nct, ad, ct);
      divmod(ad, d, F.inv_d, al, de);
      const int ga0 = 16 * ct;
      gam[tg] = tv ? ga0 + 4 * g : c;
      obase[tg] = li * LD + (al * c + ga0 + 4 * g) * d + de;
      const bool gv = tv && ga0 + li < c;
      const int voff = ad * bc + ga0 + li;
      const int xoff = li * LD + al * b * d + de;
#pragma unroll
      for (int sk = 0; sk < SK; ++sk) {
        const int be = 4 * sk + g;
        av[tg][sk] = 0.f;
        bv[tg][sk] = 0.f;
        if (tv && be < b) {
          bv[tg][sk] = in[xoff + be * d];
          if (gv) av[tg][sk] = load_in(V, voff + be * c);
        }
      }
    }
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      if (t0 + tg * kCmWaves < F.ntask) {
        f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sk = 0; sk < SK; ++sk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[tg][sk], bv[tg][sk], acc, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (gam[tg] + v < c) out[obase[tg] + v * d] = acc[v];
      }
    }
  }
}

// Factors with more than 8 beta steps: one task at a time, 8 steps per batch of loads.
template <typename TIn>
__device__ __forceinline__ void run_factor_long(const CmFactor& F, const TIn* V, const float* in, float* out, int LD) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, li = lane & 15;
  const int b = F.b, c = F.c, d = F.d, bc = b * c;
  const int nks = (b + 3) / 4;
  for (int task = w; task < F.ntask; task += kCmWaves) {
    int ad, ct, al, de;
    divmod(task, F.nct, F.inv_nct, ad, ct);
    divmod(ad, d, F.inv_d, al, de);
    const int ga0 = 16 * ct;
    const bool gv = ga0 + li < c;
    const int voff = ad * bc + ga0 + li;
    const int xoff = li * LD + al * b * d + de;
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nks; s0 += kCmKChunk) {
      float av[kCmKChunk], bv[kCmKChunk];
#pragma unroll
      for (int u = 0; u < kCmKChunk; ++u) {
        const int be = 4 * (s0 + u) + g;
        av[u] = 0.f;
        bv[u] = 0.f;
        if (be < b) {
          bv[u] = in[xoff + be * d];
          if (gv) av[u] = load_in(V, voff + be * c);
        }
      }
#pragma unroll
      for (int u = 0; u < kCmKChunk; ++u)
        if (s0 + u < nks) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], bv[u], acc, 0, 0, 0);
    }
    const int obase = li * LD + (al * c + ga0 + 4 * g) * d + de;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (ga0 + 4 * g + v < c) out[obase + v * d] = acc[v];
  }
}

template <typename TIn>
__global__ __launch_bounds__(kCmThreads) void ks_chain_mfma_kernel(ChainArgs A, int LD, int64_t ntiles) {
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int w0 = A.f[0].a * A.f[0].b * A.f[0].d;
  const int wl = A.wl;
  const int q0 = w0 / 4, ql = wl / 4;   // float4 per input and output row
  const TIn* x = static_cast<const TIn*>(A.x);
  float4 pre[kCmPre];
  // item e of a tile: row e % 16, float4 e / 16 (16 lanes cover one float4 column of the
  // tile: 64-byte runs per row in memory, LDS banks spread by the odd row pitch)
  auto fetch = [&](int64_t tile) {
#pragma unroll
    for (int u = 0; u < kCmPre; ++u) {
      const int e = tid + u * kCmThreads, r = e & (kCmRows - 1), c4 = e / kCmRows;
      const int64_t row = tile * kCmRows + r;
      pre[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c4 < q0 && row < A.N) pre[u] = load4_in(x + row * w0 + 4 * c4);
    }
  };
  auto stage = [&]() {   // registers into buffer 0
#pragma unroll
    for (int u = 0; u < kCmPre; ++u) {
      const int e = tid + u * kCmThreads, r = e & (kCmRows - 1), c4 = e / kCmRows;
      if (c4 < q0) {
        float* p = smem + r * LD + 4 * c4;
        p[0] = pre[u].x;
        p[1] = pre[u].y;
        p[2] = pre[u].z;
        p[3] = pre[u].w;
      }
    }
  };
  int64_t tile = blockIdx.x;
  fetch(tile);
  stage();
  for (; tile < ntiles; tile += gridDim.x) {
    if (tile + gridDim.x < ntiles) fetch(tile + gridDim.x);
    __syncthreads();
    int cur = 0;
    for (int fi = 0; fi < A.nf; ++fi) {
      CmFactor F;
      F.b = A.f[fi].b;
      F.c = A.f[fi].c;
      F.d = A.f[fi].d;
      F.nct = (F.c + 15) / 16;
      F.ntask = A.f[fi].a * F.d * F.nct;
      F.inv_nct = 1.f / (float)F.nct;
      F.inv_d = 1.f / (float)F.d;
      const TIn* V = static_cast<const TIn*>(A.f[fi].vals);
      const float* in = smem + cur * kCmRows * LD;
      float* out = smem + (cur ^ 1) * kCmRows * LD;
      const int nks = (F.b + 3) / 4;
      if (nks <= 2)
        run_factor<8, 2>(F, V, in, out, LD);
      else if (nks <= 4)
        run_factor<4, 4>(F, V, in, out, LD);
      else if (nks <= 8)
        run_factor<2, 8>(F, V, in, out, LD);
      else
        run_factor_long(F, V, in, out, LD);
      __syncthreads();
      cur ^= 1;
    }
    store_tile(A.y, smem + cur * kCmRows * LD, LD, tile, A.N, wl, ql);
    __syncthreads();   // buffer 0 is free again
    if (tile + gridDim.x < ntiles) stage();
  }
}

// Chains whose every factor fits a compile-time slot layout: factor f gives each wavefront
// at most TPW_f tasks of at most SK_f beta steps (b and c multiples of 4).  The factor values
// a wavefront needs never change from tile to tile, so they are loaded into registers once,
// with each slot's row and output offsets; a tile then costs only LDS reads, products and
// LDS writes.  Same tiles, buffers, task split and operand roles as ks_chain_mfma_kernel.
// Slot j of factor f for wavefront w: its values in registers (lane 16g + i: beta 4s + g,
// gamma tile + i) and a descriptor {row offset, output offset, gamma values left (c - first
// gamma of the tile; 0 for an unused slot), 0} in LDS,
// the same for every lane of the wavefront.
template <int TPW, int SK, typename TIn>
__device__ __forceinline__ void load_slots(const ChainFactor& f, int w, float* vr, int4* desc) {
  const int lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
  const int b = f.b, c = f.c, d = f.d, nct = (c + 15) / 16, ntask = f.a * d * nct;
  const TIn* V = static_cast<const TIn*>(f.vals);
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int task = w + kCmWaves * j;
    const bool valid = task < ntask;
    const int ad = task / nct, ct = task - ad * nct, al = ad / d, de = ad - al * d;
    const int ga0 = 16 * ct;
    if (lane == 0) desc[j] = valid ? make_int4(al * b * d + de, (al * c + ga0) * d + de, c - ga0, 0) : make_int4(0, 0, 0, 0);
#pragma unroll
    for (int sk = 0; sk < SK; ++sk) {
      const int be = 4 * sk + g;
      vr[j * SK + sk] = (valid && be < b && ga0 + li < c) ? load_in(V, ((int64_t)ad * b + be) * c + ga0 + li) : 0.f;
    }
  }
}

// Slots run in batches without branches, so that the compiler can overlap one
// slot's reads with another's products: an unused slot has zero values and writes into the
// wavefront's dummy area, and a beta step past b (nks < SK) multiplies zeros.
constexpr int kCmBatch = 16;   // row values (slots x beta steps) read per batch

template <int TPW, int SK>
__device__ __forceinline__ void run_slots(const float* vr, const int4* __restrict__ desc, int nks,
                                          int d, int LD, const float* __restrict__ in,
                                          float* __restrict__ out, float* __restrict__ dummy) {
  const int lane = threadIdx.x & 63, g = lane >> 4, li = lane & 15;
  const int d4 = 4 * d, lx = li * LD + g * d, lo = li * LD + 4 * g * d;
  constexpr int NB0 = kCmBatch / SK > 0 ? kCmBatch / SK : 1;   // about 16 row values in flight
  constexpr int NB = TPW < NB0 ? TPW : NB0;
  static_assert(TPW % NB == 0, "slots per wavefront in whole batches");
#pragma unroll
  for (int j0 = 0; j0 < TPW; j0 += NB) {
    float bv[NB][SK];
    float* op[NB];
    int st[NB];
#pragma unroll
    for (int jj = 0; jj < NB; ++jj) {
      const int j = j0 + jj;
      // The descriptor is the same for every lane.  With short beta loops it is moved to
      // scalar registers, so that the selects below stay selects: a select fed by a load
      // becomes a branch around the load, which splits the batch and makes each slot wait
      // for its own descriptor.  With 8 or more beta steps per slot (one or two slots per
      // batch) the extra scalar moves cost more than they save.
      const int4 dv = desc[j];
      int3 ds = make_int3(dv.x, dv.y, dv.z);
      if constexpr (SK < 8)
        ds = make_int3(__builtin_amdgcn_readfirstlane(dv.x), __builtin_amdgcn_readfirstlane(dv.y),
                       __builtin_amdgcn_readfirstlane(dv.z));
      const bool live = 4 * g < ds.z;
      op[jj] = live ? out + lo + ds.y : dummy + lane;
      st[jj] = live ? d : 64;
#pragma unroll
      for (int sk = 0; sk < SK; ++sk) {
        const float v = in[lx + ds.x + (sk < nks ? sk : 0) * d4];
        bv[jj][sk] = sk < nks ? v : 0.f;
      }
    }
#pragma unroll
    for (int jj = 0; jj < NB; ++jj) {
      const int j = j0 + jj;
      f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sk = 0; sk < SK; ++sk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[j * SK + sk], bv[jj][sk], acc, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) op[jj][v * st[jj]] = acc[v];
    }
  }
}

template <int T0, int S0, int T1, int S1, int T2, int S2>
struct SlotLayout {
  static constexpr int nf = T2 > 0 ? 3 : (T1 > 0 ? 2 : 1);
};

template <typename TIn, int T0, int S0, int T1, int S1, int T2, int S2>
__global__ __launch_bounds__(kCmThreads) void ks_chain_reg_kernel(ChainArgs A, int LD, int64_t ntiles) {
  extern __shared__ float smem[];
  constexpr int NF = SlotLayout<T0, S0, T1, S1, T2, S2>::nf;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w0 = A.f[0].a * A.f[0].b * A.f[0].d;
  const int wl = A.wl;
  const int q0 = w0 / 4, ql = wl / 4;
  const TIn* x = static_cast<const TIn*>(A.x);
  float v0[T0 * S0], v1[T1 * S1 + 1], v2[T2 * S2 + 1];
  // slot descriptors after the two row buffers: [factor][wavefront][slot]
  int4* const d0 = reinterpret_cast<int4*>(smem + 2 * kCmRows * LD) + w * T0;   // 2*16*LD floats: 16-byte multiple
  int4* const d1 = d0 + kCmWaves * T0 - w * T0 + w * T1;
  int4* const d2 = d1 + kCmWaves * T1 - w * T1 + w * T2;
  float* const dummy = reinterpret_cast<float*>(d2 + kCmWaves * T2 - w * T2) + w * 256;   // 4 x 64 per wavefront
  load_slots<T0, S0, TIn>(A.f[0], w, v0, d0);
  if constexpr (NF > 1) load_slots<T1, S1, TIn>(A.f[1], w, v1, d1);
  if constexpr (NF > 2) load_slots<T2, S2, TIn>(A.f[2], w, v2, d2);
  int nk[3], dd[3];
#pragma unroll
  for (int fi = 0; fi < 3; ++fi) {
    const int f = fi < NF ? fi : 0;
    nk[fi] = (A.f[f].b + 3) / 4;
    dd[fi] = A.f[f].d;
  }
  float4 pre[kCmPre];
  auto fetch = [&](int64_t tile) {
#pragma unroll
    for (int u = 0; u < kCmPre; ++u) {
      const int e = tid + u * kCmThreads, r = e & (kCmRows - 1), c4 = e / kCmRows;
      const int64_t row = tile * kCmRows + r;
      pre[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c4 < q0 && row < A.N) pre[u] = load4_in(x + row * w0 + 4 * c4);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < kCmPre; ++u) {
      const int e = tid + u * kCmThreads, r = e & (kCmRows - 1), c4 = e / kCmRows;
      if (c4 < q0) {
        float* p = smem + r * LD + 4 * c4;
        p[0] = pre[u].x;
        p[1] = pre[u].y;
        p[2] = pre[u].z;
        p[3] = pre[u].w;
      }
    }
  };
  float* const b0 = smem;
  float* const b1 = smem + kCmRows * LD;
  int64_t tile = blockIdx.x;
  fetch(tile);
  stage();
  // the factor values must be in registers before the loop: otherwise the loop head merges
  // the preheader's outstanding value loads with the tile's prefetch, and the first product
  // of every tile waits for that prefetch
#pragma unroll
  for (int i = 0; i < T0 * S0; ++i) asm volatile("" ::"v"(v0[i]));
  if constexpr (NF > 1) {
#pragma unroll
    for (int i = 0; i < T1 * S1; ++i) asm volatile("" ::"v"(v1[i]));
  }
  if constexpr (NF > 2) {
#pragma unroll
    for (int i = 0; i < T2 * S2; ++i) asm volatile("" ::"v"(v2[i]));
  }
  for (; tile < ntiles; tile += gridDim.x) {
    if (tile + gridDim.x < ntiles) fetch(tile + gridDim.x);
    __syncthreads();
    run_slots<T0, S0>(v0, d0, nk[0], dd[0], LD, b0, b1, dummy);
    __syncthreads();
    if constexpr (NF > 1) {
      run_slots<T1, S1>(v1, d1, nk[1], dd[1], LD, b1, b0, dummy);
      __syncthreads();
    }
    if constexpr (NF > 2) {
      run_slots<T2, S2>(v2, d2, nk[2], dd[2], LD, b0, b1, dummy);
      __syncthreads();
    }
    store_tile(A.y, (NF & 1) ? b1 : b0, LD, tile, A.N, wl, ql);
    __syncthreads();
    if (tile + gridDim.x < ntiles) stage();
  }
}

struct RegEntry {
  int nf, tpw[3], sk[3];
  const void* fn[2];   // fp32, bf16 inputs
};
#define KS_CHAIN_REG_ENTRY(T0, S0, T1, S1, T2, S2)                                                            \
  RegEntry {                                                                                                  \
    SlotLayout<T0, S0, T1, S1, T2, S2>::nf, {T0, T1, T2}, {S0, S1, S2}, {                                     \
      (const void*)ks_chain_reg_kernel<float, T0, S0, T1, S1, T2, S2>,                                        \
          (const void*)ks_chain_reg_kernel<uint16_t, T0, S0, T1, S1, T2, S2>                                  \
    }                                                                                                         \
  }
// (8x8)(x)(16x16)(x)(8x8)-like triples and Monarch-like pairs of 32x32 blocks at 1024 values per row
const RegEntry kRegTable[] = {KS_CHAIN_REG_ENTRY(16, 2, 8, 4, 16, 2), KS_CHAIN_REG_ENTRY(8, 8, 8, 8, 0, 0)};

const RegEntry* reg_find(const ChainArgs& A) {
  for (const RegEntry& E : kRegTable) {
    if (E.nf != A.nf) continue;
    bool ok = true;
    for (int f = 0; f < A.nf && ok; ++f) {
      const ChainFactor& F = A.f[f];
      const int ntask = F.a * F.d * ((F.c + 15) / 16);
      ok = F.b % 4 == 0 && F.c % 4 == 0 && (ntask + kCmWaves - 1) / kCmWaves <= E.tpw[f] && (F.b + 3) / 4 <= E.sk[f];
    }
    if (ok) return &E;
  }
  return nullptr;
}

}  // namespace

bool chain_mfma_ok(const ChainArgs& A) {
  const int w0 = A.f[0].a * A.f[0].b * A.f[0].d;
  const ChainFactor& fl = A.f[A.nf - 1];
  const int wl = fl.a * fl.c * fl.d;
  return A.maxw <= kCmMaxWidth && w0 % 4 == 0 && wl % 4 == 0;
}

int chain_rows_per_tile(int maxw) {
  int64_t T = (int64_t)(kChainLds / (2 * (size_t)maxw * sizeof(float)));
  if (T > kChainMaxRows) T = kChainMaxRows;
  return (int)T;
}

hipError_t launch_ks_chain(const ChainArgs& A, hipStream_t s) {
  if (A.N > 0 && chain_mfma_ok(A)) {
    static const bool attr = [] {
      const bool a1 = hipFuncSetAttribute((const void*)ks_chain_mfma_kernel<float>,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kChainLds) == hipSuccess;
      const bool a2 = hipFuncSetAttribute((const void*)ks_chain_mfma_kernel<uint16_t>,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kChainLds) == hipSuccess;
      return a1 && a2;
    }();
    (void)attr;
    const int LD = (A.maxw + 31) / 32 * 32 + 1;
    const int64_t ntiles = (A.N + kCmRows - 1) / kCmRows;
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    const unsigned grid = (unsigned)(ntiles < ncu ? ntiles : ncu);
    const size_t lds = 2 * (size_t)kCmRows * LD * sizeof(float);
    const RegEntry* E = reg_find(A);
    const size_t lds_reg = lds + (size_t)kCmWaves * ((E ? E->tpw[0] + E->tpw[1] + E->tpw[2] : 0) * 16 + 256 * 4);
    if (E && lds_reg <= kChainLds) {
      const void* fn = E->fn[A.dtype == KRON_F32 ? 0 : 1];
      static bool attr_set[sizeof(kRegTable) / sizeof(kRegTable[0])][2] = {};
      bool& done = attr_set[E - kRegTable][A.dtype == KRON_F32 ? 0 : 1];
      if (!done) done = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kChainLds) == hipSuccess;
      ChainArgs args = A;
      int ld = LD;
      int64_t nt = ntiles;
      void* kargs[] = {&args, &ld, &nt};
      return hipLaunchKernel(fn, dim3(grid), dim3(kCmThreads), kargs, lds_reg, s);
    }
    if (A.dtype == KRON_F32)
      hipLaunchKernelGGL(ks_chain_mfma_kernel<float>, dim3(grid), dim3(kCmThreads), lds, s, A, LD, ntiles);
    else
      hipLaunchKernelGGL(ks_chain_mfma_kernel<uint16_t>, dim3(grid), dim3(kCmThreads), lds, s, A, LD, ntiles);
    return hipGetLastError();
  }
  const int T = chain_rows_per_tile(A.maxw);
  if (T < 1) return hipErrorInvalidValue;
  const int64_t grid = (A.N + T - 1) / T;
  if (grid == 0) return hipSuccess;
  const size_t lds = 2 * (size_t)T * A.maxw * sizeof(float);
  static const bool attr = [] {
    const bool a1 = hipFuncSetAttribute((const void*)ks_chain_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                        (int)kChainLds) == hipSuccess;
    const bool a2 = hipFuncSetAttribute((const void*)ks_chain_kernel<uint16_t>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kChainLds) == hipSuccess;
    return a1 && a2;
  }();
  (void)attr;
  if (A.dtype == KRON_F32)
    hipLaunchKernelGGL(ks_chain_kernel<float>, dim3((unsigned)grid), dim3(kChainThreads), lds, s, A, T);
  else
    hipLaunchKernelGGL(ks_chain_kernel<uint16_t>, dim3((unsigned)grid), dim3(kChainThreads), lds, s, A, T);
  return hipGetLastError();
}

}  // namespace kron
