// Backward of the Kronecker-sparse matmul Y = X K, K with support I_a (x) 1_{b x c} (x) I_d
// ("Fast Inference with Kronecker-Sparse Matrices", abstract), by calculus from the forward:
//   dX = dY K^T.  K^T is again Kronecker-sparse, with the pattern (a, c, b, d) and the
//        values of each (alpha, delta) block transposed, so dX is the forward product on dY
//        with those values (transposed once per call into the workspace).
//   dvals[al][de][be][ga] = sum_n X[n, (al*b + be)*d + de] * dY[n, (al*c + ga)*d + de],
//        a reduction over the rows: each workgroup sums its chunk of rows for one
//        (alpha, delta) block (and one beta x gamma block of it) into a partial row, and the
//        fixed-order column reduction adds the partial rows (deterministic, no atomics).
#include "kron_internal.h"

namespace kron {
namespace {

constexpr int kDvThreads = 256;
constexpr int kDvOpt = 48;        // beta values per thread
constexpr int kDvMaxRows = 32;    // rows per LDS tile
constexpr size_t kDvLds = 160 * 1024;
constexpr int kDvTargetGroups = 256;

__device__ __forceinline__ float load_in(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_in(const uint16_t* p, int64_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}

template <typename T>
__global__ __launch_bounds__(256) void ks_vals_transpose_kernel(int64_t total, int b, int c, const T* __restrict__ v,
                                                                T* __restrict__ vt) {
  // vt[blk][ga][be] = v[blk][be][ga], blk = al*d + de
  const int64_t bc = (int64_t)b * c;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t blk = e / bc, r = e - blk * bc;
    const int64_t ga = r / b, be = r - ga * b;
    vt[e] = v[blk * bc + be * c + ga];
  }
}

// Work split of the dvals reduction.  Threads: CW gamma columns x G beta groups; thread
// (gi, gl) owns gamma g0 + gl and the betas b0 + gi + G*j, j < kDvOpt.
struct DvPlan {
  int CW, G, BH, ngb, nbb, T;
  int64_t Gr;   // row chunks = partial rows
};

DvPlan dv_plan(int64_t N, int a, int b, int c, int d) {
  DvPlan p{};
  p.CW = c < kDvThreads ? c : kDvThreads;
  p.G = kDvThreads / p.CW;
  p.BH = p.G * kDvOpt;
  p.ngb = (c + p.CW - 1) / p.CW;
  p.nbb = (b + p.BH - 1) / p.BH;
  const int64_t bhm = b < p.BH ? b : p.BH, gwm = p.CW;
  int64_t T = (int64_t)(kDvLds / ((bhm + gwm) * sizeof(float)));
  p.T = (int)(T > kDvMaxRows ? kDvMaxRows : (T < 1 ? 1 : T));
  const int64_t blocks = (int64_t)a * d * p.ngb * p.nbb;
  int64_t gr = (kDvTargetGroups + blocks - 1) / blocks;
  const int64_t tiles = (N + p.T - 1) / p.T;
  if (gr > tiles) gr = tiles;
  p.Gr = gr < 1 ? 1 : gr;
  return p;
}

template <typename TIn>
__global__ __launch_bounds__(kDvThreads) void ks_dv_kernel(int64_t N, int a, int b, int c, int d, DvPlan P,
                                                           const TIn* __restrict__ x, const TIn* __restrict__ dy,
                                                           float* __restrict__ part) {
  extern __shared__ float s[];
  const int n_oc = P.ngb * P.nbb;
  const int oc = blockIdx.x % n_oc;
  const int ad = (blockIdx.x / n_oc) % (a * d);
  const int64_t chunk = blockIdx.x / ((int64_t)n_oc * a * d);
  const int gb = oc % P.ngb, bb = oc / P.ngb;
  const int al = ad / d, de = ad % d;
  const int g0 = gb * P.CW, gw = c - g0 < P.CW ? c - g0 : P.CW;   // gamma block
  const int b0 = bb * P.BH, bh = b - b0 < P.BH ? b - b0 : P.BH;   // beta block
  float* Xs = s;                // T x bh
  float* Ys = s + P.T * bh;     // T x gw
  const int tid = threadIdx.x, gi = tid / P.CW, gl = tid % P.CW;
  const bool active = gi < P.G && gl < gw;
  float acc[kDvOpt];
#pragma unroll
  for (int j = 0; j < kDvOpt; ++j) acc[j] = 0.f;
  const int64_t in_w = (int64_t)a * b * d, out_w = (int64_t)a * c * d;
  const int64_t per = (N + P.Gr - 1) / P.Gr, r0 = chunk * per;
  const int64_t r1 = r0 + per < N ? r0 + per : N;
  for (int64_t t0 = r0; t0 < r1; t0 += P.T) {
    const int rows = (int)(r1 - t0 < P.T ? r1 - t0 : P.T);
    __syncthreads();
    for (int i = tid; i < rows * bh; i += kDvThreads) {
      const int t = i / bh, be = i - t * bh;
      Xs[i] = load_in(x, (t0 + t) * in_w + ((int64_t)al * b + b0 + be) * d + de);
    }
    for (int i = tid; i < rows * gw; i += kDvThreads) {
      const int t = i / gw, ga = i - t * gw;
      Ys[i] = load_in(dy, (t0 + t) * out_w + ((int64_t)al * c + g0 + ga) * d + de);
    }
    __syncthreads();
    if (active) {
      for (int t = 0; t < rows; ++t) {
        const float yv = Ys[t * gw + gl];
        const float* xr = Xs + t * bh + gi;
#pragma unroll
        for (int j = 0; j < kDvOpt; ++j)
          if (gi + P.G * j < bh) acc[j] = fmaf(xr[P.G * j], yv, acc[j]);
      }
    }
  }
  if (active) {
    const PartRow out{part, P.Gr, chunk, (int64_t)ad * b * c};
#pragma unroll
    for (int j = 0; j < kDvOpt; ++j) {
      const int be = gi + P.G * j;
      if (be < bh) out[(int64_t)(b0 + be) * c + g0 + gl] = acc[j];
    }
  }
}

// ---------------------------------------------------------------------------------
// dvals on the matrix cores, for d = 4 and b = 16*TB (TB <= 4), c = 16*NW (NW <= 16).
// A workgroup owns one alpha and a chunk of rows; wavefront w owns the gamma tile
// 16w .. 16w+15 and accumulates dvals[al][de][be][ga] for all TB beta tiles and all four
// delta in registers.  One v_mfma_f32_16x16x4_f32 step contracts four rows:
//   lane (g, c) supplies A[be = 16t + c][K = row g] = X[row g, (al*b + 16t + c)*4 + de]
//   and B[K = row g][ga = 16w + c] = dY[row g, (al*c + 16w + c)*4 + de],
// both read as one 16-byte load per lane covering the four delta.  Rows past the chunk
// read as zeros.  The next step's operands are loaded while the current step runs.
// ---------------------------------------------------------------------------------
typedef float f4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }
__device__ __forceinline__ f4 load4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ f4 load4(const uint16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return f4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
            __uint_as_float(v.y & 0xffff0000u)};
}
constexpr int kDvmChunks = 128;   // row chunks per alpha

template <int TB, typename TIn>
__global__ __launch_bounds__(1024) void ks_dv_mfma_kernel(int64_t N, int a, int c, int64_t Gr,
                                                          const TIn* __restrict__ x, const TIn* __restrict__ dy,
                                                          float* __restrict__ part) {
  constexpr int B = 16 * TB;
  const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15, w = threadIdx.x >> 6;
  const int al = blockIdx.x % a;
  const int64_t chunk = blockIdx.x / a;
  const int64_t in_w = (int64_t)a * B * 4, out_w = (int64_t)a * c * 4;
  const int64_t per = ((N + Gr - 1) / Gr + 3) / 4 * 4, r0 = chunk * per;
  const int64_t r1 = r0 + per < N ? r0 + per : N;
  const TIn* xb = x + ((int64_t)al * B + cl) * 4;
  const TIn* yb = dy + ((int64_t)al * c + 16 * w + cl) * 4;
  f4 acc[TB][4];
#pragma unroll
  for (int t = 0; t < TB; ++t)
#pragma unroll
    for (int de = 0; de < 4; ++de) acc[t][de] = f4{0.f, 0.f, 0.f, 0.f};
  f4 xn[TB], yn;
  auto load = [&](f4 (&xv)[TB], f4& yv, int64_t row) {
    const bool ok = row < r1;
    const int64_t rr = ok ? row : 0;
#pragma unroll
    for (int t = 0; t < TB; ++t) xv[t] = load4(xb + rr * in_w + 64 * t);
    yv = load4(yb + rr * out_w);
    if (!ok) {
#pragma unroll
      for (int t = 0; t < TB; ++t) xv[t] = f4{0.f, 0.f, 0.f, 0.f};
      yv = f4{0.f, 0.f, 0.f, 0.f};
    }
  };
  if (r0 < r1) load(xn, yn, r0 + g);
  for (int64_t row = r0; row < r1; row += 4) {
    f4 xv[TB], yv = yn;
#pragma unroll
    for (int t = 0; t < TB; ++t) xv[t] = xn[t];
    load(xn, yn, row + 4 + g);
#pragma unroll
    for (int de = 0; de < 4; ++de)
#pragma unroll
      for (int t = 0; t < TB; ++t) acc[t][de] = mfma4(xv[t][de], yv[de], acc[t][de]);
  }
  // acc[t][de] register v = dvals[al][de][be = 16t + 4g + v][ga = 16w + cl]
  const PartRow out{part, Gr, chunk, (int64_t)al * 4 * B * c};
#pragma unroll
  for (int de = 0; de < 4; ++de)
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) out[((int64_t)de * B + 16 * t + 4 * g + v) * c + 16 * w + cl] = acc[t][de][v];
}

// bf16 inputs on bf16 matrix instructions (v_mfma_f32_16x16x16_bf16): the contraction is
// over rows, 16 per instruction; lane group g takes rows 16s + 4g + u (u < 4).  A lane loads,
// for each of its four rows, the four delta values of its beta (and of its gamma) as one
// 8-byte piece, and regroups the 4 rows x 4 deltas into one operand per delta with byte
// permutes.  Same partial rows as the fp32 kernel.
typedef short s4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2v __attribute__((ext_vector_type(2)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

// 4 rows x 4 deltas (row-major pieces) -> op[de] = {rows 0..3 of delta de}
__device__ __forceinline__ void split_rows(const uint2 (&r)[4], s4 (&op)[4]) {
  const unsigned LO = 0x05040100u, HI = 0x07060302u;
  op[0] = __builtin_bit_cast(s4, (u2v{__builtin_amdgcn_perm(r[1].x, r[0].x, LO), __builtin_amdgcn_perm(r[3].x, r[2].x, LO)}));
  op[1] = __builtin_bit_cast(s4, (u2v{__builtin_amdgcn_perm(r[1].x, r[0].x, HI), __builtin_amdgcn_perm(r[3].x, r[2].x, HI)}));
  op[2] = __builtin_bit_cast(s4, (u2v{__builtin_amdgcn_perm(r[1].y, r[0].y, LO), __builtin_amdgcn_perm(r[3].y, r[2].y, LO)}));
  op[3] = __builtin_bit_cast(s4, (u2v{__builtin_amdgcn_perm(r[1].y, r[0].y, HI), __builtin_amdgcn_perm(r[3].y, r[2].y, HI)}));
}

constexpr int kDv16MaxWaves = 12;   // gamma tiles (c <= 192): 768 threads leave 168 VGPRs a lane

template <int TB>
__global__ __launch_bounds__(64 * kDv16MaxWaves) void ks_dv_mfma16_kernel(int64_t N, int a, int c, int64_t Gr,
                                                            const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ dy, float* __restrict__ part) {
  constexpr int B = 16 * TB;
  const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15, w = threadIdx.x >> 6;
  const int al = blockIdx.x % a;
  const int64_t chunk = blockIdx.x / a;
  const int64_t in_w = (int64_t)a * B * 4, out_w = (int64_t)a * c * 4;
  const int64_t per = ((N + Gr - 1) / Gr + 15) / 16 * 16, r0 = chunk * per;
  const int64_t r1 = r0 + per < N ? r0 + per : N;
  const uint16_t* xb = x + ((int64_t)al * B + cl) * 4;
  const uint16_t* yb = dy + ((int64_t)al * c + 16 * w + cl) * 4;
  f4 acc[TB][4];
#pragma unroll
  for (int t = 0; t < TB; ++t)
#pragma unroll
    for (int de = 0; de < 4; ++de) acc[t][de] = f4{0.f, 0.f, 0.f, 0.f};
  uint2 xn[TB][4], yn[4];
  auto load = [&](int64_t row0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t row = row0 + 4 * g + u;
      const bool ok = row < r1;
      const int64_t rr = ok ? row : 0;
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        const uint2 v = *reinterpret_cast<const uint2*>(xb + rr * in_w + 64 * t);
        xn[t][u] = ok ? v : uint2{0u, 0u};
      }
      const uint2 v = *reinterpret_cast<const uint2*>(yb + rr * out_w);
      yn[u] = ok ? v : uint2{0u, 0u};
    }
  };
  if (r0 < r1) load(r0);
  for (int64_t row = r0; row < r1; row += 16) {
    s4 yo[4], xo[TB][4];   // this step's operands, formed before the next step's loads reuse xn, yn
    split_rows(yn, yo);
#pragma unroll
    for (int t = 0; t < TB; ++t) split_rows(xn[t], xo[t]);
    load(row + 16);
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int de = 0; de < 4; ++de)
        acc[t][de] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xo[t][de], yo[de], acc[t][de], 0, 0, 0);
  }
  // acc[t][de] register v = dvals[al][de][be = 16t + 4g + v][ga = 16w + cl]
  const PartRow out{part, Gr, chunk, (int64_t)al * 4 * B * c};
#pragma unroll
  for (int de = 0; de < 4; ++de)
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) out[((int64_t)de * B + 16 * t + 4 * g + v) * c + 16 * w + cl] = acc[t][de][v];
}

bool dv_mfma_ok(int a, int b, int c, int d) {
  (void)a;
  return d == 4 && b % 16 == 0 && b / 16 >= 1 && b / 16 <= 4 && c % 16 == 0 && c / 16 >= 1 && c / 16 <= 16;
}
int64_t dv_mfma_chunks(int64_t N) {
  const int64_t steps = (N + 3) / 4;
  return steps < kDvmChunks ? (steps < 1 ? 1 : steps) : kDvmChunks;
}

template <int TB>
void launch_dv_mfma(const KSBwdArgs& k, int64_t Gr, dim3 grid, dim3 block, float* part, hipStream_t s) {
  if (k.dtype == KRON_F32)
    hipLaunchKernelGGL((ks_dv_mfma_kernel<TB, float>), grid, block, 0, s, k.N, k.a, k.c, Gr, (const float*)k.x,
                       (const float*)k.dy, part);
  else if (k.c / 16 <= kDv16MaxWaves)
    hipLaunchKernelGGL((ks_dv_mfma16_kernel<TB>), grid, block, 0, s, k.N, k.a, k.c, Gr, (const uint16_t*)k.x,
                       (const uint16_t*)k.dy, part);
  else
    hipLaunchKernelGGL((ks_dv_mfma_kernel<TB, uint16_t>), grid, block, 0, s, k.N, k.a, k.c, Gr,
                       (const uint16_t*)k.x, (const uint16_t*)k.dy, part);
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

bool ks_bwd_supported(int a, int b, int c, int d) { return ks_supported(a, c, b, d); }

size_t ks_bwd_workspace_bytes(int64_t N, int a, int b, int c, int d, int dtype) {
  const size_t es = dtype == KRON_F32 ? 4 : 2;
  const int64_t Gr = dv_mfma_ok(a, b, c, d) ? dv_mfma_chunks(N) : dv_plan(N, a, b, c, d).Gr;
  return align256((size_t)a * b * c * d * es) + align256((size_t)part_floats(Gr, (int64_t)a * b * c * d) * 4);
}

hipError_t launch_ks_bwd(const KSBwdArgs& k, void* ws, hipStream_t s) {
  const size_t es = k.dtype == KRON_F32 ? 4 : 2;
  const int64_t total = (int64_t)k.a * k.b * k.c * k.d;
  unsigned char* w = static_cast<unsigned char*>(ws);
  void* vt = w;
  float* part = reinterpret_cast<float*>(w + align256((size_t)total * es));
  if (k.dx && k.N > 0) {
    const int64_t blocks64 = (total + 255) / 256;
    const unsigned blocks = (unsigned)(blocks64 < 4096 ? blocks64 : 4096);
    if (k.dtype == KRON_F32)
      hipLaunchKernelGGL(ks_vals_transpose_kernel<float>, dim3(blocks), dim3(256), 0, s, total, k.b, k.c,
                         (const float*)k.vals, (float*)vt);
    else
      hipLaunchKernelGGL(ks_vals_transpose_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, total, k.b, k.c,
                         (const uint16_t*)k.vals, (uint16_t*)vt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const KSArgs f{k.N, k.a, k.c, k.b, k.d, k.dtype, KRON_F32, k.dy, vt, k.dx};
    if ((e = launch_ks(f, s)) != hipSuccess) return e;
  }
  if (k.dvals && dv_mfma_ok(k.a, k.b, k.c, k.d)) {
    const int64_t Gr = dv_mfma_chunks(k.N);
    const dim3 grid((unsigned)(Gr * k.a)), block((unsigned)(64 * (k.c / 16)));
    switch (k.b / 16) {
      case 1: launch_dv_mfma<1>(k, Gr, grid, block, part, s); break;
      case 2: launch_dv_mfma<2>(k, Gr, grid, block, part, s); break;
      case 3: launch_dv_mfma<3>(k, Gr, grid, block, part, s); break;
      default: launch_dv_mfma<4>(k, Gr, grid, block, part, s); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    RedPlan plan{};
    plan.seg[0] = RedSeg{k.dvals, (int32_t)total, 1.f, 0};
    plan.nseg = 1;
    if ((e = launch_column_reduce(part, (int32_t)Gr, (int32_t)total, plan, s)) != hipSuccess) return e;
  } else if (k.dvals) {
    const DvPlan P = dv_plan(k.N, k.a, k.b, k.c, k.d);
    const int bhm = k.b < P.BH ? k.b : P.BH;
    const size_t lds = (size_t)P.T * (bhm + P.CW) * sizeof(float);
    const int64_t grid = P.Gr * k.a * k.d * P.ngb * P.nbb;
    static const bool attr = [] {
      const bool a1 = hipFuncSetAttribute((const void*)ks_dv_kernel<float>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                          (int)kDvLds) == hipSuccess;
      const bool a2 = hipFuncSetAttribute((const void*)ks_dv_kernel<uint16_t>,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDvLds) == hipSuccess;
      return a1 && a2;
    }();
    (void)attr;
    if (k.dtype == KRON_F32)
      hipLaunchKernelGGL(ks_dv_kernel<float>, dim3((unsigned)grid), dim3(kDvThreads), lds, s, k.N, k.a, k.b, k.c,
                         k.d, P, (const float*)k.x, (const float*)k.dy, part);
    else
      hipLaunchKernelGGL(ks_dv_kernel<uint16_t>, dim3((unsigned)grid), dim3(kDvThreads), lds, s, k.N, k.a, k.b,
                         k.c, k.d, P, (const uint16_t*)k.x, (const uint16_t*)k.dy, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    RedPlan plan{};
    plan.seg[0] = RedSeg{k.dvals, (int32_t)total, 1.f, 0};
    plan.nseg = 1;
    if ((e = launch_column_reduce(part, (int32_t)P.Gr, (int32_t)total, plan, s)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kron
