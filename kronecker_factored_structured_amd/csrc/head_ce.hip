// Dense classification head with mean softmax cross-entropy, forward and backward
// (Kronecker layer tutorial, "Setup": the 10-class output layer stays dense; the step's
// loss is the cross-entropy).
//   z = h W + b;  loss = mean_n (logsumexp(z_n) - z_n[label_n])
//   dz = (softmax(z) - onehot) / N;  dh = dz W^T (o [h > 0]);  dW = h^T dz;  db = sum dz
// Pass 1: one wavefront per row computes z with a butterfly all-reduce across the
// 64 lanes, the softmax, dz, the row's loss and dh.  Pass 2: each thread owns one row
// k of dW (all C classes in registers) over a chunk of rows; the chunks' partial sums
// go through the shared fixed-order column reduction.
#include <type_traits>

#include "kron_internal.h"

namespace kron {
namespace {

constexpr int kThreads = 256;
constexpr int kWave = 64;
constexpr int kPass1Blocks = 512;

template <int CMAX>
__global__ __launch_bounds__(kThreads) void head_rows_kernel(
    int64_t N, int K, int C, uint32_t flags, const float* __restrict__ h, const float* __restrict__ W,
    const float* __restrict__ b, const int64_t* __restrict__ labels, float* __restrict__ dh,
    float* __restrict__ dz, float* __restrict__ lossrow) {
  extern __shared__ float Wt[];   // C x K (transposed head weight)
  for (int e = threadIdx.x; e < K * C; e += kThreads) {
    const int k = e / C, c = e - k * C;
    Wt[c * K + k] = W[e];
  }
  __syncthreads();
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / kWave);
  const float invN = 1.f / (float)N;
  for (int64_t row = (int64_t)blockIdx.x * (kThreads / kWave) + wave; row < N; row += nwaves) {
    const float* hr = h + row * K;
    float z[CMAX];
#pragma unroll
    for (int c = 0; c < CMAX; ++c) z[c] = 0.f;
    for (int k = lane; k < K; k += kWave) {
      const float hk = hr[k];
#pragma unroll
      for (int c = 0; c < CMAX; ++c)
        if (c < C) z[c] = fmaf(hk, Wt[c * K + k], z[c]);
    }
#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
      if (c < C) {
        float v = z[c];
#pragma unroll
        for (int off = kWave / 2; off >= 1; off /= 2) v += __shfl_xor(v, off, kWave);
        z[c] = v + b[c];
      }
    }
    float zmax = -INFINITY;
#pragma unroll
    for (int c = 0; c < CMAX; ++c)
      if (c < C) zmax = fmaxf(zmax, z[c]);
    const int64_t lab = labels[row];
    const bool ok = lab >= 0 && lab < C;
    float zlm = 0.f;   // z[label] - max
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CMAX; ++c)
      if (c < C) {
        const float d = z[c] - zmax;
        if (ok && c == lab) zlm = d;
        z[c] = expf(d);   // z now holds exp(z - max)
        s += z[c];
      }
    const float inv_s = 1.f / s;
    float mydz = 0.f;
#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
      if (c < C) {
        const float pc = z[c] * inv_s;
        const float d = (pc - ((ok && c == lab) ? 1.f : 0.f)) * invN;
        z[c] = d;                  // z now holds dz
        if (lane == c) mydz = d;
      }
    }
    if (lane < C) dz[row * C + lane] = mydz;
    if (lane == 0) lossrow[row] = ok ? (logf(s) - zlm) : __builtin_nanf("");
    float* dhr = dh ? dh + row * K : nullptr;
    if (dhr) {
      for (int k = lane; k < K; k += kWave) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CMAX; ++c)
          if (c < C) acc = fmaf(z[c], Wt[c * K + k], acc);
        if ((flags & KRON_DX_RELU_MASK) && !(hr[k] > 0.f)) acc = 0.f;
        dhr[k] = acc;
      }
    }
  }
}

// grid (ceil((K+1)/256), G): thread k < K owns dW[k][:] over rows [g*R, (g+1)*R);
// thread k == K owns db[:] and the loss sum of the same rows.
template <int CMAX>
__global__ __launch_bounds__(kThreads) void head_dw_kernel(int64_t N, int K, int C, int64_t R,
                                                           const float* __restrict__ h,
                                                           const float* __restrict__ dz,
                                                           const float* __restrict__ lossrow,
                                                           float* __restrict__ part) {
  const int k = blockIdx.x * kThreads + threadIdx.x;
  if (k > K) return;
  const int64_t r0 = (int64_t)blockIdx.y * R;
  const int64_t r1 = (r0 + R) < N ? (r0 + R) : N;
  const int64_t PW = (int64_t)K * C + C + 1;
  const PartRow out{part, (int64_t)gridDim.y, (int64_t)blockIdx.y, 0};
  (void)PW;
  float acc[CMAX];
#pragma unroll
  for (int c = 0; c < CMAX; ++c) acc[c] = 0.f;
  if (k < K) {
    for (int64_t n = r0; n < r1; ++n) {
      const float hv = h[n * K + k];
#pragma unroll
      for (int c = 0; c < CMAX; ++c)
        if (c < C) acc[c] = fmaf(hv, dz[n * C + c], acc[c]);
    }
#pragma unroll
    for (int c = 0; c < CMAX; ++c)
      if (c < C) out[(int64_t)k * C + c] = acc[c];
  } else {
    float ls = 0.f;
    for (int64_t n = r0; n < r1; ++n) {
#pragma unroll
      for (int c = 0; c < CMAX; ++c)
        if (c < C) acc[c] += dz[n * C + c];
      ls += lossrow[n];
    }
#pragma unroll
    for (int c = 0; c < CMAX; ++c)
      if (c < C) out[(int64_t)K * C + c] = acc[c];
    out[(int64_t)K * C + C] = ls;
  }
}

// ---------------------------------------------------------------------------------
// Matrix-core head for C <= 16 and K = KK (a multiple of 256): one pass over h.
// A workgroup (NWH wavefronts) takes 16-row tiles of h in turn and stages each in LDS
// (row stride KK + 4); wavefront w owns the columns [w*KQ, (w+1)*KQ) of h (the rows of
// W), KQ = KK / NWH.  Per tile:
//   z partial   = h[:, quarter] W[quarter, :]      64 products 16x16x4 per wavefront
//   z           = sum of the NWH partials (fixed order) + b; softmax, loss, dz per row
//                 (a row's 16 classes sit in 16 consecutive lanes)
//   dh[:, qtr]  = dz W[qtr, :]^T (o [h > 0])        16 output tiles x 4 products
//   dW[qtr, :] += h[:, qtr]^T dz                    16 accumulator tiles x 4 products
// W is held in registers in the two operand layouts.  dW, db and the loss sum stay in
// registers over the workgroup's tiles and are written once as its partial row.
// ---------------------------------------------------------------------------------
template <int KK, int NWH, bool DH>
__global__ __launch_bounds__(64 * NWH) void head_mfma_kernel(int64_t N, int C, uint32_t flags,
                                                        const float* __restrict__ h, const float* __restrict__ W,
                                                        const float* __restrict__ b,
                                                        const int64_t* __restrict__ labels,
                                                        float* __restrict__ dh, float* __restrict__ part) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int NT = 64 * NWH;
  constexpr int KQ = KK / NWH;      // columns of h per wavefront
  constexpr int SZ = KQ / 4;        // K steps of the z product per lane group: k = g*SZ + s
  constexpr int TQ = KQ / 16;       // 16-column tiles per wavefront
  constexpr int LH = KK + 4;        // LDS row stride of the h tile
  extern __shared__ float lds[];
  float* hs = lds;                  // 16 x LH
  float* zp = hs + 16 * LH;         // NWH x 16 x 16 z partials
  float* dzs = zp + NWH * 256;      // 16 x 16 dz
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15, w = tid >> 6;
  const int64_t ntile = (N + 15) / 16;
  const float invN = 1.f / (float)N;
  const bool mask = flags & KRON_DX_RELU_MASK;

  float wz[SZ];                     // W[k = w*KQ + g*SZ + s][class c]
  float wh[TQ][4];                  // W[k = w*KQ + 16t + c][class 4s + g]
#pragma unroll
  for (int s = 0; s < SZ; ++s) wz[s] = c < C ? W[(int64_t)(w * KQ + g * SZ + s) * C + c] : 0.f;
#pragma unroll
  for (int t = 0; t < TQ; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s) wh[t][s] = (4 * s + g) < C ? W[(int64_t)(w * KQ + 16 * t + c) * C + 4 * s + g] : 0.f;
  const int row_t = (tid >> 4) & 15, cls_t = tid & 15;   // the (row, class) of threads < 256 in the softmax
  const float bias_t = cls_t < C ? b[cls_t] : 0.f;

  f4 dwacc[TQ];                     // dW[k = w*KQ + 16t + 4g + v][class c]
#pragma unroll
  for (int t = 0; t < TQ; ++t) dwacc[t] = f4{0.f, 0.f, 0.f, 0.f};
  float dbacc = 0.f, lossacc = 0.f;

  // A tile's rows (and labels) are loaded during the previous tile and staged in LDS at
  // its start; full tiles run in the loop and the partial tile, if any, after it, so every
  // loop iteration issues the same stores and waiting for the prefetch never waits for them.
  constexpr int NPF = (16 * KK / 4 + NT - 1) / NT;
  f4 pf[NPF];
  int64_t lab_pf = 0;
  auto fetch = [&](int64_t tile) {
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int f = tid + i * NT;
      const int r = f / (KK / 4), o = 4 * (f % (KK / 4));
      f4 v = f4{0.f, 0.f, 0.f, 0.f};
      if ((16 * KK / 4) % NT == 0 || f < 16 * KK / 4)
        if (tile < ntile && tile * 16 + r < N) v = *reinterpret_cast<const f4*>(h + (tile * 16 + r) * KK + o);
      pf[i] = v;
    }
    lab_pf = (tid < 256 && tile < ntile && tile * 16 + row_t < N) ? labels[tile * 16 + row_t] : 0;
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int f = tid + i * NT;
      const int r = f / (KK / 4), o = 4 * (f % (KK / 4));
      if ((16 * KK / 4) % NT == 0 || f < 16 * KK / 4) *reinterpret_cast<f4*>(hs + r * LH + o) = pf[i];
    }
  };
  fetch(blockIdx.x);
  auto process = [&](int64_t tile, auto tail_c) {
    constexpr bool kTail = decltype(tail_c)::value;
    const int64_t r0 = tile * 16;
    __syncthreads();   // the previous tile's reads of hs and dzs are done
    stash();
    const int64_t lab = lab_pf;
    fetch(tile + gridDim.x);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // z partial over this wavefront's quarter (two accumulator chains)
    {
      f4 a0 = f4{0.f, 0.f, 0.f, 0.f}, a1 = a0;
      const float* hr = hs + c * LH + w * KQ + g * SZ;
#pragma unroll
      for (int s = 0; s < SZ; s += 8) {
        const f4 x0 = *reinterpret_cast<const f4*>(hr + s), x1 = *reinterpret_cast<const f4*>(hr + s + 4);
        a0 = __builtin_amdgcn_mfma_f32_16x16x4f32(x0[0], wz[s], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x4f32(x0[1], wz[s + 1], a1, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f32_16x16x4f32(x0[2], wz[s + 2], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x4f32(x0[3], wz[s + 3], a1, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f32_16x16x4f32(x1[0], wz[s + 4], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x4f32(x1[1], wz[s + 5], a1, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f32_16x16x4f32(x1[2], wz[s + 6], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x4f32(x1[3], wz[s + 7], a1, 0, 0, 0);
      }
      const f4 a = a0 + a1;   // z partial[row 4g+v][class c]
#pragma unroll
      for (int v = 0; v < 4; ++v) zp[w * 256 + (4 * g + v) * 16 + c] = a[v];
    }
    __syncthreads();
    // softmax, loss and dz of row row_t, class cls_t (16 consecutive lanes per row)
    if (tid < 256) {
      const int64_t row = r0 + row_t;
      const int e = row_t * 16 + cls_t;
      float z = zp[e];
#pragma unroll
      for (int q = 1; q < NWH; ++q) z += zp[q * 256 + e];
      z += bias_t;
      const bool valid = cls_t < C;
      float m = valid ? z : -INFINITY;
#pragma unroll
      for (int off = 8; off >= 1; off /= 2) m = fmaxf(m, __shfl_xor(m, off, 16));
      const float ex = valid ? expf(z - m) : 0.f;
      float ssum = ex;
#pragma unroll
      for (int off = 8; off >= 1; off /= 2) ssum += __shfl_xor(ssum, off, 16);
      float d = 0.f;
      if (!kTail || row < N) {
        const bool ok = lab >= 0 && lab < C;
        if (valid) d = (ex / ssum - ((ok && cls_t == lab) ? 1.f : 0.f)) * invN;
        // z[label] - max, from the label's lane
        const float zl = __shfl(z - m, (int)(ok ? lab : 0), 16);
        if (cls_t == 0) lossacc += ok ? (logf(ssum) - zl) : __builtin_nanf("");
      }
      dzs[e] = d;
      dbacc += d;
    }
    __syncthreads();
    // dh[:, quarter] = dz W[quarter, :]^T and dW[quarter, :] += h[:, quarter]^T dz.  dh is
    // formed transposed (dh^T[col][row] = sum_class W[col][class] dz[row][class]), so that a
    // lane holds four consecutive columns of one row and writes them as one 16-byte store.
    {
      float dzr[4];                                                         // dz[row c][class 4s+g]
#pragma unroll
      for (int s = 0; s < 4; ++s) dzr[s] = dzs[c * 16 + 4 * s + g];
      float dzb[4];                                                         // dz[row 4g+s][class c]
#pragma unroll
      for (int s = 0; s < 4; ++s) dzb[s] = dzs[(4 * g + s) * 16 + c];
      const bool live = !kTail || r0 + c < N;
#pragma unroll
      for (int t = 0; t < TQ; ++t) {
        const int col = w * KQ + 16 * t + c;
        if constexpr (DH) {
          f4 o = f4{0.f, 0.f, 0.f, 0.f};   // dh[row c][cols w*KQ + 16t + 4g .. +3]
#pragma unroll
          for (int s = 0; s < 4; ++s) o = __builtin_amdgcn_mfma_f32_16x16x4f32(wh[t][s], dzr[s], o, 0, 0, 0);
          const int c0 = w * KQ + 16 * t + 4 * g;
          if (mask) {
            const f4 hv = *reinterpret_cast<const f4*>(hs + c * LH + c0);
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v] = hv[v] > 0.f ? o[v] : 0.f;
          }
          if (live) __builtin_nontemporal_store(o, reinterpret_cast<f4*>(dh + (r0 + c) * KK + c0));
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
          dwacc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(hs[(4 * g + s) * LH + col], dzb[s], dwacc[t], 0, 0, 0);
      }
    }
  };
  const int64_t nfull = N / 16;
  int64_t tile = blockIdx.x;
  for (; tile < nfull; tile += gridDim.x) process(tile, std::false_type{});
  if (tile < ntile) process(tile, std::true_type{});

  // partial row: [dW (K*C) | db (C) | loss (1)]
  __syncthreads();
  const PartRow out{part, (int64_t)gridDim.x, (int64_t)blockIdx.x, 0};
#pragma unroll
  for (int t = 0; t < TQ; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (c < C) out[(int64_t)(w * KQ + 16 * t + 4 * g + v) * C + c] = dwacc[t][v];
  float* red = lds;   // 256 db values and 16 loss values, reduced in a fixed order
  if (tid < 256) red[tid] = dbacc;
  if (tid < 16) red[256 + tid] = 0.f;
  __syncthreads();
  if (tid < 256 && cls_t == 0) red[256 + row_t] = lossacc;
  __syncthreads();
  if (tid < 16) {
    float t0 = 0.f;
    for (int j = 0; j < 16; ++j) t0 += red[j * 16 + tid];
    if (tid < C) out[(int64_t)KK * C + tid] = t0;
  }
  if (tid == 0) {
    float l = 0.f;
    for (int j = 0; j < 16; ++j) l += red[256 + j];
    out[(int64_t)KK * C + C] = l;
  }
}

constexpr int kHeadMfmaK = 1024;
constexpr int kHeadMfmaWaves = 8;
constexpr size_t kHeadMfmaLds = (16 * (kHeadMfmaK + 4) + kHeadMfmaWaves * 256 + 256) * sizeof(float);

}  // namespace

bool head_mfma_ok(int K, int C) { return K == kHeadMfmaK && C <= 16; }

int head_groups(int64_t N) {
  const int64_t g = (N + 127) / 128;
  return (int)(g < 256 ? g : 256);
}

// Workgroups of the matrix-core head: two per compute unit, at most one per 16-row tile.
int head_mfma_groups(int64_t N) {
  const int64_t g = (N + 15) / 16;
  return (int)(g < 512 ? g : 512);
}

int64_t head_rows_per_group(int64_t N) {
  const int G = head_groups(N);
  return G == 0 ? 0 : (N + G - 1) / G;
}

hipError_t launch_head(const HeadArgs& a, int G, hipStream_t s) {
  if (head_mfma_ok(a.K, a.C)) {
    // as many workgroups as are resident at once (at most head_mfma_groups(N), which the
    // workspace is sized for)
    static const int per_cu = [] {
      (void)hipFuncSetAttribute((const void*)head_mfma_kernel<kHeadMfmaK, kHeadMfmaWaves, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kHeadMfmaLds);
      (void)hipFuncSetAttribute((const void*)head_mfma_kernel<kHeadMfmaK, kHeadMfmaWaves, false>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kHeadMfmaLds);
      int nb = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, head_mfma_kernel<kHeadMfmaK, kHeadMfmaWaves, true>,
                                                       64 * kHeadMfmaWaves, kHeadMfmaLds) != hipSuccess || nb < 1)
        nb = 1;
      return nb;
    }();
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    int Gm = head_mfma_groups(a.N);
    if (Gm > per_cu * cus) Gm = per_cu * cus;
    if (Gm > 0) {
      if (a.dh)
        hipLaunchKernelGGL((head_mfma_kernel<kHeadMfmaK, kHeadMfmaWaves, true>), dim3(Gm), dim3(64 * kHeadMfmaWaves),
                           kHeadMfmaLds, s, a.N, a.C, a.flags, a.h, a.W, a.b, a.labels, a.dh, a.part);
      else
        hipLaunchKernelGGL((head_mfma_kernel<kHeadMfmaK, kHeadMfmaWaves, false>), dim3(Gm), dim3(64 * kHeadMfmaWaves),
                           kHeadMfmaLds, s, a.N, a.C, a.flags, a.h, a.W, a.b, a.labels, a.dh, a.part);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    RedPlan plan{};
    plan.nseg = 3;
    plan.seg[0] = RedSeg{a.dW, a.K * a.C, 1.f, 0};
    plan.seg[1] = RedSeg{a.db, a.C, 1.f, 0};
    plan.seg[2] = RedSeg{a.loss, 1, a.N > 0 ? (float)(1.0 / (double)a.N) : 0.f, 0};
    return launch_column_reduce(a.part, Gm, a.K * a.C + a.C + 1, plan, s);
  }
  float* lossrow = a.dz + a.N * a.C;
  if (a.N > 0) {
    int64_t blocks = (a.N + 3) / 4;
    if (blocks > kPass1Blocks) blocks = kPass1Blocks;
    const size_t lds = (size_t)a.K * a.C * sizeof(float);
    if (a.C <= 16)
      hipLaunchKernelGGL(head_rows_kernel<16>, dim3((unsigned)blocks), dim3(kThreads), lds, s, a.N, a.K,
                         a.C, a.flags, a.h, a.W, a.b, a.labels, a.dh, a.dz, lossrow);
    else
      hipLaunchKernelGGL(head_rows_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), lds, s, a.N, a.K,
                         a.C, a.flags, a.h, a.W, a.b, a.labels, a.dh, a.dz, lossrow);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t R = head_rows_per_group(a.N);
    dim3 grid((unsigned)((a.K + 1 + kThreads - 1) / kThreads), (unsigned)G);
    if (a.C <= 16)
      hipLaunchKernelGGL(head_dw_kernel<16>, grid, dim3(kThreads), 0, s, a.N, a.K, a.C, R, a.h, a.dz,
                         lossrow, a.part);
    else
      hipLaunchKernelGGL(head_dw_kernel<64>, grid, dim3(kThreads), 0, s, a.N, a.K, a.C, R, a.h, a.dz,
                         lossrow, a.part);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  RedPlan plan{};
  plan.nseg = 3;
  plan.seg[0] = RedSeg{a.dW, a.K * a.C, 1.f, 0};
  plan.seg[1] = RedSeg{a.db, a.C, 1.f, 0};
  plan.seg[2] = RedSeg{a.loss, 1, a.N > 0 ? (float)(1.0 / (double)a.N) : 0.f, 0};
  return launch_column_reduce(a.part, G, a.K * a.C + a.C + 1, plan, s);
}

}  // namespace kron
