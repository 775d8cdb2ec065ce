// C ABI of libkron: argument validation (host only, before any HIP call), launch
// planning and dispatch to the kernels.  See include/kron.h for the contract.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "kron_internal.h"

namespace {

thread_local std::string g_last_error;

kron_status_t fail(kron_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kron_status_t ok() {
  g_last_error.clear();
  return KRON_OK;
}

kron_status_t hip_fail(hipError_t e, const char* where) {
  return fail(KRON_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
  const void* p;
  size_t bytes;
  const char* name;
};

bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes;
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
  return a0 < b1 && b0 < a1;
}

// Every output must be disjoint from every input and from every other output.
kron_status_t check_alias(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j]))
        return fail(KRON_E_ALIAS, "output %s overlaps input %s", outs[i].name, ins[j].name);
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j]))
        return fail(KRON_E_ALIAS, "output %s overlaps output %s", outs[i].name, outs[j].name);
  }
  return KRON_OK;
}

kron_status_t check_align(const Range* rs, int n) {
  for (int i = 0; i < n; ++i)
    if (rs[i].p && !aligned16(rs[i].p))
      return fail(KRON_E_ALIGN, "%s is not 16-byte aligned (%p)", rs[i].name, rs[i].p);
  return KRON_OK;
}

constexpr int32_t kMaxDim = 4096;
constexpr int32_t kMaxRank = 64;
constexpr int64_t kMaxFeatures = 65536;
constexpr int64_t kMaxParams = int64_t(1) << 24;
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;

kron_status_t check_shape(const kron_shape_t* s) {
  if (!s) return fail(KRON_E_NULL, "shape is NULL");
  if (s->N < 0 || s->N > kMaxRows) return fail(KRON_E_SHAPE, "N = %lld out of range", (long long)s->N);
  const int32_t d[5] = {s->p, s->q, s->m, s->n, s->r};
  const char* nm[5] = {"p", "q", "m", "n", "r"};
  for (int i = 0; i < 5; ++i)
    if (d[i] < 1) return fail(KRON_E_SHAPE, "%s = %d must be >= 1", nm[i], d[i]);
  for (int i = 0; i < 4; ++i)
    if (d[i] > kMaxDim) return fail(KRON_E_UNSUPPORTED, "%s = %d exceeds %d", nm[i], d[i], kMaxDim);
  if (s->r > kMaxRank) return fail(KRON_E_UNSUPPORTED, "r = %d exceeds %d", s->r, kMaxRank);
  const int64_t in = (int64_t)s->p * s->m, out = (int64_t)s->q * s->n;
  if (in > kMaxFeatures || out > kMaxFeatures)
    return fail(KRON_E_UNSUPPORTED, "in = %lld or out = %lld exceeds %lld", (long long)in, (long long)out,
                (long long)kMaxFeatures);
  if ((int64_t)s->r * s->p * s->q > kMaxParams || (int64_t)s->r * s->m * s->n > kMaxParams)
    return fail(KRON_E_UNSUPPORTED, "factor tensors exceed %lld elements", (long long)kMaxParams);
  if (s->flags & ~(KRON_RELU_OUT | KRON_DX_RELU_MASK | KRON_SPARSE_ROWS))
    return fail(KRON_E_ARG, "unknown flag bits 0x%x", s->flags);
  return KRON_OK;
}

// Which backward kernel runs for a shape, with how many workgroups (= partial rows).
// chunk > 0: the ranks run in passes of `chunk` ranks each (partial rows per pass).
struct BwdPlan {
  bool mfma;
  bool small;
  int chunk;
  int G;
  size_t ws_bytes;
  kron::SmallBwdPlan sp;
};

BwdPlan bwd_plan(const kron_shape_t* s, bool want_dx) {
  BwdPlan pl{false, false, 0, 0, 0, {}};
  if (kron::small_supported(s->p, s->q, s->m, s->n, s->r) &&
      !kron::mfma_bwd_supported(s->p, s->q, s->m, s->n, s->r)) {
    pl.small = true;
    pl.sp = kron::small_bwd_plan(s->N, s->p, s->q, s->m, s->n, s->r);
    pl.ws_bytes = (size_t)pl.sp.ws_floats * sizeof(float);
    return pl;
  }
  if (kron::mfma_bwd_supported(s->p, s->q, s->m, s->n, s->r)) {
    pl.mfma = true;
    pl.G = kron::mfma_bwd_groups(s->N, s->p, s->q, s->m, s->n, s->r);
  } else if ((pl.chunk = kron::mfma_bwd_chunk(s->p, s->q, s->m, s->n, s->r)) > 0) {
    pl.mfma = true;
    pl.G = kron::mfma_bwd_groups(s->N, s->p, s->q, s->m, s->n, pl.chunk);
    const int64_t PWc = kron::partial_width(s->p, s->q, s->m, s->n, pl.chunk);
    pl.ws_bytes = (size_t)kron::part_floats(pl.G, PWc) * sizeof(float);
    return pl;
  } else {
    const int T = kron::generic_bwd_rows_per_tile(s->p, s->q, s->m, s->n, want_dx);
    if (T == 0) return pl;
    pl.G = kron::generic_bwd_groups(s->N, T);
  }
  const int64_t PW = kron::partial_width(s->p, s->q, s->m, s->n, s->r);
  pl.ws_bytes = (size_t)kron::part_floats(pl.G, PW) * sizeof(float);
  return pl;
}

// Workspace bytes for a shape: the larger of the plans with and without dx, so the
// caller need not know which one a call will take.
size_t bwd_workspace(const kron_shape_t* s) {
  const BwdPlan a = bwd_plan(s, true), b = bwd_plan(s, false);
  size_t w = a.ws_bytes > b.ws_bytes ? a.ws_bytes : b.ws_bytes;
  return w == 0 ? 256 : (w + 255) & ~size_t(255);
}

}  // namespace

// Bytes of the Z cache for N rows (the saved ranks' Z_i = X B_i, p x n each, per row).
size_t zcache_need(const kron_shape_t* s) {
  return (size_t)s->N * kron::mfma_zcache_row_floats(s->p, s->q, s->m, s->n, s->r) * sizeof(float);
}

// The cache's own checks (the shape itself is checked by the caller first).
kron_status_t zcache_checks(const kron_shape_t* s, const void* zc, size_t zc_bytes) {
  if (kron::mfma_zcache_row_floats(s->p, s->q, s->m, s->n, s->r) == 0)
    return fail(KRON_E_UNSUPPORTED, "no saved-intermediate path for p=%d q=%d m=%d n=%d r=%d", s->p, s->q, s->m,
                s->n, s->r);
  if (s->flags & KRON_SPARSE_ROWS) return fail(KRON_E_ARG, "the sparse-row hint has no saved-intermediate path");
  if (zc_bytes < zcache_need(s))
    return fail(KRON_E_WORKSPACE, "zcache of %zu bytes given, %zu needed", zc_bytes, zcache_need(s));
  if (!aligned16(zc)) return fail(KRON_E_ALIGN, "zcache is not 16-byte aligned (%p)", zc);
  return KRON_OK;
}

extern "C" {

int32_t kron_abi_version(void) { return KRON_ABI_VERSION; }

const char* kron_status_str(kron_status_t st) {
  switch (st) {
    case KRON_OK: return "ok";
    case KRON_E_NULL: return "null pointer";
    case KRON_E_SHAPE: return "invalid shape";
    case KRON_E_ALIGN: return "misaligned pointer";
    case KRON_E_ALIAS: return "overlapping buffers";
    case KRON_E_DTYPE: return "unknown dtype";
    case KRON_E_WORKSPACE: return "workspace missing or too small";
    case KRON_E_UNSUPPORTED: return "unsupported by this build";
    case KRON_E_HIP: return "HIP error";
    case KRON_E_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

const char* kron_last_error(void) { return g_last_error.c_str(); }

kron_status_t kron_linear_check(const kron_shape_t* s) {
  const kron_status_t st = check_shape(s);
  if (st != KRON_OK) return st;
  if (!kron::small_supported(s->p, s->q, s->m, s->n, s->r) &&
      (kron::generic_fwd_rows_per_tile(s->p, s->q, s->m, s->n) == 0 ||
       kron::generic_bwd_rows_per_tile(s->p, s->q, s->m, s->n, true) == 0))
    return fail(KRON_E_UNSUPPORTED, "per-row working set of p=%d q=%d m=%d n=%d exceeds LDS", s->p, s->q,
                s->m, s->n);
  return ok();
}

size_t kron_linear_bwd_workspace_bytes(const kron_shape_t* s) {
  if (kron_linear_check(s) != KRON_OK) return 0;
  return bwd_workspace(s);
}

size_t kron_linear_zcache_bytes(const kron_shape_t* s) {
  if (kron_linear_check(s) != KRON_OK || kron::mfma_zcache_row_floats(s->p, s->q, s->m, s->n, s->r) == 0) return 0;
  return zcache_need(s);
}

}  // extern "C"

namespace {

// The forward, writing the Z cache as well when zc is given (zc_bytes checked here).
kron_status_t fwd_run(const kron_shape_t* s, const float* x, const float* S, const float* A, const float* B,
                      const float* bias, float* y, float* zc, size_t zc_bytes, hipStream_t stream) {
  kron_status_t st = kron_linear_check(s);
  if (st != KRON_OK) return st;
  if (s->flags & KRON_DX_RELU_MASK) return fail(KRON_E_ARG, "KRON_DX_RELU_MASK is a backward flag");
  if (!A || !B) return fail(KRON_E_NULL, "A and B are required");
  if (s->N > 0 && (!x || !y)) return fail(KRON_E_NULL, "x and y are required when N > 0");
  if (zc && (st = zcache_checks(s, zc, zc_bytes)) != KRON_OK) return st;
  const size_t in = (size_t)s->p * s->m, out = (size_t)s->q * s->n;
  const Range ins[5] = {{x, (size_t)s->N * in * 4, "x"},
                        {S, (size_t)s->p * s->q * 4, "S"},
                        {A, (size_t)s->r * s->p * s->q * 4, "A"},
                        {B, (size_t)s->r * s->m * s->n * 4, "B"},
                        {bias, out * 4, "bias"}};
  const Range outs[2] = {{y, (size_t)s->N * out * 4, "y"}, {zc, zc ? zcache_need(s) : 0, "zcache"}};
  if ((st = check_align(ins, 5)) != KRON_OK || (st = check_align(outs, 2)) != KRON_OK) return st;
  if ((st = check_alias(outs, 2, ins, 5)) != KRON_OK) return st;
  if (s->N == 0) return ok();
  kron::LayerArgs a{};
  a.N = s->N; a.p = s->p; a.q = s->q; a.m = s->m; a.n = s->n; a.r = s->r; a.flags = s->flags;
  a.x = x; a.S = S; a.A = A; a.B = B; a.bias = bias; a.y = y; a.zc = zc;
  hipError_t e = kron::mfma_fwd_supported(a.p, a.q, a.m, a.n, a.r)    ? kron::launch_fwd_mfma(a, stream)
                 : kron::small_supported(a.p, a.q, a.m, a.n, a.r) ? kron::launch_fwd_small(a, stream)
                                                                  : kron::launch_fwd_generic(a, stream);
  if (e != hipSuccess) return hip_fail(e, "kron_linear_fwd launch");
  return ok();
}

}  // namespace

extern "C" {

kron_status_t kron_linear_fwd(const kron_shape_t* s, const float* x, const float* S, const float* A,
                              const float* B, const float* bias, float* y, hipStream_t stream) {
  return fwd_run(s, x, S, A, B, bias, y, nullptr, 0, stream);
}

kron_status_t kron_linear_fwd_save(const kron_shape_t* s, const float* x, const float* S, const float* A,
                                   const float* B, const float* bias, float* y, float* zcache, size_t zcache_bytes,
                                   hipStream_t stream) {
  if (!zcache && s && s->N > 0) return fail(KRON_E_NULL, "zcache is required when N > 0");
  return fwd_run(s, x, S, A, B, bias, y, zcache, zcache_bytes, stream);
}

}  // extern "C"

namespace {

// kron_linear_bwd's argument checks (host only), with the workspace size taken as given.
kron_status_t bwd_checks(const kron_shape_t* s, const float* x, const float* S, const float* A, const float* B,
                         const float* dy, float* dx, float* dS, float* dA, float* dB, float* dbias) {
  kron_status_t st = kron_linear_check(s);
  if (st != KRON_OK) return st;
  if (s->flags & KRON_RELU_OUT) return fail(KRON_E_ARG, "KRON_RELU_OUT is a forward flag");
  if (!A || !B || !dA || !dB) return fail(KRON_E_NULL, "A, B, dA and dB are required");
  if ((S == nullptr) != (dS == nullptr)) return fail(KRON_E_NULL, "dS must be given exactly when S is");
  if (s->N > 0 && (!x || !dy)) return fail(KRON_E_NULL, "x and dy are required when N > 0");
  if ((s->flags & KRON_DX_RELU_MASK) && !dx) return fail(KRON_E_ARG, "KRON_DX_RELU_MASK needs dx");
  return KRON_OK;
}

kron_status_t bwd_run(const kron_shape_t* s, const float* x, const float* S, const float* A, const float* B,
                      const float* dy, float* dx, float* dS, float* dA, float* dB, float* dbias, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, const float* zc = nullptr, size_t zc_bytes = 0) {
  kron_status_t st = bwd_checks(s, x, S, A, B, dy, dx, dS, dA, dB, dbias);
  if (st != KRON_OK) return st;
  if (zc && (st = zcache_checks(s, zc, zc_bytes)) != KRON_OK) return st;
  const size_t need = bwd_workspace(s);
  if (!workspace || workspace_bytes < need)
    return fail(KRON_E_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0) return fail(KRON_E_ALIGN, "workspace is not 256-byte aligned");
  const size_t in = (size_t)s->p * s->m, out = (size_t)s->q * s->n;
  const size_t pq = (size_t)s->p * s->q, mn = (size_t)s->m * s->n;
  const Range ins[7] = {{x, (size_t)s->N * in * 4, "x"},     {S, pq * 4, "S"},
                        {A, s->r * pq * 4, "A"},             {B, s->r * mn * 4, "B"},
                        {dy, (size_t)s->N * out * 4, "dy"},  {workspace, need, "workspace"},
                        {zc, zc ? zcache_need(s) : 0, "zcache"}};
  const Range outs[5] = {{dx, (size_t)s->N * in * 4, "dx"}, {dS, pq * 4, "dS"}, {dA, s->r * pq * 4, "dA"},
                         {dB, s->r * mn * 4, "dB"},         {dbias, out * 4, "dbias"}};
  if ((st = check_align(ins, 7)) != KRON_OK || (st = check_align(outs, 5)) != KRON_OK) return st;
  if ((st = check_alias(outs, 5, ins, 7)) != KRON_OK) return st;

  kron::LayerArgs a{};
  a.N = s->N; a.p = s->p; a.q = s->q; a.m = s->m; a.n = s->n; a.r = s->r; a.flags = s->flags;
  a.x = x; a.S = S; a.A = A; a.B = B; a.dy = dy;
  a.dx = s->N > 0 ? dx : nullptr;
  a.dS = dS; a.dA = dA; a.dB = dB; a.dbias = dbias;
  a.part = (float*)workspace;
  a.zc = const_cast<float*>(zc);   // (read only by the backward)
  const BwdPlan pl = bwd_plan(s, a.dx != nullptr);
  if (zc && (!pl.mfma || pl.small || pl.chunk > 0))   // (a supported shape always takes the whole-row kernel)
    return fail(KRON_E_UNSUPPORTED, "the saved-intermediate backward needs the whole-row kernel");
  const int32_t pq32 = s->p * s->q, mn32 = s->m * s->n;
  if (pl.small) {
    hipError_t e = kron::launch_bwd_small(a, pl.sp, stream);
    if (e != hipSuccess) return hip_fail(e, "kron_linear_bwd launch");
    return ok();
  }
  if (pl.chunk > 0) {
    // ranks in passes of pl.chunk: pass c handles ranks [c*chunk, (c+1)*chunk); dX is
    // written by the first pass and added to by the others (the ReLU mask, if any, is
    // applied by the last pass), dS sums over the passes and dbias comes from the first
    const int passes = s->r / pl.chunk;
    const int32_t PWc = (int32_t)kron::partial_width(s->p, s->q, s->m, s->n, pl.chunk);
    for (int c = 0; c < passes; ++c) {
      kron::LayerArgs ac = a;
      ac.r = pl.chunk;
      ac.A = A + (size_t)c * pl.chunk * pq32;
      ac.B = B + (size_t)c * pl.chunk * mn32;
      ac.flags = (c == passes - 1) ? s->flags : (s->flags & ~KRON_DX_RELU_MASK);
      ac.dx_accumulate = c > 0;
      hipError_t e = kron::launch_bwd_mfma(ac, pl.G, stream);
      if (e != hipSuccess) return hip_fail(e, "kron_linear_bwd launch");
      kron::RedPlan rp{};
      rp.nseg = 4;
      rp.seg[0] = kron::RedSeg{dB + (size_t)c * pl.chunk * mn32, pl.chunk * mn32, 1.f, 0};
      rp.seg[1] = kron::RedSeg{dA + (size_t)c * pl.chunk * pq32, pl.chunk * pq32, 1.f, 0};
      rp.seg[2] = kron::RedSeg{dS, pq32, 1.f, c > 0};
      rp.seg[3] = kron::RedSeg{c == 0 ? dbias : nullptr, s->q * s->n, 1.f, 0};
      e = kron::launch_column_reduce(a.part, pl.G, PWc, rp, stream);
      if (e != hipSuccess) return hip_fail(e, "kron_linear_bwd reduce launch");
    }
    return ok();
  }
  hipError_t e = pl.mfma ? kron::launch_bwd_mfma(a, pl.G, stream) : kron::launch_bwd_generic(a, pl.G, stream);
  if (e != hipSuccess) return hip_fail(e, "kron_linear_bwd launch");
  kron::RedPlan rp{};
  rp.nseg = 4;
  rp.seg[0] = kron::RedSeg{dB, s->r * mn32, 1.f, 0};
  rp.seg[1] = kron::RedSeg{dA, s->r * pq32, 1.f, 0};
  rp.seg[2] = kron::RedSeg{dS, pq32, 1.f, 0};
  rp.seg[3] = kron::RedSeg{dbias, s->q * s->n, 1.f, 0};
  const int32_t PW = (int32_t)kron::partial_width(s->p, s->q, s->m, s->n, s->r);
  e = kron::launch_column_reduce(a.part, pl.G, PW, rp, stream);
  if (e != hipSuccess) return hip_fail(e, "kron_linear_bwd reduce launch");
  return ok();
}

}  // namespace

extern "C" {

kron_status_t kron_linear_bwd(const kron_shape_t* s, const float* x, const float* S, const float* A,
                              const float* B, const float* dy, float* dx, float* dS, float* dA, float* dB,
                              float* dbias, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_run(s, x, S, A, B, dy, dx, dS, dA, dB, dbias, workspace, workspace_bytes, stream);
}

kron_status_t kron_linear_bwd_saved(const kron_shape_t* s, const float* x, const float* S, const float* A,
                                    const float* B, const float* dy, const float* zcache, size_t zcache_bytes,
                                    float* dx, float* dS, float* dA, float* dB, float* dbias, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  if (!zcache && s && s->N > 0) return fail(KRON_E_NULL, "zcache is required when N > 0");
  return bwd_run(s, x, S, A, B, dy, dx, dS, dA, dB, dbias, workspace, workspace_bytes, stream, zcache,
                 zcache_bytes);
}

}  // extern "C"

// The fixed scratch of kron_linear_bwd_noalloc: the backward's partial-row workspace for
// callers that cannot allocate.  Each GPU the library runs on holds its own copy for the
// life of the process.  In host code `scratch` only names the symbol; its device address
// on the current GPU comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[KRON_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// The device address of `scratch` on the current device (looked up on the first call
// made with that device current).
kron_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(KRON_E_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || ((uintptr_t)p & 255u) != 0) return fail(KRON_E_HIP, "scratch has no 256-byte aligned address");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return KRON_OK;
}

}  // namespace

extern "C" {

kron_status_t kron_linear_bwd_noalloc(const kron_shape_t* s, const float* x, const float* S, const float* A,
                                      const float* B, const float* dy, float* dx, float* dS, float* dA,
                                      float* dB, float* dbias, hipStream_t stream) {
  kron_status_t st = bwd_checks(s, x, S, A, B, dy, dx, dS, dA, dB, dbias);
  if (st != KRON_OK) return st;
  const size_t need = bwd_workspace(s);
  if (need > KRON_NOALLOC_SCRATCH_BYTES)
    return fail(KRON_E_UNSUPPORTED, "this shape needs %zu bytes of scratch; the fixed scratch holds %zu", need,
                (size_t)KRON_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != KRON_OK) return st;
  return bwd_run(s, x, S, A, B, dy, dx, dS, dA, dB, dbias, ws, KRON_NOALLOC_SCRATCH_BYTES, stream);
}

size_t kron_linear_bwd_bf16_workspace_bytes(const kron_shape_t* s) {
  if (kron_linear_check(s) != KRON_OK || !kron::bf16_supported(s->p, s->q, s->m, s->n, s->r)) return 0;
  const int G = kron::bf16_bwd_groups(s->N, s->p, s->q, s->m, s->n, s->r);
  const int64_t PW = kron::partial_width(s->p, s->q, s->m, s->n, s->r);
  const size_t w = (size_t)kron::part_floats(G, PW) * sizeof(float);
  return w == 0 ? 256 : (w + 255) & ~size_t(255);
}

kron_status_t kron_linear_fwd_bf16(const kron_shape_t* s, const void* x, const void* S, const void* A, const void* B,
                             const void* bias, void* y, hipStream_t stream) {
  kron_status_t st = kron_linear_check(s);
  if (st != KRON_OK) return st;
  if (s->flags & KRON_DX_RELU_MASK) return fail(KRON_E_ARG, "KRON_DX_RELU_MASK is a backward flag");
  if (!kron::bf16_supported(s->p, s->q, s->m, s->n, s->r))
    return fail(KRON_E_UNSUPPORTED, "no bf16 kernel for (p, q, m, n, r) = (%d, %d, %d, %d, %d)", s->p, s->q, s->m,
                s->n, s->r);
  if (!A || !B) return fail(KRON_E_NULL, "A and B are required");
  if (s->N > 0 && (!x || !y)) return fail(KRON_E_NULL, "x and y are required when N > 0");
  const size_t in = (size_t)s->p * s->m, out = (size_t)s->q * s->n;
  const Range ins[5] = {{x, (size_t)s->N * in * 2, "x"},
                        {S, (size_t)s->p * s->q * 2, "S"},
                        {A, (size_t)s->r * s->p * s->q * 2, "A"},
                        {B, (size_t)s->r * s->m * s->n * 2, "B"},
                        {bias, out * 2, "bias"}};
  const Range outs[1] = {{y, (size_t)s->N * out * 2, "y"}};
  if ((st = check_align(ins, 5)) != KRON_OK || (st = check_align(outs, 1)) != KRON_OK) return st;
  if ((st = check_alias(outs, 1, ins, 5)) != KRON_OK) return st;
  if (s->N == 0) return ok();
  kron::LayerArgsBf16 a{};
  a.N = s->N; a.p = s->p; a.q = s->q; a.m = s->m; a.n = s->n; a.r = s->r; a.flags = s->flags;
  a.x = (const uint16_t*)x; a.S = (const uint16_t*)S; a.A = (const uint16_t*)A; a.B = (const uint16_t*)B;
  a.bias = (const uint16_t*)bias; a.y = (uint16_t*)y;
  hipError_t e = kron::launch_fwd_bf16(a, stream);
  if (e != hipSuccess) return hip_fail(e, "kron_linear_fwd_bf16 launch");
  return ok();
}

kron_status_t kron_linear_bwd_bf16(const kron_shape_t* s, const void* x, const void* S, const void* A, const void* B,
                             const void* dy, void* dx, float* dS, float* dA, float* dB, float* dbias, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  kron_status_t st = kron_linear_check(s);
  if (st != KRON_OK) return st;
  if (s->flags & KRON_RELU_OUT) return fail(KRON_E_ARG, "KRON_RELU_OUT is a forward flag");
  if (!kron::bf16_supported(s->p, s->q, s->m, s->n, s->r))
    return fail(KRON_E_UNSUPPORTED, "no bf16 kernel for (p, q, m, n, r) = (%d, %d, %d, %d, %d)", s->p, s->q, s->m,
                s->n, s->r);
  if (!A || !B || !dA || !dB) return fail(KRON_E_NULL, "A, B, dA and dB are required");
  if ((S == nullptr) != (dS == nullptr)) return fail(KRON_E_NULL, "dS must be given exactly when S is");
  if (s->N > 0 && (!x || !dy)) return fail(KRON_E_NULL, "x and dy are required when N > 0");
  if ((s->flags & KRON_DX_RELU_MASK) && !dx) return fail(KRON_E_ARG, "KRON_DX_RELU_MASK needs dx");
  const size_t need = kron_linear_bwd_bf16_workspace_bytes(s);
  if (!workspace || workspace_bytes < need)
    return fail(KRON_E_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0) return fail(KRON_E_ALIGN, "workspace is not 256-byte aligned");
  const size_t in = (size_t)s->p * s->m, out = (size_t)s->q * s->n;
  const size_t pq = (size_t)s->p * s->q, mn = (size_t)s->m * s->n;
  const Range ins[6] = {{x, (size_t)s->N * in * 2, "x"},     {S, pq * 2, "S"},
                        {A, s->r * pq * 2, "A"},             {B, s->r * mn * 2, "B"},
                        {dy, (size_t)s->N * out * 2, "dy"},  {workspace, need, "workspace"}};
  const Range outs[5] = {{dx, (size_t)s->N * in * 2, "dx"}, {dS, pq * 4, "dS"}, {dA, s->r * pq * 4, "dA"},
                         {dB, s->r * mn * 4, "dB"},         {dbias, out * 4, "dbias"}};
  if ((st = check_align(ins, 6)) != KRON_OK || (st = check_align(outs, 5)) != KRON_OK) return st;
  if ((st = check_alias(outs, 5, ins, 6)) != KRON_OK) return st;
  kron::LayerArgsBf16 a{};
  a.N = s->N; a.p = s->p; a.q = s->q; a.m = s->m; a.n = s->n; a.r = s->r; a.flags = s->flags;
  a.x = (const uint16_t*)x; a.S = (const uint16_t*)S; a.A = (const uint16_t*)A; a.B = (const uint16_t*)B;
  a.dy = (const uint16_t*)dy; a.dx = s->N > 0 ? (uint16_t*)dx : nullptr;
  a.part = (float*)workspace;
  const int G = kron::bf16_bwd_groups(s->N, s->p, s->q, s->m, s->n, s->r);
  hipError_t e = kron::launch_bwd_bf16(a, G, stream);
  if (e != hipSuccess) return hip_fail(e, "kron_linear_bwd_bf16 launch");
  kron::RedPlan rp{};
  rp.nseg = 4;
  rp.seg[0] = kron::RedSeg{dB, (int32_t)(s->r * mn), 1.f, 0};
  rp.seg[1] = kron::RedSeg{dA, (int32_t)(s->r * pq), 1.f, 0};
  rp.seg[2] = kron::RedSeg{dS, (int32_t)pq, 1.f, 0};
  rp.seg[3] = kron::RedSeg{dbias, s->q * s->n, 1.f, 0};
  const int32_t PW = (int32_t)kron::partial_width(s->p, s->q, s->m, s->n, s->r);
  e = kron::launch_column_reduce(a.part, G, PW, rp, stream);
  if (e != hipSuccess) return hip_fail(e, "kron_linear_bwd_bf16 reduce launch");
  return ok();
}

kron_status_t ks_matmul_out(int64_t N, int32_t a, int32_t b, int32_t c, int32_t d, int32_t in_dtype, int32_t out_dtype,
                      const void* x, const void* vals, void* y, hipStream_t stream) {
  if (N < 0 || N > kMaxRows) return fail(KRON_E_SHAPE, "N = %lld out of range", (long long)N);
  if (a < 1 || b < 1 || c < 1 || d < 1) return fail(KRON_E_SHAPE, "a, b, c, d must be >= 1");
  const int64_t in = (int64_t)a * b * d, out = (int64_t)a * c * d;
  if (in > kMaxFeatures || out > kMaxFeatures)
    return fail(KRON_E_UNSUPPORTED, "a*b*d = %lld or a*c*d = %lld exceeds %lld", (long long)in,
                (long long)out, (long long)kMaxFeatures);
  if (in_dtype != KRON_F32 && in_dtype != KRON_BF16) return fail(KRON_E_DTYPE, "input dtype %d", in_dtype);
  if (out_dtype != KRON_F32 && out_dtype != KRON_BF16) return fail(KRON_E_DTYPE, "output dtype %d", out_dtype);
  if (!kron::ks_supported(a, b, c, d)) return fail(KRON_E_UNSUPPORTED, "b*d = %lld too large", (long long)b * d);
  if (!vals) return fail(KRON_E_NULL, "vals is required");
  if (N > 0 && (!x || !y)) return fail(KRON_E_NULL, "x and y are required when N > 0");
  const size_t es = in_dtype == KRON_F32 ? 4 : 2, os = out_dtype == KRON_F32 ? 4 : 2;
  const Range ins[2] = {{x, (size_t)N * in * es, "x"}, {vals, (size_t)a * b * c * d * es, "vals"}};
  const Range outs[1] = {{y, (size_t)N * out * os, "y"}};
  kron_status_t st;
  if ((st = check_align(ins, 2)) != KRON_OK || (st = check_align(outs, 1)) != KRON_OK) return st;
  if ((st = check_alias(outs, 1, ins, 2)) != KRON_OK) return st;
  if (N == 0) return ok();
  kron::KSArgs k{N, a, b, c, d, in_dtype, out_dtype, x, vals, y};
  hipError_t e = kron::launch_ks(k, stream);
  if (e != hipSuccess) return hip_fail(e, "ks_matmul launch");
  return ok();
}

kron_status_t ks_matmul(int64_t N, int32_t a, int32_t b, int32_t c, int32_t d, int32_t in_dtype, const void* x,
                  const void* vals, float* y, hipStream_t stream) {
  return ks_matmul_out(N, a, b, c, d, in_dtype, KRON_F32, x, vals, y, stream);
}

namespace {
constexpr int64_t kMaxKsValues = int64_t{1} << 28;   // dvals columns of the reduction (int32)

kron_status_t ks_shape_check(int64_t N, int32_t a, int32_t b, int32_t c, int32_t d, int32_t in_dtype) {
  if (N < 0 || N > kMaxRows) return fail(KRON_E_SHAPE, "N = %lld out of range", (long long)N);
  if (a < 1 || b < 1 || c < 1 || d < 1) return fail(KRON_E_SHAPE, "a, b, c, d must be >= 1");
  const int64_t in = (int64_t)a * b * d, out = (int64_t)a * c * d;
  if (in > kMaxFeatures || out > kMaxFeatures)
    return fail(KRON_E_UNSUPPORTED, "a*b*d = %lld or a*c*d = %lld exceeds %lld", (long long)in,
                (long long)out, (long long)kMaxFeatures);
  if ((int64_t)a * b * c * d > kMaxKsValues)
    return fail(KRON_E_UNSUPPORTED, "a*b*c*d = %lld values exceed %lld", (long long)a * b * c * d,
                (long long)kMaxKsValues);
  if (in_dtype != KRON_F32 && in_dtype != KRON_BF16) return fail(KRON_E_DTYPE, "input dtype %d", in_dtype);
  if (!kron::ks_supported(a, b, c, d) || !kron::ks_bwd_supported(a, b, c, d))
    return fail(KRON_E_UNSUPPORTED, "b*d = %lld or c*d = %lld too large", (long long)b * d, (long long)c * d);
  return KRON_OK;
}
}  // namespace

size_t ks_matmul_bwd_workspace_bytes(int64_t N, int32_t a, int32_t b, int32_t c, int32_t d, int32_t in_dtype) {
  if (ks_shape_check(N, a, b, c, d, in_dtype) != KRON_OK) return 0;
  return kron::ks_bwd_workspace_bytes(N, a, b, c, d, in_dtype);
}

kron_status_t ks_matmul_bwd(int64_t N, int32_t a, int32_t b, int32_t c, int32_t d, int32_t in_dtype, const void* x,
                      const void* vals, const void* dy, float* dx, float* dvals, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  kron_status_t st = ks_shape_check(N, a, b, c, d, in_dtype);
  if (st != KRON_OK) return st;
  if (!dx && !dvals) return ok();
  if (dx && !vals) return fail(KRON_E_NULL, "vals is required for dx");
  if (N > 0 && !dy) return fail(KRON_E_NULL, "dy is required when N > 0");
  if (N > 0 && dvals && !x) return fail(KRON_E_NULL, "x is required for dvals when N > 0");
  const size_t need = kron::ks_bwd_workspace_bytes(N, a, b, c, d, in_dtype);
  if (!workspace || workspace_bytes < need)
    return fail(KRON_E_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0) return fail(KRON_E_ALIGN, "workspace is not 256-byte aligned");
  const size_t es = in_dtype == KRON_F32 ? 4 : 2;
  const int64_t in = (int64_t)a * b * d, out = (int64_t)a * c * d, nv = (int64_t)a * b * c * d;
  const Range ins[4] = {{x, (size_t)N * in * es, "x"},
                        {vals, (size_t)nv * es, "vals"},
                        {dy, (size_t)N * out * es, "dy"},
                        {workspace, need, "workspace"}};
  const Range outs[2] = {{dx, (size_t)N * in * 4, "dx"}, {dvals, (size_t)nv * 4, "dvals"}};
  if ((st = check_align(ins, 4)) != KRON_OK || (st = check_align(outs, 2)) != KRON_OK) return st;
  if ((st = check_alias(outs, 2, ins, 4)) != KRON_OK) return st;
  kron::KSBwdArgs k{N, a, b, c, d, in_dtype, x, vals, dy, N > 0 ? dx : nullptr, dvals};
  hipError_t e = kron::launch_ks_bwd(k, workspace, stream);
  if (e != hipSuccess) return hip_fail(e, "ks_matmul_bwd launch");
  return ok();
}

kron_status_t ks_chain(int64_t N, int32_t nfactors, const ks_factor_t* factors, int32_t in_dtype, const void* x, float* y,
                 hipStream_t stream) {
  if (N < 0 || N > kMaxRows) return fail(KRON_E_SHAPE, "N = %lld out of range", (long long)N);
  if (nfactors < 1 || nfactors > kron::kChainMaxFactors)
    return fail(KRON_E_ARG, "nfactors = %d outside 1..%d", nfactors, kron::kChainMaxFactors);
  if (!factors) return fail(KRON_E_NULL, "factors is required");
  if (in_dtype != KRON_F32 && in_dtype != KRON_BF16) return fail(KRON_E_DTYPE, "input dtype %d", in_dtype);
  const size_t es = in_dtype == KRON_F32 ? 4 : 2;
  kron::ChainArgs A{};
  A.N = N;
  A.nf = nfactors;
  A.dtype = in_dtype;
  int64_t width = 0, maxw = 0;
  Range ins[kron::kChainMaxFactors + 1];
  for (int32_t f = 0; f < nfactors; ++f) {
    const ks_factor_t& F = factors[f];
    if (F.a < 1 || F.b < 1 || F.c < 1 || F.d < 1) return fail(KRON_E_SHAPE, "factor %d: a, b, c, d must be >= 1", f);
    const int64_t win = (int64_t)F.a * F.b * F.d, wout = (int64_t)F.a * F.c * F.d;
    if (win > kron::kChainMaxWidth || wout > kron::kChainMaxWidth)
      return fail(KRON_E_UNSUPPORTED, "factor %d: width %lld -> %lld exceeds %d", f, (long long)win, (long long)wout,
                  kron::kChainMaxWidth);
    if (f > 0 && win != width)
      return fail(KRON_E_SHAPE, "factor %d takes %lld values per row, factor %d gives %lld", f, (long long)win, f - 1,
                  (long long)width);
    if (!F.vals) return fail(KRON_E_NULL, "factor %d: vals is required", f);
    ins[f + 1] = Range{F.vals, (size_t)F.a * F.b * F.c * F.d * es, "vals"};
    A.f[f] = kron::ChainFactor{F.a, F.b, F.c, F.d, F.vals};
    maxw = win > maxw ? win : maxw;
    maxw = wout > maxw ? wout : maxw;
    width = wout;
  }
  const int64_t w0 = (int64_t)factors[0].a * factors[0].b * factors[0].d;
  if (N > 0 && (!x || !y)) return fail(KRON_E_NULL, "x and y are required when N > 0");
  ins[0] = Range{x, (size_t)N * w0 * es, "x"};
  const Range outs[1] = {{y, (size_t)N * width * 4, "y"}};
  kron_status_t st;
  if ((st = check_align(ins, nfactors + 1)) != KRON_OK || (st = check_align(outs, 1)) != KRON_OK) return st;
  if ((st = check_alias(outs, 1, ins, nfactors + 1)) != KRON_OK) return st;
  if (N == 0) return ok();
  A.maxw = (int32_t)maxw;
  A.wl = (int32_t)width;
  A.x = x;
  A.y = y;
  hipError_t e = kron::launch_ks_chain(A, stream);
  if (e != hipSuccess) return hip_fail(e, "ks_chain launch");
  return ok();
}

namespace {
constexpr int kVlMaxSide = 8192;   // p*q and m*n (one workgroup orthonormalises a p*q or m*n column)

kron_status_t van_loan_check(int32_t p, int32_t q, int32_t m, int32_t n, int32_t r, int32_t s, int32_t iters) {
  if (p < 1 || q < 1 || m < 1 || n < 1) return fail(KRON_E_SHAPE, "p, q, m, n must be >= 1");
  const int64_t M = (int64_t)p * q, K = (int64_t)m * n;
  if (M > kVlMaxSide || K > kVlMaxSide)
    return fail(KRON_E_UNSUPPORTED, "p*q = %lld or m*n = %lld exceeds %d", (long long)M, (long long)K, kVlMaxSide);
  if ((int64_t)p * m > kMaxFeatures || (int64_t)q * n > kMaxFeatures)
    return fail(KRON_E_UNSUPPORTED, "W of %lld x %lld exceeds %lld per side", (long long)p * m, (long long)q * n,
                (long long)kMaxFeatures);
  if (s < 1 || s > 32 || s > M || s > K) return fail(KRON_E_ARG, "s = %d outside 1..min(32, p*q, m*n)", s);
  if (r < 1 || r > s) return fail(KRON_E_ARG, "r = %d outside 1..s", r);
  if (iters < 0 || iters > 100) return fail(KRON_E_ARG, "iters = %d outside 0..100", iters);
  return KRON_OK;
}
}  // namespace

size_t kron_van_loan_workspace_bytes(int32_t p, int32_t q, int32_t m, int32_t n, int32_t s) {
  if (van_loan_check(p, q, m, n, 1, s, 0) != KRON_OK) return 0;
  return kron::van_loan_workspace_bytes(p, q, m, n, s);
}

kron_status_t kron_van_loan(int32_t p, int32_t q, int32_t m, int32_t n, int32_t r, int32_t s, int32_t iters, const float* W,
                      const float* omega, float* C, float* B, float* sigma, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  kron_status_t st = van_loan_check(p, q, m, n, r, s, iters);
  if (st != KRON_OK) return st;
  if (!W || !omega || !C || !B || !sigma) return fail(KRON_E_NULL, "W, omega, C, B and sigma are required");
  const size_t need = kron::van_loan_workspace_bytes(p, q, m, n, s);
  if (!workspace || workspace_bytes < need)
    return fail(KRON_E_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0) return fail(KRON_E_ALIGN, "workspace is not 256-byte aligned");
  const size_t M = (size_t)p * q, K = (size_t)m * n;
  const Range ins[3] = {{W, (size_t)p * m * q * n * 4, "W"}, {omega, K * s * 4, "omega"}, {workspace, need, "workspace"}};
  const Range outs[3] = {{C, r * M * 4, "C"}, {B, r * K * 4, "B"}, {sigma, (size_t)r * 4, "sigma"}};
  if ((st = check_align(ins, 3)) != KRON_OK || (st = check_align(outs, 3)) != KRON_OK) return st;
  if ((st = check_alias(outs, 3, ins, 3)) != KRON_OK) return st;
  kron::VanLoanArgs A{p, q, m, n, r, s, iters, W, omega, C, B, sigma};
  hipError_t e = kron::launch_van_loan(A, workspace, stream);
  if (e != hipSuccess) return hip_fail(e, "kron_van_loan launch");
  return ok();
}

kron_status_t kron_adam_l1_step(int32_t ntensors, float* const* params, const float* const* grads, float* const* m,
                          float* const* v, const int64_t* numel, const float* l1, int64_t step, double lr,
                          double beta1, double beta2, double eps, hipStream_t stream) {
  if (ntensors < 0 || ntensors > 4096) return fail(KRON_E_ARG, "ntensors = %d out of range", ntensors);
  if (ntensors == 0) return ok();
  if (!params || !grads || !m || !v || !numel) return fail(KRON_E_NULL, "pointer arrays are required");
  if (step < 1) return fail(KRON_E_ARG, "step = %lld must be >= 1", (long long)step);
  if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) || !(eps >= 0.0) || !std::isfinite(lr))
    return fail(KRON_E_ARG, "hyper-parameters out of range");
  for (int32_t t = 0; t < ntensors; ++t) {
    if (numel[t] < 0) return fail(KRON_E_ARG, "numel[%d] < 0", t);
    if (numel[t] == 0) continue;
    if (!params[t] || !grads[t] || !m[t] || !v[t]) return fail(KRON_E_NULL, "tensor %d has a NULL pointer", t);
    const Range rs[4] = {{params[t], 0, "param"}, {grads[t], 0, "grad"}, {m[t], 0, "m"}, {v[t], 0, "v"}};
    kron_status_t st = check_align(rs, 4);
    if (st != KRON_OK) return st;
    const size_t by = (size_t)numel[t] * 4;
    const Range outs[3] = {{params[t], by, "param"}, {m[t], by, "m"}, {v[t], by, "v"}};
    const Range ins[1] = {{grads[t], by, "grad"}};
    if ((st = check_alias(outs, 3, ins, 1)) != KRON_OK) return st;
  }
  const double bc1 = 1.0 - std::pow(beta1, (double)step);
  const double bc2 = 1.0 - std::pow(beta2, (double)step);
  kron::AdamHyper hp{(float)lr, (float)beta1, (float)(1.0 - beta1), (float)beta2, (float)(1.0 - beta2),
                     (float)eps, (float)(1.0 / bc1), (float)(1.0 / bc2)};
  for (int32_t t0 = 0; t0 < ntensors; t0 += kron::kAdamMaxPerLaunch) {
    kron::AdamBatch batch{};
    int64_t maxn = 0;
    for (int32_t t = t0; t < ntensors && t < t0 + kron::kAdamMaxPerLaunch; ++t) {
      if (numel[t] == 0) continue;
      kron::AdamTensor& T = batch.t[batch.count++];
      T.p = params[t]; T.g = grads[t]; T.m = m[t]; T.v = v[t]; T.numel = numel[t];
      T.l1 = l1 ? l1[t] : 0.f;
      if (numel[t] > maxn) maxn = numel[t];
    }
    hipError_t e = kron::launch_adam(batch, maxn, hp, stream);
    if (e != hipSuccess) return hip_fail(e, "kron_adam_l1_step launch");
  }
  return ok();
}

kron_status_t kron_relu_bwd(int64_t n, const float* y, const float* dy, float* out, hipStream_t stream) {
  if (n < 0) return fail(KRON_E_SHAPE, "n = %lld must be >= 0", (long long)n);
  if (n == 0) return ok();
  if (!y || !dy || !out) return fail(KRON_E_NULL, "y, dy and out are required");
  const Range rs[3] = {{y, 0, "y"}, {dy, 0, "dy"}, {out, 0, "out"}};
  kron_status_t st = check_align(rs, 3);
  if (st != KRON_OK) return st;
  const size_t by = (size_t)n * 4;
  const Range outs[1] = {{out, by, "out"}};
  const Range ins[2] = {{y, by, "y"}, {dy, by, "dy"}};
  // out may be dy itself (in place); any other overlap is refused
  if ((st = check_alias(outs, 1, ins, out == dy ? 1 : 2)) != KRON_OK) return st;
  hipError_t e = kron::launch_relu_bwd(n, y, dy, out, stream);
  if (e != hipSuccess) return hip_fail(e, "kron_relu_bwd launch");
  return ok();
}

kron_status_t kron_l1_penalty(int32_t ntensors, const float* const* tensors, const int64_t* numel, float lam,
                              float* loss, uint32_t flags, hipStream_t stream) {
  if (ntensors < 0 || ntensors > kron::kL1MaxTensors)
    return fail(KRON_E_ARG, "ntensors = %d out of range [0, %d]", ntensors, kron::kL1MaxTensors);
  if (!loss) return fail(KRON_E_NULL, "loss is required");
  if (ntensors > 0 && (!tensors || !numel)) return fail(KRON_E_NULL, "tensors and numel are required");
  if (flags & ~KRON_ACCUMULATE) return fail(KRON_E_ARG, "unknown flag bits 0x%x", flags);
  if (!std::isfinite(lam)) return fail(KRON_E_ARG, "lam is not finite");
  const Range lr[1] = {{loss, 4, "loss"}};
  kron_status_t st = check_align(lr, 1);
  if (st != KRON_OK) return st;
  kron::L1Batch b{};
  for (int32_t t = 0; t < ntensors; ++t) {
    if (numel[t] < 0) return fail(KRON_E_ARG, "numel[%d] < 0", t);
    if (numel[t] == 0) continue;
    if (!tensors[t]) return fail(KRON_E_NULL, "tensor %d is NULL", t);
    const Range in[1] = {{tensors[t], (size_t)numel[t] * 4, "tensor"}};
    if ((st = check_align(in, 1)) != KRON_OK) return st;
    if ((st = check_alias(lr, 1, in, 1)) != KRON_OK) return st;
    b.t[b.count] = tensors[t];
    b.numel[b.count] = numel[t];
    ++b.count;
  }
  hipError_t e = kron::launch_l1_penalty(b, lam, loss, (flags & KRON_ACCUMULATE) != 0, stream);
  if (e != hipSuccess) return hip_fail(e, "kron_l1_penalty launch");
  return ok();
}

kron_status_t kron_l1_penalty_grad(int64_t n, const float* S, float lam, const float* g, float* dS,
                                   hipStream_t stream) {
  if (n < 0) return fail(KRON_E_SHAPE, "n = %lld must be >= 0", (long long)n);
  if (n == 0) return ok();
  if (!S || !g || !dS) return fail(KRON_E_NULL, "S, g and dS are required");
  if (!std::isfinite(lam)) return fail(KRON_E_ARG, "lam is not finite");
  const Range rs[3] = {{S, 0, "S"}, {g, 0, "g"}, {dS, 0, "dS"}};
  kron_status_t st = check_align(rs, 3);
  if (st != KRON_OK) return st;
  const Range outs[1] = {{dS, (size_t)n * 4, "dS"}};
  const Range ins[2] = {{S, (size_t)n * 4, "S"}, {g, 4, "g"}};
  if ((st = check_alias(outs, 1, ins, 2)) != KRON_OK) return st;
  hipError_t e = kron::launch_l1_grad(n, S, lam, g, dS, stream);
  if (e != hipSuccess) return hip_fail(e, "kron_l1_penalty_grad launch");
  return ok();
}

size_t kron_head_ce_workspace_bytes(int64_t N, int32_t K, int32_t C) {
  if (N < 0 || K < 1 || C < 1) return 0;
  // the larger of the two paths' partial sums (the matrix-core path uses more groups)
  const int64_t PW = (int64_t)K * C + C + 1;
  const int64_t p1 = kron::part_floats(kron::head_groups(N), PW);
  const int64_t p2 = kron::head_mfma_ok(K, C) ? kron::part_floats(kron::head_mfma_groups(N), PW) : 0;
  const size_t floats = (size_t)N * C + (size_t)N + (size_t)(p1 > p2 ? p1 : p2);
  return ((floats * 4 + 255) & ~size_t(255)) + 256;
}

kron_status_t kron_head_ce(int64_t N, int32_t K, int32_t C, const float* h, const float* Wh, const float* bh,
                     const int64_t* labels, float* loss, float* dh, float* dWh, float* dbh, uint32_t flags,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (N < 0 || N > kMaxRows) return fail(KRON_E_SHAPE, "N = %lld out of range", (long long)N);
  if (K < 1 || C < 1) return fail(KRON_E_SHAPE, "K and C must be >= 1");
  if (C > 64 || K > 8192 || (int64_t)K * C > 16384)
    return fail(KRON_E_UNSUPPORTED, "K = %d, C = %d beyond the limits (C <= 64, K <= 8192, K*C <= 16384)", K, C);
  if (flags & ~KRON_DX_RELU_MASK) return fail(KRON_E_ARG, "unknown flag bits 0x%x", flags);
  if (!Wh || !bh || !loss || !dWh || !dbh) return fail(KRON_E_NULL, "Wh, bh, loss, dWh and dbh are required");
  if (N > 0 && (!h || !labels)) return fail(KRON_E_NULL, "h and labels are required when N > 0");
  const size_t need = kron_head_ce_workspace_bytes(N, K, C);
  if (!workspace || workspace_bytes < need)
    return fail(KRON_E_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0) return fail(KRON_E_ALIGN, "workspace is not 256-byte aligned");
  const Range ins[5] = {{h, (size_t)N * K * 4, "h"},      {Wh, (size_t)K * C * 4, "Wh"}, {bh, (size_t)C * 4, "bh"},
                        {labels, (size_t)N * 8, "labels"}, {workspace, need, "workspace"}};
  const Range outs[4] = {{loss, 4, "loss"}, {dh, (size_t)N * K * 4, "dh"}, {dWh, (size_t)K * C * 4, "dWh"},
                         {dbh, (size_t)C * 4, "dbh"}};
  kron_status_t st;
  if ((st = check_align(ins, 5)) != KRON_OK || (st = check_align(outs, 4)) != KRON_OK) return st;
  if ((st = check_alias(outs, 4, ins, 5)) != KRON_OK) return st;
  kron::HeadArgs a{};
  a.N = N; a.K = K; a.C = C; a.flags = flags; a.h = h; a.W = Wh; a.b = bh; a.labels = labels;
  a.loss = loss; a.dh = dh; a.dW = dWh; a.db = dbh;
  a.dz = (float*)workspace;
  const size_t dz_floats = ((size_t)N * C + (size_t)N + 63) & ~size_t(63);
  a.part = a.dz + dz_floats;
  hipError_t e = kron::launch_head(a, kron::head_groups(N), stream);
  if (e != hipSuccess) return hip_fail(e, "kron_head_ce launch");
  return ok();
}

}  // extern "C"
