// C ABI of liblapnys (declared in include/lapnys.h): parameter validation,
// the per-call plan and workspace layout, the stage sequence, the
// library-owned workspace of lapnys_forward, and the debug/profiled forms.
//
// Stage sequence (no host synchronisation), all on the caller's stream:
//   pool      K -> K~
//   kernel    Q, K, V, K~ -> C^T, tile statistics, B V partials; for m <= 64
//             the same launch also runs the Newton-Schulz solver (K~ -> W, X)
//   finalize  partials -> mu, sigma, B V
//   output    Y = X (B V), then O = whiten(C) Y
// For 64 < m <= 256 the solver is a sequence of launches on a library-owned
// stream of the device (default priority), forked after the pool stage and
// joined before Y = X (B V), which is then its own launch in the finalize
// stage.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "lapnys.h"
#include "lapnys_internal.hpp"

using lapnys::Plan;

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// LAPNYS_LOG=1 in the environment prints each failing HIP call to stderr.
bool log_enabled() {
  static const bool on = [] {
    const char* e = getenv("LAPNYS_LOG");
    return e && *e && *e != '0';
  }();
  return on;
}

bool ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  if (log_enabled()) fprintf(stderr, "liblapnys: %s failed: %s (%d)\n", what, hipGetErrorString(e), (int)e);
  return false;
}

int validate(const lapnys_params* p) {
  if (!p) return LAPNYS_ERR_INVALID_ARG;
  if (p->B <= 0 || p->H <= 0 || p->N <= 0 || p->d <= 0 || p->grid_h <= 0 || p->grid_w <= 0 || p->pool <= 0)
    return LAPNYS_ERR_INVALID_ARG;
  if (!(isfinite(p->lambda) && p->lambda > 0.f)) return LAPNYS_ERR_INVALID_ARG;
  if (!(isfinite(p->eps) && p->eps >= 0.f)) return LAPNYS_ERR_INVALID_ARG;
  if (p->ns_iters < 0) return LAPNYS_ERR_INVALID_ARG;
  if (p->flags &
      ~(uint32_t)(LAPNYS_WHITEN | LAPNYS_NS_REFINE | LAPNYS_GAUSSIAN | LAPNYS_SOLVER_CG | LAPNYS_NS_PLAIN))
    return LAPNYS_ERR_INVALID_ARG;
  if ((p->flags & LAPNYS_SOLVER_CG) && (p->flags & LAPNYS_NS_REFINE)) return LAPNYS_ERR_INVALID_ARG;
  if (p->dtype != LAPNYS_F32 && p->dtype != LAPNYS_BF16) return LAPNYS_ERR_UNSUPPORTED;
  if ((int64_t)p->grid_h * p->grid_w != (int64_t)p->N) return LAPNYS_ERR_SHAPE;
  if (p->grid_h % p->pool || p->grid_w % p->pool) return LAPNYS_ERR_SHAPE;
  if (p->d != 32 && p->d != 64) return LAPNYS_ERR_UNSUPPORTED;
  const int64_t m = (int64_t)(p->grid_h / p->pool) * (p->grid_w / p->pool);
  if (m > lapnys::kMaxM) return LAPNYS_ERR_UNSUPPORTED;
  if ((int64_t)p->B * p->H > 65535) return LAPNYS_ERR_UNSUPPORTED;  // problems map to one grid axis
  return LAPNYS_OK;
}

int make_plan(const lapnys_params* p, Plan* pl) {
  const int st = validate(p);
  if (st != LAPNYS_OK) return st;
  Plan& P = *pl;
  memset(&P, 0, sizeof(P));
  P.P = p->B * p->H;
  P.N = p->N;
  P.ldc = (p->N + 3) & ~3;
  P.d = p->d;
  P.grid_w = p->grid_w;
  P.pool = p->pool;
  P.gw = p->grid_w / p->pool;
  P.m = (p->grid_h / p->pool) * P.gw;
  P.dtype = p->dtype;
  P.whiten = (p->flags & LAPNYS_WHITEN) != 0;
  P.ns_iters = p->ns_iters;
  P.refine = (p->flags & LAPNYS_NS_REFINE) != 0;
  P.gaussian = (p->flags & LAPNYS_GAUSSIAN) != 0;
  P.cg = (p->flags & LAPNYS_SOLVER_CG) != 0;
  // exp(-s / lambda) = exp2(s * scale)
  P.scale = (float)(-1.4426950408889634074 / (double)p->lambda);
  P.eps = p->eps;
  // m <= 64: one workgroup per problem runs the steps (inside the
  // kernel-matrix launch for the Laplacian form, a launch of its own beside
  // it for the Gaussian form).
  P.fused_ns = P.m <= lapnys::kFusedNsMaxM && !P.cg;
  // The in-launch schedule is the Laplacian default; the Gaussian form and
  // LAPNYS_NS_PLAIN run the plain steps as a launch of their own.
  P.ns_in_launch = P.fused_ns && !P.gaussian && !(p->flags & LAPNYS_NS_PLAIN);
  P.mp = P.fused_ns ? 64 : ((P.m + 63) / 64) * 64;
  P.tt = 256;
  P.ntiles = (P.N + P.tt - 1) / P.tt;
  // Landmark blocks: all m <= 64 landmarks in one block (every solver of the
  // Laplacian form; the Gaussian form beside its Newton-Schulz solver), else
  // blocks of 32.
  const bool one_block = P.m <= lapnys::kFusedNsMaxM && (!P.gaussian || P.fused_ns);
  P.lb = one_block ? P.m : (P.m < 32 ? P.m : 32);
  P.jblocks = (P.m + P.lb - 1) / P.lb;
  // Tiles per workgroup: enough workgroups to fill the chip several times,
  // few enough that the B V partials stay small.
  const int64_t jobs = (int64_t)P.ntiles * P.jblocks * P.P;
  P.tpg = (int)(jobs / 4096 > 1 ? jobs / 4096 : 1);
  P.groups = (P.ntiles + P.tpg - 1) / P.tpg;
  const size_t f = sizeof(float);
  const size_t Pn = (size_t)P.P;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  P.off_kt = take(Pn * P.m * P.d * f);
  P.off_w = take(Pn * P.mp * P.mp * f);
  P.off_x = take(Pn * P.mp * P.mp * f);
  // The second iterate and the product buffer serve the tiled solver's
  // steps, and the correction of LAPNYS_NS_REFINE at any size.
  const bool tiled = !P.fused_ns || P.refine;
  P.off_x2 = take(tiled ? Pn * P.mp * P.mp * f : 0);
  P.off_pm = take(tiled ? Pn * P.mp * P.mp * f : 0);
  P.off_ct = take(Pn * P.m * (size_t)P.ldc * f);
  P.off_stats = take(Pn * P.ntiles * P.m * 2 * f);
  P.off_bvpart = take(Pn * P.groups * P.m * P.d * f);
  P.off_bv = take(Pn * P.m * P.d * f);
  P.off_mu = take(Pn * P.m * f);
  P.off_sigma = take(Pn * P.m * f);
  P.off_rs = take(Pn * P.m * f);
  P.off_y = take(Pn * P.m * P.d * f);
  P.off_yt = take(P.fused_ns ? Pn * 2 * P.d * 64 * sizeof(uint16_t) : 0);
  P.total = off;
  return LAPNYS_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int check_buffers(const void* q, const void* k, const void* v, const float* out, const Plan& pl, const void* ws,
                  size_t ws_bytes) {
  if (!q || !k || !v || !out) return LAPNYS_ERR_INVALID_ARG;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) return LAPNYS_ERR_INVALID_ARG;
  const size_t elems = (size_t)pl.P * pl.N * pl.d;
  const size_t in_bytes = elems * (pl.dtype == LAPNYS_BF16 ? 2 : 4);
  const size_t out_bytes = elems * 4;
  if (overlaps(out, out_bytes, q, in_bytes) || overlaps(out, out_bytes, k, in_bytes) ||
      overlaps(out, out_bytes, v, in_bytes))
    return LAPNYS_ERR_INVALID_ARG;
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < pl.total) return LAPNYS_ERR_WORKSPACE;
  if (overlaps(out, out_bytes, ws, pl.total)) return LAPNYS_ERR_INVALID_ARG;
  return LAPNYS_OK;
}

lapnys::Work carve(const Plan& pl, void* ws) {
  char* b = (char*)ws;
  lapnys::Work W;
  W.kt = (float*)(b + pl.off_kt);
  W.w = (float*)(b + pl.off_w);
  W.x = (float*)(b + pl.off_x);
  W.x2 = (float*)(b + pl.off_x2);
  W.pm = (float*)(b + pl.off_pm);
  W.ct = (float*)(b + pl.off_ct);
  W.stats = (float*)(b + pl.off_stats);
  W.bvpart = (float*)(b + pl.off_bvpart);
  W.bv = (float*)(b + pl.off_bv);
  W.mu = (float*)(b + pl.off_mu);
  W.sigma = (float*)(b + pl.off_sigma);
  W.rs = (float*)(b + pl.off_rs);
  W.y = (float*)(b + pl.off_y);
  W.yt = (__bf16*)(b + pl.off_yt);
  W.x_final = W.x;
  return W;
}

// Per-device side stream and the fork/join events, created on first use.
struct DeviceCtx {
  hipStream_t side = nullptr;
  hipEvent_t pooled = nullptr, join = nullptr;
};
std::mutex g_ctx_mu;  // also serialises the fork/join sequence of concurrent callers
std::vector<DeviceCtx> g_ctx;

int device_ctx(DeviceCtx** out) {
  int dev = 0;
  if (!ok(hipGetDevice(&dev), "hipGetDevice") || dev < 0) return LAPNYS_ERR_HIP;
  if ((int)g_ctx.size() <= dev) g_ctx.resize(dev + 1);
  DeviceCtx& c = g_ctx[dev];
  if (!c.side) {
    if (!ok(hipStreamCreateWithFlags(&c.side, hipStreamNonBlocking), "hipStreamCreateWithFlags")) {
      c.side = nullptr;
      return LAPNYS_ERR_HIP;
    }
    // The fork/join events order work between two streams of one device: a
    // device-scope release is all they need (no host-visible write-back).
    const unsigned flags = hipEventDisableTiming | hipEventReleaseToDevice;
    if (!ok(hipEventCreateWithFlags(&c.join, flags), "hipEventCreateWithFlags") ||
        !ok(hipEventCreateWithFlags(&c.pooled, flags), "hipEventCreateWithFlags"))
      return LAPNYS_ERR_HIP;
  }
  *out = &c;
  return LAPNYS_OK;
}

int run(const Plan& pl, const void* q, const void* k, const void* v, float* out, lapnys::Work& W, hipEvent_t* ev,
        hipStream_t s) {
  // An error left by an earlier, unrelated runtime call would otherwise be
  // reported by the first launch check below.
  (void)hipGetLastError();
  auto span = [&](int stage) {
    lapnys::Span t;
    if (ev) {
      t.start = ev[2 * stage];
      t.stop = ev[2 * stage + 1];
    }
    return t;
  };
  auto mark = [&](int idx) { return !ev || !ev[idx] || ok(hipEventRecord(ev[idx], s), "hipEventRecord"); };
  const lapnys::Span fin = span(LAPNYS_STAGE_FINALIZE);

  if (pl.ns_in_launch) {
    // m <= 64: one stream; the solver runs inside the kernel-matrix launch,
    // and its stage events bracket that launch.
    if (!ok(lapnys::launch_pool(pl, k, W, s, span(LAPNYS_STAGE_POOL)), "pool launch")) return LAPNYS_ERR_HIP;
    if (!mark(2 * LAPNYS_STAGE_NS)) return LAPNYS_ERR_HIP;
    if (!ok(lapnys::launch_l1exp(pl, q, k, v, W, s, span(LAPNYS_STAGE_KERNEL)), "kernel-matrix launch"))
      return LAPNYS_ERR_HIP;
    if (pl.refine && !ok(lapnys::launch_refine(pl, W, s), "refinement launch")) return LAPNYS_ERR_HIP;
    if (!mark(2 * LAPNYS_STAGE_NS + 1)) return LAPNYS_ERR_HIP;
    if (!ok(lapnys::launch_reduce(pl, W, s, fin), "reduce launch")) return LAPNYS_ERR_HIP;
    if (out && !ok(lapnys::launch_output(pl, W, out, s, span(LAPNYS_STAGE_OUTPUT)), "output launch"))
      return LAPNYS_ERR_HIP;
    return LAPNYS_OK;
  }

  // Otherwise (m > 64, the Gaussian form, the plain steps, CG): the solver's
  // launches run on a library-owned stream beside the kernel-matrix stage,
  // forked from the caller's stream after the pool stage and joined before
  // the stages that read the solver's result.  Each stream waits only on an
  // event recorded last on the other stream before the wait is issued (the
  // runtime may resolve a wait on an event recorded earlier than the other
  // stream's latest work no sooner than that latest work).
  std::lock_guard<std::mutex> lock(g_ctx_mu);
  DeviceCtx* dc = nullptr;
  const int st = device_ctx(&dc);
  if (st != LAPNYS_OK) return st;
  hipStream_t side = dc->side;
  if (!ok(lapnys::launch_pool(pl, k, W, s, span(LAPNYS_STAGE_POOL)), "pool launch")) return LAPNYS_ERR_HIP;
  if (!ok(hipEventRecord(dc->pooled, s), "hipEventRecord") || !ok(hipStreamWaitEvent(side, dc->pooled, 0), "hipStreamWaitEvent"))
    return LAPNYS_ERR_HIP;
  if (!ok(lapnys::launch_ns(pl, W, side, span(LAPNYS_STAGE_NS)), "Newton-Schulz launch")) return LAPNYS_ERR_HIP;
  if (!ok(hipEventRecord(dc->join, side), "hipEventRecord")) return LAPNYS_ERR_HIP;
  const lapnys::Span ks = span(LAPNYS_STAGE_KERNEL);
  if (!ok(pl.gaussian ? lapnys::launch_gauss(pl, q, k, v, W, s, ks) : lapnys::launch_l1exp(pl, q, k, v, W, s, ks),
          "kernel-matrix launch"))
    return LAPNYS_ERR_HIP;
  if (pl.fused_ns) {
    // m <= 64 (a solver launch of its own): the reductions also form
    // Y = X (B V), so they wait for the solver.
    if (!ok(hipStreamWaitEvent(s, dc->join, 0), "hipStreamWaitEvent")) return LAPNYS_ERR_HIP;
    if (!ok(lapnys::launch_reduce(pl, W, s, fin), "reduce launch")) return LAPNYS_ERR_HIP;
  } else if (pl.cg) {
    // CG: Y = W^-1 (B V) once B V and W are both there.
    if (!ok(lapnys::launch_reduce(pl, W, s, {fin.start, nullptr}), "reduce launch")) return LAPNYS_ERR_HIP;
    if (!ok(hipStreamWaitEvent(s, dc->join, 0), "hipStreamWaitEvent")) return LAPNYS_ERR_HIP;
    if (!ok(lapnys::launch_cg(pl, W, s, fin.stop), "CG launch")) return LAPNYS_ERR_HIP;
  } else {
    if (!ok(lapnys::launch_reduce(pl, W, s, {fin.start, nullptr}), "reduce launch")) return LAPNYS_ERR_HIP;
    if (!ok(hipStreamWaitEvent(s, dc->join, 0), "hipStreamWaitEvent")) return LAPNYS_ERR_HIP;
    if (!ok(lapnys::launch_y(pl, W, s, {nullptr, fin.stop}), "Y launch")) return LAPNYS_ERR_HIP;
  }
  if (out && !ok(lapnys::launch_output(pl, W, out, s, span(LAPNYS_STAGE_OUTPUT)), "output launch"))
    return LAPNYS_ERR_HIP;
  return LAPNYS_OK;
}

int forward_impl(const void* q, const void* k, const void* v, float* out, const lapnys_params* p, void* ws,
                 size_t ws_bytes, hipEvent_t* ev, const lapnys_debug* dbg, hipStream_t s) {
  Plan pl;
  int st = make_plan(p, &pl);
  if (st != LAPNYS_OK) return st;
  st = check_buffers(q, k, v, out, pl, ws, ws_bytes);
  if (st != LAPNYS_OK) return st;
  lapnys::Work B = carve(pl, ws);
  if (dbg && dbg->kernel_clock) {
    // earliest start (atomic minimum from all ones) and latest end (atomic maximum from zero)
    if (!ok(hipMemsetAsync(dbg->kernel_clock, 0xff, sizeof(unsigned long long), s), "hipMemsetAsync") ||
        !ok(hipMemsetAsync(dbg->kernel_clock + 1, 0, sizeof(unsigned long long), s), "hipMemsetAsync"))
      return LAPNYS_ERR_HIP;
    B.kclk = dbg->kernel_clock;
  }
  if (dbg && dbg->ns_clock && pl.ns_in_launch) B.nsclk = dbg->ns_clock;
  st = run(pl, q, k, v, out, B, ev, s);
  if (st != LAPNYS_OK || !dbg) return st;
  const size_t f = sizeof(float);
  const size_t Pm = (size_t)pl.P * pl.m;
  auto cp = [&](float* dst, const float* src, size_t bytes) {
    return !dst || ok(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s), "debug copy");
  };
  // C^T rows are stored with stride ldc >= N; the debug copy is dense.
  const bool ct_ok = !dbg->C_t || ok(hipMemcpy2DAsync(dbg->C_t, pl.N * f, B.ct, pl.ldc * f, pl.N * f, Pm,
                                                      hipMemcpyDeviceToDevice, s),
                                     "debug copy");
  bool good = ct_ok && cp(dbg->landmarks, B.kt, Pm * pl.d * f) &&
              cp(dbg->BV, B.bv, Pm * pl.d * f) && cp(dbg->mu, B.mu, Pm * f) && cp(dbg->sigma, B.sigma, Pm * f);
  // Y for m <= 64 lives only in the output stage's LDS; the debug form forms
  // it once more with the tile GEMM into the workspace.
  if (good && dbg->Y && pl.fused_ns) good = ok(lapnys::launch_y(pl, B, s), "Y launch");
  if (good) good = cp(dbg->Y, B.y, Pm * pl.d * f);
  if (good && dbg->W) good = ok(lapnys::launch_extract_square(B.w, pl.mp, dbg->W, pl.m, pl.P, s), "W extract");
  if (good && dbg->X && !pl.cg)
    good = ok(lapnys::launch_extract_square(B.x_final, pl.mp, dbg->X, pl.m, pl.P, s), "X extract");
  if (!good || !ok(hipStreamSynchronize(s), "hipStreamSynchronize")) return LAPNYS_ERR_HIP;
  return LAPNYS_OK;
}

// Backward buffers after the forward's workspace (each 256-byte aligned).
constexpr int kBwdBuffers = 15;

int backward_plan(const lapnys_params* p, Plan* pl, size_t off[kBwdBuffers], size_t* total) {
  const int st = make_plan(p, pl);
  if (st != LAPNYS_OK) return st;
  if (pl->cg || pl->gaussian) return LAPNYS_ERR_UNSUPPORTED;
  const size_t f = sizeof(float), Pn = (size_t)pl->P, m = (size_t)pl->m, d = (size_t)pl->d, N = (size_t)pl->N;
  const size_t mp = (size_t)pl->mp, nt = (N + 255) / 256;
  const bool big = pl->m > lapnys::kFusedNsMaxM;
  const size_t sizes[kBwdBuffers] = {
      Pn * nt * m * d * f, Pn * nt * d * f, Pn * m * d * f, Pn * m * d * f, Pn * 2 * m * f, Pn * mp * mp * f,
      Pn * m * N * f,      Pn * m * N * f,  Pn * m * d * f,
      Pn * mp * d * f,           big ? Pn * d * mp * f : 0, Pn * d * f,           big ? Pn * mp * mp * f : 0,
      big ? Pn * mp * mp * f : 0, big ? Pn * mp * mp * f : 0};
  size_t o = pl->total;
  for (int i = 0; i < kBwdBuffers; ++i) {
    off[i] = o;
    o = align256(o + sizes[i]);
  }
  *total = o;
  return LAPNYS_OK;
}

int backward_impl(const void* q, const void* k, const void* v, const float* dout, float* dq, float* dk, float* dv,
                  const lapnys_params* p, void* ws, size_t ws_bytes, hipStream_t s) {
  Plan pl;
  size_t off[kBwdBuffers], total = 0;
  int st = backward_plan(p, &pl, off, &total);
  if (st != LAPNYS_OK) return st;
  if (!dout || !dk || !dv || (((uintptr_t)dout | (uintptr_t)dk | (uintptr_t)dv) & 15)) return LAPNYS_ERR_INVALID_ARG;
  // dq is checked as an output buffer of the forward's shape would be.
  st = check_buffers(q, k, v, dq, pl, ws, ws_bytes);
  if (st != LAPNYS_OK) return st;
  if (ws_bytes < total) return LAPNYS_ERR_WORKSPACE;
  const size_t elems = (size_t)pl.P * pl.N * pl.d;
  const size_t in_bytes = elems * (pl.dtype == LAPNYS_BF16 ? 2 : 4), out_bytes = elems * 4;
  const void* ins[4] = {q, k, v, dout};
  const size_t in_sz[4] = {in_bytes, in_bytes, in_bytes, out_bytes};
  const float* outs[3] = {dq, dk, dv};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 4; ++i)
      if (overlaps(outs[o], out_bytes, ins[i], in_sz[i])) return LAPNYS_ERR_INVALID_ARG;
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlaps(outs[o], out_bytes, outs[o2], out_bytes)) return LAPNYS_ERR_INVALID_ARG;
    if (overlaps(outs[o], out_bytes, ws, total)) return LAPNYS_ERR_INVALID_ARG;
  }
  if (overlaps(dout, out_bytes, ws, total)) return LAPNYS_ERR_INVALID_ARG;
  char* b = (char*)ws;
  lapnys::BwdWork B;
  float** slots[kBwdBuffers] = {&B.part, &B.spart, &B.y,  &B.dbv, &B.ab, &B.dw, &B.gt, &B.ht,
                                &B.dkt,  &B.dy,    &B.bvt, &B.s,   &B.xt, &B.dx, &B.r};
  for (int i = 0; i < kBwdBuffers; ++i) *slots[i] = (float*)(b + off[i]);
  // The forward leaves B in the H^T buffer, which the backward turns into H
  // in place.
  lapnys::Work W = carve(pl, ws);
  W.bt = B.ht;
  // The backward reads C, B, W, X, B V and the column statistics from the
  // workspace but not O, so the forward skips its output stage (out = null).
  st = run(pl, q, k, v, nullptr, W, nullptr, s);
  if (st != LAPNYS_OK) return st;
  if (!ok(lapnys::launch_backward(pl, B, W, q, k, v, dout, dq, dk, dv, s), "backward launch")) return LAPNYS_ERR_HIP;
  return LAPNYS_OK;
}

struct Cached {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_cache_mu;
std::vector<Cached> g_cache;

// Workspace of lapnys_forward_noalloc: a static device array of
// LAPNYS_SCRATCH_MAX_BYTES, one copy per device (each device holds its copy
// from the library's first use on it until the process ends).  In host code
// `scratch` names a host-side stand-in, not a device address: its device
// address on each device comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is used.
static __device__ __align__(256) unsigned char scratch[LAPNYS_SCRATCH_MAX_BYTES];
std::mutex g_scratch_mu;
std::vector<void*> g_scratch;  // per device: the device address of `scratch`

int scratch_address(void** out) {
  int dev = 0;
  if (!ok(hipGetDevice(&dev), "hipGetDevice") || dev < 0) return LAPNYS_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch.size() <= dev) g_scratch.resize(dev + 1, nullptr);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (!ok(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress") || !ptr) return LAPNYS_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return LAPNYS_OK;
}

}  // namespace

extern "C" {

int lapnys_landmark_count(const lapnys_params* p) {
  const int st = validate(p);
  if (st != LAPNYS_OK) return st;
  return (p->grid_h / p->pool) * (p->grid_w / p->pool);
}

int lapnys_workspace_size(const lapnys_params* p, size_t* bytes) {
  if (!bytes) return LAPNYS_ERR_INVALID_ARG;
  Plan pl;
  const int st = make_plan(p, &pl);
  if (st != LAPNYS_OK) return st;
  *bytes = pl.total;
  return LAPNYS_OK;
}

int lapnys_forward_ws(const void* q, const void* k, const void* v, float* out, const lapnys_params* p, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  return forward_impl(q, k, v, out, p, ws, ws_bytes, nullptr, nullptr, stream);
}

int lapnys_forward_profiled(const void* q, const void* k, const void* v, float* out, const lapnys_params* p,
                            void* ws, size_t ws_bytes, hipEvent_t* stage_events, hipStream_t stream) {
  if (!stage_events) return LAPNYS_ERR_INVALID_ARG;
  return forward_impl(q, k, v, out, p, ws, ws_bytes, stage_events, nullptr, stream);
}

int lapnys_forward_debug(const void* q, const void* k, const void* v, float* out, const lapnys_params* p, void* ws,
                         size_t ws_bytes, const lapnys_debug* dbg, hipStream_t stream) {
  if (!dbg) return LAPNYS_ERR_INVALID_ARG;
  return forward_impl(q, k, v, out, p, ws, ws_bytes, nullptr, dbg, stream);
}

int lapnys_forward(const void* q, const void* k, const void* v, float* out, const lapnys_params* p,
                   hipStream_t stream) {
  Plan pl;
  int st = make_plan(p, &pl);
  if (st != LAPNYS_OK) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LAPNYS_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_cache_mu);
  if ((int)g_cache.size() <= dev) g_cache.resize(dev + 1);
  Cached& c = g_cache[dev];
  if (c.bytes < pl.total) {
    if (c.ptr) {
      if (hipDeviceSynchronize() != hipSuccess) return LAPNYS_ERR_HIP;
      (void)hipFree(c.ptr);
      c.ptr = nullptr;
      c.bytes = 0;
    }
    if (hipMalloc(&c.ptr, pl.total) != hipSuccess) {
      c.ptr = nullptr;
      return LAPNYS_ERR_HIP;
    }
    c.bytes = pl.total;
  }
  return forward_impl(q, k, v, out, p, c.ptr, c.bytes, nullptr, nullptr, stream);
}

int lapnys_forward_noalloc(const void* q, const void* k, const void* v, float* out, const lapnys_params* p,
                           hipStream_t stream) {
  Plan pl;
  int st = make_plan(p, &pl);
  if (st != LAPNYS_OK) return st;
  // Only the single-stream sequence: the other forms fork a library-owned
  // stream, created on first use.
  if (!pl.ns_in_launch) return LAPNYS_ERR_UNSUPPORTED;
  if (pl.total > LAPNYS_SCRATCH_MAX_BYTES) return LAPNYS_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != LAPNYS_OK) return st;
  return forward_impl(q, k, v, out, p, ws, LAPNYS_SCRATCH_MAX_BYTES, nullptr, nullptr, stream);
}

void lapnys_release(void) {
  std::lock_guard<std::mutex> lock(g_cache_mu);
  int cur = 0;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (size_t dev = 0; dev < g_cache.size(); ++dev) {
    if (!g_cache[dev].ptr) continue;
    // Release is best effort: a failed synchronise or free leaves nothing to
    // report to (the function returns no status), and the slot is dropped.
    if (hipSetDevice((int)dev) == hipSuccess) {
      (void)hipDeviceSynchronize();
      (void)hipFree(g_cache[dev].ptr);
    }
    g_cache[dev] = Cached();
  }
  if (have_cur) (void)hipSetDevice(cur);
}

int lapnys_backward_workspace_size(const lapnys_params* p, size_t* bytes) {
  if (!bytes) return LAPNYS_ERR_INVALID_ARG;
  Plan pl;
  size_t off[kBwdBuffers], total = 0;
  const int st = backward_plan(p, &pl, off, &total);
  if (st != LAPNYS_OK) return st;
  *bytes = total;
  return LAPNYS_OK;
}

int lapnys_backward_ws(const void* q, const void* k, const void* v, const float* dout, float* dq, float* dk,
                       float* dv, const lapnys_params* p, void* ws, size_t ws_bytes, hipStream_t stream) {
  return backward_impl(q, k, v, dout, dq, dk, dv, p, ws, ws_bytes, stream);
}

const char* lapnys_status_string(int status) {
  switch (status) {
    case LAPNYS_OK: return "ok";
    case LAPNYS_ERR_INVALID_ARG: return "invalid argument";
    case LAPNYS_ERR_SHAPE: return "shape mismatch: N != grid_h*grid_w or pool does not divide the grid";
    case LAPNYS_ERR_UNSUPPORTED: return "unsupported: d must be 32 or 64, m <= 256, dtype f32 or bf16";
    case LAPNYS_ERR_WORKSPACE: return "workspace null, too small or not 256-byte aligned";
    case LAPNYS_ERR_HIP: return "HIP runtime error";
    case LAPNYS_ERR_SCRATCH:
      return "the problem's workspace exceeds the static scratch of lapnys_forward_noalloc (LAPNYS_SCRATCH_MAX_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
