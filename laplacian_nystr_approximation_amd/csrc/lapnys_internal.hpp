// Internal declarations shared by the liblapnys translation units: device
// helpers, the per-call plan (tiling and workspace layout) and the kernel
// launchers.  Nothing here is part of the public C ABI (include/lapnys.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lapnys {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Splits two floats into bf16 high parts (round to nearest even) and bf16
// low parts (the rounded remainders), each pair packed in one dword: with
// both operands of a product split this way, hi*hi + hi*lo + lo*hi on bf16
// MFMA keeps all but about 2^-16 of the product.
__device__ __forceinline__ void split2(float z0, float z1, uint32_t& hi, uint32_t& lo) {
  const bf16x2 h = __builtin_convertvector((f32x2){z0, z1}, bf16x2);
  const f32x2 hf = __builtin_convertvector(h, f32x2);
  const bf16x2 l = __builtin_convertvector((f32x2){z0 - hf.x, z1 - hf.y}, bf16x2);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

// Input element widening: float32 passes through, bfloat16 (stored as its
// 16-bit pattern) widens exactly by placing it in the high half of a float32.
__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Landmark block handled by one workgroup of the fused kernel-matrix stage.
constexpr int kLandmarkBlock = 64;
// Largest landmark count the fused single-workgroup Newton-Schulz handles.
constexpr int kFusedNsMaxM = 64;
// Largest supported landmark count.
constexpr int kMaxM = 256;
// Devices per process with cached per-device launch data.
constexpr int kMaxDevices = 64;

// Per-call plan: sizes, tiling and the workspace layout (byte offsets, each
// 256-byte aligned).  Computed on the host from the validated parameters.
struct Plan {
  int P;            // B * H problems
  int N, d, m;      // tokens, head dimension, landmarks
  int ldc;          // row stride of the stored C^T (N rounded up to 4)
  int gw;           // pooled grid width (grid_w / pool)
  int grid_w, pool;
  int dtype;        // lapnys_dtype
  bool whiten;
  int ns_iters;
  bool refine;      // one float64-residual correction after the steps
  bool gaussian;    // Gaussian kernel exp(-||x - y||_2^2 / lambda) instead of the Laplacian
  bool cg;          // conjugate gradient for Y = W^-1 (B V) instead of Newton-Schulz
  float scale;      // -log2(e) / lambda, so k = exp2(scale * L1)
  float eps;
  int mp;           // padded Newton-Schulz size (64, or m rounded up to 64)
  bool fused_ns;    // m <= kFusedNsMaxM: one workgroup per problem (64 x 64 padded X)
  bool ns_in_launch;  // ... inside the kernel-matrix launch (the Laplacian default)
  int tt;           // tokens per tile of the kernel-matrix stage (256 or 128)
  int ntiles;       // token tiles per problem
  int lb;           // landmarks per block of the kernel-matrix stage
  int jblocks;      // landmark blocks (ceil(m / lb))
  int tpg;          // tiles per workgroup (tile group)
  int groups;       // tile groups per problem
  // workspace offsets in bytes
  size_t off_kt, off_w, off_x, off_x2, off_pm, off_ct, off_stats, off_bvpart, off_bv,
      off_mu, off_sigma, off_rs, off_y, off_yt, total;
};

// Device pointers into one call's workspace.
struct Work {
  float *kt, *w, *x, *x2, *pm, *ct, *stats, *bvpart, *bv, *mu, *sigma, *rs, *y;
  __bf16* yt;          // m <= 64: Y^T as bf16 high and low parts, [P][2][d][64] (yt_index layout)
  float* x_final;      // the Newton-Schulz result (x or x2), set by launch_ns
  float* bt = nullptr; // if set (Laplacian form only): the kernel-matrix stage also stores B as [P][m][N]
  // If set (debug form): device wall-clock stamps.  nsclk [P][3]: start, first
  // step and end of each problem's in-launch solver workgroup; kclk [2]: the
  // earliest start and latest end over the Laplacian kernel-matrix workgroups
  // (kclk[0] must hold the largest value and kclk[1] zero on entry).
  unsigned long long* nsclk = nullptr;
  unsigned long long* kclk = nullptr;
};

// Backward-pass buffers, after the forward's workspace (float32; mp = m
// rounded up to 64):
//   part [P][tiles][m][d], spart [P][tiles][d]   partial C^T dO and 1^T dO
//   y, dbv [P][m][d]; ab [P][2][m]; dkt [P][m][d]
//   dw [P][mp][mp]   R X^T with R = X^T dX, i.e. -dW
//   gt, ht [P][m][N]                              G^T and H^T
//   dy [P][mp][d] (zero rows past m), s [P][d]
//   m > 64 only: bvt [P][d][mp], xt, dx, r [P][mp][mp]
struct BwdWork {
  float *part, *spart, *y, *dbv, *ab, *dw, *gt, *ht, *dkt;
  float *dy, *bvt, *s, *xt, *dx, *r;
};

// Position of Y^T element (feature f, landmark l) in a [D][rl] bf16 array (rl
// a multiple of 64), the layout the output stage reads its B operands from.
// The 8-landmark chunks of a row are XOR-swizzled by t = f / (D / 16), the
// index of the lane that reads feature f, so the 16 lanes that read one
// chunk column for 16 different features spread over distinct banks.
__device__ __forceinline__ int yt_index(int f, int l, int t, int rl) {
  const int c = l >> 3;
  return f * rl + 8 * ((c & ~7) | ((c ^ t) & 7)) + (l & 7);
}

// Optional timing events of one stage: the start time of its first kernel and
// the end time of its last kernel, taken from the kernels' own dispatch
// timestamps (hipExtLaunchKernel), so no event command sits between kernels.
// Null members are not recorded.
struct Span {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Kernel launchers (each returns the hipError_t of its launches).
hipError_t launch_pool(const Plan& pl, const void* k, const Work& w, hipStream_t s, Span t = {});
// The solver as launches of its own: 64 < m <= 256, and the Gaussian form at
// every m (sets w.x_final).
hipError_t launch_ns(const Plan& pl, Work& w, hipStream_t s, Span t = {});
// The correction X <- X + X (I - W X) of w.x_final (residual in float64),
// into the other iterate buffer; updates w.x_final.  Any m; the stop event,
// if given, is recorded by its last kernel.
hipError_t launch_refine(const Plan& pl, Work& w, hipStream_t s, hipEvent_t stop = nullptr);
// The kernel-matrix stage; for m <= 64 the same launch also runs the
// Newton-Schulz solver (and sets w.x_final).
hipError_t launch_l1exp(const Plan& pl, const void* q, const void* k, const void* v, Work& w,
                        hipStream_t s, Span t = {});
// The Gaussian-kernel form of the kernel-matrix stage (pl.gaussian; the
// solver then runs as launch_ns at every m).
hipError_t launch_gauss(const Plan& pl, const void* q, const void* k, const void* v, Work& w, hipStream_t s,
                        Span t = {});
// Reductions after the kernel-matrix stage: B V, the whitening statistics,
// and for m <= 64 also Y = X (B V) into w.yt.
hipError_t launch_reduce(const Plan& pl, const Work& w, hipStream_t s, Span t = {});
hipError_t launch_y(const Plan& pl, const Work& w, hipStream_t s, Span t = {});  // m > kFusedNsMaxM only
// pl.cg: Y = W^-1 (B V) by pl.ns_iters CG steps per column, into w.y.
hipError_t launch_cg(const Plan& pl, const Work& w, hipStream_t s, hipEvent_t stop = nullptr);
hipError_t launch_output(const Plan& pl, const Work& w, float* out, hipStream_t s, Span t = {});
// The gradients of sum(dout * O) into dq, dk, dv (float32 [B,H,N,d]) after a
// forward call on the same workspace (Laplacian kernel, Newton-Schulz).
hipError_t launch_backward(const Plan& pl, const BwdWork& b, const Work& w, const void* q, const void* k,
                           const void* v, const float* dout, float* dq, float* dk, float* dv, hipStream_t s);
// Batched C = A B on the tile GEMM (ns.hip): A rows [0, 64 ceil(crows / 64))
// and columns [0, kext) in range, B read where in [0, brows) x [0, bcols).
hipError_t launch_gemm(const float* A, int lda, long long sa, const float* B, int ldb, long long sb, int brows,
                       int bcols, float* C, int ldc, long long sc, int crows, int ccols, int kext, int P,
                       hipStream_t s);
hipError_t launch_extract_square(const float* src, int src_ld, float* dst, int n, int P, hipStream_t s);

}  // namespace lapnys
