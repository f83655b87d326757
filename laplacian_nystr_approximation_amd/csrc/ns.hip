// Landmark Gram matrix and its Newton-Schulz inverse (EN page, section 2.C.2;
// DE section 2; ZH section 2.2; KO section 2.3; JA section 2.3).
//
//   W  = k(K~, K~) + eps I,   k(x, y) = exp(-||x - y||_1 / lambda)
//   X0 = W^T / (||W||_1 ||W||_inf)
//   X <- X (2I - W X), a fixed number of times, matrix products only.
//
// W is built so that it is bit-symmetric: entry (a, b) and entry (b, a) sum
// the same |differences| in the same feature order, and the diagonal is
// exp(0) + eps = 1 + eps exactly as float32 arithmetic gives it.
//
// Two schedules:
//  * m <= 64: one workgroup per problem keeps W and the iterates in LDS and
//    runs inside the kernel-matrix stage's launch (ns_small.hpp, l1exp.hip).
//  * 64 < m <= 256 (this file): the products are too large for one LDS; W and
//    the iterates live in the workspace (L2-resident) and each product is one
//    batched launch of 64 x 64 output tiles, two launches per step.  The same
//    tile kernel also forms Y = X (B V) for these sizes.
#include "lapnys_internal.hpp"

namespace lapnys {

namespace {

// ---- 64 < m <= 256 -------------------------------------------------------

// W rows [16*blockIdx.x, +16) of problem blockIdx.y; thread b owns column b.
template <int D>
__global__ __launch_bounds__(256) void wbuild_big_kernel(const float* __restrict__ kt, float* __restrict__ w, int m,
                                                         int mp, float scale, float eps) {
  __shared__ float kl[16 * D];
  const int p = blockIdx.y, a0 = blockIdx.x * 16, b = threadIdx.x;
  const float* ktp = kt + (size_t)p * m * D;
  for (int e = threadIdx.x; e < 16 * D; e += 256) {
    const int a = a0 + e / D;
    kl[e] = (a < m) ? ktp[(size_t)a * D + e % D] : 0.f;
  }
  float xb[D];
#pragma unroll
  for (int t = 0; t < D; ++t) xb[t] = (b < m) ? ktp[(size_t)b * D + t] : 0.f;
  __syncthreads();
  if (b >= mp) return;
  for (int r = 0; r < 16; ++r) {
    const int a = a0 + r;
    float val = 0.f;
    if (a < m && b < m) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int t = 0; t < D; t += 2) {
        s0 += fabsf(kl[r * D + t] - xb[t]);
        s1 += fabsf(kl[r * D + t + 1] - xb[t + 1]);
      }
      val = exp2f((s0 + s1) * scale);
      if (a == b) val += eps;
    }
    w[((size_t)p * mp + a) * mp + b] = val;
  }
}

// alpha and X0 = W^T / alpha for problem blockIdx.x.
__global__ __launch_bounds__(256) void alpha_x0_kernel(const float* __restrict__ w, float* __restrict__ x, int mp) {
  __shared__ float red[512];
  __shared__ float alpha_s;
  const int p = blockIdx.x, tid = threadIdx.x;
  const float* wp = w + (size_t)p * mp * mp;
  float rs = 0.f, cs = 0.f;
  if (tid < mp) {
    for (int b = 0; b < mp; ++b) rs += fabsf(wp[(size_t)tid * mp + b]);
    for (int a = 0; a < mp; ++a) cs += fabsf(wp[(size_t)a * mp + tid]);
  }
  red[tid] = rs;
  red[256 + tid] = cs;
  __syncthreads();
  if (tid == 0) {
    float rm = 0.f, cm = 0.f;
    for (int i = 0; i < 256; ++i) {
      rm = fmaxf(rm, red[i]);
      cm = fmaxf(cm, red[256 + i]);
    }
    alpha_s = cm * rm;
  }
  __syncthreads();
  const float alpha = alpha_s;
  float* xp = x + (size_t)p * mp * mp;
  for (int e = tid; e < mp * mp; e += 256) {
    const int a = e / mp, b = e % mp;
    xp[e] = wp[(size_t)b * mp + a] / alpha;
  }
}

// One 64 x 64 output tile (blockIdx.x, blockIdx.y) of problem blockIdx.z:
//   C = A B (mode 0)  or  C = A (2I - B) (mode 1),
// reduction over [0, kext) (a multiple of 32) staged through LDS 32 at a time.
// B entries outside [0, brows) x [0, bcols) read as zero (before the 2I
// transform); C is stored for rows < crows and columns < ccols.  Each of the
// four wavefronts owns a 32 x 32 block and issues fp32 MFMA 32x32x2.
__global__ __launch_bounds__(256) void gemm64_kernel(const float* __restrict__ A, int lda, long long sa,
                                                     const float* __restrict__ B, int ldb, long long sb, int brows,
                                                     int bcols, float* __restrict__ C, int ldc, long long sc,
                                                     int crows, int ccols, int kext, int mode) {
  __shared__ float as[64 * 33];
  __shared__ float bs[32 * 64];
  const int p = blockIdx.z, r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wr = w >> 1, wc = w & 1, li = lane & 31, lk = lane >> 5;
  const float* Ap = A + p * sa;
  const float* Bp = B + p * sb;
  f32x16 acc = {0.f};
  for (int kc = 0; kc < kext; kc += 32) {
    for (int e = tid; e < 64 * 32; e += 256) {
      const int r = e >> 5, c = e & 31;
      as[r * 33 + c] = Ap[(size_t)(r0 + r) * lda + kc + c];
    }
    for (int e = tid; e < 32 * 64; e += 256) {
      const int r = e >> 6, c = e & 63;
      const int gr = kc + r, gc = c0 + c;
      float bv = (gr < brows && gc < bcols) ? Bp[(size_t)gr * ldb + gc] : 0.f;
      if (mode) bv = (gr == gc ? 2.f : 0.f) - bv;
      bs[r * 64 + c] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int k0 = 0; k0 < 32; k0 += 2) {
      const float a = as[(32 * wr + li) * 33 + k0 + lk];
      const float b = bs[(k0 + lk) * 64 + 32 * wc + li];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  float* Cp = C + p * sc;
  const int cc = c0 + 32 * wc + li;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rr = r0 + 32 * wr + 8 * (r >> 2) + 4 * lk + (r & 3);
    if (rr < crows && cc < ccols) Cp[(size_t)rr * ldc + cc] = acc[r];
  }
}

__global__ __launch_bounds__(256) void extract_square_kernel(const float* __restrict__ src, int src_ld,
                                                             float* __restrict__ dst, int n, long long total) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const long long p = e / ((long long)n * n);
  const int rem = (int)(e % ((long long)n * n));
  const int a = rem / n, b = rem % n;
  dst[e] = src[(p * src_ld + a) * src_ld + b];
}

}  // namespace

hipError_t launch_ns(const Plan& pl, Work& wk, hipStream_t s, Span t) {
  // m <= 64 runs inside the kernel-matrix launch (launch_l1exp).
  if (pl.fused_ns) return hipErrorInvalidValue;
  const int mp = pl.mp;
  if (pl.d == 64)
    hipExtLaunchKernelGGL(wbuild_big_kernel<64>, dim3(mp / 16, pl.P), dim3(256), 0, s, t.start, nullptr, 0, wk.kt,
                          wk.w, pl.m, mp, pl.scale, pl.eps);
  else
    hipExtLaunchKernelGGL(wbuild_big_kernel<32>, dim3(mp / 16, pl.P), dim3(256), 0, s, t.start, nullptr, 0, wk.kt,
                          wk.w, pl.m, mp, pl.scale, pl.eps);
  hipExtLaunchKernelGGL(alpha_x0_kernel, dim3(pl.P), dim3(256), 0, s, nullptr, pl.ns_iters == 0 ? t.stop : nullptr, 0,
                        wk.w, wk.x, mp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int kext = (pl.m + 31) & ~31;
  const long long sq = (long long)mp * mp;
  const dim3 grid(mp / 64, mp / 64, pl.P);
  float* xc = wk.x;
  float* xn = wk.x2;
  for (int it = 0; it < pl.ns_iters; ++it) {
    hipLaunchKernelGGL(gemm64_kernel, grid, dim3(256), 0, s, wk.w, mp, sq, xc, mp, sq, mp, mp, wk.pm, mp, sq, mp, mp,
                       kext, 0);
    hipExtLaunchKernelGGL(gemm64_kernel, grid, dim3(256), 0, s, nullptr, it + 1 == pl.ns_iters ? t.stop : nullptr, 0,
                          xc, mp, sq, wk.pm, mp, sq, mp, mp, xn, mp, sq, mp, mp, kext, 1);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    float* t = xc;
    xc = xn;
    xn = t;
  }
  wk.x_final = xc;
  return hipSuccess;
}

hipError_t launch_y(const Plan& pl, const Work& wk, hipStream_t s, Span t) {
  const int kext = (pl.m + 31) & ~31;
  const long long md = (long long)pl.m * pl.d;
  hipExtLaunchKernelGGL(gemm64_kernel, dim3((pl.m + 63) / 64, (pl.d + 63) / 64, pl.P), dim3(256), 0, s, t.start,
                        t.stop, 0, wk.x_final,
                     pl.mp, (long long)pl.mp * pl.mp, wk.bv, pl.d, md, pl.m, pl.d, wk.y, pl.d, md, pl.m, pl.d, kext, 0);
  return hipGetLastError();
}

hipError_t launch_extract_square(const float* src, int src_ld, float* dst, int n, int P, hipStream_t s) {
  const long long total = (long long)P * n * n;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(extract_square_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, src, src_ld,
                     dst, n, total);
  return hipGetLastError();
}

}  // namespace lapnys
