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
//  * m <= 64: one workgroup per problem keeps W, X and 2I - W X in LDS
//    (64 x 64, zero padded) and runs every step in one launch on fp32 MFMA;
//    padding rows and columns stay exactly zero (see ns_fused_kernel).
//  * 64 < m <= 256: the products are too large for one LDS; W and the iterates
//    live in the workspace (L2-resident) and each product is one batched launch
//    of 64 x 64 output tiles, two launches per step.  The same tile kernel also
//    forms Y = X (B V) for these sizes.
#include "lapnys_internal.hpp"

namespace lapnys {

namespace {

constexpr int kMP = 64;  // padded size of the in-LDS schedule
constexpr int kLD = 68;  // LDS row stride (floats): conflict-free column reads

// In-LDS schedule for m <= 64: one workgroup of four wavefronts per problem,
// 52 KB of LDS (so it can share a CU with the kernel-matrix stage).
//
// Each step is evaluated as X_next = 2X - X (W X), which equals X (2I - W X).
// Symmetry: W is bit-symmetric and X0 = W^T / alpha = W / alpha; for a
// symmetric X the product X W X is symmetric whatever rounding X carries, so
// Q = W X is formed in full (wavefront w: the four 16 x 16 blocks of block row
// w) and stored transposed, while S = X Q is formed only on its 10 upper
// 16 x 16 blocks (spread over the wavefronts as 3, 3, 2, 2) and stored with
// its mirror image.  X thus stays exactly symmetric in one row-major copy,
// and a column of X is read as a row.  (Mirroring a product that is not
// symmetric in exact arithmetic, such as W X, would not be a faithful step:
// the iteration then drifts away once it has converged.)
//
// The reduction runs over k in [0, 4 KS), KS = ceil(m / 4), on fp32 MFMA
// 16x16x4.  Padding rows and columns of W and X are exact zeros and stay so.
__device__ __constant__ int8_t kBlkI[4][3] = {{0, 0, 0}, {0, 1, 1}, {1, 2, -1}, {2, 3, -1}};
__device__ __constant__ int8_t kBlkJ[4][3] = {{0, 1, 2}, {3, 1, 2}, {3, 2, -1}, {3, 3, -1}};

template <int D, int KS>
__global__ __launch_bounds__(256) void ns_fused_kernel(const float* __restrict__ kt, float* __restrict__ wout,
                                                       float* __restrict__ xout, int m, float scale, float eps,
                                                       int iters) {
  constexpr int KLD = D + 4;  // landmark staging stride: 16-byte rows for broadcast reads
  __shared__ float4 xs4[2][kMP * kLD / 4];  // X (ping-pong), symmetric; [1] also stages the landmarks
  __shared__ float4 qs4[kMP * kLD / 4];     // (W X)^T; W during set-up
  __shared__ float red[128];
  __shared__ float alpha_s;
  static_assert(kMP * KLD <= kMP * kLD, "landmark staging must fit in an X buffer");
  float* wl = reinterpret_cast<float*>(qs4);
  float* ql = wl;
  float* kl = reinterpret_cast<float*>(xs4[1]);

  const int p = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* ktp = kt + (size_t)p * m * D;
  for (int e = tid; e < m * D; e += 256) kl[(e / D) * KLD + (e % D)] = ktp[e];
  __syncthreads();

  // W = k(K~, K~) + eps I, zero padded.  Lane b holds landmark b in
  // registers; wavefront w forms rows [16 w, 16 w + 16) four at a time with
  // the row landmark broadcast from LDS.  Entry (a, b) sums |K~_a - K~_b| over
  // even and odd features in increasing order, the same sums as entry (b, a),
  // so W is bit-symmetric.
  {
    const int b = lane;
    float xb[D];
#pragma unroll
    for (int t = 0; t < D; ++t) xb[t] = kl[min(b, m - 1) * KLD + t];
    for (int a0 = 16 * w; a0 < 16 * w + 16; a0 += 4) {
      if (a0 < m) {
        float s0[4] = {0.f, 0.f, 0.f, 0.f}, s1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < D; t += 2) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int a = min(a0 + u, m - 1);
            s0[u] += fabsf(kl[a * KLD + t] - xb[t]);
            s1[u] += fabsf(kl[a * KLD + t + 1] - xb[t + 1]);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int a = a0 + u;
          float val = 0.f;
          if (a < m && b < m) {
            val = exp2f((s0[u] + s1[u]) * scale);
            if (a == b) val += eps;
          }
          wl[a * kLD + b] = val;
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) wl[(a0 + u) * kLD + b] = 0.f;
      }
    }
  }
  __syncthreads();

  // alpha = ||W||_1 * ||W||_inf (largest absolute column sum times largest row
  // sum); W goes out to the workspace, the second X buffer is cleared.
  float* wp = wout + (size_t)p * kMP * kMP;
  for (int e = tid; e < kMP * kMP; e += 256) {
    wp[e] = wl[(e >> 6) * kLD + (e & 63)];
    kl[(e >> 6) * kLD + (e & 63)] = 0.f;
  }
  if (tid < 2 * kMP) {
    const int i = tid & 63;
    const bool rows = tid < kMP;
    float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b0 = 0; b0 < kMP; b0 += 8)
#pragma unroll
      for (int u = 0; u < 8; ++u) acc8[u] += fabsf(rows ? wl[i * kLD + b0 + u] : wl[(b0 + u) * kLD + i]);
    red[tid] = ((acc8[0] + acc8[1]) + (acc8[2] + acc8[3])) + ((acc8[4] + acc8[5]) + (acc8[6] + acc8[7]));
  }
  __syncthreads();
  if (tid < 64) {
    float rm = red[tid], cm = red[kMP + tid];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      rm = fmaxf(rm, __shfl_xor(rm, off, 64));
      cm = fmaxf(cm, __shfl_xor(cm, off, 64));
    }
    if (tid == 0) alpha_s = cm * rm;
  }
  __syncthreads();

  // W's A operands for every step of Q = W X, block row w:
  // A[li][lk] of step s = W[16 w + li][4 s + lk].  Then this wavefront's
  // upper blocks of S = X Q.
  // KS = ceil(m / 4) steps per product (a template parameter, so the step
  // loops unroll without branches).  Wavefronts with two upper blocks run a
  // third, unstored copy of their last block: every wavefront issues the
  // same MFMA sequence and none branches inside it.
  const int li = lane & 15, lk = lane >> 4;
  float wreg[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) wreg[st] = wl[(16 * w + li) * kLD + 4 * st + lk];
  int bI[3], bJ[3];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    bI[b] = kBlkI[w][b];
    bJ[b] = kBlkJ[w][b];
  }
  const int nb = bI[2] < 0 ? 2 : 3;
  if (nb == 2) {
    bI[2] = bI[1];
    bJ[2] = bJ[1];
  }
  // X0 = W^T / alpha = W / alpha (W is symmetric).
  {
    const float alpha = alpha_s;
    float* x0 = reinterpret_cast<float*>(xs4[0]);
    for (int e = tid; e < kMP * kMP; e += 256) {
      const int a = e >> 6, b = e & 63;
      x0[a * kLD + b] = wl[b * kLD + a] / alpha;
    }
  }
  __syncthreads();

  int cur = 0;
  for (int it = 0; it < iters; ++it) {
    const float* xc = reinterpret_cast<const float*>(xs4[cur]);
    // Q = W X, block row w, stored transposed: ql[j][i] = Q[i][j].
    {
      f32x4 acc[4];
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) acc[bj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
          const float xb = xc[(16 * bj + li) * kLD + 4 * st + lk];  // X[4 st + lk][16 bj + li]
          acc[bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(wreg[st], xb, acc[bj], 0, 0, 0);
        }
      }
      // acc[bj][r] = Q[16 w + 4 lk + r][16 bj + li]: four consecutive entries of
      // row 16 bj + li of Q^T.
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
        *reinterpret_cast<float4*>(&ql[(16 * bj + li) * kLD + 16 * w + 4 * lk]) =
            make_float4(acc[bj][0], acc[bj][1], acc[bj][2], acc[bj][3]);
    }
    __syncthreads();
    // S = X Q on the upper blocks; X_next = 2 X - S stored with its mirror.
    {
      float xij[3][4];  // X entries of this lane's outputs, read ahead of the products
#pragma unroll
      for (int b = 0; b < 3; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) xij[b][r] = xc[(16 * bI[b] + 4 * lk + r) * kLD + 16 * bJ[b] + li];
      f32x4 acc[3];
#pragma unroll
      for (int b = 0; b < 3; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
#pragma unroll
        for (int b = 0; b < 3; ++b) {
          const float xa = xc[(16 * bI[b] + li) * kLD + 4 * st + lk];  // X[16 bi + li][4 st + lk]
          const float qb = ql[(16 * bJ[b] + li) * kLD + 4 * st + lk];  // Q[4 st + lk][16 bj + li]
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa, qb, acc[b], 0, 0, 0);
        }
      }
      float* xn = reinterpret_cast<float*>(xs4[cur ^ 1]);
#pragma unroll
      for (int b = 0; b < 3; ++b) {
        if (b < nb) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = 2.f * xij[b][r] - acc[b][r];
          const int i0 = 16 * bI[b] + 4 * lk, j = 16 * bJ[b] + li;
          if (bI[b] != bJ[b]) {
            // off the diagonal every entry is upper: the mirror image is four
            // consecutive entries of row j
#pragma unroll
            for (int r = 0; r < 4; ++r) xn[(i0 + r) * kLD + j] = v[r];
            *reinterpret_cast<float4*>(&xn[j * kLD + i0]) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
            // diagonal block: only the upper-triangle entries, with their mirrors
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (i0 + r <= j) {
                xn[(i0 + r) * kLD + j] = v[r];
                xn[j * kLD + i0 + r] = v[r];
              }
            }
          }
        }
      }
    }
    __syncthreads();
    cur ^= 1;
  }

  float* xp = xout + (size_t)p * kMP * kMP;
  const float* xf = reinterpret_cast<const float*>(xs4[cur]);
  for (int e = tid; e < kMP * kMP; e += 256) xp[e] = xf[(e >> 6) * kLD + (e & 63)];
}

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

template <int D, int KS>
void launch_fused_ks(const Plan& pl, Work& wk, hipStream_t s, Span t) {
  hipExtLaunchKernelGGL(ns_fused_kernel<D, KS>, dim3(pl.P), dim3(256), 0, s, t.start, t.stop, 0, wk.kt, wk.w, wk.x,
                        pl.m, pl.scale, pl.eps, pl.ns_iters);
}

template <int D, int KS = 1>
void launch_fused(const Plan& pl, Work& wk, hipStream_t s, Span t) {
  if constexpr (KS < 16) {
    if ((pl.m + 3) / 4 > KS) {
      launch_fused<D, KS + 1>(pl, wk, s, t);
      return;
    }
  }
  launch_fused_ks<D, KS>(pl, wk, s, t);
}

}  // namespace

hipError_t launch_ns(const Plan& pl, Work& wk, hipStream_t s, Span t) {
  if (pl.fused_ns) {
    if (pl.d == 64)
      launch_fused<64>(pl, wk, s, t);
    else
      launch_fused<32>(pl, wk, s, t);
    wk.x_final = wk.x;
    return hipGetLastError();
  }
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
