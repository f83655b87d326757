// Output stage: O = Z Y with Z = (C - mu) / sigma column-wise (the diagonal
// whitening of EN page section 2.B) and Y = X (B V), i.e. O = Z W^-1 (B V).
//
// One workgroup per 256-token tile, four wavefronts of 64 tokens each.
//
// Prologue (m <= 64): the workgroup forms its problem's Y = X (B V) itself on
// fp32 MFMA (a 64 x 64 x 64 product, zero padded) into LDS, so no separate
// launch is needed; for larger m, Y comes from a batched tile GEMM and is
// copied into LDS.
//
// Main loop: a wavefront's 64 x D output is (4 x D/16) blocks of fp32 MFMA
// 16x16x4; the reduction runs over landmarks four at a time.  Lane l feeds
// A[l%16][l/16] = Z[token][landmark], whitened from the stored C^T (16
// consecutive tokens of one landmark row per 16 lanes), and
// B[l/16][l%16] = Y[landmark][feature] from LDS.  The C loads of the next
// four landmarks are issued before the current MFMAs.  Each element of C is
// read once and each element of O written once.
#include "lapnys_internal.hpp"

namespace lapnys {

namespace {

constexpr int kXLD = 65;  // LDS row stride of X in the prologue

template <int D, bool FUSED_Y>
__global__ __launch_bounds__(256) void output_kernel(const float* __restrict__ ct, const float* __restrict__ x,
                                                     int mp, const float* __restrict__ bv, const float* __restrict__ y,
                                                     const float* __restrict__ mu, const float* __restrict__ rs,
                                                     float* __restrict__ out, int N, int m) {
  extern __shared__ float lds[];
  const int m4 = (m + 3) & ~3;
  float* yl = lds;             // [m4 or 64][D], rows >= m zero
  float* mul = yl + (FUSED_Y ? 64 : m4) * D;  // [m4]
  float* rsl = mul + m4;       // [m4]
  const int tile = blockIdx.x, p = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int e = tid; e < m4; e += 256) {
    mul[e] = (e < m) ? mu[p * m + e] : 0.f;
    rsl[e] = (e < m) ? rs[p * m + e] : 0.f;
  }

  if constexpr (FUSED_Y) {
    // Y = X (B V), 64 x D, on fp32 MFMA 32x32x2; X and B V zero padded to 64 rows.
    float* xl = rsl + m4;           // [64][kXLD]
    float* bvl = xl + 64 * kXLD;    // [64][D]
    const float* xp = x + (size_t)p * mp * mp;
    const float* bp = bv + (size_t)p * m * D;
    for (int e = tid; e < 64 * 64; e += 256) {
      const int a = e >> 6, b = e & 63;
      xl[a * kXLD + b] = (a < m && b < m) ? xp[(size_t)a * mp + b] : 0.f;
    }
    for (int e = tid; e < 64 * D; e += 256) bvl[e] = (e < m * D) ? bp[e] : 0.f;
    __syncthreads();
    const int li = lane & 31, lk = lane >> 5;
    const int bi = w >> 1, bj = w & 1;
    if (32 * bj < D) {
      f32x16 acc = {0.f};
      const int kext = (m + 1) & ~1;
      for (int k0 = 0; k0 < kext; k0 += 2) {
        const float a = xl[(32 * bi + li) * kXLD + k0 + lk];
        const float b = bvl[(k0 + lk) * D + 32 * bj + li];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) yl[(32 * bi + 8 * (r >> 2) + 4 * lk + (r & 3)) * D + 32 * bj + li] = acc[r];
    }
  } else {
    const float* yp = y + (size_t)p * m * D;
    for (int e = tid; e < m4 * D; e += 256) yl[e] = (e < m * D) ? yp[e] : 0.f;
  }
  __syncthreads();

  constexpr int DB = D / 16;
  const int li = lane & 15, lk = lane >> 4;
  const int tb = tile * 256 + 64 * w;
  const float* cp = ct + (size_t)p * m * N;
  f32x4 acc[4][DB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // raw C values of landmark row j for this lane's four tokens (0 outside)
  auto load_c = [&](int j, float (&c)[4]) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int tok = tb + 16 * a + li;
      c[a] = (j < m && tok < N) ? cp[(size_t)j * N + tok] : 0.f;
    }
  };
  float cur[4], nxt[4];
  load_c(lk, cur);
  for (int j0 = 0; j0 < m4; j0 += 4) {
    const int j = j0 + lk;
    load_c(j + 4, nxt);
    const float mj = mul[j], rj = rsl[j];
    float yb[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) yb[b] = yl[j * D + 16 * b + li];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float za = (j < m) ? (cur[a] - mj) * rj : 0.f;
#pragma unroll
      for (int b = 0; b < DB; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(za, yb[b], acc[a][b], 0, 0, 0);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) cur[a] = nxt[a];
  }

  float* op = out + (size_t)p * N * D;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = tb + 16 * a + 4 * lk + r;
      if (tok < N) {
#pragma unroll
        for (int b = 0; b < DB; ++b) op[(size_t)tok * D + 16 * b + li] = acc[a][b][r];
      }
    }
}

template <int D, bool FUSED_Y>
hipError_t launch_typed(const Plan& pl, const Work& wk, float* out, hipStream_t s) {
  const int m4 = (pl.m + 3) & ~3;
  const size_t floats = FUSED_Y ? (size_t)64 * D + 2 * m4 + 64 * kXLD + 64 * D : (size_t)m4 * D + 2 * m4;
  const size_t shmem = floats * sizeof(float);
  auto kern = output_kernel<D, FUSED_Y>;
  if (shmem > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((pl.N + 255) / 256, pl.P), dim3(256), shmem, s, wk.ct, wk.x_final, pl.mp, wk.bv,
                     wk.y, wk.mu, wk.rs, out, pl.N, pl.m);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_output(const Plan& pl, const Work& wk, float* out, hipStream_t s) {
  if (pl.fused_ns) {
    if (pl.d == 64) return launch_typed<64, true>(pl, wk, out, s);
    return launch_typed<32, true>(pl, wk, out, s);
  }
  if (pl.d == 64) return launch_typed<64, false>(pl, wk, out, s);
  return launch_typed<32, false>(pl, wk, out, s);
}

}  // namespace lapnys
