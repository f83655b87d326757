// Output stage: O = Z Y with Z = (C - mu) / sigma column-wise (the diagonal
// whitening of EN page section 2.B) and Y = X (B V), i.e. O = Z W^-1 (B V).
//
// One workgroup per 256-token tile, four wavefronts of 64 tokens each.  A
// wavefront's 64 x D output is (4 x D/16) blocks of fp32 MFMA 16x16x4; the
// reduction runs over landmarks four at a time.  Lane l feeds
// A[l%16][l/16] = Z[token][landmark], whitened on the fly from the stored C^T
// (16 consecutive tokens of one landmark row per 16 lanes), and
// B[l/16][l%16] = Y[landmark][feature] from LDS.  Each element of C is read
// once and each element of O written once.
#include "lapnys_internal.hpp"

namespace lapnys {

namespace {

template <int D>
__global__ __launch_bounds__(256) void output_kernel(const float* __restrict__ ct, const float* __restrict__ y,
                                                     const float* __restrict__ mu, const float* __restrict__ rs,
                                                     float* __restrict__ out, int N, int m) {
  extern __shared__ float lds[];
  const int m4 = (m + 3) & ~3;
  float* yl = lds;               // [m4][D], rows >= m zero
  float* mul = yl + m4 * D;      // [m4]
  float* rsl = mul + m4;         // [m4]
  const int tile = blockIdx.x, p = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* yp = y + (size_t)p * m * D;
  for (int e = tid; e < m4 * D; e += 256) yl[e] = (e < m * D) ? yp[e] : 0.f;
  for (int e = tid; e < m4; e += 256) {
    mul[e] = (e < m) ? mu[p * m + e] : 0.f;
    rsl[e] = (e < m) ? rs[p * m + e] : 0.f;
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

  for (int j0 = 0; j0 < m4; j0 += 4) {
    const int j = j0 + lk;
    const float mj = mul[j], rj = rsl[j];
    float za[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int tok = tb + 16 * a + li;
      za[a] = (j < m && tok < N) ? (cp[(size_t)j * N + tok] - mj) * rj : 0.f;
    }
    float yb[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) yb[b] = yl[j * D + 16 * b + li];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < DB; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(za[a], yb[b], acc[a][b], 0, 0, 0);
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

template <int D>
hipError_t launch_typed(const Plan& pl, const float* ct, const float* y, const float* mu, const float* rs,
                        float* out, hipStream_t s) {
  const int m4 = (pl.m + 3) & ~3;
  const size_t shmem = (size_t)(m4 * D + 2 * m4) * sizeof(float);
  auto kern = output_kernel<D>;
  if (shmem > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((pl.N + 255) / 256, pl.P), dim3(256), shmem, s, ct, y, mu, rs, out, pl.N, pl.m);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_output(const Plan& pl, const float* ct, const float* y, const float* mu, const float* rs,
                         float* out, hipStream_t s) {
  if (pl.d == 64) return launch_typed<64>(pl, ct, y, mu, rs, out, s);
  return launch_typed<32>(pl, ct, y, mu, rs, out, s);
}

}  // namespace lapnys
