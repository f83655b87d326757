// Reductions between the kernel-matrix stage and the output stage.
//
//  * Whitening statistics (EN page, section 2.B; KO section 2.2): for every
//    landmark column j of C, the mean and the population standard deviation
//    over the N tokens of the problem.  The per-tile (sum, squared-deviation
//    sum) pairs are merged in float64 in tile order with the exact
//    decomposition M2 = sum_t [M2_t + n_t (mean_t - mean)^2], so the result
//    is the two-pass statistic, not a one-pass E[c^2] - E[c]^2.
//  * B V = sum over tile groups of the partial products, in group order.
//  * Y = X (B V): the Newton-Schulz inverse applied to B V (m x d).
// Every reduction runs in a fixed order, so results repeat bit for bit.
#include <math.h>

#include "lapnys_internal.hpp"

namespace lapnys {

namespace {

// One lane per (problem, landmark, feature): B V sum; feature-0 lanes also
// produce the landmark's mean, sigma and 1/sigma.
__global__ __launch_bounds__(256) void reduce_kernel(const float2* __restrict__ stats,
                                                     const float* __restrict__ bvpart, float* __restrict__ bv,
                                                     float* __restrict__ mu, float* __restrict__ sigma,
                                                     float* __restrict__ rs, int N, int m, int D, int ntiles,
                                                     int tt, int groups, int whiten) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int p = blockIdx.y;
  if (e >= m * D) return;
  const int j = e / D, t = e % D;
  const float* src = bvpart + (size_t)p * groups * m * D + (size_t)j * D + t;
  float acc = 0.f;
  for (int g = 0; g < groups; ++g) acc += src[(size_t)g * m * D];
  bv[((size_t)p * m + j) * D + t] = acc;
  if (t != 0) return;
  if (!whiten) {
    mu[p * m + j] = 0.f;
    sigma[p * m + j] = 1.f;
    rs[p * m + j] = 1.f;
    return;
  }
  const float2* st = stats + (size_t)p * ntiles * m + j;
  double total = 0.0;
  for (int i = 0; i < ntiles; ++i) total += (double)st[(size_t)i * m].x;
  const double mean = total / (double)N;
  double m2 = 0.0;
  for (int i = 0; i < ntiles; ++i) {
    const float2 sv = st[(size_t)i * m];
    const int n = min(tt, N - i * tt);
    const double dm = (double)sv.x / (double)n - mean;
    m2 += (double)sv.y + (double)n * dm * dm;
  }
  const double sd = sqrt(m2 / (double)N);
  mu[p * m + j] = (float)mean;
  sigma[p * m + j] = (float)sd;
  rs[p * m + j] = sd > 0.0 ? (float)(1.0 / sd) : 0.f;
}

// Y[p][a][t] = sum_{b < m} X[p][a][b] * BV[p][b][t], X stored with row stride mp.
__global__ __launch_bounds__(256) void y_kernel(const float* __restrict__ x, const float* __restrict__ bv,
                                                float* __restrict__ y, int m, int mp, int D) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int p = blockIdx.y;
  if (e >= m * D) return;
  const int a = e / D, t = e % D;
  const float* xr = x + ((size_t)p * mp + a) * mp;
  const float* bc = bv + (size_t)p * m * D + t;
  float acc = 0.f;
  for (int b = 0; b < m; ++b) acc = fmaf(xr[b], bc[(size_t)b * D], acc);
  y[((size_t)p * m + a) * D + t] = acc;
}

}  // namespace

hipError_t launch_finalize(const Plan& pl, const float* stats, const float* bvpart, const float* x, float* bv,
                           float* mu, float* sigma, float* rs, float* y, hipStream_t s) {
  const int n = pl.m * pl.d;
  const dim3 grid((n + 255) / 256, pl.P);
  hipLaunchKernelGGL(reduce_kernel, grid, dim3(256), 0, s, reinterpret_cast<const float2*>(stats), bvpart, bv, mu,
                     sigma, rs, pl.N, pl.m, pl.d, pl.ntiles, pl.tt, pl.groups, pl.whiten ? 1 : 0);
  hipLaunchKernelGGL(y_kernel, grid, dim3(256), 0, s, x, bv, y, pl.m, pl.mp, pl.d);
  return hipGetLastError();
}

}  // namespace lapnys
