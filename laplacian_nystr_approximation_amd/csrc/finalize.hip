// Reductions between the kernel-matrix stage and the output stage.
//
//  * B V = sum over tile groups of the partial products, in group order.
//  * Whitening statistics (EN page, section 2.B; KO section 2.2): for every
//    landmark column j of C, the mean and the population standard deviation
//    over the N tokens of the problem.  The per-tile (sum, squared deviations
//    about the tile mean) pairs are merged in float64, in tile order, with the
//    exact decomposition M2 = sum_t [M2_t + n_t (mean_t - mean)^2], so the
//    result is the two-pass statistic, not a one-pass E[c^2] - E[c]^2.
//
// One lane per B V element: the launch is wide (every partial is read once,
// in parallel across the chip) and each lane keeps up to 16 groups' loads in
// flight before its ordered adds.  Loads past the last group or tile read a
// clamped, valid address and are dropped where they are used: a load under a
// condition would become a branch with its own wait, one memory round trip
// per load.  One extra workgroup per problem produces
// the statistics, one lane per landmark.  Every reduction has a fixed order,
// so results repeat bit for bit.
#include <math.h>

#include "lapnys_internal.hpp"

namespace lapnys {

namespace {

constexpr int kChunk = 16;

__global__ __launch_bounds__(256) void reduce_kernel(const float2* __restrict__ stats,
                                                     const float* __restrict__ bvpart, float* __restrict__ bv,
                                                     float* __restrict__ mu, float* __restrict__ sigma,
                                                     float* __restrict__ rs, int N, int m, int D, int ntiles, int tt,
                                                     int groups, int whiten) {
  const int p = blockIdx.y;
  const int md = m * D;
  const int nbv = (md + 255) / 256;
  if ((int)blockIdx.x < nbv) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= md) return;
    const float* src = bvpart + (size_t)p * groups * md + e;
    float sum = 0.f;
    for (int g0 = 0; g0 < groups; g0 += kChunk) {
      float v[kChunk];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) v[u] = src[(size_t)min(g0 + u, groups - 1) * md];
#pragma unroll
      for (int u = 0; u < kChunk; ++u)
        if (g0 + u < groups) sum += v[u];
    }
    bv[(size_t)p * md + e] = sum;
    return;
  }

  const int j = threadIdx.x;
  if (j >= m) return;
  if (!whiten) {
    mu[p * m + j] = 0.f;
    sigma[p * m + j] = 1.f;
    rs[p * m + j] = 1.f;
    return;
  }
  const float2* st = stats + (size_t)p * ntiles * m + j;
  // Each chunk of (sum, M2) pairs is loaded once when the tiles fit in one
  // chunk (the common case): the mean needs every tile's sum first, and the
  // deviation pass reuses the same registers.
  double total = 0.0, m2 = 0.0;
  if (ntiles <= kChunk) {
    float2 v[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) v[u] = st[(size_t)min(u, ntiles - 1) * m];
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      if (u < ntiles) total += (double)v[u].x;
    const double mean = total / (double)N;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if (u < ntiles) {
        const int n = min(tt, N - u * tt);
        const double dm = (double)v[u].x / (double)n - mean;
        m2 += (double)v[u].y + (double)n * dm * dm;
      }
    }
  } else {
    for (int i0 = 0; i0 < ntiles; i0 += kChunk) {
      float v[kChunk];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) v[u] = st[(size_t)min(i0 + u, ntiles - 1) * m].x;
#pragma unroll
      for (int u = 0; u < kChunk; ++u)
        if (i0 + u < ntiles) total += (double)v[u];
    }
    const double mean = total / (double)N;
    for (int i0 = 0; i0 < ntiles; i0 += kChunk) {
      float2 v[kChunk];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) v[u] = st[(size_t)min(i0 + u, ntiles - 1) * m];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        if (i0 + u < ntiles) {
          const int n = min(tt, N - (i0 + u) * tt);
          const double dm = (double)v[u].x / (double)n - mean;
          m2 += (double)v[u].y + (double)n * dm * dm;
        }
      }
    }
  }
  const double mean = total / (double)N;
  const double sd = sqrt(m2 / (double)N);
  mu[p * m + j] = (float)mean;
  sigma[p * m + j] = (float)sd;
  rs[p * m + j] = sd > 0.0 ? (float)(1.0 / sd) : 0.f;
}

}  // namespace

hipError_t launch_reduce(const Plan& pl, const Work& w, hipStream_t s, Span t) {
  const int nbv = (pl.m * pl.d + 255) / 256;
  hipExtLaunchKernelGGL(reduce_kernel, dim3(nbv + 1, pl.P), dim3(256), 0, s, t.start, t.stop, 0,
                        reinterpret_cast<const float2*>(w.stats),
                     w.bvpart, w.bv, w.mu, w.sigma, w.rs, pl.N, pl.m, pl.d, pl.ntiles, pl.tt, pl.groups,
                     pl.whiten ? 1 : 0);
  return hipGetLastError();
}

}  // namespace lapnys
