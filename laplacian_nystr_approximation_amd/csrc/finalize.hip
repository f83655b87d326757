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
// m > 64: one lane per B V element: the launch is wide (every partial is
// read once, in parallel across the chip) and each lane keeps up to 16
// groups' loads in flight before its ordered adds; one extra workgroup per
// problem produces the statistics, one lane per landmark.  m <= 64: four
// workgroups per problem (two for d = 32), each reducing a 16-feature column
// slice of B V and forming the same slice of Y = X (B V) on fp32 MFMA, which
// it stores transposed as bf16 high and low parts for the output stage, and
// one more for the statistics.  Loads past the last group or tile read a
// clamped, valid address and are dropped where they are used: a load under a
// condition would become a branch with its own wait, one memory round trip
// per load.  Every reduction has a fixed order, so results repeat bit for
// bit.
#include <math.h>

#include "lapnys_internal.hpp"

namespace lapnys {

namespace {

constexpr int kChunk = 16;

// Mean, population standard deviation and its reciprocal of landmark column
// j of problem p, merged from the per-tile (sum, M2) pairs (lane j of one
// workgroup per problem).
__device__ __forceinline__ void column_stats(const float2* __restrict__ stats, float* __restrict__ mu,
                                             float* __restrict__ sigma, float* __restrict__ rs, int N, int m,
                                             int ntiles, int tt, int whiten, int p, int j) {
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

  column_stats(stats, mu, sigma, rs, N, m, ntiles, tt, whiten, p, threadIdx.x);
}

// m <= 64: workgroup (c, p), c < D / 16, reduces columns [16 c, 16 c + 16) of
// problem p's B V in group order, forms the same columns of Y = X (B V) (X
// zero padded to 64 x 64, rows of B V past m zero) on fp32 MFMA 16x16x4, and
// stores them into Y^T high and low parts; workgroup c = D / 16 merges the
// statistics, beside them.  Workgroups are handed to the XCDs in turn by
// index, and each XCD has its own L2: the index b = (p / 8) 8 (D / 16 + 1) +
// 8 c + p % 8 keeps all of a problem's workgroups on one XCD, so X and the
// B V partials come from HBM once per problem instead of once per slice
// (at 320 problems the launch took 9.4 us with the slices on four XCDs).
// Problems past P (the grid rounds P up to a multiple of 8) exit at once.
template <int D>
__global__ __launch_bounds__(256) void finalize_fused_kernel(const float2* __restrict__ stats,
                                                             const float* __restrict__ bvpart,
                                                             const float* __restrict__ x, float* __restrict__ bv,
                                                             float* __restrict__ mu, float* __restrict__ sigma,
                                                             float* __restrict__ rs, __bf16* __restrict__ yt, int N,
                                                             int m, int ntiles, int tt, int groups, int whiten, int P) {
  constexpr int DB = D / 16;
  constexpr int kXS = 68;  // X row stride in LDS: the A-operand column reads hit distinct banks
  __shared__ __align__(16) float xs[64 * kXS];
  __shared__ __align__(16) float bs[64 * 16];  // the B V column slice, [landmark][16]
  const int b = blockIdx.x, tid = threadIdx.x;
  const int p = (b / (8 * (DB + 1))) * 8 + b % 8, c = (b / 8) % (DB + 1);
  if (p >= P) return;
  if (c == DB) {
    column_stats(stats, mu, sigma, rs, N, m, ntiles, tt, whiten, p, tid);
    return;
  }
  const int md = m * D;

  // X: 64 x 64 (the solver's padded layout), four 16-byte loads per lane.
  const float4* xp4 = reinterpret_cast<const float4*>(x + (size_t)p * 64 * 64);
  float4 xv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xv[i] = xp4[tid + 256 * i];
  // B V: lane (k, q) sums row k, columns 16 c + 4 q + [0, 4), over the groups.
  const int k = tid >> 2, c4 = 16 * c + 4 * (tid & 3);
  const float* src = bvpart + (size_t)p * groups * md + (size_t)min(k, m - 1) * D + c4;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int g0 = 0; g0 < groups; g0 += kChunk) {
    float4 v[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) v[u] = *reinterpret_cast<const float4*>(src + (size_t)min(g0 + u, groups - 1) * md);
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if (g0 + u < groups) {
        sum.x += v[u].x;
        sum.y += v[u].y;
        sum.z += v[u].z;
        sum.w += v[u].w;
      }
    }
  }
  if (k < m) {
    *reinterpret_cast<float4*>(bv + ((size_t)p * m + k) * D + c4) = sum;
  } else {
    sum = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  *reinterpret_cast<float4*>(&bs[k * 16 + 4 * (tid & 3)]) = sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e4 = tid + 256 * i;
    *reinterpret_cast<float4*>(&xs[(e4 >> 4) * kXS + 4 * (e4 & 15)]) = xv[i];
  }
  __syncthreads();

  // Y rows [16 w, 16 w + 16), columns [16 c, 16 c + 16): A[li][lk] =
  // X[16 w + li][4 s + lk], B[lk][li] = (B V)[4 s + lk][16 c + li].
  const int lane = tid & 63, w = tid >> 6, li = lane & 15, lk = lane >> 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < 16; ++st)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xs[(16 * w + li) * kXS + 4 * st + lk], bs[(4 * st + lk) * 16 + li], acc,
                                              0, 0, 0);
  // acc[r] = Y[16 w + 4 lk + r][f]: four consecutive landmarks of feature f.
  const int f = 16 * c + li;
  uint32_t h0, l0, h1, l1;
  split2(acc[0], acc[1], h0, l0);
  split2(acc[2], acc[3], h1, l1);
  __bf16* yp = yt + (size_t)p * 2 * D * 64;
  const int at = yt_index(f, 16 * w + 4 * lk, f / DB, 64);
  *reinterpret_cast<uint2*>(yp + at) = make_uint2(h0, h1);
  *reinterpret_cast<uint2*>(yp + D * 64 + at) = make_uint2(l0, l1);
}

}  // namespace

hipError_t launch_reduce(const Plan& pl, const Work& w, hipStream_t s, Span t) {
  if (pl.fused_ns) {
    auto kern = pl.d == 64 ? finalize_fused_kernel<64> : finalize_fused_kernel<32>;
    const int grid = (pl.P + 7) / 8 * 8 * (pl.d / 16 + 1);
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, t.start, t.stop, 0,
                          reinterpret_cast<const float2*>(w.stats), w.bvpart, w.x_final, w.bv, w.mu, w.sigma, w.rs,
                          w.yt, pl.N, pl.m, pl.ntiles, pl.tt, pl.groups, pl.whiten ? 1 : 0, pl.P);
    return hipGetLastError();
  }
  const int nbv = (pl.m * pl.d + 255) / 256;
  hipExtLaunchKernelGGL(reduce_kernel, dim3(nbv + 1, pl.P), dim3(256), 0, s, t.start, t.stop, 0,
                        reinterpret_cast<const float2*>(w.stats),
                     w.bvpart, w.bv, w.mu, w.sigma, w.rs, pl.N, pl.m, pl.d, pl.ntiles, pl.tt, pl.groups,
                     pl.whiten ? 1 : 0);
  return hipGetLastError();
}

}  // namespace lapnys
