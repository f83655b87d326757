// Landmark average pooling (EN page, section 2.C.1: landmark keys are chosen by
// average pooling).  K~[j, t] is the mean of K over the pool x pool window of
// landmark j on the row-major token grid.
//
// One lane per output element (problem, landmark, feature): consecutive lanes
// take consecutive features, so every load instruction reads contiguous
// memory, and each element of K is read exactly once.  The window sum is
// accumulated in float64 in a fixed order (window row outer, window column
// inner), divided by pool*pool and rounded to float32 once, so the result is
// bit-for-bit the float32 rounding of the float64 mean computed in that order.
#include "lapnys_internal.hpp"

namespace lapnys {

// POOL > 0: the window size is a compile-time constant, so every load of the
// window is issued before the (dependent) float64 adds.  POOL == 0: any window
// size, loads issued a window row at a time in chunks of 8.
template <typename T, int POOL>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ k, float* __restrict__ kt, int N, int d,
                                                   int grid_w, int pool_rt, int gw, int m, long long total) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int pool = POOL > 0 ? POOL : pool_rt;
  const int t = (int)(idx % d);
  const long long rest = idx / d;
  const int j = (int)(rest % m);
  const long long p = rest / m;
  const int R = j / gw, Cc = j % gw;
  const T* base = k + p * (long long)N * d + ((long long)R * pool * grid_w + (long long)Cc * pool) * d + t;
  const long long row_stride = (long long)grid_w * d;
  double acc = 0.0;
  if constexpr (POOL > 0) {
    float vals[POOL * POOL];
#pragma unroll
    for (int r = 0; r < POOL; ++r)
#pragma unroll
      for (int c = 0; c < POOL; ++c) vals[r * POOL + c] = widen(base[r * row_stride + (long long)c * d]);
#pragma unroll
    for (int e = 0; e < POOL * POOL; ++e) acc += (double)vals[e];
  } else {
    for (int r = 0; r < pool; ++r) {
      const T* row = base + r * row_stride;
      for (int c0 = 0; c0 < pool; c0 += 8) {
        float vals[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) vals[c] = (c0 + c < pool) ? widen(row[(long long)(c0 + c) * d]) : 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (c0 + c < pool) acc += (double)vals[c];
      }
    }
  }
  kt[idx] = (float)(acc / (double)(pool * pool));
}

template <typename T>
void launch_typed(const Plan& pl, const T* k, float* kt, hipStream_t s, Span t) {
  const long long total = (long long)pl.P * pl.m * pl.d;
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  switch (pl.pool) {
    case 1: hipExtLaunchKernelGGL((pool_kernel<T, 1>), grid, block, 0, s, t.start, t.stop, 0, k, kt, pl.N, pl.d, pl.grid_w, 1, pl.gw, pl.m, total); break;
    case 2: hipExtLaunchKernelGGL((pool_kernel<T, 2>), grid, block, 0, s, t.start, t.stop, 0, k, kt, pl.N, pl.d, pl.grid_w, 2, pl.gw, pl.m, total); break;
    case 4: hipExtLaunchKernelGGL((pool_kernel<T, 4>), grid, block, 0, s, t.start, t.stop, 0, k, kt, pl.N, pl.d, pl.grid_w, 4, pl.gw, pl.m, total); break;
    case 8: hipExtLaunchKernelGGL((pool_kernel<T, 8>), grid, block, 0, s, t.start, t.stop, 0, k, kt, pl.N, pl.d, pl.grid_w, 8, pl.gw, pl.m, total); break;
    case 16: hipExtLaunchKernelGGL((pool_kernel<T, 16>), grid, block, 0, s, t.start, t.stop, 0, k, kt, pl.N, pl.d, pl.grid_w, 16, pl.gw, pl.m, total); break;
    default: hipExtLaunchKernelGGL((pool_kernel<T, 0>), grid, block, 0, s, t.start, t.stop, 0, k, kt, pl.N, pl.d, pl.grid_w, pl.pool, pl.gw, pl.m, total); break;
  }
}

hipError_t launch_pool(const Plan& pl, const void* k, const Work& w, hipStream_t s, Span t) {
  if (pl.dtype == 1)
    launch_typed<uint16_t>(pl, (const uint16_t*)k, w.kt, s, t);
  else
    launch_typed<float>(pl, (const float*)k, w.kt, s, t);
  return hipGetLastError();
}

}  // namespace lapnys
