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

template <typename T>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ k, float* __restrict__ kt,
                                                   int N, int d, int grid_w, int pool, int gw, int m,
                                                   long long total) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int t = (int)(idx % d);
  const long long rest = idx / d;
  const int j = (int)(rest % m);
  const long long p = rest / m;
  const int R = j / gw, Cc = j % gw;
  const T* kp = k + p * (long long)N * d;
  double acc = 0.0;
  for (int r = 0; r < pool; ++r) {
    const T* row = kp + ((long long)(R * pool + r) * grid_w + (long long)Cc * pool) * d + t;
    for (int c = 0; c < pool; ++c) acc += (double)widen(row[(long long)c * d]);
  }
  kt[idx] = (float)(acc / (double)(pool * pool));
}

hipError_t launch_pool(const Plan& pl, const void* k, float* kt, hipStream_t s) {
  const long long total = (long long)pl.P * pl.m * pl.d;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (pl.dtype == 1)
    hipLaunchKernelGGL(pool_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s, (const uint16_t*)k, kt, pl.N,
                       pl.d, pl.grid_w, pl.pool, pl.gw, pl.m, total);
  else
    hipLaunchKernelGGL(pool_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)k, kt, pl.N, pl.d,
                       pl.grid_w, pl.pool, pl.gw, pl.m, total);
  return hipGetLastError();
}

}  // namespace lapnys
