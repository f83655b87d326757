// Issue-rate probe for the vector ALU of one MI355X (gfx950): how many
// float32 lane-operations per CU per clock the subtract / add-with-|.| pair
// of the L1 distance loop retires, at a fixed number of wavefronts per SIMD.
//
// Every lane runs eight independent chains s_u += |x - y_u| written as
// explicit v_sub_f32 / v_add_f32 instructions (so the instruction count per
// iteration is exact: 8 subtracts then 8 adds), with register operands only.
// Occupancy is fixed by the dynamic LDS request: a workgroup of 256 lanes is
// one wavefront per SIMD, and the LDS size admits exactly `waves_per_simd`
// workgroups per CU (160 KB of LDS per CU).  The grid is 256 CUs x
// waves_per_simd x rounds workgroups.
//
// C entry point (measurement tooling, not part of liblapnys):
//   int valu_probe_run(int waves_per_simd, int iters, int rounds, float* ms,
//                      double* lane_ops)
// runs the kernel once untimed and once between two events; returns 0 or a
// hipError_t, and the kernel time and the executed VALU lane-operations of
// the L1 pair (16 per lane per inner step).
#include <hip/hip_runtime.h>

namespace {

constexpr int kLdsPerCu = 160 * 1024;
constexpr int kRepeat = 8;  // asm blocks per loop iteration

__global__ __launch_bounds__(256) void valu_probe_kernel(const float* __restrict__ in, float* __restrict__ out,
                                                         int iters) {
  extern __shared__ float lds[];
  const int g = blockIdx.x * 256 + threadIdx.x;
  const float x = in[g & 1023];
  float y[8], s[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    y[u] = in[(g + 97 * (u + 1)) & 1023];
    s[u] = 0.f;
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < kRepeat; ++r) {
      float d0, d1, d2, d3, d4, d5, d6, d7;
      asm volatile(
          "v_sub_f32 %[d0], %[x], %[y0]\n\t"
          "v_sub_f32 %[d1], %[x], %[y1]\n\t"
          "v_sub_f32 %[d2], %[x], %[y2]\n\t"
          "v_sub_f32 %[d3], %[x], %[y3]\n\t"
          "v_sub_f32 %[d4], %[x], %[y4]\n\t"
          "v_sub_f32 %[d5], %[x], %[y5]\n\t"
          "v_sub_f32 %[d6], %[x], %[y6]\n\t"
          "v_sub_f32 %[d7], %[x], %[y7]\n\t"
          "v_add_f32 %[s0], %[s0], |%[d0]|\n\t"
          "v_add_f32 %[s1], %[s1], |%[d1]|\n\t"
          "v_add_f32 %[s2], %[s2], |%[d2]|\n\t"
          "v_add_f32 %[s3], %[s3], |%[d3]|\n\t"
          "v_add_f32 %[s4], %[s4], |%[d4]|\n\t"
          "v_add_f32 %[s5], %[s5], |%[d5]|\n\t"
          "v_add_f32 %[s6], %[s6], |%[d6]|\n\t"
          "v_add_f32 %[s7], %[s7], |%[d7]|"
          : [d0] "=&v"(d0), [d1] "=&v"(d1), [d2] "=&v"(d2), [d3] "=&v"(d3), [d4] "=&v"(d4), [d5] "=&v"(d5),
            [d6] "=&v"(d6), [d7] "=&v"(d7), [s0] "+v"(s[0]), [s1] "+v"(s[1]), [s2] "+v"(s[2]), [s3] "+v"(s[3]),
            [s4] "+v"(s[4]), [s5] "+v"(s[5]), [s6] "+v"(s[6]), [s7] "+v"(s[7])
          : [x] "v"(x), [y0] "v"(y[0]), [y1] "v"(y[1]), [y2] "v"(y[2]), [y3] "v"(y[3]), [y4] "v"(y[4]),
            [y5] "v"(y[5]), [y6] "v"(y[6]), [y7] "v"(y[7]));
    }
  }
  float t = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) t += s[u];
  out[g] = t;
  if (t == -1.f) lds[threadIdx.x] = t;  // keeps the LDS request live
}

}  // namespace

extern "C" int valu_probe_run(int waves_per_simd, int iters, int rounds, float* ms, double* lane_ops) {
  if (waves_per_simd < 1 || waves_per_simd > 8 || iters < 1 || rounds < 1 || !ms || !lane_ops)
    return (int)hipErrorInvalidValue;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return (int)e;
  // exactly waves_per_simd workgroups (of one wavefront per SIMD) fit a CU
  const size_t lds = ((size_t)kLdsPerCu / waves_per_simd) & ~(size_t)255;
  e = hipFuncSetAttribute((const void*)valu_probe_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return (int)e;
  const long long grid = (long long)cus * waves_per_simd * rounds;
  float *in = nullptr, *out = nullptr;
  if ((e = hipMalloc(&in, 1024 * sizeof(float))) != hipSuccess) return (int)e;
  if ((e = hipMalloc(&out, grid * 256 * sizeof(float))) != hipSuccess) {
    (void)hipFree(in);
    return (int)e;
  }
  float host[1024];
  for (int i = 0; i < 1024; ++i) host[i] = 0.001f * (float)((i * 37) % 1000) - 0.5f;
  hipEvent_t a = nullptr, b = nullptr;
  e = hipMemcpy(in, host, sizeof(host), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(valu_probe_kernel, dim3((unsigned)grid), dim3(256), lds, 0, in, out, iters);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(a, 0);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(valu_probe_kernel, dim3((unsigned)grid), dim3(256), lds, 0, in, out, iters);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(b, 0);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, a, b);
  *lane_ops = (double)grid * 256.0 * (double)iters * kRepeat * 16.0;
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  (void)hipFree(in);
  (void)hipFree(out);
  return (int)e;
}
