// Internal declarations shared by the liblapnys translation units: device
// helpers, the per-call plan (tiling and workspace layout) and the kernel
// launchers.  Nothing here is part of the public C ABI (include/lapnys.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lapnys {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Input element widening: float32 passes through, bfloat16 (stored as its
// 16-bit pattern) widens exactly by placing it in the high half of a float32.
__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Butterfly sum over the 64 lanes of a wavefront.  The pairing is fixed, so
// the result is the same on every run.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Landmark block handled by one workgroup of the fused kernel-matrix stage.
constexpr int kLandmarkBlock = 64;
// Largest landmark count the fused single-workgroup Newton-Schulz handles.
constexpr int kFusedNsMaxM = 64;
// Largest supported landmark count.
constexpr int kMaxM = 256;

// Per-call plan: sizes, tiling and the workspace layout (byte offsets, each
// 256-byte aligned).  Computed on the host from the validated parameters.
struct Plan {
  int P;            // B * H problems
  int N, d, m;      // tokens, head dimension, landmarks
  int gw;           // pooled grid width (grid_w / pool)
  int grid_w, pool;
  int dtype;        // lapnys_dtype
  bool whiten;
  int ns_iters;
  float scale;      // -log2(e) / lambda, so k = exp2(scale * L1)
  float eps;
  int mp;           // padded Newton-Schulz size (64, or m rounded up to 64)
  bool fused_ns;    // m <= kFusedNsMaxM: one workgroup per problem
  int tt;           // tokens per tile of the kernel-matrix stage (256 or 128)
  int ntiles;       // token tiles per problem
  int lb;           // landmarks per block of the kernel-matrix stage
  int jblocks;      // landmark blocks (ceil(m / lb))
  int tpg;          // tiles per workgroup (tile group)
  int groups;       // tile groups per problem
  // workspace offsets in bytes
  size_t off_kt, off_w, off_x, off_x2, off_pm, off_ct, off_stats, off_bvpart, off_bv,
      off_mu, off_sigma, off_rs, off_y, total;
};

// Kernel launchers (each returns the hipError_t of its launch).
hipError_t launch_pool(const Plan& pl, const void* k, float* kt, hipStream_t s);
hipError_t launch_ns(const Plan& pl, const float* kt, float* w, float* x, float* x2, float* pm,
                     float** x_final, hipStream_t s);
hipError_t launch_l1exp(const Plan& pl, const void* q, const void* k, const void* v, const float* kt,
                        float* ct, float* stats, float* bvpart, hipStream_t s);
hipError_t launch_finalize(const Plan& pl, const float* stats, const float* bvpart, const float* x,
                           float* bv, float* mu, float* sigma, float* rs, float* y, hipStream_t s);
hipError_t launch_output(const Plan& pl, const float* ct, const float* y, const float* mu, const float* rs,
                         float* out, hipStream_t s);
hipError_t launch_extract_square(const float* src, int src_ld, float* dst, int n, int P, hipStream_t s);

}  // namespace lapnys
