// Conjugate-gradient solve of W Y = B V (the solver the pages' ablation sets
// against Newton-Schulz: EN page, section 4, solver robustness; DE section 4,
// ablations).  One CG run per column of B V, from Y0 = 0, no preconditioner,
// a fixed number of steps:
//   a = r.r / p.(W p);  y += a p;  r -= a W p;  b = r'.r' / r.r;  p = r' + b p
// with a = b = 0 for a column whose residual is exactly zero.  Float32
// throughout; every sum has a fixed order, so results repeat bit for bit.
// For a well-conditioned W the recursive residual keeps shrinking by a
// constant factor per step and can leave float32's range within the step
// count (float64 cannot): a step whose p.(W p) is not positive is skipped.
//
// Work layout: workgroup (cb, p) takes columns [16 cb, 16 cb + 16) of problem
// p.  W (mp x mp, zero padded, row-major) stays in the workspace and is read
// once per step (from L2); the direction vectors go through LDS, transposed,
// as the B operand of W P on fp32 MFMA 16x16x4.  Wavefront w forms row blocks
// w RBW + [0, RBW) (RBW = mp / 64) of Q = W P, and lane (li, lk) keeps in
// registers the entries of y, r, p and q it produces: rows 16 rb + 4 lk + r,
// column li.  The MFMA reduction index is permuted so that lane group lk takes
// k in [S lk, S lk + S), S = mp / 4, and both operands are 16-byte loads; the
// next row block's W values are loaded while the current one's products run.
#include "lapnys_internal.hpp"

namespace lapnys {

namespace {

template <int RBW>
__global__ __launch_bounds__(256) void cg_kernel(const float* __restrict__ w, const float* __restrict__ bv,
                                                 float* __restrict__ y, int m, int d, int iters) {
  constexpr int kMP = 64 * RBW;
  constexpr int kS = kMP / 4;       // reduction indices per lane group
  constexpr int kC = kS / 4;        // 16-byte chunks per lane group
  constexpr int kPT = kMP + 4;      // P^T row stride (floats)
  __shared__ __align__(16) float pt[16 * kPT];
  __shared__ float red[2][4][16];
  const int cb = blockIdx.x, p = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int col = 16 * cb + li;
  const float* wp = w + (size_t)p * kMP * kMP;
  const float* bvp = bv + (size_t)p * m * d;

  // Own entries: row block rb = wv RBW + i, rows 16 rb + 4 lk + r.
  float yv[RBW][4], rv[RBW][4], pv[RBW][4];
#pragma unroll
  for (int i = 0; i < RBW; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * (wv * RBW + i) + 4 * lk + r;
      const float b = bvp[(size_t)min(row, m - 1) * d + col];
      rv[i][r] = row < m ? b : 0.f;
      pv[i][r] = rv[i][r];
      yv[i][r] = 0.f;
    }

  // Column sums of this wavefront's own entries, merged over the lane groups
  // ((g0 + g1) + (g2 + g3)) and then over the wavefronts in order.
  auto column_sum = [&](float part, int buf) {
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    if (lk == 0) red[buf][wv][li] = part;
    __syncthreads();
    return ((red[buf][0][li] + red[buf][1][li]) + red[buf][2][li]) + red[buf][3][li];
  };
  auto own_dot = [&](const float (&a)[RBW][4], const float (&b)[RBW][4]) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) s = fmaf(a[i][r], b[i][r], s);
    return s;
  };
  float rr = column_sum(own_dot(rv, rv), 0);

  for (int it = 0; it < iters; ++it) {
    // P^T into LDS: four consecutive rows of one column per row block.  The
    // previous step's reads of P^T ended before the barriers of its sums.
#pragma unroll
    for (int i = 0; i < RBW; ++i)
      *reinterpret_cast<f32x4*>(&pt[li * kPT + 16 * (wv * RBW + i) + 4 * lk]) =
          f32x4{pv[i][0], pv[i][1], pv[i][2], pv[i][3]};
    __syncthreads();

    // Q = W P for the own row blocks.
    f32x4 q[RBW];
    f32x4 wa[2][kC];
    auto load_w = [&](int i, int buf) {
      const float* wr = wp + (size_t)(16 * (wv * RBW + i) + li) * kMP + kS * lk;
#pragma unroll
      for (int c = 0; c < kC; ++c) wa[buf][c] = *reinterpret_cast<const f32x4*>(wr + 4 * c);
    };
    load_w(0, 0);
#pragma unroll
    for (int i = 0; i < RBW; ++i) {
      if (i + 1 < RBW) load_w(i + 1, (i + 1) & 1);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kC; ++c) {
        const f32x4 b = *reinterpret_cast<const f32x4*>(&pt[li * kPT + kS * lk + 4 * c]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[i & 1][c][e], b[e], acc, 0, 0, 0);
      }
      q[i] = acc;  // q[i][r] = (W P)[16 rb + 4 lk + r][col]
    }
    float qv[RBW][4];
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) qv[i][r] = q[i][r];

    const float pq = column_sum(own_dot(pv, qv), 0);
    // p.(W p) is positive for any p != 0; a column whose residual has run
    // below float32's range (p.(W p) rounds to 0 while r.r may not) takes no
    // further steps, as a column with r = 0 does.
    const float a = rr > 0.f && pq > 0.f ? rr / pq : 0.f;
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        yv[i][r] = fmaf(a, pv[i][r], yv[i][r]);
        rv[i][r] = fmaf(-a, qv[i][r], rv[i][r]);
      }
    const float rr_new = column_sum(own_dot(rv, rv), 1);
    const float b = rr > 0.f ? rr_new / rr : 0.f;
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) pv[i][r] = fmaf(b, pv[i][r], rv[i][r]);
    rr = rr_new;
  }

  float* yp = y + (size_t)p * m * d;
#pragma unroll
  for (int i = 0; i < RBW; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * (wv * RBW + i) + 4 * lk + r;
      if (row < m) yp[(size_t)row * d + col] = yv[i][r];
    }
}

}  // namespace

hipError_t launch_cg(const Plan& pl, const Work& wk, hipStream_t s, hipEvent_t stop) {
  if (!pl.cg || pl.fused_ns) return hipErrorInvalidValue;
  const dim3 grid(pl.d / 16, pl.P);
  switch (pl.mp / 64) {
    case 1: hipExtLaunchKernelGGL(cg_kernel<1>, grid, dim3(256), 0, s, nullptr, stop, 0, wk.w, wk.bv, wk.y, pl.m, pl.d,
                                  pl.ns_iters); break;
    case 2: hipExtLaunchKernelGGL(cg_kernel<2>, grid, dim3(256), 0, s, nullptr, stop, 0, wk.w, wk.bv, wk.y, pl.m, pl.d,
                                  pl.ns_iters); break;
    case 3: hipExtLaunchKernelGGL(cg_kernel<3>, grid, dim3(256), 0, s, nullptr, stop, 0, wk.w, wk.bv, wk.y, pl.m, pl.d,
                                  pl.ns_iters); break;
    case 4: hipExtLaunchKernelGGL(cg_kernel<4>, grid, dim3(256), 0, s, nullptr, stop, 0, wk.w, wk.bv, wk.y, pl.m, pl.d,
                                  pl.ns_iters); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lapnys
