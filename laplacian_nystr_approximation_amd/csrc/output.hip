// Output stage: O = Z Y with Z = (C - mu) / sigma column-wise (the diagonal
// whitening of EN page section 2.B) and Y = X (B V), i.e. O = Z W^-1 (B V).
//
// One workgroup per 256-token tile, four wavefronts of 64 tokens each.  The
// stage streams C once and writes O once; its arithmetic (2 N m d flops per
// problem) is small, so the design goal is to keep every C load in flight
// early and every store full-width.
//
//  * Each lane loads C^T[landmark][4 consecutive tokens] as one 16-byte load;
//    16 lanes cover a 256-byte run of one landmark row.  All of a wavefront's
//    C loads (up to 64 landmarks) are issued before anything else, so their
//    latency overlaps the Y prologue.  For m > 64 the loads of the next 64
//    landmarks are issued group by group as the current ones are consumed.
//  * Prologue (m <= 64): the workgroup forms Y = X (B V) itself on fp32 MFMA
//    (a 64 x 64 x 64 product, zero padded) into LDS; for larger m, Y comes
//    from a batched tile GEMM and is copied into LDS.
//  * Main loop: a wavefront's 64 x D output is (4 x D/16) blocks of fp32
//    MFMA 16x16x4 reducing over four landmarks per step.  Lane (li, lk)
//    feeds A[li][lk] = Z[token tb + 4 li + a][landmark] for token block a,
//    and B[lk][li] = Y[landmark][D/16 li + b] for feature block b, so that a
//    lane ends up holding D/16 consecutive features of each of its tokens and
//    writes them with one 16-byte (D = 64) or 8-byte (D = 32) store.
#include "lapnys_internal.hpp"

namespace lapnys {

namespace {

constexpr int kXLD = 65;   // LDS row stride of X in the prologue
constexpr int kGroups = 16;  // landmark groups of four held in registers (64 landmarks)

// All-ones when ok, else zero, opaque to the optimiser: masking a loaded
// value with it (instead of a select) keeps the load unconditional, so it
// issues with the others and no early wait is needed for it.
__device__ __forceinline__ uint32_t lane_mask(bool ok) {
  uint32_t mk = ok ? 0xffffffffu : 0u;
  asm volatile("" : "+v"(mk));
  return mk;
}

__device__ __forceinline__ float masked(float v, uint32_t mk) { return __uint_as_float(__float_as_uint(v) & mk); }

template <int D>
struct OutVec;
template <>
struct OutVec<64> {
  using type = float4;
};
template <>
struct OutVec<32> {
  using type = float2;
};

template <int D, bool FUSED_Y>
__global__ __launch_bounds__(256) void output_kernel(const float* __restrict__ ct, int ldc,
                                                     const float* __restrict__ x, int mp,
                                                     const float* __restrict__ bv, const float* __restrict__ y,
                                                     const float* __restrict__ mu, const float* __restrict__ rs,
                                                     float* __restrict__ out, int N, int m) {
  constexpr int DB = D / 16;
  extern __shared__ float lds[];
  const int m4 = (m + 3) & ~3;
  const int ym = FUSED_Y ? 64 : m4;  // rows of Y in LDS; rows >= m are zero
  float* yl = lds;                   // [ym][D]
  float2* mrs = reinterpret_cast<float2*>(yl + ym * D);  // [m4]: (mu, 1/sigma), zero past m
  const int tile = blockIdx.x, p = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int tb = tile * 256 + 64 * w;  // first token of this wavefront
  const int tok4 = tb + 4 * li;        // first of this lane's four tokens
  const bool tok_ok = tok4 < N;

  // C loads: landmark rows past m and tokens past N are read from a clamped,
  // in-bounds address and masked to zero where they are used, so the loads
  // are unconditional and all issue before the first wait.
  float4 cr[kGroups];
  const float* cpc = ct + (size_t)p * m * ldc + min(tok4, ldc - 4);
  auto load_group = [&](int c0, int g) {
    cr[g] = *reinterpret_cast<const float4*>(cpc + (size_t)min(c0 + 4 * g + lk, m - 1) * ldc);
  };

  if constexpr (FUSED_Y) {
    // Prologue operands are loaded into registers ahead of the C loads, and
    // nothing consumes a loaded value before the scheduling barrier, so the
    // wait for the prologue operands leaves the C loads in flight.
    constexpr int kXPer = 64 * 64 / 256, kBPer = 64 * D / 256;
    const float* xp = x + (size_t)p * mp * mp;
    const float* bp = bv + (size_t)p * m * D;
    float xr[kXPer], br[kBPer];
#pragma unroll
    for (int i = 0; i < kXPer; ++i) xr[i] = xp[(size_t)(i * 4 + (tid >> 6)) * mp + (tid & 63)];  // row, col < 64 <= mp
#pragma unroll
    for (int i = 0; i < kBPer; ++i) br[i] = bp[min(tid + 256 * i, m * D - 1)];
    const int jt = tid & 63;
    const float mu_t = mu[p * m + min(jt, m - 1)], rs_t = rs[p * m + min(jt, m - 1)];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) load_group(0, g);
    __builtin_amdgcn_sched_barrier(0);

    // Y = X (B V), 64 x D, on fp32 MFMA 32x32x2; X and B V zero padded to 64 rows.
    float* xl = reinterpret_cast<float*>(mrs + 64);  // [64][kXLD]
    float* bvl = xl + 64 * kXLD;                    // [64][D]
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int r = i * 4 + (tid >> 6), c = tid & 63;
      xl[r * kXLD + c] = masked(xr[i], lane_mask(r < m && c < m));
    }
#pragma unroll
    for (int i = 0; i < kBPer; ++i) bvl[tid + 256 * i] = masked(br[i], lane_mask(tid + 256 * i < m * D));
    {
      // Every wavefront stores the same 64 pairs (an unconditional store keeps
      // the two loads from being moved behind the C loads' wait).
      const uint32_t mk = lane_mask(jt < m);
      mrs[jt] = make_float2(masked(mu_t, mk), masked(rs_t, mk));
    }
    __syncthreads();
    const int yi = lane & 31, yk = lane >> 5;
    const int bi = w >> 1, bj = w & 1;
    if (32 * bj < D) {
      f32x16 acc = {0.f};
      // Full 64-deep product over the zero-padded operands, unrolled so that
      // the LDS reads run ahead of the MFMA chain.
#pragma unroll
      for (int k0 = 0; k0 < 64; k0 += 2) {
        const float a = xl[(32 * bi + yi) * kXLD + k0 + yk];
        const float b = bvl[(k0 + yk) * D + 32 * bj + yi];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) yl[(32 * bi + 8 * (r >> 2) + 4 * yk + (r & 3)) * D + 32 * bj + yi] = acc[r];
    }
  } else {
#pragma unroll
    for (int g = 0; g < kGroups; ++g) load_group(0, g);
    for (int e = tid; e < m4; e += 256)
      mrs[e] = (e < m) ? make_float2(mu[p * m + e], rs[p * m + e]) : make_float2(0.f, 0.f);
    const float* yp = y + (size_t)p * m * D;
    for (int e = tid; e < m4 * D; e += 256) yl[e] = (e < m * D) ? yp[e] : 0.f;
  }
  __syncthreads();

  f32x4 acc[4][DB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < m4; c0 += 4 * kGroups) {
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      if (c0 + 4 * g < m4) {
        const int j = c0 + 4 * g + lk;
        const float2 s = mrs[j];
        float yb[DB];
        if constexpr (DB == 4) {
          const float4 t = *reinterpret_cast<const float4*>(yl + j * D + 4 * li);
          yb[0] = t.x; yb[1] = t.y; yb[2] = t.z; yb[3] = t.w;
        } else {
          const float2 t = *reinterpret_cast<const float2*>(yl + j * D + 2 * li);
          yb[0] = t.x; yb[1] = t.y;
        }
        const uint32_t mk = lane_mask(tok_ok && j < m);
        const float c4[4] = {masked(cr[g].x, mk), masked(cr[g].y, mk), masked(cr[g].z, mk), masked(cr[g].w, mk)};
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          // Landmarks past m have mu = 1/sigma = 0 and a zero C value: z = 0.
          const float za = (c4[a] - s.x) * s.y;
#pragma unroll
          for (int b = 0; b < DB; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(za, yb[b], acc[a][b], 0, 0, 0);
        }
        if constexpr (!FUSED_Y) {
          if (c0 + 4 * kGroups + 4 * g < m4) load_group(c0 + 4 * kGroups, g);
        }
      }
    }
  }

  // acc[a][b][r] = O[token tb + 4 (4 lk + r) + a][feature DB li + b]
  using V = typename OutVec<D>::type;
  float* op = out + (size_t)p * N * D + DB * li;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int tok = tb + 16 * lk + 4 * r + a;
      if (tok < N) {
        V o;
        if constexpr (DB == 4) {
          o = make_float4(acc[a][0][r], acc[a][1][r], acc[a][2][r], acc[a][3][r]);
        } else {
          o = make_float2(acc[a][0][r], acc[a][1][r]);
        }
        *reinterpret_cast<V*>(op + (size_t)tok * D) = o;
      }
    }
}

template <int D, bool FUSED_Y>
hipError_t launch_typed(const Plan& pl, const Work& wk, float* out, hipStream_t s, Span t) {
  const int m4 = (pl.m + 3) & ~3;
  // yl, then the (mu, 1/sigma) pairs (64 of them in the fused form, so that
  // the prologue's X and B V buffers start at a fixed offset).
  const size_t floats = FUSED_Y ? (size_t)64 * D + 2 * 64 + 64 * kXLD + 64 * D : (size_t)m4 * D + 2 * m4;
  const size_t shmem = floats * sizeof(float);
  auto kern = output_kernel<D, FUSED_Y>;
  if (shmem > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  hipExtLaunchKernelGGL(kern, dim3((pl.N + 255) / 256, pl.P), dim3(256), shmem, s, t.start, t.stop, 0, wk.ct, pl.ldc,
                        wk.x_final, pl.mp,
                     wk.bv, wk.y, wk.mu, wk.rs, out, pl.N, pl.m);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_output(const Plan& pl, const Work& wk, float* out, hipStream_t s, Span t) {
  if (pl.fused_ns) {
    if (pl.d == 64) return launch_typed<64, true>(pl, wk, out, s, t);
    return launch_typed<32, true>(pl, wk, out, s, t);
  }
  if (pl.d == 64) return launch_typed<64, false>(pl, wk, out, s, t);
  return launch_typed<32, false>(pl, wk, out, s, t);
}

}  // namespace lapnys
