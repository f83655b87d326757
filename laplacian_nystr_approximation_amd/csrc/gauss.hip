// Gaussian-kernel form of the kernel-matrix stage: C = k(Q, K~) and
// B = k(K~, K) with k(x, y) = exp(-||x - y||_2^2 / lambda), the kernel the
// Laplacian one replaces (EN page, section 1, first flaw; section 2.A puts the
// L1 distance in its place).  Everything after the kernel values (statistics,
// C^T store, B V partials) is the Laplacian stage's (kmat_tile.hpp), so the
// reductions, the solver and the output stage serve both kernels unchanged.
//
// Unlike the L1 distance, the squared L2 distance is a dense contraction:
//   ||x - y||^2 = ||x||^2 + ||y||^2 - 2 x . y,
// so each tile's 256 x lb dot products run on fp32 MFMA 16x16x4 (float32
// products and sums, as the Laplacian stage uses), and only the norms, the
// combination and the exponential are vector work.  The combination can round
// below zero for nearly equal points; it is clamped at 0.
//
// Work layout: wavefront w takes tokens t0 + 64 w + [0, 64) of the tile as
// four 16-token column blocks and the block's landmarks as LBB 16-row blocks,
// LBB x 4 accumulator tiles.  The reduction index of the MFMA is a permutation
// of the features: lane group lk holds features [D/4 lk, D/4 (lk + 1)) of its
// tokens, read as contiguous 16-byte loads, and the landmark operand is read
// from LDS in the same order, so every product pairs equal features.
#include "kmat_tile.hpp"
#include "lapnys_internal.hpp"

namespace lapnys {

namespace {

using namespace kmat;

// The features of each of a lane's four tokens that it holds, and the number
// of raw 16-byte words they take.
template <typename T, int D>
struct TokenSlice {
  static constexpr int kF = D / 4;
  static constexpr int kWords = kF * (int)sizeof(T) / 16;
  uint4 raw[4][kWords];
  float f[4][kF];
  float norm[4];  // ||row||^2 over all D features, the same in the four lane groups

  // Token rows tok_base + 16 bt (bt < 4) of src (row stride D), features
  // [kF lk, kF lk + kF); rows past tok_last read the last row.
  __device__ __forceinline__ void issue(const T* __restrict__ src, int tok_base, int tok_last, int lk) {
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) {
      const uint4* s4 = reinterpret_cast<const uint4*>(src + (size_t)min(tok_base + 16 * bt, tok_last) * D + kF * lk);
#pragma unroll
      for (int c = 0; c < kWords; ++c) raw[bt][c] = s4[c];
    }
  }

  __device__ __forceinline__ void widen_and_norm() {
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) {
#pragma unroll
      for (int c = 0; c < kWords; ++c) {
        const uint32_t w4[4] = {raw[bt][c].x, raw[bt][c].y, raw[bt][c].z, raw[bt][c].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          if constexpr (sizeof(T) == 4) {
            f[bt][4 * c + h] = __uint_as_float(w4[h]);
          } else {
            f[bt][8 * c + 2 * h + 0] = __uint_as_float(w4[h] << 16);
            f[bt][8 * c + 2 * h + 1] = __uint_as_float(w4[h] & 0xffff0000u);
          }
        }
      }
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < kF; ++e) s = fmaf(f[bt][e], f[bt][e], s);
      norm[bt] = s;
    }
    // Sum over the four lane groups (lanes li, li + 16, li + 32, li + 48):
    // (g0 + g1) + (g2 + g3) in every group, bit for bit.
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) norm[bt] += __shfl_xor(norm[bt], 16, 64);
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) norm[bt] += __shfl_xor(norm[bt], 32, 64);
  }
};

// The kernel values of one tile for this wavefront's 64 tokens: acc[bj][bt]
// = K~ rows 16 bj + [0, 16) dotted with tokens 16 bt + [0, 16), then
// exp2(scale * max(||x||^2 + ||k||^2 - 2 x.k, 0)) into the tile buffer: float32
// rows of stride kTP (SPLIT false), or bf16 high parts and, rows further on,
// low parts of stride kRB (SPLIT true) plus the zero row lb.  Rows past lb are
// computed (from zero-filled landmark rows) and not written; tokens past N
// are written as 0.
template <typename T, int D, int LBB, bool SPLIT>
__device__ __forceinline__ void gauss_rows(const TokenSlice<T, D>& x, const float* __restrict__ kl,
                                           const float* __restrict__ kn, int lb, int rows, float scale,
                                           float* __restrict__ tl, int w, int lane, int nvalid) {
  constexpr int kF = D / 4;
  constexpr int kKS = D + 4;
  const int li = lane & 15, lk = lane >> 4;
  f32x4 acc[LBB][4];
#pragma unroll
  for (int bj = 0; bj < LBB; ++bj)
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) acc[bj][bt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s4 = 0; s4 < kF / 4; ++s4) {
    f32x4 a[LBB];
#pragma unroll
    for (int bj = 0; bj < LBB; ++bj)
      a[bj] = *reinterpret_cast<const f32x4*>(kl + (16 * bj + li) * kKS + kF * lk + 4 * s4);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int bj = 0; bj < LBB; ++bj)
#pragma unroll
        for (int bt = 0; bt < 4; ++bt)
          acc[bj][bt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[bj][e], x.f[bt][4 * s4 + e], acc[bj][bt], 0, 0, 0);
  }
  // acc[bj][bt][r] = landmark 16 bj + 4 lk + r, token 16 bt + li of the wavefront.
#pragma unroll
  for (int bj = 0; bj < LBB; ++bj) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 16 * bj + 4 * lk + r;
      const float knj = kn[j];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const int col = 64 * w + 16 * bt + li;
        const float dist = fmaxf(fmaf(-2.f, acc[bj][bt][r], x.norm[bt] + knj), 0.f);
        const float val = col < nvalid ? exp2f(dist * scale) : 0.f;
        if (j < lb) {
          if constexpr (SPLIT) {
            __bf16* th = reinterpret_cast<__bf16*>(tl);
            const __bf16 hi = (__bf16)val;
            th[j * kRB + col] = hi;
            th[(rows + j) * kRB + col] = (__bf16)(val - (float)hi);
          } else {
            tl[j * kTP + col] = val;
          }
        }
      }
    }
  }
  if constexpr (SPLIT) {
    __bf16* th = reinterpret_cast<__bf16*>(tl);
    th[lb * kRB + 64 * w + lane] = (__bf16)0.f;
    th[(rows + lb) * kRB + 64 * w + lane] = (__bf16)0.f;
  }
}

// One workgroup: landmark block jb (lb <= lbmax landmarks from j0 = jb *
// lbmax), tile group g, problem p; the tiles in order, as the Laplacian
// stage.  LDS: the tile buffer, (lbmax + 1) * kTileRow floats; the block's
// landmark rows, 16 LBB rows of stride D + 4 (rows past lb zero); their
// squared norms, 16 LBB floats.
template <typename T, int D, int LBB>
__global__ __launch_bounds__(kTT) void gauss_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                    const T* __restrict__ v, const float* __restrict__ kt,
                                                    float* __restrict__ ct, float2* __restrict__ stats,
                                                    float* __restrict__ bvpart, int N, int ldc, int m, int lbmax,
                                                    int ntiles, int tpg, int groups, int jblocks, float scale) {
  extern __shared__ __align__(16) float lds[];
  constexpr int kKS = D + 4;
  constexpr int kRows = 16 * LBB;
  float* tl = lds;
  float* kl = tl + (lbmax + 1) * kTileRow;
  float* kn = kl + kRows * kKS;
  const __bf16* bh = reinterpret_cast<const __bf16*>(tl);
  const __bf16* bl = bh + (lbmax + 1) * kRB;

  const int b = blockIdx.x;
  const int jb = b % jblocks, g = (b / jblocks) % groups, p = b / (jblocks * groups);
  const int j0 = jb * lbmax;
  const int lb = min(lbmax, m - j0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  {
    // Landmark rows j0 + [0, kRows) as float4s, rows past lb zero: every load
    // (clamped to a valid row) issued before the first store.
    constexpr int kQ = D / 4;                      // float4s per row
    constexpr int kV = (kRows * kQ + kTT - 1) / kTT;
    const float4* kg4 = reinterpret_cast<const float4*>(kt + ((size_t)p * m + j0) * D);
    float4 kv[kV];
#pragma unroll
    for (int i = 0; i < kV; ++i) {
      const int e = min(tid + kTT * i, kRows * kQ - 1);
      kv[i] = kg4[min(e / kQ, lb - 1) * kQ + e % kQ];
    }
#pragma unroll
    for (int i = 0; i < kV; ++i) {
      const int e = tid + kTT * i;
      if (e < kRows * kQ) {
        const float4 val = e / kQ < lb ? kv[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(kl + (e / kQ) * kKS + 4 * (e % kQ)) = val;
      }
    }
    __syncthreads();
    if (tid < kRows) {
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < D; ++t) s = fmaf(kl[tid * kKS + t], kl[tid * kKS + t], s);
      kn[tid] = s;
    }
  }

  BvTile<T, D, LBB> bv;
  bv.init(w, lane, lb);
  const size_t prob = (size_t)p * N * D;
  const int tile_begin = g * tpg;
  const int tile_end = min(ntiles, tile_begin + tpg);
  const T* vcol = v + prob + 16 * bv.bt0 + bv.li;
  const int tok_last = N - 1;
  const int li = lane & 15, lk = lane >> 4;

  TokenSlice<T, D> x;
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    const int t0 = tile * kTT;
    const int nvalid = min(kTT, N - t0);
    const int tok_base = t0 + 64 * w + li;

    // ---- C = k(Q, K~) ----
    x.issue(q + prob, tok_base, tok_last, lk);
    x.widen_and_norm();
    __syncthreads();  // tile buffer free (previous tile's MFMA reads done); kn ready
    gauss_rows<T, D, LBB, false>(x, kl, kn, lb, lbmax + 1, scale, tl, w, lane, nvalid);
    __syncthreads();

    // The key rows and this lane's V operands are issued now and arrive while
    // the statistics pass runs.
    x.issue(k + prob, tok_base, tok_last, lk);
    VHalf<T, D> v0;
    v0.issue(vcol, t0, bv.lk, 0, tok_last);

    // ---- column statistics of C over the tile, and the C^T store ----
    tile_stats_store(tl, stats, ct, p, ntiles, tile, m, j0, lb, ldc, t0, nvalid, lane, w);

    // ---- B = k(K~, K), kept on chip ----
    x.widen_and_norm();
    __syncthreads();  // statistics pass done with the tile buffer
    gauss_rows<T, D, LBB, true>(x, kl, kn, lb, lbmax + 1, scale, tl, w, lane, nvalid);
    __syncthreads();

    // ---- B V partial ----
    VHalf<T, D> v1;
    v1.issue(vcol, t0, bv.lk, 1, tok_last);
    bv.accumulate(bh, bl, v0, v1);
  }
  bv.store(bvpart + ((size_t)p * groups + g) * m * D, j0, lb);
}

template <typename T, int D, int LBB>
hipError_t launch_lbb(const Plan& pl, const void* q, const void* k, const void* v, Work& w, hipStream_t s, Span t) {
  const size_t floats = (size_t)(pl.lb + 1) * kTileRow + (size_t)16 * LBB * (D + 4) + 16 * LBB;
  const size_t shmem = floats * sizeof(float);
  auto kern = gauss_kernel<T, D, LBB>;
  if (shmem > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  const long long grid = (long long)pl.jblocks * pl.groups * pl.P;
  hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kTT), shmem, s, t.start, t.stop, 0, (const T*)q,
                        (const T*)k, (const T*)v, w.kt, w.ct, reinterpret_cast<float2*>(w.stats), w.bvpart, pl.N,
                        pl.ldc, pl.m, pl.lb, pl.ntiles, pl.tpg, pl.groups, pl.jblocks, pl.scale);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_typed(const Plan& pl, const void* q, const void* k, const void* v, Work& w, hipStream_t s, Span t) {
  switch ((pl.lb + 15) / 16) {
    case 1: return launch_lbb<T, D, 1>(pl, q, k, v, w, s, t);
    case 2: return launch_lbb<T, D, 2>(pl, q, k, v, w, s, t);
    case 3: return launch_lbb<T, D, 3>(pl, q, k, v, w, s, t);
    case 4: return launch_lbb<T, D, 4>(pl, q, k, v, w, s, t);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gauss(const Plan& pl, const void* q, const void* k, const void* v, Work& w, hipStream_t s,
                        Span t) {
  if (!pl.gaussian) return hipErrorInvalidValue;
  if (pl.dtype == 1) {
    return pl.d == 64 ? launch_typed<uint16_t, 64>(pl, q, k, v, w, s, t)
                      : launch_typed<uint16_t, 32>(pl, q, k, v, w, s, t);
  }
  return pl.d == 64 ? launch_typed<float, 64>(pl, q, k, v, w, s, t) : launch_typed<float, 32>(pl, q, k, v, w, s, t);
}

}  // namespace lapnys
