// Fused L1-distance + exponential stage: the kernel matrices C = k(Q, K~) and
// B = k(K~, K) with k(x, y) = exp(-||x - y||_1 / lambda) (EN page, section
// 2.A; the pages' own implementation fuses the distance with the exponential,
// EN section 2.C.3 and ZH section 2.2), plus everything that needs C or B
// while it is on chip:
//   * C is written once to the workspace, landmark-major (C^T, [m][N] per
//     problem), for the output stage;
//   * per token tile and landmark: the sum of C and the sum of squared
//     deviations from the tile mean (whitening statistics, EN section 2.B);
//   * B V partial products over the tile, on fp32 MFMA.  B itself never
//     leaves the chip.
//
// Layout of the work: one lane per token.  A workgroup of 256 lanes takes a
// tile of 256 consecutive tokens of one problem and a block of landmarks whose
// K~ rows sit in LDS; every landmark value is read by a wave-uniform LDS
// address (a broadcast), so the inner loop is pure VALU: one subtract and one
// add with an |.| source modifier per (token, landmark, feature).  This stage
// is not a dense contraction; it runs on the vector ALUs, not on MFMA.
//
// LDS per workgroup: K~ block [lb][D] and a tile buffer [lb][256 + 2] that
// holds C, then B, transposed (landmark-major) so that the statistics pass and
// the C store are coalesced and the MFMA reads B columns without bank
// conflicts.
#include "lapnys_internal.hpp"

namespace lapnys {

namespace {

constexpr int kTT = 256;        // tokens per tile = lanes per workgroup
constexpr int kTP = kTT + 2;    // tile buffer row stride (floats)
constexpr int kNW = kTT / 64;   // wavefronts per workgroup

template <int D>
__device__ __forceinline__ void load_row(const float* __restrict__ src, bool valid, float (&x)[D]) {
  if (valid) {
    const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const float4 u = s4[c];
      x[4 * c + 0] = u.x;
      x[4 * c + 1] = u.y;
      x[4 * c + 2] = u.z;
      x[4 * c + 3] = u.w;
    }
  } else {
#pragma unroll
    for (int t = 0; t < D; ++t) x[t] = 0.f;
  }
}

template <int D>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ src, bool valid, float (&x)[D]) {
  if (valid) {
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const uint4 u = s4[c];
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        x[8 * c + 2 * h + 0] = __uint_as_float(w4[h] << 16);
        x[8 * c + 2 * h + 1] = __uint_as_float(w4[h] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < D; ++t) x[t] = 0.f;
  }
}

// tl[j][col] = exp2(scale * sum_t |x[t] - kl[j][t]|) for the lb landmarks of the
// block (0 for a lane past the last token).  Two partial sums per landmark
// (even / odd features) and four landmarks at a time give eight independent
// add chains.  The K~ values are broadcast-read from LDS one 4-feature chunk
// ahead of their use (double buffer); the compiler barriers keep the
// compiler from hoisting every load of the unrolled loop, which would cost
// more registers than the loop has.
template <int D>
__device__ __forceinline__ void kernel_row(const float (&x)[D], const float* kl, int lb, float scale,
                                           float* __restrict__ tl, int col, bool valid) {
  int j = 0;
  for (; j + 4 <= lb; j += 4) {
    float sa[4] = {0.f, 0.f, 0.f, 0.f}, sb[4] = {0.f, 0.f, 0.f, 0.f};
    float4 kv[2][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) kv[0][u] = *reinterpret_cast<const float4*>(&kl[(j + u) * D]);
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const int cur = c & 1;
      if (c + 1 < D / 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) kv[cur ^ 1][u] = *reinterpret_cast<const float4*>(&kl[(j + u) * D + 4 * (c + 1)]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sa[u] += fabsf(x[4 * c + 0] - kv[cur][u].x);
        sb[u] += fabsf(x[4 * c + 1] - kv[cur][u].y);
        sa[u] += fabsf(x[4 * c + 2] - kv[cur][u].z);
        sb[u] += fabsf(x[4 * c + 3] - kv[cur][u].w);
      }
      // Accumulators are in/out operands: this chunk's adds finish before the
      // next chunk's loads issue.
      asm volatile("" : "+v"(sa[0]), "+v"(sa[1]), "+v"(sa[2]), "+v"(sa[3]), "+v"(sb[0]), "+v"(sb[1]),
                   "+v"(sb[2]), "+v"(sb[3])::"memory");
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) tl[(j + u) * kTP + col] = valid ? exp2f((sa[u] + sb[u]) * scale) : 0.f;
  }
  for (; j < lb; ++j) {
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int t = 0; t < D; t += 4) {
      const float4 kv = *reinterpret_cast<const float4*>(&kl[j * D + t]);
      sa += fabsf(x[t + 0] - kv.x);
      sb += fabsf(x[t + 1] - kv.y);
      sa += fabsf(x[t + 2] - kv.z);
      sb += fabsf(x[t + 3] - kv.w);
    }
    tl[j * kTP + col] = valid ? exp2f((sa + sb) * scale) : 0.f;
  }
}

// Grid: (landmark block, tile group, problem).  Dynamic LDS: lb*D + lb*kTP floats.
template <typename T, int D>
__global__ __launch_bounds__(kTT) void l1exp_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                    const T* __restrict__ v, const float* __restrict__ kt,
                                                    float* __restrict__ ct, float2* __restrict__ stats,
                                                    float* __restrict__ bvpart, int N, int m, int lbmax, int ntiles,
                                                    int tpg, int groups, float scale) {
  extern __shared__ float4 lds4[];
  float* kl = reinterpret_cast<float*>(lds4);  // [lb][D]
  float* tl = kl + lbmax * D;                   // [lb][kTP]

  const int jb = blockIdx.x, g = blockIdx.y, p = blockIdx.z;
  const int j0 = jb * lbmax;
  const int lb = min(lbmax, m - j0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  const float4* ktp4 = reinterpret_cast<const float4*>(kt + ((size_t)p * m + j0) * D);
  for (int e = tid; e < lb * D / 4; e += kTT) lds4[e] = ktp4[e];

  // B V output blocks (16 x 16) of this wavefront: rows are landmarks of the
  // block (up to 64, four 16-row blocks), columns are features (D/16 blocks).
  constexpr int DB = D / 16;
  constexpr int BTW = (kNW <= DB) ? DB / kNW : 1;
  constexpr int BIW = (kNW <= DB) ? 4 : 4 / (kNW / DB);
  const int bt0 = (kNW <= DB) ? w * BTW : (w % DB);
  const int bi0 = (kNW <= DB) ? 0 : (w / DB) * BIW;
  f32x4 acc[BIW][BTW];
#pragma unroll
  for (int a = 0; a < BIW; ++a)
#pragma unroll
    for (int b = 0; b < BTW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t prob = (size_t)p * N * D;
  const int tile_begin = g * tpg;
  const int tile_end = min(ntiles, tile_begin + tpg);
  float x[D];
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    const int t0 = tile * kTT;
    const int nvalid = min(kTT, N - t0);
    const bool valid = tid < nvalid;
    const size_t row = prob + (size_t)(t0 + (valid ? tid : 0)) * D;

    // ---- C = k(Q, K~) ----
    load_row<D>(q + row, valid, x);
    __syncthreads();  // K~ staged (first tile); tile buffer free (later tiles)
    kernel_row<D>(x, kl, lb, scale, tl, tid, valid);
    __syncthreads();
    for (int j = w; j < lb; j += kNW) {
      float vals[kTT / 64];
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < kTT / 64; ++c) {
        const int col = lane + 64 * c;
        vals[c] = tl[j * kTP + col];
        if (col < nvalid) s += vals[c];
      }
      s = wave_sum(s);
      const float mean = s / (float)nvalid;
      float m2 = 0.f;
#pragma unroll
      for (int c = 0; c < kTT / 64; ++c) {
        const int col = lane + 64 * c;
        if (col < nvalid) {
          const float dv = vals[c] - mean;
          m2 += dv * dv;
        }
      }
      m2 = wave_sum(m2);
      if (lane == 0) stats[((size_t)p * ntiles + tile) * m + j0 + j] = make_float2(s, m2);
      float* crow = ct + ((size_t)p * m + j0 + j) * N + t0;
#pragma unroll
      for (int c = 0; c < kTT / 64; ++c) {
        const int col = lane + 64 * c;
        if (col < nvalid) crow[col] = vals[c];
      }
    }

    // ---- B = k(K~, K), kept on chip ----
    load_row<D>(k + row, valid, x);
    __syncthreads();  // statistics pass done with the tile buffer
    kernel_row<D>(x, kl, lb, scale, tl, tid, valid);
    __syncthreads();

    // ---- B V partial: acc[landmark][feature] += sum over the tile's tokens ----
    // fp32 MFMA 16x16x4: lane l supplies A[l%16][l/16] = B[landmark][token] and
    // B[l/16][l%16] = V[token][feature]; four tokens per step.
    const int li = lane & 15, lk = lane >> 4;
#pragma unroll 8
    for (int s4 = 0; s4 < kTT / 4; ++s4) {
      const int tk = 4 * s4 + lk;
      const int tok = t0 + tk;
      float bv[BTW];
#pragma unroll
      for (int b = 0; b < BTW; ++b)
        bv[b] = (tok < N) ? widen(v[prob + (size_t)tok * D + 16 * (bt0 + b) + li]) : 0.f;
#pragma unroll
      for (int a = 0; a < BIW; ++a) {
        const int r0 = 16 * (bi0 + a);
        if (r0 < lb) {
          const float av = (r0 + li < lb) ? tl[(r0 + li) * kTP + tk] : 0.f;
#pragma unroll
          for (int b = 0; b < BTW; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv[b], acc[a][b], 0, 0, 0);
        }
      }
    }
  }

  // Partial B V of this tile group: rows j0 + [0, lb) of bvpart[p][g].
  float* bvp = bvpart + ((size_t)p * groups + g) * m * D;
  const int li = lane & 15, lk = lane >> 4;
#pragma unroll
  for (int a = 0; a < BIW; ++a) {
    const int r0 = 16 * (bi0 + a);
    if (r0 >= lb) continue;
#pragma unroll
    for (int b = 0; b < BTW; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = r0 + 4 * lk + r;
        if (rr < lb) bvp[(size_t)(j0 + rr) * D + 16 * (bt0 + b) + li] = acc[a][b][r];
      }
  }
}

template <typename T, int D>
hipError_t launch_typed(const Plan& pl, const void* q, const void* k, const void* v, const float* kt, float* ct,
                        float* stats, float* bvpart, hipStream_t s) {
  const int lbmax = pl.lb;
  const size_t shmem = (size_t)(lbmax * D + lbmax * kTP) * sizeof(float);
  auto kern = l1exp_kernel<T, D>;
  if (shmem > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(pl.jblocks, pl.groups, pl.P), dim3(kTT), shmem, s, (const T*)q, (const T*)k,
                     (const T*)v, kt, ct, reinterpret_cast<float2*>(stats), bvpart, pl.N, pl.m, lbmax, pl.ntiles,
                     pl.tpg, pl.groups, pl.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_l1exp(const Plan& pl, const void* q, const void* k, const void* v, const float* kt, float* ct,
                        float* stats, float* bvpart, hipStream_t s) {
  if (pl.dtype == 1) {
    if (pl.d == 64) return launch_typed<uint16_t, 64>(pl, q, k, v, kt, ct, stats, bvpart, s);
    return launch_typed<uint16_t, 32>(pl, q, k, v, kt, ct, stats, bvpart, s);
  }
  if (pl.d == 64) return launch_typed<float, 64>(pl, q, k, v, kt, ct, stats, bvpart, s);
  return launch_typed<float, 32>(pl, q, k, v, kt, ct, stats, bvpart, s);
}

}  // namespace lapnys
