// Fused L1-distance + exponential stage: the kernel matrices C = k(Q, K~) and
// B = k(K~, K) with k(x, y) = exp(-||x - y||_1 / lambda) (EN page, section
// 2.A; the pages' own implementation fuses the distance with the exponential,
// EN section 2.C.3 and ZH section 2.2), plus everything that needs C or B
// while it is on chip:
//   * C is written once to the workspace, landmark-major (C^T, [m][N] per
//     problem), for the output stage;
//   * per token tile and landmark: the sum of C and the sum of squared
//     deviations from the tile mean (whitening statistics, EN section 2.B);
//   * B V partial products over each tile group, on fp32 MFMA.  B itself
//     never leaves the chip.
// The partials are reduced by the finalize stage (finalize.hip).
//
// Layout of the work: one lane per token.  A workgroup of 256 lanes takes a
// tile of 256 consecutive tokens of one problem and a block of landmarks.  A
// landmark row is spread over the 16 lanes of each DPP row and reaches every
// lane through a row_newbcast source operand, so the inner loop is pure VALU:
// one subtract (with the broadcast folded in) and one add with an |.| source
// modifier per (token, landmark, feature), and one 16-byte load per lane feeds
// a whole landmark row.  This stage is not a dense contraction; it runs on the
// vector ALUs, not on MFMA.
//
// LDS per workgroup: a tile buffer [lb + 1][256 + 2] (the extra row is zero) that
// holds C, then B, transposed (landmark-major) so that the statistics pass and
// the C store are coalesced and the MFMA reads B columns without bank
// conflicts.
#include "lapnys_internal.hpp"
#include "ns_small.hpp"

namespace lapnys {

namespace {

constexpr int kTT = 256;        // tokens per tile = lanes per workgroup
constexpr int kTP = kTT + 4;    // tile buffer row stride (floats; rows stay 16-byte aligned)
constexpr int kNW = kTT / 64;   // wavefronts per workgroup

// A token row held as raw 16-byte words: issued early, widened later.
template <typename T, int D>
struct RawRow {
  static constexpr int kWords = D * (int)sizeof(T) / 16;
  uint4 w[kWords];
};

template <typename T, int D>
__device__ __forceinline__ void issue_row(const T* __restrict__ src, bool valid, RawRow<T, D>& r) {
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
  for (int c = 0; c < RawRow<T, D>::kWords; ++c) r.w[c] = valid ? s4[c] : make_uint4(0u, 0u, 0u, 0u);
}

template <int D>
__device__ __forceinline__ void widen_row(const RawRow<float, D>& r, float (&x)[D]) {
#pragma unroll
  for (int c = 0; c < D / 4; ++c) {
    x[4 * c + 0] = __uint_as_float(r.w[c].x);
    x[4 * c + 1] = __uint_as_float(r.w[c].y);
    x[4 * c + 2] = __uint_as_float(r.w[c].z);
    x[4 * c + 3] = __uint_as_float(r.w[c].w);
  }
}

template <int D>
__device__ __forceinline__ void widen_row(const RawRow<uint16_t, D>& r, float (&x)[D]) {
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const uint32_t w4[4] = {r.w[c].x, r.w[c].y, r.w[c].z, r.w[c].w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      x[8 * c + 2 * h + 0] = __uint_as_float(w4[h] << 16);
      x[8 * c + 2 * h + 1] = __uint_as_float(w4[h] & 0xffff0000u);
    }
  }
}

// Half of the V operand of the B V MFMA for one tile, per lane:
// V[t0 + 64 lk + s][col] for the kTT/8 steps s of half h (s in [32h, 32h+32)).
// (Step s of lane group lk takes token 64 lk + s of the tile: every token is
// summed exactly once, and one lane's B values for four consecutive steps are
// contiguous in LDS.)  Tokens past N read the last token's row (their B column
// is zero).  Each half is issued well before its MFMAs.
template <typename T, int D>
struct VHalf {
  T w[kTT / 8];
  __device__ __forceinline__ void issue(const T* __restrict__ vcol, int t0, int lk, int h, int tok_last) {
#pragma unroll
    for (int i = 0; i < kTT / 8; ++i) w[i] = vcol[min(t0 + 64 * lk + 32 * h + i, tok_last) * D];
  }
  __device__ __forceinline__ float get(int i) const { return widen(w[i]); }
};

// Where each of the four landmarks of a group reads its features from:
// kLds = broadcast reads of the block's landmark rows staged in LDS (every
// lane reads the same 16 bytes); kSgpr = scalar loads of the rows in global
// memory (wave-uniform addresses), feeding the subtract as an SGPR operand.
// Both leave the VALU free to dual-issue from two wavefronts (a DPP-broadcast
// operand does not).  Scalar loads are as fast when the scalar cache holds
// the rows, but workgroups of different problems sharing a CU evict each
// other's rows, so every landmark reads from LDS.
constexpr int kLds = 0, kSgpr = 1;
constexpr int kSrc[4] = {kLds, kLds, kLds, kLds};

// tl[j][col] = exp2(scale * sum_t |x[t] - k_j[t]|) for the lb landmarks of the
// block (0 for a lane past the last token).  kl: the block's landmark rows in
// LDS; kg: the same rows in global memory.  Four landmarks at a time, each
// with two partial sums (even / odd features), give eight independent add
// chains; the operands of the next 4-feature chunk are loaded while the
// current chunk is summed, and the compiler barriers keep that shape.
template <int D>
__device__ __forceinline__ void kernel_row(const float (&x)[D], const float* __restrict__ kl,
                                           const float* __restrict__ kg, int lb, float scale, float* __restrict__ tl,
                                           int col, bool valid) {
  int j = 0;
  for (; j + 4 <= lb; j += 4) {
    float sa[4] = {0.f, 0.f, 0.f, 0.f}, sb[4] = {0.f, 0.f, 0.f, 0.f};
    float4 kv[2][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      kv[0][u] = *reinterpret_cast<const float4*>((kSrc[u] == kLds ? kl : kg) + (j + u) * D);
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const int cur = c & 1;
      if (c + 1 < D / 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          kv[cur ^ 1][u] = *reinterpret_cast<const float4*>((kSrc[u] == kLds ? kl : kg) + (j + u) * D + 4 * (c + 1));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sa[u] += fabsf(x[4 * c + 0] - kv[cur][u].x);
        sb[u] += fabsf(x[4 * c + 1] - kv[cur][u].y);
        sa[u] += fabsf(x[4 * c + 2] - kv[cur][u].z);
        sb[u] += fabsf(x[4 * c + 3] - kv[cur][u].w);
      }
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
      const float4 kv = *reinterpret_cast<const float4*>(kl + j * D + t);
      sa += fabsf(x[t + 0] - kv.x);
      sb += fabsf(x[t + 1] - kv.y);
      sa += fabsf(x[t + 2] - kv.z);
      sb += fabsf(x[t + 3] - kv.w);
    }
    tl[j * kTP + col] = valid ? exp2f((sa + sb) * scale) : 0.f;
  }
}

// One workgroup's share of the stage: landmark block jb (lb <= lbmax
// landmarks from j0 = jb * lbmax), tile group g, problem p.  LBB = 16-row
// blocks per landmark block (lbmax rounded up to 16, over 16).  tl: the
// workgroup's LDS, (lbmax + 1) * kTP + lbmax * D floats.
template <typename T, int D, int LBB>
__device__ __forceinline__ void l1exp_body(const T* __restrict__ q, const T* __restrict__ k,
                                           const T* __restrict__ v, const float* __restrict__ kt,
                                           float* __restrict__ ct, float2* __restrict__ stats,
                                           float* __restrict__ bvpart, int N, int ldc, int m, int lbmax, int ntiles,
                                           int tpg, int groups, float scale, int jb, int g, int p,
                                           float* __restrict__ tl) {
  // tl: [lb + 1][kTP], row lb stays zero; then kl: [lb][D], this block's landmark rows
  float* kl = tl + (lbmax + 1) * kTP;

  const int j0 = jb * lbmax;
  const int lb = min(lbmax, m - j0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  const float* kg = kt + ((size_t)p * m + j0) * D;  // this block's K~ rows
  for (int e = lb * kTP + tid; e < (lb + 1) * kTP; e += kTT) tl[e] = 0.f;
  for (int e = tid; e < lb * D; e += kTT) kl[e] = kg[e];
  const int li = lane & 15, lk = lane >> 4;

  // B V output blocks (16 x 16) of this wavefront: one 16-feature column block
  // bt0 and BIW of the LBB 16-row landmark blocks, starting at bi0.  When the
  // row blocks do not split evenly, a wavefront's last block may lie past
  // LBB: it reads a valid (zero-padded) row block and is not stored, so every
  // MFMA issues unconditionally.
  constexpr int DB = D / 16;
  static_assert(kNW % DB == 0, "wavefronts must cover the feature blocks");
  constexpr int SPLIT = kNW / DB;
  constexpr int BIW = (LBB + SPLIT - 1) / SPLIT;
  const int bt0 = w % DB;
  const int bi0 = (w / DB) * BIW;
  f32x4 acc[BIW];
#pragma unroll
  for (int a = 0; a < BIW; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t prob = (size_t)p * N * D;
  const int tile_begin = g * tpg;
  const int tile_end = min(ntiles, tile_begin + tpg);
  // Lane li of row block bi reads landmark row 16 bi + li, or the zero row lb
  // past the block's landmarks.
  const float* arow[BIW];
#pragma unroll
  for (int a = 0; a < BIW; ++a) arow[a] = tl + min(16 * min(bi0 + a, LBB - 1) + li, lb) * kTP + 64 * lk;
  const T* vcol = v + prob + 16 * bt0 + li;
  const int tok_last = N - 1;

  float x[D];
  RawRow<T, D> raw;
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    const int t0 = tile * kTT;
    const int nvalid = min(kTT, N - t0);
    const bool valid = tid < nvalid;
    const size_t row = prob + (size_t)(t0 + (valid ? tid : 0)) * D;

    // ---- C = k(Q, K~) ----
    issue_row<T, D>(q + row, valid, raw);
    widen_row<D>(raw, x);
    __syncthreads();  // tile buffer free (previous tile's MFMA reads done)
    kernel_row<D>(x, kl, kg, lb, scale, tl, tid, valid);
    __syncthreads();

    // The key row and this lane's V operands are issued now and arrive while
    // the statistics pass runs.
    issue_row<T, D>(k + row, valid, raw);
    VHalf<T, D> v0;
    v0.issue(vcol, t0, lk, 0, tok_last);

    // ---- column statistics of C over the tile, and the C^T store ----
    // Wavefront w takes landmarks w, w + 4, ..., four of them at a time so
    // that their wavefront reductions overlap.
    for (int jq = w; jq < lb; jq += 4 * kNW) {
      float vals[4][kTT / 64];
      float s[4], m2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jj = min(jq + kNW * u, lb - 1);  // rows past lb: read, not stored
        s[u] = 0.f;
#pragma unroll
        for (int c = 0; c < kTT / 64; ++c) {
          const int col = lane + 64 * c;
          vals[u][c] = tl[jj * kTP + col];
          if (col < nvalid) s[u] += vals[u][c];
        }
      }
      wave_sum_dpp_n<4>(s);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float mean = s[u] / (float)nvalid;
        m2[u] = 0.f;
#pragma unroll
        for (int c = 0; c < kTT / 64; ++c) {
          const int col = lane + 64 * c;
          if (col < nvalid) {
            const float dv = vals[u][c] - mean;
            m2[u] += dv * dv;
          }
        }
      }
      wave_sum_dpp_n<4>(m2);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = jq + kNW * u;
        if (j < lb) {
          if (lane == 0) stats[((size_t)p * ntiles + tile) * m + j0 + j] = make_float2(s[u], m2[u]);
          float* crow = ct + ((size_t)p * m + j0 + j) * ldc + t0;
#pragma unroll
          for (int c = 0; c < kTT / 64; ++c) {
            const int col = lane + 64 * c;
            if (col < nvalid) crow[col] = vals[u][c];
          }
        }
      }
    }

    // ---- B = k(K~, K), kept on chip ----
    widen_row<D>(raw, x);
    __syncthreads();  // statistics pass done with the tile buffer
    kernel_row<D>(x, kl, kg, lb, scale, tl, tid, valid);
    __syncthreads();

    // ---- B V partial: acc[landmark][feature] += sum over the tile's tokens ----
    // fp32 MFMA 16x16x4: lane l supplies A[l%16][l/16] = B[landmark][token] and
    // B[l/16][l%16] = V[token][feature], token = 64 (l/16) + step.  A lane's B
    // values for four steps are one 16-byte LDS read; the first half of V is
    // already in registers and the second half lands during the first half's
    // MFMAs; tile-buffer rows past the block's landmarks are zero.
    VHalf<T, D> v1;
    v1.issue(vcol, t0, lk, 1, tok_last);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const VHalf<T, D>& vh = h ? v1 : v0;
#pragma unroll
      for (int i = 0; i < kTT / 8; i += 4) {
        float4 av[BIW];
#pragma unroll
        for (int a = 0; a < BIW; ++a) av[a] = *reinterpret_cast<const float4*>(arow[a] + 32 * h + i);
#pragma unroll
        for (int a = 0; a < BIW; ++a) {
          acc[a] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a].x, vh.get(i + 0), acc[a], 0, 0, 0);
          acc[a] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a].y, vh.get(i + 1), acc[a], 0, 0, 0);
          acc[a] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a].z, vh.get(i + 2), acc[a], 0, 0, 0);
          acc[a] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a].w, vh.get(i + 3), acc[a], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Partial B V of this tile group: rows j0 + [0, lb) of bvpart[p][g].
  float* bvp = bvpart + ((size_t)p * groups + g) * m * D;
#pragma unroll
  for (int a = 0; a < BIW; ++a) {
    const int r0 = 16 * (bi0 + a);
    if (bi0 + a >= LBB) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = r0 + 4 * lk + r;
      if (rr < lb) bvp[(size_t)(j0 + rr) * D + 16 * bt0 + li] = acc[a][r];
    }
  }

}

// The stage's launch.  For m <= 64 (KS > 0) the first nns workgroups each run
// one problem's Newton-Schulz schedule (ns_small.hpp) and the rest the
// kernel-matrix work, so the two share the machine without a second stream or
// any cross-stream wait: workgroups start in index order, the solver's first,
// and the workgroups [gap, gap + nns) that would share a CU with them exit at
// once.  Grid: nns + jblocks * groups * P workgroups (plus nns empty ones),
// the kernel-matrix ones numbered landmark block fastest, then tile group,
// then problem.
// Dynamic LDS: the larger of the two parts' needs, 16-byte aligned.  The
// register budget of the union of both parts is held to three wavefronts per
// SIMD (the L1 loop needs at least two to dual-issue).
template <typename T, int D, int LBB, int KS>
__global__ __launch_bounds__(kTT) void l1exp_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ kt,
    float* __restrict__ ct, float2* __restrict__ stats, float* __restrict__ bvpart, float* __restrict__ wout,
    float* __restrict__ xout, int N, int ldc, int m, int lbmax, int ntiles, int tpg, int groups, int jblocks,
    float scale, float eps, int iters, int nns, int gap) {
  extern __shared__ __align__(16) float lds[];
  int b = blockIdx.x;
  if constexpr (KS > 0) {
    if (b < nns) {
      ns_detail::ns_small<D, KS>(kt, wout, xout, m, scale, eps, iters, b, lds);
      return;
    }
    // Workgroups [gap, gap + nns) do nothing (see launch_kernel).
    if (b >= gap && b < gap + nns) return;
    b -= b >= gap ? 2 * nns : nns;
  }
  const int jb = b % jblocks, g = (b / jblocks) % groups, p = b / (jblocks * groups);
  l1exp_body<T, D, LBB>(q, k, v, kt, ct, stats, bvpart, N, ldc, m, lbmax, ntiles, tpg, groups, scale, jb, g, p, lds);
}

// CUs of the current device (queried once per device; 0 if unknown).
int cu_count() {
  static int cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

template <typename T, int D, int LBB, int KS>
hipError_t launch_kernel(const Plan& pl, const void* q, const void* k, const void* v, Work& w, hipStream_t s,
                         Span t) {
  const int lbmax = pl.lb;
  size_t floats = (size_t)(lbmax + 1) * kTP + (size_t)lbmax * D;
  if (KS > 0 && floats < (size_t)ns_detail::kNsLdsFloats) floats = ns_detail::kNsLdsFloats;
  const size_t shmem = floats * sizeof(float);
  auto kern = l1exp_kernel<T, D, LBB, KS>;
  if (shmem > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  // Workgroups are placed on the CUs in index order, one per CU per round, so
  // workgroup i and workgroup i + (CU count) share a CU.  The second-round
  // workgroups that would land beside the solver workgroups (ids cus .. cus +
  // nns - 1) exit at once: a kernel-matrix workgroup there would only get the
  // issue slots the solver leaves, and finish last.  (If the placement differs,
  // only the balance changes.)
  const int nns = KS > 0 ? pl.P : 0;
  long long grid = (long long)nns + (long long)pl.jblocks * pl.groups * pl.P;
  int gap = 0x7fffffff;
  if (nns > 0) {
    const int cus = cu_count();
    if (cus > 0 && nns <= cus && grid > cus) {
      gap = cus;
      grid += nns;
    }
  }
  hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kTT), shmem, s, t.start, t.stop, 0, (const T*)q,
                        (const T*)k, (const T*)v, w.kt, w.ct, reinterpret_cast<float2*>(w.stats), w.bvpart, w.w,
                        w.x, pl.N, pl.ldc, pl.m, lbmax, pl.ntiles, pl.tpg, pl.groups, pl.jblocks, pl.scale, pl.eps,
                        pl.ns_iters, nns, gap);
  if (KS > 0) w.x_final = w.x;
  return hipGetLastError();
}

// m <= 64: the Newton-Schulz step count KS = ceil(m / 4) and the landmark
// row blocks LBB = ceil(m / 16) are compile-time constants.
template <typename T, int D, int KS = 1>
hipError_t launch_fused(const Plan& pl, const void* q, const void* k, const void* v, Work& w, hipStream_t s,
                        Span t) {
  if constexpr (KS < 16) {
    if ((pl.m + 3) / 4 > KS) return launch_fused<T, D, KS + 1>(pl, q, k, v, w, s, t);
  }
  return launch_kernel<T, D, (KS + 3) / 4, KS>(pl, q, k, v, w, s, t);
}

template <typename T, int D>
hipError_t launch_typed(const Plan& pl, const void* q, const void* k, const void* v, Work& w, hipStream_t s,
                        Span t) {
  if (pl.fused_ns) return launch_fused<T, D>(pl, q, k, v, w, s, t);
  // m > 64: landmark blocks of 32 (two row blocks); the solver runs on its own.
  return launch_kernel<T, D, 2, 0>(pl, q, k, v, w, s, t);
}

}  // namespace

hipError_t launch_l1exp(const Plan& pl, const void* q, const void* k, const void* v, Work& w,
                        hipStream_t s, Span t) {
  if (pl.dtype == 1) {
    if (pl.d == 64) return launch_typed<uint16_t, 64>(pl, q, k, v, w, s, t);
    return launch_typed<uint16_t, 32>(pl, q, k, v, w, s, t);
  }
  if (pl.d == 64) return launch_typed<float, 64>(pl, q, k, v, w, s, t);
  return launch_typed<float, 32>(pl, q, k, v, w, s, t);
}

}  // namespace lapnys
