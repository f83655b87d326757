// Fused L1-distance + exponential stage: the kernel matrices C = k(Q, K~) and
// B = k(K~, K) with k(x, y) = exp(-||x - y||_1 / lambda) (EN page, section
// 2.A; the pages' own implementation fuses the distance with the exponential,
// EN section 2.C.3 and ZH section 2.2), plus everything that needs C or B
// while it is on chip:
//   * C is written once to the workspace, landmark-major (C^T, [m][N] per
//     problem), for the output stage;
//   * per token tile and landmark: the sum of C and the sum of squared
//     deviations from the tile mean (whitening statistics, EN section 2.B);
//   * B V partial products over each tile group, on bf16 MFMA with B split
//     into bf16 high and low parts (and V too for float32 inputs; bf16 V is
//     exact).  B itself never leaves the chip.
// The partials are reduced by the finalize stage (finalize.hip).
//
// Layout of the work: one lane per token.  A workgroup of 256 lanes takes a
// tile of 256 consecutive tokens of one problem and a block of landmarks,
// whose rows it stages in LDS.  Every landmark value reaches all 64 lanes of
// a wavefront as a wave-uniform LDS broadcast read (one 16-byte read gives
// four features of one landmark, loaded two 4-feature chunks ahead),
// so the inner loop is one subtract and one add with an |.| source modifier
// per (token, landmark, feature), eight independent sums at a time (four
// landmarks, even and odd features).  This stage is not a dense contraction;
// it runs on the vector ALUs, not on MFMA.
//
// LDS per workgroup: a tile buffer that holds C as float32 [lb][256 + 4], then
// B as bf16 high and low parts [lb + 1][264] each (the extra row is zero),
// both landmark-major, so that the statistics pass and the C store are
// coalesced and the MFMA reads eight tokens of a landmark row as one 16-byte
// access without bank conflicts.
#include "kmat_tile.hpp"
#include "lapnys_internal.hpp"
#include "ns_small.hpp"

namespace lapnys {

namespace {

using namespace kmat;

// Where each of the four landmarks of a group reads its features from:
// kLds = broadcast reads of the block's landmark rows staged in LDS (every
// lane reads the same 16 bytes); kSgpr = scalar loads of the rows in global
// memory (wave-uniform addresses), feeding the subtract as an SGPR operand.
// Both leave the VALU free to dual-issue from two wavefronts (a DPP-broadcast
// operand does not).  Scalar loads are as fast when the scalar cache holds
// the rows, but workgroups of different problems sharing a CU evict each
// other's rows, so every landmark reads from LDS.
constexpr int kLds = 0;
[[maybe_unused]] constexpr int kSgpr = 1;
constexpr int kSrc[4] = {kLds, kLds, kLds, kLds};

// Row j of the tile = exp2(scale * sum_t |x[t] - k_j[t]|) for the lb landmarks
// of the block (0 for a lane past the last token): float32 rows of stride kTP
// at tl, or (SPLIT) bf16 high parts at tl and low parts rows * kRB further,
// rows of stride kRB, followed by a zero row lb.  kl: the block's landmark
// rows in LDS; kg: the same rows in global memory.  Four landmarks at a time, each
// with two partial sums (even / odd features), give eight independent add
// chains; the operands of the next RING - 1 4-feature chunks are in flight
// while the current chunk is summed (with one chunk ahead instead of two the
// 28x28 and 56x56 float32 workloads ran 1-3 % slower; the kernel held to
// three wavefronts per SIMD keeps one, as two spilled more of its
// registers), and the compiler barriers keep that shape.
template <int D, bool SPLIT, int RING = 3>
__device__ __forceinline__ void kernel_row(const float (&x)[D], const float* __restrict__ kl,
                                           const float* __restrict__ kg, int lb, float scale, float* __restrict__ tl,
                                           int rows, int col, bool valid, float* __restrict__ bout = nullptr,
                                           int ldb = 0) {
  auto put = [&](int j, float sum) {
    const float val = valid ? exp2f(sum * scale) : 0.f;
    if constexpr (SPLIT) {
      __bf16* th = reinterpret_cast<__bf16*>(tl);
      const __bf16 hi = (__bf16)val;
      th[j * kRB + col] = hi;
      th[(rows + j) * kRB + col] = (__bf16)(val - (float)hi);
      if (bout != nullptr && valid) bout[(size_t)j * ldb] = val;
    } else {
      tl[j * kTP + col] = val;
    }
  };
  int j = 0;
  for (; j + 4 <= lb; j += 4) {
    float sa[4] = {0.f, 0.f, 0.f, 0.f}, sb[4] = {0.f, 0.f, 0.f, 0.f};
    float4 kv[RING][4];
#pragma unroll
    for (int c0 = 0; c0 < RING - 1; ++c0)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        kv[c0][u] = *reinterpret_cast<const float4*>((kSrc[u] == kLds ? kl : kg) + (j + u) * D + 4 * c0);
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const int cur = c % RING;
      if (c + RING - 1 < D / 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          kv[(c + RING - 1) % RING][u] =
              *reinterpret_cast<const float4*>((kSrc[u] == kLds ? kl : kg) + (j + u) * D + 4 * (c + RING - 1));
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
    for (int u = 0; u < 4; ++u) put(j + u, sa[u] + sb[u]);
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
    put(j, sa + sb);
  }
  if constexpr (SPLIT) {
    __bf16* th = reinterpret_cast<__bf16*>(tl);
    th[lb * kRB + col] = (__bf16)0.f;
    th[(rows + lb) * kRB + col] = (__bf16)0.f;
  }
}

// One workgroup's share of the stage: landmark block jb (lb <= lbmax
// landmarks from j0 = jb * lbmax), tile group g, problem p.  LBB = 16-row
// blocks per landmark block (lbmax rounded up to 16, over 16).  tl: the
// workgroup's LDS, (lbmax + 1) * kTileRow + lbmax * D floats.  PART 0 forms
// both C and B of each tile; PART 1 only C (statistics and the C^T store),
// PART 2 only B (the B V partial; its V operands are then issued after the B
// rows, so they do not hold registers during them).
template <typename T, int D, int LBB, int PART = 0, int RING = 3>
__device__ __forceinline__ void l1exp_body(const T* __restrict__ q, const T* __restrict__ k,
                                           const T* __restrict__ v, const float* __restrict__ kt,
                                           float* __restrict__ ct, float2* __restrict__ stats,
                                           float* __restrict__ bvpart, float* __restrict__ bt, int N, int ldc,
                                           int m, int lbmax, int ntiles, int tpg, int groups, float scale, int jb,
                                           int g, int p, float* __restrict__ tl, unsigned long long* __restrict__ kclk) {
  if (kclk != nullptr && threadIdx.x == 0) atomicMin(kclk, (unsigned long long)wall_clock64());
  // tl: the tile buffer, (lbmax + 1) * kTileRow floats; then kl: [lb][D],
  // this block's landmark rows
  float* kl = tl + (lbmax + 1) * kTileRow;
  const __bf16* bh = reinterpret_cast<const __bf16*>(tl);  // B tile high parts, [lbmax + 1][kRB]
  const __bf16* bl = bh + (lbmax + 1) * kRB;               // low parts

  const int j0 = jb * lbmax;
  const int lb = min(lbmax, m - j0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  const float* kg = kt + ((size_t)p * m + j0) * D;  // this block's K~ rows
  {
    // The block's landmark rows into LDS, every load issued before the first
    // store (lb <= 64 rows, at most four 16-byte loads per lane).
    constexpr int kV = 64 * D / 4 / kTT;
    const int n4 = lb * D / 4;
    const float4* kg4 = reinterpret_cast<const float4*>(kg);
    float4 kv[kV];
#pragma unroll
    for (int i = 0; i < kV; ++i) kv[i] = kg4[min(tid + kTT * i, n4 - 1)];
#pragma unroll
    for (int i = 0; i < kV; ++i)
      if (tid + kTT * i < n4) reinterpret_cast<float4*>(kl)[tid + kTT * i] = kv[i];
  }
  BvTile<T, D, LBB> bv;
  bv.init(w, lane, lb);

  const size_t prob = (size_t)p * N * D;
  const int tile_begin = g * tpg;
  const int tile_end = min(ntiles, tile_begin + tpg);
  const T* vcol = v + prob + 16 * bv.bt0 + bv.li;
  const int tok_last = N - 1;

  float x[D];
  RawRow<T, D> raw;
  for (int tile = tile_begin; tile < tile_end; ++tile) {
    const int t0 = tile * kTT;
    const int nvalid = min(kTT, N - t0);
    const bool valid = tid < nvalid;
    const size_t row = prob + (size_t)(t0 + (valid ? tid : 0)) * D;

    // ---- C = k(Q, K~) ----
    if constexpr (PART != 2) {
      issue_row<T, D>(q + row, valid, raw);
      widen_row<D>(raw, x);
      __syncthreads();  // tile buffer free (previous tile's MFMA reads done)
      kernel_row<D, false, RING>(x, kl, kg, lb, scale, tl, lbmax + 1, tid, valid);
      __syncthreads();
    }
    if constexpr (PART == 1) {
      tile_stats_store(tl, stats, ct, p, ntiles, tile, m, j0, lb, ldc, t0, nvalid, lane, w);
      continue;
    }

    // The key row and this lane's V operands are issued now and arrive while
    // the statistics pass runs.
    issue_row<T, D>(k + row, valid, raw);
    VHalf<T, D> v0;
    if constexpr (PART == 0) v0.issue(vcol, t0, bv.lk, 0, tok_last);

    // ---- column statistics of C over the tile, and the C^T store ----
    if constexpr (PART == 0) tile_stats_store(tl, stats, ct, p, ntiles, tile, m, j0, lb, ldc, t0, nvalid, lane, w);

    // ---- B = k(K~, K), kept on chip ----
    widen_row<D>(raw, x);
    __syncthreads();  // statistics pass done with the tile buffer
    kernel_row<D, true, RING>(x, kl, kg, lb, scale, tl, lbmax + 1, tid, valid,
                        bt != nullptr ? bt + ((size_t)p * m + j0) * N + t0 + tid : nullptr, N);
    __syncthreads();

    // ---- B V partial: acc[landmark][feature] += sum over the tile's tokens ----
    if constexpr (PART == 2) v0.issue(vcol, t0, bv.lk, 0, tok_last);
    VHalf<T, D> v1;
    v1.issue(vcol, t0, bv.lk, 1, tok_last);
    bv.accumulate(bh, bl, v0, v1);
  }

  // Partial B V of this tile group: rows j0 + [0, lb) of bvpart[p][g].
  if constexpr (PART != 1) bv.store(bvpart + ((size_t)p * groups + g) * m * D, j0, lb);
  if (kclk != nullptr && threadIdx.x == 0) atomicMax(kclk + 1, (unsigned long long)wall_clock64());
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
// union of both parts takes 212 registers at d = 64: two wavefronts per SIMD
// (the L1 loop needs at least two to dual-issue).
template <typename T, int D, int LBB, int KS>
__global__ __launch_bounds__(kTT) void l1exp_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ kt,
    float* __restrict__ ct, float2* __restrict__ stats, float* __restrict__ bvpart, float* __restrict__ bt,
    float* __restrict__ wout, float* __restrict__ xout, int N, int ldc, int m, int lbmax, int ntiles, int tpg, int groups, int jblocks,
    float scale, float eps, int iters, int nns, int gap, unsigned long long* __restrict__ nsclk,
    unsigned long long* __restrict__ kclk) {
  extern __shared__ __align__(16) float lds[];
  int b = blockIdx.x;
  if constexpr (KS > 0) {
    if (b < nns) {
      ns_detail::ns_small<D, KS>(kt, wout, xout, m, scale, eps, iters, b, lds, nsclk);
      return;
    }
    // Workgroups [gap, gap + nns) do nothing (see launch_kernel).
    if (b >= gap && b < gap + nns) return;
    b -= b >= gap ? 2 * nns : nns;
  }
  const int jb = b % jblocks, g = (b / jblocks) % groups, p = b / (jblocks * groups);
  l1exp_body<T, D, LBB>(q, k, v, kt, ct, stats, bvpart, bt, N, ldc, m, lbmax, ntiles, tpg, groups, scale, jb, g, p,
                        lds, kclk);
}

// The same launch with the work of each (landmark block, tile group) in two
// workgroups: one forms C (with its statistics and the C^T store), the other
// B (with the B V partial, its V operands loaded after the B rows).  Neither
// holds the other's registers, so the launch fits three wavefronts per SIMD
// (162 registers, the solver's; 53 KB of LDS with the landmarks in two
// blocks), for shapes where the unsplit workgroups would leave most CUs a
// single one (see launch_typed).  Grid: nns + 8 S ceil(units / 8) workgroups
// (plus nns empty ones), S = 2 jblocks, unit u = g + groups p: workgroup b =
// (u / 8) 8 S + 8 sub + u % 8 takes sub = jb + jblocks part of unit u, so
// the S workgroups of a unit run on one XCD and share its L2.
template <typename T, int D, int LBB, int KS>
__global__ __launch_bounds__(kTT) void l1exp_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ kt,
    float* __restrict__ ct, float2* __restrict__ stats, float* __restrict__ bvpart, float* __restrict__ bt,
    float* __restrict__ wout, float* __restrict__ xout, int N, int ldc, int m, int lbmax, int ntiles, int tpg, int groups, int jblocks,
    float scale, float eps, int iters, int nns, int gap, unsigned long long* __restrict__ nsclk,
    unsigned long long* __restrict__ kclk) {
  extern __shared__ __align__(16) float lds[];
  int b = blockIdx.x;
  if constexpr (KS > 0) {
    if (b < nns) {
      ns_detail::ns_small<D, KS>(kt, wout, xout, m, scale, eps, iters, b, lds, nsclk);
      return;
    }
    if (b >= gap && b < gap + nns) return;
    b -= b >= gap ? 2 * nns : nns;
  }
  const int S = 2 * jblocks;
  const int u = (b / (8 * S)) * 8 + b % 8, sub = (b / 8) % S;
  if (u >= groups * nns) return;
  const int jb = sub % jblocks, part = sub / jblocks, g = u % groups, p = u / groups;
  if (part == 0)
    l1exp_body<T, D, LBB, 1>(q, k, v, kt, ct, stats, bvpart, bt, N, ldc, m, lbmax, ntiles, tpg, groups, scale, jb, g,
                             p, lds, kclk);
  else
    l1exp_body<T, D, LBB, 2>(q, k, v, kt, ct, stats, bvpart, bt, N, ldc, m, lbmax, ntiles, tpg, groups, scale, jb, g,
                             p, lds, kclk);
}

// The same stage without the solver at landmark blocks of at most 32 (m > 64,
// and the forms whose solver runs beside it), with registers held to three
// wavefronts per SIMD: the L1 loop issues faster with three than with two,
// and the 43 KB of LDS of such a block allows three workgroups per CU.  At
// d = 64 this spills a few registers of the cold path and still runs the
// m = 256 kernel-matrix stage 16 % faster.  Same parameters as l1exp_kernel.
template <typename T, int D, int LBB>
__global__ __launch_bounds__(kTT) __attribute__((amdgpu_waves_per_eu(3))) void l1exp_solo_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ kt,
    float* __restrict__ ct, float2* __restrict__ stats, float* __restrict__ bvpart, float* __restrict__ bt,
    float* __restrict__ wout, float* __restrict__ xout, int N, int ldc, int m, int lbmax, int ntiles, int tpg, int groups, int jblocks,
    float scale, float eps, int iters, int nns, int gap, unsigned long long* __restrict__ nsclk,
    unsigned long long* __restrict__ kclk) {
  extern __shared__ __align__(16) float lds[];
  const int b = blockIdx.x;
  const int jb = b % jblocks, g = (b / jblocks) % groups, p = b / (jblocks * groups);
  l1exp_body<T, D, LBB, 0, 2>(q, k, v, kt, ct, stats, bvpart, bt, N, ldc, m, lbmax, ntiles, tpg, groups, scale, jb, g, p,
                        lds, kclk);
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

template <typename T, int D, int LBB, int KS, bool SPLIT = false>
hipError_t launch_kernel(const Plan& pl, const void* q, const void* k, const void* v, Work& w, hipStream_t s,
                         Span t) {
  static_assert(!SPLIT || KS > 0, "the split launch carries the solver");
  const int lbmax = pl.lb;
  size_t floats = (size_t)(lbmax + 1) * kTileRow + (size_t)lbmax * D;
  if (KS > 0 && floats < (size_t)ns_detail::kNsLdsFloats) floats = ns_detail::kNsLdsFloats;
  const size_t shmem = floats * sizeof(float);
  auto kern = l1exp_kernel<T, D, LBB, KS>;
  if constexpr (KS == 0 && LBB <= 2) kern = l1exp_solo_kernel<T, D, LBB>;
  if constexpr (SPLIT) kern = l1exp_split_kernel<T, D, LBB, KS>;
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
  if (SPLIT) grid = (long long)nns + ((long long)pl.groups * pl.P + 7) / 8 * 8 * 2 * pl.jblocks;
  int gap = 0x7fffffff;
  if (nns > 0) {
    const int cus = cu_count();
    if (cus > 0 && nns <= cus && grid > cus) {
      gap = cus;
      grid += nns;
    }
  }
  hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kTT), shmem, s, t.start, t.stop, 0, (const T*)q,
                        (const T*)k, (const T*)v, w.kt, w.ct, reinterpret_cast<float2*>(w.stats), w.bvpart, w.bt, w.w,
                        w.x, pl.N, pl.ldc, pl.m, lbmax, pl.ntiles, pl.tpg, pl.groups, pl.jblocks, pl.scale, pl.eps,
                        pl.ns_iters, nns, gap, w.nsclk, w.kclk);
  if (KS > 0) w.x_final = w.x;
  return hipGetLastError();
}

// m <= 64: the Newton-Schulz step count KS = ceil(m / 4) and the landmark
// row blocks LBB are compile-time constants: ceil(m / 16) for one landmark
// block, ceil(ceil(m / 2) / 16) when HALF splits the landmarks in two.
template <typename T, int D, bool HALF, bool SPLIT = false, int KS = 1>
hipError_t launch_fused(const Plan& pl, const void* q, const void* k, const void* v, Work& w, hipStream_t s,
                        Span t) {
  if constexpr (KS < 16) {
    if ((pl.m + 3) / 4 > KS) return launch_fused<T, D, HALF, SPLIT, KS + 1>(pl, q, k, v, w, s, t);
  }
  if constexpr (HALF) {
    if constexpr (KS >= 8) return launch_kernel<T, D, (2 * KS + 15) / 16, KS, SPLIT>(pl, q, k, v, w, s, t);
    return hipErrorInvalidValue;  // not planned below 29 landmarks
  } else {
    return launch_kernel<T, D, (KS + 3) / 4, KS>(pl, q, k, v, w, s, t);
  }
}

template <typename T, int D>
hipError_t launch_typed(const Plan& pl, const void* q, const void* k, const void* v, Work& w, hipStream_t s,
                        Span t) {
  if (pl.ns_in_launch) {
    // The landmarks go in two blocks when the solver and kernel-matrix
    // workgroups need more than two rounds of the CUs (two workgroups of
    // either kind fit a CU): the half-length kernel-matrix workgroups then
    // fill the slots that free up while the solver workgroups run, instead of
    // a third round of full-length ones starting only when the first solvers
    // end.  They also go in two blocks when even then every workgroup has a
    // CU of its own (a few problems): the halves run side by side.  In
    // between, when the unsplit workgroups would average at most 1.5 per CU
    // the solvers leave free (most of those CUs then run one workgroup, one
    // wavefront per SIMD), the two blocks' C and B halves run as separate
    // workgroups at three wavefronts per SIMD (l1exp_split_kernel): the
    // 28x28 workload (64 problems) went from 68.6 to 62.9 us; at the 56x56
    // workloads (1.86 per free CU) the split was slower (80.3 against 71.9).
    const int cus = cu_count();
    const long long kwg = (long long)pl.groups * pl.P;
    if (cus > 0 && pl.m >= 29) {
      Plan half = pl;
      half.lb = (pl.m + 1) / 2;
      half.jblocks = 2;
      if (pl.P + kwg > 2LL * cus || pl.P + 2 * kwg <= cus) return launch_fused<T, D, true>(half, q, k, v, w, s, t);
      if (pl.P < cus && 2 * kwg <= 3LL * (cus - pl.P)) return launch_fused<T, D, true, true>(half, q, k, v, w, s, t);
    }
    return launch_fused<T, D, false>(pl, q, k, v, w, s, t);
  }
  // The solver runs on its own: one block of m <= 64 landmarks (up to four
  // 16-row blocks), or landmark blocks of at most 32 (two row blocks).
  if (pl.lb > 48) return launch_kernel<T, D, 4, 0>(pl, q, k, v, w, s, t);
  if (pl.lb > 32) return launch_kernel<T, D, 3, 0>(pl, q, k, v, w, s, t);
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
