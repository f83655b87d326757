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
// tile of 256 consecutive tokens of one problem and a block of landmarks.  A
// landmark row is spread over the 16 lanes of each DPP row and reaches every
// lane through a row_newbcast source operand, so the inner loop is pure VALU:
// one subtract (with the broadcast folded in) and one add with an |.| source
// modifier per (token, landmark, feature), and one 16-byte load per lane feeds
// a whole landmark row.  This stage is not a dense contraction; it runs on the
// vector ALUs, not on MFMA.
//
// LDS per workgroup: a tile buffer that holds C as float32 [lb][256 + 4], then
// B as bf16 high and low parts [lb + 1][264] each (the extra row is zero),
// both landmark-major, so that the statistics pass and the C store are
// coalesced and the MFMA reads eight tokens of a landmark row as one 16-byte
// access without bank conflicts.
#include "lapnys_internal.hpp"
#include "ns_small.hpp"

namespace lapnys {

namespace {

constexpr int kTT = 256;        // tokens per tile = lanes per workgroup
constexpr int kTP = kTT + 4;    // C tile row stride (floats; rows stay 16-byte aligned)
constexpr int kRB = kTT + 8;    // B tile row stride (bf16; 528-byte rows: 16-byte aligned, and
                                // 16 consecutive rows start in distinct 4-bank groups)
constexpr int kTileRow = kRB;   // tile buffer floats per landmark row: max(kTP, 2 kRB / 2)
constexpr int kNW = kTT / 64;   // wavefronts per workgroup
static_assert(kTileRow >= kTP, "the C tile must fit in the tile buffer");

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

// Half of the V operand of the B V MFMA for one tile, per lane: for the four
// 32-token steps s = 4 h + sp of half h, V[t0 + 32 s + 8 lk + e][col], e < 8
// (step s covers tokens t0 + 32 s + [0, 32), lane group lk eight of them).
// Tokens past N read the last token's row (their B column is zero).  Each
// half is issued well before its MFMAs.
template <typename T, int D>
struct VHalf {
  T w[kTT / 8];
  __device__ __forceinline__ void issue(const T* __restrict__ vcol, int t0, int lk, int h, int tok_last) {
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        w[8 * sp + e] = vcol[min(t0 + 128 * h + 32 * sp + 8 * lk + e, tok_last) * D];
  }
  // The eight values of step sp as a bf16 MFMA operand: bf16 inputs as they
  // are (lo unused), float32 inputs split into high and low parts.
  __device__ __forceinline__ void operand(int sp, u32x4& hi, u32x4& lo) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (sizeof(T) == 2) {
        hi[i] = (uint32_t)w[8 * sp + 2 * i] | ((uint32_t)w[8 * sp + 2 * i + 1] << 16);
      } else {
        uint32_t h, l;
        split2(widen(w[8 * sp + 2 * i]), widen(w[8 * sp + 2 * i + 1]), h, l);
        hi[i] = h;
        lo[i] = l;
      }
    }
  }
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

// Row j of the tile = exp2(scale * sum_t |x[t] - k_j[t]|) for the lb landmarks
// of the block (0 for a lane past the last token): float32 rows of stride kTP
// at tl, or (SPLIT) bf16 high parts at tl and low parts rows * kRB further,
// rows of stride kRB, followed by a zero row lb.  kl: the block's landmark
// rows in LDS; kg: the same rows in global memory.  Four landmarks at a time, each
// with two partial sums (even / odd features), give eight independent add
// chains; the operands of the next 4-feature chunk are loaded while the
// current chunk is summed, and the compiler barriers keep that shape.
template <int D, bool SPLIT>
__device__ __forceinline__ void kernel_row(const float (&x)[D], const float* __restrict__ kl,
                                           const float* __restrict__ kg, int lb, float scale, float* __restrict__ tl,
                                           int rows, int col, bool valid) {
  auto put = [&](int j, float sum) {
    const float val = valid ? exp2f(sum * scale) : 0.f;
    if constexpr (SPLIT) {
      __bf16* th = reinterpret_cast<__bf16*>(tl);
      const __bf16 hi = (__bf16)val;
      th[j * kRB + col] = hi;
      th[(rows + j) * kRB + col] = (__bf16)(val - (float)hi);
    } else {
      tl[j * kTP + col] = val;
    }
  };
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
// workgroup's LDS, (lbmax + 1) * kTileRow + lbmax * D floats.
template <typename T, int D, int LBB>
__device__ __forceinline__ void l1exp_body(const T* __restrict__ q, const T* __restrict__ k,
                                           const T* __restrict__ v, const float* __restrict__ kt,
                                           float* __restrict__ ct, float2* __restrict__ stats,
                                           float* __restrict__ bvpart, int N, int ldc, int m, int lbmax, int ntiles,
                                           int tpg, int groups, float scale, int jb, int g, int p,
                                           float* __restrict__ tl) {
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
  // Lane li of row block bi reads landmark row 16 bi + li of the B tile, or
  // the zero row lb past the block's landmarks; lane group lk reads tokens
  // 8 lk + [0, 8) of each 32-token step.
  int aoff[BIW];
#pragma unroll
  for (int a = 0; a < BIW; ++a) aoff[a] = min(16 * min(bi0 + a, LBB - 1) + li, lb) * kRB + 8 * lk;
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
    kernel_row<D, false>(x, kl, kg, lb, scale, tl, lbmax + 1, tid, valid);
    __syncthreads();

    // The key row and this lane's V operands are issued now and arrive while
    // the statistics pass runs.
    issue_row<T, D>(k + row, valid, raw);
    VHalf<T, D> v0;
    v0.issue(vcol, t0, lk, 0, tok_last);

    // ---- column statistics of C over the tile, and the C^T store ----
    // Lane l takes tokens 4 l + [0, 4) of the tile: one 16-byte LDS read and
    // one 16-byte store of the C^T row per landmark.  Wavefront w takes
    // landmarks w, w + 4, ..., four of them at a time so that their
    // wavefront reductions overlap.  Tokens past N hold C = 0 (kernel_row),
    // so the sums need no mask; the squared deviations do.  The C^T row
    // stride is N rounded up to 4, so a lane's 16-byte store past N stays in
    // the row's padding.
    const bool full = nvalid == kTT;
    const float inv_n = 1.f / (float)nvalid;  // 1/256 exactly for a full tile
    for (int jq = w; jq < lb; jq += 4 * kNW) {
      float4 vals[4];
      float s[4], m2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jj = min(jq + kNW * u, lb - 1);  // rows past lb: read, not stored
        vals[u] = *reinterpret_cast<const float4*>(tl + jj * kTP + 4 * lane);
        s[u] = (vals[u].x + vals[u].y) + (vals[u].z + vals[u].w);
      }
      wave_sum_dpp_n<4>(s);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float mean = s[u] * inv_n;
        float d[4] = {vals[u].x - mean, vals[u].y - mean, vals[u].z - mean, vals[u].w - mean};
        if (!full) {
#pragma unroll
          for (int i = 0; i < 4; ++i) d[i] = (4 * lane + i < nvalid) ? d[i] : 0.f;
        }
        m2[u] = (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
      }
      wave_sum_dpp_n<4>(m2);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = jq + kNW * u;
        if (j < lb) {
          if (lane == 0) stats[((size_t)p * ntiles + tile) * m + j0 + j] = make_float2(s[u], m2[u]);
          float* crow = ct + ((size_t)p * m + j0 + j) * ldc + t0;
          if (4 * lane < nvalid) *reinterpret_cast<float4*>(crow + 4 * lane) = vals[u];
        }
      }
    }

    // ---- B = k(K~, K), kept on chip ----
    widen_row<D>(raw, x);
    __syncthreads();  // statistics pass done with the tile buffer
    kernel_row<D, true>(x, kl, kg, lb, scale, tl, lbmax + 1, tid, valid);
    __syncthreads();

    // ---- B V partial: acc[landmark][feature] += sum over the tile's tokens ----
    // bf16 MFMA 16x16x32, one 32-token step at a time: lane (li, lk) supplies
    // A[li][8 lk + e] = B[landmark][token 32 s + 8 lk + e] (one 16-byte LDS
    // read of the high parts, one of the low parts) and B[8 lk + e][li] =
    // V[same token][feature].  Per step and row block: Blo V + Bhi V for bf16
    // V, plus Bhi Vlo for float32 V.  The first half of V is already in
    // registers and the second half lands during the first half's MFMAs; tile
    // rows past the block's landmarks are zero.
    VHalf<T, D> v1;
    v1.issue(vcol, t0, lk, 1, tok_last);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const VHalf<T, D>& vh = h ? v1 : v0;
#pragma unroll
      for (int sp = 0; sp < 4; ++sp) {
        const int s32 = 32 * (4 * h + sp);
        u32x4 vhi, vlo;
        vh.operand(sp, vhi, vlo);
        bf16x8 ah[BIW], al[BIW];
#pragma unroll
        for (int a = 0; a < BIW; ++a) {
          ah[a] = *reinterpret_cast<const bf16x8*>(bh + aoff[a] + s32);
          al[a] = *reinterpret_cast<const bf16x8*>(bl + aoff[a] + s32);
        }
        const bf16x8 vb = __builtin_bit_cast(bf16x8, vhi);
#pragma unroll
        for (int a = 0; a < BIW; ++a) acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[a], vb, acc[a], 0, 0, 0);
        if constexpr (sizeof(T) == 4) {
          const bf16x8 vl = __builtin_bit_cast(bf16x8, vlo);
#pragma unroll
          for (int a = 0; a < BIW; ++a) acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[a], vl, acc[a], 0, 0, 0);
        }
#pragma unroll
        for (int a = 0; a < BIW; ++a) acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[a], vb, acc[a], 0, 0, 0);
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
  size_t floats = (size_t)(lbmax + 1) * kTileRow + (size_t)lbmax * D;
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
