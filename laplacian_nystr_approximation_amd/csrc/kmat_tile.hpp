// Pieces of the kernel-matrix stage shared by its Laplacian (l1exp.hip) and
// Gaussian (gauss.hip) forms.  A workgroup of 256 lanes takes a tile of 256
// consecutive tokens of one problem and a block of lb <= 64 landmarks; once
// the tile's kernel values are in LDS, the rest does not depend on the kernel:
//   * tile_stats_store: per landmark, the tile's sum of C and sum of squared
//     deviations from the tile mean (the whitening statistics, EN page,
//     section 2.B), and the C^T store, from C as float32 [lb][kTP] in LDS;
//   * BvTile: the B V partial product over the tile on bf16 MFMA, from B as
//     bf16 high and low parts [lb + 1][kRB] each in LDS (row lb zero).
#pragma once

#include "lapnys_internal.hpp"

namespace lapnys {
namespace kmat {

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

// bf16 V: each pair of consecutive values of a step is loaded straight into
// the two halves of one register (the packed MFMA operand word), so a half
// holds 16 registers instead of 32.
template <int D>
struct VHalf<uint16_t, D> {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 w[kTT / 16];
  __device__ __forceinline__ void issue(const uint16_t* __restrict__ vcol, int t0, int lk, int h, int tok_last) {
#pragma unroll
    for (int sp = 0; sp < 4; ++sp)
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int t = t0 + 128 * h + 32 * sp + 8 * lk + 2 * e2;
        w[4 * sp + e2].x = vcol[min(t, tok_last) * D];
        w[4 * sp + e2].y = vcol[min(t + 1, tok_last) * D];
      }
  }
  __device__ __forceinline__ void operand(int sp, u32x4& hi, u32x4& lo) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) hi[i] = __builtin_bit_cast(uint32_t, w[4 * sp + i]);
    (void)lo;
  }
};

// Column statistics of the tile's C (float32 rows of stride kTP at tl) and
// the C^T store.
//   * Statistics: L lanes per landmark (lane L j + q, j < lb; L = 4, 8 or 16
//     as the block has more than 32, more than 16 or at most 16 landmarks),
//     lane q summing its 256 / L tokens of row j as 16-byte LDS reads in token
//     order; the partial sums merge pairwise by lane exchanges ((q0 + q1) +
//     (q2 + q3) and so on), so all L lanes hold the same tile sum and mean, and
//     the squared deviations about that mean go the same way.  No
//     wavefront-wide reduction: the sixteen DPP steps per landmark pair those
//     took were half of this pass.  Tokens past N hold C = 0, so the sums need
//     no mask; the squared deviations do.
//   * C^T: lane l stores tokens 4 l + [0, 4) of each of its wavefront's rows
//     (w, w + 4, ...) with one 16-byte store.  The C^T row stride is N rounded
//     up to 4, so a store past N stays in the row's padding.
__device__ __forceinline__ void tile_stats_store(const float* __restrict__ tl, float2* __restrict__ stats,
                                                 float* __restrict__ ct, int p, int ntiles, int tile, int m, int j0,
                                                 int lb, int ldc, int t0, int nvalid, int lane, int w) {
  const bool full = nvalid == kTT;
  const float inv_n = 1.f / (float)nvalid;  // 1/256 exactly for a full tile
  {
    // L lanes per landmark (4 up to 64 landmarks, 8 up to 32, 16 up to 16),
    // so every wavefront takes part however few landmarks the block has;
    // lane q of landmark j sums tokens SEG q + [0, SEG), SEG = 256 / L.
    const int lsh = lb > 32 ? 2 : (lb > 16 ? 3 : 4), L = 1 << lsh, seg = kTT >> lsh;
    const int tid = 64 * w + lane, j = tid >> lsh, q = tid & (L - 1);
    const float* row = tl + min(j, lb - 1) * kTP + seg * q;  // rows past lb: read, not stored
    // The row segment is read twice (sum, then deviations) rather than held:
    // the pass runs beside the next row's loads in flight.
    float s = 0.f;
#pragma unroll 4
    for (int i = 0; i < seg / 4; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(row + 4 * i);
      s += (v.x + v.y) + (v.z + v.w);
    }
    for (int off = 1; off < L; off <<= 1) s += __shfl_xor(s, off, 64);
    const float mean = s * inv_n;
    float m2 = 0.f;
#pragma unroll 4
    for (int i = 0; i < seg / 4; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(row + 4 * i);
      float d[4] = {v.x - mean, v.y - mean, v.z - mean, v.w - mean};
      if (!full) {
#pragma unroll
        for (int e = 0; e < 4; ++e) d[e] = (seg * q + 4 * i + e < nvalid) ? d[e] : 0.f;
      }
      m2 += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
    }
    for (int off = 1; off < L; off <<= 1) m2 += __shfl_xor(m2, off, 64);
    if (q == 0 && j < lb) stats[((size_t)p * ntiles + tile) * m + j0 + j] = make_float2(s, m2);
  }
  if (4 * lane < nvalid) {
    for (int j = w; j < lb; j += kNW) {
      const float4 c4 = *reinterpret_cast<const float4*>(tl + j * kTP + 4 * lane);
      *reinterpret_cast<float4*>(ct + ((size_t)p * m + j0 + j) * ldc + t0 + 4 * lane) = c4;
    }
  }
}

// The B V partial of one workgroup, acc[landmark][feature] summed over its
// tiles, on bf16 MFMA 16x16x32.  Output blocks (16 x 16) of wavefront w: one
// 16-feature column block bt0 and BIW of the LBB 16-row landmark blocks,
// starting at bi0.  When the row blocks do not split evenly, a wavefront's
// last block may lie past LBB: it reads a valid (zero-padded) row block and
// is not stored, so every MFMA issues unconditionally.
template <typename T, int D, int LBB>
struct BvTile {
  static constexpr int DB = D / 16;
  static_assert(kNW % DB == 0, "wavefronts must cover the feature blocks");
  static constexpr int SPLIT = kNW / DB;
  static constexpr int BIW = (LBB + SPLIT - 1) / SPLIT;
  int bt0, bi0, li, lk;
  int aoff[BIW];
  f32x4 acc[BIW];

  // Lane li of row block bi reads landmark row 16 bi + li of the B tile, or
  // the zero row lb past the block's landmarks; lane group lk reads tokens
  // 8 lk + [0, 8) of each 32-token step.
  __device__ __forceinline__ void init(int w, int lane, int lb) {
    bt0 = w % DB;
    bi0 = (w / DB) * BIW;
    li = lane & 15;
    lk = lane >> 4;
#pragma unroll
    for (int a = 0; a < BIW; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int a = 0; a < BIW; ++a) aoff[a] = min(16 * min(bi0 + a, LBB - 1) + li, lb) * kRB + 8 * lk;
  }

  // acc += the tile's B (high parts bh, low parts bl, rows of stride kRB)
  // times V.  One 32-token step at a time: lane (li, lk) supplies A[li][8 lk +
  // e] = B[landmark][token 32 s + 8 lk + e] (one 16-byte LDS read of the high
  // parts, one of the low parts) and B[8 lk + e][li] = V[same token][feature].
  // Per step and row block: Blo V + Bhi V for bf16 V, plus Bhi Vlo for float32
  // V.  The first half of V (v0) is in registers and the second (v1) lands
  // during the first half's MFMAs.
  __device__ __forceinline__ void accumulate(const __bf16* __restrict__ bh, const __bf16* __restrict__ bl,
                                             const VHalf<T, D>& v0, const VHalf<T, D>& v1) {
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

  // Rows j0 + [0, lb) of the group's partial, bvp = bvpart[p][g].
  __device__ __forceinline__ void store(float* __restrict__ bvp, int j0, int lb) const {
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
};

}  // namespace kmat
}  // namespace lapnys
