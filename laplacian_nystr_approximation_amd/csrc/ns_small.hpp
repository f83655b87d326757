// Newton-Schulz inverse of the landmark Gram matrix for m <= 64, one
// workgroup per problem with every operand in LDS (EN page, section 2.C.2;
// DE section 2; ZH section 2.2; KO section 2.3; JA section 2.3):
//
//   W  = k(K~, K~) + eps I,   k(x, y) = exp(-||x - y||_1 / lambda)
//   X0 = W^T / (||W||_1 ||W||_inf)
//   X <- X (2I - W X), a fixed number of times, matrix products only.
//
// W is built so that it is bit-symmetric: entry (a, b) and entry (b, a) sum
// the same |differences| in the same feature order, and the diagonal is
// exp(0) + eps = 1 + eps exactly as float32 arithmetic gives it.  These
// workgroups run inside the kernel-matrix stage's launch (l1exp.hip).
//
// Precision of the steps: the iteration corrects its own errors (from
// X = W^-1 (I + E) one exact step gives W^-1 (I - E^2)), so only the last
// steps decide the accuracy of the result.  All but the last kFp32Steps steps
// take their products on bf16 MFMA with both operands split into high and
// low parts (hi*hi + hi*lo + lo*hi, about 2^-16 of each product); the last
// kFp32Steps steps are float32 products on fp32 MFMA, which square the
// error left by the split steps and end at the float32 floor.  X itself is
// kept in float32 throughout: each lane holds the entries it produces in
// registers, and only the MFMA operands in LDS are split.
#pragma once

#include "lapnys_internal.hpp"

namespace lapnys {
namespace ns_detail {

constexpr int kMP = 64;  // padded size of the in-LDS schedule
constexpr int kLD = 68;  // float32 LDS row stride (floats): conflict-free column reads
constexpr int kLB = 72;  // bf16 LDS row stride (144-byte rows: 16-byte aligned, and
                         // 16 consecutive rows start in distinct 4-bank groups)
constexpr int kXB = kMP * kLB;  // bf16 elements of one 64 x 64 high or low array
constexpr int kFp32Steps = 2;   // final steps on float32 products
// LDS of one problem's schedule (floats).  Split steps: X (high, low) twice
// and (W X)^T (high, low), 6 kXB bf16 = 3 kXB floats.  Float32 steps (the
// same bytes): X twice and (W X)^T, 3 kMP kLD floats.  Then 256 partial sums
// and alpha.
constexpr int kNsRegion = 3 * kXB;
static_assert(3 * kMP * kLD <= kNsRegion, "the float32 layout must fit in the split layout's bytes");
constexpr int kNsLdsFloats = kNsRegion + 260;

// In-LDS schedule for m <= 64: one workgroup of four wavefronts per problem,
// 57 KB of LDS (so it can share a CU with the kernel-matrix stage).
//
// Each step is evaluated as X_next = 2X - X (W X), which equals X (2I - W X).
// Symmetry: W is bit-symmetric and X0 = W^T / alpha = W / alpha; for a
// symmetric X the product X W X is symmetric whatever rounding X carries, so
// Q = W X is formed in full (wavefront w: the four 16 x 16 blocks of block row
// w) and stored transposed, while S = X Q is formed only on its 10 upper
// 16 x 16 blocks (spread over the wavefronts as 3, 3, 2, 2) and stored with
// its mirror image.  X thus stays exactly symmetric in one row-major copy,
// and a column of X is read as a row.  (Mirroring a product that is not
// symmetric in exact arithmetic, such as W X, would not be a faithful step:
// the iteration then drifts away once it has converged.)
//
// The float32 steps reduce over k in [0, 4 KS), KS = ceil(m / 4), on fp32
// MFMA 16x16x4; the split steps over k in [0, 32 KB), KB = ceil(m / 32), on
// bf16 MFMA 16x16x32.  Padding rows and columns of W and X are exact zeros
// and stay so, and every step writes all 64 x 64 entries of X_next.
__device__ __constant__ int8_t kBlkI[4][3] = {{0, 0, 0}, {0, 1, 1}, {1, 2, -1}, {2, 3, -1}};
__device__ __constant__ int8_t kBlkJ[4][3] = {{0, 1, 2}, {3, 1, 2}, {3, 2, -1}, {3, 3, -1}};

// Problem p's W and X, for one workgroup of 256 lanes.  lds: kNsLdsFloats
// floats, 16-byte aligned.
template <int D, int KS>
__device__ __forceinline__ void ns_small(const float* __restrict__ kt, float* __restrict__ wout,
                                         float* __restrict__ xout, int m, float scale, float eps, int iters, int p,
                                         float* __restrict__ lds) {
  constexpr int KLD = D + 4;  // landmark staging stride: 16-byte rows for broadcast reads
  static_assert(kMP * KLD <= kMP * kLD, "landmark staging must fit in an X buffer");
  // Float32 layout: X (ping-pong, symmetric), then (W X)^T.
  float4(*xs4)[kMP * kLD / 4] = reinterpret_cast<float4(*)[kMP * kLD / 4]>(lds);
  float* ql = lds + 2 * kMP * kLD;
  // Split layout (same bytes): X high/low parts ping-pong, then (W X)^T high/low.
  __bf16* xb16 = reinterpret_cast<__bf16*>(lds);
  __bf16* qb16 = xb16 + 4 * kXB;
  // Set-up: W in the float32 (W X)^T buffer, the landmarks in the second
  // float32 X buffer.  X0 goes to the first split X buffer (2 kXB bf16 =
  // kXB floats), which ends before W starts; the landmarks are dead by then.
  float* wl = ql;
  float* kl = reinterpret_cast<float*>(xs4[1]);
  static_assert(kXB <= 2 * kMP * kLD, "X0 must not overlap W");
  float* red = lds + kNsRegion;  // [256] partial column sums, then alpha
  float& alpha_s = red[256];

  // Beside the kernel-matrix workgroups on the same CUs, the solver's chain
  // of dependent products is the longer one: its wavefronts take issue
  // priority.
  __builtin_amdgcn_s_setprio(3);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // Landmark rows into LDS: every load of the (at most 64 x D) block is
  // issued before the first store, so the staging costs one memory latency.
  {
    constexpr int kV = kMP * D / 4 / 256;  // float4 per lane
    const float4* ktp4 = reinterpret_cast<const float4*>(kt + (size_t)p * m * D);
    float4 kv[kV];
#pragma unroll
    for (int i = 0; i < kV; ++i) {
      const int e4 = tid + 256 * i;
      kv[i] = (4 * e4 < m * D) ? ktp4[e4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < kV; ++i) {
      const int e = 4 * (tid + 256 * i);
      *reinterpret_cast<float4*>(&kl[(e / D) * KLD + (e % D)]) = kv[i];
    }
  }
  __syncthreads();

  // W = k(K~, K~) + eps I, zero padded.  Lane b holds landmark b in
  // registers; wavefront w forms rows [16 w, 16 w + 16) four at a time with
  // the row landmark broadcast from LDS.  Entry (a, b) sums |K~_a - K~_b| over
  // even and odd features in increasing order, the same sums as entry (b, a),
  // so W is bit-symmetric.
  {
    const int b = lane;
    float csum = 0.f;  // |W[a][b]| over this wavefront's rows a, in increasing a
    float xb[D];
#pragma unroll
    for (int t = 0; t < D; ++t) xb[t] = kl[min(b, m - 1) * KLD + t];
    for (int a0 = 16 * w; a0 < 16 * w + 16; a0 += 4) {
      if (a0 < m) {
        float s0[4] = {0.f, 0.f, 0.f, 0.f}, s1[4] = {0.f, 0.f, 0.f, 0.f};
        const float* ka[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) ka[u] = kl + min(a0 + u, m - 1) * KLD;
#pragma unroll
        for (int t = 0; t < D; t += 4) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float4 r = *reinterpret_cast<const float4*>(ka[u] + t);
            s0[u] += fabsf(r.x - xb[t]);
            s1[u] += fabsf(r.y - xb[t + 1]);
            s0[u] += fabsf(r.z - xb[t + 2]);
            s1[u] += fabsf(r.w - xb[t + 3]);
          }
          // The sums are in/out operands here: each 4-feature chunk's row
          // values are read just before use (bounded registers).
          asm volatile("" : "+v"(s0[0]), "+v"(s0[1]), "+v"(s0[2]), "+v"(s0[3]), "+v"(s1[0]), "+v"(s1[1]),
                       "+v"(s1[2]), "+v"(s1[3])::"memory");
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int a = a0 + u;
          float val = 0.f;
          if (a < m && b < m) {
            val = exp2f((s0[u] + s1[u]) * scale);
            if (a == b) val += eps;
          }
          wl[a * kLD + b] = val;
          csum += val;  // entries are positive
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) wl[(a0 + u) * kLD + b] = 0.f;
      }
    }
    red[w * kMP + b] = csum;
  }
  __syncthreads();

  // alpha = ||W||_1 ||W||_inf.  W is symmetric, so its largest absolute
  // column sum (the 1-norm) is also its largest row sum (the inf-norm):
  // alpha = (max_b sum_a |W[a][b]|)^2, the column sums merged from the four
  // wavefronts' partial sums in wavefront order.  W goes out to the
  // workspace.
  float* wp = wout + (size_t)p * kMP * kMP;
  for (int e = tid; e < kMP * kMP; e += 256) wp[e] = wl[(e >> 6) * kLD + (e & 63)];
  if (tid < 64) {
    float cm = ((red[tid] + red[kMP + tid]) + red[2 * kMP + tid]) + red[3 * kMP + tid];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off, 64));
    if (tid == 0) alpha_s = cm * cm;
  }
  __syncthreads();

  const int li = lane & 15, lk = lane >> 4;
  // This wavefront's upper blocks of S = X Q.  Wavefronts with two upper
  // blocks run a third, unstored copy of their last block: every wavefront
  // issues the same MFMA sequence and none branches inside it.
  int bI[3], bJ[3];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    bI[b] = kBlkI[w][b];
    bJ[b] = kBlkJ[w][b];
  }
  const int nb = bI[2] < 0 ? 2 : 3;
  if (nb == 2) {
    bI[2] = bI[1];
    bJ[2] = bJ[1];
  }
  // W's A operands for every step of Q = W X, block row w.  fp32 MFMA
  // 16x16x4: A[li][lk] of step s = W[16 w + li][4 s + lk], KS = ceil(m / 4)
  // steps (a template parameter, so the step loops unroll without branches).
  // bf16 MFMA 16x16x32: A[li][8 lk + e] of step kb = W[16 w + li][32 kb +
  // 8 lk + e], KB = ceil(m / 32) steps, as high and low parts.
  constexpr int KB = (4 * KS + 31) / 32;
  float wreg[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) wreg[st] = wl[(16 * w + li) * kLD + 4 * st + lk];
  u32x4 wh[KB], wlo[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* wr = wl + (16 * w + li) * kLD + 32 * kb + 8 * lk + 2 * i;
      uint32_t h, l;
      split2(wr[0], wr[1], h, l);
      wh[kb][i] = h;
      wlo[kb][i] = l;
    }

  // X0 = W^T / alpha.  xij[b][r] = X[16 bI + 4 lk + r][16 bJ + li], the
  // entries this lane produces (the upper-triangle ones of its blocks are
  // the ones it stores); the split steps keep them in these registers.
  const int n16 = iters > kFp32Steps ? iters - kFp32Steps : 0;
  const float alpha = alpha_s;
  float xij[3][4];
#pragma unroll
  for (int b = 0; b < 3; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) xij[b][r] = wl[(16 * bJ[b] + li) * kLD + 16 * bI[b] + 4 * lk + r] / alpha;
  if (n16 > 0) {
    // Every entry of X0, as high and low parts.
    for (int e = tid; e < kMP * kMP / 2; e += 256) {
      const int a = e >> 5, c = 2 * (e & 31);
      uint32_t h, l;
      split2(wl[c * kLD + a] / alpha, wl[(c + 1) * kLD + a] / alpha, h, l);
      *reinterpret_cast<uint32_t*>(xb16 + a * kLB + c) = h;
      *reinterpret_cast<uint32_t*>(xb16 + kXB + a * kLB + c) = l;
    }
  } else {
    float* x0 = reinterpret_cast<float*>(xs4[0]);
    for (int e = tid; e < kMP * kMP; e += 256) {
      const int a = e >> 6, b = e & 63;
      x0[a * kLD + b] = wl[b * kLD + a] / alpha;
    }
  }
  __syncthreads();

  // ---- split steps: X (hi, lo) in buffer cur -> buffer cur ^ 1 ----
  int cur = 0;
  for (int it = 0; it < n16; ++it) {
    const __bf16* xh = xb16 + cur * 2 * kXB;
    const __bf16* xlo = xh + kXB;
    // Q = W X, block row w, stored transposed: Q^T[j][i] = Q[i][j].  The B
    // operand X[32 kb + 8 lk + e][16 bj + li] is read as row 16 bj + li (X is
    // symmetric).
    {
      f32x4 acc[4];
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) acc[bj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
          const int o = (16 * bj + li) * kLB + 32 * kb + 8 * lk;
          const bf16x8 bh = *reinterpret_cast<const bf16x8*>(xh + o);
          const bf16x8 bl = *reinterpret_cast<const bf16x8*>(xlo + o);
          acc[bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wlo[kb]), bh, acc[bj], 0, 0, 0);
          acc[bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wh[kb]), bl, acc[bj], 0, 0, 0);
          acc[bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wh[kb]), bh, acc[bj], 0, 0, 0);
        }
      }
      // acc[bj][r] = Q[16 w + 4 lk + r][16 bj + li]: four consecutive entries
      // of row 16 bj + li of Q^T.
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) {
        uint32_t h0, l0, h1, l1;
        split2(acc[bj][0], acc[bj][1], h0, l0);
        split2(acc[bj][2], acc[bj][3], h1, l1);
        const int o = (16 * bj + li) * kLB + 16 * w + 4 * lk;
        *reinterpret_cast<uint2*>(qb16 + o) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(qb16 + kXB + o) = make_uint2(l0, l1);
      }
    }
    __syncthreads();
    // S = X Q on the upper blocks; X_next = 2 X - S, stored with its mirror.
    {
      f32x4 acc[3];
#pragma unroll
      for (int b = 0; b < 3; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int b = 0; b < 3; ++b) {
          const int oa = (16 * bI[b] + li) * kLB + 32 * kb + 8 * lk;  // X[16 bI + li][32 kb + 8 lk + e]
          const int ob = (16 * bJ[b] + li) * kLB + 32 * kb + 8 * lk;  // Q[32 kb + 8 lk + e][16 bJ + li]
          const bf16x8 ah = *reinterpret_cast<const bf16x8*>(xh + oa);
          const bf16x8 al = *reinterpret_cast<const bf16x8*>(xlo + oa);
          const bf16x8 qh = *reinterpret_cast<const bf16x8*>(qb16 + ob);
          const bf16x8 ql2 = *reinterpret_cast<const bf16x8*>(qb16 + kXB + ob);
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, qh, acc[b], 0, 0, 0);
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, ql2, acc[b], 0, 0, 0);
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, qh, acc[b], 0, 0, 0);
        }
      }
      __bf16* nh = xb16 + (cur ^ 1) * 2 * kXB;
      __bf16* nl = nh + kXB;
#pragma unroll
      for (int b = 0; b < 3; ++b) {
#pragma unroll
        for (int r = 0; r < 4; ++r) xij[b][r] = 2.f * xij[b][r] - acc[b][r];
        if (b < nb) {
          uint32_t h0, l0, h1, l1;
          split2(xij[b][0], xij[b][1], h0, l0);
          split2(xij[b][2], xij[b][3], h1, l1);
          const uint32_t hw[4] = {h0 & 0xffffu, h0 >> 16, h1 & 0xffffu, h1 >> 16};
          const uint32_t lw[4] = {l0 & 0xffffu, l0 >> 16, l1 & 0xffffu, l1 >> 16};
          const int i0 = 16 * bI[b] + 4 * lk, j = 16 * bJ[b] + li;
          uint16_t* nh16 = reinterpret_cast<uint16_t*>(nh);
          uint16_t* nl16 = reinterpret_cast<uint16_t*>(nl);
          if (bI[b] != bJ[b]) {
            // off the diagonal every entry is upper: the mirror image is four
            // consecutive entries of row j
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              nh16[(i0 + r) * kLB + j] = (uint16_t)hw[r];
              nl16[(i0 + r) * kLB + j] = (uint16_t)lw[r];
            }
            *reinterpret_cast<uint2*>(nh + j * kLB + i0) = make_uint2(h0, h1);
            *reinterpret_cast<uint2*>(nl + j * kLB + i0) = make_uint2(l0, l1);
          } else {
            // diagonal block: only the upper-triangle entries, with their mirrors
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (i0 + r <= j) {
                nh16[(i0 + r) * kLB + j] = (uint16_t)hw[r];
                nl16[(i0 + r) * kLB + j] = (uint16_t)lw[r];
                nh16[j * kLB + i0 + r] = (uint16_t)hw[r];
                nl16[j * kLB + i0 + r] = (uint16_t)lw[r];
              }
            }
          }
        }
      }
    }
    __syncthreads();
    cur ^= 1;
  }
  if (n16 > 0) {
    // Into the float32 layout for the last steps: the stored (upper) entries
    // and their mirrors, from the registers.  The split buffers are dead
    // (every wavefront passed the last step's barrier).
    float* x0 = reinterpret_cast<float*>(xs4[0]);
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      if (b < nb) {
        const int i0 = 16 * bI[b] + 4 * lk, j = 16 * bJ[b] + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (bI[b] != bJ[b] || i0 + r <= j) {
            x0[(i0 + r) * kLD + j] = xij[b][r];
            x0[j * kLD + i0 + r] = xij[b][r];
          }
        }
      }
    }
    __syncthreads();
    cur = 0;
  }

  // ---- float32 steps ----
  for (int it = n16; it < iters; ++it) {
    const float* xc = reinterpret_cast<const float*>(xs4[cur]);
    // Q = W X, block row w, stored transposed: ql[j][i] = Q[i][j].
    {
      f32x4 acc[4];
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) acc[bj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
          const float xb = xc[(16 * bj + li) * kLD + 4 * st + lk];  // X[4 st + lk][16 bj + li]
          acc[bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(wreg[st], xb, acc[bj], 0, 0, 0);
        }
      }
      // acc[bj][r] = Q[16 w + 4 lk + r][16 bj + li]: four consecutive entries of
      // row 16 bj + li of Q^T.
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
        *reinterpret_cast<float4*>(&ql[(16 * bj + li) * kLD + 16 * w + 4 * lk]) =
            make_float4(acc[bj][0], acc[bj][1], acc[bj][2], acc[bj][3]);
    }
    __syncthreads();
    // S = X Q on the upper blocks; X_next = 2 X - S stored with its mirror.
    {
      float xo[3][4];  // X entries of this lane's outputs, read ahead of the products
#pragma unroll
      for (int b = 0; b < 3; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) xo[b][r] = xc[(16 * bI[b] + 4 * lk + r) * kLD + 16 * bJ[b] + li];
      f32x4 acc[3];
#pragma unroll
      for (int b = 0; b < 3; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
#pragma unroll
        for (int b = 0; b < 3; ++b) {
          const float xa = xc[(16 * bI[b] + li) * kLD + 4 * st + lk];  // X[16 bi + li][4 st + lk]
          const float qb = ql[(16 * bJ[b] + li) * kLD + 4 * st + lk];  // Q[4 st + lk][16 bj + li]
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa, qb, acc[b], 0, 0, 0);
        }
      }
      float* xn = reinterpret_cast<float*>(xs4[cur ^ 1]);
#pragma unroll
      for (int b = 0; b < 3; ++b) {
        if (b < nb) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = 2.f * xo[b][r] - acc[b][r];
          const int i0 = 16 * bI[b] + 4 * lk, j = 16 * bJ[b] + li;
          if (bI[b] != bJ[b]) {
            // off the diagonal every entry is upper: the mirror image is four
            // consecutive entries of row j
#pragma unroll
            for (int r = 0; r < 4; ++r) xn[(i0 + r) * kLD + j] = v[r];
            *reinterpret_cast<float4*>(&xn[j * kLD + i0]) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
            // diagonal block: only the upper-triangle entries, with their mirrors
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (i0 + r <= j) {
                xn[(i0 + r) * kLD + j] = v[r];
                xn[j * kLD + i0 + r] = v[r];
              }
            }
          }
        }
      }
    }
    __syncthreads();
    cur ^= 1;
  }

  float* xp = xout + (size_t)p * kMP * kMP;
  const float* xf = reinterpret_cast<const float*>(xs4[cur]);
  for (int e = tid; e < kMP * kMP; e += 256) xp[e] = xf[(e >> 6) * kLD + (e & 63)];
}


}  // namespace ns_detail
}  // namespace lapnys
