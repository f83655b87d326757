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
// Form of a step: X_next = 2X - X (W X), every entry formed.  With Q = W X
// rounded to Q + dQ, the step's own error is X dQ, whose residual W X dQ is
// about dQ once W X is near I.  Copying one triangle of the product onto the
// other (to keep X exactly symmetric) would put dQ^T X there instead, whose
// residual W dQ^T X is larger by up to cond(W): that drives the iteration
// away from the inverse for cond(W) of about 1e4 and more.  So X is not
// assumed symmetric: it is kept both row-major and transposed.
//
// Precision of the steps: the iteration corrects its own errors (from
// X = W^-1 (I + E) one exact step gives W^-1 (I - E^2)), so only the last
// steps decide the accuracy of the result.  Steps take their products on
// bf16 MFMA with both operands split into high and low parts (hi*hi + hi*lo
// + lo*hi: each entry of W X is off by about 2^-16 of sum_k |W_ik| |X_kj|,
// at most 2^-16 rho with rho = ||W||_1 max|X|), while rho stays at most
// kSplitGuard and until kFp32Steps steps remain; every later step takes
// float32 products on fp32 MFMA, which square the error the split steps
// left and end at the float32 floor.  In exact arithmetic rho after k steps
// is at most 2^(k/2) (the iterate's eigenvalues are at most sqrt(2^k / alpha)
// and ||W||_1 = sqrt(alpha)), so the guard cannot act before step 12, and
// for a well-conditioned W (rho stays below 11 on the pooled heavy-tailed
// landmarks) it never acts.  X itself is float32 throughout: each lane holds
// the entries it produces in registers, and only the MFMA operands in LDS
// are split.
#pragma once

#include "lapnys_internal.hpp"

namespace lapnys {
namespace ns_detail {

constexpr int kMP = 64;  // padded size of the in-LDS schedule
constexpr int kLD = 68;  // float32 LDS row stride (floats): conflict-free column reads
constexpr int kLB = 72;  // bf16 LDS row stride (144-byte rows: 16-byte aligned, and
                         // 16 consecutive rows start in distinct 4-bank groups)
constexpr int kXB = kMP * kLB;  // bf16 elements of one 64 x 64 high or low array
constexpr int kFp32Steps = 2;   // final steps on float32 products, at least
constexpr float kSplitGuard = 64.f;  // largest rho = ||W||_1 max|X| for a split step
// LDS of one problem's schedule (floats).  Split steps: X, X^T and (W X)^T,
// each as high and low parts, 6 kXB bf16 = 3 kXB floats.  Float32 steps (the
// same bytes): X, X^T and (W X)^T, 3 kMP kLD floats.  Then 256 partial sums,
// alpha and ||W||_1.
constexpr int kNsRegion = 3 * kXB;
static_assert(3 * kMP * kLD <= kNsRegion, "the float32 layout must fit in the split layout's bytes");
constexpr int kNsLdsFloats = kNsRegion + 260;

// Largest value over the 64 lanes of a wavefront of a non-negative x,
// returned to every lane: DPP row rotations leave each 16-lane row's
// largest value in every lane of the row, then row_bcast:15 and row_bcast:31
// carry rows 0 and 2 into rows 1 and 3 and rows 0 + 1 into row 3 (rows the
// mask leaves out read 0, which does not change a maximum of non-negative
// values), and lane 63 is read.
__device__ __forceinline__ float wave_max_nonneg(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xa, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xc, 0xf, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// In-LDS schedule for m <= 64: one workgroup of four wavefronts per problem,
// 57 KB of LDS (so it can share a CU with the kernel-matrix stage).
//
// Wavefront w owns block row w (rows [16 w, 16 w + 16)) of Q = W X, of
// S = X Q and of X: each lane holds the 16 entries X[16 w + 4 lk + r]
// [16 bj + li] (bj, r in [0, 4)) in registers.  A step forms Q's block row
// (W's rows from registers, X's columns read as rows of X^T), stores it
// transposed, and after a barrier forms S's block row (X's rows, Q's columns
// read as rows of Q^T), then writes X_next = 2X - S into both X (row-major)
// and X^T.  Only wavefront w reads X's block row w, and X^T is read only in
// the first half of a step, so both are updated in place.
//
// The float32 steps reduce over k in [0, 4 KS), KS = ceil(m / 4), on fp32
// MFMA 16x16x4; the split steps over k in [0, 32 KB), KB = ceil(m / 32), on
// bf16 MFMA 16x16x32.  Padding rows and columns of W and X are exact zeros
// and stay so, and every step writes all 64 x 64 entries of X_next.
//
// Problem p's W and X, for one workgroup of 256 lanes.  lds: kNsLdsFloats
// floats, 16-byte aligned.
template <int D, int KS>
__device__ __forceinline__ void ns_small(const float* __restrict__ kt, float* __restrict__ wout,
                                         float* __restrict__ xout, int m, float scale, float eps, int iters, int p,
                                         float* __restrict__ lds, unsigned long long* __restrict__ clk) {
  // Debug stamps (clk non-null): start, first step, end, device wall clock.
  const unsigned long long t_start = clk ? (unsigned long long)wall_clock64() : 0ull;
  constexpr int KLD = D + 4;  // landmark staging stride: 16-byte rows for broadcast reads
  static_assert(kMP * KLD <= kMP * kLD, "landmark staging must fit in one float32 buffer");
  // Float32 layout: X, X^T, (W X)^T.
  float* xf = lds;
  float* xtf = lds + kMP * kLD;
  float* qf = lds + 2 * kMP * kLD;
  // Split layout (same bytes): X, X^T, (W X)^T, each high parts then low parts.
  __bf16* xb = reinterpret_cast<__bf16*>(lds);
  __bf16* xtb = xb + 2 * kXB;
  __bf16* qb = xb + 4 * kXB;
  // Set-up: W in the float32 (W X)^T buffer, the landmarks in the float32
  // X^T buffer.  Both are dead once every lane holds its operands in
  // registers (a barrier before X0 is stored).
  float* wl = qf;
  float* kl = xtf;
  float* red = lds + kNsRegion;  // [256] partial column sums, then alpha and ||W||_1
  float& alpha_s = red[256];
  float& norm1_s = red[257];

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
    float xb_[D];
#pragma unroll
    for (int t = 0; t < D; ++t) xb_[t] = kl[min(b, m - 1) * KLD + t];
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
            s0[u] += fabsf(r.x - xb_[t]);
            s1[u] += fabsf(r.y - xb_[t + 1]);
            s0[u] += fabsf(r.z - xb_[t + 2]);
            s1[u] += fabsf(r.w - xb_[t + 3]);
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
    if (tid == 0) {
      alpha_s = cm * cm;
      norm1_s = cm;
    }
  }
  __syncthreads();

  const int li = lane & 15, lk = lane >> 4;
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

  // X0 = W^T / alpha.  xr[bj][r] = X[16 w + 4 lk + r][16 bj + li], the
  // entries this lane produces in every step.
  const int n16 = iters > kFp32Steps ? iters - kFp32Steps : 0;
  const float alpha = alpha_s, norm1 = norm1_s;
  float xr[4][4];
#pragma unroll
  for (int bj = 0; bj < 4; ++bj)
#pragma unroll
    for (int r = 0; r < 4; ++r) xr[bj][r] = wl[(16 * bj + li) * kLD + 16 * w + 4 * lk + r] / alpha;
  __syncthreads();  // every lane has read W and the landmarks: their buffers are free

  const int i0 = 16 * w + 4 * lk;  // first row of this lane's entries
  // This lane's entries of X into the split layout: row-major X (four
  // 16-bit stores per part) and X^T (four consecutive entries of row
  // 16 bj + li, one 8-byte store per part).
  auto store_split = [&]() {
    uint16_t* xh16 = reinterpret_cast<uint16_t*>(xb);
    uint16_t* xl16 = xh16 + kXB;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      uint32_t h0, l0, h1, l1;
      split2(xr[bj][0], xr[bj][1], h0, l0);
      split2(xr[bj][2], xr[bj][3], h1, l1);
      const int j = 16 * bj + li;
      const uint32_t hw[4] = {h0 & 0xffffu, h0 >> 16, h1 & 0xffffu, h1 >> 16};
      const uint32_t lw[4] = {l0 & 0xffffu, l0 >> 16, l1 & 0xffffu, l1 >> 16};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        xh16[(i0 + r) * kLB + j] = (uint16_t)hw[r];
        xl16[(i0 + r) * kLB + j] = (uint16_t)lw[r];
      }
      *reinterpret_cast<uint2*>(xtb + j * kLB + i0) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(xtb + kXB + j * kLB + i0) = make_uint2(l0, l1);
    }
  };
  // The same entries into the float32 layout.
  auto store_f32 = [&]() {
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const int j = 16 * bj + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) xf[(i0 + r) * kLD + j] = xr[bj][r];
      *reinterpret_cast<float4*>(&xtf[j * kLD + i0]) = make_float4(xr[bj][0], xr[bj][1], xr[bj][2], xr[bj][3]);
    }
  };
  if (n16 > 0)
    store_split();
  else
    store_f32();
  __syncthreads();
  const unsigned long long t_steps = clk ? (unsigned long long)wall_clock64() : 0ull;

  // ---- split steps ----
  int it = 0;
  while (it < n16) {
    // Q = W X, block row w, stored transposed: Q^T[j][i] = Q[i][j].  The B
    // operand X[32 kb + 8 lk + e][16 bj + li] is row 16 bj + li of X^T.
    {
      f32x4 acc[4];
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) acc[bj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
          const int o = (16 * bj + li) * kLB + 32 * kb + 8 * lk;
          const bf16x8 bh = *reinterpret_cast<const bf16x8*>(xtb + o);
          const bf16x8 bl = *reinterpret_cast<const bf16x8*>(xtb + kXB + o);
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
        const int o = (16 * bj + li) * kLB + i0;
        *reinterpret_cast<uint2*>(qb + o) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(qb + kXB + o) = make_uint2(l0, l1);
      }
    }
    __syncthreads();
    // S = X Q, block row w; X_next = 2 X - S.
    {
      f32x4 acc[4];
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) acc[bj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int oa = (16 * w + li) * kLB + 32 * kb + 8 * lk;  // X[16 w + li][32 kb + 8 lk + e]
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(xb + oa);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(xb + kXB + oa);
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
          const int ob = (16 * bj + li) * kLB + 32 * kb + 8 * lk;  // Q[32 kb + 8 lk + e][16 bj + li]
          const bf16x8 qh = *reinterpret_cast<const bf16x8*>(qb + ob);
          const bf16x8 ql = *reinterpret_cast<const bf16x8*>(qb + kXB + ob);
          acc[bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, qh, acc[bj], 0, 0, 0);
          acc[bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, ql, acc[bj], 0, 0, 0);
          acc[bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, qh, acc[bj], 0, 0, 0);
        }
      }
      float amax = 0.f;
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          xr[bj][r] = 2.f * xr[bj][r] - acc[bj][r];
          amax = fmaxf(amax, fabsf(xr[bj][r]));
        }
      // X's block row w is read by this wavefront only, and its reads above
      // feed the products these stores depend on; X^T is not read in this
      // half of the step.
      store_split();
      amax = wave_max_nonneg(amax);
      if (lane == 0) red[w] = amax;
    }
    __syncthreads();
    ++it;
    // The guard: the same four values in every wavefront, so the decision
    // is uniform across the workgroup.  red[0..3] is next written after the
    // next step's first barrier, which every wavefront passes after this read.
    const float4 mx = *reinterpret_cast<const float4*>(red);
    if (norm1 * fmaxf(fmaxf(mx.x, mx.y), fmaxf(mx.z, mx.w)) > kSplitGuard) break;
  }
  if (n16 > 0) {
    // Into the float32 layout for the remaining steps (at least kFp32Steps),
    // from the registers.  The split buffers are dead: every wavefront passed
    // the last split step's barrier.
    store_f32();
    __syncthreads();
  }

  // ---- float32 steps ----
  for (; it < iters; ++it) {
    // Q = W X, block row w, stored transposed: qf[j][i] = Q[i][j].  B operand
    // X[4 st + lk][16 bj + li] = X^T[16 bj + li][4 st + lk].
    {
      f32x4 acc[4];
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) acc[bj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
          const float xv = xtf[(16 * bj + li) * kLD + 4 * st + lk];
          acc[bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(wreg[st], xv, acc[bj], 0, 0, 0);
        }
      }
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
        *reinterpret_cast<float4*>(&qf[(16 * bj + li) * kLD + i0]) =
            make_float4(acc[bj][0], acc[bj][1], acc[bj][2], acc[bj][3]);
    }
    __syncthreads();
    // S = X Q, block row w; X_next = 2 X - S into X and X^T.
    {
      f32x4 acc[4];
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) acc[bj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const float xa = xf[(16 * w + li) * kLD + 4 * st + lk];  // X[16 w + li][4 st + lk]
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
          const float qv = qf[(16 * bj + li) * kLD + 4 * st + lk];  // Q[4 st + lk][16 bj + li]
          acc[bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa, qv, acc[bj], 0, 0, 0);
        }
      }
#pragma unroll
      for (int bj = 0; bj < 4; ++bj)
#pragma unroll
        for (int r = 0; r < 4; ++r) xr[bj][r] = 2.f * xr[bj][r] - acc[bj][r];
      store_f32();
    }
    __syncthreads();
  }

  // X (row-major, float32 layout) to the workspace.
  float* xp = xout + (size_t)p * kMP * kMP;
  for (int e = tid; e < kMP * kMP; e += 256) xp[e] = xf[(e >> 6) * kLD + (e & 63)];
  if (clk != nullptr && tid == 0) {
    clk[3 * p + 0] = t_start;
    clk[3 * p + 1] = t_steps;
    clk[3 * p + 2] = (unsigned long long)wall_clock64();
  }
}

}  // namespace ns_detail
}  // namespace lapnys
