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
// float32 products on fp32 MFMA.  One such step squares the error the split
// steps left (at most about 1e-3 with the guard) and ends at the float32
// floor: in a float32 emulation of the schedule over the workloads and
// near-duplicate landmarks (cond(W) 40 to 1.6e5) the final residual with
// one float32 step was within 1.3x of the all-float32 schedule's, and equal
// to it wherever the guard acts.  In exact arithmetic rho after k steps
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
constexpr int kFp32Steps = 1;   // final steps on float32 products, at least
constexpr float kSplitGuard = 64.f;  // largest rho = ||W||_1 max|X| for a split step
// First step after which the guard is evaluated: in exact arithmetic rho is
// at most 2^(k/2) after k steps, at most 64 up to step 12.
constexpr int kGuardFrom = 11;
// LDS of one problem's schedule (floats).  Split steps: the row-major copy
// of X twice (the current iterate and the next), each as high and low parts,
// 4 kXB bf16 = 2 kXB floats.  Float32 steps (the same bytes): the two copies,
// 2 kMP kLD floats.  Before the steps the same region holds the staged
// landmark rows (kMP rows of D + 4 floats), then 256 partial column sums,
// alpha and ||W||_1 (at kNsRed).  Then W itself (float32, kMP rows of kLD),
// kept for the whole schedule; its padding columns 64..67 of row 0 carry the
// four wavefronts' max|X| for the guard.  54272 bytes in all: three such
// workgroups fit in a CU's 160 KB.
constexpr int kNsRegion = 2 * kXB;
static_assert(2 * kMP * kLD <= kNsRegion, "the float32 layout must fit in the split layout's bytes");
constexpr int kNsRed = kMP * (64 + 4);
static_assert(kNsRed + 260 <= kNsRegion, "the set-up sums must fit beside the staged landmarks");
constexpr int kNsWOffset = kNsRegion;
static_assert(kNsWOffset % 4 == 0, "W must start 16-byte aligned");
constexpr int kNsLdsFloats = kNsWOffset + kMP * kLD;

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
// 54272 bytes of LDS.
//
// Wavefront w owns block column w (columns [16 w, 16 w + 16)) of Q = W X,
// of S = X Q and of X: each lane holds the 16 entries X[16 bo + 4 lk + r]
// [16 w + li] (bo, r in [0, 4)) in registers, the MFMA result layout.  A
// step forms Q's block column (all of W's rows from registers, times X's
// block column from registers), then S's block column (all of X's rows,
// from the shared row-major copy, times Q's block column, still in
// registers), and writes X_next = 2X - S into the other row-major copy.
// Both products take their reduction index in the order the result layout
// holds it (see the step loops), which is what lets a block column feed the
// next product without going through LDS.  Only the row-major copy is
// shared between wavefronts, and it alternates between two buffers, so one
// barrier per step orders everything: a wavefront reads the current copy
// after every wavefront wrote it, and writes the next copy, which nobody
// reads until the following barrier.
//
// The float32 steps reduce over k in [0, 4 KS), KS = ceil(m / 4), on fp32
// MFMA 16x16x4; the split steps over k in [0, 32 KB), KB = ceil(m / 32), on
// bf16 MFMA 16x16x32.  Padding rows and columns of W and X are exact zeros
// and stay so, and every step writes all 64 x 64 entries of X_next.
//
// Problem p's W and X, for one workgroup of 256 lanes.  lds: kNsLdsFloats
// floats, 16-byte aligned.
template <int D, int KS, bool GAUSS = false>
__device__ __forceinline__ void ns_small(const float* __restrict__ kt, float* __restrict__ wout,
                                         float* __restrict__ xout, int m, float scale, float eps, int iters, int p,
                                         float* __restrict__ lds, unsigned long long* __restrict__ clk) {
  // Debug stamps (clk non-null): start, first step, end, device wall clock.
  const unsigned long long t_start = clk ? (unsigned long long)wall_clock64() : 0ull;
  // Float32 layout: the row-major X twice.
  float* xrf0 = lds;
  // Split layout (same bytes): the same two copies, each high parts then low
  // parts, columns in the split steps' reduction order.
  __bf16* xrb0 = reinterpret_cast<__bf16*>(lds);
  float* wl = lds + kNsWOffset;  // W, float32
  float* red = lds + kNsRed;     // [256] partial column sums, then alpha and ||W||_1
  float& alpha_s = red[256];
  float& norm1_s = red[257];
  float* gmax = wl + kMP;        // the guard's four max|X| (W's row 0 padding)

  // Beside the kernel-matrix workgroups on the same CUs, the solver's chain
  // of dependent products is the longer one: its wavefronts take issue
  // priority.
  __builtin_amdgcn_s_setprio(3);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const float* ktp = kt + (size_t)p * m * D;

  // W = k(K~, K~) + eps I, zero padded.  The landmark rows are staged in
  // LDS (in the X region, free until the steps start; rows of D + 4 floats,
  // so lanes reading different rows hit different banks) and W's LDS rows
  // are cleared.  Entry (b, a) for a = (b + r) mod m is formed once, by lane
  // b of the wavefront that owns the shift r (r = w, w + 4, ... up to m / 2),
  // from landmark b in registers and landmark a read from LDS, and written to
  // both (b, a) and (a, b): W is bit-symmetric by construction.  The sum runs
  // over even and odd features in increasing order, four entries at a time
  // (eight independent chains), with the next two 4-feature chunks of their
  // rows loaded ahead.
  {
    constexpr int NC = D / 4;   // 4-feature chunks
    constexpr int KSTR = D + 4;  // staged row stride (floats)
    float* ks = lds;
    {
      constexpr int kV = 64 * D / 4 / 256;  // float4 loads per lane, at most
      const int n4 = m * D / 4;
      const float4* k4 = reinterpret_cast<const float4*>(ktp);
      float4 kv[kV];
#pragma unroll
      for (int i = 0; i < kV; ++i) kv[i] = k4[min(tid + 256 * i, n4 - 1)];
#pragma unroll
      for (int i = 0; i < kV; ++i) {
        const int e4 = tid + 256 * i;
        if (e4 < n4) *reinterpret_cast<float4*>(ks + (e4 / NC) * KSTR + 4 * (e4 % NC)) = kv[i];
      }
      for (int e = tid; e < kMP * kLD; e += 256) wl[e] = 0.f;
    }
    __syncthreads();
    const int b = lane;
    const bool live = b < m;
    float xb_[D];
    {
      const float* kb = ks + min(b, m - 1) * KSTR;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float4 v4 = *reinterpret_cast<const float4*>(kb + 4 * c);
        xb_[4 * c] = v4.x;
        xb_[4 * c + 1] = v4.y;
        xb_[4 * c + 2] = v4.z;
        xb_[4 * c + 3] = v4.w;
      }
    }
    const int rmax = m / 2;
    for (int r0 = w; r0 <= rmax; r0 += 16) {  // shifts r0 + 4 u, u < 4 (wave-uniform)
      float s0[4] = {0.f, 0.f, 0.f, 0.f}, s1[4] = {0.f, 0.f, 0.f, 0.f};
      int arow[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int a = b + r0 + 4 * u;
        arow[u] = min(a >= m ? a - m : a, m - 1);
      }
      const float* ka[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) ka[u] = ks + arow[u] * KSTR;
      float4 kv[3][4];  // ring of three chunks: the current one and the next two
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int u = 0; u < 4; ++u) kv[c][u] = *reinterpret_cast<const float4*>(ka[u] + 4 * c);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c + 2 < NC) {
#pragma unroll
          for (int u = 0; u < 4; ++u) kv[(c + 2) % 3][u] = *reinterpret_cast<const float4*>(ka[u] + 4 * (c + 2));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 r = kv[c % 3][u];
          if constexpr (GAUSS) {
            const float e0 = r.x - xb_[4 * c], e1 = r.y - xb_[4 * c + 1];
            const float e2 = r.z - xb_[4 * c + 2], e3 = r.w - xb_[4 * c + 3];
            s0[u] = fmaf(e0, e0, s0[u]);
            s1[u] = fmaf(e1, e1, s1[u]);
            s0[u] = fmaf(e2, e2, s0[u]);
            s1[u] = fmaf(e3, e3, s1[u]);
          } else {
            s0[u] += fabsf(r.x - xb_[4 * c]);
            s1[u] += fabsf(r.y - xb_[4 * c + 1]);
            s0[u] += fabsf(r.z - xb_[4 * c + 2]);
            s1[u] += fabsf(r.w - xb_[4 * c + 3]);
          }
        }
        // The sums are in/out operands here, so the loads of a chunk stay
        // two chunks ahead of its arithmetic (bounded registers).
        asm volatile("" : "+v"(s0[0]), "+v"(s0[1]), "+v"(s0[2]), "+v"(s0[3]), "+v"(s1[0]), "+v"(s1[1]),
                     "+v"(s1[2]), "+v"(s1[3])::"memory");
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + 4 * u;
        // At r = m / 2 (m even) lanes b and b + r form the same pair: the
        // lower one writes it.
        if (live && r <= rmax && (2 * r != m || b < r)) {
          const int a = arow[u];
          float val = exp2f((s0[u] + s1[u]) * scale);
          if (r == 0) val += eps;
          wl[b * kLD + a] = val;
          wl[a * kLD + b] = val;
        }
      }
    }
    __syncthreads();
    // Column sums of this wavefront's rows 16 w + [0, 16), in increasing row
    // order (entries are positive).
    float csum = 0.f;
#pragma unroll
    for (int a = 0; a < 16; ++a) csum += wl[(16 * w + a) * kLD + b];
    red[w * kMP + b] = csum;
  }
  __syncthreads();

  // alpha = ||W||_1 ||W||_inf.  W is symmetric, so its largest absolute
  // column sum (the 1-norm) is also its largest row sum (the inf-norm):
  // alpha = (max_b sum_a |W[a][b]|)^2, the column sums merged from the four
  // wavefront's partial sums in wavefront order.  W goes out to the
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
  // The Gaussian kernel's iterate is usually still far from converged after
  // the given steps, where a split step's error is carried to the end: every
  // step of that form takes float32 products.
  const int n16 = !GAUSS && iters > kFp32Steps ? iters - kFp32Steps : 0;
  // Reduction index of the split steps' products: bf16 MFMA 16x16x32 kb takes
  // from lane group lk the eight k = 32 kb + 4 lk + r and 32 kb + 16 + 4 lk + r
  // (r < 4).  Those are the entries a lane holds of a block column in the
  // MFMA result layout (rows 16 bo + 4 lk + r, bo = 2 kb and 2 kb + 1), so the
  // block columns of X and Q are B operands straight from registers.  The
  // shared row-major copy of X keeps its columns in the order kpos(k), which
  // puts each lane group's eight at 32 kb + 8 lk + [0, 8): one 16-byte read.
  constexpr int KB = (4 * KS + 31) / 32;
  auto kpos = [](int k) { return (k & ~31) | (((k & 15) >> 2) << 3) | (((k >> 4) & 1) << 2) | (k & 3); };
  // W's A operands for the split steps, every row block, as high and low
  // parts: A[li][8 lk + e] of step kb for row block bi = W[16 bi + li][k(kb,
  // lk, e)] with k as above.
  u32x4 wh[4][KB], wlo[4][KB];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* wr = wl + (16 * bi + li) * kLD + 32 * kb + 16 * (i >> 1) + 4 * lk + 2 * (i & 1);
        uint32_t h, l;
        split2(wr[0], wr[1], h, l);
        wh[bi][kb][i] = h;
        wlo[bi][kb][i] = l;
      }

  // X0 = W^T / alpha (times the float32 reciprocal of alpha).  xr[bo][r] =
  // X[16 bo + 4 lk + r][16 w + li], the entries this lane produces in every
  // step.
  const float ralpha = 1.f / alpha_s, norm1 = norm1_s;
  float xr[4][4];
#pragma unroll
  for (int bo = 0; bo < 4; ++bo)
#pragma unroll
    for (int r = 0; r < 4; ++r) xr[bo][r] = wl[(16 * w + li) * kLD + 16 * bo + 4 * lk + r] * ralpha;
  __syncthreads();  // X0 read before the stores below (W stays in place)

  const int jc = 16 * w + li;  // the column of X this lane holds
  // A block column in the result layout (v[bo][r] = M[16 bo + 4 lk + r][jc])
  // split into bf16 high and low parts, two entries per word: words (bo, 0)
  // and (bo, 1) hold rows r = 0, 1 and r = 2, 3.
  auto split_cols = [&](const float (&v)[4][4], uint32_t (&hw)[4][2], uint32_t (&lw)[4][2]) {
#pragma unroll
    for (int bo = 0; bo < 4; ++bo) {
      split2(v[bo][0], v[bo][1], hw[bo][0], lw[bo][0]);
      split2(v[bo][2], v[bo][3], hw[bo][1], lw[bo][1]);
    }
  };
  // The same words as the B operands of the split steps' MFMAs kb (rows
  // 32 kb + [0, 32) of the block column: row blocks 2 kb and 2 kb + 1).
  auto b_words = [&](const uint32_t (&hw)[4][2], const uint32_t (&lw)[4][2], bf16x8 (&bh)[KB], bf16x8 (&bl)[KB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      bh[kb] = __builtin_bit_cast(bf16x8, u32x4{hw[2 * kb][0], hw[2 * kb][1], hw[2 * kb + 1][0], hw[2 * kb + 1][1]});
      bl[kb] = __builtin_bit_cast(bf16x8, u32x4{lw[2 * kb][0], lw[2 * kb][1], lw[2 * kb + 1][0], lw[2 * kb + 1][1]});
    }
  };
  // This lane's entries of X (as split words) into the split row-major copy
  // `buf`, column jc at kpos(jc): sixteen 16-bit stores per part.
  auto store_split = [&](int buf, const uint32_t (&hw)[4][2], const uint32_t (&lw)[4][2]) {
    uint16_t* xh16 = reinterpret_cast<uint16_t*>(xrb0 + buf * 2 * kXB);
    uint16_t* xl16 = xh16 + kXB;
    const int cp = kpos(jc);
#pragma unroll
    for (int bo = 0; bo < 4; ++bo) {
      const int i0 = 16 * bo + 4 * lk;
      const uint32_t h4[4] = {hw[bo][0] & 0xffffu, hw[bo][0] >> 16, hw[bo][1] & 0xffffu, hw[bo][1] >> 16};
      const uint32_t l4[4] = {lw[bo][0] & 0xffffu, lw[bo][0] >> 16, lw[bo][1] & 0xffffu, lw[bo][1] >> 16};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        xh16[(i0 + r) * kLB + cp] = (uint16_t)h4[r];
        xl16[(i0 + r) * kLB + cp] = (uint16_t)l4[r];
      }
    }
  };
  // The same entries into the float32 row-major copy (natural column order).
  auto store_f32 = [&](int buf) {
    float* xrf = xrf0 + buf * kMP * kLD;
#pragma unroll
    for (int bo = 0; bo < 4; ++bo) {
      const int i0 = 16 * bo + 4 * lk;
#pragma unroll
      for (int r = 0; r < 4; ++r) xrf[(i0 + r) * kLD + jc] = xr[bo][r];
    }
  };
  // The split words of this lane's entries of the current iterate: written
  // to the row-major copy and reused as the next step's B operands.
  uint32_t xhw[4][2], xlw[4][2];
  if (n16 > 0) {
    split_cols(xr, xhw, xlw);
    store_split(0, xhw, xlw);
  } else {
    store_f32(0);
  }
  __syncthreads();
  const unsigned long long t_steps = clk ? (unsigned long long)wall_clock64() : 0ull;

  // ---- split steps ----
  int it = 0, cur = 0;
  while (it < n16) {
    // The A operands of S = X Q[:, w], X[16 bo + li][k] from the current
    // row-major copy (every wavefront's, written before the last barrier),
    // are issued first and arrive during the first product.
    const __bf16* xh = xrb0 + cur * 2 * kXB;
    bf16x8 ah[4][KB], al[4][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int bo = 0; bo < 4; ++bo) {
        const int oa = (16 * bo + li) * kLB + 32 * kb + 8 * lk;
        ah[bo][kb] = *reinterpret_cast<const bf16x8*>(xh + oa);
        al[bo][kb] = *reinterpret_cast<const bf16x8*>(xh + kXB + oa);
      }
    // Q[:, w] = W X[:, w], the B operand from this lane's entries of X.
    f32x4 acc[4];
    {
      bf16x8 bh[KB], bl[KB];
      b_words(xhw, xlw, bh, bl);
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) acc[bi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
          acc[bi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wlo[bi][kb]), bh[kb], acc[bi], 0, 0, 0);
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
          acc[bi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wh[bi][kb]), bl[kb], acc[bi], 0, 0, 0);
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
          acc[bi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wh[bi][kb]), bh[kb], acc[bi], 0, 0, 0);
      }
    }
    // S[:, w] = X Q[:, w], the B operand from Q's block column in registers.
    {
      float q[4][4];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int r = 0; r < 4; ++r) q[bi][r] = acc[bi][r];
      uint32_t qhw[4][2], qlw[4][2];
      split_cols(q, qhw, qlw);
      bf16x8 qh[KB], ql[KB];
      b_words(qhw, qlw, qh, ql);
#pragma unroll
      for (int bo = 0; bo < 4; ++bo) acc[bo] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int bo = 0; bo < 4; ++bo) acc[bo] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[bo][kb], qh[kb], acc[bo], 0, 0, 0);
#pragma unroll
        for (int bo = 0; bo < 4; ++bo) acc[bo] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[bo][kb], ql[kb], acc[bo], 0, 0, 0);
#pragma unroll
        for (int bo = 0; bo < 4; ++bo) acc[bo] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[bo][kb], qh[kb], acc[bo], 0, 0, 0);
      }
    }
#pragma unroll
    for (int bo = 0; bo < 4; ++bo)
#pragma unroll
      for (int r = 0; r < 4; ++r) xr[bo][r] = 2.f * xr[bo][r] - acc[bo][r];
    // X_next into the other row-major copy (last read before the previous
    // barrier).
    split_cols(xr, xhw, xlw);
    store_split(cur ^ 1, xhw, xlw);
    if (it >= kGuardFrom) {
      float amax = 0.f;
#pragma unroll
      for (int bo = 0; bo < 4; ++bo)
#pragma unroll
        for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(xr[bo][r]));
      amax = wave_max_nonneg(amax);
      if (lane == 0) gmax[w] = amax;
    }
    __syncthreads();
    cur ^= 1;
    // The guard: the same four values in every wavefront, so the decision
    // is uniform across the workgroup.  gmax[0..3] is next written after
    // every wavefront has passed the next barrier, and so this read.
    if (it >= kGuardFrom) {
      const float4 mx = *reinterpret_cast<const float4*>(gmax);
      if (norm1 * fmaxf(fmaxf(mx.x, mx.y), fmaxf(mx.z, mx.w)) > kSplitGuard) {
        ++it;
        break;
      }
    }
    ++it;
  }

  // ---- float32 steps (n16 < iters whenever iters > 0, so at least kFp32Steps
  // of them follow the split steps) ----
  if (it < iters) {
    if (n16 > 0) {
      // Into the float32 layout, from the registers.  The split buffers are
      // dead: every wavefront passed the last split step's barrier.
      store_f32(0);
      cur = 0;
      __syncthreads();
    }
    // fp32 MFMA 16x16x4 (bo, r) takes k = 16 bo + 4 lk + r from lane group
    // lk: the B operands are this lane's entries of a block column (xr, then
    // Q's), and W's A operands are W[16 bi + li][16 bo + 4 lk + r].  Row
    // blocks of the reduction past the last landmark are zero and skipped.
    constexpr int NBO = (4 * KS + 15) / 16;
    float wreg[4][NBO][4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bo = 0; bo < NBO; ++bo)
#pragma unroll
        for (int r = 0; r < 4; ++r) wreg[bi][bo][r] = wl[(16 * bi + li) * kLD + 16 * bo + 4 * lk + r];
    for (; it < iters; ++it) {
      // The A operands of S = X Q[:, w]: X[16 bo + li][16 bk + 4 lk + r] from
      // the current row-major copy, one 16-byte read per (bo, bk).
      const float* xrf = xrf0 + cur * kMP * kLD;
      float4 xa[4][NBO];
#pragma unroll
      for (int bo = 0; bo < 4; ++bo)
#pragma unroll
        for (int bk = 0; bk < NBO; ++bk)
          xa[bo][bk] = *reinterpret_cast<const float4*>(xrf + (16 * bo + li) * kLD + 16 * bk + 4 * lk);
      // Q[:, w] = W X[:, w].
      f32x4 acc[4];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) acc[bi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int bk = 0; bk < NBO; ++bk)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int bi = 0; bi < 4; ++bi)
            acc[bi] = __builtin_amdgcn_mfma_f32_16x16x4f32(wreg[bi][bk][r], xr[bk][r], acc[bi], 0, 0, 0);
      float q[4][4];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int r = 0; r < 4; ++r) q[bi][r] = acc[bi][r];
      // S[:, w] = X Q[:, w].
#pragma unroll
      for (int bo = 0; bo < 4; ++bo) acc[bo] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int bk = 0; bk < NBO; ++bk) {
#pragma unroll
        for (int bo = 0; bo < 4; ++bo) acc[bo] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[bo][bk].x, q[bk][0], acc[bo], 0, 0, 0);
#pragma unroll
        for (int bo = 0; bo < 4; ++bo) acc[bo] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[bo][bk].y, q[bk][1], acc[bo], 0, 0, 0);
#pragma unroll
        for (int bo = 0; bo < 4; ++bo) acc[bo] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[bo][bk].z, q[bk][2], acc[bo], 0, 0, 0);
#pragma unroll
        for (int bo = 0; bo < 4; ++bo) acc[bo] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[bo][bk].w, q[bk][3], acc[bo], 0, 0, 0);
      }
#pragma unroll
      for (int bo = 0; bo < 4; ++bo)
#pragma unroll
        for (int r = 0; r < 4; ++r) xr[bo][r] = 2.f * xr[bo][r] - acc[bo][r];
      store_f32(cur ^ 1);
      __syncthreads();
      cur ^= 1;
    }
  }

  // X (row-major, float32 layout, copy cur) to the workspace.
  float* xp = xout + (size_t)p * kMP * kMP;
  const float* xf = xrf0 + cur * kMP * kLD;
  for (int e = tid; e < kMP * kMP; e += 256) xp[e] = xf[(e >> 6) * kLD + (e & 63)];
  if (clk != nullptr && tid == 0) {
    clk[3 * p + 0] = t_start;
    clk[3 * p + 1] = t_steps;
    clk[3 * p + 2] = (unsigned long long)wall_clock64();
  }
}

}  // namespace ns_detail
}  // namespace lapnys
