// Landmark Gram matrix and its Newton-Schulz inverse (EN page, section 2.C.2;
// DE section 2; ZH section 2.2; KO section 2.3; JA section 2.3).
//
//   W  = k(K~, K~) + eps I,   k(x, y) = exp(-||x - y||_1 / lambda)
//   X0 = W^T / (||W||_1 ||W||_inf)
//   X <- X (2I - W X), a fixed number of times, matrix products only.
//
// W is built so that it is bit-symmetric: entry (a, b) and entry (b, a) sum
// the same |differences| in the same feature order, and the diagonal is
// exp(0) + eps = 1 + eps exactly as float32 arithmetic gives it.
//
// Two schedules:
//  * m <= 64: one workgroup per problem keeps W and the iterates in LDS and
//    runs inside the kernel-matrix stage's launch (ns_small.hpp, l1exp.hip).
//  * 64 < m <= 256 (this file): the products are too large for one LDS; W and
//    the iterates live in the workspace (L2-resident) and each step is one
//    batched launch (ns_step_kernel) that forms the next iterate column block
//    by column block.  A general 64 x 64 tile product (gemm64_kernel) forms
//    Y = X (B V) for these sizes and the optional correction below.
//
// Optional correction (LAPNYS_NS_REFINE, beyond the pages' fixed-count
// iteration), for either schedule: R = I - W X with float64 accumulation, then
// X <- X + X R on the tile kernel.  Exactly, the new residual is R^2; the
// float64 residual lets it reach the float32 representation floor of W^-1
// where the float32 products of the steps themselves stall above it.
#include "lapnys_internal.hpp"
#include "ns_small.hpp"

namespace lapnys {

namespace {

// ---- 64 < m <= 256 -------------------------------------------------------

// W rows [16*blockIdx.x, +16) of problem blockIdx.y (the Laplacian kernel,
// or with GAUSS the Gaussian one, exp(-sum_t (x_t - y_t)^2 / lambda), its
// squared differences summed directly); thread b owns column b
// and also writes the sum of its 16 entries (all positive) to
// part[p][blockIdx.x][b], the block's share of the column sums.  Loads read
// clamped, in-bounds addresses (rows past m are masked where used), so every
// load of the block issues before the first wait.
template <int D, bool GAUSS>
__global__ __launch_bounds__(256) void wbuild_big_kernel(const float* __restrict__ kt, float* __restrict__ w,
                                                         float* __restrict__ part, int m, int mp, float scale,
                                                         float eps) {
  __shared__ float kl[16 * D];
  const int p = blockIdx.y, a0 = blockIdx.x * 16, b = threadIdx.x;
  const float* ktp = kt + (size_t)p * m * D;
  constexpr int kPer = 16 * D / 256;
  float kv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = threadIdx.x + 256 * i;
    kv[i] = ktp[(size_t)min(a0 + e / D, m - 1) * D + e % D];
  }
  // Column landmark b: D / 4 16-byte loads (rows are 16-byte aligned).
  float xb[D];
  const float4* kb4 = reinterpret_cast<const float4*>(ktp + (size_t)min(b, m - 1) * D);
#pragma unroll
  for (int t = 0; t < D / 4; ++t) {
    const float4 v4 = kb4[t];
    xb[4 * t] = v4.x;
    xb[4 * t + 1] = v4.y;
    xb[4 * t + 2] = v4.z;
    xb[4 * t + 3] = v4.w;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) kl[threadIdx.x + 256 * i] = kv[i];
  __syncthreads();
  if (b >= mp) return;
  float csum = 0.f;
  for (int r = 0; r < 16; ++r) {
    const int a = a0 + r;
    float val = 0.f;
    if (a < m && b < m) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int t = 0; t < D; t += 2) {
        const float e0 = kl[r * D + t] - xb[t], e1 = kl[r * D + t + 1] - xb[t + 1];
        if constexpr (GAUSS) {
          s0 = fmaf(e0, e0, s0);
          s1 = fmaf(e1, e1, s1);
        } else {
          s0 += fabsf(e0);
          s1 += fabsf(e1);
        }
      }
      val = exp2f((s0 + s1) * scale);
      if (a == b) val += eps;
    }
    w[((size_t)p * mp + a) * mp + b] = val;
    csum += val;
  }
  part[((size_t)p * (mp / 16) + blockIdx.x) * mp + b] = csum;
}

// alpha and rows [blockIdx.y mp / 16, +mp / 16) of X0 = W^T / alpha for
// problem blockIdx.x (every workgroup of a problem forms the same alpha from
// the same partials, in the same order).  W is bit-symmetric
// (entry (a, b) sums the same |differences| in the same order as (b, a)), so
// its 1-norm and inf-norm are the same largest column sum and W^T = W: alpha
// = (max column sum)^2 and X0 = W / alpha, read row-major.  Column sums: one
// lane per column adds the W build's mp / 16 (<= 16) partial sums in block
// order, all loaded at once.
__global__ __launch_bounds__(256) void alpha_x0_kernel(const float* __restrict__ w, const float* __restrict__ part,
                                                       float* __restrict__ x, int mp) {
  __shared__ float red[4];
  const int p = blockIdx.x, tid = threadIdx.x;
  const float* wp = w + (size_t)p * mp * mp;
  const int nblk = mp / 16;  // also the rows of this workgroup's X0 slab
  float cs = 0.f;
  if (tid < mp) {
    const float* pp = part + (size_t)p * nblk * mp + tid;
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = pp[(size_t)min(u, nblk - 1) * mp];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (u < nblk) cs += v[u];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cs = fmaxf(cs, __shfl_xor(cs, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = cs;
  __syncthreads();
  const float cm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float alpha = cm * cm;
  // The slab: nblk rows of mp = 16 nblk^2 entries, nblk^2 / 16 per lane.
  const size_t slab = (size_t)blockIdx.y * nblk * mp;
  float* xp = x + (size_t)p * mp * mp + slab;
  const float* ws = wp + slab;
  for (int e0 = tid; e0 < nblk * mp; e0 += 256 * 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = ws[min(e0 + 256 * u, nblk * mp - 1)];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (e0 + 256 * u < nblk * mp) xp[e0 + 256 * u] = v[u] / alpha;
  }
}

// One 64 x 64 output tile (blockIdx.x, blockIdx.y) of problem blockIdx.z:
//   C = A B (mode 0),  C = A (2I - B) (mode 1)  or  C = A + A B (mode 2),
// reduction over [0, kext) (a multiple of 32), 32 at a time.  A stage's A
// (64 x 32) and B (32 x 64) values are loaded into registers, two 16-byte
// loads of each per lane, one stage ahead, and stored to the LDS buffer not
// being read, so the loads overlap the products of the stage before.  B
// entries outside [0, brows) x [0, bcols) read a clamped, in-bounds address
// and are zeroed (before the 2I transform); C is stored for rows < crows and
// columns < ccols.  Each of the four wavefronts owns a 32 x 32 block and
// issues fp32 MFMA 32x32x2.  A's rows r0 + [0, 64) and columns [0, kext)
// must be in range (lda and the row count are multiples of 64, kext <= lda).
__global__ __launch_bounds__(256) void gemm64_kernel(const float* __restrict__ A, int lda, long long sa,
                                                     const float* __restrict__ B, int ldb, long long sb, int brows,
                                                     int bcols, float* __restrict__ C, int ldc, long long sc,
                                                     int crows, int ccols, int kext, int mode) {
  __shared__ float as[2][64 * 33];
  __shared__ __align__(16) float bs[2][32 * 64];
  const int p = blockIdx.z, r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wr = w >> 1, wc = w & 1, li = lane & 31, lk = lane >> 5;
  const float* Ap = A + p * sa;
  const float* Bp = B + p * sb;
  float4 ra[2], rb[2];
  auto load = [&](int kc) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e4 = tid + 256 * i;
      const int r = e4 >> 3, c4 = 4 * (e4 & 7);  // A: 64 rows of 8 float4
      ra[i] = *reinterpret_cast<const float4*>(Ap + (size_t)(r0 + r) * lda + kc + c4);
      const int br = e4 >> 4, bc4 = 4 * (e4 & 15);  // B: 32 rows of 16 float4
      const int gr = kc + br, gc = c0 + bc4;
      rb[i] = *reinterpret_cast<const float4*>(Bp + (size_t)min(gr, brows - 1) * ldb + min(gc, bcols - 4));
    }
  };
  auto store = [&](int kc, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e4 = tid + 256 * i;
      const int r = e4 >> 3, c4 = 4 * (e4 & 7);
      float* ad = &as[buf][r * 33 + c4];
      ad[0] = ra[i].x;
      ad[1] = ra[i].y;
      ad[2] = ra[i].z;
      ad[3] = ra[i].w;
      const int br = e4 >> 4, bc4 = 4 * (e4 & 15);
      const int gr = kc + br, gc = c0 + bc4;
      float bv[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (!(gr < brows && gc + u < bcols)) bv[u] = 0.f;
        if (mode == 1) bv[u] = (gr == gc + u ? 2.f : 0.f) - bv[u];
      }
      *reinterpret_cast<float4*>(&bs[buf][br * 64 + bc4]) = make_float4(bv[0], bv[1], bv[2], bv[3]);
    }
  };
  f32x16 acc = {0.f};
  load(0);
  store(0, 0);
  __syncthreads();
  for (int kc = 0; kc < kext; kc += 32) {
    const int cur = (kc >> 5) & 1;
    const bool more = kc + 32 < kext;
    if (more) load(kc + 32);  // lands during this stage's products
#pragma unroll
    for (int k0 = 0; k0 < 32; k0 += 2) {
      const float a = as[cur][(32 * wr + li) * 33 + k0 + lk];
      const float b = bs[cur][(k0 + lk) * 64 + 32 * wc + li];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    // The other buffer was last read in the stage before, behind the barrier
    // that ended it.
    if (more) store(kc + 32, cur ^ 1);
    __syncthreads();
  }
  float* Cp = C + p * sc;
  const int cc = c0 + 32 * wc + li;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rr = r0 + 32 * wr + 8 * (r >> 2) + 4 * lk + (r & 3);
    if (rr < crows && cc < ccols) Cp[(size_t)rr * ldc + cc] = mode == 2 ? Ap[(size_t)rr * lda + cc] + acc[r] : acc[r];
  }
}

// ---- the Newton-Schulz steps at 64 < m <= 256 ------------------------------
//
// One launch per step.  Column block c (16 columns) of the next iterate,
//   X'[:, c] = X (2 E_c - W X[:, c]),    E_c the same columns of I,
// needs W, X and that block of X only, so a workgroup forms it from the
// previous iterate alone: Q_c = W X[:, c] (mp x 16), T_c = 2 E_c - Q_c, then
// X T_c for its share of the rows.  Column by column this is the step
// X (2I - W X) itself, so the iteration keeps its self-correction of the
// residual I - W X.  (The row-block form (2I - X W) X corrects I - X W
// instead; emulated in float32 at m = 256 it left W X - I ten times larger.)
// A workgroup that forms only part of the rows of X T_c repeats Q_c, which the
// other parts of its column block form too: at m = 256 and eight problems two
// parts of 128 rows give 256 workgroups, one per CU, for 1.5 times the
// step's flops (pick_step weighs this against the number of workgroups).
//
// Every product is float32 on fp32 MFMA 16x16x4.  (Split bf16 products, as in
// the in-LDS schedule for m <= 64, lose here: while the iteration has not yet
// converged along W's small eigenvalues, the error of a step is carried to
// the end at the same relative size instead of being squared away.)  MFMA
// (q, c), c < 8, takes k = 32 q + 8 lk + c from lane group lk, so every
// operand is a 16-byte read.  W's rows and X's rows come from global memory
// (each element read once per workgroup; L2-resident), kStepPD chunks of k
// ahead of the products; X[:, c] and T_c sit transposed in LDS.  Workgroup b
// takes problem b % P: when P is a multiple of 8 all workgroups of a problem
// run on one XCD and share its L2.  Measured at m = 256 and eight problems:
// 11.5 us per launch, bound by the L2-to-CU transfer of the 384 KB each
// workgroup reads (W whole and its part of X, about 35 GB/s per CU), not by
// the MFMAs (5.5 us at their issue rate).  Rows and columns past m hold zeros
// in W and X and stay zero (T_c's identity there meets zero columns of X),
// and a reduction over all mp terms equals the one over m: the added terms
// are exact zeros.
constexpr int kStepPD = 2;  // 32-deep chunks of k loaded ahead of the products

// Eight consecutive k of one row, k = 32 q + [0, 8) from row (the caller
// adds 8 lk): two adjacent 16-byte loads.  Across the four lane groups each
// load instruction touches every 128-byte line of a row's chunk, so a row's
// chunk costs the L2 two line requests, not four.
struct K8 {
  float4 lo, hi;
};
__device__ __forceinline__ K8 load_k8(const float* row, int q) {
  const float* a = row + 32 * q;
  return K8{*reinterpret_cast<const float4*>(a), *reinterpret_cast<const float4*>(a + 4)};
}

// acc += A B over the eight k of a chunk: MFMA c takes k = 32 q + 8 lk + c
// from lane group lk (A from a, B from b).
__device__ __forceinline__ f32x4 mfma_k8(const K8& a, const K8& b, f32x4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
  return acc;
}

// Column block blockIdx.x / P % (MP / 16), rows [64 TPW part, +64 TPW) with
// part = blockIdx.x / P / (MP / 16), of problem blockIdx.x % P, with NW
// wavefronts (eight give each SIMD two, whose loads and products overlap).
// Matrices are MP x MP float32 row-major, problem p at p MP^2.  xn must not
// alias x.
template <int MP, int TPW, int NW>
__global__ __launch_bounds__(64 * NW) void ns_step_kernel(const float* __restrict__ w, const float* __restrict__ x,
                                                          float* __restrict__ xn, int P) {
  static_assert((MP / 16) % NW == 0 && (4 * TPW) % NW == 0, "row tiles must split evenly over the wavefronts");
  constexpr int NT = 64 * NW;          // lanes
  constexpr int NT1 = MP / 16 / NW;    // Q_c row tiles per wavefront
  constexpr int NT2 = 4 * TPW / NW;    // output row tiles per wavefront
  constexpr int NCB = MP / 16;  // column blocks
  constexpr int NQ = MP / 32;   // 32-deep chunks of k
  constexpr int KS = MP + 4;    // LDS row stride (floats) of the transposed blocks
  __shared__ __align__(16) float xc[16 * KS];  // xc[j][k] = X[k][c0 + j]
  __shared__ __align__(16) float tt[16 * KS];  // tt[j][k] = T_c[k][j]
  const int b = blockIdx.x, p = b % P, rest = b / P;
  const int c0 = 16 * (rest % NCB), r0 = 64 * TPW * (rest / NCB);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, li = lane & 15, lk = lane >> 4;
  const size_t sq = (size_t)MP * MP;
  const float* wp = w + p * sq;
  const float* xp = x + p * sq;

  // X[:, c0 + [0, 16)): MP rows of four 16-byte loads, transposed into xc.
  constexpr int kXc = 4 * MP / NT;
  float4 xv[kXc];
#pragma unroll
  for (int i = 0; i < kXc; ++i) {
    const int e = tid + NT * i;
    xv[i] = *reinterpret_cast<const float4*>(xp + (size_t)(e >> 2) * MP + c0 + 4 * (e & 3));
  }
  // W rows 16 (wv + NW u) + li of Q_c's row tiles u, the first kStepPD chunks.
  const float* wrow = wp + (size_t)(16 * wv + li) * MP + 8 * lk;
  K8 wa[kStepPD][NT1];
#pragma unroll
  for (int s = 0; s < kStepPD; ++s)
#pragma unroll
    for (int u = 0; u < NT1; ++u) wa[s][u] = load_k8(wrow + (size_t)16 * NW * u * MP, s);
#pragma unroll
  for (int i = 0; i < kXc; ++i) {
    const int e = tid + NT * i, k = e >> 2, j = 4 * (e & 3);
    xc[j * KS + k] = xv[i].x;
    xc[(j + 1) * KS + k] = xv[i].y;
    xc[(j + 2) * KS + k] = xv[i].z;
    xc[(j + 3) * KS + k] = xv[i].w;
  }
  __syncthreads();

  // Q_c row tiles wv + NW u: acc1[u][q & 1] accumulates chunk q.  Chunk q's
  // products, then chunk q + 1's LDS operand and chunk q + kStepPD's W loads;
  // the scheduling barrier keeps the compiler from sinking the loads to
  // their use, which would expose their latency at every chunk.
  f32x4 acc1[NT1][2];
#pragma unroll
  for (int u = 0; u < NT1; ++u) acc1[u][0] = acc1[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float* xcl = xc + li * KS + 8 * lk;
  K8 bx = load_k8(xcl, 0);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int s = q % kStepPD, h = q & 1;
#pragma unroll
    for (int u = 0; u < NT1; ++u) acc1[u][h] = mfma_k8(wa[s][u], bx, acc1[u][h]);
    if (q + 1 < NQ) bx = load_k8(xcl, q + 1);
    if (q + kStepPD < NQ) {
#pragma unroll
      for (int u = 0; u < NT1; ++u) wa[s][u] = load_k8(wrow + (size_t)16 * NW * u * MP, q + kStepPD);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // X rows r0 + 16 (wv + NW v) + li of the output row tiles v, issued before
  // T_c goes to LDS.
  const float* xrow = xp + (size_t)(r0 + 16 * wv + li) * MP + 8 * lk;
  K8 xa[kStepPD][NT2];
#pragma unroll
  for (int s = 0; s < kStepPD; ++s)
#pragma unroll
    for (int v = 0; v < NT2; ++v) xa[s][v] = load_k8(xrow + (size_t)16 * NW * v * MP, s);
  // acc1[u][.][r] sums to Q[16 (wv + NW u) + 4 lk + r][c0 + li]; T_c = 2 E_c - Q_c.
#pragma unroll
  for (int u = 0; u < NT1; ++u) {
    const int k0 = 16 * (wv + NW * u) + 4 * lk;
    float t4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) t4[r] = (k0 + r == c0 + li ? 2.f : 0.f) - (acc1[u][0][r] + acc1[u][1][r]);
    *reinterpret_cast<float4*>(tt + li * KS + k0) = make_float4(t4[0], t4[1], t4[2], t4[3]);
  }
  __syncthreads();

  // X' rows: X T_c, row tiles wv + NW v of this part.
  f32x4 acc2[NT2][2];
#pragma unroll
  for (int v = 0; v < NT2; ++v) acc2[v][0] = acc2[v][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float* ttl = tt + li * KS + 8 * lk;
  K8 bt = load_k8(ttl, 0);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int s = q % kStepPD, h = q & 1;
#pragma unroll
    for (int v = 0; v < NT2; ++v) acc2[v][h] = mfma_k8(xa[s][v], bt, acc2[v][h]);
    if (q + 1 < NQ) bt = load_k8(ttl, q + 1);
    if (q + kStepPD < NQ) {
#pragma unroll
      for (int v = 0; v < NT2; ++v) xa[s][v] = load_k8(xrow + (size_t)16 * NW * v * MP, q + kStepPD);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // acc2[v][.][r] sums to X'[r0 + 16 (wv + NW v) + 4 lk + r][c0 + li]: 16
  // lanes write 64 contiguous bytes of a row.
  float* xo = xn + p * sq + c0 + li;
#pragma unroll
  for (int v = 0; v < NT2; ++v)
#pragma unroll
    for (int r = 0; r < 4; ++r) xo[(size_t)(r0 + 16 * (wv + NW * v) + 4 * lk + r) * MP] = acc2[v][0][r] + acc2[v][1][r];
}

using StepKernel = void (*)(const float*, const float*, float*, int);

// The step kernel for padded size mp and P problems, its grid and workgroup
// size.  Row parts of 64 TPW rows: fewer parts repeat Q_c less, more parts
// give more workgroups; the choice minimises (rounds of 256 workgroups) x
// (MFMAs per SIMD, proportional to MP / 64 + TPW), ties to fewer workgroups.
struct StepChoice {
  StepKernel k;
  unsigned grid, threads;
};
StepChoice pick_step(int mp, int P) {
  struct Cand { int tpw, nw; StepKernel k; };
  static const Cand c256[] = {{4, 8, ns_step_kernel<256, 4, 8>}, {2, 8, ns_step_kernel<256, 2, 8>},
                              {1, 4, ns_step_kernel<256, 1, 4>}};
  static const Cand c192[] = {{3, 4, ns_step_kernel<192, 3, 4>}, {1, 4, ns_step_kernel<192, 1, 4>}};
  static const Cand c128[] = {{2, 8, ns_step_kernel<128, 2, 8>}, {1, 4, ns_step_kernel<128, 1, 4>}};
  StepChoice best{nullptr, 0, 0};
  if (mp != 128 && mp != 192 && mp != 256) return best;
  const Cand* c = mp == 256 ? c256 : mp == 192 ? c192 : c128;
  const int n = mp == 256 ? 3 : 2;
  long long best_cost = 0;
  for (int i = 0; i < n; ++i) {
    const long long wgs = (long long)P * (mp / 16) * (mp / (64 * c[i].tpw));
    const long long cost = ((wgs + 255) / 256) * (mp / 64 + c[i].tpw);
    if (!best.k || cost < best_cost) {
      best = StepChoice{c[i].k, (unsigned)wgs, 64u * c[i].nw};
      best_cost = cost;
    }
  }
  return best;
}

// The residual R = I - W X of one 32 x 32 tile (blockIdx.x, blockIdx.y) of
// problem blockIdx.z, accumulated in float64: every product of two float32
// values is exact in float64, and the sums of at most 256 of them carry
// about 2^-45 relative error, so R keeps its leading digits even where
// W X agrees with I to float32 precision (there a float32 sum would return
// mostly rounding noise).  The identity is restricted to [0, m); W's rows and
// X's columns past m are zero, so R is zero outside the m x m block.  The
// reduction runs over [0, kext), 32 at a time, in ascending order.  Each
// stage's operands are widened to float64 once, as they are staged in LDS (W
// transposed); lane (ty, tx) owns rows 2 ty + [0, 2) and columns 2 tx + [0, 2)
// and reads both operand pairs as 16-byte loads.  Small tiles give the launch
// 16 (mp / 64)^2 workgroups per problem, enough to cover the chip at m = 256.
__global__ __launch_bounds__(256) void residual_kernel(const float* __restrict__ W, const float* __restrict__ X,
                                                       float* __restrict__ R, int m, int mp, int kext) {
  constexpr int kS = 34;
  __shared__ __align__(16) double at[32 * kS];  // at[k][row] = W[r0 + row][kc + k]
  __shared__ __align__(16) double bt[32 * kS];  // bt[k][col] = X[kc + k][c0 + col]
  const int p = blockIdx.z, r0 = blockIdx.x * 32, c0 = blockIdx.y * 32;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int sr = tid >> 3, s4 = 4 * (tid & 7);  // staging: row (or k) and 4 consecutive columns
  const size_t sq = (size_t)mp * mp;
  const float* Wp = W + p * sq;
  const float* Xp = X + p * sq;
  double acc[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
  for (int kc = 0; kc < kext; kc += 32) {
    const f32x4 wa = *reinterpret_cast<const f32x4*>(Wp + (size_t)(r0 + sr) * mp + kc + s4);
    const f32x4 xb = *reinterpret_cast<const f32x4*>(Xp + (size_t)(kc + sr) * mp + c0 + s4);
    __syncthreads();  // the stage before has finished reading
#pragma unroll
    for (int u = 0; u < 4; ++u) at[(s4 + u) * kS + sr] = (double)wa[u];
    *reinterpret_cast<double2*>(&bt[sr * kS + s4]) = make_double2(xb[0], xb[1]);
    *reinterpret_cast<double2*>(&bt[sr * kS + s4 + 2]) = make_double2(xb[2], xb[3]);
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
      const double2 a = *reinterpret_cast<const double2*>(&at[k * kS + 2 * ty]);
      const double2 b = *reinterpret_cast<const double2*>(&bt[k * kS + 2 * tx]);
      acc[0][0] = fma(a.x, b.x, acc[0][0]);
      acc[0][1] = fma(a.x, b.y, acc[0][1]);
      acc[1][0] = fma(a.y, b.x, acc[1][0]);
      acc[1][1] = fma(a.y, b.y, acc[1][1]);
    }
  }
  float* Rp = R + p * sq;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = r0 + 2 * ty + i, col = c0 + 2 * tx;
    const double d0 = row == col && row < m ? 1.0 : 0.0;
    const double d1 = row == col + 1 && row < m ? 1.0 : 0.0;
    *reinterpret_cast<f32x2*>(Rp + (size_t)row * mp + col) = (f32x2){(float)(d0 - acc[i][0]), (float)(d1 - acc[i][1])};
  }
}

// m <= 64, the plain steps (LAPNYS_NS_PLAIN, the Laplacian kernel): W, alpha,
// X0 and the steps X <- X (2I - W X) of one problem per workgroup, with W and
// the iterates in LDS (64 x 64, zero padded).  W's entries are formed as in
// wbuild_big_kernel (absolute differences over even and odd features, in
// increasing order, so W is bit-symmetric, and the diagonal is 1 + eps) and
// written out; alpha = (max column sum)^2 and X0 = W / alpha as in
// alpha_x0_kernel.  The steps take the tiled steps' form: T = 2I - W X in
// full, then X T, float32 products on fp32 MFMA 16x16x4 over k in [0, kext):
// the reference schedule the default one is compared with (the default forms
// 2X - X (W X) inside the kernel-matrix launch and takes its early products
// on bf16-split MFMA).
//
// Eight wavefronts: wavefront v forms block row v / 2 and column blocks
// 2 (v % 2) + [0, 2) of each product.  The reduction index is permuted so
// that lane group lk takes k in [S lk, S lk + S), S = kext / 4: every operand
// is then read as 16-byte LDS loads, four steps at a time, from row-major
// copies of W (symmetric), X, X^T and T^T.  X is double-buffered (two
// wavefronts share a block row); X^T and T^T are rewritten only after every
// wavefront has passed the barrier behind their last reads.
template <int D, int KEXT>
__global__ __launch_bounds__(512) void ns_plain_kernel(const float* __restrict__ kt, float* __restrict__ w,
                                                       float* __restrict__ x, int m, float scale, float eps,
                                                       int iters) {
  constexpr int kS = 68;  // row stride (floats): 16-byte rows, quarter-waves on distinct banks
  constexpr int kN = 64 * kS;
  extern __shared__ __align__(16) float lds[];
  float* ws = lds;            // W
  float* xr = ws + kN;        // X, two buffers
  float* xt = xr + 2 * kN;    // X^T
  float* tt = xt + kN;        // T^T
  const int p = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int br = wv >> 1, bc0 = 2 * (wv & 1);
  // The reduction extent is a compile-time constant, so each product's loop
  // unrolls and its LDS reads are issued ahead of the MFMAs (with a runtime
  // extent every four k-steps waited for their reads).
  constexpr int S = KEXT / 4;
  f32x4* w4 = reinterpret_cast<f32x4*>(w + (size_t)p * 64 * 64);
  f32x4* x4 = reinterpret_cast<f32x4*>(x + (size_t)p * 64 * 64);
  {
    // Landmark rows (zero past m) into the T^T buffer, every load issued
    // before the first store.
    constexpr int kQ = D / 4;
    constexpr int kV = 64 * kQ / 512;
    const f32x4* k4 = reinterpret_cast<const f32x4*>(kt + (size_t)p * m * D);
    f32x4 kv[kV];
#pragma unroll
    for (int i = 0; i < kV; ++i) {
      const int e = tid + 512 * i;
      kv[i] = k4[min(e / kQ, m - 1) * kQ + e % kQ];
    }
#pragma unroll
    for (int i = 0; i < kV; ++i) {
      const int e = tid + 512 * i;
      *reinterpret_cast<f32x4*>(&tt[(e / kQ) * kS + 4 * (e % kQ)]) = e / kQ < m ? kv[i] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  __syncthreads();
  {
    // W: lane b = tid % 64 forms column b for rows a = 8 g + [0, 8), g = tid / 64.
    const int b = tid & 63, g = tid >> 6;
    float kb[D];
#pragma unroll
    for (int t = 0; t < D; ++t) kb[t] = tt[b * kS + t];
    float csum = 0.f;
    for (int a = 8 * g; a < 8 * g + 8; ++a) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int t = 0; t < D; t += 2) {
        const float e0 = tt[a * kS + t] - kb[t], e1 = tt[a * kS + t + 1] - kb[t + 1];
        s0 += fabsf(e0);
        s1 += fabsf(e1);
      }
      float val = 0.f;
      if (a < m && b < m) {
        val = exp2f((s0 + s1) * scale);
        if (a == b) val += eps;
      }
      ws[a * kS + b] = val;
      csum += val;
    }
    xr[kN + g * 64 + b] = csum;  // partial column sums in the second X buffer
  }
  __syncthreads();
  if (tid < 64) {
    float cs = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) cs += xr[kN + g * 64 + tid];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cs = fmaxf(cs, __shfl_xor(cs, off, 64));
    if (tid == 0) xr[kN + 512] = cs * cs;
  }
  __syncthreads();
  const float alpha = xr[kN + 512];
  // X0 = W^T / alpha = W / alpha; W goes out to the workspace.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e4 = tid + 512 * i, row = e4 >> 4, c4 = 4 * (e4 & 15);
    const f32x4 wrow = *reinterpret_cast<const f32x4*>(&ws[row * kS + c4]);
    w4[e4] = wrow;
    f32x4 x0;
#pragma unroll
    for (int u = 0; u < 4; ++u) x0[u] = wrow[u] / alpha;
    *reinterpret_cast<f32x4*>(&xr[row * kS + c4]) = x0;
#pragma unroll
    for (int u = 0; u < 4; ++u) xt[(c4 + u) * kS + row] = x0[u];
  }
  __syncthreads();
  const int arow = (16 * br + li) * kS + S * lk;  // A operand: row 16 br + li, this lane group's k
  int brow[2];                                    // B operand: transposed row 16 bj + li
#pragma unroll
  for (int j = 0; j < 2; ++j) brow[j] = (16 * (bc0 + j) + li) * kS + S * lk;
  int cur = 0;
  for (int it = 0; it < iters; ++it) {
    const float* xc = xr + cur * kN;
    float* xn = xr + (cur ^ 1) * kN;
    f32x4 acc[2];
    // T = 2I - W X, stored transposed
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < S; c += 4) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&ws[arow + c]);
      f32x4 b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const f32x4*>(&xt[brow[j] + c]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[j][e], acc[j], 0, 0, 0);
    }
    // acc[j][r] = (W X)[16 br + 4 lk + r][16 (bc0 + j) + li]
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = 16 * (bc0 + j) + li, row0 = 16 * br + 4 * lk;
      f32x4 t;
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] = (row0 + r == col ? 2.f : 0.f) - acc[j][r];
      *reinterpret_cast<f32x4*>(&tt[col * kS + row0]) = t;
    }
    __syncthreads();  // T complete; every wavefront is done reading X^T
    // X_next = X T
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < S; c += 4) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&xc[arow + c]);
      f32x4 b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const f32x4*>(&tt[brow[j] + c]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[j][e], acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = 16 * (bc0 + j) + li, row0 = 16 * br + 4 * lk;
#pragma unroll
      for (int r = 0; r < 4; ++r) xn[(row0 + r) * kS + col] = acc[j][r];
      *reinterpret_cast<f32x4*>(&xt[col * kS + row0]) = acc[j];
    }
    __syncthreads();  // X_next and its transpose complete; T^T free
    cur ^= 1;
  }
  const float* xf = xr + cur * kN;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e4 = tid + 512 * i;
    x4[e4] = *reinterpret_cast<const f32x4*>(&xf[(e4 >> 4) * kS + 4 * (e4 & 15)]);
  }
}

// LDS of ns_plain_kernel: W, X twice, X^T and T^T, 64 rows of 68 floats each.
constexpr size_t kPlainLds = 5 * 64 * 68 * sizeof(float);

__global__ __launch_bounds__(256) void extract_square_kernel(const float* __restrict__ src, int src_ld,
                                                             float* __restrict__ dst, int n, long long total) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total) return;
  const long long p = e / ((long long)n * n);
  const int rem = (int)(e % ((long long)n * n));
  const int a = rem / n, b = rem % n;
  dst[e] = src[(p * src_ld + a) * src_ld + b];
}

// The Gaussian kernel's solver for m <= 64: the Laplacian form's in-LDS
// schedule (ns_small.hpp: each entry of W formed once per pair, the block
// columns of X in registers, one barrier per step) with W from squared
// differences and every step on float32 products, as a launch of its own
// beside the kernel-matrix stage: one workgroup of 256 lanes per problem.
template <int D, int KS>
__global__ __launch_bounds__(256) void ns_gauss_kernel(const float* __restrict__ kt, float* __restrict__ w,
                                                       float* __restrict__ x, int m, float scale, float eps,
                                                       int iters) {
  extern __shared__ __align__(16) float lds[];
  ns_detail::ns_small<D, KS, true>(kt, w, x, m, scale, eps, iters, blockIdx.x, lds, nullptr);
}

// KS = ceil(m / 4), a compile-time constant of the schedule's loops.
template <int D, int KS = 1>
hipError_t launch_ns_gauss(const Plan& pl, Work& wk, hipStream_t s, Span t) {
  if constexpr (KS < 16) {
    if ((pl.m + 3) / 4 > KS) return launch_ns_gauss<D, KS + 1>(pl, wk, s, t);
  }
  hipExtLaunchKernelGGL((ns_gauss_kernel<D, KS>), dim3(pl.P), dim3(256), ns_detail::kNsLdsFloats * sizeof(float), s,
                        t.start, pl.refine ? nullptr : t.stop, 0, wk.kt, wk.w, wk.x, pl.m, pl.scale, pl.eps,
                        pl.ns_iters);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ns(const Plan& pl, Work& wk, hipStream_t s, Span t) {
  const int kext = (pl.m + 31) & ~31;
  if (pl.fused_ns) {
    // m <= 64: the default Laplacian schedule runs inside the kernel-matrix
    // launch (launch_l1exp); the plain steps run one workgroup per problem
    // here.  kext (m rounded up to 32) is a multiple of 16, as the operand
    // reads need.
    if (pl.ns_in_launch) return hipErrorInvalidValue;
    if (pl.gaussian) {
      hipError_t err = pl.d == 64 ? launch_ns_gauss<64>(pl, wk, s, t) : launch_ns_gauss<32>(pl, wk, s, t);
      if (err != hipSuccess) return err;
      wk.x_final = wk.x;
      return pl.refine ? launch_refine(pl, wk, s, t.stop) : hipSuccess;
    }
    auto pick = [&](auto k32, auto k64) { return kext > 32 ? k64 : k32; };
    auto kern = pl.d == 64 ? pick(ns_plain_kernel<64, 32>, ns_plain_kernel<64, 64>)
                           : pick(ns_plain_kernel<32, 32>, ns_plain_kernel<32, 64>);
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)kPlainLds);
    if (err != hipSuccess) return err;
    hipExtLaunchKernelGGL(kern, dim3(pl.P), dim3(512), kPlainLds, s, t.start, pl.refine ? nullptr : t.stop, 0, wk.kt,
                          wk.w, wk.x, pl.m, pl.scale, pl.eps, pl.ns_iters);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    wk.x_final = wk.x;
    return pl.refine ? launch_refine(pl, wk, s, t.stop) : hipSuccess;
  }
  const int mp = pl.mp;
  auto wbuild = pl.d == 64 ? (pl.gaussian ? wbuild_big_kernel<64, true> : wbuild_big_kernel<64, false>)
                           : (pl.gaussian ? wbuild_big_kernel<32, true> : wbuild_big_kernel<32, false>);
  hipExtLaunchKernelGGL(wbuild, dim3(mp / 16, pl.P), dim3(256), 0, s, t.start, pl.cg ? t.stop : nullptr, 0, wk.kt,
                        wk.w, wk.pm, pl.m, mp, pl.scale, pl.eps);
  if (pl.cg) return hipGetLastError();  // the CG solve (cg.hip) needs W only
  // The column-sum partials go to the product buffer, which the steps only
  // write after alpha_x0 has read them.
  const int T = pl.ns_iters;
  hipExtLaunchKernelGGL(alpha_x0_kernel, dim3(pl.P, 16), dim3(256), 0, s, nullptr,
                        T == 0 && !pl.refine ? t.stop : nullptr, 0, wk.w, wk.pm, wk.x, mp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // Iterates alternate by step between the two buffers.
  float* const xf[2] = {wk.x, wk.x2};
  const StepChoice step = pick_step(mp, pl.P);
  if (!step.k) return hipErrorInvalidValue;
  for (int it = 0; it < T; ++it) {
    hipExtLaunchKernelGGL(step.k, dim3(step.grid), dim3(step.threads), 0, s, nullptr,
                          it + 1 == T && !pl.refine ? t.stop : nullptr,
                          0, (const float*)wk.w, (const float*)xf[it & 1], xf[(it + 1) & 1], pl.P);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  wk.x_final = xf[T & 1];
  return pl.refine ? launch_refine(pl, wk, s, t.stop) : hipSuccess;
}

hipError_t launch_refine(const Plan& pl, Work& wk, hipStream_t s, hipEvent_t stop) {
  const int mp = pl.mp;
  const int kext = (pl.m + 31) & ~31;
  const long long sq = (long long)mp * mp;
  const dim3 grid(mp / 64, mp / 64, pl.P);
  float* xc = wk.x_final;
  float* xn = xc == wk.x ? wk.x2 : wk.x;
  hipLaunchKernelGGL(residual_kernel, dim3(mp / 32, mp / 32, pl.P), dim3(256), 0, s, wk.w, xc, wk.pm, pl.m, mp, kext);
  hipExtLaunchKernelGGL(gemm64_kernel, grid, dim3(256), 0, s, nullptr, stop, 0, xc, mp, sq, wk.pm, mp, sq, mp, mp,
                        xn, mp, sq, mp, mp, kext, 2);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  wk.x_final = xn;
  return hipSuccess;
}

hipError_t launch_y(const Plan& pl, const Work& wk, hipStream_t s, Span t) {
  const int kext = (pl.m + 31) & ~31;
  const long long md = (long long)pl.m * pl.d;
  hipExtLaunchKernelGGL(gemm64_kernel, dim3((pl.m + 63) / 64, (pl.d + 63) / 64, pl.P), dim3(256), 0, s, t.start,
                        t.stop, 0, wk.x_final,
                     pl.mp, (long long)pl.mp * pl.mp, wk.bv, pl.d, md, pl.m, pl.d, wk.y, pl.d, md, pl.m, pl.d, kext, 0);
  return hipGetLastError();
}

hipError_t launch_gemm(const float* A, int lda, long long sa, const float* B, int ldb, long long sb, int brows,
                       int bcols, float* C, int ldc, long long sc, int crows, int ccols, int kext, int P,
                       hipStream_t s) {
  hipLaunchKernelGGL(gemm64_kernel, dim3((crows + 63) / 64, (ccols + 63) / 64, P), dim3(256), 0, s, A, lda, sa, B,
                     ldb, sb, brows, bcols, C, ldc, sc, crows, ccols, kext, 0);
  return hipGetLastError();
}

hipError_t launch_extract_square(const float* src, int src_ld, float* dst, int n, int P, hipStream_t s) {
  const long long total = (long long)P * n * n;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(extract_square_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, src, src_ld,
                     dst, n, total);
  return hipGetLastError();
}

}  // namespace lapnys
