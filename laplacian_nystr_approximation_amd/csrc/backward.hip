// Backward pass of the Laplacian-kernel Nystrom attention (the pages' kernels
// serve the forward and the backward pass: EN page, section 3; the L1 kernel's
// gradient stays away from zero near coincident points: EN section 2.A).  The
// gradients of sum(dO * O) with respect to Q, K and V after a forward call has
// filled the workspace.  X stands for W^-1 in the derivative
// (the implicit reading: dW = -X^T dX X^T), which the converged Newton-Schulz
// iterate approximates.  Per problem, with Z = (C - mu) / sigma, Y = X (B V),
// O = Z Y, g = dO:
//
//   dY = Z^T g = (C^T g - mu (1^T g)) / sigma
//   dC_ij = (g_i . Y_j - a_j - Z_ij b_j) / sigma_j,
//       a_j = (1^T g) . Y_j / N,  b_j = Y_j . dY_j / N   (the whitening backward)
//   G = dC (.) C;  dQ_i = -(1/lambda) sum_j G_ij sign(q_i - K~_j)
//   dBV = X^T dY;  dX = dY BV^T;  dW = -X^T dX X^T
//   H_jn = (dBV_j . v_n) B_jn;  dV_n = sum_j B_jn dBV_j
//   dK_n = (1/lambda) sum_j H_jn sign(K~_j - k_n) + dK~_{j(n)} / pool^2
//   dK~_j = (1/lambda) [sum_i G_ij sign(q_i - K~_j) - sum_n H_jn sign(K~_j - k_n)
//                       - sum_b (dW_jb + dW_bj) W'_jb sign(K~_j - K~_b)]
//
// (W' = W without eps.)  With whitening off, mu = 0, 1/sigma = 1 and a = b = 0.
// Every kernel works in float32 with a fixed summation order, so results
// repeat bit for bit.  B comes from the forward (stored into the H^T buffer);
// the products over d or over 64-row blocks (C^T g, g Y^T, dBV V^T, B^T dBV
// and the m x m ones) run on fp32 MFMA; the sign sums run on the vector ALUs,
// the token-side ones one lane per token and 16 features, the landmark-side
// one one lane per (feature, 4 landmarks) with the tokens streamed through LDS.
#include "lapnys_internal.hpp"

namespace lapnys {

namespace {

constexpr int kBT = 256;  // tokens per tile of the token-side kernels

__device__ __forceinline__ float sgn(float x) { return x > 0.f ? 1.f : (x < 0.f ? -1.f : 0.f); }

// sign(x - y) in two instructions for the hot loops: with ys = y * 2^64
// (exact), fma(x, 2^64, -ys) is (x - y) * 2^64 rounded once, so it is zero
// exactly when x == y and has the sign of x - y; the median with -1 and 1 then
// gives -1, 0 or 1 whenever |x - y| >= 2^-64 (smaller nonzero gaps, between
// values below ~2^-40, would give a fraction).  Inputs must stay below 2^63 in
// magnitude.
constexpr float kSgnScale = 1.8446744073709552e19f;  // 2^64
__device__ __forceinline__ float sgn_diff(float x, float ys) {
  return __builtin_amdgcn_fmed3f(fmaf(x, kSgnScale, -ys), -1.f, 1.f);
}

template <typename T, int D>
__device__ __forceinline__ void load_row(const T* __restrict__ src, float (&x)[D]) {
#pragma unroll
  for (int t = 0; t < D; ++t) x[t] = widen(src[t]);
}

// Partial C^T g and 1^T g over one tile of tokens: part[p][tile][j][f],
// spart[p][tile][f].  Workgroup (tile, p, jb) takes landmarks [64 jb, 64 jb +
// 64).  The tile's tokens pass through LDS in chunks of 64 (the C^T entries of
// those landmarks, zero past m, and the rows of g); C^T g runs on fp32 MFMA
// 16x16x4, wavefront w forming landmark rows 64 jb + [16 w, 16 w + 16), and
// lanes tid < D of block 0 add up 1^T g in token order.
template <int D>
__global__ __launch_bounds__(256) void bwd_ctg_kernel(const float* __restrict__ ct, int ldc,
                                                      const float* __restrict__ dout, float* __restrict__ part,
                                                      float* __restrict__ spart, int N, int m, int ntiles) {
  constexpr int kC = 64;
  constexpr int kCS = kC + 1, kGS = D + 1;
  __shared__ float cs[64 * kCS];  // [j][i]
  __shared__ float gs[kC * kGS];  // [i][f]
  const int tile = blockIdx.x, p = blockIdx.y, j0 = 64 * blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, li = lane & 15, lk = lane >> 4;
  const int t0 = tile * kBT, nv = min(kBT, N - t0);
  const bool sums = blockIdx.z == 0;
  f32x4 acc[D / 16];
#pragma unroll
  for (int bj = 0; bj < D / 16; ++bj) acc[bj] = f32x4{0.f, 0.f, 0.f, 0.f};
  float s = 0.f;
  // Per lane, one chunk's loads (kCE entries of C^T, kGE of g), issued a chunk
  // ahead so that they land while the current chunk's products run.
  constexpr int kCE = 64 * kC / 256, kGE = kC * D / 256;
  float cr[kCE], gr[kGE];
  auto fetch = [&](int c0) {
    const int nc = min(kC, nv - c0);
#pragma unroll
    for (int u = 0; u < kCE; ++u) {
      const int e = tid + 256 * u, j = j0 + e / kC, i = e % kC;
      cr[u] = ct[((size_t)p * m + min(j, m - 1)) * ldc + t0 + c0 + min(i, nc - 1)];
    }
#pragma unroll
    for (int u = 0; u < kGE; ++u) {
      const int e = tid + 256 * u, i = e / D, f = e % D;
      gr[u] = dout[((size_t)p * N + t0 + c0 + min(i, nc - 1)) * D + f];
    }
  };
  fetch(0);
  for (int c0 = 0; c0 < nv; c0 += kC) {
    const int nc = min(kC, nv - c0);
    __syncthreads();  // the previous chunk's reads are done
#pragma unroll
    for (int u = 0; u < kCE; ++u) {
      const int e = tid + 256 * u, j = j0 + e / kC, i = e % kC;
      cs[(e / kC) * kCS + i] = (j < m && i < nc) ? cr[u] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kGE; ++u) {
      const int e = tid + 256 * u, i = e / D, f = e % D;
      gs[i * kGS + f] = i < nc ? gr[u] : 0.f;
    }
    __syncthreads();
    if (c0 + kC < nv) fetch(c0 + kC);
#pragma unroll 4
    for (int k0 = 0; k0 < kC; k0 += 4) {
      const float a = cs[(16 * w + li) * kCS + k0 + lk];
#pragma unroll
      for (int bj = 0; bj < D / 16; ++bj)
        acc[bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, gs[(k0 + lk) * kGS + 16 * bj + li], acc[bj], 0, 0, 0);
    }
    if (sums && tid < D)
      for (int i = 0; i < nc; ++i) s += gs[i * kGS + tid];
  }
  // acc[bj][r] = (C^T g)[16 w + 4 lk + r][16 bj + li]
  float* pp = part + (((size_t)p * ntiles + tile) * m) * D;
#pragma unroll
  for (int bj = 0; bj < D / 16; ++bj)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = j0 + 16 * w + 4 * lk + r;
      if (j < m) pp[(size_t)j * D + 16 * bj + li] = acc[bj][r];
    }
  if (sums && tid < D) spart[((size_t)p * ntiles + tile) * D + tid] = s;
}

// LDS of bwd_small_kernel: five 64-row matrices of row stride 65 (X, the m x m
// scratch dX, R, and B V, dY, Y of D columns), and 1^T g (D).
template <int D>
constexpr size_t bwd_small_lds() {
  return (size_t)(6 * 64 * 65 + D) * sizeof(float);
}

// out[i][j] = sum_{k < K} A(i, k) B(k, j) for i < 64, j < NC, on fp32 MFMA
// 16x16x4: wavefront w forms rows [16 w, 16 w + 16).  A(i, k) = a[i][k] or,
// with TA, a[k][i]; B(k, j) = b[k][j] or, with TB, b[j][k]; all row stride 65.
template <int NC, bool TA, bool TB>
__device__ __forceinline__ void mm64(const float* __restrict__ a, const float* __restrict__ b,
                                     float* __restrict__ out, int K, float sign) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, li = lane & 15, lk = lane >> 4;
  f32x4 acc[NC / 16];
#pragma unroll
  for (int bj = 0; bj < NC / 16; ++bj) acc[bj] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += 4) {
    const int i = 16 * w + li, k = k0 + lk;
    const float av = TA ? a[k * 65 + i] : a[i * 65 + k];
#pragma unroll
    for (int bj = 0; bj < NC / 16; ++bj) {
      const int j = 16 * bj + li;
      const float bv = TB ? b[j * 65 + k] : b[k * 65 + j];
      acc[bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[bj], 0, 0, 0);
    }
  }
#pragma unroll
  for (int bj = 0; bj < NC / 16; ++bj)
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(16 * w + 4 * lk + r) * 65 + 16 * bj + li] = sign * acc[bj][r];
}

// m <= 64, per problem (one workgroup), from dY and 1^T g (bwd_dy_kernel):
// Y, a, b, dBV and R X^T = X^T (dY BV^T) X^T = -dW, every matrix zero padded
// to 64 rows in LDS and the products on fp32 MFMA.  x: the Newton-Schulz
// result, row stride mp (= 64); dyg: dY [P][mp][D], zero rows past m.
// Outputs: y, dbv [P][m][D]; ab [P][2][m]; dw [P][mp][mp].
template <int D>
__global__ __launch_bounds__(256) void bwd_small_kernel(const float* __restrict__ dyg, const float* __restrict__ sg,
                                                        const float* __restrict__ x, int mp,
                                                        const float* __restrict__ bv, float* __restrict__ y,
                                                        float* __restrict__ dbv, float* __restrict__ ab,
                                                        float* __restrict__ dw, int N, int m, int whiten) {
  extern __shared__ __align__(16) float lds[];
  constexpr int kS = 64 * 65;
  float* xs = lds;
  float* dxs = xs + kS;
  float* rsm = dxs + kS;
  float* bvs = rsm + kS;
  float* dys = bvs + kS;
  float* ys = dys + kS;
  float* ss = ys + kS;
  const int p = blockIdx.x, tid = threadIdx.x;
  {
    // Every load is issued before the first LDS store.
    constexpr int kXE = 64 * 64 / 256, kBE = 64 * D / 256;
    float xr[kXE], br[kBE], dr[kBE];
#pragma unroll
    for (int u = 0; u < kXE; ++u) {
      const int e = tid + 256 * u, r = e >> 6, c = e & 63;
      xr[u] = x[(size_t)p * mp * mp + (size_t)min(r, m - 1) * mp + min(c, m - 1)];
    }
#pragma unroll
    for (int u = 0; u < kBE; ++u) {
      const int e = tid + 256 * u, r = e / D, c = e % D;
      br[u] = bv[((size_t)p * m + min(r, m - 1)) * D + c];
      dr[u] = dyg[((size_t)p * mp + r) * D + c];
    }
    const float sv = sg[(size_t)p * D + tid % D];
#pragma unroll
    for (int u = 0; u < kXE; ++u) {
      const int e = tid + 256 * u, r = e >> 6, c = e & 63;
      xs[r * 65 + c] = (r < m && c < m) ? xr[u] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kBE; ++u) {
      const int e = tid + 256 * u, r = e / D, c = e % D;
      bvs[r * 65 + c] = r < m ? br[u] : 0.f;
      dys[r * 65 + c] = dr[u];
    }
    if (tid < D) ss[tid] = sv;
  }
  __syncthreads();
  mm64<D, false, false>(xs, bvs, ys, 64, 1.f);  // Y = X BV
  __syncthreads();
  for (int e = tid; e < m * D; e += 256) y[(size_t)p * m * D + e] = ys[(e / D) * 65 + e % D];
  {
    // a_j = (1^T g) . Y_j / N, b_j = Y_j . dY_j / N: four lanes per landmark,
    // D / 4 features each, then merged ((0 + 1) + (2 + 3)).
    const int j = tid >> 2, q4 = tid & 3;
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int f = q4 * (D / 4); f < (q4 + 1) * (D / 4); ++f) {
      a = fmaf(ss[f], ys[j * 65 + f], a);
      b = fmaf(ys[j * 65 + f], dys[j * 65 + f], b);
    }
    a += __shfl_xor(a, 1, 64);
    b += __shfl_xor(b, 1, 64);
    a += __shfl_xor(a, 2, 64);
    b += __shfl_xor(b, 2, 64);
    if (q4 == 0 && j < m) {
      ab[(size_t)p * 2 * m + j] = whiten ? a / (float)N : 0.f;
      ab[(size_t)p * 2 * m + m + j] = whiten ? b / (float)N : 0.f;
    }
  }
  __syncthreads();
  mm64<D, true, false>(xs, dys, ys, 64, 1.f);    // dBV = X^T dY (into the Y buffer)
  mm64<64, false, true>(dys, bvs, dxs, D, 1.f);  // dX = dY BV^T
  __syncthreads();
  for (int e = tid; e < m * D; e += 256) dbv[(size_t)p * m * D + e] = ys[(e / D) * 65 + e % D];
  mm64<64, true, false>(xs, dxs, rsm, 64, 1.f);  // R = X^T dX
  __syncthreads();
  mm64<64, false, true>(rsm, xs, dxs, 64, 1.f);  // R X^T = -dW (into the dX buffer)
  __syncthreads();
  for (int e = tid; e < m * m; e += 256) dw[((size_t)p * mp + e / m) * mp + e % m] = dxs[(e / m) * 65 + e % m];
}

// dY = (C^T g - mu (1^T g)) / sigma from the partials into dy
// [P][mp][D] (zero rows past m), and 1^T g into s [P][D].
template <int D>
__global__ __launch_bounds__(256) void bwd_dy_kernel(const float* __restrict__ part, const float* __restrict__ spart,
                                                     const float* __restrict__ mu, const float* __restrict__ rs,
                                                     float* __restrict__ dy, float* __restrict__ sg, int m, int mp,
                                                     int ntiles) {
  const int p = blockIdx.y, e = blockIdx.x * 256 + threadIdx.x;
  if (e >= mp * D) return;
  const int j = e / D, f = e % D;
  float sv = 0.f;
#pragma unroll 8
  for (int t = 0; t < ntiles; ++t) sv += spart[((size_t)p * ntiles + t) * D + f];
  if (j == 0) sg[(size_t)p * D + f] = sv;
  float c = 0.f;
  if (j < m) {
#pragma unroll 8
    for (int t = 0; t < ntiles; ++t) c += part[(((size_t)p * ntiles + t) * m + j) * D + f];
    c = (c - mu[p * m + j] * sv) * rs[p * m + j];
  }
  dy[(size_t)p * mp * D + e] = c;
}

// m > 64: a_j = (1^T g) . Y_j / N and b_j = Y_j . dY_j / N (0 with whitening off).
template <int D>
__global__ __launch_bounds__(256) void bwd_ab_kernel(const float* __restrict__ y, const float* __restrict__ dy,
                                                     const float* __restrict__ sg, float* __restrict__ ab, int N,
                                                     int m, int mp, int whiten) {
  const int p = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
  if (j >= m) return;
  float a = 0.f, b = 0.f;
  for (int f = 0; f < D; ++f) {
    const float yv = y[((size_t)p * m + j) * D + f];
    a = fmaf(sg[(size_t)p * D + f], yv, a);
    b = fmaf(yv, dy[((size_t)p * mp + j) * D + f], b);
  }
  ab[(size_t)p * 2 * m + j] = whiten ? a / (float)N : 0.f;
  ab[(size_t)p * 2 * m + m + j] = whiten ? b / (float)N : 0.f;
}

// dst[c][r] = src[r][c] for r < rows, c < cols; zero for r in [rows, rp) (per
// problem; src row stride lds, dst row stride rp).
__global__ __launch_bounds__(256) void bwd_transpose_kernel(const float* __restrict__ src, int lds_, long long ss,
                                                            float* __restrict__ dst, long long sd, int rows, int cols,
                                                            int rp) {
  const int p = blockIdx.y;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= (long long)cols * rp) return;
  const int c = (int)(e / rp), r = (int)(e % rp);
  dst[p * sd + e] = r < rows ? src[p * ss + (long long)r * lds_ + c] : 0.f;
}

// Query side, first pass: G_ij = dC_ij C_ij, stored as G^T[p][j][i], with
// dC_ij = (g_ij - a_j - z_ij b_j) r_j, z_ij = (C_ij - mu_j) r_j and g = dO Y^T.
// Workgroup (tile, p) takes kGT tokens; per block of 64 landmarks, g^T for the
// tile runs on fp32 MFMA 16x16x4 from Y and the tile's rows of dO in LDS
// (2 x 64 rows of D + 1 floats at lds; wavefront w: landmarks 16 w + [0, 16)),
// and the lanes finish G^T from C^T in their own accumulator positions.
constexpr int kGT = 64;  // tokens per tile

template <int D>
__device__ __forceinline__ void bwd_g_body(float* __restrict__ lds, const float* __restrict__ dout,
                                           const float* __restrict__ ct, int ldc, const float* __restrict__ y,
                                           const float* __restrict__ mu, const float* __restrict__ rs,
                                           const float* __restrict__ ab, float* __restrict__ gt, int N, int m) {
  constexpr int kS = D + 1;
  float* ys = lds;            // [64][D+1] the block's Y rows
  float* gs = ys + 64 * kS;   // [kGT][D+1] the tile's dO rows
  const int tile = blockIdx.x, p = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, li = lane & 15, lk = lane >> 4;
  const int n0 = tile * kGT, nv = min(kGT, N - n0);
  constexpr int kE = 64 * D / 256;
  float gr[kE], yr[kE];
#pragma unroll
  for (int u = 0; u < kE; ++u) {
    const int e = tid + 256 * u, i = e / D, f = e % D;
    gr[u] = dout[((size_t)p * N + n0 + min(i, nv - 1)) * D + f];
  }
  for (int j0 = 0; j0 < m; j0 += 64) {
    const int jv = min(64, m - j0);
#pragma unroll
    for (int u = 0; u < kE; ++u) {
      const int e = tid + 256 * u, jj = e / D, f = e % D;
      yr[u] = y[((size_t)p * m + j0 + min(jj, jv - 1)) * D + f];
    }
    __syncthreads();  // the previous block's reads are done
#pragma unroll
    for (int u = 0; u < kE; ++u) {
      const int e = tid + 256 * u, r = e / D, f = e % D;
      ys[r * kS + f] = r < jv ? yr[u] : 0.f;
      if (j0 == 0) gs[r * kS + f] = r < nv ? gr[u] : 0.f;
    }
    __syncthreads();
    if (16 * w >= jv) continue;
    // The epilogue's operands are loaded before the products, from clamped
    // addresses (entries past m or past the tile are not stored), so their
    // latency overlaps the MFMAs instead of following them one load at a time.
    float cv[4][kGT / 16], rjv[4], mjv[4], ajv[4], bjv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int jc = min(j0 + 16 * w + 4 * lk + r, m - 1);
      rjv[r] = rs[p * m + jc];
      mjv[r] = mu[p * m + jc];
      ajv[r] = ab[(size_t)p * 2 * m + jc];
      bjv[r] = ab[(size_t)p * 2 * m + m + jc];
#pragma unroll
      for (int bj = 0; bj < kGT / 16; ++bj) cv[r][bj] = ct[((size_t)p * m + jc) * ldc + n0 + min(16 * bj + li, nv - 1)];
    }
    f32x4 acc[kGT / 16];
#pragma unroll
    for (int bj = 0; bj < kGT / 16; ++bj) acc[bj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int k0 = 0; k0 < D; k0 += 4) {
      const float av = ys[(16 * w + li) * kS + k0 + lk];
#pragma unroll
      for (int bj = 0; bj < kGT / 16; ++bj)
        acc[bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, gs[(16 * bj + li) * kS + k0 + lk], acc[bj], 0, 0, 0);
    }
    // acc[bj][r] = g[token n0 + 16 bj + li][landmark j0 + 16 w + 4 lk + r]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = j0 + 16 * w + 4 * lk + r;
      if (j >= m) continue;
#pragma unroll
      for (int bj = 0; bj < kGT / 16; ++bj) {
        const int i = 16 * bj + li;
        if (i < nv) {
          const float c = cv[r][bj];
          const float z = (c - mjv[r]) * rjv[r];
          const float dc = (acc[bj][r] - ajv[r] - z * bjv[r]) * rjv[r];
          gt[((size_t)p * m + j) * N + n0 + i] = dc * c;
        }
      }
    }
  }
}

// Key side, first pass, on fp32 MFMA 16x16x4.  The forward left B in the
// H^T buffer ([P][m][N]); workgroup (tile, p) takes kHT tokens (LDS at lds,
// bwd_hv_lds bytes) and, per block
// of 64 landmarks, stages that block's B, dBV and the tile's V in LDS, forms
// dBV V^T (wavefront w: landmarks 16 w + [0, 16)) and overwrites B with
// H = (dBV V^T) (.) B in place, and accumulates dV = B^T dBV over the blocks
// (wavefront w: tokens 16 w + [0, 16)).  The dV reduction runs over the
// block's landmarks rounded up to 4 (rows past m are zero).
constexpr int kHT = 64;  // tokens per tile

template <int D>
constexpr size_t bwd_hv_lds() {
  return (size_t)(64 * (D + 1) + kHT * (D + 1) + 64 * (kHT + 4)) * sizeof(float);
}

template <typename T, int D>
__device__ __forceinline__ void bwd_hv_body(float* __restrict__ lds, const T* __restrict__ v,
                                            const float* __restrict__ dbv, float* __restrict__ ht,
                                            float* __restrict__ dv, int N, int m) {
  constexpr int kVS = D + 1, kBS = kHT + 4;
  float* dbl = lds;             // [64][D+1]  the block's dBV rows
  float* vs = dbl + 64 * kVS;   // [kHT][D+1] the tile's V rows
  float* bs = vs + kHT * kVS;   // [64][kHT+4] B of the block and tile
  const int tile = blockIdx.x, p = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, li = lane & 15, lk = lane >> 4;
  const int n0 = tile * kHT, nv = min(kHT, N - n0);
  const size_t prob = (size_t)p * N * D;
  // Staging: every global load of a phase is issued before its LDS stores.
  constexpr int kVE = kHT * D / 256, kDE = 64 * D / 256, kBE = 64 * kHT / 256;
  float vr[kVE], dr[kDE], br[kBE];
  auto load_block = [&](int j0, int jv) {
#pragma unroll
    for (int i = 0; i < kDE; ++i) {
      const int e = tid + 256 * i, jj = e / D, f = e % D;
      dr[i] = dbv[((size_t)p * m + j0 + min(jj, jv - 1)) * D + f];
    }
#pragma unroll
    for (int i = 0; i < kBE; ++i) {
      const int e = tid + 256 * i, jj = e / kHT, n = e % kHT;
      br[i] = ht[((size_t)p * m + j0 + min(jj, jv - 1)) * N + n0 + min(n, nv - 1)];
    }
  };
  auto store_block = [&](int jv) {
#pragma unroll
    for (int i = 0; i < kDE; ++i) {
      const int e = tid + 256 * i, jj = e / D, f = e % D;
      dbl[jj * kVS + f] = jj < jv ? dr[i] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kBE; ++i) {
      const int e = tid + 256 * i, jj = e / kHT, n = e % kHT;
      bs[jj * kBS + n] = (jj < jv && n < nv) ? br[i] : 0.f;
    }
  };
#pragma unroll
  for (int i = 0; i < kVE; ++i) {
    const int e = tid + 256 * i, n = e / D, f = e % D;
    vr[i] = widen(v[prob + (size_t)(n0 + min(n, nv - 1)) * D + f]);
  }
  load_block(0, min(64, m));
#pragma unroll
  for (int i = 0; i < kVE; ++i) {
    const int e = tid + 256 * i, n = e / D, f = e % D;
    vs[n * kVS + f] = n < nv ? vr[i] : 0.f;
  }
  f32x4 adv[D / 16];
#pragma unroll
  for (int bj = 0; bj < D / 16; ++bj) adv[bj] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < m; j0 += 64) {
    const int jv = min(64, m - j0);
    if (j0 > 0) {
      load_block(j0, jv);
      __syncthreads();  // the previous block's reads are done
    }
    store_block(jv);
    __syncthreads();
    // H = (dBV V^T) (.) B: landmarks 16 w + [0, 16) of the block, every token.
    if (16 * w < jv) {
      f32x4 acc[kHT / 16];
#pragma unroll
      for (int bj = 0; bj < kHT / 16; ++bj) acc[bj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int k0 = 0; k0 < D; k0 += 4) {
        const float a = dbl[(16 * w + li) * kVS + k0 + lk];
#pragma unroll
        for (int bj = 0; bj < kHT / 16; ++bj)
          acc[bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, vs[(16 * bj + li) * kVS + k0 + lk], acc[bj], 0, 0, 0);
      }
#pragma unroll
      for (int bj = 0; bj < kHT / 16; ++bj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int jj = 16 * w + 4 * lk + r, n = 16 * bj + li;
          if (jj < jv && n < nv) ht[((size_t)p * m + j0 + jj) * N + n0 + n] = acc[bj][r] * bs[jj * kBS + n];
        }
    }
    // dV += B^T dBV: tokens 16 w + [0, 16).
    const int kend = (jv + 3) & ~3;
    for (int k0 = 0; k0 < kend; k0 += 4) {
      const float bt = bs[(k0 + lk) * kBS + 16 * w + li];
#pragma unroll
      for (int bj = 0; bj < D / 16; ++bj)
        adv[bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(bt, dbl[(k0 + lk) * kVS + 16 * bj + li], adv[bj], 0, 0, 0);
    }
  }
#pragma unroll
  for (int bj = 0; bj < D / 16; ++bj)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = 16 * w + 4 * lk + r;
      if (n < nv) dv[prob + (size_t)(n0 + n) * D + 16 * bj + li] = adv[bj][r];
    }
}

// The two first passes in one launch: blockIdx.z = 0 runs the query side
// (bwd_g_body), 1 the key side (bwd_hv_body), on the same 64-token tiles; one
// dynamic LDS buffer serves either.
static_assert(kGT == kHT, "both first passes take the same token tiles");

template <int D>
constexpr size_t bwd_first_lds() {
  return bwd_hv_lds<D>() > 2 * 64 * (D + 1) * sizeof(float) ? bwd_hv_lds<D>() : 2 * 64 * (D + 1) * sizeof(float);
}

template <typename T, int D>
__global__ __launch_bounds__(256, 3) void bwd_first_kernel(const float* __restrict__ dout,
                                                           const float* __restrict__ ct, int ldc,
                                                           const float* __restrict__ y, const float* __restrict__ mu,
                                                           const float* __restrict__ rs, const float* __restrict__ ab,
                                                           float* __restrict__ gt, const T* __restrict__ v,
                                                           const float* __restrict__ dbv, float* __restrict__ ht,
                                                           float* __restrict__ dv, int N, int m) {
  extern __shared__ __align__(16) float lds[];
  if (blockIdx.z == 0)
    bwd_g_body<D>(lds, dout, ct, ldc, y, mu, rs, ab, gt, N, m);
  else
    bwd_hv_body<T, D>(lds, v, dbv, ht, dv, N, m);
}

// Token-side sign sums: out_n = -(1/lambda) sum_j w[j][n] sign(x_n - K~_j),
// per feature.  With x = Q and w = G^T this is dQ; with x = K and w = H^T it
// is the B part of dK (sign(K~_j - k_n) = -sign(k_n - K~_j)), to which the
// pooling adjoint then adds dK~_{j(n)} / pool^2 when dkt is given (grid_w,
// pool, gw locate token n's window).  Workgroup (tile, p) takes kST tokens
// with D / 16 wavefronts: wavefront fb holds features 16 fb + [0, 16) of
// every token of the tile, one lane per token, so each lane keeps 16 inputs
// and 16 sums in registers; the weights of the next group of landmarks are
// loaded while the current group is summed.
constexpr int kST = 64;  // tokens per tile

template <typename T, int D>
__global__ __launch_bounds__(4 * D) void bwd_sign_kernel(const T* __restrict__ x0, const float* __restrict__ wt0,
                                                         float* __restrict__ out0, const T* __restrict__ x1,
                                                         const float* __restrict__ wt1, float* __restrict__ out1,
                                                         const float* __restrict__ dkt1, const float* __restrict__ kt,
                                                         int N, int m, float inv_lam, int grid_w, int pool, int gw) {
  extern __shared__ __align__(16) float kls[];  // [m][D] K~ * 2^64
  const int tile = blockIdx.x, p = blockIdx.y, tid = threadIdx.x;
  // blockIdx.z picks the side: 0 = (x0, wt0, out0), 1 = (x1, wt1, out1, dkt1).
  const bool second = blockIdx.z != 0;
  const T* __restrict__ x = second ? x1 : x0;
  const float* __restrict__ wt = second ? wt1 : wt0;
  float* __restrict__ out = second ? out1 : out0;
  const float* __restrict__ dkt = second ? dkt1 : nullptr;
  const int lane = tid & 63, f0 = 16 * (tid >> 6);
  {
    // K~ into LDS in batches of kB loads per lane, each batch's loads issued
    // before its stores.
    constexpr int kB = 16;
    const float* kp = kt + (size_t)p * m * D;
    for (int base = 0; base < m * D; base += kB * 4 * D) {
      float r[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) r[u] = kp[min(base + tid + 4 * D * u, m * D - 1)];
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (base + tid + 4 * D * u < m * D) kls[base + tid + 4 * D * u] = r[u] * kSgnScale;
    }
  }
  __syncthreads();
  const int n = tile * kST + lane;
  if (n >= N) return;
  float xv[16], acc[16];
  load_row<T, 16>(x + ((size_t)p * N + n) * D + f0, xv);
#pragma unroll
  for (int t = 0; t < 16; ++t) acc[t] = 0.f;
  const float* wc = wt + (size_t)p * m * N + n;
  constexpr int kJU = 8;  // landmarks per group; the next group's weights load during this one
  float wcur[kJU], wnext[kJU];
  auto fetch_w = [&](int j0, float (&dst)[kJU]) {
#pragma unroll
    for (int u = 0; u < kJU; ++u) dst[u] = wc[(size_t)min(j0 + u, m - 1) * N];
  };
  fetch_w(0, wcur);
  for (int j0 = 0; j0 < m; j0 += kJU) {
    if (j0 + kJU < m) fetch_w(j0 + kJU, wnext);
#pragma unroll
    for (int u = 0; u < kJU; ++u) {
      if (j0 + u < m) {
        const float* kr = kls + (j0 + u) * D + f0;
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[t] = fmaf(wcur[u], sgn_diff(xv[t], kr[t]), acc[t]);
      }
    }
#pragma unroll
    for (int u = 0; u < kJU; ++u) wcur[u] = wnext[u];
  }
  float* op = out + ((size_t)p * N + n) * D + f0;
  if (dkt) {
    const int jn = (n / grid_w / pool) * gw + (n % grid_w) / pool;
    const float* dr = dkt + ((size_t)p * m + jn) * D + f0;
    const float inv_area = 1.f / (float)(pool * pool);
#pragma unroll
    for (int t = 0; t < 16; ++t) op[t] = fmaf(dr[t], inv_area, -inv_lam * acc[t]);
  } else {
#pragma unroll
    for (int t = 0; t < 16; ++t) op[t] = -inv_lam * acc[t];
  }
}

// Landmark side: lane (jl, t) takes feature t of landmarks jb LW + jl + LG u,
// u < kJPL (LG = 256 / D, LW = kJPL LG landmarks per workgroup), so that each
// token value read from LDS serves kJPL landmarks; workgroup (jb, p, sl) takes
// the tokens of slice sl (kKC-token chunks, slice_chunks of them).  The chunks
// are streamed through LDS: the chunk's rows of Q (then K) and its G^T (then
// H^T) entries for the workgroup's landmarks, loaded coalesced by all lanes one
// chunk ahead, then summed per lane in token order on two chains per landmark
// (even and odd tokens).  The slice's sum of both sides goes to
// kpart[sl][p][j][t]; bwd_kt_combine_kernel adds the slices in order and the W
// term.
constexpr int kKC = 64;
constexpr int kJPL = 4;  // the pipelined loop below names its four accumulators

template <typename T, int D>
__global__ __launch_bounds__(256, 3) void bwd_kt_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                        const float* __restrict__ kt, const float* __restrict__ gt,
                                                        const float* __restrict__ ht, float* __restrict__ kpart,
                                                        int N, int m, int slice_chunks) {
  constexpr int LG = 256 / D, LW = kJPL * LG;
  __shared__ float xs[kKC * D];
  __shared__ __align__(16) float gs[LW * kKC];
  const int p = blockIdx.y, sl = blockIdx.z, tid = threadIdx.x;
  const int jl = tid / D, t = tid % D;
  const int j0 = blockIdx.x * LW;
  float kjs[kJPL];
#pragma unroll
  for (int u = 0; u < kJPL; ++u) kjs[u] = kt[((size_t)p * m + min(j0 + jl + LG * u, m - 1)) * D + t] * kSgnScale;
  const int n_begin = sl * slice_chunks * kKC, n_end = min(N, n_begin + slice_chunks * kKC);
  // Per lane, the chunk's loads: kX row values and kG weights.  Tokens past
  // the slice read a valid row and carry weight 0.
  constexpr int kX = kKC * D / 256, kG = LW * kKC / 256;
  float total[kJPL];
#pragma unroll
  for (int u = 0; u < kJPL; ++u) total[u] = 0.f;
#pragma unroll
  for (int side = 0; side < 2; ++side) {
    const T* rows = (side == 0 ? q : k) + (size_t)p * N * D;
    const float* wt = (side == 0 ? gt : ht) + (size_t)p * m * N;
    float xr[kX], gr[kG];
    auto fetch = [&](int c0) {
#pragma unroll
      for (int u = 0; u < kX; ++u) {
        const int e = tid + 256 * u, i = e / D;
        xr[u] = widen(rows[(size_t)min(c0 + i, N - 1) * D + e % D]);
      }
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        const int e = tid + 256 * u, l = e / kKC, i = e % kKC;
        const float g = wt[(size_t)min(j0 + l, m - 1) * N + min(c0 + i, N - 1)];
        gr[u] = c0 + i < n_end ? g : 0.f;
      }
    };
    float a0[kJPL], a1[kJPL];
#pragma unroll
    for (int u = 0; u < kJPL; ++u) a0[u] = a1[u] = 0.f;
    fetch(n_begin);
    for (int c0 = n_begin; c0 < n_end; c0 += kKC) {
      __syncthreads();  // the previous chunk's reads are done
#pragma unroll
      for (int u = 0; u < kX; ++u) xs[tid + 256 * u] = xr[u];
#pragma unroll
      for (int u = 0; u < kG; ++u) gs[tid + 256 * u] = gr[u];
      __syncthreads();
      if (c0 + kKC < n_end) fetch(c0 + kKC);
      // Both sides sum w_i sign(x_i - K~_jt); the B side's sign is flipped in
      // the combine.  Four tokens per step; the weights (one 16-byte read per
      // landmark) and token values of the step after next are read while the
      // current step is summed, so the LDS latency is not waited out per step
      // (72.9 -> 65.7 us at the 56x56 workload; one step ahead: 67.8).  a0
      // takes the even tokens and a1 the odd ones, in token order.
      float4 gq[3][kJPL];
      float xq[3][4];
      auto read_step = [&](int i, float4 (&g4)[kJPL], float (&x4)[4]) {
#pragma unroll
        for (int u = 0; u < kJPL; ++u) g4[u] = *reinterpret_cast<const float4*>(gs + (jl + LG * u) * kKC + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) x4[e] = xs[(i + e) * D + t];
      };
      read_step(0, gq[0], xq[0]);
      read_step(4, gq[1], xq[1]);
#pragma unroll
      for (int i = 0; i < kKC; i += 4) {
        const int cur = (i >> 2) % 3;
        if (i + 8 < kKC) read_step(i + 8, gq[(cur + 2) % 3], xq[(cur + 2) % 3]);
#pragma unroll
        for (int u = 0; u < kJPL; ++u) {
          a0[u] = fmaf(gq[cur][u].x, sgn_diff(xq[cur][0], kjs[u]), a0[u]);
          a1[u] = fmaf(gq[cur][u].y, sgn_diff(xq[cur][1], kjs[u]), a1[u]);
          a0[u] = fmaf(gq[cur][u].z, sgn_diff(xq[cur][2], kjs[u]), a0[u]);
          a1[u] = fmaf(gq[cur][u].w, sgn_diff(xq[cur][3], kjs[u]), a1[u]);
        }
        asm volatile("" : "+v"(a0[0]), "+v"(a0[1]), "+v"(a0[2]), "+v"(a0[3]), "+v"(a1[0]), "+v"(a1[1]),
                     "+v"(a1[2]), "+v"(a1[3])::"memory");
      }
    }
#pragma unroll
    for (int u = 0; u < kJPL; ++u) total[u] += a0[u] + a1[u];
  }
#pragma unroll
  for (int u = 0; u < kJPL; ++u) {
    const int j = j0 + jl + LG * u;
    if (j < m) kpart[(((size_t)sl * gridDim.y + p) * m + j) * D + t] = total[u];
  }
}

// dK~_jt = (1/lambda) (sum over slices of kpart + c_jt), one lane per (j, t);
// workgroup (jb, p) takes landmarks jb LG + [0, LG), LG = 256 / D:
// c_jt = sum_b a_jb sign(K~_jt - K~_bt), a_jb = (dw_jb + dw_bj)(W_jb - eps [j = b]).
// dw holds -dW, so the W term of the gradient, -(1/lambda) sum_b (dW_jb +
// dW_bj)(W_jb - eps [j = b]) sign(K~_jt - K~_bt), is +c_jt / lambda.  The
// coefficients a_jb go to LDS first.  sum_n H_jn sign(K~_j - k_n) is minus
// the K side of kpart.
template <int D>
__global__ __launch_bounds__(256) void bwd_kt_combine_kernel(const float* __restrict__ kpart, int slices,
                                                             const float* __restrict__ kt,
                                                             const float* __restrict__ w, int mp,
                                                             const float* __restrict__ dw, float* __restrict__ dkt,
                                                             int m, float eps, float inv_lam) {
  constexpr int LG = 256 / D;
  __shared__ float coef[LG * kMaxM];
  const int p = blockIdx.y, tid = threadIdx.x, jl = tid / D, t = tid % D;
  const int j0 = blockIdx.x * LG, j = j0 + jl;
  const float* wp = w + (size_t)p * mp * mp;
  const float* dwp = dw + (size_t)p * mp * mp;
  for (int e = tid; e < LG * m; e += 256) {
    const int l = e / m, bb = e % m, jj = min(j0 + l, m - 1);
    const float wv = wp[(size_t)jj * mp + bb] - (bb == jj ? eps : 0.f);
    coef[l * kMaxM + bb] = (dwp[(size_t)jj * mp + bb] + dwp[(size_t)bb * mp + jj]) * wv;
  }
  __syncthreads();
  if (j >= m) return;
  const size_t slice_stride = (size_t)gridDim.y * m * D;
  float s = 0.f;
  for (int sl = 0; sl < slices; ++sl) s += kpart[sl * slice_stride + ((size_t)p * m + j) * D + t];
  const float* ktp = kt + (size_t)p * m * D + t;
  const float kj = ktp[(size_t)j * D];
  const float* cl = coef + jl * kMaxM;
  float c = 0.f;
#pragma unroll 8
  for (int bb = 0; bb < m; ++bb) c = fmaf(cl[bb], sgn(kj - ktp[(size_t)bb * D]), c);
  dkt[((size_t)p * m + j) * D + t] = (s + c) * inv_lam;
}

template <typename T, int D>
hipError_t launch_typed(const Plan& pl, const BwdWork& b, const Work& w, const void* q, const void* k,
                        const void* v, const float* dout, float* dq, float* dk, float* dv, hipStream_t s) {
  const int nt = (pl.N + kBT - 1) / kBT;
  const float inv_lam = -pl.scale / 1.4426950408889634f;  // 1 / lambda from scale = -log2(e) / lambda
  const int mp = pl.mp, m = pl.m;
  hipLaunchKernelGGL(bwd_ctg_kernel<D>, dim3(nt, pl.P, (m + 63) / 64), dim3(256), 0, s, w.ct, pl.ldc, dout, b.part,
                     b.spart, pl.N, m, nt);
  hipError_t e;
  if (m <= 64) {
    constexpr size_t small_lds = bwd_small_lds<D>();
    e = hipFuncSetAttribute((const void*)bwd_small_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)small_lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dy_kernel<D>, dim3((mp * D + 255) / 256, pl.P), dim3(256), 0, s, b.part, b.spart, w.mu,
                       w.rs, b.dy, b.s, m, mp, nt);
    hipLaunchKernelGGL(bwd_small_kernel<D>, dim3(pl.P), dim3(256), small_lds, s, b.dy, b.s, w.x_final, mp, w.bv,
                       b.y, b.dbv, b.ab, b.dw, pl.N, m, pl.whiten ? 1 : 0);
  } else {
    // The same quantities with the products on the tile GEMM, in the workspace.
    const long long sq = (long long)mp * mp, md = (long long)m * D, mpd = (long long)mp * D;
    const int kext = (m + 31) & ~31;
    hipLaunchKernelGGL(bwd_dy_kernel<D>, dim3((mp * D + 255) / 256, pl.P), dim3(256), 0, s, b.part, b.spart, w.mu,
                       w.rs, b.dy, b.s, m, mp, nt);
    e = launch_gemm(w.x_final, mp, sq, w.bv, D, md, m, D, b.y, D, md, m, D, kext, pl.P, s);  // Y = X BV
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_ab_kernel<D>, dim3((m + 255) / 256, pl.P), dim3(256), 0, s, b.y, b.dy, b.s, b.ab, pl.N, m,
                       mp, pl.whiten ? 1 : 0);
    hipLaunchKernelGGL(bwd_transpose_kernel, dim3((unsigned)((sq + 255) / 256), pl.P), dim3(256), 0, s, w.x_final,
                       mp, sq, b.xt, sq, mp, mp, mp);  // X^T
    hipLaunchKernelGGL(bwd_transpose_kernel, dim3((unsigned)((D * mp + 255) / 256), pl.P), dim3(256), 0, s, w.bv, D,
                       md, b.bvt, (long long)D * mp, m, D, mp);  // BV^T, zero past m
    e = launch_gemm(b.xt, mp, sq, b.dy, D, mpd, mp, D, b.dbv, D, md, m, D, kext, pl.P, s);  // dBV = X^T dY
    if (e != hipSuccess) return e;
    e = launch_gemm(b.dy, D, mpd, b.bvt, mp, (long long)D * mp, D, mp, b.dx, mp, sq, mp, mp, D, pl.P, s);  // dX
    if (e != hipSuccess) return e;
    e = launch_gemm(b.xt, mp, sq, b.dx, mp, sq, mp, mp, b.r, mp, sq, mp, mp, kext, pl.P, s);  // R = X^T dX
    if (e != hipSuccess) return e;
    e = launch_gemm(b.r, mp, sq, b.xt, mp, sq, mp, mp, b.dw, mp, sq, mp, mp, kext, pl.P, s);  // R X^T = -dW
    if (e != hipSuccess) return e;
  }
  const size_t row_lds = (size_t)m * D * sizeof(float);  // <= 64 KB
  const int nst = (pl.N + kST - 1) / kST;
  // G (query side) and H, dV (key side) in one launch.
  constexpr size_t first_lds = bwd_first_lds<D>();
  static_assert(first_lds <= 65536, "the first passes fit in static-size LDS");
  hipLaunchKernelGGL((bwd_first_kernel<T, D>), dim3((pl.N + kHT - 1) / kHT, pl.P, 2), dim3(256), first_lds, s, dout,
                     w.ct, pl.ldc, b.y, w.mu, w.rs, b.ab, b.gt, (const T*)v, b.dbv, b.ht, dv, pl.N, m);
  // Landmark side in token slices of kSliceChunks chunks; the partials reuse
  // the C^T g partial buffer ([P][tiles][m][d], tiles >= slices), which is
  // free once dY is formed.
  constexpr int LG = 256 / D, kSliceChunks = 4;
  const int chunks = (pl.N + kKC - 1) / kKC;
  const int slices = (chunks + kSliceChunks - 1) / kSliceChunks;
  if (slices > nt) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_kt_kernel<T, D>), dim3((m + kJPL * LG - 1) / (kJPL * LG), pl.P, slices), dim3(256), 0, s,
                     (const T*)q, (const T*)k, w.kt, b.gt, b.ht, b.part, pl.N, m, kSliceChunks);
  hipLaunchKernelGGL(bwd_kt_combine_kernel<D>, dim3((m + LG - 1) / LG, pl.P), dim3(256), 0, s, b.part, slices,
                     w.kt, w.w, pl.mp, b.dw, b.dkt, m, pl.eps, inv_lam);
  // dQ, and dK: the B part plus the pooling adjoint of dK~, in one launch.
  hipLaunchKernelGGL((bwd_sign_kernel<T, D>), dim3(nst, pl.P, 2), dim3(4 * D), row_lds, s, (const T*)q, b.gt, dq,
                     (const T*)k, b.ht, dk, b.dkt, w.kt, pl.N, m, inv_lam, pl.grid_w, pl.pool, pl.gw);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const Plan& pl, const BwdWork& b, const Work& w, const void* q, const void* k,
                           const void* v, const float* dout, float* dq, float* dk, float* dv, hipStream_t s) {
  if (pl.dtype == 1) {
    return pl.d == 64 ? launch_typed<uint16_t, 64>(pl, b, w, q, k, v, dout, dq, dk, dv, s)
                      : launch_typed<uint16_t, 32>(pl, b, w, q, k, v, dout, dq, dk, dv, s);
  }
  return pl.d == 64 ? launch_typed<float, 64>(pl, b, w, q, k, v, dout, dq, dk, dv, s)
                    : launch_typed<float, 32>(pl, b, w, q, k, v, dout, dq, dk, dv, s);
}

}  // namespace lapnys
