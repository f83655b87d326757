// Output stage: O = Z Y with Z = (C - mu) / sigma column-wise (the diagonal
// whitening of EN page section 2.B) and Y = X (B V), i.e. O = Z W^-1 (B V).
//
// One workgroup per 256-token tile, four wavefronts of 64 tokens each.  The
// stage streams C once and writes O once.
//
//  * Each lane loads C^T[landmark][4 consecutive tokens] as one 16-byte load;
//    16 lanes cover a 256-byte run of one landmark row.  All of a wavefront's
//    C loads (up to 64 landmarks) are issued before anything else, so their
//    latency overlaps the Y prologue.  For m > 64 the loads of the next 64
//    landmarks are issued slot by slot as the current ones are consumed.
//  * Prologue: Y = X (B V) is stored in LDS transposed, as bf16 high and low
//    parts (y = hi + lo to about 16 bits).  For m <= 64 the finalize stage
//    has already formed it in this layout (once per problem) and the
//    workgroup copies 16 KB; for larger m it comes from a batched tile GEMM
//    in float32 and is split here.
//  * Main loop: Z Y on bf16 MFMA 16x16x32 with three products per step,
//    Zhi Yhi + Zhi Ylo + Zlo Yhi: the dropped Zlo Ylo term and the rounding
//    of the low parts are about 2^-16 of each product, so the stage keeps
//    near-fp32 accuracy at a fifth of the fp32 MFMA cycles.  Lane (li, lk)
//    holds 8 landmarks (32 h + 8 lk + e, e < 8) of its 4 tokens tb + 4 li + a
//    and feeds them as the A operand of token block a; the B operand of
//    feature block b is Y[same 8 landmarks][D/16 li + b], one 16-byte LDS read.
//    A lane thus ends up holding D/16 consecutive features of each of its
//    tokens and writes them with one 16-byte (D = 64) or 8-byte (D = 32)
//    streaming store.
//  * Workgroups go to the eight XCDs in turn by index, each XCD with its own
//    L2.  For m <= 64 with P a multiple of 8 the workgroup index b =
//    (p / 8) 8 T + 8 tile + p % 8 (T tiles per problem) keeps all of a
//    problem's tiles on one XCD, so Y^T and the column statistics come from
//    HBM once per problem (the 56x56 workload's stage: 9.2 -> 8.8 us).
//    Otherwise tiles are numbered problem-major (b = p T + tile): at m = 256
//    with 8 problems of 256 tiles the grouping put each problem's whole C
//    stream behind one XCD and was slower (139 -> 144 us).
#include "lapnys_internal.hpp"

namespace lapnys {

namespace {

constexpr int kSlots = 16; // C loads of four tokens each held per lane (64 landmarks)

// All-ones when ok, else zero, opaque to the optimiser: masking a loaded
// value with it (instead of a select) keeps the load unconditional, so it
// issues with the others and no early wait is needed for it.
__device__ __forceinline__ uint32_t lane_mask(bool ok) {
  uint32_t mk = ok ? 0xffffffffu : 0u;
  asm volatile("" : "+v"(mk));
  return mk;
}

__device__ __forceinline__ float masked(float v, uint32_t mk) { return __uint_as_float(__float_as_uint(v) & mk); }

template <int D, bool FUSED_Y>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void output_kernel(const float* __restrict__ ct, int ldc,
                                                     const __bf16* __restrict__ yt, const float* __restrict__ y,
                                                     const float* __restrict__ mu, const float* __restrict__ rs,
                                                     float* __restrict__ out, int N, int m, int xcd_group) {
  constexpr int DB = D / 16;
  extern __shared__ __align__(16) float lds[];
  const int rl = FUSED_Y ? 64 : (m + 63) & ~63;  // landmarks per Y^T row; rows past m are zero
  __bf16* yth = reinterpret_cast<__bf16*>(lds);  // [D][rl] high parts
  __bf16* ytl = yth + D * rl;                    // [D][rl] low parts
  float2* mrs = reinterpret_cast<float2*>(ytl + D * rl);  // [rl]: (mu, 1/sigma), zero past m
  const int nt = (N + 255) / 256, b = blockIdx.x;
  const int tile = xcd_group ? (b / 8) % nt : b % nt;
  const int p = xcd_group ? (b / (8 * nt)) * 8 + b % 8 : b / nt;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int tb = tile * 256 + 64 * w;  // first token of this wavefront
  const int tok4 = tb + 4 * li;        // first of this lane's four tokens
  const bool tok_ok = tok4 < N;

  // C loads: slot s holds landmark c0 + 32 (s / 8) + 8 lk + s % 8.  Landmark
  // rows past m and tokens past N are read from a clamped, in-bounds address
  // and masked to zero where they are used, so the loads are unconditional
  // and all issue before the first wait.
  float4 cr[kSlots];
  const float* cpc = ct + (size_t)p * m * ldc + min(tok4, ldc - 4);
  auto load_slot = [&](int c0, int s) {
    const int j = c0 + 32 * (s >> 3) + 8 * lk + (s & 7);
    cr[s] = *reinterpret_cast<const float4*>(cpc + (size_t)min(j, m - 1) * ldc);
  };

  if constexpr (FUSED_Y) {
    // Y^T high and low parts come from the finalize stage in this LDS layout
    // (2 D 64 bf16): they are loaded into registers ahead of the C loads, and
    // nothing consumes a loaded value before the scheduling barrier, so the
    // wait for them leaves the C loads in flight.
    constexpr int kYv = 2 * D * 64 * 2 / 16 / 256;  // 16-byte loads per lane
    const float4* ysrc = reinterpret_cast<const float4*>(yt + (size_t)p * 2 * D * 64);
    float4 yv[kYv];
#pragma unroll
    for (int i = 0; i < kYv; ++i) yv[i] = ysrc[tid + 256 * i];
    const int jt = tid & 63;
    const float mu_t = mu[p * m + min(jt, m - 1)], rs_t = rs[p * m + min(jt, m - 1)];
#pragma unroll
    for (int s = 0; s < kSlots; ++s) load_slot(0, s);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kYv; ++i) reinterpret_cast<float4*>(yth)[tid + 256 * i] = yv[i];
    {
      // Every wavefront stores the same 64 pairs (an unconditional store keeps
      // the two loads from being moved behind the C loads' wait).
      const uint32_t mk = lane_mask(jt < m);
      mrs[jt] = make_float2(masked(mu_t, mk), masked(rs_t, mk));
    }
  } else {
#pragma unroll
    for (int s = 0; s < kSlots; ++s) load_slot(0, s);
    for (int e = tid; e < rl; e += 256)
      mrs[e] = (e < m) ? make_float2(mu[p * m + e], rs[p * m + e]) : make_float2(0.f, 0.f);
    // Y^T into LDS in batches of kB loads per lane, each batch's loads
    // issued before its stores.
    const float* yp = y + (size_t)p * m * D;
    constexpr int kB = 16;
    for (int base = 0; base < rl * D; base += kB * 256) {
      float r[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) r[u] = yp[min(base + tid + 256 * u, m * D - 1)];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int e = base + tid + 256 * u;
        if (e < rl * D) {
          const int l = e / D, f = e % D;
          const float v = l < m ? r[u] : 0.f;
          const __bf16 hi = (__bf16)v;
          const int at = yt_index(f, l, f / DB, rl);
          yth[at] = hi;
          ytl[at] = (__bf16)(v - (float)hi);
        }
      }
    }
  }
  __syncthreads();

  f32x4 acc[4][DB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One pass over 64 landmarks when Y is formed here (m <= 64).
  const int mc = FUSED_Y ? 64 : m;
  for (int c0 = 0; c0 < mc; c0 += 64) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (c0 + 32 * h < m) {  // else the half is past m (uniform)
        // A operands: z of landmarks c0 + 32 h + 8 lk + e for token block a,
        // split into bf16 high and low parts, two landmarks per dword.
        u32x4 ah[4], al[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float z[2][4];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int s = 8 * h + e + u;
            const int j = c0 + 32 * h + 8 * lk + e + u;
            const float2 st = mrs[j];
            // Landmarks past m have mu = 1/sigma = 0 and a zero C value: z = 0.
            const uint32_t mk = lane_mask(tok_ok && j < m);
            z[u][0] = (masked(cr[s].x, mk) - st.x) * st.y;
            z[u][1] = (masked(cr[s].y, mk) - st.x) * st.y;
            z[u][2] = (masked(cr[s].z, mk) - st.x) * st.y;
            z[u][3] = (masked(cr[s].w, mk) - st.x) * st.y;
            if constexpr (!FUSED_Y) {
              if (c0 + 64 < m) load_slot(c0 + 64, s);
            }
          }
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            uint32_t hw, lw;
            split2(z[0][a], z[1][a], hw, lw);
            ah[a][e / 2] = hw;
            al[a][e / 2] = lw;
          }
        }
        const int chunk = 4 * h + lk + (c0 >> 3);
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const int at = (DB * li + b) * rl + 8 * ((chunk & ~7) | ((chunk ^ li) & 7));
          const bf16x8 bh = *reinterpret_cast<const bf16x8*>(yth + at);
          const bf16x8 bl = *reinterpret_cast<const bf16x8*>(ytl + at);
#pragma unroll
          for (int a = 0; a < 4; ++a)
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, al[a]), bh, acc[a][b], 0, 0, 0);
#pragma unroll
          for (int a = 0; a < 4; ++a)
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ah[a]), bl, acc[a][b], 0, 0, 0);
#pragma unroll
          for (int a = 0; a < 4; ++a)
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ah[a]), bh, acc[a][b], 0, 0, 0);
        }
      }
    }
  }

  // acc[a][b][r] = O[token tb + 4 (4 lk + r) + a][feature DB li + b].  O is
  // written with streaming (nontemporal) stores: it is not read again here,
  // and the writes drain to memory while the kernel runs instead of being
  // written back from L2 when it ends.
  float* op = out + (size_t)p * N * D + DB * li;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int tok = tb + 16 * lk + 4 * r + a;
      if (tok < N) {
        if constexpr (DB == 4) {
          const f32x4 o = {acc[a][0][r], acc[a][1][r], acc[a][2][r], acc[a][3][r]};
          __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(op + (size_t)tok * D));
        } else {
          const f32x2 o = {acc[a][0][r], acc[a][1][r]};
          __builtin_nontemporal_store(o, reinterpret_cast<f32x2*>(op + (size_t)tok * D));
        }
      }
    }
}

template <int D, bool FUSED_Y>
hipError_t launch_typed(const Plan& pl, const Work& wk, float* out, hipStream_t s, Span t) {
  // Y^T high and low parts (bf16, rl landmarks per row), then the
  // (mu, 1/sigma) pairs.
  const size_t rl = FUSED_Y ? 64 : (size_t)(pl.m + 63) & ~(size_t)63;
  const size_t shmem = 2 * D * rl * 2 + rl * 8;
  auto kern = output_kernel<D, FUSED_Y>;
  if (shmem > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  const int xcd_group = FUSED_Y && pl.P % 8 == 0 ? 1 : 0;
  const long long grid = (long long)((pl.N + 255) / 256) * pl.P;
  if (grid * 256 > 0xffffffffLL) return hipErrorInvalidConfiguration;  // one grid axis of 2^32 lanes
  hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), shmem, s, t.start, t.stop, 0, wk.ct, pl.ldc,
                        wk.yt, wk.y, wk.mu, wk.rs, out, pl.N, pl.m, xcd_group);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_output(const Plan& pl, const Work& wk, float* out, hipStream_t s, Span t) {
  if (pl.fused_ns) {
    if (pl.d == 64) return launch_typed<64, true>(pl, wk, out, s, t);
    return launch_typed<32, true>(pl, wk, out, s, t);
  }
  if (pl.d == 64) return launch_typed<64, false>(pl, wk, out, s, t);
  return launch_typed<32, false>(pl, wk, out, s, t);
}

}  // namespace lapnys
