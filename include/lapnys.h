/*
 * liblapnys -- forward pass of LaplacianFormer's Laplacian-kernel Nystrom
 * linear attention on AMD Instinct MI355X (gfx950).
 *
 * Sources: the summary pages of "LaplacianFormer: Rethinking Linear Attention
 * with Laplacian Kernel" (gist.science; English page cited as EN, others by
 * language).  Per independent (batch, head) problem with N tokens on a
 * grid_h x grid_w token grid and head dimension d, one call computes:
 *
 *   K~ = average pool of K over pool x pool windows        (EN 2.C.1)
 *   C  = k(Q, K~)  [N x m],  B = k(K~, K)  [m x N],
 *   W  = k(K~, K~) + eps I  [m x m],
 *        with k(x, y) = exp(-||x - y||_1 / lambda)          (EN 2.A)
 *   X  = Newton-Schulz inverse of W: X0 = W^T/(||W||_1 ||W||_inf),
 *        then ns_iters steps X <- X (2I - W X)             (EN 2.C.2)
 *   Z  = C with each landmark column centred and divided by its standard
 *        deviation over the N tokens (population variance) (EN 2.B)
 *   O  = Z (X (B V))
 *
 * m = (grid_h / pool) * (grid_w / pool).  Tokens are the row-major cells of
 * the grid (token n = r * grid_w + c); landmark j = R * (grid_w / pool) + C.
 *
 * Layouts: q, k, v and out are dense, C-order [B, H, N, d] arrays; problem
 * (b, h) is the contiguous block starting at element (b * H + h) * N * d.
 * q, k and v are float32 or bfloat16 (dtype); out is always float32.
 *
 * Precision.  Every value is held in float32 after the input load (bf16
 * inputs widen exactly).  Landmark pooling sums in float64 and rounds once.
 * The L1 distances, exponentials, W and the whitening statistics are float32
 * vector arithmetic (the statistics are merged in float64).  The products
 * B V and Z Y, and the Newton-Schulz steps for m <= 64 except the last ones,
 * run on bf16 MFMA with every float32 operand split into a bf16 high part and
 * a bf16 low part and three of the four partial products (hi*hi, hi*lo,
 * lo*hi) accumulated in float32: each product keeps all but about 2^-16 of
 * its value.  The last Newton-Schulz steps (at least one, and every step once
 * ||W||_1 max|X| exceeds 64), Y = X (B V), the m > 64 solver and the CG
 * solver use float32 products (fp32 MFMA).  Measured against the float64
 * oracle the output stays within 1e-4 of max|O| (normwise) for float32 and
 * bf16 inputs alike.  Results do not depend on the input storage type beyond
 * the input values themselves.
 *
 * Ownership and threading: every pointer argument belongs to the caller.  The
 * library keeps no pointer after a call returns.  Device pointers must point
 * to memory of the current HIP device.  Work is enqueued on `stream` (0 means
 * the null stream); no call synchronises the stream except
 * lapnys_forward_debug, which returns after its copies are complete.  Calls
 * do not throw; every call returns LAPNYS_OK (0) or a negative status, and on
 * any validation error nothing is enqueued.  Faults inside kernels surface as
 * HIP errors at the caller's next synchronisation.
 */
#ifndef LAPNYS_H_
#define LAPNYS_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of q, k and v. */
typedef enum { LAPNYS_F32 = 0, LAPNYS_BF16 = 1 } lapnys_dtype;

/* flags.
 * LAPNYS_WHITEN: apply the diagonal whitening to C (EN 2.B).  Without it
 *   Z = C.
 * LAPNYS_NS_REFINE: after the ns_iters Newton-Schulz steps (EN 2.C.2), one
 *   correction X <- X + X R with the residual R = I - W X accumulated in
 *   float64 from the float32 W and X.  This is an extension beyond the pages'
 *   fixed-count iteration, not part of the method: exactly, the step leaves
 *   the residual R^2 (it is the Newton-Schulz update X (2I - W X) with W X
 *   formed more accurately), so a large, poorly conditioned W whose float32
 *   iterate stops short of the wanted residual (for example 256 landmarks of
 *   a 256 x 256 grid, condition number near 1.4e3) reaches the float32
 *   representation floor of its inverse.  Off, the result is the pages'
 *   fixed-count X.
 * LAPNYS_GAUSSIAN: the Gaussian kernel k(x, y) = exp(-||x - y||_2^2 / lambda)
 *   in place of the Laplacian one, for C, B and W alike: the kernel the
 *   pages' method replaces (EN section 1 and 2.A), read with the same scale
 *   lambda.  Every other step is unchanged.  The squared distances of C and
 *   B are formed as ||x||^2 + ||y||^2 - 2 x.y (the dot products on fp32
 *   MFMA) and clamped at 0; W's are summed directly.  The solver then runs
 *   as launches of its own, beside the kernel-matrix stage, at every m.
 * LAPNYS_SOLVER_CG: the conjugate-gradient solver of the pages' solver
 *   ablation (EN section 4) in place of Newton-Schulz: Y = W^-1 (B V) is
 *   computed directly by ns_iters CG steps per column of B V, from Y0 = 0,
 *   without a preconditioner, in float32 (a column whose residual is exactly
 *   zero, or so small that p.(W p) underflows to zero, stops changing).  X is not formed: the debug form leaves its X
 *   buffer untouched.  Not combinable with LAPNYS_NS_REFINE.
 * LAPNYS_NS_PLAIN: m <= 64 only (larger m always runs so): the Newton-Schulz
 *   steps X <- X (2I - W X) with every product in float32, as a launch of
 *   its own beside the kernel-matrix stage.  The default schedule for
 *   m <= 64 runs inside the kernel-matrix launch, forms every entry of
 *   2X - X (W X) and takes the early steps on bf16-split products while
 *   ||W||_1 max|X| <= 64; it reaches the same float32 floor as the plain
 *   steps at every condition number (near-singular W included).  Kept as the
 *   reference schedule of the solver study; slower. */
enum { LAPNYS_WHITEN = 1u, LAPNYS_NS_REFINE = 2u, LAPNYS_GAUSSIAN = 4u, LAPNYS_SOLVER_CG = 8u,
       LAPNYS_NS_PLAIN = 16u };

/* Status codes. */
enum {
  LAPNYS_OK = 0,
  LAPNYS_ERR_INVALID_ARG = -1, /* null/misaligned pointer, non-positive size,
                                  lambda <= 0, eps < 0, ns_iters < 0, unknown
                                  flag bits, LAPNYS_SOLVER_CG together with
                                  LAPNYS_NS_REFINE, non-finite lambda/eps, or
                                  out overlapping an input */
  LAPNYS_ERR_SHAPE = -2,       /* N != grid_h * grid_w, or pool does not divide
                                  grid_h and grid_w */
  LAPNYS_ERR_UNSUPPORTED = -3, /* d not in {32, 64}, m > 256, unknown dtype, or
                                  sizes beyond 32-bit element counts */
  LAPNYS_ERR_WORKSPACE = -4,   /* workspace null, smaller than
                                  lapnys_workspace_size, or not 256-B aligned */
  LAPNYS_ERR_HIP = -5,         /* a HIP runtime call or kernel launch failed */
  LAPNYS_ERR_SCRATCH = -6      /* lapnys_forward_noalloc: the workspace the
                                  problem needs exceeds LAPNYS_SCRATCH_MAX_BYTES */
};

/* Problem description.  lambda is the kernel scale (the pages find 4 best,
 * EN section 4), eps the diagonal shift of W (EN 2.C.2). */
typedef struct {
  int32_t B, H;          /* batch and heads: B * H independent problems */
  int32_t N;             /* tokens per problem, = grid_h * grid_w */
  int32_t d;             /* head dimension: 32 or 64 */
  int32_t grid_h, grid_w;
  int32_t pool;          /* landmark pooling window (pool x pool, stride pool) */
  float lambda;          /* > 0 */
  float eps;             /* >= 0 */
  int32_t ns_iters;      /* Newton-Schulz steps, >= 0 */
  int32_t dtype;         /* lapnys_dtype */
  uint32_t flags;        /* LAPNYS_WHITEN | LAPNYS_NS_REFINE | LAPNYS_GAUSSIAN |
                            LAPNYS_SOLVER_CG | LAPNYS_NS_PLAIN, or 0 */
} lapnys_params;

/* Optional device buffers for the intermediates of one call (debug form).
 * Each pointer may be NULL (not written).  Shapes per problem p = b * H + h,
 * all float32, C order:
 *   landmarks [B*H, m, d]   C_t [B*H, m, N] (C transposed: landmark-major)
 *   W, X      [B*H, m, m]   BV, Y [B*H, m, d]   mu, sigma [B*H, m]
 * With whitening off, mu = 0 and sigma = 1.
 * Timing stamps (device wall clock, hipDeviceAttributeWallClockRate kHz):
 *   ns_clock [B*H, 3]: start, first Newton-Schulz step and end of each
 *     problem's solver workgroup, written only by the default m <= 64
 *     schedule (the solver runs inside the kernel-matrix launch);
 *   kernel_clock [2]: earliest start and latest end over the workgroups of
 *     the Laplacian kernel-matrix stage (the solver's excluded). */
typedef struct {
  float* landmarks;
  float* C_t;
  float* W;
  float* X;
  float* BV;
  float* Y;
  float* mu;
  float* sigma;
  unsigned long long* ns_clock;
  unsigned long long* kernel_clock;
} lapnys_debug;

/* Stage indices for lapnys_forward_profiled. */
enum {
  LAPNYS_STAGE_POOL = 0,     /* landmark average pooling */
  LAPNYS_STAGE_NS = 1,       /* W build, scaling, Newton-Schulz (and the
                                correction of LAPNYS_NS_REFINE); with
                                LAPNYS_SOLVER_CG the W build only */
  LAPNYS_STAGE_KERNEL = 2,   /* fused distance + exp: C, column statistics, B V */
  LAPNYS_STAGE_FINALIZE = 3, /* statistics and B V reductions, Y = X (B V)
                                (the CG solve with LAPNYS_SOLVER_CG) */
  LAPNYS_STAGE_OUTPUT = 4,   /* O = whiten(C) Y */
  LAPNYS_NUM_STAGES = 5
};

/* Number of landmarks m for valid params, else a negative status. */
int lapnys_landmark_count(const lapnys_params* p);

/* Device workspace (bytes) that lapnys_forward_ws needs for params p.
 * Host-only arithmetic: touches no device.  Returns a status; *bytes is
 * written only on success. */
int lapnys_workspace_size(const lapnys_params* p, size_t* bytes);

/* Forward with a caller-provided device workspace (allocates nothing).
 * q, k, v: device, [B,H,N,d] of dtype, 16-byte aligned.  out: device float32
 * [B,H,N,d], 16-byte aligned, not overlapping q, k, v or ws.  ws: device,
 * 256-byte aligned, at least lapnys_workspace_size bytes; its contents on
 * entry do not matter and on return are unspecified.  Two calls that share a
 * workspace must be ordered (same stream or synchronised). */
int lapnys_forward_ws(const void* q, const void* k, const void* v, float* out,
                      const lapnys_params* p, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* Forward with a library-owned workspace: the call form
 * lapnys_forward(q, k, v, out, params, stream).  The library keeps one
 * workspace per device, grown with hipMalloc on demand (the first call for a
 * size may allocate and synchronise the device), and reuses it; calls on one
 * device must therefore be ordered on a single stream.  lapnys_release frees
 * it.  Arguments as for lapnys_forward_ws. */
int lapnys_forward(const void* q, const void* k, const void* v, float* out,
                   const lapnys_params* p, hipStream_t stream);

/* lapnys_forward_ws, then copies of the intermediates into the non-NULL
 * buffers of dbg (layouts above); synchronises `stream` before returning. */
int lapnys_forward_debug(const void* q, const void* k, const void* v, float* out,
                         const lapnys_params* p, void* ws, size_t ws_bytes,
                         const lapnys_debug* dbg, hipStream_t stream);

/* lapnys_forward_ws that also times its stages: stage_events[2*s] receives
 * the start time of the first kernel of stage s (LAPNYS_STAGE_*) and
 * stage_events[2*s+1] the end time of its last kernel, taken from the
 * kernels' own dispatch timestamps (hipExtLaunchKernel's start/stop events),
 * so hipEventElapsedTime gives the stage's device time and no event command
 * is inserted between kernels.  stage_events: array of 2 * LAPNYS_NUM_STAGES
 * events created by the caller; a NULL entry is not recorded. */
int lapnys_forward_profiled(const void* q, const void* k, const void* v, float* out,
                            const lapnys_params* p, void* ws, size_t ws_bytes,
                            hipEvent_t* stage_events, hipStream_t stream);

/* Backward pass (EN section 3: the kernels serve forward and backward): the
 * gradients of sum(dout * O) with respect to q, k and v, where O is the
 * forward's output for the same inputs and params.  The call runs the forward
 * itself into the workspace (all but its output stage: O is not needed)
 * and then the backward kernels.  The inverse enters as X = W^-1 (dW = -X^T dX X^T, with X
 * the Newton-Schulz result).  Supported: the Laplacian kernel with the
 * Newton-Schulz solver (with or without LAPNYS_NS_REFINE / LAPNYS_NS_PLAIN),
 * every m the forward supports; with LAPNYS_GAUSSIAN or LAPNYS_SOLVER_CG,
 * LAPNYS_ERR_UNSUPPORTED.  The sign of q - K~ and K~ - k is taken exactly (0
 * on ties) for inputs below 2^63 in magnitude.  dout: device float32 [B,H,N,d]; dq, dk,
 * dv: device float32 [B,H,N,d] outputs; all 16-byte aligned, the outputs
 * overlapping neither each other, the inputs nor ws.  ws: at least
 * lapnys_backward_workspace_size bytes, 256-byte aligned. */
int lapnys_backward_workspace_size(const lapnys_params* p, size_t* bytes);
int lapnys_backward_ws(const void* q, const void* k, const void* v, const float* dout, float* dq, float* dk,
                       float* dv, const lapnys_params* p, void* ws, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * lapnys_forward_ws with the library's static device scratch array as the
 * workspace.  Allocates nothing and calls no allocating routine; the first
 * call on a device resolves the array's device address (hipGetSymbolAddress)
 * and keeps it.  Each device holds one array of LAPNYS_SCRATCH_MAX_BYTES
 * (64 MiB) from then until the process ends; it covers every problem whose
 * lapnys_workspace_size is at most that (for example 32 problems of 3136
 * tokens, or 320 problems of 196 tokens, at 49 landmarks), larger ones return
 * LAPNYS_ERR_SCRATCH before anything is enqueued.  Only the single-stream
 * sequence is offered: m <= 64 with the Laplacian kernel and the default
 * Newton-Schulz schedule (LAPNYS_WHITEN and LAPNYS_NS_REFINE allowed); other
 * flags or m > 64 return LAPNYS_ERR_UNSUPPORTED.  Every call on a device
 * shares that device's array and its contents on entry do not matter (the
 * previous call's values are overwritten): calls that overlap in time on one
 * device race, so order them on one stream.  Other arguments as for
 * lapnys_forward_ws. */
#define LAPNYS_SCRATCH_MAX_BYTES ((size_t)64 << 20)
int lapnys_forward_noalloc(const void* q, const void* k, const void* v, float* out,
                           const lapnys_params* p, hipStream_t stream);

/* Frees the library-owned workspaces of lapnys_forward (all devices).
 * Synchronises each device that had one. */
void lapnys_release(void);

/* Static, human-readable text for a status code. */
const char* lapnys_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* LAPNYS_H_ */
