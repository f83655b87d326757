"""Throughput of the Laplacian-kernel Nystrom attention forward on one MI355X.

One step = one full forward (landmark pooling, W + Newton-Schulz, fused
L1+exp kernel matrices with statistics and B V, reductions and Y = X (B V),
whitened output) over the whole synthetic workload, through the C ABI with
inputs already resident in device memory.

Default workload: B=32, H=1, 56x56 token grid (N=3136), d=64, 8x8 pooling
(m=49), lambda=4, eps=1e-3, 20 Newton-Schulz steps, bf16 inputs (float32
arithmetic).  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from lapnys_inputs import HEADLINE, WORKLOADS, make_inputs  # noqa: E402

HEADLINE_METRIC = "attention tokens/s (N=3136,d=64,m=49 bf16) + % VALU/MFMA/HBM roofline"
EVERY = 4  # timed steps per kernel-duration sample

# Measured HBM traffic of the fused kernel-matrix kernel (rocprofv3 FETCH_SIZE
# and WRITE_SIZE passes, scaled by a copy kernel of known size).  Reported only
# while the kernel's sources hash to the value recorded with the counters.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "l1exp_kernel_stage1_56x56_bf16_hbm_traffic.md")
KERNEL_SOURCES = ("l1exp.hip", "kmat_tile.hpp", "ns_small.hpp", "lapnys_internal.hpp", "lapnys_api.hip")

# MI355X figures: 256 CUs at 2.4 GHz; published fp32 vector peak 157.3 TFLOP/s,
# i.e. 78.6e12 fp32 lane-instructions/s counting an FMA as two flops:
# 128 lanes per CU per clock (each of the 4 SIMDs retires 32 lanes a clock when
# two wavefronts co-issue).  The L1 stage's subtract and add are one
# lane-instruction each.  HBM3E 8 TB/s; fp32 MFMA 157.3 TFLOP/s.
CUS, CLOCK_HZ = 256, 2.4e9
VALU_F32_LANE_OPS = CUS * 128 * CLOCK_HZ
HBM_BYTES_S = 8.0e12
MFMA_F32_FLOPS = 157.3e12


def gauss_stage_flops(w) -> float:
    """Algorithmic fp32 MFMA flops of one launch of the Gaussian kernel-matrix
    stage: the dot products of C (N x m) and B (m x N), d multiply-adds each."""
    return 2.0 * (2.0 * w.N * w.m * w.d) * w.P


def kernel_stage_ops(w) -> float:
    """Algorithmic VALU ops of one launch of the fused L1+exp kernel: C = k(Q, K~)
    and B = k(K~, K) are N*m pair-dims each per feature, and every pair-dim is one
    subtract plus one add of the absolute value."""
    pair_dims = 2.0 * w.N * w.m * w.d * w.P
    return 2.0 * pair_dims


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "laplacian_nystr_approximation_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, or None when the
    summary is missing, covers another workload, or predates the current
    kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith("traffic_json:"):
                    rec = json.loads(line.split(":", 1)[1])
                    break
            else:
                return None
    except OSError:
        return None
    if rec.get("workload") != workload or rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return float(rec["bytes_per_launch"])


_CPU_JOB = {}  # the workload and its inputs, inherited by forked oracle workers


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _cpu_problem(p):
    import oracle
    w, x = _CPU_JOB["w"], _CPU_JOB["x"]
    b, h = divmod(p, w.H)
    oracle.attention_problem(x.qf[b, h], x.kf[b, h], x.vf[b, h], grid_h=w.grid_h, grid_w=w.grid_w, pool=w.pool,
                             lam=float(np.float32(w.lam)), eps=float(np.float32(w.eps)), ns_iters=w.ns_iters,
                             whiten=w.whiten, refine=w.refine, kernel=w.kernel, solver=w.solver)
    return p


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, budget_s: float):
    """The oracle as it stands over the workload's (batch, head) problems on a
    process pool of one single-threaded worker per available host core (at
    most 16, the host share of one GPU): problems are handed out in order,
    cycling over the workload as repeated forwards do, until about budget_s
    seconds of CPU work are done (at least one per worker); scaled to
    tokens/s over the completed problems.  Runs before the GPU is touched (the workers are forked)."""
    import multiprocessing as mp
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    _CPU_JOB.update(w=w, x=x)
    ctx = mp.get_context("fork")
    done = 0
    with ctx.Pool(cores, initializer=_cpu_worker_init) as pool:
        t0 = time.perf_counter()
        pending = [pool.apply_async(_cpu_problem, (i % w.P,)) for i in range(cores)]
        issued = len(pending)
        while pending:
            pending.pop(0).get()
            done += 1
            el = time.perf_counter() - t0
            # CPU work so far ~ elapsed x busy workers; keep handing out problems until the budget
            if el * cores < budget_s and issued < 1000 * cores:
                pending.append(pool.apply_async(_cpu_problem, (issued % w.P,)))
                issued += 1
        el = time.perf_counter() - t0
    _CPU_JOB.clear()
    return {"value": done * w.N / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done} (batch, head) problems of the same workload, handed out in order over its {w.P} "
                      f"(N={w.N} tokens each), float64 numpy, {cores} worker processes of one thread "
                      f"each, {el:.2f} s wall"}


def wall_clock_hz() -> float:
    """Rate of the device wall clock (hipDeviceAttributeWallClockRate, kHz)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    v = ctypes.c_int(0)
    dev = ctypes.c_int(0)
    if hip.hipGetDevice(ctypes.byref(dev)) != 0 or hip.hipDeviceGetAttribute(ctypes.byref(v), 10017, dev) != 0:
        raise RuntimeError("hipDeviceGetAttribute(hipDeviceAttributeWallClockRate) failed")
    return v.value * 1e3


def solver_timing(w, L, q, k, v, out, params, ws, dev):
    """The in-launch Newton-Schulz solver's own time, from its workgroups'
    wall-clock stamps (debug form, one warm call), beside the span of the
    kernel-matrix workgroups of the same launch.  MFMA fraction per occupied
    CU: the method's 4 m^3 T flops per problem (float32 products) over the
    solver workgroup's time, against one CU's share of the fp32 MFMA peak."""
    import torch
    nsc = torch.zeros((w.P, 3), dtype=torch.int64, device=dev)
    kc = torch.zeros(2, dtype=torch.int64, device=dev)
    L.lapnys_forward_debug(q, k, v, out, params, ws, {"ns_clock": nsc, "kernel_clock": kc})
    hz = wall_clock_hz()
    c = nsc.cpu().numpy().astype(np.float64)
    kcl = kc.cpu().numpy().astype(np.float64)
    us = 1e6 / hz
    per = (c[:, 2] - c[:, 0]) * us
    steps = (c[:, 2] - c[:, 1]) * us
    flops = 4.0 * w.m ** 3 * w.ns_iters
    cu_peak = MFMA_F32_FLOPS / CUS
    return {"source": "solver workgroups' wall-clock stamps (lapnys_forward_debug ns_clock / kernel_clock)",
            "solver_span_us": float((c[:, 2].max() - c[:, 0].min()) * us),
            "per_problem_us_mean": float(per.mean()), "per_problem_us_max": float(per.max()),
            "setup_us_mean": float(((c[:, 1] - c[:, 0]) * us).mean()), "steps_us_mean": float(steps.mean()),
            "kernel_matrix_span_us": float((kcl[1] - kcl[0]) * us),
            "solver_end_after_kernel_matrix_start_us": float((c[:, 2].max() - kcl[0]) * us),
            "mfma_flops_per_problem": flops,
            "mfma_frac_per_occupied_cu": float(flops / (per.mean() * 1e-6) / cu_peak),
            "mfma_frac_per_occupied_cu_steps_only": float(flops / (steps.mean() * 1e-6) / cu_peak),
            "chip_wide_mfma_frac": float(flops * w.P / ((c[:, 2].max() - c[:, 0].min()) * us * 1e-6)
                                         / MFMA_F32_FLOPS)}


def stage_hbm_bytes(w):
    """Algorithmic HBM bytes per forward of the stages bounded by memory (all
    problems): what each must read and write at least, from the sizes alone."""
    s_in = 2 if w.dtype == "bf16" else 4
    P, N, d, m = w.P, w.N, w.d, w.m
    ntiles = -(-N // 256)
    jblocks = 1 if m <= 64 else -(-m // 32)
    tpg = max(1, ntiles * jblocks * P // 4096)
    groups = -(-ntiles // tpg)
    mp = 64 if m <= 64 else -(-m // 64) * 64
    pool = P * (N * d * s_in + m * d * 4)
    # partials in; B V, statistics out; X in and Y (split, or float32 for m > 64) out
    y_out = 2 * d * 64 * 2 if m <= 64 else m * d * 4
    finalize = P * (groups * m * d * 4 + ntiles * m * 8 + mp * mp * 4 + m * d * 4 + 3 * m * 4 + y_out)
    output = P * (m * N * 4 + N * d * 4 + y_out + 2 * m * 4)
    return {"pool": pool, "finalize": finalize, "output": output}


def stage_rooflines(w, stage_ms):
    out = {}
    for name, nbytes in stage_hbm_bytes(w).items():
        t = stage_ms[name] * 1e-3
        gbs = nbytes / t / 1e9
        out[name] = {"bound": "hbm", "achieved": gbs, "peak": HBM_BYTES_S / 1e9, "unit": "GB/s",
                     "frac": gbs * 1e9 / HBM_BYTES_S, "bytes": nbytes, "ms": stage_ms[name]}
    return out


# (workload, LAPNYS_NS_REFINE): the refined lines price the float64-residual
# correction of the Newton-Schulz result.
SWEEP = (("sweep_64x64_bf16", False), ("sweep_128x128_bf16", False), ("long_256x256_bf16", False),
         ("long_256x256_bf16", True), (HEADLINE, False), (HEADLINE, True))


def sweep_main(args):
    """Time against N at m = 256 (and the headline workload), warm and cold.

    Per workload: the median, 10th and 90th percentile of single-call device
    times (events around one forward on the stream); warm = back to back, cold
    = a 512 MiB buffer written between calls so the last-level cache holds
    none of the inputs; and the peak device memory of inputs, workspace and
    output (the _ws form allocates nothing itself); and the median device time
    of the solver stage (its own kernels' dispatch timestamps, warm).  One JSON
    line each."""
    import dataclasses

    import torch
    import laplacian_nystr_approximation_amd.lapnys as L
    from lapnys_inputs import make_inputs

    dev = torch.device("cuda:0")
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for name, refine in SWEEP:
        w = dataclasses.replace(WORKLOADS[name], refine=refine)
        x = make_inputs(w)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)

        def up(a):
            a = np.ascontiguousarray(a)
            return torch.from_numpy(a.view(np.int16) if w.dtype == "bf16" else a).to(dev)

        q, k, v = up(x.q), up(x.k), up(x.v)
        del x
        params = L.params_for(w)
        out = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
        ws = torch.empty(L.lapnys_workspace_size(params), dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream()
        reps = 50 if w.N <= 16384 else 20
        times = {}
        for mode in ("warm", "cold"):
            for _ in range(5):
                L.lapnys_forward_ws(q, k, v, out, params, ws, stream)
            ts = []
            for _ in range(reps):
                if mode == "cold":
                    flush.fill_(1)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                L.lapnys_forward_ws(q, k, v, out, params, ws, stream)
                e1.record(stream)
                e1.synchronize()
                ts.append(e0.elapsed_time(e1))
            times[mode] = {"median_ms": float(np.median(ts)), "p10_ms": float(np.percentile(ts, 10)),
                           "p90_ms": float(np.percentile(ts, 90))}
        ns = 2 * L.LAPNYS_STAGE_NS
        evs = L.HipEvents(2 * reps)
        for i in range(reps):
            slots = [None] * (2 * L.LAPNYS_NUM_STAGES)
            slots[ns], slots[ns + 1] = evs.handles[2 * i], evs.handles[2 * i + 1]
            L.lapnys_forward_profiled(q, k, v, out, params, ws, slots, stream)
        torch.cuda.synchronize()
        ns_ms = float(np.median([evs.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps)]))
        evs.close()
        peak = torch.cuda.max_memory_allocated(dev) - base
        print(json.dumps({"workload": name, "refine": refine, "N": w.N, "m": w.m, "P": w.P, "d": w.d,
                          "ns_iters": w.ns_iters, "ns_stage_ms": ns_ms,
                          "tokens_per_s_warm": w.P * w.N / (times["warm"]["median_ms"] * 1e-3),
                          "warm": times["warm"], "cold": times["cold"], "peak_device_bytes": int(peak),
                          "workspace_bytes": int(ws.numel())}), flush=True)
        del q, k, v, out, ws
        torch.cuda.empty_cache()
    return 0


def kernel_value_comparison(w, q, k, v, dev):
    """Both kernels' C = k(Q, K~) on the same inputs, from the GPU's own
    intermediates (the debug form): quantiles of all entries, the share below
    1e-6, and per query the largest landmark's share of the row sum (how far
    one landmark dominates), averaged over queries.  The pages' argument
    against the Gaussian kernel on heavy-tailed distances is that it
    suppresses moderate interactions and lets outliers dominate."""
    import dataclasses

    import torch
    import laplacian_nystr_approximation_amd as L

    out = {}
    for kern in ("laplacian", "gaussian"):
        wk = dataclasses.replace(w, kernel=kern)
        params = L.params_for(wk)
        ws = torch.empty(L.lapnys_workspace_size(params), dtype=torch.uint8, device=dev)
        o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
        ct = torch.empty((w.P, w.m, w.N), dtype=torch.float32, device=dev)
        L.lapnys_forward_debug(q, k, v, o, params, ws, {"C_t": ct})
        c = ct.double()
        qs = torch.quantile(c.flatten()[:: -(-c.numel() // (1 << 23))],
                            torch.tensor([0.01, 0.1, 0.5, 0.9, 0.99], dtype=torch.float64, device=dev))
        top_share = (c.max(dim=1).values / c.sum(dim=1).clamp_min(1e-300)).mean()
        out[kern] = {"quantiles_1_10_50_90_99": [float(t) for t in qs.cpu()],
                     "share_below_1e-6": float((c < 1e-6).double().mean()),
                     "mean_top_landmark_share": float(top_share)}
        del ws, o, ct, c
    return out


def solver_study_main(args):
    """Residual against iterations, Newton-Schulz against CG, on W made
    ill-conditioned by a small eps or by near-duplicate landmarks (the pages'
    solver ablation, reproduced on synthetic inputs).  Solvers: "ns" (the
    default m <= 64 schedule), "ns_plain" (LAPNYS_NS_PLAIN) and "cg".  Per
    condition and step count T, for each solver, on the GPU (float32, the library's own W, X, Y
    and B V from the debug form) and in float64 on the same W and B V (the
    oracle's solvers): the relative residual of the solve, ||W Y - B V|| /
    ||B V||, the quantity the output depends on.  One JSON line each."""
    import dataclasses

    import torch
    import laplacian_nystr_approximation_amd as L
    import oracle
    from lapnys_inputs import make_inputs

    dev = torch.device("cuda:0")
    base = dataclasses.replace(WORKLOADS["stage1_56x56_f32"], B=4, name="study_56x56_f32")
    conditions = [("eps=1e-1", 1e-1, None), ("eps=1e-3", 1e-3, None),
                  ("eps=1e-3, near-duplicate landmarks (delta=1e-2)", 1e-3, 1e-2),
                  ("eps=1e-5, near-duplicate landmarks (delta=1e-3)", 1e-5, 1e-3),
                  ("eps=1e-6, near-duplicate landmarks (delta=1e-4)", 1e-6, 1e-4)]
    steps = (4, 8, 12, 16, 20, 24, 32, 48)
    P, m = base.P, base.m
    for label, eps, delta in conditions:
        # Near-duplicate landmarks: every odd pooled window column of K copies
        # its left neighbour plus delta-scaled noise (lapnys_inputs).
        x = make_inputs(base if delta is None else base.with_(near_dup=delta))
        q, k, v = (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev) for a in (x.q, x.k, x.v))
        kappa = None
        for solver in ("ns", "ns_plain", "cg"):
            for T in steps:
                w = dataclasses.replace(base, eps=eps, ns_iters=T, solver="cg" if solver == "cg" else "ns",
                                        ns_plain=solver == "ns_plain")
                params = L.params_for(w)
                ws = torch.empty(L.lapnys_workspace_size(params), dtype=torch.uint8, device=dev)
                out = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
                dbg = {"W": torch.empty((P, m, m), device=dev), "X": torch.zeros((P, m, m), device=dev),
                       "Y": torch.empty((P, m, w.d), device=dev), "BV": torch.empty((P, m, w.d), device=dev)}
                L.lapnys_forward_debug(q, k, v, out, params, ws, dbg)
                W_, Y_, BV_ = (dbg[key].cpu().double().numpy() for key in ("W", "Y", "BV"))
                gpu_res, f64_res = [], []
                for p_ in range(P):
                    nb = np.linalg.norm(BV_[p_])
                    gpu_res.append(float(np.linalg.norm(W_[p_] @ Y_[p_] - BV_[p_]) / nb))
                    if solver != "cg":
                        y64 = oracle.newton_schulz_inverse(W_[p_], T) @ BV_[p_]
                    else:
                        y64 = oracle.conjugate_gradient(W_[p_], BV_[p_], T)
                    f64_res.append(float(np.linalg.norm(W_[p_] @ y64 - BV_[p_]) / nb))
                if kappa is None:
                    ev = [np.linalg.eigvalsh(W_[p_]) for p_ in range(P)]
                    kappa = [float(e[-1] / e[0]) for e in ev]
                print(json.dumps({"condition": label, "solver": solver, "steps": T,
                                  "gpu_rel_residual_max": max(gpu_res), "f64_rel_residual_max": max(f64_res),
                                  "kappa_W": [min(kappa), max(kappa)], "finite": bool(np.isfinite(Y_).all())}),
                      flush=True)
                del ws, out, dbg
    return 0


def valu_probe_main(args):
    """VALU issue rate of the L1 loop's instruction pair (v_sub_f32, then
    v_add_f32 with an |.| source) with register operands, at 1, 2, 3, 4 and 8
    wavefronts per SIMD (laplacian_nystr_approximation_amd/probe/valu_probe.hip).
    One JSON line per occupancy: kernel time (events) and lane-operations per
    CU per clock at the 2.4 GHz peak clock; a counter pass (SQ_INSTS_VALU,
    GRBM_GUI_ACTIVE) gives the same per the clock actually run."""
    import ctypes

    import torch  # noqa: F401  (loads the HIP runtime the probe links against)
    lib = ctypes.CDLL(os.path.join(ROOT, "laplacian_nystr_approximation_amd", "libvaluprobe.so"))
    lib.valu_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float),
                                   ctypes.POINTER(ctypes.c_double)]
    lib.valu_probe_run.restype = ctypes.c_int
    for waves in (1, 2, 3, 4, 8):
        ms, ops = ctypes.c_float(), ctypes.c_double()
        rc = lib.valu_probe_run(waves, args.probe_iters, 4, ctypes.byref(ms), ctypes.byref(ops))
        if rc != 0:
            print(json.dumps({"waves_per_simd": waves, "hip_error": rc}), flush=True)
            return 1
        per_clk = ops.value / (ms.value * 1e-3) / (CUS * CLOCK_HZ)
        print(json.dumps({"probe": "valu_sub_add_abs", "waves_per_simd": waves, "kernel_ms": ms.value,
                          "lane_ops": ops.value, "lane_ops_per_s": ops.value / (ms.value * 1e-3),
                          "lane_ops_per_cu_per_clock_at_2.4GHz": per_clk}), flush=True)
    return 0


def backward_main(args):
    """The backward pass (lapnys_backward_ws: the forward, then the gradients of
    sum(dO * O) with respect to Q, K, V) on the bench workload: warm-up, then
    K timed calls; one JSON line with tokens/s of forward + backward."""
    import torch
    import laplacian_nystr_approximation_amd as L
    from lapnys_inputs import make_grad_out, make_inputs

    w = WORKLOADS[args.workload]
    x = make_inputs(w)
    dev = torch.device("cuda:0")

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if w.dtype == "bf16" else a).to(dev)

    q, k, v = up(x.q), up(x.k), up(x.v)
    dout = torch.from_numpy(make_grad_out(w)).to(dev)
    dq, dk, dv = (torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev) for _ in range(3))
    params = L.params_for(w)
    ws = torch.empty(L.lapnys_backward_workspace_size(params), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        L.lapnys_backward_ws(q, k, v, dout, dq, dk, dv, params, ws, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        L.lapnys_backward_ws(q, k, v, dout, dq, dk, dv, params, ws, stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    print(json.dumps({"metric": f"attention forward+backward tokens/s ({w.name})",
                      "value": w.P * w.N / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "dtype": "f32",
                      "data": "synthetic", "config": {"workload": w.name, "N": w.N, "m": w.m, "d": w.d, "P": w.P,
                                                       "input_dtype": w.dtype}}), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--kernel", default="laplacian", choices=("laplacian", "gaussian"),
                    help="gaussian: the Gaussian-kernel variant of the same forward (LAPNYS_GAUSSIAN)")
    ap.add_argument("--solver", default="ns", choices=("ns", "cg"),
                    help="cg: the conjugate-gradient solver variant (LAPNYS_SOLVER_CG)")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the bench line: forward + backward (lapnys_backward_ws) on the workload")
    ap.add_argument("--solver-study", action="store_true",
                    help="instead of the bench line: solve residual against steps, Newton-Schulz and CG, on "
                         "ill-conditioned W (small eps, near-duplicate landmarks), GPU and float64")
    ap.add_argument("--valu-probe", action="store_true",
                    help="instead of the bench line: the VALU issue-rate probe of the L1 instruction pair")
    ap.add_argument("--probe-iters", type=int, default=4000)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time (0: skip)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the bench line: warm and cold single-call times and peak memory over the "
                         "length sweep at m = 256 and the headline workload")
    ap.add_argument("--all-configs", action="store_true",
                    help="one bench line per configuration (the five forward workloads, the headline workload and "
                         "the length-sweep points), each from a child process running that workload's bench")
    ap.add_argument("--fill-baseline", default=None,
                    help="rewrite BASELINE.md section 4 from the bench lines in this file (no GPU)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="after the measurements, run a plain float32 copy kernel of this many MiB three times "
                         "(the known-size reference for HBM traffic counters)")
    args = ap.parse_args(argv)
    if args.sweep:
        return sweep_main(args)
    if args.solver_study:
        return solver_study_main(args)
    if args.backward:
        return backward_main(args)
    if args.valu_probe:
        return valu_probe_main(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this forward has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    if args.fill_baseline:
        return fill_baseline_main(args)
    if args.all_configs:
        # One child process per configuration, each the same command as a
        # single-workload run (its oracle leg, then its GPU line), so no line
        # is measured after another configuration's work in the same process.
        # This process touches no GPU.
        import subprocess
        for name in ALL_CONFIGS:
            cmd = [sys.executable, os.path.abspath(__file__), "--workload", name, "--steps", str(args.steps),
                   "--warmup", str(args.warmup), "--cpu-budget", str(args.cpu_budget), "--kernel", args.kernel,
                   "--solver", args.solver]
            r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
            if r.returncode != 0:
                print(f"bench.py --workload {name} failed ({r.returncode})", file=sys.stderr)
                return r.returncode
            lines = [line for line in r.stdout.splitlines() if line.startswith("{")]
            print(lines[-1], flush=True)
        return 0
    names = [args.workload]
    ws_ = []
    for name in names:
        w = WORKLOADS[name]
        if args.kernel != "laplacian" or args.solver != "ns":
            import dataclasses
            w = dataclasses.replace(w, kernel=args.kernel, solver=args.solver)
        ws_.append(w)
    inputs = [make_inputs(w) for w in ws_]
    # The CPU legs run before the GPU is touched (their workers are forked).
    cpus = [cpu_baseline(w, x, args.cpu_budget) if args.cpu_budget > 0 else None for w, x in zip(ws_, inputs)]
    for w, x, cpu in zip(ws_, inputs, cpus):
        line = gpu_line(w, x, cpu, args)
        print(json.dumps(line), flush=True)
    return 0


PRECISION = ("float32 values throughout (bf16 inputs widen exactly); L1 distances, exp, W and whitening statistics "
             "on the float32 vector ALU (statistics merged in float64, landmarks summed in float64); B V, Z Y and "
             "the Newton-Schulz steps for m <= 64 (all but the last) on bf16 MFMA with every float32 operand "
             "split into bf16 high and low parts, three partial products accumulated in float32; Y = X (B V), the "
             "last Newton-Schulz steps and the m > 64 solver on fp32 MFMA")

# The configurations the bench lines cover: the five forward workloads, the
# headline workload (the 56x56 shape with bf16 inputs) and the two smaller
# points of the length sweep at 256 landmarks.
ALL_CONFIGS = ["tiny_f32", "stage1_56x56_f32", "stage2_28x28_bf16", "stage3_14x14_bf16", "long_256x256_bf16",
               HEADLINE, "sweep_64x64_bf16", "sweep_128x128_bf16"]
CLOCK_WARMUP_S = 0.03  # the GPU reaches its steady clock after ~15 ms of sustained work


def gpu_line(w, x, cpu, args):
    """One bench line for workload w: warm-up, exactly K timed steps, the
    kernel-matrix kernel's duration from its dispatch timestamps, a per-stage
    breakdown, the in-launch solver's stamps."""
    import torch

    import laplacian_nystr_approximation_amd as L
    from laplacian_nystr_approximation_amd.lapnys import LAPNYS_NUM_STAGES, LAPNYS_STAGE_KERNEL, STAGE_NAMES

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if w.dtype == "bf16" else a).to(dev)

    q, k, v = up(x.q), up(x.k), up(x.v)
    params = L.params_for(w)
    out = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
    ws = torch.empty(L.lapnys_workspace_size(params), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    K, W = args.steps, args.warmup
    per_step = 2 * LAPNYS_NUM_STAGES
    kern = 2 * LAPNYS_STAGE_KERNEL

    # Clock warm-up (untimed, before the W warm-up steps): forward calls until
    # CLOCK_WARMUP_S of wall time have passed, so the timed steps run at the
    # GPU's steady clock whatever W is.
    clock_steps = 0
    tw = time.perf_counter()
    while time.perf_counter() - tw < CLOCK_WARMUP_S:
        for _ in range(8):
            L.lapnys_forward_ws(q, k, v, out, params, ws, stream)
        clock_steps += 8
        torch.cuda.synchronize()
    for _ in range(W):
        L.lapnys_forward_ws(q, k, v, out, params, ws, stream)
    torch.cuda.synchronize()

    # Timed region: K steps.  Every EVERY-th step goes through the profiled
    # entry point, whose timing events take the fused kernel-matrix kernel's own
    # dispatch timestamps on the stream that runs it; the others through the
    # plain entry point (an event-carrying launch costs the step a few
    # microseconds, so timing every step would understate the throughput).
    sampled = list(range(0, K, EVERY))
    ev = L.HipEvents(2 * len(sampled))
    t0 = time.perf_counter()
    for i in range(K):
        if i % EVERY == 0:
            e = i // EVERY
            slots = [None] * per_step
            slots[kern], slots[kern + 1] = ev.handles[2 * e], ev.handles[2 * e + 1]
            L.lapnys_forward_profiled(q, k, v, out, params, ws, slots, stream)
        else:
            L.lapnys_forward_ws(q, k, v, out, params, ws, stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    kernel_ms = float(np.mean([ev.elapsed_ms(2 * e, 2 * e + 1) for e in range(len(sampled))]))
    ev.close()

    # Untimed breakdown: every stage bracketed by events (the extra event
    # records lengthen these steps slightly); the median over the K steps, so
    # that one stalled step does not move a stage of a few microseconds.
    evs = L.HipEvents(per_step * K)
    for i in range(K):
        L.lapnys_forward_profiled(q, k, v, out, params, ws, evs.handles[i * per_step:(i + 1) * per_step], stream)
    torch.cuda.synchronize()
    stage_ms = {name: float(np.median([evs.elapsed_ms(i * per_step + 2 * s, i * per_step + 2 * s + 1)
                                       for i in range(K)]))
                for s, name in enumerate(STAGE_NAMES)}
    evs.close()

    solver = None
    in_launch = (w.kernel == "laplacian" and w.solver == "ns" and w.m <= 64 and not w.ns_plain)
    if in_launch:
        # The solver runs inside the kernel-matrix launch: its own stamps, not
        # events around the launch, give its time.
        solver = solver_timing(w, L, q, k, v, out, params, ws, dev)
        stage_ms.pop("ns", None)
    elif w.solver == "ns":
        # The solver's own launches on the side stream: the stage span.
        flops = 4.0 * (((w.m + 63) // 64) * 64) ** 3 * w.ns_iters * w.P
        solver = {"source": "events at the first and last solver launch (side stream)", "stage_ms": stage_ms["ns"],
                  "padded_mfma_flops": flops,
                  "chip_wide_mfma_frac": flops / (stage_ms["ns"] * 1e-3) / MFMA_F32_FLOPS,
                  "algorithmic_mfma_frac": 4.0 * w.m ** 3 * w.ns_iters * w.P / (stage_ms["ns"] * 1e-3)
                                           / MFMA_F32_FLOPS}

    # Same work without any stage events.
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(K):
        L.lapnys_forward_ws(q, k, v, out, params, ws, stream)
    torch.cuda.synchronize()
    plain_ms = (time.perf_counter() - t2) * 1e3 / K

    if args.copy_mb > 0:
        n = args.copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    tokens = w.P * w.N
    gauss = w.kernel == "gaussian"
    if gauss:
        roof = {"kernel": "gauss_kernel (squared L2 on fp32 MFMA + exp, C store, column statistics, B V)",
                "bound": "mfma", "unit": "TFLOP/s", "peak": MFMA_F32_FLOPS / 1e12,
                "achieved": gauss_stage_flops(w) / (kernel_ms * 1e-3) / 1e12, "traffic": None}
    else:
        roof = {"kernel": "l1exp_kernel (fused L1 + exp, C store, column statistics, B V)",
                "bound": "alu", "unit": "TOP/s", "peak": VALU_F32_LANE_OPS / 1e12,
                "achieved": kernel_stage_ops(w) / (kernel_ms * 1e-3) / 1e12, "traffic": measured_traffic(w.name)}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel_ms"] = kernel_ms
    roof["kernel_ms_samples"] = f"HIP events on every {EVERY}th timed step ({len(sampled)} of {K})"
    if w.name == HEADLINE and not gauss and w.solver == "ns":
        metric = HEADLINE_METRIC
    else:
        variant = (", Gaussian kernel" if gauss else "") + (", CG solver" if w.solver == "cg" else "")
        metric = f"attention tokens/s ({w.name}{variant})"
    # Z Y in the output stage: 2 N m d flops per problem (run as three bf16 products)
    zy_flops = 2.0 * w.N * w.m * w.d * w.P
    line = {
        "metric": metric,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "clock_warmup_steps": clock_steps,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32+bf16x3",
        "precision": PRECISION,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "grid": [w.grid_h, w.grid_w], "N": w.N, "d": w.d,
                   "pool": w.pool, "m": w.m, "input_dtype": w.dtype, "lambda": w.lam, "eps": w.eps,
                   "ns_iters": w.ns_iters, "whiten": w.whiten, "kernel": w.kernel, "solver": w.solver},
        "roofline": roof,
        "cpu_baseline": cpu,
        "stage_ms": stage_ms,
        "solver": solver,
        "stage_roofline": stage_rooflines(w, stage_ms),
        "output_zy_mfma": {"flops": zy_flops, "ms": stage_ms["output"],
                           "frac_of_fp32_mfma_peak": zy_flops / (stage_ms["output"] * 1e-3) / MFMA_F32_FLOPS,
                           "note": "algorithmic flops of Z Y over the whole output stage time (HBM-bound stage)"},
        "ms_per_step_without_events": plain_ms,
    }
    if gauss:
        line["kernel_values"] = kernel_value_comparison(w, q, k, v, dev)
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    return line


def fill_baseline_main(args):
    """Rewrite the benchmark spec section 4 from the bench lines recorded in a file
    (lines starting with '{'), one table row per workload."""
    rows = []
    with open(args.fill_baseline) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                rows.append(json.loads(line))
    out = ["## 4. Results", "",
           f"Filled by `python bench.py --fill-baseline {os.path.relpath(args.fill_baseline, ROOT)}` from the bench "
           "lines recorded there (one MI355X, `python bench.py --all-configs`); no value is entered by hand.", "",
           "| Workload | P | N | m | tokens/s (GPU) | ms per forward | L1+exp VALU frac | NS MFMA frac | "
           "pool / output HBM frac | oracle tokens/s (cores) |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        c = r["config"]
        sol = r.get("solver") or {}
        if "mfma_frac_per_occupied_cu" in sol:
            ns = f"{sol['mfma_frac_per_occupied_cu']:.2f} per occupied CU ({sol['per_problem_us_mean']:.0f} us per problem)"
        elif "algorithmic_mfma_frac" in sol:
            ns = f"{sol['algorithmic_mfma_frac']:.3f} chip-wide ({sol['stage_ms'] * 1e3:.0f} us stage)"
        else:
            ns = "-"
        sr = r.get("stage_roofline", {})
        hbm = f"{sr['pool']['frac']:.2f} / {sr['output']['frac']:.2f}" if "pool" in sr else "-"
        cpu = r.get("cpu_baseline") or {}
        cpus = f"{cpu['value']:.3g} ({cpu['cores']})" if cpu else "-"
        out.append(f"| `{c['workload']}` | {c['B'] * c['H']} | {c['N']} | {c['m']} | {r['value']:.3g} | "
                   f"{r['ms_per_step']:.4f} | {r['roofline']['frac']:.2f} | {ns} | {hbm} | {cpus} |")
    out.append("")
    path = os.path.join(ROOT, "BASELINE.md")
    text = open(path).read()
    i = text.index("## 4. Results")
    with open(path, "w") as f:
        f.write(text[:i] + "\n".join(out))
    print("\n".join(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
