"""Benchmark of the fused GEMM-RMSNorm-GEMM + SwiGLU block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

One step = one pass of the fused hot path over the LLaMA-3-1B-shaped MLP
block (M = 8192 tokens, d = 2048, ffn = 8192, bf16, fp32 accumulate):
GEMM1 (residual add + partial sums of squares) -> RMS reduce -> GEMM2 (row
scale + SwiGLU).  Inputs are seeded synthetic tensors already resident in
HBM; the RMSNorm gain is folded into the gate/up weights once, before timing
(weight preparation, not per-token work).

Prints ONE JSON line: fused-block TFLOP/s (the metric), the unfused GPU
sequence timed the same way, the dominant kernel's roofline figure measured
with HIP events on the launch stream, and the CPU oracle's throughput on a
bounded row sample (a baseline only).
"""

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, 2.4 GHz
WORKLOAD = "mlp_1b"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=100,
                   help="untimed steps (fused and unfused sequence each) before timing; the "
                        "shader clock settles over the first ~35 ms of sustained load, so the "
                        "default covers about 100 ms")
    p.add_argument("--warmup-ms", type=float, default=200.0,
                   help="GPU-time floor of the warm-up: after the --warmup steps, fused and "
                        "unfused steps keep alternating until this much GPU time has passed, so "
                        "the timed steps start on a settled shader clock")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-rows", action="store_true",
                   help="skip the other_rows workloads (attention input, LM head, the layer "
                        "at 1B / 7B / 70B, the 7B and 70B MLP blocks, the backward, fp8)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="before timing, copy a buffer of this many MiB three times (a plain "
                        "copy kernel of known size, to scale HBM byte counters)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time budget of the oracle baseline")
    p.add_argument("--row-min-ms", type=float, default=60.0,
                   help="minimum GPU time of the warm-up and of the timed steps of each "
                        "other_rows workload (0: exactly --steps / 3 warm-up steps)")
    p.add_argument("--no-cold", action="store_true",
                   help="skip the pass that overwrites 1 GiB between steps (operands evicted "
                        "from the 256 MB memory-side cache)")
    return p.parse_args()


_ROW_MIN_MS = 60.0


def main():
    global _ROW_MIN_MS
    args = parse()
    _ROW_MIN_MS = args.row_min_ms
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    from gemm_epilogue_transformer_gemm1_amd import inputs, ops

    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = inputs.make_workload(WORKLOAD)
    M, d, K1, ffn = (w.sizes[k] for k in ("M", "d", "K1", "ffn"))
    eps = 1e-5

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(dev)

    x, res, w1 = bf(w.arrays["x"]), bf(w.arrays["res"]), bf(w.arrays["w1"])
    wg, wu = bf(w.arrays["wg"]), bf(w.arrays["wu"])
    gamma = torch.from_numpy(w.arrays["gamma"]).to(dev)
    # weight preparation (untimed): fold gamma into gate / up weights
    wg_f, wu_f = torch.empty_like(wg), torch.empty_like(wu)
    ops.fold_gamma(wg, gamma, wg_f)
    ops.fold_gamma(wu, gamma, wu_f)
    wgu = torch.cat([wg, wu], 0).contiguous()  # unfused path: one GEMM for gate|up

    T = ops.rms_tiles(d)
    h = torch.empty(M, d, dtype=torch.bfloat16, device=dev)
    P = torch.empty(T, M, dtype=torch.float32, device=dev)
    r = torch.empty(M, dtype=torch.float32, device=dev)
    out = torch.empty(M, ffn, dtype=torch.bfloat16, device=dev)
    # unfused buffers
    y_u, h_u, n_u = (torch.empty(M, d, dtype=torch.bfloat16, device=dev) for _ in range(3))
    gu_u = torch.empty(M, 2 * ffn, dtype=torch.bfloat16, device=dev)
    out_u = torch.empty(M, ffn, dtype=torch.bfloat16, device=dev)

    stream = torch.cuda.current_stream()
    flops_g1 = 2.0 * M * d * K1
    flops_g2 = 2.0 * M * (2 * ffn) * d
    flops = flops_g1 + flops_g2

    def fused_step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        ops.gemm_residual_partialrms(x, w1, res, h, P)
        if ev is not None:
            ev[1].record(stream)
        ops.rms_reduce(P, d, eps, r)
        if ev is not None:
            ev[2].record(stream)
        ops.gemm_rowscale_swiglu(h, wg_f, wu_f, r, out)
        if ev is not None:
            ev[3].record(stream)

    def unfused_step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        ops.gemm_bf16(x, w1, y_u)
        ops.residual_add(y_u, res, h_u)
        ops.rmsnorm(h_u, gamma, eps, n_u)
        ops.gemm_bf16(n_u, wgu, gu_u)
        ops.swiglu(gu_u, out_u)
        if ev is not None:
            ev[3].record(stream)

    def timed(step_fn, steps, per_kernel=False):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for s in range(steps):
            step_fn(evs[s]) if per_kernel else step_fn()
        stop.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        total_ms = start.elapsed_time(stop)
        per = None
        if per_kernel:
            per = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(3)] for e in evs])
        return total_ms, wall, per

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copied {args.calibrate_copy} MiB x3", file=sys.stderr, flush=True)
        del src, dst

    print(f"[bench] warmup {args.warmup} steps (floor {args.warmup_ms:.0f} ms of GPU time)",
          file=sys.stderr, flush=True)
    wa, wb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wa.record(stream)
    for _ in range(args.warmup):
        fused_step()
        unfused_step()
    wb.record(stream)
    torch.cuda.synchronize()
    warm_ms, warm_pairs = wa.elapsed_time(wb), args.warmup
    while warm_ms < args.warmup_ms:
        # one fused + unfused pair takes about 1 ms; top up in chunks
        pair_ms = warm_ms / warm_pairs if warm_pairs else 1.0
        extra = int(min(500, max(1, np.ceil((args.warmup_ms - warm_ms) / max(pair_ms, 0.05)))))
        wa.record(stream)
        for _ in range(extra):
            fused_step()
            unfused_step()
        wb.record(stream)
        torch.cuda.synchronize()
        warm_ms += wa.elapsed_time(wb)
        warm_pairs += extra

    print(f"[bench] timing {args.steps} fused steps", file=sys.stderr, flush=True)
    # 1) whole-step throughput, no events between kernels: the headline pass, right after
    #    the warm-up
    fused_ms, fused_wall, _ = timed(fused_step, args.steps)
    print(f"[bench] timing {args.steps} unfused steps", file=sys.stderr, flush=True)
    unfused_ms, _, _ = timed(unfused_step, args.steps)
    # the same two passes twice more, alternating, so that the fused/unfused ratio does not
    # depend on which sequence ran first
    fused_passes, unfused_passes = [fused_ms], [unfused_ms]
    for _ in range(2):
        fused_passes.append(timed(fused_step, args.steps)[0])
        unfused_passes.append(timed(unfused_step, args.steps)[0])
    # 2) per-kernel durations with events on the launch stream
    _, _, per = timed(fused_step, args.steps, per_kernel=True)
    # per-step distribution (events before and after every step)
    fused_steps = np.array([per[k].sum() for k in range(args.steps)])
    unf_steps = step_times(torch, stream, unfused_step, args.steps)

    # context only: the same unfused block in eager PyTorch (torch.mm on hipBLASLt, torch
    # elementwise and reduction kernels), the analogue of the vendor-BLAS + PyTorch baseline the
    # page compares against; weights transposed once, outside the timed region
    print("[bench] torch eager unfused sequence (context)", file=sys.stderr, flush=True)
    w1_t, wgu_t = w1.t().contiguous(), wgu.t().contiguous()
    g32 = gamma.to(torch.float32)

    def torch_step():
        hh = torch.mm(x, w1_t) + res
        h32 = hh.float()
        nn = (h32 * torch.rsqrt(h32.pow(2).mean(-1, keepdim=True) + eps) * g32).to(torch.bfloat16)
        gu = torch.mm(nn, wgu_t)
        return torch.nn.functional.silu(gu[:, :ffn]) * gu[:, ffn:]
    for _ in range(max(3, args.warmup // 10)):
        torch_step()
    torch_ms = float(np.median(step_times(torch, stream, torch_step, args.steps)))
    del w1_t, wgu_t

    cold = None
    if not args.no_cold:
        print("[bench] cold pass (1 GiB overwritten before every step)", file=sys.stderr,
              flush=True)
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        cold = {"fused_step_ms": pctl(step_times_cold(torch, stream, fused_step, args.steps,
                                                      scratch)),
                "unfused_step_ms": pctl(step_times_cold(torch, stream, unfused_step,
                                                        args.steps, scratch)),
                "note": "events around each step only; before each step a 1 GiB buffer is "
                        "overwritten so the step's operands are not resident in the "
                        "256 MB memory-side cache"}
        del scratch

    ms_step = fused_ms / args.steps
    tflops = flops / (ms_step * 1e-3) / 1e12
    unf_ms_step = unfused_ms / args.steps
    unf_tflops = flops / (unf_ms_step * 1e-3) / 1e12
    g1_ms, red_ms, g2_ms = (float(np.mean(per[:, i])) for i in range(3))
    g2_tflops = flops_g2 / (g2_ms * 1e-3) / 1e12

    clock = measured_clock_ghz("gemm_rowscale_swiglu")
    rows = {}
    if not args.no_rows:
        rows = time_other_rows(torch, ops, inputs, stream, min(args.steps, 10), 3)

    cpu = None
    if not args.no_cpu:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, eps, args.cpu_seconds)

    line = {
        "metric": "fused block TFLOP/s (GEMM1 residual+partial-RMS -> reduce -> GEMM2 "
                  "row-scale+SwiGLU), LLaMA-1B-shaped MLP",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/d) weights, random init)",
        "config": {"workload": "mlp_1b: M=8192 tokens (4x2048), d=2048, ffn=8192, "
                               "gate/up with SwiGLU, eps=1e-5",
                   "M": M, "d": d, "K1": K1, "ffn": ffn, "parallelism": "none (1 GPU)"},
        "pct_of_mfma_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "step_ms": pctl(fused_steps),
        "cold_cache": cold,
        "torch_eager_unfused": {"ms_per_step": round(torch_ms, 4),
                                "tflops": round(flops / (torch_ms * 1e-3) / 1e12, 2),
                                "speedup_fused_vs_torch": round(torch_ms / ms_step, 3),
                                "note": "context, not the baseline: median step of the same block "
                                        "in eager PyTorch (torch.mm on hipBLASLt, bf16; RMSNorm "
                                        "in fp32; SwiGLU)"},
        "unfused": {"ms_per_step": round(unf_ms_step, 4), "tflops": round(unf_tflops, 2),
                    "speedup_fused_vs_unfused": round(unf_ms_step / ms_step, 3),
                    "step_ms": pctl(unf_steps),
                    "alternating_passes": {
                        "fused_ms_per_step": [round(v / args.steps, 4) for v in fused_passes],
                        "unfused_ms_per_step": [round(v / args.steps, 4) for v in unfused_passes],
                        "speedup_of_medians": round(float(np.median(unfused_passes)) /
                                                    float(np.median(fused_passes)), 3),
                        "note": "three passes of --steps steps each, fused and unfused in "
                                "turn; the first fused pass is the headline"}},
        "warmup_floor": {"min_gpu_ms": args.warmup_ms, "gpu_ms": round(warm_ms, 1),
                         "fused_unfused_pairs_run": warm_pairs,
                         "note": "the --warmup steps, extended until the warm-up has run this "
                                 "much GPU time (fused and unfused alternating)"},
        "kernels_ms": {"gemm_residual_partialrms": round(g1_ms, 4),
                       "rms_reduce": round(red_ms, 4),
                       "gemm_rowscale_swiglu": round(g2_ms, 4)},
        "roofline": {"kernel": "gemm_rowscale_swiglu", "bound": "mfma",
                     "achieved": round(g2_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(g2_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("gemm_rowscale_swiglu"),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE, "
                                     "copy-calibrated)",
                     "clock_ghz_measured": clock,
                     "frac_at_measured_clock":
                         None if clock is None else round(g2_tflops / (PEAK_BF16_TFLOPS * clock / 2.4), 4)},
        "cpu_baseline": cpu,
        "other_rows": rows,
    }
    print(json.dumps(line), flush=True)


PEAK_FP8_TFLOPS = 5033.2  # MI355X dense OCP fp8 MFMA, 2.4 GHz


def pctl(ms):
    """Median, 10th and 90th percentile of per-step times (ms)."""
    ms = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(ms)), 4), "p10": round(float(np.percentile(ms, 10)), 4),
            "p90": round(float(np.percentile(ms, 90)), 4)}


def step_times(torch, stream, fn, steps):
    """Per-step times (ms) from events recorded before and after every step
    (no synchronisation between steps)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def step_times_cold(torch, stream, fn, steps, scratch):
    """Per-step times (ms) with `scratch` overwritten before every step (not
    timed), so the step starts with its operands evicted from the caches."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for k, (e0, e1) in enumerate(evs):
        scratch.fill_(float(k))
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def splitk_parts(M, N, K, cus):
    """Reduction parts for an M x N output over K: doubled while the
    256 x 256 tiles times the parts stay below the compute-unit count."""
    tiles = -(-M // 256) * -(-N // 256)
    p = 1
    while tiles * p < cus and p < 16 and K % (128 * p) == 0:
        p *= 2
    return p


def _events_time(torch, stream, fn, steps, warmup, min_ms=None):
    """Mean step time (ms) over back-to-back steps.  Warmup and timed region
    each cover at least `min_ms` of GPU work (the shader clock settles over
    tens of milliseconds under sustained MFMA load), so short steps are
    repeated more often than `steps`/`warmup`."""
    if min_ms is None:
        min_ms = _ROW_MIN_MS
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    est = max(e0.elapsed_time(e1), 1e-3)
    reps = int(min(2000, max(1, np.ceil(min_ms / est))))
    steps, warmup = max(steps, reps), max(warmup, reps)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _mlp_bwd_row(torch, ops, inputs, stream, steps, warmup, bf, name="mlp_1b_bwd", **sizes):
    """Backward of the MLP sub-layer given dY: fused (SwiGLU-backward GEMM ->
    row-coefficient reduce -> RMSNorm-backward GEMM -> dx GEMM) against the
    unfused sequence (plain GEMMs with a SwiGLU-backward pass and an
    RMSNorm-backward pass between them), and the forward that saves z plus
    the backward against the unfused forward plus backward."""
    dev = "cuda:0"
    eps = 1e-5
    print(f"[bench] {name}", file=sys.stderr, flush=True)
    w = inputs.make_workload(name, **sizes)
    M, d, K1, ffn = (w.sizes[k] for k in ("M", "d", "K1", "ffn"))
    x, res, wo, wd, dy = (bf(w.arrays[k]) for k in ("x", "res", "w1", "wd", "dy"))
    # gate and up weights live in one [2 ffn, d] buffer (the unfused gate|up GEMM
    # reads it whole, the fused path its two halves)
    wgu = torch.cat([bf(w.arrays["wg"]), bf(w.arrays["wu"])], 0).contiguous()
    wg, wu = wgu[:ffn], wgu[ffn:]
    gamma = torch.from_numpy(w.arrays["gamma"]).to(dev)
    del w
    bf16 = dict(dtype=torch.bfloat16, device=dev)
    # weight preparation: gamma folded, transposed copies for the backward
    # GEMMs.  Weights change every training step, so the training-step timings
    # below include it (both sequences need the same copies); the backward and
    # weight-gradient timings alone do not.
    wg_f, wu_f = torch.empty_like(wg), torch.empty_like(wu)
    WdT, W2T, WoT = (torch.empty(ffn, d, **bf16), torch.empty(d, 2 * ffn, **bf16),
                     torch.empty(K1, d, **bf16))

    def prep():
        ops.fold_gamma(wg, gamma, wg_f)
        ops.fold_gamma(wu, gamma, wu_f)
        ops.transpose(wd, WdT)
        ops.transpose(wg_f, W2T[:, :ffn])
        ops.transpose(wu_f, W2T[:, ffn:])
        ops.transpose(wo, WoT)
    prep()
    h = torch.empty(M, d, **bf16)
    P = torch.empty(ops.rms_tiles(d), M, dtype=torch.float32, device=dev)
    r = torch.empty(M, dtype=torch.float32, device=dev)
    o = torch.empty(M, ffn, **bf16)
    gu = torch.empty(M, 2 * ffn, **bf16)
    dz = torch.empty(M, 2 * ffn, **bf16)
    pdot = torch.empty(ops.rms_tiles(ffn), M, dtype=torch.float32, device=dev)
    c = torch.empty(M, dtype=torch.float32, device=dev)
    dh = torch.empty(M, d, **bf16)
    dx = torch.empty(M, K1, **bf16)

    def fwd_save():
        ops.gemm_residual_partialrms(x, wo, res, h, P)
        ops.rms_reduce(P, d, eps, r)
        ops.gemm_rowscale_swiglu_save(h, wg_f, wu_f, r, o, gu)
    bwd_k = [lambda: ops.gemm_swiglu_bwd(dy, WdT, gu, dz, pdot),
             lambda: ops.rms_bwd_reduce(pdot, d, r, c),
             lambda: ops.gemm_rmsnorm_bwd(dz, W2T, h, dy, r, c, dh),
             lambda: ops.gemm_bf16(dh, WoT, dx)]

    def bwd():
        for f in bwd_k:
            f()

    # weight gradients: token-major copies (the row scale r applied while
    # copying h), then plain GEMMs reducing over the tokens
    x_T, h_T, dy_T, dh_T = (torch.empty(n, M, **bf16) for n in (K1, d, d, d))
    dz_T, o_T = torch.empty(2 * ffn, M, **bf16), torch.empty(ffn, M, **bf16)
    dW2, dWd, dWo = (torch.empty(2 * ffn, d, **bf16), torch.empty(d, ffn, **bf16),
                     torch.empty(d, K1, **bf16))
    # dWo (d x K1) has too few output tiles for the chip: split its reduction
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    parts_o = splitk_parts(d, K1, M, cus)
    ws_o = torch.empty(parts_o, d, K1, dtype=torch.float32, device=dev)

    def gemm_dwo():
        if parts_o > 1:
            ops.gemm_bf16_splitk(dh_T, x_T, dWo, ws_o)
        else:
            ops.gemm_bf16(dh_T, x_T, dWo)

    # gradient of the RMSNorm gain: partial sums over 128-row slices of the
    # gate|up weight gradient, then the light reduce
    pdg = torch.empty(ops.dgamma_slices(2 * ffn), d, dtype=torch.float32, device=dev)
    dgamma = torch.empty(d, dtype=torch.float32, device=dev)

    def dw():
        ops.transpose(h, h_T, row_scale=r)
        ops.transpose(dz, dz_T)
        ops.transpose(dy, dy_T)
        ops.transpose(o, o_T)
        ops.transpose(dh, dh_T)
        ops.transpose(x, x_T)
        # dW = dW' diag(gamma) (unfolded gate|up) and the dgamma partials in its epilogue
        ops.gemm_wgrad_gamma(dz_T, h_T, wgu, gamma, dW2, pdg)
        ops.dgamma_reduce(pdg, dgamma)
        ops.gemm_bf16(dy_T, o_T, dWd)
        gemm_dwo()

    def train():
        prep()
        fwd_save()
        bwd()
        dw()
    fwd_save()
    ms_b = _events_time(torch, stream, bwd, steps, warmup)
    kb = _kernel_times(torch, stream, bwd_k, steps)
    ms_w = _events_time(torch, stream, dw, steps, warmup)
    ms_p = _events_time(torch, stream, prep, steps, warmup)
    ms_t = _events_time(torch, stream, train, steps, warmup)
    # unfused: forward stores g|u from one plain GEMM (the backward reads it)
    y_u, h_u, n_u, G_u, dh_u = (torch.empty(M, d, **bf16) for _ in range(5))
    gu_u, dz_u = torch.empty(M, 2 * ffn, **bf16), torch.empty(M, 2 * ffn, **bf16)
    o_u, dout_u = torch.empty(M, ffn, **bf16), torch.empty(M, ffn, **bf16)
    dx_u = torch.empty(M, K1, **bf16)

    def fwd_u():
        ops.gemm_bf16(x, wo, y_u)
        ops.residual_add(y_u, res, h_u)
        ops.rmsnorm(h_u, gamma, eps, n_u)
        ops.gemm_bf16(n_u, wgu, gu_u)
        ops.swiglu(gu_u, o_u)
    bwd_uk = [lambda: ops.gemm_bf16(dy, WdT, dout_u),
              lambda: ops.swiglu_bwd(dout_u, gu_u, dz_u),
              lambda: ops.gemm_bf16(dz_u, W2T, G_u),
              lambda: ops.rmsnorm_bwd(G_u, h_u, dy, eps, dh_u),
              lambda: ops.gemm_bf16(dh_u, WoT, dx_u)]

    def bwd_u():
        for f in bwd_uk:
            f()

    n_T = torch.empty(d, M, **bf16)

    pdg_u = torch.empty_like(pdg)

    def dw_u():  # the same GEMMs; the normalised n (with gamma) is stored here
        ops.transpose(n_u, n_T)
        ops.transpose(dz_u, dz_T)
        ops.transpose(dy, dy_T)
        ops.transpose(o_u, o_T)
        ops.transpose(dh_u, dh_T)
        ops.transpose(x, x_T)
        ops.gemm_bf16(dz_T, n_T, dW2)  # the unfolded gate|up gradient directly
        # dgamma = sum_n dW * W / gamma: a column-dot pass over the stored gradient
        ops.col_dot_partial(dW2, wgu, pdg_u)
        ops.dgamma_reduce(pdg_u, dgamma, gamma_div=gamma)
        ops.gemm_bf16(dy_T, o_T, dWd)
        gemm_dwo()

    def train_u():
        prep()
        fwd_u()
        bwd_u()
        dw_u()
    fwd_u()
    ms_bu = _events_time(torch, stream, bwd_u, steps, warmup)
    kbu = _kernel_times(torch, stream, bwd_uk, steps)
    ms_wu = _events_time(torch, stream, dw_u, steps, warmup)
    ms_tu = _events_time(torch, stream, train_u, steps, warmup)
    # context only: the same backward chain in eager PyTorch (torch.mm on hipBLASLt with
    # contiguous operands; the SwiGLU gradient on bf16 tensors as autograd would run it, the
    # RMSNorm gradient in fp32), from the unfused forward's g|u
    w2 = torch.cat([wg_f, wu_f], 0).contiguous()  # W' = [Wg; Wu] diag(gamma), [2 ffn, d]

    def bwd_torch():
        dout = torch.mm(dy, wd)
        g, u = gu_u[:, :ffn], gu_u[:, ffn:]
        sg = torch.sigmoid(g)
        sl = g * sg
        dzt = torch.cat([dout * u * (sg + sl * (1 - sg)), dout * sl], 1)
        G = torch.mm(dzt, w2).float()
        h32 = h_u.float()
        rr = torch.rsqrt(h32.pow(2).mean(-1, keepdim=True) + eps)
        dhh = rr * G - (rr.pow(3) / d) * (h32 * G).sum(-1, keepdim=True) * h32 + dy.float()
        return torch.mm(dhh.to(torch.bfloat16), wo)
    ms_bt = _events_time(torch, stream, bwd_torch, steps, warmup)
    del w2
    fl_b = 2.0 * M * ffn * d + 2.0 * M * d * 2 * ffn + 2.0 * M * K1 * d
    fl_w = 2.0 * M * 2 * ffn * d + 2.0 * M * d * ffn + 2.0 * M * d * K1
    fl_t = fl_b + fl_w + 2.0 * M * d * K1 + 2.0 * M * 2 * ffn * d
    return {"workload": f"M={M}, d={d}, K1={K1}, ffn={ffn}: backward of the MLP sub-layer "
                        "given dY (dx and dres), its weight gradients, and the training step "
                        "(weight preparation, forward saving g|u, backward, weight gradients)",
            "bwd_ms": round(ms_b, 4), "bwd_tflops": round(fl_b / ms_b / 1e9, 1),
            "bwd_pct_of_bf16_peak": round(100 * fl_b / ms_b / 1e9 / PEAK_BF16_TFLOPS, 2),
            "bwd_kernels_ms": dict(zip(("gemm_swiglu_bwd", "rms_bwd_reduce", "gemm_rmsnorm_bwd",
                                        "gemm_bf16_dx"), kb)),
            "dw_ms": round(ms_w, 4), "dwo_reduction_parts": parts_o, "dw_tflops": round(fl_w / ms_w / 1e9, 1),
            "dw_note": "weight gradients of the unfolded weights (dWg|dWu = dW' diag(gamma) from "
                       "the GEMM epilogue), dWd, dWo and dgamma (partial sums in the same "
                       "epilogue + light reduce); the unfused sequence gives the same gradients",
            "weight_prep_ms": round(ms_p, 4),
            "train_step_ms": round(ms_t, 4), "train_step_tflops": round(fl_t / ms_t / 1e9, 1),
            "unfused": {"bwd_ms": round(ms_bu, 4), "bwd_tflops": round(fl_b / ms_bu / 1e9, 1),
                        "bwd_speedup_fused_vs_unfused": round(ms_bu / ms_b, 3),
                        "bwd_kernels_ms": dict(zip(("gemm_bf16_dout", "swiglu_bwd",
                                                    "gemm_bf16_G", "rmsnorm_bwd",
                                                    "gemm_bf16_dx"), kbu)),
                        "dw_ms": round(ms_wu, 4),
                        "train_step_ms": round(ms_tu, 4),
                        "train_step_speedup_fused_vs_unfused": round(ms_tu / ms_t, 3)},
            "torch_eager_bwd": {"bwd_ms": round(ms_bt, 4),
                                "bwd_speedup_fused_vs_torch": round(ms_bt / ms_b, 3),
                                "note": "context, not the baseline: the same backward chain in "
                                        "eager PyTorch (torch.mm on hipBLASLt; SwiGLU gradient "
                                        "on bf16 tensors, RMSNorm gradient in fp32)"}}


def _kernel_times(torch, stream, fns, steps):
    """Mean duration (ms) of each launch in `fns`, from events recorded on the
    launch stream between consecutive launches over `steps` passes."""
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
           for _ in range(steps)]
    torch.cuda.synchronize()
    for e in evs:
        e[0].record(stream)
        for i, f in enumerate(fns):
            f()
            e[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(len(fns))] for e in evs])
    return [round(float(v), 4) for v in per.mean(axis=0)]


def time_other_rows(torch, ops, inputs, stream, steps, warmup):
    """Fused-path step time of the other hot-path workloads (same timing
    policy: inputs resident in HBM, one stream, HIP events)."""
    dev = "cuda:0"
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
        torch.bfloat16).to(dev)
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    out = {}
    eps = 1e-5

    # attention-input block: GEMM1 (K=8192) -> reduce -> QKV GEMM + RoPE
    print("[bench] attn_rope", file=sys.stderr, flush=True)
    w = inputs.make_workload("attn_rope")
    sz = w.sizes
    M, d, K1 = sz["M"], sz["d"], sz["K1"]
    nq, nkv, hd = sz["n_q"], sz["n_kv"], sz["head_dim"]
    x, res, w1, wqkv = (bf(w.arrays[k]) for k in ("x", "res", "w1", "wqkv"))
    gamma = torch.from_numpy(w.arrays["gamma"]).to(dev)
    wqkv_f = torch.empty_like(wqkv)
    ops.fold_gamma(wqkv, gamma, wqkv_f)
    cos = torch.empty(sz["seq_len"], hd // 2, dtype=torch.float32, device=dev)
    sin = torch.empty_like(cos)
    ops.rope_tables(sz["theta"], sz["seq_len"], hd, cos, sin)
    pos = torch.from_numpy(w.arrays["pos"]).to(dev)
    h = torch.empty(M, d, dtype=torch.bfloat16, device=dev)
    P = torch.empty(ops.rms_tiles(d), M, dtype=torch.float32, device=dev)
    r = torch.empty(M, dtype=torch.float32, device=dev)
    qkv = torch.empty(M, (nq + 2 * nkv) * hd, dtype=torch.bfloat16, device=dev)

    def attn_step():
        ops.gemm_residual_partialrms(x, w1, res, h, P)
        ops.rms_reduce(P, d, eps, r)
        ops.gemm_rope(h, wqkv_f, r, cos, sin, pos, qkv, nq, nkv, hd)
    ms = _events_time(torch, stream, attn_step, steps, warmup)
    # unfused: plain GEMM -> add -> RMSNorm -> plain QKV GEMM -> RoPE in place
    y_u, h_u, n_u = (torch.empty(M, d, dtype=torch.bfloat16, device=dev) for _ in range(3))
    qkv_u = torch.empty_like(qkv)

    def attn_unfused():
        ops.gemm_bf16(x, w1, y_u)
        ops.residual_add(y_u, res, h_u)
        ops.rmsnorm(h_u, gamma, eps, n_u)
        ops.gemm_bf16(n_u, wqkv, qkv_u)
        ops.rope_apply(qkv_u, cos, sin, pos, nq, nkv, hd)
    ms_u = _events_time(torch, stream, attn_unfused, steps, warmup)
    fl = 2.0 * M * d * K1 + 2.0 * M * (nq + 2 * nkv) * hd * d
    out["attn_rope"] = {"workload": "M=8192, d=2048, GEMM1 K=8192, 32 q / 8 kv heads of 64, "
                                    "RoPE theta=5e5", "ms_per_step": round(ms, 4),
                        "tflops": round(fl / ms / 1e9, 1),
                        "pct_of_bf16_peak": round(100 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
                        "unfused": {"ms_per_step": round(ms_u, 4),
                                    "tflops": round(fl / ms_u / 1e9, 1),
                                    "speedup_fused_vs_unfused": round(ms_u / ms, 3)}}
    del x, res, w1, wqkv, wqkv_f, h, P, r, qkv, w, y_u, h_u, n_u, qkv_u

    # LM head: block log-sum-exp GEMM + merge
    print("[bench] lm_head", file=sys.stderr, flush=True)
    w = inputs.make_workload("lm_head")
    M, d, V = w.sizes["M"], w.sizes["d"], w.sizes["V"]
    x, wl = bf(w.arrays["x"]), bf(w.arrays["wlm"])
    lab = torch.from_numpy(w.arrays["labels"]).to(dev)
    T = ops.lse_tiles(V)
    tmax = torch.empty(T, M, dtype=torch.float32, device=dev)
    tsum = torch.empty_like(tmax)
    zl, loss = (torch.empty(M, dtype=torch.float32, device=dev) for _ in range(2))
    ms = _events_time(torch, stream, lambda: ops.gemm_block_lse(x, wl, lab, tmax, tsum, zl, loss),
                      steps, warmup)
    # unfused: plain GEMM -> bf16 logits in HBM (2.1 GB) -> row cross entropy
    logits = torch.empty(M, V, dtype=torch.bfloat16, device=dev)
    lse_u, loss_u = (torch.empty(M, dtype=torch.float32, device=dev) for _ in range(2))

    def lm_unfused():
        ops.gemm_bf16(x, wl, logits)
        ops.cross_entropy_rows(logits, lab, lse_u, loss_u)
    ms_u = _events_time(torch, stream, lm_unfused, steps, warmup)
    fl = 2.0 * M * V * d
    out["lm_head"] = {"workload": "M=8192, d=2048, V=128256, per-row CE via block LSE",
                      "ms_per_step": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                      "pct_of_bf16_peak": round(100 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
                      "unfused": {"ms_per_step": round(ms_u, 4),
                                  "tflops": round(fl / ms_u / 1e9, 1),
                                  "speedup_fused_vs_unfused": round(ms_u / ms, 3),
                                  "max_loss_diff_vs_fused":
                                      round(float((loss_u - loss).abs().max().item()), 6)}}
    del x, wl, tmax, tsum, w, logits, lse_u, loss_u

    # one whole layer at the 1B shape: attention-input block, attention, MLP block
    for name in ("layer_1b", "layer_7b", "layer_70b"):
        out[name] = _layer_row(torch, ops, inputs, stream, steps, warmup, bf, name)

    # the bf16 MLP block at the 7B and 70B hidden sizes
    for name in ("mlp_7b", "mlp_70b"):
        out[name] = _mlp_row(torch, ops, inputs, stream, name, steps, warmup, bf)

    # backward of the 1B-shaped MLP sub-layer (and forward + backward)
    out["mlp_1b_bwd"] = _mlp_bwd_row(torch, ops, inputs, stream, steps, warmup, bf)

    # fp8 8B-shaped MLP block (delayed scaling: the previous step's scale)
    print("[bench] mlp_8b_fp8", file=sys.stderr, flush=True)
    w = inputs.make_workload("mlp_8b_fp8")
    M, d, K1, ffn = (w.sizes[k] for k in ("M", "d", "K1", "ffn"))
    x, w1, wg, wu = (u8(w.arrays[k]) for k in ("x", "w1", "wg", "wu"))
    res = bf(w.arrays["res"])
    sc = {k: torch.tensor([w.scales[k]], dtype=torch.float32, device=dev)
          for k in ("x", "w1", "wg", "wu")}
    h = torch.empty(M, d, dtype=torch.bfloat16, device=dev)
    h8 = torch.empty(M, d, dtype=torch.uint8, device=dev)
    T = ops.rms_tiles(d)
    P, PA = (torch.empty(T, M, dtype=torch.float32, device=dev) for _ in range(2))
    r = torch.empty(M, dtype=torch.float32, device=dev)
    amax = torch.empty(1, dtype=torch.float32, device=dev)
    scales = [torch.ones(1, dtype=torch.float32, device=dev) for _ in range(2)]
    o = torch.empty(M, ffn, dtype=torch.bfloat16, device=dev)
    flip = [0]

    def fp8_step():
        s_in, s_out = scales[flip[0]], scales[1 - flip[0]]
        ops.gemm_residual_partialrms(x, w1, res, h, P, a_scale=sc["x"], w_scale=sc["w1"],
                                     h8_scale=s_in, h8=h8, partial_amax=PA)
        ops.rms_reduce(P, d, eps, r, partial_amax=PA, h_amax=amax, h8_scale_out=s_out)
        ops.gemm_rowscale_swiglu(h8, wg, wu, r, o, x_scale=s_in, wg_scale=sc["wg"],
                                 wu_scale=sc["wu"])
        flip[0] = 1 - flip[0]
    ms = _events_time(torch, stream, fp8_step, steps, warmup)
    # unfused: fp8 GEMM -> bf16 y; add; RMSNorm (gain folded into the weights);
    # quantise to e4m3 (delayed scale); two fp8 GEMMs into g|u; SwiGLU
    y_u, h_u, n_u = (torch.empty(M, d, dtype=torch.bfloat16, device=dev) for _ in range(3))
    n8 = torch.empty(M, d, dtype=torch.uint8, device=dev)
    gu = torch.empty(M, 2 * ffn, dtype=torch.bfloat16, device=dev)
    o_u = torch.empty(M, ffn, dtype=torch.bfloat16, device=dev)
    ones_d = torch.ones(d, dtype=torch.float32, device=dev)
    amax_u = torch.empty(1, dtype=torch.float32, device=dev)
    scales_u = [torch.ones(1, dtype=torch.float32, device=dev) for _ in range(2)]
    flip_u = [0]

    def fp8_unfused():
        s_in, s_out = scales_u[flip_u[0]], scales_u[1 - flip_u[0]]
        ops.gemm_fp8(x, w1, sc["x"], sc["w1"], y_u)
        ops.residual_add(y_u, res, h_u)
        ops.rmsnorm(h_u, ones_d, eps, n_u)
        ops.quantize_e4m3(n_u, s_in, n8, amax_u, s_out)
        ops.gemm_fp8(n8, wg, s_in, sc["wg"], gu[:, :ffn])
        ops.gemm_fp8(n8, wu, s_in, sc["wu"], gu[:, ffn:])
        ops.swiglu(gu, o_u)
        flip_u[0] = 1 - flip_u[0]
    ms_u = _events_time(torch, stream, fp8_unfused, steps, warmup)
    fl = 2.0 * M * d * K1 + 2.0 * M * 2 * ffn * d
    out["mlp_8b_fp8"] = {"workload": "M=16384, d=4096, ffn=14336, e4m3 operands, "
                                     "delayed per-tensor scale of h",
                         "ms_per_step": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
                         "pct_of_fp8_peak": round(100 * fl / ms / 1e9 / PEAK_FP8_TFLOPS, 2),
                         "unfused": {"ms_per_step": round(ms_u, 4),
                                     "tflops": round(fl / ms_u / 1e9, 1),
                                     "speedup_fused_vs_unfused": round(ms_u / ms, 3)}}
    return out


def attention_flops(M, L, nq, hd):
    """Algorithmic FLOPs of causal attention: q.k and p.v, 2 hd each, for every
    (query, visible key) pair, L (L + 1) / 2 pairs per sequence and head."""
    return 4.0 * hd * nq * (M // L) * L * (L + 1) / 2


def _layer_row(torch, ops, inputs, stream, steps, warmup, bf, name="layer_1b"):
    """Forward of one transformer layer (layer_1b: M=8192 as 4 sequences of
    2048, d=2048, previous-MLP width 8192, ffn=8192, 32 q / 8 kv heads of 64;
    layer_7b and layer_70b: the 7B and 70B hidden sizes with heads of 128):
    the fused chain of seven launches against the unfused sequence with the
    same attention kernel, plus per-launch times of the fused chain."""
    print(f"[bench] {name}", file=sys.stderr, flush=True)
    dev = "cuda:0"
    eps = 1e-5
    w = inputs.make_workload(name)
    sz = w.sizes
    M, d, K1, ffn = sz["M"], sz["d"], sz["K1"], sz["ffn"]
    nq, nkv, hd, L = sz["n_q"], sz["n_kv"], sz["head_dim"], sz["seq_len"]
    x, res, wdn, wqkv, wo, wg, wu = (bf(w.arrays[k])
                                     for k in ("x", "res", "w1", "wqkv", "wo", "wg", "wu"))
    g1, g2 = (torch.from_numpy(w.arrays[k]).to(dev) for k in ("gamma", "gamma2"))
    wqkv_f, wg_f, wu_f = torch.empty_like(wqkv), torch.empty_like(wg), torch.empty_like(wu)
    ops.fold_gamma(wqkv, g1, wqkv_f)
    ops.fold_gamma(wg, g2, wg_f)
    ops.fold_gamma(wu, g2, wu_f)
    cos = torch.empty(L, hd // 2, dtype=torch.float32, device=dev)
    sin = torch.empty_like(cos)
    ops.rope_tables(sz["theta"], L, hd, cos, sin)
    pos = torch.from_numpy(w.arrays["pos"]).to(dev)
    e = dict(dtype=torch.bfloat16, device=dev)
    h1, h2 = torch.empty(M, d, **e), torch.empty(M, d, **e)
    T = ops.rms_tiles(d)
    P1, P2 = (torch.empty(T, M, dtype=torch.float32, device=dev) for _ in range(2))
    r1, r2 = (torch.empty(M, dtype=torch.float32, device=dev) for _ in range(2))
    qkv = torch.empty(M, (nq + 2 * nkv) * hd, **e)
    o = torch.empty(M, nq * hd, **e)
    act = torch.empty(M, ffn, **e)
    fused = [lambda: ops.gemm_residual_partialrms(x, wdn, res, h1, P1),
             lambda: ops.rms_reduce(P1, d, eps, r1),
             lambda: ops.gemm_rope(h1, wqkv_f, r1, cos, sin, pos, qkv, nq, nkv, hd),
             lambda: ops.attention_fwd(qkv, o, L, nq, nkv, hd),
             lambda: ops.gemm_residual_partialrms(o, wo, h1, h2, P2),
             lambda: ops.rms_reduce(P2, d, eps, r2),
             lambda: ops.gemm_rowscale_swiglu(h2, wg_f, wu_f, r2, act)]
    names = ["gemm1_down_residual_partialrms", "rms_reduce", "qkv_rope", "attention",
             "gemm1_o_residual_partialrms", "rms_reduce", "gemm2_rowscale_swiglu"]

    def layer():
        for f in fused:
            f()
    ms = _events_time(torch, stream, layer, steps, warmup)
    per = _kernel_times(torch, stream, fused, steps)
    # unfused: every GEMM plain, residual add, RMSNorm, RoPE in place and
    # SwiGLU as their own launches; the same attention kernel
    y, hu1, nu, hu2 = (torch.empty(M, d, **e) for _ in range(4))
    qkv_u, o_u = torch.empty_like(qkv), torch.empty_like(o)
    gu = torch.empty(M, 2 * ffn, **e)
    wgu = torch.cat([wg, wu], 0)  # gate rows then up rows: one GEMM writes g | u
    act_u = torch.empty_like(act)

    def layer_u():
        ops.gemm_bf16(x, wdn, y)
        ops.residual_add(y, res, hu1)
        ops.rmsnorm(hu1, g1, eps, nu)
        ops.gemm_bf16(nu, wqkv, qkv_u)
        ops.rope_apply(qkv_u, cos, sin, pos, nq, nkv, hd)
        ops.attention_fwd(qkv_u, o_u, L, nq, nkv, hd)
        ops.gemm_bf16(o_u, wo, y)
        ops.residual_add(y, hu1, hu2)
        ops.rmsnorm(hu2, g2, eps, nu)
        ops.gemm_bf16(nu, wgu, gu)
        ops.swiglu(gu, act_u)
    ms_u = _events_time(torch, stream, layer_u, steps, warmup)
    fl_att = attention_flops(M, L, nq, hd)
    fl = (2.0 * M * d * K1 + 2.0 * M * (nq + 2 * nkv) * hd * d + fl_att
          + 2.0 * M * d * nq * hd + 2.0 * M * 2 * ffn * d)
    att_ms = per[3]
    return {"workload": f"M={M} ({M // L} sequences of {L}), d={d}, previous-MLP width {K1}, "
                        f"ffn={ffn}, {nq} q / {nkv} kv heads of {hd}, causal attention, "
                        f"RoPE theta={sz['theta']:g}",
            "ms_per_step": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
            "pct_of_bf16_peak": round(100 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
            "flops_note": "GEMM FLOPs 2MNK each; attention 4 hd per causal (query, key) pair",
            "kernels_ms": dict(zip([f"{i}_{n}" for i, n in enumerate(names)], per)),
            "attention": {"ms": att_ms, "gflop": round(fl_att / 1e9, 2),
                          "tflops": round(fl_att / att_ms / 1e9, 1),
                          "pct_of_bf16_peak": round(100 * fl_att / att_ms / 1e9
                                                    / PEAK_BF16_TFLOPS, 2)},
            "unfused": {"ms_per_step": round(ms_u, 4), "tflops": round(fl / ms_u / 1e9, 1),
                        "speedup_fused_vs_unfused": round(ms_u / ms, 3)}}


def _mlp_row(torch, ops, inputs, stream, name, steps, warmup, bf, **sizes):
    """Fused and unfused step time of a bf16 MLP workload (same kernels and
    timing policy as the headline line, inputs resident in HBM)."""
    dev = "cuda:0"
    eps = 1e-5
    print(f"[bench] {name}", file=sys.stderr, flush=True)
    w = inputs.make_workload(name, **sizes)
    M, d, K1, ffn = (w.sizes[k] for k in ("M", "d", "K1", "ffn"))
    x, res, w1, wg, wu = (bf(w.arrays[k]) for k in ("x", "res", "w1", "wg", "wu"))
    gamma = torch.from_numpy(w.arrays["gamma"]).to(dev)
    del w
    wg_f, wu_f = torch.empty_like(wg), torch.empty_like(wu)
    ops.fold_gamma(wg, gamma, wg_f)
    ops.fold_gamma(wu, gamma, wu_f)
    h = torch.empty(M, d, dtype=torch.bfloat16, device=dev)
    P = torch.empty(ops.rms_tiles(d), M, dtype=torch.float32, device=dev)
    r = torch.empty(M, dtype=torch.float32, device=dev)
    o = torch.empty(M, ffn, dtype=torch.bfloat16, device=dev)

    fused_k = [lambda: ops.gemm_residual_partialrms(x, w1, res, h, P),
               lambda: ops.rms_reduce(P, d, eps, r),
               lambda: ops.gemm_rowscale_swiglu(h, wg_f, wu_f, r, o)]

    def fused():
        for f in fused_k:
            f()
    ms = _events_time(torch, stream, fused, steps, warmup)
    k_ms = _kernel_times(torch, stream, fused_k, steps)
    del wg_f, wu_f
    wgu = torch.cat([wg, wu], 0).contiguous()
    del wg, wu
    y_u, h_u, n_u = (torch.empty(M, d, dtype=torch.bfloat16, device=dev) for _ in range(3))
    gu = torch.empty(M, 2 * ffn, dtype=torch.bfloat16, device=dev)
    o_u = torch.empty(M, ffn, dtype=torch.bfloat16, device=dev)

    unfused_k = [lambda: ops.gemm_bf16(x, w1, y_u),
                 lambda: ops.residual_add(y_u, res, h_u),
                 lambda: ops.rmsnorm(h_u, gamma, eps, n_u),
                 lambda: ops.gemm_bf16(n_u, wgu, gu),
                 lambda: ops.swiglu(gu, o_u)]

    def unfused():
        for f in unfused_k:
            f()
    ms_u = _events_time(torch, stream, unfused, steps, warmup)
    ku_ms = _kernel_times(torch, stream, unfused_k, steps)
    fl = 2.0 * M * d * K1 + 2.0 * M * 2 * ffn * d
    return {"workload": f"M={M}, d={d}, K1={K1}, ffn={ffn}, gate/up with SwiGLU, eps=1e-5",
            "ms_per_step": round(ms, 4), "tflops": round(fl / ms / 1e9, 1),
            "pct_of_bf16_peak": round(100 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
            "kernels_ms": dict(zip(("gemm_residual_partialrms", "rms_reduce",
                                    "gemm_rowscale_swiglu"), k_ms)),
            "unfused": {"ms_per_step": round(ms_u, 4), "tflops": round(fl / ms_u / 1e9, 1),
                        "speedup_fused_vs_unfused": round(ms_u / ms, 3),
                        "kernels_ms": dict(zip(("gemm_bf16", "residual_add", "rmsnorm",
                                                "gemm_bf16_gate_up", "swiglu"), ku_ms))}}


# the sources the bf16 GEMM kernels are compiled from
KERNEL_SOURCES = ("coda_device.hpp", "gemm_core.hpp", "gemm_bf16.hip")


def kernel_sources_sha256():
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        h.update(name.encode())
        with open(os.path.join(root, "gemm_epilogue_transformer_gemm1_amd", "csrc", name),
                  "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_clock_ghz(kernel):
    """Average shader clock during `kernel` from the committed rocprofv3 counter
    summary, or None when the kernel's sources changed since it was taken."""
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(root, "profiles", "clock.json")) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if kernel_sources_sha256() != rec.get("sources_sha256"):
        return None
    return float(rec["clock_ghz"])


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when the kernel's sources changed since it was taken."""
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(root, "profiles", "traffic.json")) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if kernel_sources_sha256() != rec.get("sources_sha256"):
        return None
    return int(rec["fetch_bytes"] + rec["write_bytes"])


def cpu_baseline(w, eps, budget_s):
    """The CPU oracle (fp64, unfused) on a bounded row sample of the same
    workload; TFLOP/s of the same algorithmic FLOP count."""
    import oracle
    from oracle import codecs
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        threads = None
    M, d, K1, ffn = (w.sizes[k] for k in ("M", "d", "K1", "ffn"))
    W1 = codecs.bf16_decode(w.arrays["w1"])
    Wg = codecs.bf16_decode(w.arrays["wg"])
    Wu = codecs.bf16_decode(w.arrays["wu"])
    g = w.arrays["gamma"].astype(np.float64)
    # row chunks of the workload, in order, wrapping around, until the time
    # budget is spent (at least one chunk)
    rows = 512
    elapsed, done = 0.0, 0
    while True:
        m0 = done % M
        m1 = min(M, m0 + rows)
        x = codecs.bf16_decode(w.arrays["x"][m0:m1])
        res = codecs.bf16_decode(w.arrays["res"][m0:m1])
        t0 = time.perf_counter()
        oracle.mlp_block(x, res, W1, Wg, Wu, g, eps)
        elapsed += time.perf_counter() - t0
        done += m1 - m0
        if elapsed >= budget_s:
            break
    flops = 2.0 * done * (d * K1 + 2 * ffn * d)
    cpu_model, blas = None, None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                             None)
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        b = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if b:
            blas = f"{b[0].get('internal_api')} {b[0].get('version')}"
    except Exception:  # pragma: no cover
        pass
    return {"value": round(flops / elapsed / 1e12, 5), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model, "blas": blas,
            "sample": f"{done} token rows of mlp_1b ({done / M:.2f} passes over its {M} rows, "
                      f"chunks of 512; fp64 numpy, unfused) in {elapsed:.1f} s; "
                      f"host cores visible {len(os.sched_getaffinity(0))}"}


if __name__ == "__main__":
    main()
