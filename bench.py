"""Benchmark: fused linear cross-entropy forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one full pass of the hot path over one batch: flce_forward
(logit tiles with online log-sum-exp, split combine, reduction) followed by
flce_backward (recompute, grad_hidden, grad_weight) on the head-vocabulary
workload N=4096 tokens, H=4096, V=128256, bf16, mean reduction, Zipf(1.1)
targets with 5% ignored rows.  Inputs are synthetic (seeded), generated on
the GPU and resident in HBM before the timed region; outputs and workspaces
are allocated once and reused.  Without --warmup the untimed warmup runs at
least 3 steps and at least 0.5 s (the JSON line gives the count), since a
sub-millisecond step otherwise starts at an idle clock.

Prints one JSON line: throughput as TFLOP/s counting 8*N*H*V flops per step,
the fraction of the dense bf16 MFMA peak, peak device memory above the
inputs, a roofline entry for the forward logit-tile kernel, and the fp64
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd+bwd TFLOP/s (8*N*H*V) and MFMA util at N=4096,H=4096,V=128256 bf16"
PEAK_BF16_TFLOPS = 2516.6          # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_TFLOPS = {"bf16": PEAK_BF16_TFLOPS, "f16": PEAK_BF16_TFLOPS, "f32": 157.3}  # dense MFMA per dtype
PEAK_HBM_GBS = 8000.0
# The sources that decide what a launch reads and writes: the kernels, their
# device headers (tile order, record layouts) and the host planner (splits,
# chunks, grids).
KERNEL_SOURCES = ["linear_cross_entropy_fwd_amd/csrc/flce_kernels.hip",
                  "linear_cross_entropy_fwd_amd/csrc/flce_small.hip",
                  "linear_cross_entropy_fwd_amd/csrc/flce_device.h",
                  "linear_cross_entropy_fwd_amd/csrc/flce_plan.h",
                  "linear_cross_entropy_fwd_amd/csrc/flce_api.cpp"]


def code_text(src: str) -> str:
    """C/C++ source with its comments removed and every run of white space made one
    blank: a change to a comment or to the layout does not change the code."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":  # string or character literal, copied whole
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the code (comments and layout excluded) of the sources a launch depends on."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_file(kernel: str, workload_key: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload_key}_traffic.json")


def kernel_template(dtype: str, metrics: bool, bias: bool, cap: bool) -> str:
    """The forward tile kernel's template instance a run launches."""
    return f"{dtype}, metrics={int(metrics)}, bias={int(bias)}, softcap={int(cap)}"


def stored_traffic(kernel: str, workload_key: str, template: str, variants: bool):
    """HBM bytes per launch of `kernel` (fwd_tiles, bwd_step) from the
    committed counter runs of this workload and kernel template, or None:
    when no such record exists, when the run has options the record was not
    taken with, or when the kernel sources changed since the counters were
    read."""
    if variants:
        return None
    try:
        with open(traffic_file(kernel, workload_key)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if (rec.get("workload_key") != workload_key or rec.get("template") != template
            or rec.get("kernel_source_hash") != kernel_source_hash()):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_info():
    """CPU model name, physical cores and logical CPUs this process may use."""
    model, cores = None, set()
    try:
        phys = None
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model is None:
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    cores.add((phys, v))
    except OSError:
        pass
    return model, (len(cores) or None), len(os.sched_getaffinity(0))


def argmax_targets_gpu(w, d):
    """Rows chosen for argmax targets get their row's first-index argmax of
    the final logits, computed on the GPU with torch in fp32 blocks (inputs
    of the timed run only; the parity tests take the oracle's ids)."""
    import torch
    rows = d["argmax_rows"]
    if not bool(rows.any()):
        return d["targets"]
    wt = d["weight"].float()
    b = None if d["bias"] is None else d["bias"].float()
    ids = torch.empty(w.n, dtype=torch.int64, device=d["targets"].device)
    for r0 in range(0, w.n, 1024):
        z = d["hidden"][r0:r0 + 1024].float() @ wt.T
        if b is not None:
            z += b
        z *= w.logit_scale
        if w.softcap is not None:
            z = w.softcap * torch.tanh(z / w.softcap)
        ids[r0:r0 + 1024] = torch.argmax(z, dim=1)
        del z
    del wt
    return torch.where(rows, ids, d["targets"])


def cpu_baseline(d, w, rows: int):
    """fp64 oracle (as it stands) on the first `rows` rows of the same inputs
    (all of them when rows >= N); "cores" is the BLAS threads it ran with."""
    import numpy as np
    import threadpoolctl
    from oracle import flce_reference

    h = d["hidden"][:rows].float().cpu().numpy()
    t = d["targets"][:rows].cpu().numpy()
    wt = d["weight"].float().cpu().numpy()
    np.dot(np.ones((2, 2)), np.ones((2, 2)))   # load BLAS so its thread pool is visible
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [1])
    t0 = time.perf_counter()
    flce_reference(h, wt, t, None, ignore_index=w.ignore_index, logit_scale=w.logit_scale,
                   softcap=w.softcap, reduction=w.reduction)
    dt = time.perf_counter() - t0
    flops = 8.0 * rows * w.h * w.v
    model, phys, logical = cpu_info()
    what = (f"the whole workload ({rows} rows)" if rows >= w.n else f"first {rows} of {w.n} rows") + \
        f", H={w.h}, V={w.v}, fwd+bwd in fp64 with numpy BLAS, {dt:.2f} s wall, 8*rows*H*V flops"
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "sample": what, "cpu_model": model, "physical_cores": phys,
            "logical_cpus_available": logical, "wall_s": round(dt, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: at least 3 and at least 0.5 s of them, so that "
                         "short steps are timed at the clock a running job holds)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="rows of the workload the CPU oracle baseline runs (the whole head-shape "
                         "workload by default, about 20 s on 16 threads)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="run one device-to-device copy of this size first (HBM counter calibration)")
    ap.add_argument("--workload", default="headvocab_bf16")
    ap.add_argument("--phase", choices=["both", "fwd"], default="both",
                    help="'fwd' runs forward passes only (for per-kernel counter runs); "
                         "the headline line is 'both'")
    ap.add_argument("--reduction", choices=["mean", "sum", "none"], default=None,
                    help="override the workload's reduction (not the headline)")
    ap.add_argument("--label-smoothing", type=float, default=0.0,
                    help="loss variant (not the headline): label smoothing eps")
    ap.add_argument("--z-loss", type=float, default=0.0, help="loss variant (not the headline): z-loss coefficient")
    ap.add_argument("--class-weights", action="store_true",
                    help="loss variant (not the headline): seeded class weights, uniform in [0.5, 1.5)")
    ap.add_argument("--dtype", choices=["bf16", "f16", "f32"], default=None,
                    help="run the workload in another dtype (not the headline)")
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MiB scrub buffer before every step, outside the step's timed window, "
                         "so that no operand is left in L2 or the last-level cache (not the headline)")
    ap.add_argument("--grad-weight-fp32", action="store_true",
                    help="write grad_weight / grad_bias in fp32 (not the headline)")
    ap.add_argument("--vocab-shards", type=int, default=1,
                    help="time one device's share of a vocabulary split into this many equal shards "
                         "(flce_forward_shard + flce_combine_shards + the shard's flce_backward; not the headline)")
    ap.add_argument("--shard", type=int, default=0, help="which shard --vocab-shards times")
    ap.add_argument("--bwd-vocab-chunk", type=int, default=0,
                    help="plan override: vocabulary ids per backward chunk (not the headline)")
    ap.add_argument("--fwd-tiles-per-split", type=int, default=0,
                    help="plan override: vocabulary tiles per forward split (not the headline)")
    args = ap.parse_args()
    variants = bool(args.label_smoothing or args.z_loss or args.class_weights or args.grad_weight_fp32
                    or args.vocab_shards > 1 or args.bwd_vocab_chunk or args.fwd_tiles_per_split)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              f"multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import flce_inputs as fi
    import linear_cross_entropy_fwd_amd as flce
    from linear_cross_entropy_fwd_amd import _abi

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = fi.WORKLOADS[args.workload]
    if args.dtype and args.dtype != w.dtype:
        w = w.resized(dtype=args.dtype, name=w.name.replace(w.dtype, args.dtype))
        variants = True
    if args.cold:
        variants = True
    if args.reduction and args.reduction != w.reduction:
        w = w.resized(reduction=args.reduction)
        variants = True
    # options beyond the workload's own (the stored counter records hold none)
    options_changed = variants
    if args.workload != "headvocab_bf16":
        variants = True
    d = fi.generate(w, device=dev)
    d["targets"] = argmax_targets_gpu(w, d)
    hidden, weight, targets, bias = d["hidden"], d["weight"], d["targets"], d["bias"]
    torch.cuda.synchronize()
    base_mem = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()

    cw = None
    if args.class_weights:
        gen = torch.Generator().manual_seed(7)
        cw = (torch.rand(w.v, generator=gen, dtype=torch.float32) + 0.5).to(dev)
    plan = dict(bwd_vocab_chunk=args.bwd_vocab_chunk, fwd_tiles_per_split=args.fwd_tiles_per_split)
    p = flce.problem_for(hidden, weight, bias, w.ignore_index, w.logit_scale, w.softcap,
                         w.reduction, w.return_metrics, label_smoothing=args.label_smoothing,
                         z_loss=args.z_loss, class_weight=cw, grad_weight_fp32=args.grad_weight_fp32, **plan)
    n_shards = args.vocab_shards
    v_eff = w.v  # the vocabulary ids one step sweeps
    shard = None
    if n_shards > 1:
        # One device's share of a vocabulary split into n_shards equal shards:
        # its forward, the combine of all shards' per-row outputs (the other
        # shards' rows of those arrays stand in for what the other devices
        # would send), and its backward with the combined lse.
        if args.class_weights or args.label_smoothing or args.z_loss or w.return_metrics:
            print("--vocab-shards takes no metrics or loss variants", file=sys.stderr)
            sys.exit(2)
        size = -(-w.v // n_shards)
        a0 = args.shard * size
        a1 = min(w.v, a0 + size)
        if not 0 <= a0 < a1:
            print(f"--shard {args.shard} of {n_shards} is empty", file=sys.stderr)
            sys.exit(2)
        v_eff = a1 - a0
        weight = weight[a0:a1]
        bias = None if bias is None else bias[a0:a1]
        p = flce.problem_for(hidden, weight, bias, w.ignore_index, w.logit_scale, w.softcap, w.reduction,
                             False, grad_weight_fp32=args.grad_weight_fp32, vocab_offset=a0, vocab_total=w.v,
                             grad_hidden_fp32=True, **plan)
        pc = _abi.make_problem(w.n, 8, w.v, _abi.BF16, w.reduction, w.ignore_index)
        shard = dict(a0=a0, a1=a1, pc=pc,
                     lse_all=torch.empty(n_shards, w.n, dtype=torch.float32, device=dev),
                     tl_all=torch.empty(n_shards, w.n, dtype=torch.float32, device=dev),
                     cws=torch.empty(_abi.flce_combine_shards_workspace_size(pc), dtype=torch.uint8, device=dev))
    fws = torch.empty(_abi.flce_forward_workspace_size(p), dtype=torch.uint8, device=dev)
    bws = torch.empty(_abi.flce_backward_workspace_size(p), dtype=torch.uint8, device=dev)
    loss = torch.empty(w.n if w.reduction == "none" else 1, dtype=torch.float32, device=dev)
    lse = torch.empty(w.n, dtype=torch.float32, device=dev)
    metrics = torch.empty(2, dtype=torch.float32, device=dev) if w.return_metrics else None
    gh = torch.empty(hidden.shape, dtype=torch.float32 if shard else hidden.dtype, device=dev)
    gdt = torch.float32 if args.grad_weight_fp32 else weight.dtype
    gw = torch.empty(weight.shape, dtype=gdt, device=dev)
    gb = torch.empty(bias.shape, dtype=gdt, device=dev) if bias is not None else None
    ptr = lambda t: 0 if t is None else t.data_ptr()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def forward():
        if shard is not None:
            k = args.shard
            _abi.check(_abi.flce_forward_shard(p, ptr(hidden), ptr(weight), ptr(targets), ptr(bias),
                                               ptr(shard["lse_all"][k]), ptr(shard["tl_all"][k]), 0, 0, 0,
                                               ptr(fws), fws.numel(), sh))
            _abi.check(_abi.flce_combine_shards(shard["pc"], n_shards, ptr(shard["lse_all"]),
                                                ptr(shard["tl_all"]), 0, 0, 0, ptr(targets), ptr(loss), ptr(lse), 0,
                                                ptr(shard["cws"]), shard["cws"].numel(), sh))
            return
        _abi.check(_abi.flce_forward(p, ptr(hidden), ptr(weight), ptr(targets), ptr(bias), ptr(loss),
                                     ptr(lse), ptr(metrics), ptr(fws), fws.numel(), sh))

    if shard is not None:
        # the other shards' per-row outputs: this shard's, as stand-ins
        # (target logits zeroed there, as a row's target lies in one shard)
        _abi.check(_abi.flce_forward_shard(p, ptr(hidden), ptr(weight), ptr(targets), ptr(bias),
                                           ptr(shard["lse_all"][args.shard]), ptr(shard["tl_all"][args.shard]),
                                           0, 0, 0, ptr(fws), fws.numel(), sh))
        for k in range(n_shards):
            if k != args.shard:
                shard["lse_all"][k].copy_(shard["lse_all"][args.shard])
                shard["tl_all"][k].zero_()
        torch.cuda.synchronize()

    def backward():
        _abi.check(_abi.flce_backward(p, ptr(hidden), ptr(weight), ptr(targets), ptr(bias), ptr(lse), 0,
                                      ptr(gh), ptr(gw), ptr(gb), ptr(bws), bws.numel(), sh))

    if args.copy_calibration_mb > 0:
        src = torch.ones(args.copy_calibration_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    run_bwd = args.phase == "both"
    if args.warmup is not None:
        for _ in range(args.warmup):
            forward()
            if run_bwd:
                backward()
        torch.cuda.synchronize()
        warmup = args.warmup
    else:
        # Sub-millisecond steps start at an idle clock that takes tens of
        # milliseconds of load to rise: warm for a time, not a step count.
        warmup, group, t_warm = 0, 1, time.perf_counter()
        while warmup < 3 or time.perf_counter() - t_warm < 0.5:
            for _ in range(group):
                forward()
                if run_bwd:
                    backward()
            torch.cuda.synchronize()
            warmup += group
            group = min(2 * group, 64)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    # 512 MiB is twice the MI355X last-level cache (256 MB) and far above the L2s.
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for i, (e0, e1, e2) in enumerate(ev):
        if scrub is not None:
            scrub.fill_(i & 0xFF)
        e0.record(stream)
        forward()
        e1.record(stream)
        if run_bwd:
            backward()
        e2.record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    step_times = sorted(e0.elapsed_time(e2) for e0, _, e2 in ev)
    total_ms = start.elapsed_time(stop) if scrub is None else sum(step_times)
    ms_step = total_ms / args.steps
    fwd_ms = sum(e0.elapsed_time(e1) for e0, e1, _ in ev) / args.steps
    bwd_ms = sum(e1.elapsed_time(e2) for _, e1, e2 in ev) / args.steps
    peak_incr = torch.cuda.max_memory_allocated() - base_mem - (scrub.numel() if scrub is not None else 0)
    if not torch.isfinite(loss).all() or (run_bwd and not torch.isfinite(gw.float().abs().max())):
        print("non-finite result", file=sys.stderr)
        sys.exit(3)

    flops = (8.0 if run_bwd else 2.0) * w.n * w.h * v_eff
    tflops = flops / (ms_step * 1e-3) / 1e12
    fwd_tflops = 2.0 * w.n * w.h * v_eff / (fwd_ms * 1e-3) / 1e12
    template = kernel_template(w.dtype, w.return_metrics, bias is not None, w.softcap is not None)
    traffic = stored_traffic("fwd_tiles", args.workload, template, options_changed or not run_bwd)
    chunk, n_chunks, _, one_launch = _abi.flce_backward_plan(p, with_launches=True)
    out = {
        "metric": (METRIC if not variants else f"fwd+bwd TFLOP/s (8*N*H*V) on {w.name}" + ", other workload or options (not the headline)")
                  if run_bwd else "forward only TFLOP/s (2*N*H*V), not the headline",
        **({"metric": f"one vocabulary shard's fwd+bwd TFLOP/s (8*N*H*V_shard) on {w.name}, shard "
                      f"{args.shard} of {n_shards} (not the headline)"} if shard is not None and run_bwd else {}),
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded counter-hash inputs generated on the GPU)",
        "config": {"workload": w.name, "n_tokens": w.n, "hidden": w.h, "vocab": w.v,
                   "reduction": w.reduction, "targets": f"{w.targets}, {w.ignore_frac:.0%} ignored",
                   "global_batch": w.n, "parallelism": "none (1 GPU)",
                   **({"parallelism": f"one of {n_shards} vocabulary shards on 1 GPU (the other shards' "
                                      f"per-row outputs are stand-ins; no collective)",
                       "vocab_shard": {"offset": shard["a0"], "ids": v_eff, "of": w.v,
                                       "shards": n_shards}} if shard is not None else {}),
                   **({"label_smoothing": args.label_smoothing, "z_loss": args.z_loss,
                       "class_weights": bool(args.class_weights),
                       "grad_weight_fp32": bool(args.grad_weight_fp32),
                       "bwd_vocab_chunk": chunk, "fwd_tiles_per_split": args.fwd_tiles_per_split or "default",
                       "cold_cache": bool(args.cold)} if variants else {})},
        "mfma_util": round(tflops / PEAK_TFLOPS[w.dtype], 4),
        "step_ms": {"p50": round(step_times[len(step_times) // 2], 4), "min": round(step_times[0], 4),
                    "max": round(step_times[-1], 4),
                    "cache": "cold (512 MiB scrub before each step)" if scrub is not None else "warm"},
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "peak_mem_incr_mb": round(peak_incr / 2**20, 1),
        "workspace_mb": round((fws.numel() + bws.numel()) / 2**20, 1),
        "outputs_mb": round(sum(t.numel() * t.element_size()
                                for t in (loss, lse, metrics, gh, gw, gb) if t is not None) / 2**20, 1),
        "n_by_v_bytes_mb": round(w.n * v_eff * 2 / 2**20, 1),
        "wall_s_timed": round(t_wall, 3),
        "roofline_forward": {"kernel": "fwd_tiles_kernel (forward logit tiles + online LSE)",
                             "bound": "mfma", "achieved": round(fwd_tflops, 3), "peak": PEAK_TFLOPS[w.dtype],
                             "unit": "TFLOP/s", "frac": round(fwd_tflops / PEAK_TFLOPS[w.dtype], 4),
                             "traffic": traffic, "template": template,
                             "flops_per_launch": 2 * w.n * w.h * v_eff,
                             "window": "HIP events around flce_forward (tile kernel + combine + reduce)"},
    }
    out["roofline"] = out["roofline_forward"]
    if run_bwd and one_launch:
        # The dominant kernel: the backward's n_chunks + 1 launches of bwd_step_kernel (each the
        # recompute of one vocabulary chunk with both contractions of the previous one) hold
        # 6*N*H*V flops per backward pass, so per launch on average 6*N*H*V / (n_chunks + 1).
        # Achieved = that over the average launch duration, i.e. 6*N*H*V over the backward's
        # HIP-event window (which also holds the 5 us prep kernel and the hidden transpose).
        launches = n_chunks + 1
        bwd_tflops = 6.0 * w.n * w.h * v_eff / (bwd_ms * 1e-3) / 1e12
        step_traffic = stored_traffic("bwd_step", args.workload, "bwd_step " + template, options_changed)
        out["roofline"] = {"kernel": "bwd_step_kernel (per vocabulary chunk: recompute + grad_weight + "
                                     "grad_hidden in one launch)",
                           "bound": "mfma", "achieved": round(bwd_tflops, 3), "peak": PEAK_TFLOPS[w.dtype],
                           "unit": "TFLOP/s", "frac": round(bwd_tflops / PEAK_TFLOPS[w.dtype], 4),
                           "traffic": step_traffic,
                           "template": "bwd_step " + template,
                           "launches_per_backward": launches, "vocab_chunk": chunk,
                           "flops_per_launch": round(6 * w.n * w.h * v_eff / launches),
                           "avg_launch_ms": round(bwd_ms / launches, 4),
                           "window": "HIP events around flce_backward (the bwd_step_kernel launches, "
                                     "prep and hidden transpose), divided by the launch count"}
    if w.dtype == "f32":
        # fp32 at small H is memory- and launch-bound, not MFMA-bound: the
        # roofline entry is HBM bandwidth over the whole step, counting the
        # algorithmic bytes (forward reads W and H; the backward reads them
        # for the recompute and again for the contractions, and writes
        # grad_weight and grad_hidden)
        wh = (v_eff * w.h + w.n * w.h) * 4
        step_bytes = (wh if not run_bwd else 4 * wh) + w.n * 8
        gbs = step_bytes / (ms_step * 1e-3) / 1e9
        out["roofline"] = {"kernel": "whole step (every launch of the forward and backward)",
                           "bound": "hbm", "achieved": round(gbs, 3), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(gbs / PEAK_HBM_GBS, 6), "traffic": None,
                           "bytes_per_step": step_bytes,
                           "window": "HIP events around each step"}
    if not args.no_cpu_baseline and shard is None:
        out["cpu_baseline"] = cpu_baseline(d, w, min(args.cpu_rows, w.n))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
