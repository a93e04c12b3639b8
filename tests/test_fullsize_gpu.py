"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (default plan).

Stored expected values (tests/golden/fullsize_<workload>.npz, written by
tests/golden/make_fullsize.py with the fp64 oracle only): every row's lse and
loss, the metrics and the targets (the peaked workload's argmax rows hold the
oracle's argmax ids), plus gradient entries at a few sampled rows and ids.

Whole tiles, computed here by the oracle (``oracle.gradient_samples``, fp64,
given the stored oracle lse): every grad_hidden row of one full 256-token
tile and of the last tile; every grad_weight row of the first vocabulary
tile, of the tiles on both sides of the first and the last backward chunk
boundary, of one tile inside the second chunk (the second of a pair where
grad_hidden runs per pair of chunks) and of the last tile; grad_bias on the
same ids.  The chunk boundaries are the library's own default plan
(flce_backward_plan).  Each output is compared element by element at the
bf16 tolerance (relative max-norm); the achieved errors are appended to
test_output/parity_margins_fullsize.txt (or to the file FLCE_PARITY_MARGINS
names).

The inputs are drawn on the GPU; the test first checks that they are
bit-identical to the CPU draw the oracle saw (hidden in full, a band of
weight rows)."""
import os

import numpy as np
import pytest
import torch

import flce_inputs as fi
from flce_testutil import TIE, TOL, log_case, maxnorm_rel, rel_err, to_np

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")
MARGINS = os.environ.get("FLCE_PARITY_MARGINS", os.path.join(ROOT, "test_output", "parity_margins_fullsize.txt"))
NAMES = ["midvocab_bf16", "headvocab_bf16", "transforms_bf16", "peaked_bf16"]
T = 256


def load(name):
    path = os.path.join(GOLDEN, f"fullsize_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (tests/golden/make_fullsize.py)")
    return dict(np.load(path))


def record(name, what, count, got, ref, tol):
    """Max-norm relative error of one output; appended to the margins file."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = maxnorm_rel(got, ref)
    absmax = float(np.max(np.abs(got - ref))) if got.size else 0.0
    line = (f"{name:16s} {what:34s} entries {count:9d}  max|diff| {absmax:.3e}  max-norm rel {err:.3e}  "
            f"tol {tol:.0e}  margin x{tol / max(err, 1e-30):.1f}")
    print("  " + line, flush=True)
    os.makedirs(os.path.dirname(MARGINS), exist_ok=True)
    with open(MARGINS, "a") as f:
        f.write(line + "\n")
    return err


def tile_ids(w, plan):
    """Token rows and vocabulary ids of the whole tiles compared at full size."""
    chunk, n_chunks, _ = plan
    rows = list(range(T, 2 * T)) + list(range((w.n - 1) // T * T, w.n))
    last_b = (n_chunks - 1) * chunk
    starts = {0, chunk - T, chunk, last_b - T, last_b, (w.v - 1) // T * T}
    if n_chunks > 1:
        starts.add(chunk + (min(chunk, w.v - chunk) // T // 2) * T)   # inside the second chunk
    vids = sorted({v for s in starts if 0 <= s < w.v for v in range(s, min(s + T, w.v))})
    return np.array(sorted(set(rows)), np.int64), np.array(vids, np.int64)


@pytest.mark.parametrize("name", NAMES)
def test_fullsize_parity(name):
    import linear_cross_entropy_fwd_amd as flce
    from linear_cross_entropy_fwd_amd import _abi
    from oracle import gradient_samples
    g = load(name)
    w = fi.WORKLOADS[name]
    log_case(f"full size {w.name}")
    tol = TOL[w.dtype]
    d = fi.generate(w, device="cuda")
    # inputs: GPU draw == CPU draw
    hid_cpu = fi.normal_((w.n, w.h), 1.0, w.seed * 16 + 0, w.torch_dtype)
    assert torch.equal(d["hidden"].cpu(), hid_cpu)
    r0 = w.v // 2
    assert torch.equal(d["weight"][r0:r0 + 64].cpu(), fi.weight_rows(w, r0, r0 + 64))
    targets = torch.from_numpy(g["targets"].astype(np.int64)).cuda()
    gen_t = d["targets"]
    keep = ~d["argmax_rows"]
    assert torch.equal(gen_t[keep], targets[keep])

    hidden, weight, bias = d["hidden"], d["weight"], d["bias"]
    reds = [w.reduction] + (["none"] if name == "peaked_bf16" else [])
    for red in reds:
        loss, lse, metrics = flce.flce_forward(hidden, weight, targets, bias, ignore_index=w.ignore_index,
                                               logit_scale=w.logit_scale, softcap=w.softcap,
                                               reduction=red, return_metrics=w.return_metrics)
        torch.cuda.synchronize()
        assert record(name, f"lse ({red})", w.n, to_np(lse), g["lse"], tol["loss"]) <= tol["loss"]
        if red == "none":
            assert record(name, "per-row loss (none)", w.n, to_np(loss), g["row_loss"], tol["loss"]) <= tol["loss"]
        else:
            e = record(name, f"loss ({red})", 1, [loss.item()], [float(g["loss"])], tol["loss"])
            assert rel_err(loss.item(), float(g["loss"])) <= tol["loss"], (e, loss.item(), float(g["loss"]))
        if metrics is not None:
            m = to_np(metrics)
            nv = int(g["n_valid"])
            assert record(name, "entropy metric", 1, [m[1]], [float(g["entropy"])], tol["loss"]) <= tol["loss"]
            valid = g["targets"] != w.ignore_index
            ties = valid & (g["gap"] <= TIE[w.dtype] * np.maximum(1.0, np.abs(g["lse"])))
            assert abs(int(round(float(m[0]) * nv)) - int(g["hit"].sum())) <= int(ties.sum())
    # backward in the benchmark's configuration (the run's own reduction)
    loss, lse, _ = flce.flce_forward(hidden, weight, targets, bias, ignore_index=w.ignore_index,
                                     logit_scale=w.logit_scale, softcap=w.softcap, reduction=w.reduction)
    gh, gw, gb = flce.flce_backward(hidden, weight, targets, bias, lse, ignore_index=w.ignore_index,
                                    logit_scale=w.logit_scale, softcap=w.softcap, reduction=w.reduction)
    torch.cuda.synchronize()
    rows = torch.from_numpy(g["rows"]).cuda()
    vids = torch.from_numpy(g["vocab_ids"]).cuda()
    e_h = record(name, "grad_hidden, stored sample rows", int(rows.numel()) * w.h, to_np(gh[rows]),
                 g["grad_hidden_rows"], tol["grad"])
    e_w = record(name, "grad_weight, stored sample ids", int(vids.numel()) * w.h, to_np(gw[vids]),
                 g["grad_weight_rows"], tol["grad"])
    assert e_h <= tol["grad"] and e_w <= tol["grad"]
    if gb is not None:
        assert record(name, "grad_bias, stored sample ids", int(vids.numel()), to_np(gb[vids]),
                      g["grad_bias_entries"], tol["grad"]) <= tol["grad"]
    # whole tiles around the default plan's chunk boundaries, by the oracle from the stored lse
    plan = _abi.flce_backward_plan(_abi.make_problem(w.n, w.h, w.v, _abi.BF16, has_bias=bias is not None))
    trows, tvids = tile_ids(w, plan)
    log_case(f"  plan {plan}: {len(trows)} grad_hidden rows, {len(tvids)} grad_weight rows")
    ref = gradient_samples(to_np(hidden), to_np(weight), g["targets"].astype(np.int64), g["lse"], trows, tvids,
                           None if bias is None else to_np(bias), ignore_index=w.ignore_index,
                           logit_scale=w.logit_scale, softcap=w.softcap, reduction=w.reduction)
    e_th = record(name, "grad_hidden, 2 whole token tiles", len(trows) * w.h, to_np(gh[torch.from_numpy(trows).cuda()]),
                  ref["grad_hidden"], tol["grad"])
    e_tw = record(name, "grad_weight, whole vocab tiles", len(tvids) * w.h, to_np(gw[torch.from_numpy(tvids).cuda()]),
                  ref["grad_weight"], tol["grad"])
    assert e_th <= tol["grad"] and e_tw <= tol["grad"]
    if gb is not None:
        assert record(name, "grad_bias, whole vocab tiles", len(tvids), to_np(gb[torch.from_numpy(tvids).cuda()]),
                      ref["grad_bias"], tol["grad"]) <= tol["grad"]
    # properties over the whole gradient at full size
    assert torch.isfinite(gw).all() and torch.isfinite(gh).all()
    ign = targets == w.ignore_index
    if bool(ign.any()):
        assert torch.all(gh[ign] == 0)
    if w.softcap is None:
        col = gw.double().sum(0).abs().max().item()
        assert col <= tol["grad"] * gw.double().abs().sum(0).max().item()
