"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (default plan).  Expected values come from
tests/golden/fullsize_<workload>.npz, written by tests/golden/make_fullsize.py
with the fp64 oracle only: every row's lse / loss and the metrics, plus
gradient entries at sampled token rows and vocabulary ids.  The inputs are
drawn on the GPU; the test first checks that they are bit-identical to the
CPU draw the oracle saw (hidden in full, a band of weight rows)."""
import math
import os

import numpy as np
import pytest
import torch

import flce_inputs as fi
from flce_testutil import TIE, TOL, log_case, maxnorm_rel, rel_err, to_np

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NAMES = ["midvocab_bf16", "headvocab_bf16", "transforms_bf16", "peaked_bf16"]


def load(name):
    path = os.path.join(GOLDEN, f"fullsize_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated (tests/golden/make_fullsize.py)")
    return dict(np.load(path))


@pytest.mark.parametrize("name", NAMES)
def test_fullsize_parity(name):
    import linear_cross_entropy_fwd_amd as flce
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
        assert maxnorm_rel(to_np(lse), g["lse"]) <= tol["loss"]
        if red == "none":
            assert maxnorm_rel(to_np(loss), g["row_loss"]) <= tol["loss"]
        else:
            assert rel_err(loss.item(), float(g["loss"])) <= tol["loss"], (loss.item(), float(g["loss"]))
        if metrics is not None:
            m = to_np(metrics)
            nv = int(g["n_valid"])
            assert rel_err(m[1], float(g["entropy"])) <= tol["loss"]
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
    e_h = maxnorm_rel(to_np(gh[rows]), g["grad_hidden_rows"])
    e_w = maxnorm_rel(to_np(gw[vids]), g["grad_weight_rows"])
    print(f"  sampled gradient errors: hidden {e_h:.2e}, weight {e_w:.2e}", flush=True)
    assert e_h <= tol["grad"] and e_w <= tol["grad"]
    if gb is not None:
        assert maxnorm_rel(to_np(gb[vids]), g["grad_bias_entries"]) <= tol["grad"]
    # properties over the whole gradient at full size
    assert torch.isfinite(gw).all() and torch.isfinite(gh).all()
    ign = targets == w.ignore_index
    if bool(ign.any()):
        assert torch.all(gh[ign] == 0)
    if w.softcap is None:
        col = gw.double().sum(0).abs().max().item()
        assert col <= tol["grad"] * gw.double().abs().sum(0).max().item()
