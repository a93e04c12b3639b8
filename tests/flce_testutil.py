"""Shared helpers for the parity tests: run the GPU path and the oracle on the
same seeded inputs and compare them at the stated tolerances."""
from __future__ import annotations

import math
import os

import numpy as np
import torch

import flce_inputs as fi

# Acceptance: relative error of scalar / per-row losses, relative max-norm of gradients.
TOL = {"f32": dict(loss=1e-5, grad=1e-4), "bf16": dict(loss=2e-3, grad=2e-2),
       "f16": dict(loss=2e-3, grad=2e-2)}
# Argmax tie margin (rows whose top-1/top-2 gap is within it may legitimately differ).
TIE = {"f32": 1e-6, "bf16": 1e-4, "f16": 1e-4}

GOLDEN_DIR = os.path.join(os.path.dirname(__file__), "golden")


def log_case(msg: str) -> None:
    print(f"\n[case] {msg}", flush=True)


def to_np(t):
    if t is None:
        return None
    return t.detach().float().cpu().numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def rel_err(a, b) -> float:
    a, b = float(a), float(b)
    if math.isnan(b):
        return 0.0 if math.isnan(a) else math.inf
    return abs(a - b) / max(abs(b), 1e-30)


def maxnorm_rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0))


def oracle_inputs(d: dict):
    """numpy copies (exact fp32 widening) of generated inputs, for the oracle."""
    return (to_np(d["hidden"]), to_np(d["weight"]), to_np(d["targets"]),
            None if d["bias"] is None else to_np(d["bias"]))


def fill_argmax_targets(w: fi.Workload, d: dict) -> dict:
    """Rows chosen for argmax targets get the oracle's first-index argmax id."""
    if not bool(d["argmax_rows"].any()):
        return d
    from oracle import row_argmax_ids
    h, wt, _, b = oracle_inputs(d)
    ids = torch.from_numpy(row_argmax_ids(h, wt, b, w.logit_scale, w.softcap))
    d = dict(d)
    d["targets"] = torch.where(d["argmax_rows"], ids.to(d["targets"].device), d["targets"])
    return d


def gpu_inputs(d: dict, device="cuda") -> dict:
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def check_against_oracle(w: fi.Workload, d_gpu: dict, ref: dict, *, loss, lse=None, metrics=None,
                         grads=None, what=""):
    """Compare GPU outputs with the oracle dict at the workload dtype's tolerances."""
    tol = TOL[w.dtype]
    out = {}
    if w.reduction == "none":
        out["row_loss"] = maxnorm_rel(to_np(loss), ref["loss"])
        assert out["row_loss"] <= tol["loss"], (what, out)
    else:
        out["loss"] = rel_err(loss.item(), ref["loss"])
        assert out["loss"] <= tol["loss"], (what, out, loss.item(), ref["loss"])
    if lse is not None:
        out["lse"] = maxnorm_rel(to_np(lse), ref["lse"])
        assert out["lse"] <= tol["loss"], (what, out)
    if metrics is not None:
        m = to_np(metrics)
        nv = ref["n_valid"]
        if nv == 0:
            assert np.isnan(m[0]) and np.isnan(m[1]), (what, m)
        else:
            out["entropy"] = rel_err(m[1], ref["entropy"])
            assert out["entropy"] <= tol["loss"], (what, out, m[1], ref["entropy"])
            valid = to_np(d_gpu["targets"]) != w.ignore_index
            zmax_scale = np.maximum(1.0, np.abs(ref["lse"]))
            ties = valid & (ref["gap"] <= TIE[w.dtype] * zmax_scale)
            gpu_hits = int(round(float(m[0]) * nv))
            ref_hits = int(ref["hit"].sum())
            out["hits"] = (gpu_hits, ref_hits, int(ties.sum()))
            assert abs(gpu_hits - ref_hits) <= int(ties.sum()), (what, out)
    if grads is not None:
        gh, gw, gb = grads
        for name, g, r in (("grad_hidden", gh, ref["grad_hidden"]), ("grad_weight", gw, ref["grad_weight"]),
                           ("grad_bias", gb, ref.get("grad_bias"))):
            if g is None or r is None:
                continue
            out[name] = maxnorm_rel(to_np(g), r)
            assert out[name] <= tol["grad"], (what, name, out)
    return out
