"""GPU test of flce_forward_noalloc, the forward entry point that allocates
nothing (its workspace is a fixed 32 MiB device array inside the library).

Two calls in a row through the C ABI, the second on a smaller problem (so it
runs on the array the first call left behind): each call's loss, lse and
metrics must equal those of flce_forward with a workspace of its own bit for
bit (the same kernels and plan), and sit within the bf16 tolerance of the
fp64 oracle.  A problem whose forward workspace exceeds the array is refused
before anything is launched."""
import numpy as np
import pytest
import torch

import flce_inputs as fi
from flce_testutil import TOL, gpu_inputs, log_case, maxnorm_rel, oracle_inputs, rel_err, to_np

pytestmark = pytest.mark.gpu


def _noalloc(p, g, n, metrics_on, reduction):
    from linear_cross_entropy_fwd_amd import _abi
    dev = g["hidden"].device
    loss = torch.full((n if reduction == "none" else 1,), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    metrics = torch.full((2,), float("nan"), dtype=torch.float32, device=dev) if metrics_on else None
    ptr = lambda t: 0 if t is None else t.data_ptr()
    torch.cuda.synchronize()
    _abi.check(_abi.flce_forward_noalloc(p, ptr(g["hidden"]), ptr(g["weight"]), ptr(g["targets"]),
                                         ptr(g["bias"]), ptr(loss), ptr(lse), ptr(metrics),
                                         torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return loss, lse, metrics


@pytest.mark.parametrize("first,second", [
    (dict(n=1000, h=256, v=5000), dict(n=300, h=128, v=3000)),
])
def test_noalloc_forward_matches_flce_forward_twice(first, second):
    import linear_cross_entropy_fwd_amd as flce
    from oracle import flce_reference
    base = fi.WORKLOADS["transforms_bf16"]     # bias, scale 0.5, cap 30, sum, metrics, 3 % ignored
    for k, sz in enumerate((first, second)):
        w = base.resized(**sz)
        log_case(f"no-alloc forward, call {k + 1}: {w.name} N={w.n} H={w.h} V={w.v}")
        d = fi.generate(w)
        g = gpu_inputs(d)
        p = flce.problem_for(g["hidden"], g["weight"], g["bias"], w.ignore_index, w.logit_scale, w.softcap,
                             w.reduction, w.return_metrics)
        loss, lse, metrics = _noalloc(p, g, w.n, w.return_metrics, w.reduction)
        rl, rlse, rm = flce.flce_forward(g["hidden"], g["weight"], g["targets"], g["bias"],
                                         ignore_index=w.ignore_index, logit_scale=w.logit_scale,
                                         softcap=w.softcap, reduction=w.reduction,
                                         return_metrics=w.return_metrics)
        torch.cuda.synchronize()
        assert torch.equal(loss, rl.reshape(loss.shape)) and torch.equal(lse, rlse)
        assert torch.equal(metrics, rm)
        h, wt, t, b = oracle_inputs(d)
        ref = flce_reference(h, wt, t, b, ignore_index=w.ignore_index, logit_scale=w.logit_scale,
                             softcap=w.softcap, reduction=w.reduction, compute_grads=False)
        tol = TOL[w.dtype]
        assert rel_err(loss.item(), ref["loss"]) <= tol["loss"]
        assert maxnorm_rel(to_np(lse), ref["lse"]) <= tol["loss"]
        assert rel_err(to_np(metrics)[1], ref["entropy"]) <= tol["loss"]


def test_noalloc_forward_refuses_a_problem_past_its_scratch():
    from linear_cross_entropy_fwd_amd import _abi
    # 128 splits x 5 fields (metrics) x 20000 rows x 4 B = 51.2 MB > 32 MiB
    p = _abi.make_problem(20000, 128, 262144, _abi.BF16, return_metrics=True)
    assert _abi.flce_forward_workspace_size(p) > 32 << 20
    fake = 0x100000
    st = _abi.flce_forward_noalloc(p, fake, fake, fake, 0, fake, fake, 0, 0)
    assert st == 3 and "fixed scratch" in _abi.last_error()
