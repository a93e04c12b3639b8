"""GPU invariants of the definition that hold at any size: bit-identity under
the metrics flag, run-to-run determinism, ignored rows contributing nothing,
per-row independence from the batch, closed forms (zero scale, zero weight),
vanishing gradient sums, and the out-of-range-target status."""
import math

import numpy as np
import pytest
import torch

import flce_inputs as fi
from flce_testutil import gpu_inputs, log_case, maxnorm_rel, to_np

pytestmark = pytest.mark.gpu

W = fi.WORKLOADS


def fwd_bwd(g, w, return_metrics=None, reduction=None, **kw):
    import linear_cross_entropy_fwd_amd as flce
    red = reduction or w.reduction
    rm = w.return_metrics if return_metrics is None else return_metrics
    loss, lse, m = flce.flce_forward(g["hidden"], g["weight"], g["targets"], g["bias"],
                                     ignore_index=w.ignore_index, logit_scale=w.logit_scale,
                                     softcap=w.softcap, reduction=red, return_metrics=rm,
                                     fwd_tiles_per_split=kw.get("tps", 0))
    grads = flce.flce_backward(g["hidden"], g["weight"], g["targets"], g["bias"], lse,
                               ignore_index=w.ignore_index, logit_scale=w.logit_scale,
                               softcap=w.softcap, reduction=red,
                               bwd_vocab_chunk=kw.get("chunk", 0))
    torch.cuda.synchronize()
    return loss, lse, m, grads


def _bits(t):
    t = t.contiguous().view(-1)
    return t.view({1: torch.int8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[t.element_size()])


def bitwise_equal(a, b):
    if a is None or b is None:
        return a is None and b is None
    return a.shape == b.shape and torch.equal(_bits(a), _bits(b))


def small_transforms():
    return W["transforms_bf16"].resized(n=300, h=256, v=2600)


def test_metrics_flag_leaves_loss_and_grads_bit_identical():
    w = small_transforms()
    log_case("metrics toggle " + w.name)
    g = gpu_inputs(fi.generate(w))
    a = fwd_bwd(g, w, return_metrics=False, chunk=1024)
    b = fwd_bwd(g, w, return_metrics=True, chunk=1024)
    assert bitwise_equal(a[0], b[0]) and bitwise_equal(a[1], b[1])
    for x, y in zip(a[3], b[3]):
        assert bitwise_equal(x, y)


def test_run_to_run_bitwise_determinism():
    w = small_transforms()
    log_case("determinism " + w.name)
    g = gpu_inputs(fi.generate(w))
    a = fwd_bwd(g, w, chunk=512)
    b = fwd_bwd(g, w, chunk=512)
    for x, y in zip(a[:3], b[:3]):
        assert bitwise_equal(x, y)
    for x, y in zip(a[3], b[3]):
        assert bitwise_equal(x, y)


def test_ignored_rows_contribute_nothing():
    w = small_transforms()
    log_case("ignored rows " + w.name)
    d = fi.generate(w)
    g = gpu_inputs(d)
    a = fwd_bwd(g, w)
    ign = g["targets"] == w.ignore_index
    assert int(ign.sum()) > 0
    g2 = dict(g)
    h2 = g["hidden"].clone()
    h2[ign] = (torch.randn(int(ign.sum()), w.h, device="cuda") * 50).to(h2.dtype)
    g2["hidden"] = h2
    b = fwd_bwd(g2, w)
    assert bitwise_equal(a[0], b[0])
    assert bitwise_equal(a[2], b[2])  # metrics
    assert bitwise_equal(a[3][1], b[3][1]) and bitwise_equal(a[3][2], b[3][2])  # dW, db
    assert torch.all(a[3][0][ign] == 0) and torch.all(b[3][0][ign] == 0)


def test_per_row_loss_independent_of_batch_split():
    w = W["headvocab_bf16"].resized(n=600, h=256, v=5000, reduction="none")
    log_case("batch split " + w.name)
    g = gpu_inputs(fi.generate(w))
    full = fwd_bwd(g, w)
    for lo, hi in ((0, 300), (300, 600), (17, 341)):
        part = {k: (v[lo:hi].contiguous() if k in ("hidden", "targets") else v) for k, v in g.items()}
        sub = fwd_bwd(part, w)
        assert bitwise_equal(sub[0], full[0][lo:hi].contiguous())
        assert bitwise_equal(sub[1], full[1][lo:hi].contiguous())
        assert bitwise_equal(sub[3][0], full[3][0][lo:hi].contiguous())  # grad_hidden rows


def test_forward_rows_independent_of_split_grouping():
    # V = 128256: 501 vocabulary tiles in 126 splits of 4 (by V only).  A forward
    # workgroup walks a run of consecutive splits chosen from N: 4 splits at
    # N = 4096 (16 token tiles), 2 at N = 1024, 1 at N = 256.  Each split ends in
    # its own record, so every row's lse, loss and argmax must keep its bits.
    import linear_cross_entropy_fwd_amd as flce
    w = W["transforms_bf16"].resized(n=4096, h=64, v=128256, reduction="none")
    log_case("split grouping " + w.name)
    g = gpu_inputs(fi.generate(w))

    def rows(n):
        pred = torch.empty(n, dtype=torch.int64, device="cuda")
        loss, lse, m = flce.flce_forward(g["hidden"][:n].contiguous(), g["weight"], g["targets"][:n].contiguous(),
                                         g["bias"], ignore_index=w.ignore_index, logit_scale=w.logit_scale,
                                         softcap=w.softcap, reduction="none", return_metrics=True, predictions=pred)
        torch.cuda.synchronize()
        return loss, lse, pred

    from linear_cross_entropy_fwd_amd import _abi
    groups = [_abi.flce_forward_plan(flce.problem_for(g["hidden"][:n], g["weight"], g["bias"], softcap=w.softcap,
                                                      return_metrics=True)) for n in (4096, 1024, 256)]
    assert groups == [(4, 126, 4), (4, 126, 2), (4, 126, 1)], groups
    full = rows(4096)
    for n in (1024, 256):
        sub = rows(n)
        for a, b in zip(sub, full):
            assert bitwise_equal(a, b[:n].contiguous())


def test_zero_scale_gives_ln_v_and_zero_grads():
    w = W["transforms_bf16"].resized(n=200, h=128, v=3000, logit_scale=0.0, reduction="mean")
    log_case("zero scale " + w.name)
    g = gpu_inputs(fi.generate(w))
    loss, lse, m, (gh, gw, gb) = fwd_bwd(g, w)
    assert abs(loss.item() - math.log(3000)) <= 1e-6 * math.log(3000)
    assert abs(m[1].item() - math.log(3000)) <= 1e-6 * math.log(3000)
    assert torch.all(gh == 0) and torch.all(gw == 0) and torch.all(gb == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_weight_closed_form(dtype):
    v = 1000
    w = W["tiny_f32"].resized(n=300, h=64, v=v, dtype=dtype, return_metrics=True)
    log_case("zero weight " + dtype)
    d = fi.generate(w)
    d["weight"] = torch.zeros_like(d["weight"])
    d["targets"] = torch.where(d["targets"] >= 0, d["targets"] % 4, d["targets"])  # many id-0 rows
    g = gpu_inputs(d)
    loss, lse, m, (gh, gw, gb) = fwd_bwd(g, w)
    t = to_np(d["targets"])
    h = to_np(d["hidden"]).astype(np.float64)
    valid = t != -100
    nv = int(valid.sum())
    lnv = math.log(v)
    assert abs(loss.item() - lnv) <= 1e-6 * lnv
    assert abs(m[1].item() - lnv) <= 1e-6 * lnv
    # every logit ties: first-index argmax is id 0
    assert int(round(m[0].item() * nv)) == int(np.sum(valid & (t == 0)))
    assert torch.all(gh == 0)
    exp_dw = np.repeat(h[valid].sum(0)[None, :] / v, v, axis=0)
    for i in np.nonzero(valid)[0]:
        exp_dw[t[i]] -= h[i]
    exp_dw /= nv
    tol = 1e-4 if dtype == "f32" else 2e-2
    assert maxnorm_rel(to_np(gw), exp_dw) <= tol


def test_gradient_sums_vanish_without_softcap():
    w = W["transforms_bf16"].resized(n=256, h=256, v=4000, softcap=None)
    log_case("gradient sums " + w.name)
    g = gpu_inputs(fi.generate(w))
    _, _, _, (gh, gw, gb) = fwd_bwd(g, w, chunk=1024)
    gwf = gw.double()
    col = gwf.sum(0).abs().max().item()
    assert col <= 2e-2 * gwf.abs().sum(0).max().item()
    gbf = gb.double()
    assert abs(gbf.sum().item()) <= 2e-2 * gbf.abs().sum().item()


def test_out_of_range_target_sets_status_and_nan_row():
    import linear_cross_entropy_fwd_amd as flce
    from linear_cross_entropy_fwd_amd import _abi
    w = W["tiny_f32"].resized(n=70, h=64, v=300, reduction="none", return_metrics=False)
    log_case("bad target")
    g = gpu_inputs(fi.generate(w))
    g["targets"][5] = 300
    g["targets"][9] = -7
    p = flce.problem_for(g["hidden"], g["weight"], g["bias"], reduction="none")
    ws = torch.empty(_abi.flce_forward_workspace_size(p), dtype=torch.uint8, device="cuda")
    loss, lse, _ = flce.flce_forward(g["hidden"], g["weight"], g["targets"], g["bias"],
                                     reduction="none", workspace=ws)
    status = _abi.flce_forward_status(p, ws.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert status & 1
    lossc = loss.cpu()
    assert math.isnan(lossc[5]) and math.isnan(lossc[9])
    assert torch.isfinite(torch.cat([lossc[:5], lossc[10:]])).all()
    # the documented spread: the bad rows' grad_hidden rows are NaN, the other rows are finite,
    # and every grad_weight entry is NaN (grad_weight contracts over every row)
    gh, gw, _ = flce.flce_backward(g["hidden"], g["weight"], g["targets"], g["bias"], lse,
                                   reduction="none")
    ghc = gh.cpu()
    assert torch.isnan(ghc[5]).all() and torch.isnan(ghc[9]).all()
    assert torch.isfinite(torch.cat([ghc[:5], ghc[6:9], ghc[10:]])).all()
    assert torch.isnan(gw.cpu()).all()
    # a mean loss is NaN; with a bias, every grad_bias entry is NaN too
    wb = W["transforms_bf16"].resized(n=64, h=64, v=600, softcap=None, reduction="mean", return_metrics=False)
    gb_in = gpu_inputs(fi.generate(wb))
    gb_in["targets"][3] = 600
    lossm, lsem, _ = flce.flce_forward(gb_in["hidden"], gb_in["weight"], gb_in["targets"], gb_in["bias"],
                                       reduction="mean", logit_scale=wb.logit_scale)
    assert math.isnan(lossm.item())
    ghm, gwm, gbm = flce.flce_backward(gb_in["hidden"], gb_in["weight"], gb_in["targets"], gb_in["bias"], lsem,
                                       reduction="mean", logit_scale=wb.logit_scale)
    ghm = ghm.float().cpu()
    assert torch.isnan(ghm[3]).all() and torch.isfinite(torch.cat([ghm[:3], ghm[4:]])).all()
    assert torch.isnan(gwm.float().cpu()).all() and torch.isnan(gbm.float().cpu()).all()
