"""CPU pins of the fp64 oracle.

Each pin checks the oracle against something other than itself: a library
routine (torch cross_entropy and autograd, scipy logsumexp / softmax /
entropy), a closed form (zero weight, zero scale, two classes), an invariant
of the definition, brute force, or central finite differences.  The mutation
tests at the end plant plausible mistakes in the oracle and check that at
least one pin catches each of them.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch
import torch.nn.functional as F

import oracle.flce_oracle as orc
from oracle import flce_reference

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.txt")


def golden_ln_v():
    out = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        v, val = line.split()
        out[int(v)] = float(val)
    return out


def problem(seed, n, hd, v, bias=False, ignore_frac=0.2, ignore_index=-100, wstd=0.5):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((n, hd))
    w = rng.standard_normal((v, hd)) * wstd
    b = rng.standard_normal(v) * 0.3 if bias else None
    t = rng.integers(0, v, n)
    t[rng.random(n) < ignore_frac] = ignore_index
    return h, w, b, t


def torch_loss(h, w, b, t, ignore_index, s, cap, reduction, g=None, grads=True):
    """Library routine: torch cross_entropy on fp64 logits, gradients by autograd."""
    th = torch.tensor(h, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    tb = torch.tensor(b, requires_grad=True) if b is not None else None
    logits = F.linear(th, tw, tb) * s
    if cap is not None:
        logits = cap * torch.tanh(logits / cap)
    loss = F.cross_entropy(logits, torch.tensor(t), ignore_index=ignore_index, reduction=reduction)
    if not grads:
        return loss.detach().numpy(), None, None, None
    if reduction == "none":
        gv = torch.tensor(g if g is not None else np.ones(len(t)))
        (loss * gv).sum().backward()
    else:
        (loss * (1.0 if g is None else float(g))).backward()
    return (loss.detach().numpy(), th.grad.numpy(), tw.grad.numpy(),
            tb.grad.numpy() if tb is not None else None)


def maxnorm_rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    den = np.max(np.abs(b))
    return np.max(np.abs(a - b)) / (den if den > 0 else 1.0)


# --------------------------------------------------------------------------- library routines

@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("ignore_index", [-100, 3])
def test_plain_loss_and_grads_match_torch(reduction, bias, ignore_index):
    h, w, b, t = problem(11, 37, 16, 53, bias=bias, ignore_index=ignore_index)
    g = np.random.default_rng(5).standard_normal(37) if reduction == "none" else 0.75
    ref = flce_reference(h, w, t, b, ignore_index=ignore_index, reduction=reduction, grad_output=g)
    tl, gh, gw, gb = torch_loss(h, w, b, t, ignore_index, 1.0, None, reduction, g)
    np.testing.assert_allclose(ref["loss"], tl, rtol=1e-12, atol=1e-13)
    assert maxnorm_rel(ref["grad_hidden"], gh) < 1e-12
    assert maxnorm_rel(ref["grad_weight"], gw) < 1e-12
    if bias:
        assert maxnorm_rel(ref["grad_bias"], gb) < 1e-12


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_scale_softcap_chain_rule_matches_autograd(reduction):
    # The transform order (bias, scale, cap) is the reading the test encodes;
    # the derivative comes from autograd, independently of the oracle's formula.
    h, w, b, t = problem(12, 29, 24, 61, bias=True, wstd=2.0)
    g = np.random.default_rng(6).standard_normal(29) if reduction == "none" else 1.3
    for s, cap in [(0.5, 3.0), (2.0, 1.5), (0.7, None)]:
        ref = flce_reference(h, w, t, b, logit_scale=s, softcap=cap, reduction=reduction, grad_output=g)
        tl, gh, gw, gb = torch_loss(h, w, b, t, -100, s, cap, reduction, g)
        np.testing.assert_allclose(ref["loss"], tl, rtol=1e-12, atol=1e-13)
        assert maxnorm_rel(ref["grad_hidden"], gh) < 1e-11
        assert maxnorm_rel(ref["grad_weight"], gw) < 1e-11
        assert maxnorm_rel(ref["grad_bias"], gb) < 1e-11


def test_row_statistics_match_scipy():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((40, 300)) * 4.0
    z[0] = 0.0                         # uniform row
    z[1, 17] = 60.0                    # nearly one-hot row
    lse, p, ent, am, gap = orc.row_statistics(z)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(z, axis=1), rtol=1e-14)
    np.testing.assert_allclose(p, scipy.special.softmax(z, axis=1), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(ent, scipy.stats.entropy(scipy.special.softmax(z, axis=1), axis=1),
                               rtol=1e-10, atol=1e-12)


def test_argmax_and_gap_brute_force():
    rng = np.random.default_rng(4)
    z = rng.integers(-3, 4, size=(60, 9)).astype(np.float64)   # many exact ties
    _, _, _, am, gap = orc.row_statistics(z)
    for i in range(z.shape[0]):
        row = list(z[i])
        best = 0
        for j in range(1, len(row)):
            if row[j] > row[best]:
                best = j
        assert am[i] == best
        srt = sorted(row, reverse=True)
        assert gap[i] == srt[0] - srt[1]


def test_hit_and_accuracy_brute_force():
    h, w, b, t = problem(13, 50, 8, 7, ignore_frac=0.3)
    ref = flce_reference(h, w, t, compute_grads=False)
    z = h @ w.T
    hits = valid = 0
    for i in range(50):
        if t[i] == -100:
            continue
        valid += 1
        best = max(range(7), key=lambda j: (z[i, j], -j))
        hits += int(best == t[i])
    assert ref["n_valid"] == valid
    assert ref["accuracy"] == hits / valid


# --------------------------------------------------------------------------- finite differences

@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_finite_differences(reduction):
    h, w, b, t = problem(14, 3, 4, 6, bias=True, ignore_frac=0.0, wstd=1.0)
    t[1] = -100
    g = np.array([0.7, -1.1, 1.9]) if reduction == "none" else 1.0
    s, cap = 0.8, 1.2
    ref = flce_reference(h, w, t, b, logit_scale=s, softcap=cap, reduction=reduction, grad_output=g)

    def f(hh, ww, bb):
        out = flce_reference(hh, ww, t, bb, logit_scale=s, softcap=cap, reduction=reduction,
                             compute_grads=False)["loss"]
        return float(np.sum(out * g)) if reduction == "none" else float(out)

    eps = 1e-6
    for name, arr, grad in [("h", h, ref["grad_hidden"]), ("w", w, ref["grad_weight"]),
                            ("b", b, ref["grad_bias"])]:
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += eps
            am[idx] -= eps
            args_p = {"h": (ap, w, b), "w": (h, ap, b), "b": (h, w, ap)}[name]
            args_m = {"h": (am, w, b), "w": (h, am, b), "b": (h, w, am)}[name]
            fd[idx] = (f(*args_p) - f(*args_m)) / (2 * eps)
        assert maxnorm_rel(grad, fd) < 1e-6, name


# --------------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("v", [7, 1000])
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_zero_weight_closed_form(v, reduction):
    lnv = golden_ln_v()[v]
    n, hd = 40, 6
    rng = np.random.default_rng(v)
    h = rng.standard_normal((n, hd))
    t = rng.integers(0, min(v, 4), n)          # many targets at id 0
    t[::5] = -100
    w = np.zeros((v, hd))
    b = np.zeros(v)
    ref = flce_reference(h, w, t, b, reduction=reduction)
    valid = t != -100
    nv = int(valid.sum())
    c = 1.0 / nv if reduction == "mean" else 1.0
    np.testing.assert_allclose(ref["row_loss"][valid], lnv, rtol=1e-15)
    np.testing.assert_allclose(ref["loss"], lnv if reduction == "mean" else nv * lnv, rtol=1e-14)
    np.testing.assert_allclose(ref["entropy"], lnv, rtol=1e-14)
    assert ref["accuracy"] == np.sum(valid & (t == 0)) / nv      # first-index tie-break
    assert np.all(ref["grad_hidden"] == 0.0)
    exp_dw = c * (h[valid].sum(0)[None, :] / v)
    exp_dw = np.repeat(exp_dw, v, axis=0)
    exp_db = np.full(v, c * nv / v)
    for i in np.nonzero(valid)[0]:
        exp_dw[t[i]] -= c * h[i]
        exp_db[t[i]] -= c
    np.testing.assert_allclose(ref["grad_weight"], exp_dw, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(ref["grad_bias"], exp_db, rtol=1e-12, atol=1e-15)


def test_zero_scale_closed_form():
    h, w, b, t = problem(15, 30, 10, 1000, bias=True)
    ref = flce_reference(h, w, t, b, logit_scale=0.0, softcap=5.0)
    np.testing.assert_allclose(ref["loss"], golden_ln_v()[1000], rtol=1e-14)
    for k in ("grad_hidden", "grad_weight", "grad_bias"):
        assert np.all(ref[k] == 0.0)


def test_two_class_closed_form():
    h, w, b, t = problem(16, 25, 5, 2, bias=True, ignore_frac=0.0)
    ref = flce_reference(h, w, t, b, reduction="none")
    z = h @ w.T + b
    other = z[np.arange(25), 1 - t]
    mine = z[np.arange(25), t]
    np.testing.assert_allclose(ref["row_loss"], np.log1p(np.exp(other - mine)), rtol=1e-13)
    p0 = 1.0 / (1.0 + np.exp(z[:, 1] - z[:, 0]))
    ent = -(p0 * np.log(p0) + (1 - p0) * np.log(1 - p0))
    np.testing.assert_allclose(ref["row_entropy"], ent, rtol=1e-11, atol=1e-14)


def test_all_rows_ignored():
    h, w, b, t = problem(17, 9, 4, 11, bias=True)
    t[:] = -100
    m = flce_reference(h, w, t, b, reduction="mean")
    assert math.isnan(m["loss"]) and math.isnan(m["accuracy"]) and math.isnan(m["entropy"])
    for k in ("grad_hidden", "grad_weight", "grad_bias"):
        assert np.all(m[k] == 0.0)
    s = flce_reference(h, w, t, b, reduction="sum")
    assert s["loss"] == 0.0
    nn = flce_reference(h, w, t, b, reduction="none")
    assert np.all(nn["loss"] == 0.0)


# --------------------------------------------------------------------------- invariants

def test_gradient_rows_sum_to_zero():
    h, w, b, t = problem(18, 33, 12, 97, bias=True, wstd=1.5)
    ref = flce_reference(h, w, t, b, logit_scale=0.6)
    scale = np.max(np.abs(ref["grad_weight"]))
    assert abs(ref["grad_bias"].sum()) < 1e-13 * max(1.0, np.abs(ref["grad_bias"]).max())
    assert np.max(np.abs(ref["grad_weight"].sum(axis=0))) < 1e-12 * max(1.0, scale)


def test_ignored_rows_contribute_nothing():
    h, w, b, t = problem(19, 40, 8, 31, bias=True, ignore_frac=0.3)
    ign = t == -100
    ref = flce_reference(h, w, t, b)
    assert np.all(ref["grad_hidden"][ign] == 0.0)
    h2 = h.copy()
    h2[ign] = np.random.default_rng(0).standard_normal((ign.sum(), 8)) * 100
    ref2 = flce_reference(h2, w, t, b)
    assert ref2["loss"] == ref["loss"]
    np.testing.assert_array_equal(ref2["grad_weight"], ref["grad_weight"])
    np.testing.assert_array_equal(ref2["grad_bias"], ref["grad_bias"])


def test_shift_invariance():
    h, w, b, t = problem(20, 30, 8, 40, bias=True)
    ref = flce_reference(h, w, t, b, compute_grads=False)
    shifted_b = flce_reference(h, w, t, b + 3.25, compute_grads=False)
    u = np.random.default_rng(1).standard_normal(8)
    shifted_w = flce_reference(h, w + u[None, :], t, b, compute_grads=False)
    np.testing.assert_allclose(shifted_b["loss"], ref["loss"], rtol=1e-13)
    np.testing.assert_allclose(shifted_w["loss"], ref["loss"], rtol=1e-12)


def test_row_block_invariance():
    h, w, b, t = problem(21, 70, 8, 45, bias=True)
    a = flce_reference(h, w, t, b, logit_scale=0.9, softcap=4.0, row_block=1)
    c = flce_reference(h, w, t, b, logit_scale=0.9, softcap=4.0, row_block=256)
    for k in ("row_loss", "lse", "row_entropy", "grad_hidden", "grad_weight", "grad_bias"):
        np.testing.assert_allclose(a[k], c[k], rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(a["argmax"], c["argmax"])


def test_out_of_range_target_raises():
    h, w, b, t = problem(22, 5, 4, 6)
    t[0] = 6
    with pytest.raises(ValueError):
        flce_reference(h, w, t)
    t[0] = -1                                       # not the ignore index: invalid
    with pytest.raises(ValueError):
        flce_reference(h, w, t)


# --------------------------------------------------------------------------- planted mistakes

def _pins_fail(check):
    with pytest.raises(AssertionError):
        check()


def test_mutation_dropped_cap_factor_is_caught(monkeypatch):
    monkeypatch.setattr(orc, "transform_derivative", lambda z, s, c: np.full_like(z, s))
    _pins_fail(lambda: test_finite_differences("mean"))


def test_mutation_scale_before_bias_is_caught(monkeypatch):
    def wrong(raw, bias, s, cap):
        y = s * raw + (bias[None, :] if bias is not None else 0.0)
        return cap * np.tanh(y / cap) if cap is not None else y
    monkeypatch.setattr(orc, "transform_logits", wrong)
    _pins_fail(lambda: test_scale_softcap_chain_rule_matches_autograd("sum"))


def test_mutation_entropy_sign_is_caught(monkeypatch):
    real = orc.row_statistics

    def wrong(z):
        lse, p, ent, am, gap = real(z)
        return lse, p, lse + (p * z).sum(axis=1), am, gap
    monkeypatch.setattr(orc, "row_statistics", wrong)
    _pins_fail(test_row_statistics_match_scipy)


def test_mutation_unnormalised_softmax_is_caught(monkeypatch):
    real = orc.row_statistics

    def wrong(z):
        lse, p, ent, am, gap = real(z)
        return lse, p * 0.999, ent, am, gap       # a probability that does not sum to 1
    monkeypatch.setattr(orc, "row_statistics", wrong)
    _pins_fail(lambda: test_plain_loss_and_grads_match_torch("mean", False, -100))
    _pins_fail(test_gradient_rows_sum_to_zero)


def test_mutation_last_index_argmax_is_caught(monkeypatch):
    real = orc.row_statistics

    def wrong(z):
        lse, p, ent, am, gap = real(z)
        return lse, p, ent, z.shape[1] - 1 - z[:, ::-1].argmax(axis=1), gap
    monkeypatch.setattr(orc, "row_statistics", wrong)
    _pins_fail(lambda: test_zero_weight_closed_form(7, "mean"))
    _pins_fail(test_argmax_and_gap_brute_force)


# --------------------------------------------------------------------------- sampled gradients

@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_gradient_samples_match_autograd(reduction):
    h, w, b, t = problem(23, 41, 12, 70, bias=True, ignore_frac=0.25, wstd=1.5)
    g = np.random.default_rng(9).standard_normal(41) if reduction == "none" else 0.6
    for s, cap in [(1.0, None), (0.5, 2.5)]:
        fwd = flce_reference(h, w, t, b, logit_scale=s, softcap=cap, reduction=reduction,
                             compute_grads=False)
        rows = [0, 3, 17, 40] + list(np.nonzero(t == -100)[0][:1])
        vids = [0, 5, int(t[t >= 0][0]), 69]
        smp = orc.gradient_samples(h, w, t, fwd["lse"], rows, vids, b, logit_scale=s, softcap=cap,
                                   reduction=reduction, grad_output=g)
        _, gh, gw, gb = torch_loss(h, w, b, t, -100, s, cap, reduction, g)
        np.testing.assert_allclose(smp["grad_hidden"], gh[rows], rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(smp["grad_weight"], gw[vids], rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(smp["grad_bias"], gb[vids], rtol=1e-10, atol=1e-13)


# --------------------------------------------------------------------------- loss variants
# Label smoothing and class weights each against torch's cross_entropy (value
# and autograd gradients); the z-loss against torch's logsumexp under
# autograd and a closed form; the three together by finite differences.

def torch_variant_loss(h, w, b, t, ignore_index, s, cap, reduction, g, eps=0.0, cw=None, zl=0.0):
    th = torch.tensor(h, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    tb = torch.tensor(b, requires_grad=True) if b is not None else None
    logits = F.linear(th, tw, tb) * s
    if cap is not None:
        logits = cap * torch.tanh(logits / cap)
    tt = torch.tensor(t)
    loss = F.cross_entropy(logits, tt, ignore_index=ignore_index, reduction=reduction,
                           label_smoothing=eps, weight=None if cw is None else torch.tensor(cw))
    if zl:
        # z-loss term per row, zero on ignored rows, reduced like the loss (no class weights here)
        valid = (tt != ignore_index).double()
        zrow = zl * torch.logsumexp(logits, dim=1) ** 2 * valid
        if reduction == "none":
            loss = loss + zrow
        elif reduction == "sum":
            loss = loss + zrow.sum()
        else:
            loss = loss + zrow.sum() / valid.sum()
    if reduction == "none":
        (loss * torch.tensor(g)).sum().backward()
    else:
        (loss * float(g)).backward()
    return (loss.detach().numpy(), th.grad.numpy(), tw.grad.numpy(),
            tb.grad.numpy() if tb is not None else None)


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_label_smoothing_matches_torch(reduction):
    h, w, b, t = problem(21, 31, 12, 47, bias=True, wstd=1.0)
    g = np.random.default_rng(7).standard_normal(31) if reduction == "none" else 0.9
    for eps, s, cap in [(0.1, 1.0, None), (0.3, 0.7, 2.5), (1.0, 1.0, None)]:
        ref = flce_reference(h, w, t, b, logit_scale=s, softcap=cap, reduction=reduction, grad_output=g,
                             label_smoothing=eps)
        tl, gh, gw, gb = torch_variant_loss(h, w, b, t, -100, s, cap, reduction, g, eps=eps)
        np.testing.assert_allclose(ref["loss"], tl, rtol=1e-12, atol=1e-13)
        assert maxnorm_rel(ref["grad_hidden"], gh) < 1e-11
        assert maxnorm_rel(ref["grad_weight"], gw) < 1e-11
        assert maxnorm_rel(ref["grad_bias"], gb) < 1e-11


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_class_weights_match_torch(reduction):
    h, w, b, t = problem(22, 33, 10, 29, bias=False, wstd=1.0)
    cw = np.random.default_rng(8).uniform(0.2, 3.0, 29)
    cw[5] = 0.0
    g = np.random.default_rng(9).standard_normal(33) if reduction == "none" else 1.4
    ref = flce_reference(h, w, t, None, reduction=reduction, grad_output=g, class_weight=cw)
    tl, gh, gw, _ = torch_variant_loss(h, w, None, t, -100, 1.0, None, reduction, g, cw=cw)
    np.testing.assert_allclose(ref["loss"], tl, rtol=1e-12, atol=1e-13)
    assert maxnorm_rel(ref["grad_hidden"], gh) < 1e-11
    assert maxnorm_rel(ref["grad_weight"], gw) < 1e-11


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_z_loss_matches_autograd(reduction):
    h, w, b, t = problem(23, 27, 14, 41, bias=True, wstd=1.0)
    g = np.random.default_rng(10).standard_normal(27) if reduction == "none" else 0.6
    for zl, s, cap in [(1e-4, 1.0, None), (0.05, 0.8, 3.0)]:
        ref = flce_reference(h, w, t, b, logit_scale=s, softcap=cap, reduction=reduction, grad_output=g,
                             z_loss=zl)
        tl, gh, gw, gb = torch_variant_loss(h, w, b, t, -100, s, cap, reduction, g, zl=zl)
        np.testing.assert_allclose(ref["loss"], tl, rtol=1e-12, atol=1e-13)
        assert maxnorm_rel(ref["grad_hidden"], gh) < 1e-11
        assert maxnorm_rel(ref["grad_weight"], gw) < 1e-11
        assert maxnorm_rel(ref["grad_bias"], gb) < 1e-11


def test_z_loss_and_smoothing_zero_weight_closed_form():
    # zero weight: every z is 0, lse = ln V, the smoothed cross-entropy is ln V
    # for any eps, and the z-loss adds zl (ln V)^2; dL/dz_j = (1 + 2 zl ln V)/V
    # - (1 - eps)[j = t] - eps/V, so grad_weight[j] = sum_i coef_i dL/dz_ij h_i.
    v = 1000
    lnv = golden_ln_v()[v]
    rng = np.random.default_rng(24)
    n, hd = 9, 5
    h = rng.standard_normal((n, hd))
    w = np.zeros((v, hd))
    t = rng.integers(0, v, n)
    zl, eps = 0.01, 0.2
    ref = flce_reference(h, w, t, reduction="sum", label_smoothing=eps, z_loss=zl)
    assert abs(ref["loss"] - n * (lnv + zl * lnv ** 2)) < 1e-9 * n * lnv
    dz = np.full((n, v), (1.0 + 2.0 * zl * lnv) / v - eps / v)
    dz[np.arange(n), t] -= 1.0 - eps
    assert maxnorm_rel(ref["grad_weight"], dz.T @ h) < 1e-12
    assert np.max(np.abs(ref["grad_hidden"])) == 0.0


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_variants_together_finite_differences(reduction):
    h, w, b, t = problem(25, 3, 4, 6, bias=True, ignore_frac=0.0, wstd=1.0)
    t[1] = -100
    cw = np.array([0.5, 2.0, 1.0, 0.0, 1.5, 3.0])
    g = np.array([0.7, -1.1, 1.9]) if reduction == "none" else 1.0
    kw = dict(logit_scale=0.8, softcap=1.2, reduction=reduction, label_smoothing=0.15, z_loss=0.03,
              class_weight=cw)
    ref = flce_reference(h, w, t, b, grad_output=g, **kw)

    def f(hh, ww, bb):
        out = flce_reference(hh, ww, t, bb, compute_grads=False, **kw)["loss"]
        return float(np.sum(out * g)) if reduction == "none" else float(out)

    eps = 1e-6
    for name, arr, grad in [("h", h, ref["grad_hidden"]), ("w", w, ref["grad_weight"]),
                            ("b", b, ref["grad_bias"])]:
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += eps
            am[idx] -= eps
            args_p = {"h": (ap, w, b), "w": (h, ap, b), "b": (h, w, ap)}[name]
            args_m = {"h": (am, w, b), "w": (h, am, b), "b": (h, w, am)}[name]
            fd[idx] = (f(*args_p) - f(*args_m)) / (2 * eps)
        assert maxnorm_rel(grad, fd) < 1e-6, name


def test_class_weights_scale_whole_row_loss():
    # the combination reading: with uniform weights c the mean is unchanged and
    # the sum scales by c; every variant term is inside the weighted row loss
    h, w, b, t = problem(26, 20, 6, 15, bias=False)
    kw = dict(label_smoothing=0.1, z_loss=0.02)
    base_m = flce_reference(h, w, t, compute_grads=False, reduction="mean", **kw)["loss"]
    base_s = flce_reference(h, w, t, compute_grads=False, reduction="sum", **kw)["loss"]
    cw = np.full(15, 2.5)
    assert abs(flce_reference(h, w, t, compute_grads=False, reduction="mean", class_weight=cw, **kw)["loss"]
               - base_m) < 1e-12 * abs(base_m)
    assert abs(flce_reference(h, w, t, compute_grads=False, reduction="sum", class_weight=cw, **kw)["loss"]
               - 2.5 * base_s) < 1e-12 * abs(base_s)


# --------------------------------------------------------------------------- row argmax targets
# row_argmax_ids builds the peaked workload's "target = row argmax" rows; it is
# pinned to torch's argmax (first maximal index) of logits that torch computes
# itself, with a bias, a scale and a soft cap, and exact ties planted by
# duplicated weight rows.

def _torch_argmax(h, w, b, s, cap):
    logits = F.linear(torch.tensor(h), torch.tensor(w), None if b is None else torch.tensor(b)) * s
    if cap is not None:
        logits = cap * torch.tanh(logits / cap)
    return torch.argmax(logits, dim=1).numpy()


def test_row_argmax_ids_match_torch():
    h, w, b, _ = problem(31, 37, 10, 53, bias=True, wstd=0.8)
    b = b * 10.0                     # a bias large enough to move most rows' argmax
    w[41] = w[12]                    # exact ties between ids 12 and 41 (same row, same bias)
    b[41] = b[12]
    h[5] = w[12] * 3.0               # row 5 peaks on the tied pair
    for s, cap, bb in [(1.0, None, None), (1.0, None, b), (0.5, 2.0, b), (2.5, 30.0, b)]:
        got = orc.row_argmax_ids(h, w, bb, s, cap, row_block=8)
        np.testing.assert_array_equal(got, _torch_argmax(h, w, bb, s, cap))
    # the tie resolves to the smaller id
    assert orc.row_argmax_ids(h, w, b, 1.0, None)[5] == 12
    # zero weight: every row is an all-way tie, so every argmax is id 0
    assert np.all(orc.row_argmax_ids(h, np.zeros_like(w)) == 0)


def test_mutation_argmax_of_raw_logits_is_caught(monkeypatch):
    monkeypatch.setattr(orc, "transform_logits", lambda raw, bias, s, cap: raw)
    _pins_fail(test_row_argmax_ids_match_torch)


def test_mutation_argmax_without_bias_is_caught(monkeypatch):
    real = orc.transform_logits
    monkeypatch.setattr(orc, "transform_logits", lambda raw, bias, s, cap: real(raw, None, s, cap))
    _pins_fail(test_row_argmax_ids_match_torch)


# --------------------------------------------------------------------------- streaming reference
# streaming_reference serves shapes whose weight cannot be held in fp64 at
# once.  It is pinned to torch (logsumexp, cross_entropy, autograd) directly,
# with weight and token blocks that do not divide the sizes.

@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_streaming_reference_matches_torch(reduction):
    h, w, b, t = problem(41, 29, 12, 61, bias=True, ignore_frac=0.2, wstd=1.2)
    g = np.random.default_rng(3).standard_normal(29) if reduction == "none" else 0.8
    rows = [0, 4, 17, 28] + list(np.nonzero(t == -100)[0][:1])
    vids = [0, 7, int(t[t >= 0][0]), 60]
    for s, cap, bb in [(1.0, None, None), (0.6, 3.0, b), (1.0, None, b)]:
        out = orc.streaming_reference(h, lambda r0, r1: w[r0:r1], 61, t, rows, vids, bb,
                                      logit_scale=s, softcap=cap, reduction=reduction, grad_output=g,
                                      weight_block=7, row_block=5)
        th = torch.tensor(h)
        logits = F.linear(th, torch.tensor(w), None if bb is None else torch.tensor(bb)) * s
        if cap is not None:
            logits = cap * torch.tanh(logits / cap)
        np.testing.assert_allclose(out["lse"], torch.logsumexp(logits, dim=1).numpy(), rtol=1e-12)
        ref_loss, gh, gw, gb = torch_loss(h, w, bb, t, -100, s, cap, reduction, g)
        np.testing.assert_allclose(out["loss"], ref_loss, rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(out["grad_hidden"], gh[rows], rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(out["grad_weight"], gw[vids], rtol=1e-10, atol=1e-13)
        if bb is not None:
            np.testing.assert_allclose(out["grad_bias"], gb[vids], rtol=1e-10, atol=1e-13)
        else:
            assert out["grad_bias"] is None


def test_mutation_streaming_merge_without_rescale_is_caught(monkeypatch):
    def wrong(m, s, z):
        m_new = np.maximum(m, z.max(axis=1))
        return m_new, s + np.exp(z - m_new[:, None]).sum(axis=1)   # old sum not rescaled
    monkeypatch.setattr(orc, "_lse_merge", wrong)
    _pins_fail(lambda: test_streaming_reference_matches_torch("mean"))

