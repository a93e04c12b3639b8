"""GPU parity of vocabulary shards, the single-device part of a
vocabulary-parallel loss: each shard's forward and backward through the C
ABI, the combine of the shards' per-row outputs, and the whole against the
fp64 oracle.  One shard covering the vocabulary must reproduce the unsharded
path bit for bit."""
import numpy as np
import pytest
import torch

import flce_inputs as fi
from flce_testutil import TIE, TOL, gpu_inputs, log_case, maxnorm_rel, oracle_inputs, rel_err, to_np
from oracle import flce_reference

pytestmark = pytest.mark.gpu

W = fi.WORKLOADS


def shard_pass(w, g, bounds, *, grad_output=None, bwd_vocab_chunk=0, fwd_tiles_per_split=0, backward=True,
               predictions=None):
    """Every shard's forward, the combine, then every shard's backward with the
    combined lse; grad_hidden summed over the shards in fp32, in shard order.
    Returns (shard_lse, target_logit, loss, lse, grads, metrics or None)."""
    import linear_cross_entropy_fwd_amd as flce
    kw = dict(ignore_index=w.ignore_index, logit_scale=w.logit_scale, softcap=w.softcap)
    V = w.v
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        bias = None if g["bias"] is None else g["bias"][a:b]
        parts.append(flce.flce_forward_shard(g["hidden"], g["weight"][a:b], g["targets"], bias, vocab_offset=a,
                                             vocab_total=V, fwd_tiles_per_split=fwd_tiles_per_split,
                                             return_metrics=w.return_metrics, **kw))
    slse = torch.stack([p[0] for p in parts])
    stl = torch.stack([p[1] for p in parts])
    sm = tuple(torch.stack([p[i] for p in parts]) for i in (2, 3, 4)) if w.return_metrics else None
    loss, lse, metrics = flce.flce_combine_shards(slse, stl, g["targets"], V, ignore_index=w.ignore_index,
                                                  reduction=w.reduction, shard_metrics=sm, predictions=predictions)
    grads = None
    if backward:
        go = None if grad_output is None else torch.as_tensor(grad_output, dtype=torch.float32)
        gh, gws, gbs = None, [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            bias = None if g["bias"] is None else g["bias"][a:b]
            gh_k, gw_k, gb_k = flce.flce_backward(g["hidden"], g["weight"][a:b], g["targets"], bias, lse, go,
                                                  reduction=w.reduction, bwd_vocab_chunk=bwd_vocab_chunk,
                                                  grad_hidden_fp32=True, vocab_offset=a, vocab_total=V, **kw)
            gh = gh_k if gh is None else gh + gh_k
            gws.append(gw_k)
            gbs.append(gb_k)
        grads = (gh, torch.cat(gws), None if g["bias"] is None else torch.cat(gbs))
    return slse, stl, loss, lse, grads, metrics


def run_shards(w, bounds, *, grad_output=None, bwd_vocab_chunk=0, fwd_tiles_per_split=0, d=None):
    log_case(f"shards {list(bounds)} of {w.name} n={w.n} h={w.h} v={w.v} dtype={w.dtype} red={w.reduction} "
             f"chunk={bwd_vocab_chunk} tps={fwd_tiles_per_split}")
    assert bounds[0] == 0 and bounds[-1] == w.v
    if d is None:
        d = fi.generate(w)
    g = gpu_inputs(d)
    pred = torch.empty(w.n, dtype=torch.int64, device="cuda") if w.return_metrics else None
    slse, stl, loss, lse, (gh, gw, gb), metrics = shard_pass(w, g, bounds, grad_output=grad_output,
                                                             bwd_vocab_chunk=bwd_vocab_chunk,
                                                             fwd_tiles_per_split=fwd_tiles_per_split,
                                                             predictions=pred)
    torch.cuda.synchronize()
    h, wt, t, bb = oracle_inputs(d)
    okw = dict(ignore_index=w.ignore_index, logit_scale=w.logit_scale, softcap=w.softcap)
    ref = flce_reference(h, wt, t, bb, reduction=w.reduction, grad_output=grad_output, **okw)
    tol = TOL[w.dtype]
    valid = t != w.ignore_index
    # the plain loss of a valid row is lse - z_t, so a target logit is compared
    # at the scale of the row losses it enters with weight 1
    zt = ref["lse"] - ref["row_loss"]
    zt_scale = max(float(np.max(np.abs(ref["row_loss"][valid]))) if valid.any() else 0.0, 1e-30)
    errs = {}
    for k, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        rs = flce_reference(h, wt[a:b], np.full_like(t, w.ignore_index), None if bb is None else bb[a:b],
                            compute_grads=False, **okw)
        errs[f"lse{k}"] = maxnorm_rel(to_np(slse[k]), rs["lse"])
        assert errs[f"lse{k}"] <= tol["loss"], errs
        own = valid & (t >= a) & (t < b)
        got = to_np(stl[k])
        assert np.all(got[~own] == 0.0), np.nonzero(got[~own])
        errs[f"zt{k}"] = float(np.max(np.abs(got[own] - zt[own]))) / zt_scale if own.any() else 0.0
        assert errs[f"zt{k}"] <= tol["loss"], errs
    if w.reduction == "none":
        errs["loss"] = maxnorm_rel(to_np(loss), ref["loss"])
    else:
        errs["loss"] = rel_err(loss.item(), ref["loss"])
    errs["lse"] = maxnorm_rel(to_np(lse), ref["lse"])
    assert errs["loss"] <= tol["loss"] and errs["lse"] <= tol["loss"], errs
    if w.return_metrics:
        # metrics as the unsharded path is checked: entropy at the loss tolerance,
        # hits and predicted ids exact away from near-ties of the top two logits
        m = to_np(metrics)
        ties = ref["gap"] <= TIE[w.dtype] * np.maximum(1.0, np.abs(ref["lse"]))
        errs["entropy"] = rel_err(m[1], ref["entropy"])
        assert errs["entropy"] <= tol["loss"], errs
        gpu_hits, ref_hits = int(round(float(m[0]) * ref["n_valid"])), int(ref["hit"].sum())
        assert abs(gpu_hits - ref_hits) <= int((ties & valid).sum()), (gpu_hits, ref_hits)
        got_pred = to_np(pred)
        assert np.all((got_pred == ref["argmax"]) | ties), np.nonzero((got_pred != ref["argmax"]) & ~ties)
    for name, got, r in (("grad_hidden", gh, ref["grad_hidden"]), ("grad_weight", gw, ref["grad_weight"]),
                         ("grad_bias", gb, ref["grad_bias"])):
        if r is None:
            continue
        errs[name] = maxnorm_rel(to_np(got), r)
        assert errs[name] <= tol["grad"], (name, errs)
    print("  errors:", errs, flush=True)


def test_two_shards_bf16_transforms():
    w = W["transforms_bf16"].resized(n=300, h=256, v=2600, reduction="mean")
    run_shards(w, [0, 1000, 2600])


def test_three_shards_f16_with_a_one_id_shard():
    w = W["headvocab_bf16"].resized(n=413, h=200, v=2600, dtype="f16", reduction="sum")
    run_shards(w, [0, 300, 301, 2600])


def test_shards_f32_none_reduction_with_upstream_gradient():
    w = W["transforms_bf16"].resized(n=290, h=132, v=2600, dtype="f32", reduction="none")
    go = np.random.default_rng(5).standard_normal(w.n).astype(np.float32)
    run_shards(w, [0, 1300, 2600], grad_output=go)


def test_shards_with_several_chunks_and_splits_each():
    w = W["midvocab_bf16"].resized(n=700, h=200, v=6000)
    run_shards(w, [0, 2048, 4096, 6000], bwd_vocab_chunk=512, fwd_tiles_per_split=1)


def test_shards_with_unequal_sizes_and_ragged_tokens():
    w = W["peaked_bf16"].resized(n=1030, h=256, v=5003, softcap=30.0)
    run_shards(w, [0, 17, 2500, 2501, 5003])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_shard_is_the_unsharded_path_bit_for_bit(dtype):
    """A single shard of the whole vocabulary runs the same kernels on the
    same ids: its lse, loss, accuracy and gradients equal flce_forward /
    flce_backward's bits (grad_hidden in fp32 rounds to the unsharded dtype
    output)."""
    import linear_cross_entropy_fwd_amd as flce
    w = W["transforms_bf16"].resized(n=300, h=256, v=2600, dtype=dtype, reduction="mean")
    log_case(f"one shard against the unsharded path, {dtype}")
    d = fi.generate(w)
    g = gpu_inputs(d)
    kw = dict(ignore_index=w.ignore_index, logit_scale=w.logit_scale, softcap=w.softcap)
    slse, stl, loss_s, lse_s, (gh_s, gw_s, gb_s), metrics_s = shard_pass(w, g, [0, w.v])
    loss, lse, metrics = flce.flce_forward(g["hidden"], g["weight"], g["targets"], g["bias"],
                                           reduction=w.reduction, return_metrics=True, **kw)
    gh, gw, gb = flce.flce_backward(g["hidden"], g["weight"], g["targets"], g["bias"], lse, reduction=w.reduction,
                                    **kw)
    torch.cuda.synchronize()
    assert torch.equal(slse[0], lse) and torch.equal(lse_s, lse)
    assert torch.equal(loss_s, loss)
    assert torch.equal(gw_s, gw) and torch.equal(gb_s, gb)
    assert gh_s.dtype == torch.float32 and torch.equal(gh_s.to(gh.dtype), gh)
    # the same argmax, so the same accuracy; the entropy formed as lse - (lse_0 - H_0)
    # rounds differently from the unsharded log S - U/S
    assert metrics_s[0].item() == metrics[0].item()
    assert rel_err(metrics_s[1].item(), metrics[1].item()) <= 1e-5


def test_grad_hidden_fp32_rounds_to_the_dtype_output():
    """grad_hidden_fp32 on the unsharded path, in the one-launch backward's
    K-split class (2 x 1 tiles: a separate sum writes grad_hidden) and without
    the split (9 x 8 tiles: the last launch writes it): the fp32 output
    rounded to the dtype (nearest even) is the dtype output."""
    import linear_cross_entropy_fwd_amd as flce
    for n, h, v in ((300, 256, 2600), (2304, 2048, 3000)):
        w = W["midvocab_bf16"].resized(n=n, h=h, v=v)
        log_case(f"grad_hidden_fp32 n={n} h={h} v={v}")
        g = gpu_inputs(fi.generate(w))
        _, lse, _ = flce.flce_forward(g["hidden"], g["weight"], g["targets"], None)
        gh, _, _ = flce.flce_backward(g["hidden"], g["weight"], g["targets"], None, lse, need_weight=False)
        gh32, _, _ = flce.flce_backward(g["hidden"], g["weight"], g["targets"], None, lse, need_weight=False,
                                        grad_hidden_fp32=True)
        torch.cuda.synchronize()
        assert gh32.dtype == torch.float32 and torch.equal(gh32.to(gh.dtype), gh)


def test_strided_tokens_with_shards_match_contiguous():
    """Shards read the (S, T+1) views of a causal batch in place: the same bits
    as the shards on contiguous copies."""
    w = W["midvocab_bf16"].resized(n=4 * 130, h=128, v=2600)
    log_case("shards on strided token views")
    d = fi.generate(w)
    g = gpu_inputs(d)
    S, T = 4, 130
    hid = torch.zeros(S, T + 1, w.h, dtype=g["hidden"].dtype, device="cuda")
    hid[:, :-1] = g["hidden"].view(S, T, w.h)
    lab = torch.full((S, T + 1), 7, dtype=torch.int64, device="cuda")
    lab[:, 1:] = g["targets"].view(S, T)
    gs = dict(g, hidden=hid[:, :-1], targets=lab[:, 1:])
    bounds = [0, 1111, 2600]
    a = shard_pass(w, g, bounds)
    b = shard_pass(w, gs, bounds)
    torch.cuda.synchronize()
    for x, y in ((a[0], b[0]), (a[1], b[1]), (a[2], b[2]), (a[3], b[3])):
        assert torch.equal(x, y)
    assert a[5] is None and b[5] is None
    for x, y in zip(a[4], b[4]):
        if x is not None:
            assert torch.equal(x.reshape(y.shape), y)


def test_out_of_range_target_with_shards():
    """A target outside the whole vocabulary: NaN in every shard's target
    logit and in the combined row loss, the combine's status bit set; a
    target of another shard is not out of range."""
    import linear_cross_entropy_fwd_amd as flce
    from linear_cross_entropy_fwd_amd import _abi
    w = W["midvocab_bf16"].resized(n=64, h=128, v=1000, reduction="none")
    log_case("out-of-range target with shards")
    d = fi.generate(w)
    g = gpu_inputs(d)
    g["targets"][5] = w.v + 3
    g["targets"][6] = 999
    slse, stl, loss, lse, _, _ = shard_pass(w, g, [0, 500, 1000], backward=False)
    torch.cuda.synchronize()
    assert torch.isnan(stl[:, 5]).all() and torch.isnan(loss[5])
    assert stl[0, 6].item() == 0.0 and torch.isfinite(stl[1, 6]) and torch.isfinite(loss[6])
    others = torch.ones(w.n, dtype=torch.bool, device="cuda")
    others[5] = False
    assert torch.isfinite(loss[others]).all() and torch.isfinite(lse).all()
    # the combine's status word (a workspace of its own)
    p = _abi.make_problem(w.n, 8, w.v, _abi.BF16, "none", w.ignore_index)
    ws = torch.empty(_abi.flce_combine_shards_workspace_size(p), dtype=torch.uint8, device="cuda")
    loss2 = torch.empty(w.n, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    _abi.check(_abi.flce_combine_shards(p, 2, slse.data_ptr(), stl.data_ptr(), 0, 0, 0, g["targets"].data_ptr(),
                                        loss2.data_ptr(), 0, 0, ws.data_ptr(), ws.numel(), stream))
    assert _abi.flce_forward_status(p, ws.data_ptr(), stream) == 1
    assert torch.equal(loss2.nan_to_num(), loss.nan_to_num())


def test_head_shape_shard_lse_matches_the_plain_forward_on_its_rows():
    """One eighth of the head-shape vocabulary (ids 16032..32063 of 128256),
    at its real size: the shard's lse equals the plain forward's lse over the
    same weight rows bit for bit (the same kernels and splits), and its
    target logits are 0 off the shard and give the plain row loss on it."""
    import linear_cross_entropy_fwd_amd as flce
    w = W["headvocab_bf16"]
    log_case("head-shape shard 1 of 8")
    g = fi.generate(w, device="cuda")
    a, b = 16032, 32064
    slse, stl = flce.flce_forward_shard(g["hidden"], g["weight"][a:b], g["targets"], None, vocab_offset=a,
                                        vocab_total=w.v)
    t = g["targets"]
    own = (t >= a) & (t < b)
    local = torch.where(own, t - a, torch.full_like(t, w.ignore_index))
    loss, lse, _ = flce.flce_forward(g["hidden"], g["weight"][a:b], local, None, reduction="none")
    torch.cuda.synchronize()
    assert torch.equal(slse, lse)
    assert torch.equal(stl[~own], torch.zeros_like(stl[~own]))
    assert torch.equal((slse - stl)[own], loss[own])  # the plain row loss is lse - z_t, rounded once


def _random_shard_configs(count, seed=20261204):
    """Seeded draws over sizes, dtypes, options and shard bounds (1 to 5
    shards of random, unequal sizes, one-id shards included)."""
    rng = np.random.default_rng(seed)
    out = []
    for k in range(count):
        dtype = ["bf16", "f16", "f32"][k % 3]
        step = 4 if dtype == "f32" else 8
        n = int(rng.integers(1, 600))
        h = int(step * rng.integers(1, 50))
        v = int(rng.integers(2, 4000))
        n_sh = int(rng.integers(1, 6))
        cuts = sorted(set(int(c) for c in rng.integers(1, v, size=n_sh - 1))) if n_sh > 1 else []
        bounds = [0] + cuts + [v]
        w = W["transforms_bf16"].resized(
            n=n, h=h, v=v, dtype=dtype, softcap=[None, 5.0, 30.0][int(rng.integers(0, 3))],
            bias_std=None if rng.random() < 0.5 else 0.1, logit_scale=[1.0, 0.5, 2.0][int(rng.integers(0, 3))],
            reduction=["mean", "sum", "none"][int(rng.integers(0, 3))], return_metrics=bool(rng.random() < 0.5),
            ignore_frac=[0.0, 0.1][int(rng.integers(0, 2))], seed=3000 + k)
        go = rng.standard_normal(n).astype(np.float32) if w.reduction == "none" else None
        out.append(pytest.param(w, bounds, go, id=f"{k}-{dtype}-n{n}-h{h}-v{v}-s{len(bounds) - 1}"))
    return out


@pytest.mark.parametrize("w,bounds,go", _random_shard_configs(10))
def test_random_shard_configurations(w, bounds, go):
    """Shards of random shapes and options against the oracle."""
    run_shards(w, bounds, grad_output=go)
