"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element, at sizes the oracle finishes in
seconds that still span several 256-wide tiles and ragged tails."""
import math

import numpy as np
import pytest
import torch

import flce_inputs as fi
from flce_testutil import (TOL, check_against_oracle, fill_argmax_targets, gpu_inputs, log_case,
                           oracle_inputs, to_np)
from oracle import flce_reference

pytestmark = pytest.mark.gpu


def run_case(w: fi.Workload, *, backward=True, bwd_vocab_chunk=0, fwd_tiles_per_split=0,
             grad_output=None, d=None, label_smoothing=0.0, z_loss=0.0, class_weight=None):
    import linear_cross_entropy_fwd_amd as flce
    log_case(f"{w.name} n={w.n} h={w.h} v={w.v} dtype={w.dtype} red={w.reduction} "
             f"chunk={bwd_vocab_chunk} tps={fwd_tiles_per_split} eps={label_smoothing} zl={z_loss} "
             f"cw={class_weight is not None}")
    if d is None:
        d = fill_argmax_targets(w, fi.generate(w))
    g = gpu_inputs(d)
    cw = None if class_weight is None else torch.as_tensor(class_weight, dtype=torch.float32).cuda()
    var = dict(label_smoothing=label_smoothing, z_loss=z_loss, class_weight=cw)
    pred = torch.empty(w.n, dtype=torch.int64, device="cuda") if w.return_metrics else None
    loss, lse, metrics = flce.flce_forward(
        g["hidden"], g["weight"], g["targets"], g["bias"], ignore_index=w.ignore_index,
        logit_scale=w.logit_scale, softcap=w.softcap, reduction=w.reduction,
        return_metrics=w.return_metrics, fwd_tiles_per_split=fwd_tiles_per_split,
        predictions=pred, **var)
    grads = None
    if backward:
        go = None if grad_output is None else torch.as_tensor(grad_output, dtype=torch.float32)
        grads = flce.flce_backward(
            g["hidden"], g["weight"], g["targets"], g["bias"], lse, go, ignore_index=w.ignore_index,
            logit_scale=w.logit_scale, softcap=w.softcap, reduction=w.reduction,
            bwd_vocab_chunk=bwd_vocab_chunk, **var)
    torch.cuda.synchronize()
    h, wt, t, b = oracle_inputs(d)
    ref = flce_reference(h, wt, t, b, ignore_index=w.ignore_index, logit_scale=w.logit_scale,
                         softcap=w.softcap, reduction=w.reduction, grad_output=grad_output,
                         compute_grads=backward, label_smoothing=label_smoothing, z_loss=z_loss,
                         class_weight=None if class_weight is None else np.asarray(class_weight, np.float64))
    out = check_against_oracle(w, d, ref, loss=loss, lse=lse, metrics=metrics, grads=grads,
                               what=w.name)
    if pred is not None and w.n > 0:
        # predicted tokens: the oracle's first-index argmax, except on near-ties
        from flce_testutil import TIE
        ties = ref["gap"] <= TIE[w.dtype] * np.maximum(1.0, np.abs(ref["lse"]))
        got = to_np(pred)
        assert np.all((got == ref["argmax"]) | ties), np.nonzero((got != ref["argmax"]) & ~ties)
    print("  errors:", out, flush=True)
    return loss, lse, metrics, grads, ref, d


W = fi.WORKLOADS


def test_tiny_f32_full_config():
    run_case(W["tiny_f32"])


def test_midvocab_shape_ragged_bf16():
    run_case(W["midvocab_bf16"].resized(n=300, h=256, v=3000))


def test_headvocab_shape_multichunk_bf16():
    run_case(W["headvocab_bf16"].resized(n=512, h=512, v=8200), bwd_vocab_chunk=2048)


@pytest.mark.parametrize("n,h,dtype,split", [(2304, 2048, "bf16", 1), (1030, 512, "bf16", 2),
                                             (1030, 512, "f32", 4), (4352, 1024, "f32", 2), (4352, 2048, "f32", 1)])
def test_grad_hidden_k_split_classes(n, h, dtype, split):
    """grad_hidden's grid (token tiles x hidden tiles) picks how many
    workgroups share each tile's K.  16-bit types, where grad_hidden shares
    its launches with the recompute and grad_weight: up to 64 tiles -> 2,
    more -> 1.  fp32, launched alone: up to 64 -> 4, up to 128 -> 2, more
    -> 1.  Each class against the oracle over several chunks."""
    tiles = -(-n // 256) * -(-h // 256)
    if dtype == "f32":
        assert split == (4 if tiles <= 64 else 2 if tiles <= 128 else 1)
    else:
        assert split == (2 if tiles <= 64 else 1)
    run_case(W["midvocab_bf16"].resized(n=n, h=h, v=1300, dtype=dtype), bwd_vocab_chunk=512)


@pytest.mark.parametrize("v,dtype", [(5000, "bf16"), (4700, "f16"), (4700, "f32")])
def test_grad_hidden_over_pairs_of_chunks(v, dtype):
    """16 chunks or more: grad_hidden runs once per pair of chunks (20
    chunks: ten pairs; 19: nine pairs and a last chunk alone)."""
    run_case(W["transforms_bf16"].resized(n=1030, h=256, v=v, dtype=dtype), bwd_vocab_chunk=256)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_default_plan_with_an_absorbed_last_chunk(dtype):
    """V = 3100 in default chunks of 1024 ids leaves 28 ids, which join the
    previous chunk (1052 ids); with 5 token tiles the 16-bit recompute kernel
    also writes W_c^T for that longer chunk."""
    run_case(W["transforms_bf16"].resized(n=1030, h=256, v=3100, dtype=dtype))


def test_transforms_shape_bias_scale_cap_sum_metrics():
    run_case(W["transforms_bf16"].resized(n=384, h=384, v=5000), bwd_vocab_chunk=1024)


def test_peaked_shape_none_forward_and_mean_backward():
    w = W["peaked_bf16"].resized(n=512, h=1024, v=4096)
    d = fill_argmax_targets(w, fi.generate(w))
    run_case(w.resized(reduction="none"), backward=False, d=d)
    run_case(w, d=d)


def test_f16_replica_of_midvocab():
    run_case(W["midvocab_bf16"].resized(n=320, h=256, v=2500, dtype="f16"))


def test_none_reduction_backward_with_row_gradients():
    w = W["transforms_bf16"].resized(n=200, h=128, v=1500, reduction="none", return_metrics=False)
    go = np.random.default_rng(0).standard_normal(200).astype(np.float32)
    run_case(w, grad_output=go)


@pytest.mark.parametrize("n", [1, 63, 65, 257])
def test_token_tails(n):
    run_case(W["tiny_f32"].resized(n=n, h=64, v=700))
    run_case(W["midvocab_bf16"].resized(n=n, h=128, v=1000))


@pytest.mark.parametrize("v", [1, 7, 255, 257, 32001])
def test_vocab_tails(v):
    run_case(W["headvocab_bf16"].resized(n=96, h=128, v=v, targets="uniform"))


@pytest.mark.parametrize("h,dtype", [(36, "f32"), (72, "bf16"), (200, "f16")])
def test_hidden_not_multiple_of_stage(h, dtype):
    run_case(W["midvocab_bf16"].resized(n=100, h=h, v=600, dtype=dtype))


# At least 4 token tiles: the recompute kernel itself writes the transposed
# weight chunk for grad_hidden (16-bit types).  Ragged hidden stage, ragged
# vocabulary tile in the last chunk, several chunks, exactly 4 and 5 tiles.
@pytest.mark.parametrize("n,h,v,dtype,chunk", [(1030, 200, 2600, "bf16", 1024),
                                               (1024, 328, 1800, "f16", 512),
                                               (1100, 256, 700, "bf16", 0)])
def test_many_token_tiles(n, h, v, dtype, chunk):
    run_case(W["transforms_bf16"].resized(n=n, h=h, v=v, dtype=dtype), bwd_vocab_chunk=chunk)


@pytest.mark.parametrize("tps,chunk", [(1, 256), (3, 768), (100, 0)])
def test_plan_overrides(tps, chunk):
    run_case(W["transforms_bf16"].resized(n=300, h=256, v=2600), fwd_tiles_per_split=tps,
             bwd_vocab_chunk=chunk)


def _random_configs(count, seed=20261202):
    """Seeded draws over sizes, dtypes and loss options (ragged N, H and V,
    plan overrides and every transform), for the sweep below."""
    rng = np.random.default_rng(seed)
    out = []
    for k in range(count):
        dtype = ["bf16", "f16", "f32"][k % 3]
        step = 4 if dtype == "f32" else 8  # a row must be whole 16-byte pieces
        n = int(rng.integers(1, 700))
        h = int(step * rng.integers(1, 66))
        v = int(rng.integers(1, 3200))
        cap = [None, 5.0, 30.0][int(rng.integers(0, 3))]
        bias = None if rng.random() < 0.5 else 0.1
        scale = [1.0, 0.5, 2.0][int(rng.integers(0, 3))]
        red = ["mean", "sum", "none"][int(rng.integers(0, 3))]
        metrics = bool(rng.random() < 0.5)
        ign = [0.0, 0.1][int(rng.integers(0, 2))]
        chunk = [0, 256, 512][int(rng.integers(0, 3))]
        tps = [0, 1, 2][int(rng.integers(0, 3))]
        go = rng.standard_normal(n).astype(np.float32) if red == "none" else None
        w = W["transforms_bf16"].resized(n=n, h=h, v=v, dtype=dtype, softcap=cap, bias_std=bias,
                                         logit_scale=scale, reduction=red, return_metrics=metrics,
                                         ignore_frac=ign, seed=1000 + k)
        out.append(pytest.param(w, chunk, tps, go, id=f"{k}-{dtype}-n{n}-h{h}-v{v}"))
    return out


@pytest.mark.parametrize("w,chunk,tps,go", _random_configs(24))
def test_random_configurations(w, chunk, tps, go):
    """A seeded sweep of random shapes and options against the oracle: the
    fixed cases above pin each feature, this one checks their combinations
    at sizes nobody picked by hand."""
    run_case(w, bwd_vocab_chunk=chunk, fwd_tiles_per_split=tps, grad_output=go)


def _random_default_plans(count, seed=20261203):
    """Seeded draws with larger vocabularies (4000 to 40000 ids) and the
    default plans: chunks of 4 to 40 tiles, rounded-up quarters of V, joined
    last chunks and forward split groups, at small N and H."""
    rng = np.random.default_rng(seed)
    out = []
    for k in range(count):
        dtype = ["bf16", "f16"][k % 2]
        n = int(rng.integers(1, 400))
        h = int(8 * rng.integers(1, 33))
        v = int(rng.integers(4000, 40001))
        w = W["midvocab_bf16"].resized(n=n, h=h, v=v, dtype=dtype, return_metrics=bool(k % 3 == 0),
                                       bias_std=0.1 if k % 4 == 1 else None, seed=2000 + k)
        out.append(pytest.param(w, id=f"{k}-{dtype}-n{n}-h{h}-v{v}"))
    return out


@pytest.mark.parametrize("w", _random_default_plans(6))
def test_random_default_plans(w):
    """The default backward chunking and forward splits at vocabularies the
    fixed cases do not reach, against the oracle."""
    run_case(w)


def test_ignore_index_edge_cases():
    base = W["tiny_f32"].resized(n=130, h=64, v=500)
    d = fi.generate(base)
    d_all = dict(d, targets=torch.full_like(d["targets"], -100))
    for red in ("mean", "sum", "none"):
        run_case(base.resized(reduction=red), d=d_all)
    d_none = dict(d, targets=d["targets"].clamp(min=0))
    run_case(base, d=d_none)
    # an ignore index that is also a valid id: rows whose target is 0 are ignored
    w0 = base.resized(ignore_index=0)
    d0 = dict(d, targets=torch.where(d["targets"] < 0, torch.zeros_like(d["targets"]), d["targets"]))
    run_case(w0, d=d0)


def test_empty_batch():
    import linear_cross_entropy_fwd_amd as flce
    log_case("N=0")
    h = torch.empty(0, 64, device="cuda")
    w = torch.randn(50, 64, device="cuda")
    t = torch.empty(0, dtype=torch.int64, device="cuda")
    b = torch.randn(50, device="cuda")
    loss, lse, m = flce.flce_forward(h, w, t, b, return_metrics=True)
    assert math.isnan(loss.item()) and torch.isnan(m).all()
    loss, _, _ = flce.flce_forward(h, w, t, b, reduction="sum")
    assert loss.item() == 0.0
    gh, gw, gb = flce.flce_backward(h, w, t, b, lse)
    assert gh.numel() == 0 and torch.all(gw == 0) and torch.all(gb == 0)


@pytest.mark.parametrize("cap,scale", [(5.0, 3.0), (30.0, 1.0), (0.5, 4.0)])
def test_softcap_f32_tight(cap, scale):
    """fp32 at the tight tolerance through the softcap (deep into tanh's
    saturation for the small caps), with metrics and both passes."""
    w = W["tiny_f32"].resized(n=300, h=64, v=700, softcap=cap, logit_scale=scale)
    run_case(w)
    run_case(w.resized(reduction="sum"), bwd_vocab_chunk=256)


# --------------------------------------------------------------------------- loss variants

def class_weights(v, seed):
    cw = np.random.default_rng(seed).uniform(0.2, 3.0, v).astype(np.float32)
    cw[::7] = 0.0
    return cw


@pytest.mark.parametrize("red", ["mean", "sum", "none"])
def test_variants_f32_tight(red):
    w = W["tiny_f32"].resized(n=200, h=64, v=700, reduction=red)
    run_case(w, label_smoothing=0.2, z_loss=1e-3, class_weight=class_weights(700, 1))
    run_case(w, label_smoothing=0.1)
    run_case(w, z_loss=0.01)
    run_case(w, class_weight=class_weights(700, 2))


def test_variants_bias_scale_cap_metrics():
    w = W["transforms_bf16"].resized(n=300, h=256, v=2600)
    run_case(w, label_smoothing=0.1, z_loss=1e-4, class_weight=class_weights(2600, 3), bwd_vocab_chunk=1024)
    run_case(w.resized(reduction="none"), label_smoothing=1.0, backward=False)


def test_variants_multichunk_and_fused_transpose():
    # several chunks, at least 4 token tiles (the recompute kernel writes W_c^T), f16
    w = W["headvocab_bf16"].resized(n=1030, h=200, v=2600, dtype="f16")
    run_case(w, label_smoothing=0.05, z_loss=2e-4, class_weight=class_weights(2600, 4), bwd_vocab_chunk=1024)


def test_variants_leave_plain_loss_bit_identical():
    import linear_cross_entropy_fwd_amd as flce
    w = W["midvocab_bf16"].resized(n=300, h=256, v=3000)
    d = fi.generate(w)
    g = gpu_inputs(d)
    args = (g["hidden"], g["weight"], g["targets"], g["bias"])
    a = flce.flce_forward(*args, reduction="sum")
    b = flce.flce_forward(*args, reduction="sum", label_smoothing=0.0, z_loss=0.0,
                          class_weight=torch.ones(3000, dtype=torch.float32, device="cuda"))
    ga = flce.flce_backward(*args, a[1], reduction="sum")
    gb = flce.flce_backward(*args, a[1], reduction="sum",
                            class_weight=torch.ones(3000, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(ga[0], gb[0]) and torch.equal(ga[1], gb[1])


# --------------------------------------------------------------------------- small fp32 path

@pytest.mark.parametrize("red", ["mean", "sum", "none"])
def test_small_fp32_path_and_tiled_path(red):
    """fp32 problems of at most 256 tokens (8192 ids, H <= 1024) run the small
    path with the default plan (the plan query reports one chunk); a plan
    override sends the same problem down the tiled path.  Both against the
    oracle with bias, scale, cap, metrics, predictions and, for none, per-row
    upstream gradients; then a single token with H = 4 and an odd V."""
    from linear_cross_entropy_fwd_amd import _abi
    w = W["transforms_bf16"].resized(n=256, h=128, v=3000, dtype="f32", reduction=red)
    assert _abi.flce_backward_plan(_abi.make_problem(w.n, w.h, w.v, _abi.F32, has_bias=True)) == (3000, 1, 3000)
    go = np.random.default_rng(5).standard_normal(w.n) if red == "none" else 0.7
    run_case(w, grad_output=go)
    run_case(w, grad_output=go, fwd_tiles_per_split=2, bwd_vocab_chunk=1024)
    run_case(W["tiny_f32"].resized(n=1, h=4, v=37, reduction=red))


# --------------------------------------------------------------------------- fp32 gradient output

@pytest.mark.parametrize("dtype,chunk", [("bf16", 1024), ("f16", 0)])
def test_fp32_grad_weight_output(dtype, chunk):
    """grad_weight_fp32 stores the same fp32 accumulators the 16-bit outputs
    are rounded from: rounding them to the input dtype (nearest even) gives
    the 16-bit gradients bit for bit, grad_hidden is untouched, and the fp32
    gradients meet the oracle at the 16-bit tolerance."""
    import linear_cross_entropy_fwd_amd as flce
    w = W["transforms_bf16"].resized(n=1030, h=200, v=2600, dtype=dtype)
    d = fill_argmax_targets(w, fi.generate(w))
    g = gpu_inputs(d)
    log_case(f"fp32 grads {w.name} n={w.n} h={w.h} v={w.v} dtype={dtype} chunk={chunk}")
    args = (g["hidden"], g["weight"], g["targets"], g["bias"])
    kw = dict(ignore_index=w.ignore_index, logit_scale=w.logit_scale, softcap=w.softcap,
              reduction=w.reduction)
    loss, lse, _ = flce.flce_forward(*args, **kw)
    g16 = flce.flce_backward(*args, lse, None, bwd_vocab_chunk=chunk, **kw)
    g32 = flce.flce_backward(*args, lse, None, bwd_vocab_chunk=chunk, grad_weight_fp32=True, **kw)
    torch.cuda.synchronize()
    assert g32[1].dtype == torch.float32 and g32[2].dtype == torch.float32
    assert torch.equal(g16[0], g32[0])
    assert torch.equal(g16[1], g32[1].to(g16[1].dtype))
    assert torch.equal(g16[2], g32[2].to(g16[2].dtype))
    h, wt, t, b = oracle_inputs(d)
    ref = flce_reference(h, wt, t, b, **kw)
    check_against_oracle(w, d, ref, loss=loss, lse=lse, grads=g32, what="fp32 grads")


def test_fp32_grad_weight_output_f32_inputs_and_empty():
    import linear_cross_entropy_fwd_amd as flce
    w = W["tiny_f32"].resized(n=300, h=64, v=700)
    d = fi.generate(w)
    g = gpu_inputs(d)
    args = (g["hidden"], g["weight"], g["targets"], g["bias"])
    _, lse, _ = flce.flce_forward(*args)
    a = flce.flce_backward(*args, lse)
    b = flce.flce_backward(*args, lse, grad_weight_fp32=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b) if x is not None)
    # no tokens: the fp32 gradients are zero-filled over their full size
    h = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    wt = torch.randn(700, 64, device="cuda").bfloat16()
    t = torch.empty(0, dtype=torch.int64, device="cuda")
    b = torch.randn(700, device="cuda").bfloat16()
    lse0 = torch.empty(0, dtype=torch.float32, device="cuda")
    gh, gw, gb = flce.flce_backward(h, wt, t, b, lse0, grad_weight_fp32=True)
    torch.cuda.synchronize()
    assert gh.numel() == 0
    assert gw.dtype == torch.float32 and gw.shape == (700, 64) and bool((gw == 0).all())
    assert gb.dtype == torch.float32 and gb.shape == (700,) and bool((gb == 0).all())


# --------------------------------------------------------------------------- one call

@pytest.mark.parametrize("wname,red,lse_out,g32", [("transforms_bf16", "sum", False, False),
                                                   ("transforms_bf16", "mean", False, True),
                                                   ("midvocab_bf16", "none", True, False),
                                                   ("tiny_f32", "mean", False, False)])
def test_forward_backward_in_one_call(wname, red, lse_out, g32):
    """flce_forward_backward gives the two calls' results bit for bit, and
    the oracle's within tolerance."""
    import linear_cross_entropy_fwd_amd as flce
    w = W[wname].resized(n=700, h=200 if wname != "tiny_f32" else 64, v=2600, reduction=red)
    log_case(f"one call {w.name} red={red} lse_out={lse_out}")
    d = fill_argmax_targets(w, fi.generate(w))
    g = gpu_inputs(d)
    args = (g["hidden"], g["weight"], g["targets"], g["bias"])
    kw = dict(ignore_index=w.ignore_index, logit_scale=w.logit_scale, softcap=w.softcap, reduction=red)
    go = torch.linspace(0.25, 2.0, w.n, device="cuda") if red == "none" else torch.tensor([0.75], device="cuda")
    var = dict(label_smoothing=0.1, z_loss=1e-4) if red != "none" else {}
    loss, lse, metrics, grads = flce.flce_forward_backward(*args, go, return_metrics=True, want_lse=lse_out,
                                                           bwd_vocab_chunk=1024, grad_weight_fp32=g32,
                                                           **var, **kw)
    loss2, lse2, metrics2 = flce.flce_forward(*args, return_metrics=True, **var, **kw)
    grads2 = flce.flce_backward(*args, lse2, go, bwd_vocab_chunk=1024, grad_weight_fp32=g32, **var, **kw)
    if g32:
        assert grads[1].dtype == torch.float32 and grads[2].dtype == torch.float32
    torch.cuda.synchronize()
    assert torch.equal(loss, loss2) and torch.equal(metrics, metrics2)
    assert (lse is None) != lse_out and (lse is None or torch.equal(lse, lse2))
    for a, b in zip(grads, grads2):
        assert (a is None and b is None) or torch.equal(a, b)
    h, wt, t, b = oracle_inputs(d)
    ref = flce_reference(h, wt, t, b, grad_output=to_np(go) if red == "none" else 0.75, **var, **kw)
    check_against_oracle(w, d, ref, loss=loss, lse=lse2, metrics=metrics, grads=grads, what="one call")
