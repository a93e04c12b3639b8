"""GPU tests of strided token layouts: hidden and targets passed as views
(the shifted hidden[:, :-1] / labels[:, 1:] of a causal-LM batch, a wider
row pitch, strided targets).  Each run is compared bit for bit with the same
call on contiguous copies (the kernels see the same operands either way) and
with the fp64 oracle on the compacted inputs."""
import numpy as np
import pytest
import torch

import flce_inputs as fi
from flce_testutil import check_against_oracle, log_case, to_np
from oracle import flce_reference

pytestmark = pytest.mark.gpu

W = fi.WORKLOADS


def _outputs(hidden, weight, targets, bias, *, reduction="mean", return_metrics=True, chunk=0, **kw):
    import linear_cross_entropy_fwd_amd as flce
    n = targets.numel()
    pred = torch.empty(n, dtype=torch.int64, device="cuda") if return_metrics else None
    loss, lse, metrics = flce.flce_forward(hidden, weight, targets, bias, reduction=reduction,
                                           return_metrics=return_metrics, predictions=pred, **kw)
    go = torch.linspace(0.5, 1.5, n, device="cuda") if reduction == "none" else None
    grads = flce.flce_backward(hidden, weight, targets, bias, lse, go, reduction=reduction,
                               bwd_vocab_chunk=chunk, **kw)
    torch.cuda.synchronize()
    return dict(loss=loss, lse=lse, metrics=metrics, pred=pred, gh=grads[0], gw=grads[1], gb=grads[2]), go


def _assert_same(a, b):
    for k in a:
        if a[k] is None:
            assert b[k] is None, k
            continue
        x, y = a[k], b[k]
        if k == "gh":
            x, y = x.reshape(-1, x.shape[-1]), y.reshape(-1, y.shape[-1])
        assert torch.equal(x, y) or (x.is_floating_point() and torch.equal(torch.isnan(x), torch.isnan(y))
                                     and torch.equal(x.nan_to_num(), y.nan_to_num())), k


def _oracle_check(w, hidden_c, weight, targets_c, bias, out, go, reduction, **kw):
    w = w.resized(reduction=reduction)
    h = to_np(hidden_c).reshape(-1, hidden_c.shape[-1])
    t = to_np(targets_c).reshape(-1)
    ref = flce_reference(h, to_np(weight), t, None if bias is None else to_np(bias),
                         reduction=reduction, grad_output=None if go is None else to_np(go), **kw)
    d = {"targets": targets_c.reshape(-1)}
    gh = out["gh"].reshape(-1, out["gh"].shape[-1])
    return check_against_oracle(w, d, ref, loss=out["loss"], lse=out["lse"], metrics=out["metrics"],
                                grads=(gh, out["gw"], out["gb"]), what="layout")


@pytest.mark.parametrize("dtype,s,t,h,v,bias,chunk", [
    ("bf16", 3, 300, 200, 2600, False, 1024),   # ragged sequences, several chunks
    ("f16", 2, 129, 64, 1000, True, 0),         # bias, sequences shorter than a tile
    ("f32", 4, 40, 36, 700, True, 0),           # fp32 tile path
])
def test_shifted_views_of_a_batch(dtype, s, t, h, v, bias, chunk):
    """hidden[:, :-1] and labels[:, 1:] of an (S, T+1) batch."""
    w = W["transforms_bf16" if bias else "midvocab_bf16"].resized(n=s * (t + 1), h=h, v=v, dtype=dtype)
    log_case(f"shifted views {dtype} S={s} T={t} H={h} V={v} bias={bias} chunk={chunk}")
    d = fi.generate(w)
    hid = d["hidden"].cuda().view(s, t + 1, h)
    lab = d["targets"].cuda().view(s, t + 1)
    wt = d["weight"].cuda()
    b = d["bias"].cuda() if d["bias"] is not None else None
    hv, tv = hid[:, :-1], lab[:, 1:]
    assert not hv.is_contiguous() and not tv.is_contiguous()
    kw = dict(ignore_index=w.ignore_index, logit_scale=w.logit_scale, softcap=w.softcap)
    for red in ("mean", "none"):
        got, go = _outputs(hv, wt, tv, b, reduction=red, chunk=chunk, **kw)
        want, _ = _outputs(hv.contiguous(), wt, tv.contiguous(), b, reduction=red, chunk=chunk, **kw)
        _assert_same(got, want)
        print("  errors:", _oracle_check(w, hv, wt, tv, b, got, go, red, **kw), flush=True)
    assert got["gh"].shape == hv.shape


def test_wider_row_pitch_and_strided_targets():
    """A wider row pitch and strided targets give the contiguous call's results."""
    w = W["transforms_bf16"].resized(n=700, h=200, v=2600)
    log_case("row pitch 264, target stride 3")
    d = fi.generate(w)
    wide = torch.zeros(700, 264, dtype=torch.bfloat16, device="cuda")
    wide[:, :200] = d["hidden"].cuda()
    hv = wide[:, :200]
    tbig = torch.full((2100,), -7, dtype=torch.int64, device="cuda")
    tbig[::3] = d["targets"].cuda()
    tv = tbig[::3]
    wt, b = d["weight"].cuda(), d["bias"].cuda()
    kw = dict(ignore_index=w.ignore_index, logit_scale=w.logit_scale, softcap=w.softcap)
    got, _ = _outputs(hv, wt, tv, b, chunk=1024, **kw)
    want, _ = _outputs(hv.contiguous(), wt, tv.contiguous(), b, chunk=1024, **kw)
    _assert_same(got, want)
    print("  errors:", _oracle_check(w, hv, wt, tv, b, got, None, "mean", **kw), flush=True)


def test_sequences_back_to_back_at_a_wider_row_pitch():
    """(S, T, H) views of an (N, H+8) buffer."""
    import linear_cross_entropy_fwd_amd as flce
    w = W["midvocab_bf16"].resized(n=4 * 90, h=128, v=1500)
    log_case("S=4 T=90 row pitch 136")
    d = fi.generate(w)
    buf = torch.zeros(360, 136, dtype=torch.bfloat16, device="cuda")
    buf[:, :128] = d["hidden"].cuda()
    hv = buf.view(4, 90, 136)[:, :, :128]
    lay = flce.token_layout(hv, d["targets"].cuda().view(4, 90))
    assert lay["hidden_seq_stride"] == 90 * lay["hidden_row_stride"]
    tv = d["targets"].cuda().view(4, 90)
    wt = d["weight"].cuda()
    got, _ = _outputs(hv, wt, tv, None)
    want, _ = _outputs(hv.contiguous(), wt, tv, None)
    _assert_same(got, want)


def test_row_pitch_of_16_mib():
    """A row pitch past what 32-bit tile offsets could reach (rows are
    gathered with 64-bit addresses)."""
    w = W["midvocab_bf16"].resized(n=5, h=64, v=700)
    log_case("row pitch 16 MiB")
    d = fi.generate(w)
    pitch = 1 << 23   # elements: 16 MiB of bf16
    store = torch.zeros(4 * pitch + 64, dtype=torch.bfloat16, device="cuda")
    hv = store.as_strided((5, 64), (pitch, 1))
    hv.copy_(d["hidden"].cuda())
    tv = d["targets"].cuda()
    wt = d["weight"].cuda()
    got, _ = _outputs(hv, wt, tv, None)
    want, _ = _outputs(hv.contiguous(), wt, tv, None)
    _assert_same(got, want)


def test_autograd_through_shifted_views():
    import linear_cross_entropy_fwd_amd as flce
    w = W["midvocab_bf16"].resized(n=2 * 301, h=128, v=3000)
    log_case("autograd, shifted views S=2 T=300")
    d = fi.generate(w)
    hid = d["hidden"].cuda().view(2, 301, 128).clone().requires_grad_(True)
    lab = d["targets"].cuda().view(2, 301)
    wt = d["weight"].cuda().clone().requires_grad_(True)
    loss = flce.fused_linear_cross_entropy(hid[:, :-1], wt, lab[:, 1:])
    loss.backward()
    hid2 = hid.detach()[:, :-1].contiguous().requires_grad_(True)
    wt2 = wt.detach().clone().requires_grad_(True)
    loss2 = flce.fused_linear_cross_entropy(hid2, wt2, lab[:, 1:].contiguous())
    loss2.backward()
    torch.cuda.synchronize()
    assert torch.equal(loss, loss2)
    assert torch.equal(hid.grad[:, :-1], hid2.grad)
    assert bool((hid.grad[:, -1] == 0).all())
    assert torch.equal(wt.grad, wt2.grad)
    ref = flce_reference(to_np(hid2).reshape(-1, 128), to_np(wt2), to_np(lab[:, 1:]).reshape(-1))
    assert abs(loss.item() - ref["loss"]) <= 2e-3 * abs(ref["loss"])
    gw = to_np(wt.grad)
    assert np.max(np.abs(gw - ref["grad_weight"])) <= 2e-2 * np.max(np.abs(ref["grad_weight"]))
