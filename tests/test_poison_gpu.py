"""GPU debug checks of memory discipline, through the C ABI.

Workspace poison: each configuration runs twice, once with its workspaces
filled with zero bytes and once with 0xFF bytes (NaN for fp32 words, -1 for
integers).  Every output must be bit-identical between the two runs, so no
kernel reads a workspace byte that the same call has not written first (a
stale or uninitialised read would turn into NaN or a changed value).

Output canaries: every output buffer (loss, lse, metrics, predictions,
grad_hidden, grad_weight, grad_bias) sits between two 4 KiB guard regions
filled with 0xA5; after the calls the guards must be unchanged, so no kernel
writes before or past its outputs.

The configurations cover the one-launch 16-bit backward (several chunks,
pairs of chunks), the f16 path with every loss variant and per-row upstream
gradients, the fp32 tiled path, the small fp32 path and a strided token
layout that is gathered into the workspace."""
import numpy as np
import pytest
import torch

import flce_inputs as fi
from flce_testutil import gpu_inputs, log_case

pytestmark = pytest.mark.gpu

W = fi.WORKLOADS
PAD = 4096      # guard bytes on each side (keeps 16-byte alignment)
GUARD = 0xA5


def _padded(nbytes):
    buf = torch.full((nbytes + 2 * PAD,), GUARD, dtype=torch.uint8, device="cuda")
    return buf, buf.data_ptr() + PAD


def _run(case, fill):
    """One forward + backward with workspaces full of `fill`; returns the output bytes."""
    from linear_cross_entropy_fwd_amd import _abi
    g, w, kw, layout, hidden, targets = case["g"], case["w"], case["kw"], case["layout"], case["hidden"], case["targets"]
    n, v, h = w.n, w.v, w.h
    eb = hidden.element_size()
    geb = 4 if kw.get("grad_weight_fp32") else eb
    sizes = {"loss": 4 * (n if w.reduction == "none" else 1), "lse": 4 * n,
             "metrics": 8 if w.return_metrics else 0, "pred": 8 * n if w.return_metrics else 0,
             "gh": n * h * eb, "gw": v * h * geb, "gb": v * geb if g["bias"] is not None else 0}
    bufs = {k: _padded(s) for k, s in sizes.items() if s}
    ptr = lambda k: bufs[k][1] if k in bufs else 0
    cw = case.get("cw")
    p = _abi.make_problem(n, h, v, _abi.BF16 if hidden.dtype == torch.bfloat16 else
                          _abi.F16 if hidden.dtype == torch.float16 else _abi.F32,
                          w.reduction, w.ignore_index, w.logit_scale, w.softcap, w.return_metrics,
                          g["bias"] is not None, class_weight=0 if cw is None else cw.data_ptr(),
                          predictions=ptr("pred"), **kw, **layout)
    fs, bs = _abi.flce_forward_workspace_size(p), _abi.flce_backward_workspace_size(p)
    ws_f = torch.full((max(fs, 1),), fill, dtype=torch.uint8, device="cuda")
    ws_b = torch.full((max(bs, 1),), fill, dtype=torch.uint8, device="cuda")
    gl = case.get("grad_loss")
    st = torch.cuda.current_stream().cuda_stream
    b = 0 if g["bias"] is None else g["bias"].data_ptr()
    _abi.check(_abi.flce_forward(p, hidden.data_ptr(), g["weight"].data_ptr(), targets.data_ptr(), b,
                                 ptr("loss"), ptr("lse"), ptr("metrics"), ws_f.data_ptr(), fs, st))
    _abi.check(_abi.flce_backward(p, hidden.data_ptr(), g["weight"].data_ptr(), targets.data_ptr(), b,
                                  ptr("lse"), 0 if gl is None else gl.data_ptr(), ptr("gh"), ptr("gw"),
                                  ptr("gb"), ws_b.data_ptr(), bs, st))
    torch.cuda.synchronize()
    out = {}
    for k, (buf, _) in bufs.items():
        host = buf.cpu()
        s = sizes[k]
        assert torch.all(host[:PAD] == GUARD), f"{case['name']}: write before {k}"
        assert torch.all(host[PAD + s:] == GUARD), f"{case['name']}: write past {k}"
        out[k] = host[PAD:PAD + s].clone()
    return out


def _cases():
    out = []

    def add(name, w, kw=None, grad_loss=None, cw=None, strided=False):
        out.append(dict(name=name, w=w, kw=kw or {}, grad_loss=grad_loss, cw=cw, strided=strided))

    add("bf16 one-launch steps, bias/scale/cap/metrics", W["transforms_bf16"].resized(n=700, h=256, v=2600))
    add("bf16 pairs of chunks", W["headvocab_bf16"].resized(n=1030, h=256, v=5000), dict(bwd_vocab_chunk=256))
    add("f16 none, every variant", W["midvocab_bf16"].resized(n=600, h=128, v=3000, dtype="f16", reduction="none"),
        dict(label_smoothing=0.1, z_loss=1e-3), grad_loss="rows", cw=True)
    add("fp32 tiled path", W["tiny_f32"].resized(n=300, h=64, v=700), dict(grad_weight_fp32=0))
    add("fp32 small path, bias/cap/metrics", W["transforms_bf16"].resized(n=200, h=64, v=700, dtype="f32"))
    add("bf16 strided tokens (gathered)", W["midvocab_bf16"].resized(n=520, h=128, v=2600), strided=True)
    add("bf16 fp32 grad_weight", W["transforms_bf16"].resized(n=300, h=128, v=2600), dict(grad_weight_fp32=1))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_workspace_poison_and_output_canaries(case):
    import linear_cross_entropy_fwd_amd as flce
    w = case["w"]
    log_case(f"poison/canary: {case['name']} n={w.n} h={w.h} v={w.v} dtype={w.dtype} red={w.reduction}")
    g = gpu_inputs(fi.generate(w))
    hidden, targets = g["hidden"], g["targets"]
    if case["strided"]:
        # (S, T+1, H) and (S, T+1) batches and their shifted views of T = 26 tokens a sequence
        s_, t_ = 20, w.n // 20
        big_h = torch.zeros(s_, t_ + 1, w.h, dtype=hidden.dtype, device="cuda")
        big_h[:, :-1] = hidden.view(s_, t_, w.h)
        big_t = torch.full((s_, t_ + 1), w.ignore_index, dtype=torch.int64, device="cuda")
        big_t[:, 1:] = targets.view(s_, t_)
        hidden, targets = big_h[:, :-1], big_t[:, 1:]
        case["layout"] = flce.token_layout(hidden, targets)
        assert case["layout"]["hidden_seq_stride"] != 0
    else:
        case["layout"] = {}
    if case["cw"] is True:
        case["cw"] = torch.from_numpy(np.random.default_rng(3).uniform(0.2, 3.0, w.v).astype(np.float32)).cuda()
    if case["grad_loss"] == "rows":
        case["grad_loss"] = torch.from_numpy(np.random.default_rng(4).standard_normal(w.n).astype(np.float32)).cuda()
    case.update(g=g, hidden=hidden, targets=targets)
    a = _run(case, 0x00)
    b = _run(case, 0xFF)
    for k in a:
        assert torch.equal(a[k], b[k]), f"{case['name']}: {k} depends on stale workspace bytes"
    assert a["gh"].numel() > 0 and bool(torch.any(a["gh"] != 0))


def _run_shards(g, w, bounds, fill):
    """Two-level vocabulary-shard pass through the C ABI (each shard's forward
    with metrics, the combine, each shard's backward with fp32 grad_hidden),
    workspaces full of `fill`, every output between guards; returns the bytes."""
    from linear_cross_entropy_fwd_amd import _abi
    n, h, V = w.n, w.h, w.v
    eb = g["hidden"].element_size()
    dt = _abi.BF16 if g["hidden"].dtype == torch.bfloat16 else _abi.F16
    P = len(bounds) - 1
    st = torch.cuda.current_stream().cuda_stream
    sizes = {"slse": 4 * P * n, "stl": 4 * P * n, "smax": 4 * P * n, "sarg": 8 * P * n, "sent": 4 * P * n,
             "loss": 4, "lse": 4 * n, "metrics": 8, "pred": 8 * n}
    for k, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        sizes[f"gh{k}"] = 4 * n * h
        sizes[f"gw{k}"] = (b - a) * h * eb
        sizes[f"gb{k}"] = (b - a) * eb
    bufs = {k: _padded(s) for k, s in sizes.items()}
    ptr = lambda k: bufs[k][1]
    for k, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        p = _abi.make_problem(n, h, b - a, dt, w.reduction, w.ignore_index, w.logit_scale, w.softcap, True, True,
                              vocab_offset=a, vocab_total=V, grad_hidden_fp32=True)
        ws = torch.full((_abi.flce_forward_workspace_size(p),), fill, dtype=torch.uint8, device="cuda")
        _abi.check(_abi.flce_forward_shard(p, g["hidden"].data_ptr(), g["weight"][a:b].data_ptr(),
                                           g["targets"].data_ptr(), g["bias"][a:b].data_ptr(),
                                           ptr("slse") + 4 * k * n, ptr("stl") + 4 * k * n, ptr("smax") + 4 * k * n,
                                           ptr("sarg") + 8 * k * n, ptr("sent") + 4 * k * n, ws.data_ptr(),
                                           ws.numel(), st))
    pc = _abi.make_problem(n, 8, V, _abi.BF16, w.reduction, w.ignore_index, return_metrics=True,
                           predictions=ptr("pred"))
    ws = torch.full((_abi.flce_combine_shards_workspace_size(pc),), fill, dtype=torch.uint8, device="cuda")
    _abi.check(_abi.flce_combine_shards(pc, P, ptr("slse"), ptr("stl"), ptr("smax"), ptr("sarg"), ptr("sent"),
                                        g["targets"].data_ptr(), ptr("loss"), ptr("lse"), ptr("metrics"),
                                        ws.data_ptr(), ws.numel(), st))
    for k, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        p = _abi.make_problem(n, h, b - a, dt, w.reduction, w.ignore_index, w.logit_scale, w.softcap, False, True,
                              vocab_offset=a, vocab_total=V, grad_hidden_fp32=True, bwd_vocab_chunk=512)
        ws = torch.full((_abi.flce_backward_workspace_size(p),), fill, dtype=torch.uint8, device="cuda")
        _abi.check(_abi.flce_backward(p, g["hidden"].data_ptr(), g["weight"][a:b].data_ptr(), g["targets"].data_ptr(),
                                      g["bias"][a:b].data_ptr(), ptr("lse"), 0, ptr(f"gh{k}"), ptr(f"gw{k}"),
                                      ptr(f"gb{k}"), ws.data_ptr(), ws.numel(), st))
    torch.cuda.synchronize()
    out = {}
    for k, (buf, _) in bufs.items():
        host = buf.cpu()
        s = sizes[k]
        assert torch.all(host[:PAD] == GUARD), f"shards: write before {k}"
        assert torch.all(host[PAD + s:] == GUARD), f"shards: write past {k}"
        out[k] = host[PAD:PAD + s].clone()
    return out


def test_shard_workspace_poison_and_output_canaries():
    """The vocabulary-shard path (target codes gathered into the workspace,
    shard metrics, the combine's workspace, fp32 grad_hidden parts) under the
    same poison and canary checks."""
    w = W["transforms_bf16"].resized(n=700, h=256, v=2600)
    log_case("poison/canary: bf16 shards [0, 1111, 2600] with metrics")
    g = gpu_inputs(fi.generate(w))
    a = _run_shards(g, w, [0, 1111, 2600], 0x00)
    b = _run_shards(g, w, [0, 1111, 2600], 0xFF)
    for k in a:
        assert torch.equal(a[k], b[k]), f"shards: {k} depends on stale workspace bytes"
    assert bool(torch.any(a["gh0"] != 0)) and bool(torch.any(a["gh1"] != 0))
