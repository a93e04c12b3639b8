"""The forward and backward calls under HIP graph capture: the library
allocates nothing and synchronises nothing, so both calls record into one
graph.  Every replay (with the program's own eager work and synchronisations
between replays, and new input values written into the captured buffers)
must equal the eager result bit for bit (the path is deterministic)."""
import pytest
import torch

import flce_inputs as fi
from flce_testutil import gpu_inputs, log_case

pytestmark = pytest.mark.gpu

W = fi.WORKLOADS


def _run(flce, g, w, ws_f, ws_b):
    loss, lse, m = flce.flce_forward(g["hidden"], g["weight"], g["targets"], g["bias"],
                                     ignore_index=w.ignore_index, logit_scale=w.logit_scale,
                                     softcap=w.softcap, reduction=w.reduction,
                                     return_metrics=w.return_metrics, workspace=ws_f)
    gh, gw, gb = flce.flce_backward(g["hidden"], g["weight"], g["targets"], g["bias"], lse,
                                    ignore_index=w.ignore_index, logit_scale=w.logit_scale,
                                    softcap=w.softcap, reduction=w.reduction, workspace=ws_b,
                                    bwd_vocab_chunk=1024)
    return [x for x in (loss, lse, m, gh, gw, gb) if x is not None]


def test_graph_replays_match_eager():
    import linear_cross_entropy_fwd_amd as flce
    w = W["transforms_bf16"].resized(n=1030, h=256, v=2600)   # bias, scale, cap, metrics; fused W_c^T
    log_case(f"graph capture {w.name} n={w.n} h={w.h} v={w.v}")
    d1 = fi.generate(w)
    d2 = fi.generate(w.resized(seed=w.seed + 100))
    g = gpu_inputs(d1)
    g2 = gpu_inputs(d2)
    p = flce.problem_for(g["hidden"], g["weight"], g["bias"], w.ignore_index, w.logit_scale, w.softcap,
                         w.reduction, w.return_metrics, bwd_vocab_chunk=1024)
    ws_f = torch.empty(flce._abi.flce_forward_workspace_size(p), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(flce._abi.flce_backward_workspace_size(p), dtype=torch.uint8, device="cuda")

    eager1 = [x.clone() for x in _run(flce, g, w, ws_f, ws_b)]
    g_alt = {k: (v.clone() if v is not None else None) for k, v in g.items()}
    for k in ("hidden", "weight", "bias"):
        if g_alt[k] is not None:
            g_alt[k].copy_(g2[k])
    eager2 = [x.clone() for x in _run(flce, g_alt, w, ws_f, ws_b)]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(flce, g, w, ws_f, ws_b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _run(flce, g, w, ws_f, ws_b)

    for rep in range(4):
        # eager work and a synchronisation between replays
        x = torch.randn(512, 512, device="cuda")
        (x @ x).sum().item()
        src = g2 if rep % 2 else None
        for k in ("hidden", "weight", "bias"):
            if g[k] is not None:
                g[k].copy_(src[k] if src is not None else gpu_inputs(d1)[k])
        graph.replay()
        torch.cuda.synchronize()
        want = eager2 if rep % 2 else eager1
        for got, ref in zip(outs, want):
            assert torch.equal(got, ref), f"replay {rep}"


def test_graph_one_call_with_shifted_views():
    """flce_forward_backward on hidden[:, :-1] / labels[:, 1:] views (the
    gather kernels and the split grad_hidden sum in the graph too)."""
    import linear_cross_entropy_fwd_amd as flce
    w = W["midvocab_bf16"].resized(n=3 * 301, h=256, v=2600)
    log_case(f"graph capture, one call on shifted views {w.name}")
    d1, d2 = fi.generate(w), fi.generate(w.resized(seed=w.seed + 100))
    hid = d1["hidden"].cuda().view(3, 301, 256)
    lab = d1["targets"].cuda().view(3, 301)
    wt = d1["weight"].cuda()
    hv, tv = hid[:, :-1], lab[:, 1:]
    p = flce.problem_for(hv, wt, None, layout=flce.token_layout(hv, tv))
    ws = torch.empty(flce._abi.flce_forward_backward_workspace_size(p), dtype=torch.uint8, device="cuda")

    def run():
        loss, lse, _, (gh, gw, _) = flce.flce_forward_backward(hv, wt, tv, None, want_lse=True, workspace=ws,
                                                               bwd_vocab_chunk=1024)
        return [loss, lse, gh, gw]

    def load(d):
        hid.copy_(d["hidden"].cuda().view(3, 301, 256))
        wt.copy_(d["weight"].cuda())

    eager1 = [x.clone() for x in run()]
    load(d2)
    eager2 = [x.clone() for x in run()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = run()
    for rep in range(4):
        x = torch.randn(256, 256, device="cuda")
        (x @ x).sum().item()
        load(d2 if rep % 2 else d1)
        graph.replay()
        torch.cuda.synchronize()
        want = eager2 if rep % 2 else eager1
        for got, ref in zip(outs, want):
            assert torch.equal(got, ref), f"replay {rep}"


def test_graph_vocabulary_shards():
    """Two vocabulary shards with metrics (their forwards, the combine and
    their backwards with fp32 grad_hidden parts) captured in one graph:
    every replay equals the eager pass bit for bit."""
    import linear_cross_entropy_fwd_amd as flce
    w = W["transforms_bf16"].resized(n=700, h=256, v=2600)
    log_case(f"graph capture, vocabulary shards of {w.name}")
    d1, d2 = fi.generate(w), fi.generate(w.resized(seed=w.seed + 100))
    g = gpu_inputs(d1)
    kw = dict(ignore_index=w.ignore_index, logit_scale=w.logit_scale, softcap=w.softcap)
    bounds = [0, 1111, 2600]

    def run():
        parts = [flce.flce_forward_shard(g["hidden"], g["weight"][a:b], g["targets"], g["bias"][a:b],
                                         vocab_offset=a, vocab_total=w.v, return_metrics=True, **kw)
                 for a, b in zip(bounds[:-1], bounds[1:])]
        st = [torch.stack([p[i] for p in parts]) for i in range(5)]
        loss, lse, metrics = flce.flce_combine_shards(st[0], st[1], g["targets"], w.v, ignore_index=w.ignore_index,
                                                      reduction=w.reduction, shard_metrics=st[2:])
        outs = [loss, lse, metrics]
        for a, b in zip(bounds[:-1], bounds[1:]):
            outs += list(flce.flce_backward(g["hidden"], g["weight"][a:b], g["targets"], g["bias"][a:b], lse,
                                            reduction=w.reduction, vocab_offset=a, vocab_total=w.v,
                                            grad_hidden_fp32=True, **kw))
        return outs

    def load(d):
        for k in ("hidden", "weight", "bias"):
            g[k].copy_(d[k].cuda())

    eager1 = [x.clone() for x in run()]
    load(d2)
    eager2 = [x.clone() for x in run()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = run()
    for rep in range(4):
        x = torch.randn(256, 256, device="cuda")
        (x @ x).sum().item()
        load(d2 if rep % 2 else d1)
        graph.replay()
        torch.cuda.synchronize()
        want = eager2 if rep % 2 else eager1
        for got, ref in zip(outs, want):
            assert torch.equal(got, ref), f"replay {rep}"
