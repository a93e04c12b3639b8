"""CPU tests of the seeded synthetic input generator."""
import torch

import flce_inputs as fi


def small(name, **kw):
    w = fi.WORKLOADS[name]
    return w.resized(n=min(w.n, 512), h=min(w.h, 64), v=min(w.v, 3000), **kw)


def test_deterministic_and_seed_dependent():
    w = small("headvocab_bf16")
    a, b = fi.generate(w), fi.generate(w)
    for k in ("hidden", "weight", "targets", "ignored"):
        assert torch.equal(a[k], b[k])
    c = fi.generate(w.resized(seed=99))
    assert not torch.equal(a["hidden"], c["hidden"])
    assert not torch.equal(a["weight"], c["weight"])


def test_block_size_does_not_change_values():
    a = fi.normal_((300, 70), 0.02, 11, torch.bfloat16, block=1 << 8)
    b = fi.normal_((300, 70), 0.02, 11, torch.bfloat16, block=1 << 20)
    assert torch.equal(a, b)


def test_irwin_hall_normal_moments_and_grid():
    x = fi.normal_((1 << 20,), 1.0, 5, torch.float32)
    assert abs(x.mean().item()) < 5e-3
    assert abs(x.std().item() - 1.0) < 5e-3
    assert x.abs().max().item() <= 6.0
    q = x * 65536.0                      # every draw sits on the 1/65536 grid before scaling
    assert torch.equal(q, q.round())
    # fourth moment of Irwin-Hall(12) standardised: 3 - 1/10
    k4 = (x.double() ** 4).mean().item()
    assert abs(k4 - 2.9) < 0.05


def test_exact_ignore_counts_and_ids_in_range():
    for name, w in fi.WORKLOADS.items():
        ws = small(name)
        d = fi.generate(ws)
        t = d["targets"]
        assert int(d["ignored"].sum()) == int(round(ws.ignore_frac * ws.n))
        assert torch.all((t == ws.ignore_index) == d["ignored"])
        live = t[~d["ignored"]]
        assert int(live.min()) >= 0 and int(live.max()) < ws.v
        assert d["hidden"].dtype == ws.torch_dtype and d["hidden"].shape == (ws.n, ws.h)
        assert d["weight"].shape == (ws.v, ws.h)
        assert (d["bias"] is None) == (ws.bias_std is None)


def test_workload_ignore_counts_at_full_size():
    expect = {"tiny_f32": 6, "midvocab_bf16": 0, "headvocab_bf16": 205,
              "transforms_bf16": 246, "peaked_bf16": 328}
    for name, count in expect.items():
        w = fi.WORKLOADS[name]
        assert int(fi.chosen_rows(w.n, int(round(w.ignore_frac * w.n)), w.seed * 16 + 4).sum()) == count


def test_zipf_support_and_head():
    ids = fi.zipf_ids(200000, 1000, 1.1, 77)
    assert int(ids.min()) >= 0 and int(ids.max()) < 1000
    counts = torch.bincount(ids, minlength=1000)
    assert int(counts.argmax()) == 0
    # P(0) / P(1) = 2^1.1 for the finite-support Zipf law
    ratio = counts[0].item() / counts[1].item()
    assert abs(ratio - 2 ** 1.1) < 0.1


def test_peaked_rows_exclude_ignored():
    w = small("peaked_bf16")
    d = fi.generate(w)
    assert not torch.any(d["argmax_rows"] & d["ignored"])
    assert int(d["argmax_rows"].sum()) == int(round(w.peaked_frac * w.n)) - int(
        (fi.chosen_rows(w.n, int(round(w.peaked_frac * w.n)), w.seed * 16 + 5) & d["ignored"]).sum())
