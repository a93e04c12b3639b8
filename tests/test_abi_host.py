"""CPU tests of the C ABI: the library loads, exports every function the
header declares, sizes workspaces, and rejects invalid arguments with the
documented status before anything is launched.  No compute call here reaches
a GPU: every call is invalid, and the one valid call runs only when no GPU
is present (where it must report FLCE_ERR_HIP)."""
import os
import re

import pytest

from linear_cross_entropy_fwd_amd import _abi
from linear_cross_entropy_fwd_amd._abi import BF16, F16, F32, make_problem

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "flce.h")
OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4
FAKE = 0x100000  # a 1 MiB-aligned non-null address; never dereferenced by these tests


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(flce_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = _abi.library()
    names = declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(lib, name), name
    assert _abi.flce_version().startswith("flce-gfx950")


def test_problem_struct_matches_the_library():
    import ctypes
    assert _abi.library().flce_problem_size() == ctypes.sizeof(_abi.Problem)


def test_status_strings():
    lib = _abi.library()
    for code, name in _abi.STATUS.items():
        assert lib.flce_status_str(code).decode() == name


def base(**kw):
    args = dict(n=64, h=128, v=1000, dtype=F32)
    args.update(kw)
    return make_problem(args.pop("n"), args.pop("h"), args.pop("v"), args.pop("dtype"), **args)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), INVALID),
    (dict(reduction=5), INVALID),
    (dict(n=-1), INVALID),
    (dict(h=0), INVALID),
    (dict(v=0), INVALID),
    (dict(v=1 << 31), UNSUPPORTED),
    (dict(h=30, dtype=F32), UNSUPPORTED),      # 120 bytes per row
    (dict(h=12, dtype=BF16), UNSUPPORTED),     # 24 bytes per row
    (dict(logit_scale=float("inf")), INVALID),
    (dict(logit_scale=float("nan")), INVALID),
    (dict(softcap=-1.0), INVALID),
    (dict(softcap=float("nan")), INVALID),
    (dict(softcap=float("inf")), INVALID),
    (dict(fwd_tiles_per_split=-2), INVALID),
    (dict(bwd_vocab_chunk=1000), INVALID),
    (dict(label_smoothing=-0.1), INVALID),
    (dict(label_smoothing=1.5), INVALID),
    (dict(label_smoothing=float("nan")), INVALID),
    (dict(z_loss=float("inf")), INVALID),
    (dict(class_weight=(1 << 40) + 2), INVALID),    # misaligned fp32 array
    (dict(predictions=(1 << 40) + 4, return_metrics=True), INVALID),  # misaligned int64 array
    (dict(predictions=1 << 40), INVALID),            # predictions without return_metrics
    (dict(grad_weight_fp32=2), INVALID),
    (dict(seq_len=-1), INVALID),
    (dict(seq_len=48), INVALID),                     # 64 tokens are not whole sequences of 48
    (dict(hidden_row_stride=129), INVALID),          # 516-byte rows: not 16-byte multiples
    (dict(hidden_seq_stride=-4), INVALID),
    (dict(targets_stride=-1), INVALID),
    (dict(seq_len=16, hidden_seq_stride=2049), INVALID),
    (dict(targets_seq_stride=1 << 40), INVALID),
    (dict(vocab_offset=10), INVALID),                             # an offset without a vocabulary total
    (dict(vocab_offset=-1, vocab_total=2000), INVALID),
    (dict(vocab_offset=1500, vocab_total=2000), INVALID),         # the shard runs past the vocabulary
    (dict(vocab_total=1 << 31), UNSUPPORTED),
    (dict(vocab_offset=500, vocab_total=2000, z_loss=1e-3), UNSUPPORTED),   # no loss variants with a shard
    (dict(grad_hidden_fp32=2), INVALID),
])
def test_invalid_problems(kw, status):
    p = base(**kw)
    assert _abi.flce_forward_workspace_size(p) == 0
    assert _abi.flce_backward_workspace_size(p) == 0
    st = _abi.flce_forward(p, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 0, FAKE, 1 << 30, 0)
    assert st == status, _abi.last_error()
    assert _abi.last_error()


def test_shard_problems_take_their_own_entry_points():
    """A valid vocabulary shard has workspaces, but flce_forward and
    flce_forward_backward refuse it (the shard forward and the combine are
    its path), and the combine refuses a shard problem."""
    import ctypes
    p = base(vocab_offset=500, vocab_total=2000, dtype=BF16)
    assert _abi.flce_forward_workspace_size(p) > 0 and _abi.flce_backward_workspace_size(p) > 0
    assert _abi.flce_forward(p, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 0, FAKE, 1 << 30, 0) == INVALID
    assert "flce_forward_shard" in _abi.last_error()
    assert _abi.flce_forward_backward(p, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 0, 0, FAKE, FAKE, 0, FAKE,
                                      1 << 40, 0) == INVALID
    assert _abi.flce_combine_shards_workspace_size(p) == 0
    whole = base(v=2000, dtype=BF16)
    assert _abi.flce_combine_shards_workspace_size(whole) > 0
    assert _abi.flce_combine_shards(whole, 0, FAKE, FAKE, 0, 0, 0, FAKE, FAKE, FAKE, 0, FAKE, 1 << 30, 0) == INVALID
    # metrics in the combine need the three per-shard metric arrays
    wm = base(v=2000, dtype=BF16, return_metrics=True)
    assert _abi.flce_combine_shards(wm, 2, FAKE, FAKE, 0, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 0) == INVALID
    # the shard's own metric outputs: all three or none
    sm = base(vocab_offset=500, vocab_total=2000, dtype=BF16, return_metrics=True)
    assert _abi.flce_forward_shard(sm, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 1 << 30, 0) == INVALID


def test_problem_null():
    import ctypes
    lib = _abi.library()
    assert lib.flce_forward_workspace_size(None) == 0
    assert lib.flce_forward(None, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, 1 << 30, None) == INVALID


def test_forward_pointer_and_workspace_validation():
    p = base()
    need = _abi.flce_forward_workspace_size(p)
    assert need > 0
    call = lambda **kw: _abi.flce_forward(
        p, kw.get("h", FAKE), kw.get("w", FAKE), kw.get("t", FAKE), kw.get("b", 0), kw.get("loss", FAKE),
        kw.get("lse", FAKE), kw.get("m", 0), kw.get("ws", FAKE), kw.get("wsb", need), 0)
    assert call(h=0) == INVALID
    assert call(t=0) == INVALID
    assert call(loss=0) == INVALID
    assert call(b=FAKE) == INVALID              # bias without has_bias
    assert call(m=FAKE) == INVALID              # metrics without return_metrics
    assert call(h=FAKE + 4) == INVALID          # misaligned hidden
    assert call(t=FAKE + 4) == INVALID          # misaligned targets
    assert call(ws=0) == WORKSPACE
    assert call(wsb=need - 1) == WORKSPACE
    assert call(ws=FAKE + 64) == INVALID        # misaligned workspace
    pb = base(has_bias=True, return_metrics=True)
    assert _abi.flce_forward(pb, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, 1 << 30, 0) == INVALID
    assert _abi.flce_forward(pb, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1 << 30, 0) == INVALID


def test_backward_pointer_and_workspace_validation():
    p = base()
    need = _abi.flce_backward_workspace_size(p)
    assert need > 0
    call = lambda **kw: _abi.flce_backward(
        p, kw.get("h", FAKE), kw.get("w", FAKE), kw.get("t", FAKE), kw.get("b", 0), kw.get("lse", FAKE),
        0, kw.get("gh", FAKE), kw.get("gw", FAKE), kw.get("gb", 0), kw.get("ws", FAKE), kw.get("wsb", need), 0)
    assert call(lse=0) == INVALID
    assert call(gb=FAKE) == INVALID             # grad_bias without has_bias
    assert call(gh=FAKE + 8) == INVALID         # misaligned grad_hidden
    assert call(ws=0) == WORKSPACE
    assert call(wsb=need - 1) == WORKSPACE
    # nothing requested: a no-op that succeeds without touching anything
    assert call(gh=0, gw=0, ws=0, wsb=0) == OK


def test_workspace_sizes_scale_and_never_hold_n_by_v():
    for n, h, v, dt in [(64, 128, 1000, F32), (2048, 2048, 32000, BF16), (4096, 4096, 128256, BF16),
                        (8192, 3584, 152064, BF16), (16384, 2048, 262144, BF16)]:
        for bias in (False, True):
            p = make_problem(n, h, v, dt, has_bias=bias)
            fwd = _abi.flce_forward_workspace_size(p)
            bwd = _abi.flce_backward_workspace_size(p)
            nv_bytes = n * v * (4 if dt == F32 else 2)
            assert 0 < fwd < nv_bytes or n * v < 1 << 20
            # the largest single backward buffer is a (N x chunk) gradient slab, about N x V / 4 at most;
            # all of them together (with the split grad_hidden accumulators of small N x H grids)
            # stay within 1.5 N x V bytes
            assert bwd < 1.5 * nv_bytes or n * v < 1 << 20
    # default plan at the head shape: the chunk buffers stay well under an N x V buffer
    big = make_problem(4096, 4096, 128256, BF16)
    assert _abi.flce_backward_workspace_size(big) < 0.4 * 4096 * 128256 * 2


def test_plan_overrides_change_workspace():
    a = _abi.flce_forward_workspace_size(make_problem(512, 256, 50000, BF16))
    b = _abi.flce_forward_workspace_size(make_problem(512, 256, 50000, BF16, fwd_tiles_per_split=1))
    assert b > a                                  # more splits -> more partial state
    c = _abi.flce_backward_workspace_size(make_problem(512, 256, 50000, BF16, bwd_vocab_chunk=1024))
    d = _abi.flce_backward_workspace_size(make_problem(512, 256, 50000, BF16))
    assert c < d


def test_token_layout_workspace():
    """Contiguous rows are read in place; any other layout adds one gathered
    copy of hidden (N*H elements) and / or of the targets (N int64)."""
    n, h, v = 512, 256, 50000
    for size in (_abi.flce_forward_workspace_size, _abi.flce_backward_workspace_size):
        plain = size(make_problem(n, h, v, BF16))
        # explicit defaults, and sequences back to back: contiguous, no gather
        assert size(make_problem(n, h, v, BF16, hidden_row_stride=h, targets_stride=1)) == plain
        assert size(make_problem(n, h, v, BF16, seq_len=128, hidden_seq_stride=128 * h,
                                 targets_seq_stride=128)) == plain
        # a wider row pitch: hidden gathered
        wide = size(make_problem(n, h, v, BF16, hidden_row_stride=h + 64))
        assert n * h * 2 <= wide - plain < n * h * 2 + 256
        # hidden[:, :-1] of (4, 129, h) and labels[:, 1:] of (4, 129): both gathered
        shifted = size(make_problem(n, h, v, BF16, seq_len=128, hidden_seq_stride=129 * h,
                                    targets_seq_stride=129))
        assert n * h * 2 + n * 8 <= shifted - plain < n * h * 2 + n * 8 + 2 * 256
        # strided targets alone
        t_only = size(make_problem(n, h, v, BF16, targets_stride=2))
        assert n * 8 <= t_only - plain < n * 8 + 256


def test_valid_call_without_gpu_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this test covers the no-device path only")
    p = base(n=0)
    st = _abi.flce_forward(p, 0, 0, 0, 0, FAKE, 0, 0, FAKE, 1 << 20, 0)
    assert st == HIP
    assert "device" in _abi.last_error().lower() or _abi.last_error()


def test_token_layout_from_tensor_views():
    import torch
    from linear_cross_entropy_fwd_amd import token_layout
    h = torch.zeros(4, 129, 64, dtype=torch.bfloat16)
    lab = torch.zeros(4, 129, dtype=torch.int64)
    # contiguous (N, H) / (N,): the defaults, read in place
    lay = token_layout(h.view(-1, 64), lab.view(-1))
    assert lay == dict(seq_len=0, hidden_row_stride=64, hidden_seq_stride=0, targets_stride=1,
                       targets_seq_stride=0)
    # the shifted views of a causal LM batch
    lay = token_layout(h[:, :-1], lab[:, 1:])
    assert lay == dict(seq_len=128, hidden_row_stride=64, hidden_seq_stride=129 * 64, targets_stride=1,
                       targets_seq_stride=129)
    p = make_problem(4 * 128, 64, 1000, BF16, **lay)
    plain = _abi.flce_forward_workspace_size(make_problem(4 * 128, 64, 1000, BF16))
    assert _abi.flce_forward_workspace_size(p) >= plain + 4 * 128 * (64 * 2 + 8)
    # (S, T, H) with contiguous (S*T,) targets
    lay = token_layout(h, lab.view(-1))
    assert lay["seq_len"] == 129 and lay["targets_stride"] == 1 and lay["targets_seq_stride"] == 129
    # a size-1 sequence dimension: its stride is irrelevant
    lay = token_layout(h[:1, :-1], lab[:1, 1:])
    assert lay["hidden_seq_stride"] == 0 and lay["targets_seq_stride"] == 0
    # one token per sequence: no row stride
    lay = token_layout(h[:, :1], lab[:, :1])
    assert lay["hidden_row_stride"] == 0 and lay["targets_stride"] == 0 and lay["seq_len"] == 1
    with pytest.raises(ValueError):
        token_layout(h[:, :, ::2], lab)                      # no unit stride along H
    with pytest.raises(ValueError):
        token_layout(h[:1].expand(4, 129, 64), lab)          # broadcast rows
    with pytest.raises(ValueError):
        token_layout(torch.zeros(4, 129, 68, dtype=torch.bfloat16)[:, :, :64], lab)  # 136-byte pitch


def test_forward_backward_workspace_holds_both_passes():
    for n, h, v in [(0, 128, 1000), (64, 128, 1000), (4096, 4096, 128256)]:
        p = make_problem(n, h, v, BF16)
        f, b = _abi.flce_forward_workspace_size(p), _abi.flce_backward_workspace_size(p)
        both = _abi.flce_forward_backward_workspace_size(p)
        assert f + b + 4 * n <= both < f + b + 4 * n + 3 * 256
    assert _abi.flce_forward_backward_workspace_size(base(n=-1)) == 0


def test_forward_backward_validates_like_the_two_calls():
    p = base()
    need = _abi.flce_forward_backward_workspace_size(p)
    # NULL inputs, a short workspace, an invalid problem: rejected before any launch
    assert _abi.flce_forward_backward(p, 0, FAKE, FAKE, 0, FAKE, 0, 0, 0, FAKE, FAKE, 0, FAKE, need, 0) == INVALID
    assert _abi.flce_forward_backward(p, FAKE, FAKE, FAKE, 0, FAKE, 0, 0, 0, FAKE, FAKE, 0, FAKE, need - 1,
                                      0) == WORKSPACE
    assert _abi.flce_forward_backward(base(reduction=9), FAKE, FAKE, FAKE, 0, FAKE, 0, 0, 0, FAKE, FAKE, 0,
                                      FAKE, need, 0) == INVALID
    # a gradient the backward would refuse (grad_bias without a bias) is caught before the forward runs
    assert _abi.flce_forward_backward(p, FAKE, FAKE, FAKE, 0, FAKE, 0, 0, 0, FAKE, FAKE, FAKE, FAKE, need,
                                      0) == INVALID
    assert "grad_bias" in _abi.last_error()


# The default forward plan at the five workloads (tiles a split, splits, splits a workgroup).  A
# split is at least 4 tiles and there are at most 128 of them (by V only); a workgroup walks the
# run of splits with the fewest rounds of 256 workgroups times tiles walked, at most 16 tiles,
# ties to the longer run.
@pytest.mark.parametrize("n,h,v,dtype,plan", [
    (2048, 2048, 32000, BF16, (4, 32, 1)),       # 8 x 32 = 256 workgroups: one round
    (4096, 4096, 128256, BF16, (4, 126, 4)),     # 16 x 32 groups of 16 tiles: two rounds
    (8192, 3584, 152064, BF16, (5, 119, 3)),     # 32 x 40 groups of 15 tiles: five rounds
    (16384, 2048, 262144, BF16, (8, 128, 2)),    # 64 x 64 groups of 16 tiles: sixteen rounds
    (64, 128, 1000, F32, (0, 0, 0)),             # the small fp32 path: no splits
])
def test_forward_plan_at_the_workloads(n, h, v, dtype, plan):
    assert _abi.flce_forward_plan(make_problem(n, h, v, dtype)) == plan


def test_forward_plan_split_by_v_only_and_override():
    for v in (1000, 32000, 128256, 262144, 1 << 20):
        plans = [_abi.flce_forward_plan(make_problem(n, 1024, v, BF16)) for n in (257, 1024, 4096, 16384, 65536)]
        assert len({(t, s) for t, s, _ in plans}) == 1, plans       # the split: V only
        for t, s, g in plans:
            tiles = -(-v // 256)
            assert t >= min(4, tiles) and s <= 128 and (s - 1) * t < tiles <= s * t
            assert 1 <= g <= s and (g == 1 or g * t <= 16)
    assert _abi.flce_forward_plan(make_problem(4096, 4096, 128256, BF16, fwd_tiles_per_split=3)) == (3, 167, 1)
    with pytest.raises(_abi.FlceError):
        _abi.flce_forward_plan(make_problem(64, 100, 1000, BF16))


# The default backward plan at the four bf16 workloads (chunk ids, chunks, last chunk).  The
# chunk is at most a quarter of V, rounded up to whole tiles, and 48 tiles, scored by how full
# grad_weight's last round of 256 workgroups is; a last chunk under a quarter of a chunk joins
# the one before it.
@pytest.mark.parametrize("n,h,v,plan", [
    (2048, 2048, 32000, (8192, 4, 7424)),       # 32-tile chunks: whole rounds of 256 workgroups
    (4096, 4096, 128256, (12288, 11, 5376)),
    (8192, 3584, 152064, (12288, 13, 4608)),
    (16384, 2048, 262144, (8192, 32, 8192)),    # 32 tiles: one full round of 8 x 32 grad_weight tiles
])
def test_backward_plan_at_the_workloads(n, h, v, plan):
    assert _abi.flce_backward_plan(make_problem(n, h, v, BF16)) == plan


def test_default_backward_plan_properties():
    """Over many (H, V): the default chunk is whole tiles, at most a quarter of
    V rounded up to a tile and at most 48 tiles (either that cap or a multiple
    of 16 tiles), the chunks cover V exactly, a longer last chunk is one that
    absorbed under a quarter of a chunk, and the plan is the same for every N
    (grad_hidden's summation order must not depend on the batch)."""
    import random
    rng = random.Random(20261202)
    vs = [1, 255, 256, 257, 1000, 1023, 1024, 1025, 4096, 32000, 32001, 50257, 128256, 152064, 256000,
          262144, 1 << 20] + [rng.randrange(1, 400000) for _ in range(40)]
    for h in (128, 1024, 2048, 3584, 4096, 8192):
        for v in vs:
            plans = {_abi.flce_backward_plan(make_problem(n, h, v, BF16)) for n in (300, 4096, 50000)}
            assert len(plans) == 1, (h, v, plans)
            chunk, n_chunks, last = plans.pop()
            cap = min(48, max(1, -(-v // 1024)))
            tiles = chunk // 256
            assert chunk % 256 == 0 and 1 <= tiles <= cap, (h, v, chunk)
            assert tiles == cap or tiles % 16 == 0, (h, v, chunk)
            assert (n_chunks - 1) * chunk + last == v and last > 0, (h, v, chunk, n_chunks, last)
            assert last <= chunk or 4 * (last - chunk) < chunk, (h, v, chunk, last)


def test_backward_plan_override_and_invalid():
    assert _abi.flce_backward_plan(make_problem(4096, 4096, 128256, BF16, bwd_vocab_chunk=4096)) == (4096, 32, 1280)
    # one launch per chunk for 16-bit inputs; fp32 and operands past 32-bit offsets keep three kernels
    assert _abi.flce_backward_plan(make_problem(4096, 4096, 128256, BF16), with_launches=True)[3] == 1
    assert _abi.flce_backward_plan(make_problem(64, 128, 1000, F32), with_launches=True)[3] == 0
    assert _abi.flce_backward_plan(make_problem(65536, 128, 32768, BF16, bwd_vocab_chunk=32768),
                                   with_launches=True)[3] == 0
    with pytest.raises(_abi.FlceError):
        _abi.flce_backward_plan(make_problem(64, 100, 1000, BF16))   # 200-byte rows: refused


# No buffer of N x V elements: the whole workspace of a forward + backward stays below the bytes
# of one N x V matrix in the input dtype at every 16-bit workload (the memory claim of the fused
# method), with and without the all-transforms options.
@pytest.mark.parametrize("n,h,v,kw", [
    (2048, 2048, 32000, {}),
    (4096, 4096, 128256, {}),
    (8192, 3584, 152064, dict(has_bias=True, logit_scale=0.5, softcap=30.0, reduction="sum",
                              return_metrics=True)),
    (16384, 2048, 262144, {}),
    (16384, 2048, 262144, dict(reduction="none")),
])
def test_workspace_below_one_n_by_v_matrix(n, h, v, kw):
    # and the forward alone fits the allocation-free forward's fixed 32 MiB
    assert _abi.flce_forward_workspace_size(make_problem(n, h, v, BF16, **kw)) <= 32 << 20
    p = make_problem(n, h, v, BF16, **kw)
    total = _abi.flce_forward_workspace_size(p) + _abi.flce_backward_workspace_size(p)
    assert 0 < total < n * v * 2, (total, n * v * 2)
    assert _abi.flce_forward_backward_workspace_size(p) < n * v * 2


def test_noalloc_forward_refuses_past_its_scratch_before_any_launch():
    # 128 splits x 5 fields (metrics) x 20000 rows x 4 B: more than the fixed 32 MiB scratch
    p = make_problem(20000, 128, 262144, BF16, return_metrics=True)
    assert _abi.flce_forward_workspace_size(p) > 32 << 20
    st = _abi.flce_forward_noalloc(p, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 0, 0)
    assert st == WORKSPACE and "fixed scratch" in _abi.last_error()
    # invalid problems get the forward's own status first
    assert _abi.flce_forward_noalloc(base(h=30), FAKE, FAKE, FAKE, 0, FAKE, FAKE, 0, 0) == UNSUPPORTED
