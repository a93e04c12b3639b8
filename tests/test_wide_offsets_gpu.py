"""GPU tests of the 16-bit backward at shapes whose K-major operand copies
would need offsets past 32 bits, so that the older operand layout runs:
grad_weight from G^T written by the recompute kernel (many tokens times a
wide chunk), and grad_hidden from W_c^T written as the recompute kernel's
side job (a chunk of 2^20 weight rows of 2048).  Every other 16-bit test
takes the K-major path.

Sizes are too large for the dense oracle, so sampled outputs are checked
against fp64 sums written out here from the definition (softmax minus
one-hot, mean over the rows that are not ignored): lse and grad_hidden on
sampled rows, grad_weight on sampled vocabulary rows (with the library's
lse, itself checked on the sampled rows).  Tolerances: bf16 inputs, 2e-2
max-norm on gradients, 1e-3 on lse."""
import numpy as np
import pytest
import torch

from flce_testutil import log_case

pytestmark = pytest.mark.gpu

IGN = -100


def _inputs(n, h, v, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    hidden = torch.randn(n, h, generator=g, device="cuda").to(torch.bfloat16)
    weight = (torch.randn(v, h, generator=g, device="cuda") / h ** 0.5).to(torch.bfloat16)
    targets = torch.randint(0, v, (n,), generator=g, device="cuda")
    targets[::17] = IGN
    return hidden, weight, targets


def _weight_rows_f32(weight, rows=1 << 17):
    for r0 in range(0, weight.shape[0], rows):
        yield r0, weight[r0:r0 + rows].float().cpu().numpy().astype(np.float64)


def _check(hidden, weight, targets, lse, gh, gw, rows, vrows):
    tg = targets.cpu().numpy()
    valid = tg != IGN
    nv = int(valid.sum())
    hs = hidden[rows].float().cpu().numpy().astype(np.float64)          # sampled token rows
    # pass 1: lse of the sampled rows over the whole vocabulary
    m = np.full(len(rows), -np.inf)
    ssum = np.zeros(len(rows))
    for _, wc in _weight_rows_f32(weight):
        z = wc @ hs.T
        mn = np.maximum(m, z.max(axis=0))
        ssum = ssum * np.exp(m - mn) + np.exp(z - mn).sum(axis=0)
        m = mn
    lse_ref = m + np.log(ssum)
    lse_got = lse[rows].double().cpu().numpy()
    assert np.max(np.abs(lse_got - lse_ref)) <= 1e-3, (lse_got, lse_ref)
    # pass 2: grad_hidden of the sampled rows = (sum_v p_v w_v - w_t) / n_valid
    acc = np.zeros_like(hs)
    for r0, wc in _weight_rows_f32(weight):
        p = np.exp(wc @ hs.T - lse_ref)                                      # (rows of W, sampled)
        acc += p.T @ wc
    ref_gh = np.zeros_like(hs)
    for k, n in enumerate(rows):
        if valid[n]:
            ref_gh[k] = (acc[k] - weight[tg[n]].float().cpu().numpy()) / nv
    got_gh = gh[rows].float().cpu().numpy()
    err = np.max(np.abs(got_gh - ref_gh)) / np.max(np.abs(ref_gh))
    assert err <= 2e-2, err
    # grad_weight of sampled vocabulary rows = sum_n (p[n, v] - [t_n = v]) h_n / n_valid
    hid = hidden.float().cpu().numpy().astype(np.float64)
    lse_all = lse.double().cpu().numpy()
    wv = weight[vrows].float().cpu().numpy().astype(np.float64)
    p = np.exp(hid @ wv.T - lse_all[:, None])                                # (N, sampled v)
    p -= (tg[:, None] == np.asarray(vrows)[None, :])
    p[~valid] = 0.0
    ref_gw = p.T @ hid / nv
    got_gw = gw[vrows].float().cpu().numpy()
    errw = np.max(np.abs(got_gw - ref_gw)) / np.max(np.abs(ref_gw))
    assert errw <= 2e-2, errw
    return err, errw


def _run(n, h, v, chunk, seed):
    import linear_cross_entropy_fwd_amd as flce
    hidden, weight, targets = _inputs(n, h, v, seed)
    loss, lse, _ = flce.flce_forward(hidden, weight, targets, ignore_index=IGN)
    gh, gw, _ = flce.flce_backward(hidden, weight, targets, None, lse, ignore_index=IGN, bwd_vocab_chunk=chunk)
    torch.cuda.synchronize()
    return hidden, weight, targets, loss, lse, gh, gw


def test_grad_weight_through_g_transposed_when_offsets_are_wide():
    """N = 65536 tokens and one 32768-id chunk: G is 4 GiB, past what the K-major copy offsets reach."""
    from linear_cross_entropy_fwd_amd import _abi
    n, h, v, chunk = 65536, 128, 32768, 32768
    p = _abi.make_problem(n, h, v, _abi.BF16, bwd_vocab_chunk=chunk)
    # the G^T buffer (chunk x N) is in the workspace on this path
    assert _abi.flce_backward_workspace_size(p) >= 2 * n * chunk * 2
    log_case(f"wide G offsets: N={n} H={h} V={v} chunk={chunk}")
    hidden, weight, targets, loss, lse, gh, gw = _run(n, h, v, chunk, 11)
    rows = [0, 1, 4097, 30000, n - 1]
    vrows = [0, 5, 12345, v - 1]
    print("  errors:", _check(hidden, weight, targets, lse, gh, gw, rows, vrows), flush=True)


def test_grad_hidden_through_wct_side_job_when_offsets_are_wide():
    """A chunk of 2^20 weight rows of H = 2048: the weight rows' K-major offsets pass 32 bits,
    so the recompute kernel writes W_c^T (1024 tokens: four token tiles) for grad_hidden."""
    from linear_cross_entropy_fwd_amd import _abi
    n, h, v, chunk = 1024, 2048, 1 << 20, 1 << 20
    p = _abi.make_problem(n, h, v, _abi.BF16, bwd_vocab_chunk=chunk)
    # the W_c^T buffer (H x chunk) is in the workspace on this path
    assert _abi.flce_backward_workspace_size(p) >= h * chunk * 2
    log_case(f"wide weight offsets: N={n} H={h} V={v} chunk={chunk}")
    hidden, weight, targets, loss, lse, gh, gw = _run(n, h, v, chunk, 12)
    rows = [0, 3, 700, n - 1]
    vrows = [0, 77, 500000, v - 1]
    print("  errors:", _check(hidden, weight, targets, lse, gh, gw, rows, vrows), flush=True)
