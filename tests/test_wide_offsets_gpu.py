"""GPU tests of the 16-bit backward at shapes whose K-major operand copies
would need offsets past 32 bits, so that the older operand layout runs:
grad_weight from G^T written by the recompute kernel (many tokens times a
wide chunk), and grad_hidden from W_c^T written as the recompute kernel's
side job (a chunk of 2^20 weight rows of 2048).  Every other 16-bit test
takes the K-major path.

The weights are too large for the dense oracle, so the expected values come
from the oracle's streaming form (``oracle.streaming_reference``, fp64, the
weight visited in row blocks): the lse of every row, grad_hidden on sampled
token rows and grad_weight on sampled vocabulary rows.  Tolerances: bf16
inputs, 2e-3 relative max-norm on lse, 2e-2 on gradients."""
import numpy as np
import pytest
import torch

from flce_testutil import TOL, log_case, maxnorm_rel, to_np

pytestmark = pytest.mark.gpu

IGN = -100


def _inputs(n, h, v, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    hidden = torch.randn(n, h, generator=g, device="cuda").to(torch.bfloat16)
    weight = (torch.randn(v, h, generator=g, device="cuda") / h ** 0.5).to(torch.bfloat16)
    targets = torch.randint(0, v, (n,), generator=g, device="cuda")
    targets[::17] = IGN
    return hidden, weight, targets


def _check(hidden, weight, targets, lse, gh, gw, rows, vrows):
    from oracle import streaming_reference
    ref = streaming_reference(to_np(hidden), lambda r0, r1: to_np(weight[r0:r1]), weight.shape[0],
                              to_np(targets), rows, vrows, ignore_index=IGN, weight_block=1 << 16,
                              row_block=2048)
    tol = TOL["bf16"]
    e_lse = maxnorm_rel(to_np(lse), ref["lse"])
    e_h = maxnorm_rel(to_np(gh[rows]), ref["grad_hidden"])
    e_w = maxnorm_rel(to_np(gw[vrows]), ref["grad_weight"])
    print(f"  errors: lse {e_lse:.2e}, grad_hidden rows {e_h:.2e}, grad_weight rows {e_w:.2e}", flush=True)
    assert e_lse <= tol["loss"] and e_h <= tol["grad"] and e_w <= tol["grad"], (e_lse, e_h, e_w)


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
    _check(hidden, weight, targets, lse, gh, gw, [0, 1, 4097, 30000, n - 1], [0, 5, 12345, v - 1])


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
    _check(hidden, weight, targets, lse, gh, gw, [0, 3, 700, n - 1], [0, 77, 500000, v - 1])
