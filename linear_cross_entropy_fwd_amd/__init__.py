"""Fused linear cross-entropy on MI355X (gfx950).

``fused_linear_cross_entropy`` has the signature of the trl-lib
"fused-linear-ce" kernel card ("Full signature"): the cross-entropy of
``hidden @ weight.T (+ bias)`` against int64 targets, with ignore_index,
logit_scale, softcap, mean / sum / none reductions and optional metrics
(mean token accuracy, mean softmax entropy), differentiable with respect to
hidden, weight and bias.  The N x V logit matrix is never materialised.

Every step runs in the hand-written HIP kernels of ``libflce.so`` through
its C ABI (include/flce.h); this module only allocates tensors with
PyTorch's caching allocator and passes device pointers and the current
stream.  There is no CPU or PyTorch fallback.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _abi
from ._abi import FlceError, Problem, library, make_problem  # noqa: F401

__all__ = ["fused_linear_cross_entropy", "flce_forward", "flce_backward", "flce_forward_backward",
           "flce_forward_shard", "flce_combine_shards", "FlceError", "Problem", "make_problem", "library",
           "token_layout"]

_DTYPES = {torch.float32: _abi.F32, torch.float16: _abi.F16, torch.bfloat16: _abi.BF16}


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def _check_inputs(hidden, weight, targets, bias):
    """Validates shapes, dtypes and devices; returns the token layout keywords
    of ``make_problem`` for the strides of hidden and targets.

    hidden is (N, H) or (S, T, H) with unit stride along H; targets is (N,)
    or (S, T) (or (S*T,)).  Other strides are passed to the library as they
    are (e.g. ``hidden[:, :-1]`` and ``labels[:, 1:]``), so no copy is made."""
    if not hidden.is_cuda:
        raise ValueError("hidden must be a GPU tensor (there is no CPU path)")
    if hidden.dim() not in (2, 3) or weight.dim() != 2 or targets.dim() not in (1, 2):
        raise ValueError("expected hidden (N,H) or (S,T,H), weight (V,H), targets (N,) or (S,T)")
    lead = tuple(hidden.shape[:-1])
    n = 1
    for d in lead:
        n *= d
    if weight.shape[1] != hidden.shape[-1] or (tuple(targets.shape) != lead and tuple(targets.shape) != (n,)):
        raise ValueError(f"shape mismatch: hidden {tuple(hidden.shape)}, weight {tuple(weight.shape)}, "
                         f"targets {tuple(targets.shape)}")
    if hidden.dtype not in _DTYPES or weight.dtype != hidden.dtype:
        raise ValueError("hidden and weight must share one of float32 / float16 / bfloat16")
    if targets.dtype != torch.int64:
        raise ValueError("targets must be int64")
    if bias is not None and (bias.shape != (weight.shape[0],) or bias.dtype != hidden.dtype):
        raise ValueError("bias must be (V,) in the dtype of hidden")
    for t in (hidden, weight, targets) + ((bias,) if bias is not None else ()):
        if t.device != hidden.device:
            raise ValueError("all tensors must be on one device")
    for t in (weight,) + ((bias,) if bias is not None else ()):
        if not t.is_contiguous():
            raise ValueError("weight and bias must be contiguous")
    return token_layout(hidden, targets)


def token_layout(hidden, targets) -> dict:
    """The token layout keywords of ``make_problem`` (seq_len and strides in
    elements, 0 = default) for hidden (N, H) / (S, T, H) and targets (N,) /
    (S, T) / (S*T,) as they sit in memory."""
    lead = tuple(hidden.shape[:-1])
    n = 1
    for d in lead:
        n *= d
    if hidden.shape[-1] > 1 and hidden.stride(-1) != 1:
        raise ValueError("hidden must have unit stride along its last dimension")
    seq = lead[-1] if len(lead) == 2 else n
    n_seq = lead[0] if len(lead) == 2 else 1
    # strides of size-1 dimensions do not matter: pass the default (0)
    hr = hidden.stride(-2) if seq > 1 else 0
    hs = hidden.stride(0) if (len(lead) == 2 and n_seq > 1) else 0
    if targets.dim() == 2:
        ts = targets.stride(1) if seq > 1 else 0
        tss = targets.stride(0) if n_seq > 1 else 0
        t_broadcast = (seq > 1 and ts == 0) or (n_seq > 1 and tss == 0)
    else:
        ts = targets.stride(0) if n > 1 else 0
        tss = seq * ts if (len(lead) == 2 and n_seq > 1) else 0
        t_broadcast = n > 1 and ts == 0
    if (seq > 1 and hr == 0) or (n_seq > 1 and hs == 0) or t_broadcast:
        raise ValueError("broadcast (zero-stride) hidden rows or targets are not supported")
    eb = hidden.element_size()
    if (hr * eb) % 16 or (hs * eb) % 16:
        raise ValueError("hidden row and sequence strides must be multiples of 16 bytes")
    return dict(seq_len=seq if len(lead) == 2 else 0, hidden_row_stride=hr, hidden_seq_stride=hs,
                targets_stride=ts, targets_seq_stride=tss)


def _check_class_weight(class_weight, weight):
    if class_weight is None:
        return
    if (class_weight.shape != (weight.shape[0],) or class_weight.dtype != torch.float32
            or class_weight.device != weight.device or not class_weight.is_contiguous()):
        raise ValueError("class_weight must be a contiguous float32 (V,) tensor on the device of weight")


def problem_for(hidden, weight, bias, ignore_index=-100, logit_scale=1.0, softcap=None,
                reduction="mean", return_metrics=False, fwd_tiles_per_split=0,
                bwd_vocab_chunk=0, label_smoothing=0.0, z_loss=0.0, class_weight=None,
                predictions=None, grad_weight_fp32=False, layout=None, vocab_offset=0, vocab_total=0,
                grad_hidden_fp32=False) -> Problem:
    """``layout``: the token layout keywords ``_check_inputs`` returns (None = contiguous).
    ``vocab_offset`` / ``vocab_total``: weight holds ids [vocab_offset, vocab_offset + V)
    of a vocabulary of vocab_total ids (0 / 0: the whole vocabulary)."""
    _check_class_weight(class_weight, weight)
    n = hidden.numel() // hidden.shape[-1] if hidden.shape[-1] else 0
    return make_problem(n, hidden.shape[-1], weight.shape[0], _DTYPES[hidden.dtype],
                        reduction, ignore_index, logit_scale, softcap, return_metrics,
                        bias is not None, fwd_tiles_per_split, bwd_vocab_chunk, label_smoothing,
                        z_loss, _ptr(class_weight), _ptr(predictions), grad_weight_fp32,
                        **(layout or {}), vocab_offset=vocab_offset, vocab_total=vocab_total,
                        grad_hidden_fp32=grad_hidden_fp32)


def flce_forward(hidden, weight, targets, bias=None, *, ignore_index=-100, logit_scale=1.0,
                 softcap=None, reduction="mean", return_metrics=False, want_lse=True,
                 workspace: Optional[torch.Tensor] = None, fwd_tiles_per_split=0,
                 label_smoothing=0.0, z_loss=0.0, class_weight=None,
                 predictions: Optional[torch.Tensor] = None):
    """Tensor-level ``flce_forward``: returns (loss, lse or None, metrics or None).
    ``predictions`` (int64 (N,), needs return_metrics) receives each row's argmax id.
    hidden may be (S, T, H) and targets (S, T), strided (see ``_check_inputs``);
    per-token outputs are flat (N,) = (S*T,)."""
    layout = _check_inputs(hidden, weight, targets, bias)
    n = targets.numel()
    if predictions is not None and (predictions.shape != (n,) or predictions.dtype != torch.int64
                                    or predictions.device != hidden.device or not predictions.is_contiguous()):
        raise ValueError("predictions must be an int64 (N,) tensor on the device of hidden")
    p = problem_for(hidden, weight, bias, ignore_index, logit_scale, softcap, reduction,
                    return_metrics, fwd_tiles_per_split=fwd_tiles_per_split,
                    label_smoothing=label_smoothing, z_loss=z_loss, class_weight=class_weight,
                    predictions=predictions, layout=layout)
    dev = hidden.device
    loss = torch.empty(n if reduction == "none" else 1, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev) if want_lse else None
    metrics = torch.empty(2, dtype=torch.float32, device=dev) if return_metrics else None
    need = _abi.flce_forward_workspace_size(p)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream().cuda_stream
    _abi.check(_abi.flce_forward(p, _ptr(hidden), _ptr(weight), _ptr(targets), _ptr(bias),
                                 _ptr(loss), _ptr(lse), _ptr(metrics), _ptr(workspace),
                                 workspace.numel(), stream))
    if reduction != "none":
        loss = loss.view(())
    return loss, lse, metrics


def flce_backward(hidden, weight, targets, bias, lse, grad_loss=None, *, ignore_index=-100,
                  logit_scale=1.0, softcap=None, reduction="mean", need_hidden=True,
                  need_weight=True, need_bias=True, workspace: Optional[torch.Tensor] = None,
                  bwd_vocab_chunk=0, label_smoothing=0.0, z_loss=0.0, class_weight=None,
                  grad_weight_fp32=False, grad_hidden_fp32=False, vocab_offset=0, vocab_total=0):
    """Tensor-level ``flce_backward``: returns (grad_hidden, grad_weight, grad_bias);
    grad_weight and grad_bias are fp32 with ``grad_weight_fp32``, grad_hidden
    with ``grad_hidden_fp32``; grad_hidden is contiguous, in the shape of hidden.
    With a vocabulary shard (``vocab_total`` > 0; weight and bias hold ids
    [vocab_offset, vocab_offset + V)), ``lse`` is the whole vocabulary's
    (``flce_combine_shards``), grad_weight and grad_bias are the shard's rows
    and grad_hidden is the shard's part of the gradient."""
    layout = _check_inputs(hidden, weight, targets, bias)
    p = problem_for(hidden, weight, bias, ignore_index, logit_scale, softcap, reduction,
                    False, bwd_vocab_chunk=bwd_vocab_chunk, label_smoothing=label_smoothing,
                    z_loss=z_loss, class_weight=class_weight, grad_weight_fp32=grad_weight_fp32,
                    layout=layout, vocab_offset=vocab_offset, vocab_total=vocab_total,
                    grad_hidden_fp32=grad_hidden_fp32)
    dev = hidden.device
    if grad_loss is not None:
        grad_loss = grad_loss.to(device=dev, dtype=torch.float32).contiguous()
        expect = targets.numel() if reduction == "none" else 1
        if grad_loss.numel() != expect:
            raise ValueError(f"grad_loss must have {expect} elements")
    hdt = torch.float32 if grad_hidden_fp32 else hidden.dtype
    gh = torch.empty(hidden.shape, dtype=hdt, device=dev) if need_hidden else None
    gdt = torch.float32 if grad_weight_fp32 else weight.dtype
    gw = torch.empty(weight.shape, dtype=gdt, device=dev) if need_weight else None
    gb = torch.empty(bias.shape, dtype=gdt, device=dev) if (need_bias and bias is not None) else None
    need = _abi.flce_backward_workspace_size(p)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream().cuda_stream
    _abi.check(_abi.flce_backward(p, _ptr(hidden), _ptr(weight), _ptr(targets), _ptr(bias),
                                  _ptr(lse), _ptr(grad_loss), _ptr(gh), _ptr(gw), _ptr(gb),
                                  _ptr(workspace), workspace.numel(), stream))
    return gh, gw, gb


def flce_forward_backward(hidden, weight, targets, bias=None, grad_loss=None, *, ignore_index=-100,
                          logit_scale=1.0, softcap=None, reduction="mean", return_metrics=False,
                          want_lse=False, need_hidden=True, need_weight=True, need_bias=True,
                          workspace: Optional[torch.Tensor] = None, fwd_tiles_per_split=0,
                          bwd_vocab_chunk=0, label_smoothing=0.0, z_loss=0.0, class_weight=None,
                          predictions: Optional[torch.Tensor] = None, grad_weight_fp32=False):
    """Loss and gradients in one library call (``flce_forward_backward``):
    returns (loss, lse or None, metrics or None, (grad_hidden, grad_weight,
    grad_bias)).  ``grad_loss`` is the upstream gradient as in
    ``flce_backward`` (None = 1)."""
    layout = _check_inputs(hidden, weight, targets, bias)
    n = targets.numel()
    if predictions is not None and (predictions.shape != (n,) or predictions.dtype != torch.int64
                                    or predictions.device != hidden.device or not predictions.is_contiguous()):
        raise ValueError("predictions must be an int64 (N,) tensor on the device of hidden")
    p = problem_for(hidden, weight, bias, ignore_index, logit_scale, softcap, reduction,
                    return_metrics, fwd_tiles_per_split=fwd_tiles_per_split,
                    bwd_vocab_chunk=bwd_vocab_chunk, label_smoothing=label_smoothing, z_loss=z_loss,
                    class_weight=class_weight, predictions=predictions,
                    grad_weight_fp32=grad_weight_fp32, layout=layout)
    dev = hidden.device
    if grad_loss is not None:
        grad_loss = grad_loss.to(device=dev, dtype=torch.float32).contiguous()
        if grad_loss.numel() != (n if reduction == "none" else 1):
            raise ValueError("grad_loss must have N elements for reduction 'none', else 1")
    loss = torch.empty(n if reduction == "none" else 1, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev) if want_lse else None
    metrics = torch.empty(2, dtype=torch.float32, device=dev) if return_metrics else None
    gh = torch.empty(hidden.shape, dtype=hidden.dtype, device=dev) if need_hidden else None
    gdt = torch.float32 if grad_weight_fp32 else weight.dtype
    gw = torch.empty(weight.shape, dtype=gdt, device=dev) if need_weight else None
    gb = torch.empty(bias.shape, dtype=gdt, device=dev) if (need_bias and bias is not None) else None
    need = _abi.flce_forward_backward_workspace_size(p)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream().cuda_stream
    _abi.check(_abi.flce_forward_backward(p, _ptr(hidden), _ptr(weight), _ptr(targets), _ptr(bias),
                                          _ptr(loss), _ptr(lse), _ptr(metrics), _ptr(grad_loss),
                                          _ptr(gh), _ptr(gw), _ptr(gb), _ptr(workspace),
                                          workspace.numel(), stream))
    if reduction != "none":
        loss = loss.view(())
    return loss, lse, metrics, (gh, gw, gb)


def flce_forward_shard(hidden, weight, targets, bias=None, *, vocab_offset, vocab_total, ignore_index=-100,
                       logit_scale=1.0, softcap=None, return_metrics=False,
                       workspace: Optional[torch.Tensor] = None, fwd_tiles_per_split=0):
    """One vocabulary shard's part of the forward (``flce_forward_shard``):
    weight and bias hold ids [vocab_offset, vocab_offset + V) of a vocabulary
    of ``vocab_total`` ids; targets are ids of the whole vocabulary.  Returns
    (shard_lse, target_logit), fp32 (N,): the row's log-sum-exp over the
    shard's ids, and its target logit when the target is one of them (else 0);
    with ``return_metrics`` also (shard_max, shard_argmax, shard_entropy): the
    row's largest logit, its first id (of the whole vocabulary, int64) and the
    entropy of the softmax over the shard's ids."""
    layout = _check_inputs(hidden, weight, targets, bias)
    p = problem_for(hidden, weight, bias, ignore_index, logit_scale, softcap, "none", return_metrics,
                    fwd_tiles_per_split=fwd_tiles_per_split, layout=layout, vocab_offset=vocab_offset,
                    vocab_total=vocab_total)
    dev = hidden.device
    n = targets.numel()
    shard_lse = torch.empty(n, dtype=torch.float32, device=dev)
    target_logit = torch.empty(n, dtype=torch.float32, device=dev)
    sm = ((torch.empty(n, dtype=torch.float32, device=dev), torch.empty(n, dtype=torch.int64, device=dev),
           torch.empty(n, dtype=torch.float32, device=dev)) if return_metrics else (None, None, None))
    need = _abi.flce_forward_workspace_size(p)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream().cuda_stream
    _abi.check(_abi.flce_forward_shard(p, _ptr(hidden), _ptr(weight), _ptr(targets), _ptr(bias),
                                       _ptr(shard_lse), _ptr(target_logit), _ptr(sm[0]), _ptr(sm[1]), _ptr(sm[2]),
                                       _ptr(workspace), workspace.numel(), stream))
    return (shard_lse, target_logit) + (sm if return_metrics else ())


def flce_combine_shards(shard_lse, target_logit, targets, vocab_total, *, ignore_index=-100,
                        reduction="mean", shard_metrics=None, predictions: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None):
    """The loss of a vocabulary split into shards (``flce_combine_shards``),
    from the shards' ``flce_forward_shard`` outputs stacked as (n_shards, N)
    tensors (shards in the order of their ids; that order is also the
    summation order).  Returns (loss, lse, metrics or None): loss per
    ``reduction`` ((), or (N,) for "none"), the whole vocabulary's per-row lse
    (the input of ``flce_backward``), and with ``shard_metrics`` = the stacked
    (shard_max, shard_argmax, shard_entropy) the two metrics; ``predictions``
    (int64 (N,), needs shard_metrics) receives each row's argmax id."""
    if shard_lse.dim() != 2 or target_logit.shape != shard_lse.shape:
        raise ValueError("shard_lse and target_logit must be (n_shards, N) tensors of one shape")
    arrays = (shard_lse, target_logit) + (tuple(shard_metrics) if shard_metrics is not None else ())
    for k, t in enumerate(arrays):
        want = torch.int64 if k == 3 else torch.float32
        if (t.dtype != want or not t.is_cuda or not t.is_contiguous() or t.device != targets.device
                or t.shape != shard_lse.shape):
            raise ValueError("shard arrays must be contiguous (n_shards, N) tensors on the targets' device "
                             "(int64 argmax, float32 otherwise)")
    if predictions is not None and (shard_metrics is None or predictions.dtype != torch.int64
                                    or predictions.shape != (targets.numel(),) or not predictions.is_contiguous()):
        raise ValueError("predictions must be an int64 (N,) tensor and needs shard_metrics")
    if targets.dtype != torch.int64 or targets.numel() != shard_lse.shape[1] or targets.dim() not in (1, 2):
        raise ValueError("targets must be int64 (N,) or (S, T) with N = shard_lse.shape[1]")
    n = targets.numel()
    if targets.dim() == 2:
        seq = targets.shape[1]
        lay = dict(seq_len=seq, targets_stride=targets.stride(1) if seq > 1 else 0,
                   targets_seq_stride=targets.stride(0) if targets.shape[0] > 1 else 0)
    else:
        lay = dict(targets_stride=targets.stride(0) if n > 1 else 0)
    # the combine reads no hidden rows: H = 8 bf16 elements stands for any width
    mon = shard_metrics is not None
    p = make_problem(n, 8, vocab_total, _abi.BF16, reduction, ignore_index, return_metrics=mon,
                     predictions=_ptr(predictions), **lay)
    dev = targets.device
    loss = torch.empty(n if reduction == "none" else 1, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    metrics = torch.empty(2, dtype=torch.float32, device=dev) if mon else None
    sm = tuple(shard_metrics) if mon else (None, None, None)
    need = _abi.flce_combine_shards_workspace_size(p)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream().cuda_stream
    _abi.check(_abi.flce_combine_shards(p, shard_lse.shape[0], _ptr(shard_lse), _ptr(target_logit), _ptr(sm[0]),
                                        _ptr(sm[1]), _ptr(sm[2]), _ptr(targets), _ptr(loss), _ptr(lse),
                                        _ptr(metrics), _ptr(workspace), workspace.numel(), stream))
    if reduction != "none":
        loss = loss.view(())
    return loss, lse, metrics


class _FusedLinearCrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, weight, targets, bias, ignore_index, logit_scale, softcap,
                reduction, return_metrics, label_smoothing, z_loss, class_weight):
        loss, lse, metrics = flce_forward(hidden, weight, targets, bias, ignore_index=ignore_index,
                                          logit_scale=logit_scale, softcap=softcap,
                                          reduction=reduction, return_metrics=return_metrics,
                                          label_smoothing=label_smoothing, z_loss=z_loss,
                                          class_weight=class_weight)
        ctx.save_for_backward(hidden, weight, targets, bias, lse, class_weight)
        ctx.opts = (ignore_index, logit_scale, softcap, reduction, label_smoothing, z_loss)
        if metrics is None:
            metrics = torch.empty(0, device=hidden.device)
        ctx.mark_non_differentiable(metrics)
        return loss, metrics

    @staticmethod
    def backward(ctx, grad_loss, _grad_metrics):
        hidden, weight, targets, bias, lse, class_weight = ctx.saved_tensors
        ignore_index, logit_scale, softcap, reduction, label_smoothing, z_loss = ctx.opts
        nh, nw, _, nb = ctx.needs_input_grad[:4]
        gh, gw, gb = flce_backward(hidden, weight, targets, bias, lse, grad_loss,
                                   ignore_index=ignore_index, logit_scale=logit_scale,
                                   softcap=softcap, reduction=reduction, need_hidden=nh,
                                   need_weight=nw, need_bias=nb and bias is not None,
                                   label_smoothing=label_smoothing, z_loss=z_loss,
                                   class_weight=class_weight)
        return gh, gw, None, gb, None, None, None, None, None, None, None, None


def fused_linear_cross_entropy(hidden, weight, targets, bias=None, ignore_index=-100,
                               logit_scale=1.0, softcap=None, reduction="mean",
                               return_metrics=False, label_smoothing=0.0, z_loss=0.0,
                               class_weight=None):
    """Cross-entropy of ``hidden @ weight.T (+ bias)`` without materialising logits.

    Returns ``loss`` (fp32; scalar for mean/sum, (N,) for none), or
    ``(loss, {"mean_token_accuracy": ..., "entropy": ...})`` with
    ``return_metrics=True``.  hidden, weight and bias receive gradients.
    ``label_smoothing``, ``z_loss`` and ``class_weight`` (fp32 (V,), not
    differentiated) select the variants described in include/flce.h.
    """
    if reduction not in ("mean", "sum", "none"):
        raise ValueError(f"unknown reduction {reduction!r}")
    loss, metrics = _FusedLinearCrossEntropy.apply(hidden, weight, targets, bias, ignore_index,
                                                   logit_scale, softcap, reduction,
                                                   return_metrics, label_smoothing, z_loss,
                                                   class_weight)
    if not return_metrics:
        return loss
    return loss, {"mean_token_accuracy": metrics[0], "entropy": metrics[1]}
