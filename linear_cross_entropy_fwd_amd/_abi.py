"""ctypes view of the C ABI in include/flce.h (argument marshalling only).

Every function here forwards to the gfx950 library ``libflce.so`` built
in-tree by ``linear_cross_entropy_fwd_amd.build``.  There is no fallback: if
the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

from . import build as _build

LIB_PATH = _build.LIB

F32, F16, BF16 = 0, 1, 2
MEAN, SUM, NONE = 0, 1, 2
REDUCTIONS = {"mean": MEAN, "sum": SUM, "none": NONE}

STATUS = {0: "FLCE_OK", 1: "FLCE_ERR_INVALID_ARGUMENT", 2: "FLCE_ERR_UNSUPPORTED",
          3: "FLCE_ERR_WORKSPACE", 4: "FLCE_ERR_HIP"}


class Problem(ctypes.Structure):
    """Mirror of ``flce_problem_t``."""
    _fields_ = [
        ("n_tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int64),
        ("vocab", ctypes.c_int64),
        ("ignore_index", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("reduction", ctypes.c_int32),
        ("logit_scale", ctypes.c_float),
        ("softcap", ctypes.c_float),
        ("return_metrics", ctypes.c_int32),
        ("has_bias", ctypes.c_int32),
        ("fwd_tiles_per_split", ctypes.c_int32),
        ("bwd_vocab_chunk", ctypes.c_int32),
        ("label_smoothing", ctypes.c_float),
        ("z_loss", ctypes.c_float),
        ("class_weight", ctypes.c_void_p),
        ("predictions", ctypes.c_void_p),
        ("grad_weight_fp32", ctypes.c_int32),
        ("seq_len", ctypes.c_int64),
        ("hidden_row_stride", ctypes.c_int64),
        ("hidden_seq_stride", ctypes.c_int64),
        ("targets_stride", ctypes.c_int64),
        ("targets_seq_stride", ctypes.c_int64),
        ("vocab_offset", ctypes.c_int64),
        ("vocab_total", ctypes.c_int64),
        ("grad_hidden_fp32", ctypes.c_int32),
    ]


class FlceError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None
_lock = threading.Lock()

_VP = ctypes.c_void_p
_PP = ctypes.POINTER(Problem)

_SIGNATURES = {
    "flce_forward_workspace_size": (ctypes.c_size_t, [_PP]),
    "flce_backward_workspace_size": (ctypes.c_size_t, [_PP]),
    "flce_forward": (ctypes.c_int, [_PP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    "flce_backward": (ctypes.c_int, [_PP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                     ctypes.c_size_t, _VP]),
    "flce_forward_noalloc": (ctypes.c_int, [_PP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "flce_forward_backward_workspace_size": (ctypes.c_size_t, [_PP]),
    "flce_forward_backward": (ctypes.c_int, [_PP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                             _VP, ctypes.c_size_t, _VP]),
    "flce_forward_status": (ctypes.c_int, [_PP, _VP, ctypes.POINTER(ctypes.c_uint32), _VP]),
    "flce_forward_shard": (ctypes.c_int, [_PP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                          ctypes.c_size_t, _VP]),
    "flce_combine_shards_workspace_size": (ctypes.c_size_t, [_PP]),
    "flce_combine_shards": (ctypes.c_int, [_PP, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                           _VP, ctypes.c_size_t, _VP]),
    "flce_forward_plan": (ctypes.c_int, [_PP, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                         ctypes.POINTER(ctypes.c_int32)]),
    "flce_backward_plan": (ctypes.c_int, [_PP, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)]),
    "flce_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "flce_last_error": (ctypes.c_char_p, []),
    "flce_version": (ctypes.c_char_p, []),
    "flce_problem_size": (ctypes.c_size_t, []),
}


def library() -> ctypes.CDLL:
    """The loaded gfx950 library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with `python -m linear_cross_entropy_fwd_amd.build`")
                lib = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in _SIGNATURES.items():
                    fn = getattr(lib, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = lib
    return _lib


def last_error() -> str:
    return library().flce_last_error().decode()


def check(status: int) -> None:
    if status != 0:
        raise FlceError(status, last_error())


def make_problem(n, h, v, dtype, reduction="mean", ignore_index=-100, logit_scale=1.0,
                 softcap=None, return_metrics=False, has_bias=False, fwd_tiles_per_split=0,
                 bwd_vocab_chunk=0, label_smoothing=0.0, z_loss=0.0, class_weight=0,
                 predictions=0, grad_weight_fp32=False, seq_len=0, hidden_row_stride=0,
                 hidden_seq_stride=0, targets_stride=0, targets_seq_stride=0, vocab_offset=0,
                 vocab_total=0, grad_hidden_fp32=False) -> Problem:
    """class_weight / predictions: integer device addresses (fp32 [V] in,
    int64 [N] out), or 0.  grad_weight_fp32: 1 for fp32 grad_weight / grad_bias.
    seq_len and the strides (elements) describe a strided token layout; 0 = default.
    vocab_offset / vocab_total: a vocabulary shard (ids [vocab_offset,
    vocab_offset + v) of vocab_total); 0 / 0 = none.  grad_hidden_fp32: 1 for
    an fp32 grad_hidden."""
    return Problem(int(n), int(h), int(v), int(ignore_index), int(dtype),
                   REDUCTIONS[reduction] if isinstance(reduction, str) else int(reduction),
                   float(logit_scale), 0.0 if softcap is None else float(softcap),
                   int(bool(return_metrics)), int(bool(has_bias)), int(fwd_tiles_per_split),
                   int(bwd_vocab_chunk), float(label_smoothing), float(z_loss),
                   int(class_weight) or None, int(predictions) or None, int(grad_weight_fp32),
                   int(seq_len), int(hidden_row_stride), int(hidden_seq_stride), int(targets_stride),
                   int(targets_seq_stride), int(vocab_offset), int(vocab_total), int(grad_hidden_fp32))


def flce_forward_workspace_size(p: Problem) -> int:
    return int(library().flce_forward_workspace_size(ctypes.byref(p)))


def flce_backward_workspace_size(p: Problem) -> int:
    return int(library().flce_backward_workspace_size(ctypes.byref(p)))


def flce_forward(p: Problem, hidden, weight, targets, bias, loss, lse, metrics, workspace,
                 workspace_bytes, stream) -> int:
    """Raw call with integer device addresses (0 = NULL); returns the status."""
    return library().flce_forward(ctypes.byref(p), hidden, weight, targets, bias, loss, lse,
                                  metrics, workspace, workspace_bytes, stream)


def flce_forward_noalloc(p: Problem, hidden, weight, targets, bias, loss, lse, metrics, stream) -> int:
    """Raw call of the allocation-free forward (workspace inside the library)."""
    return library().flce_forward_noalloc(ctypes.byref(p), hidden, weight, targets, bias, loss, lse,
                                          metrics, stream)


def flce_forward_backward_workspace_size(p: Problem) -> int:
    return int(library().flce_forward_backward_workspace_size(ctypes.byref(p)))


def flce_forward_backward(p: Problem, hidden, weight, targets, bias, loss, lse, metrics, grad_loss,
                          grad_hidden, grad_weight, grad_bias, workspace, workspace_bytes, stream) -> int:
    return library().flce_forward_backward(ctypes.byref(p), hidden, weight, targets, bias, loss, lse,
                                           metrics, grad_loss, grad_hidden, grad_weight, grad_bias,
                                           workspace, workspace_bytes, stream)


def flce_backward(p: Problem, hidden, weight, targets, bias, lse, grad_loss, grad_hidden,
                  grad_weight, grad_bias, workspace, workspace_bytes, stream) -> int:
    return library().flce_backward(ctypes.byref(p), hidden, weight, targets, bias, lse,
                                   grad_loss, grad_hidden, grad_weight, grad_bias, workspace,
                                   workspace_bytes, stream)


def flce_forward_shard(p: Problem, hidden, weight, targets, bias, shard_lse, target_logit, shard_max,
                       shard_argmax, shard_entropy, workspace, workspace_bytes, stream) -> int:
    return library().flce_forward_shard(ctypes.byref(p), hidden, weight, targets, bias, shard_lse, target_logit,
                                        shard_max, shard_argmax, shard_entropy, workspace, workspace_bytes, stream)


def flce_combine_shards_workspace_size(p: Problem) -> int:
    return int(library().flce_combine_shards_workspace_size(ctypes.byref(p)))


def flce_combine_shards(p: Problem, n_shards, shard_lse, target_logit, shard_max, shard_argmax, shard_entropy,
                        targets, loss, lse, metrics, workspace, workspace_bytes, stream) -> int:
    return library().flce_combine_shards(ctypes.byref(p), int(n_shards), shard_lse, target_logit, shard_max,
                                         shard_argmax, shard_entropy, targets, loss, lse, metrics, workspace,
                                         workspace_bytes, stream)


def flce_forward_status(p: Problem, workspace, stream) -> int:
    out = ctypes.c_uint32(0)
    check(library().flce_forward_status(ctypes.byref(p), workspace, ctypes.byref(out), stream))
    return int(out.value)


def flce_forward_plan(p: Problem):
    """(tiles_per_split, n_splits, splits_per_workgroup): the forward's
    vocabulary splits and how many consecutive ones a workgroup walks."""
    t, n, g = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    check(library().flce_forward_plan(ctypes.byref(p), ctypes.byref(t), ctypes.byref(n), ctypes.byref(g)))
    return int(t.value), int(n.value), int(g.value)


def flce_backward_plan(p: Problem, with_launches: bool = False):
    """(chunk, n_chunks, last_chunk): the backward's vocabulary chunking; with
    ``with_launches`` also whether each chunk is one launch (1) or three (0)."""
    c, n, last, one = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int32(0)
    check(library().flce_backward_plan(ctypes.byref(p), ctypes.byref(c), ctypes.byref(n), ctypes.byref(last),
                                       ctypes.byref(one)))
    out = (int(c.value), int(n.value), int(last.value))
    return out + (int(one.value),) if with_launches else out


def flce_version() -> str:
    return library().flce_version().decode()
