"""Seeded synthetic inputs for fused linear cross-entropy workloads.

This module is shared by the tests, the benchmark and the oracle-side scripts.
It holds no arithmetic of the loss itself: it only draws hidden states,
weights, biases and target ids of the shapes and distributions that the
workloads name.

Every value comes from a counter-based integer hash evaluated with plain torch
integer ops, so the same call yields bit-identical tensors on the CPU and on a
GPU (all intermediates stay below 2**63; no floating point is involved until a
final exact conversion):

* N(0, std): Irwin-Hall sum of twelve 16-bit uniforms,
  x = (sum - 393210) / 65536, which has mean 0 and variance 1 (to 1 part in
  4e9), is exact in fp32, and is then multiplied by ``std`` in fp32 (one IEEE
  rounding) and rounded to the storage dtype (round-to-nearest-even).
* uniform ids in [0, V): ``(w * V) >> 32`` for a 32-bit hash word ``w``.
* Zipf(s) over [0, V): P(k) proportional to (k+1)^-s, by inverse CDF
  (``searchsorted`` on an fp64 CDF built on the CPU) at u = (w + 0.5) / 2^32.
* "exactly round(f*N) rows" (ignored rows, argmax rows): the rows with the
  smallest hash words (a seeded permutation; words are distinct).

The hash is the 32-bit "lowbias32" integer mixer (xor-shift / multiply),
applied twice with per-stream keys derived by the same mixer.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import torch

_M32 = 0xFFFFFFFF

# per-tensor stream ids (key = seed * 16 + stream)
_S_HIDDEN, _S_WEIGHT, _S_BIAS, _S_TARGETS, _S_IGNORE, _S_ARGMAX = 0, 1, 2, 3, 4, 5


def _mix32_int(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & _M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & _M32
    x ^= x >> 16
    return x


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for int64 x in [0, 2^32) without int64 overflow."""
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & _M32


def _mix32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def hash_words(key: int, word: int, idx: torch.Tensor) -> torch.Tensor:
    """32-bit hash word ``word`` of stream ``key`` for element indices ``idx``."""
    k1 = _mix32_int(key * 0x9E3779B1 + word * 0x85EBCA77 + 0x165667B1)
    k2 = _mix32_int(k1 ^ 0xC2B2AE3D)
    return _mix32(_mix32(idx ^ k1) ^ k2)


def _indices(n: int, device, start: int = 0) -> torch.Tensor:
    if start + n > (1 << 32):
        raise ValueError("stream longer than 2^32 elements")
    return torch.arange(start, start + n, dtype=torch.int64, device=device)


def normal_range(start: int, count: int, std: float, key: int, dtype: torch.dtype,
                 device="cpu") -> torch.Tensor:
    """Elements [start, start+count) of the flattened N(0, std) stream ``key``."""
    idx = _indices(count, device, start)
    acc = torch.zeros(count, dtype=torch.int64, device=device)
    for w in range(6):
        h = hash_words(key, w, idx)
        acc += (h >> 16) + (h & 0xFFFF)
    x = (acc - 393210).to(torch.float32) * (1.0 / 65536.0)  # exact
    x = x * torch.tensor(std, dtype=torch.float32)          # one fp32 rounding
    return x.to(dtype)


def normal_(shape, std: float, key: int, dtype: torch.dtype, device="cpu",
            block: Optional[int] = None) -> torch.Tensor:
    """N(0, std) draws (Irwin-Hall of 12 16-bit uniforms), rounded to dtype.

    ``block`` only sets how many elements are hashed per pass (cache-sized on
    the CPU, large on a GPU); it does not change the values.
    """
    if block is None:
        block = (1 << 18) if torch.device(device).type == "cpu" else (1 << 24)
    numel = 1
    for s in shape:
        numel *= int(s)
    out = torch.empty(numel, dtype=dtype, device=device)
    for b0 in range(0, numel, block):
        n = min(block, numel - b0)
        out[b0:b0 + n] = normal_range(b0, n, std, key, dtype, device)
    return out.view(*shape)


def weight_rows(w: "Workload", r0: int, r1: int, device="cpu") -> torch.Tensor:
    """Rows [r0, r1) of workload w's weight, drawn alone (same values as generate)."""
    wstd = 1.0 / w.h if w.weight_std_is_inv_h else w.weight_std
    return normal_range(r0 * w.h, (r1 - r0) * w.h, wstd, w.seed * 16 + _S_WEIGHT,
                        w.torch_dtype, device).view(r1 - r0, w.h)


def uniform_ids(n: int, v: int, key: int, device="cpu") -> torch.Tensor:
    w = hash_words(key, 0, _indices(n, device))
    return (w * v) >> 32


def zipf_ids(n: int, v: int, s: float, key: int, device="cpu") -> torch.Tensor:
    k = torch.arange(1, v + 1, dtype=torch.float64)
    cdf = torch.cumsum(k.pow(-s), 0)
    cdf = (cdf / cdf[-1]).to(device)
    w = hash_words(key, 0, _indices(n, device))
    u = (w.to(torch.float64) + 0.5) * (1.0 / 4294967296.0)
    return torch.searchsorted(cdf, u, right=True).clamp_(max=v - 1)


def chosen_rows(n: int, count: int, key: int, device="cpu") -> torch.Tensor:
    """Boolean mask of exactly ``count`` rows (those with the smallest words)."""
    w = hash_words(key, 0, _indices(n, device))
    mask = torch.zeros(n, dtype=torch.bool, device=device)
    if count > 0:
        mask[torch.argsort(w)[:count]] = True
    return mask


_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: sizes, value distributions and loss options."""
    name: str
    n: int
    h: int
    v: int
    dtype: str              # "f32" | "bf16" | "f16"
    weight_std: float       # None-able only through ``weight_std_is_inv_h``
    bias_std: Optional[float]
    logit_scale: float
    softcap: Optional[float]
    reduction: str
    ignore_frac: float
    targets: str            # "uniform" | "zipf" | "peaked"
    return_metrics: bool
    seed: int
    ignore_index: int = -100
    weight_std_is_inv_h: bool = False
    zipf_s: float = 1.1
    peaked_frac: float = 0.5

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype]

    def resized(self, n=None, h=None, v=None, **kw) -> "Workload":
        return replace(self, n=n or self.n, h=h or self.h, v=v or self.v, **kw)

    @property
    def flops_fwd_bwd(self) -> int:
        return 8 * self.n * self.h * self.v


# The five workloads of fused linear cross-entropy at LM-head shapes.
WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32_N64_H128_V1000", 64, 128, 1000, "f32", 0.0, None, 1.0, None,
        "mean", 0.10, "uniform", True, seed=1, weight_std_is_inv_h=True),
    "midvocab_bf16": Workload(
        "midvocab_bf16_N2048_H2048_V32000", 2048, 2048, 32000, "bf16", 0.02, None,
        1.0, None, "mean", 0.0, "uniform", False, seed=2),
    "headvocab_bf16": Workload(
        "headvocab_bf16_N4096_H4096_V128256", 4096, 4096, 128256, "bf16", 0.02, None,
        1.0, None, "mean", 0.05, "zipf", False, seed=3),
    "transforms_bf16": Workload(
        "transforms_bf16_N8192_H3584_V152064", 8192, 3584, 152064, "bf16", 0.02, 0.1,
        0.5, 30.0, "sum", 0.03, "uniform", True, seed=4),
    "peaked_bf16": Workload(
        "peaked_bf16_N16384_H2048_V262144", 16384, 2048, 262144, "bf16", 0.2, None,
        1.0, None, "mean", 0.02, "peaked", False, seed=5),
}


def generate(w: Workload, device="cpu") -> dict:
    """Draw the inputs of workload ``w`` on ``device``.

    Returns hidden (N,H), weight (V,H), bias (V,) or None, targets (N,) int64,
    ``ignored`` (N,) bool and ``argmax_rows`` (N,) bool.  For "peaked" targets
    the rows in ``argmax_rows`` still hold a uniform draw: the caller replaces
    them with that row's argmax logit id (a property of the loss inputs, so it
    is computed by whoever owns the arithmetic), ignored rows excluded.
    """
    dt = w.torch_dtype
    key = lambda s: w.seed * 16 + s
    wstd = 1.0 / w.h if w.weight_std_is_inv_h else w.weight_std
    hidden = normal_((w.n, w.h), 1.0, key(_S_HIDDEN), dt, device)
    weight = normal_((w.v, w.h), wstd, key(_S_WEIGHT), dt, device)
    bias = None
    if w.bias_std is not None:
        bias = normal_((w.v,), w.bias_std, key(_S_BIAS), dt, device)
    if w.targets == "zipf":
        targets = zipf_ids(w.n, w.v, w.zipf_s, key(_S_TARGETS), device)
    else:
        targets = uniform_ids(w.n, w.v, key(_S_TARGETS), device)
    argmax_rows = torch.zeros(w.n, dtype=torch.bool, device=device)
    if w.targets == "peaked":
        argmax_rows = chosen_rows(w.n, int(round(w.peaked_frac * w.n)), key(_S_ARGMAX), device)
    ignored = chosen_rows(w.n, int(round(w.ignore_frac * w.n)), key(_S_IGNORE), device)
    targets = torch.where(ignored, torch.full_like(targets, w.ignore_index), targets)
    argmax_rows &= ~ignored
    return dict(hidden=hidden, weight=weight, bias=bias, targets=targets,
                ignored=ignored, argmax_rows=argmax_rows)
