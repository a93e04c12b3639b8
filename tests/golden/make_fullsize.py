"""Writes the full-size expected values used by tests/test_fullsize_gpu.py.

    python tests/golden/make_fullsize.py [workload ...]

For each workload at its full size it draws the seeded inputs on the CPU
(bit-identical to the GPU draw) and runs only the fp64 oracle:
  * the forward pass over every row (lse, per-row loss, metrics, top-1/top-2
    gap for argmax ties),
  * gradient entries at fixed sampled token rows and vocabulary ids, given
    that forward pass's lse.
For the peaked workload the argmax rows' targets are the oracle's
first-index argmax ids; the full target vector is stored so that the GPU
test uses exactly the same targets.

Output: tests/golden/fullsize_<workload>.npz (compressed).  Existing files
are kept (delete one to recompute it).
"""
import os
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import flce_inputs as fi  # noqa: E402
from oracle import flce_reference, gradient_samples, row_argmax_ids  # noqa: E402

WORKLOADS = ["midvocab_bf16", "headvocab_bf16", "transforms_bf16", "peaked_bf16"]


def sample_indices(w, targets):
    n, v = w.n, w.v
    t = targets
    valid_rows = np.nonzero(t != w.ignore_index)[0]
    ign_rows = np.nonzero(t == w.ignore_index)[0]
    rows = sorted({0, 1, n // 3, n // 2 + 7, n - 1, int(valid_rows[5]), int(valid_rows[-3])}
                  | ({int(ign_rows[0])} if len(ign_rows) else set()))
    # the most frequent ids, the ids of some sampled rows' targets, a ragged-tail id
    common = np.bincount(t[t >= 0], minlength=v).argsort()[::-1][:3]
    vids = sorted({0, 1, v // 2, v - 1, *map(int, common), int(t[valid_rows[5]]), int(t[valid_rows[-3]])})
    return np.array(rows, dtype=np.int64), np.array(vids, dtype=np.int64)


def make(name):
    out = os.path.join(HERE, f"fullsize_{name}.npz")
    if os.path.exists(out):
        print(f"{name}: exists, skipped", flush=True)
        return
    w = fi.WORKLOADS[name]
    t0 = time.time()
    d = fi.generate(w)
    h = d["hidden"].float().numpy()
    wt = d["weight"].float().numpy()
    b = None if d["bias"] is None else d["bias"].float().numpy()
    targets = d["targets"].numpy().copy()
    print(f"{name}: inputs drawn in {time.time() - t0:.0f} s", flush=True)
    if bool(d["argmax_rows"].any()):
        am = row_argmax_ids(h, wt, b, w.logit_scale, w.softcap, row_block=512)
        rows_am = d["argmax_rows"].numpy()
        targets[rows_am] = am[rows_am]
        print(f"{name}: argmax targets in {time.time() - t0:.0f} s", flush=True)
    fwd = flce_reference(h, wt, targets, b, ignore_index=w.ignore_index, logit_scale=w.logit_scale,
                         softcap=w.softcap, reduction=w.reduction, compute_grads=False, row_block=512)
    print(f"{name}: forward in {time.time() - t0:.0f} s", flush=True)
    rows, vids = sample_indices(w, targets)
    smp = gradient_samples(h, wt, targets, fwd["lse"], rows, vids, b, ignore_index=w.ignore_index,
                           logit_scale=w.logit_scale, softcap=w.softcap, reduction=w.reduction)
    print(f"{name}: gradient samples in {time.time() - t0:.0f} s", flush=True)
    np.savez_compressed(
        out, targets=targets.astype(np.int32), loss=np.asarray(fwd["loss"], np.float64),
        row_loss=fwd["row_loss"], lse=fwd["lse"], hit=fwd["hit"], gap=fwd["gap"].astype(np.float32),
        n_valid=fwd["n_valid"], accuracy=fwd["accuracy"], entropy=fwd["entropy"],
        rows=rows, vocab_ids=vids, grad_hidden_rows=smp["grad_hidden"],
        grad_weight_rows=smp["grad_weight"], grad_bias_entries=smp["grad_bias"])
    print(f"{name}: wrote {out} ({os.path.getsize(out) / 1e3:.0f} KB)", flush=True)


if __name__ == "__main__":
    torch.set_num_threads(os.cpu_count() or 1)
    for name in (sys.argv[1:] or WORKLOADS):
        make(name)
