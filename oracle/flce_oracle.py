"""Plain fp64 CPU oracle for fused linear cross-entropy.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: it is used by ``tests/``, by the package entry point's
smoke check and by the benchmark's CPU-baseline leg.  It shares no code with
the GPU library and imports nothing from it.

What it computes is the plain definition of the loss that the trl-lib
"fused-linear-ce" kernel card describes (sections "Full signature", "Metrics
for free" and "Algorithm"): cross-entropy of ``hidden @ weight.T (+ bias)``
against integer targets, with an ignore index, a logit scale, an optional
soft cap, mean / sum / none reductions, the two forward-only metrics (mean
token accuracy over non-ignored positions, mean softmax entropy in nats), and
the gradients of the loss with respect to hidden, weight and bias.

Unlike the fused method it DOES materialise logits, one block of rows at a
time (the row block only bounds memory; every row is independent), and does
all arithmetic in fp64 after an exact upcast of the inputs.  Library
primitives used as steps: numpy matmul (BLAS), exp, log, tanh, argmax.

Readings of points the card leaves open (each is stated where it is used):
  * transform order: bias, then scale, then soft cap:
        z = c * tanh(s * (raw + b) / c)      (c = softcap; identity if None)
  * soft cap form c*tanh(x/c); logit_scale multiplies;
  * mean divides by the number of non-ignored rows; with none of them the
    mean loss and both metrics are NaN and every gradient is zero;
  * ignored rows have per-row loss 0 under reduction "none";
  * argmax ties resolve to the smallest vocabulary index (numpy's argmax);
  * metrics average over non-ignored rows;
  * a non-ignored target outside [0, V) raises ValueError.

Three loss variants that run on the same vocabulary sweep (not defined on
the pages; textbook definitions, each a stated reading):
  * label smoothing eps: the target distribution is (1 - eps) one-hot plus
    eps / V uniform, so row_loss = lse - (1 - eps) z_t - (eps / V) sum_j z_j;
  * z-loss coefficient zl: row_loss += zl * lse^2 (penalises the partition
    function's log);
  * class weights w (V,): row i's whole loss (including the z-loss term) is
    multiplied by w[t_i], and the mean divides by the sum of w[t_i] over
    non-ignored rows.  Alone, label smoothing and class weights each match
    torch's cross_entropy; together, torch weights the smoothing term per
    class instead, which this reading does not.
  Metrics (accuracy, entropy) are unweighted and unaffected.

Every function here is pinned by CPU tests against library routines
(torch cross_entropy and autograd, scipy logsumexp / softmax / entropy),
closed forms (zero weight, zero scale, two classes), invariants and central
finite differences.
"""
from __future__ import annotations

import math

import numpy as np


def _f64(a):
    """Exact upcast to fp64 (inputs are fp32, or bf16/f16 already widened to fp32)."""
    return None if a is None else np.asarray(a, dtype=np.float64)


def transform_logits(raw, bias, logit_scale, softcap):
    """Bias, then logit scale, then soft cap (card: "Algorithm" -- the tile
    "applies bias / logit_scale / softcap"; the order as listed)."""
    y = raw + bias[None, :] if bias is not None else raw
    y = logit_scale * y
    if softcap is not None:
        y = softcap * np.tanh(y / softcap)
    return y


def transform_derivative(z, logit_scale, softcap):
    """d z / d raw for the transform above, written in terms of the final z:
    s for no cap; s * (1 - (z/c)^2) with the cap (derivative of c*tanh(x/c))."""
    if softcap is None:
        return np.full_like(z, logit_scale)
    return logit_scale * (1.0 - (z / softcap) ** 2)


def row_statistics(z):
    """Per-row log-sum-exp, softmax, entropy, argmax and top-1/top-2 gap.

    lse_i = m_i + log sum_j exp(z_ij - m_i) with m_i = max_j z_ij; the softmax
    p = exp(z - lse); entropy H_i = -sum_j p_ij log p_ij = lse_i - sum_j p_ij z_ij
    in nats (card: "Metrics for free"); argmax is the smallest index attaining
    the row maximum; gap = top-1 minus top-2 value (inf when V == 1).
    """
    m = z.max(axis=1)
    lse = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    p = np.exp(z - lse[:, None])
    entropy = lse - (p * z).sum(axis=1)
    argmax = z.argmax(axis=1)
    if z.shape[1] >= 2:
        top2 = np.partition(z, z.shape[1] - 2, axis=1)[:, -2:]
        gap = top2[:, 1] - top2[:, 0]
    else:
        gap = np.full(z.shape[0], np.inf)
    return lse, p, entropy, argmax, gap


def _row_weights(t, valid, class_weight):
    """w[t_i] on non-ignored rows (1 without class weights), 0 on ignored ones."""
    if class_weight is None:
        return valid.astype(np.float64)
    cw = np.asarray(class_weight, dtype=np.float64)
    return np.where(valid, cw[np.where(valid, t, 0)], 0.0)


def _reduction_coef(reduction, grad_output, rw, n):
    """Per-row factor of the gradient of the reduced loss w.r.t. each row's
    unweighted loss: row weight times the upstream gradient, divided by the
    weight total for mean."""
    if reduction == "none":
        g = np.ones(n) if grad_output is None else np.asarray(grad_output, np.float64).reshape(n)
        return rw * g
    g = 1.0 if grad_output is None else float(np.asarray(grad_output, np.float64).reshape(()))
    wsum = rw.sum()
    if reduction == "sum":
        return rw * g
    return rw * (g / wsum) if wsum > 0 else np.zeros(n)


def flce_reference(hidden, weight, targets, bias=None, ignore_index=-100,
                   logit_scale=1.0, softcap=None, reduction="mean",
                   grad_output=None, compute_grads=True, row_block=256,
                   label_smoothing=0.0, z_loss=0.0, class_weight=None):
    """Forward and backward of the loss, by its definition, in fp64.

    Arguments follow the card's "Full signature": hidden (N,H), weight (V,H),
    targets (N,) integer ids, bias (V,) or None, ignore_index, logit_scale,
    softcap (None or > 0), reduction "mean" | "sum" | "none".  ``grad_output``
    is the upstream gradient of the returned loss: a scalar for mean/sum, an
    (N,) vector for none; None means 1.  ``label_smoothing``, ``z_loss`` and
    ``class_weight`` are the variants described in the module docstring.

    Returns a dict with
      loss            scalar (mean/sum) or (N,) (none)
      row_loss        (N,)  the row's (weighted) loss, 0 on ignored rows
      lse             (N,)  log-sum-exp of the final logits
      argmax, gap     (N,)  first-index argmax and top-1/top-2 gap of z
      hit             (N,)  valid and argmax == target
      row_entropy     (N,)  softmax entropy of the row (nats)
      n_valid         number of non-ignored rows
      accuracy, entropy   the two metrics (card: "Metrics for free")
      grad_hidden (N,H), grad_weight (V,H), grad_bias (V,) or None  (if compute_grads)
    """
    if reduction not in ("mean", "sum", "none"):
        raise ValueError(f"unknown reduction {reduction!r}")
    if softcap is not None and not softcap > 0:
        raise ValueError("softcap must be None or > 0")
    h = _f64(hidden)
    w = _f64(weight)
    b = _f64(bias)
    t = np.asarray(targets, dtype=np.int64)
    n, hd = h.shape
    v = w.shape[0]
    valid = t != ignore_index
    if np.any(valid & ((t < 0) | (t >= v))):
        raise ValueError("target id outside [0, V) on a non-ignored row")
    n_valid = int(valid.sum())
    eps = float(label_smoothing)
    zl = float(z_loss)
    rw = _row_weights(t, valid, class_weight)

    # Per-row coefficient of the gradient of the reduced loss w.r.t. the
    # row's unweighted loss (row weight folded in).
    coef = _reduction_coef(reduction, grad_output, rw, n)

    row_loss = np.zeros(n)
    lse = np.zeros(n)
    argmax = np.zeros(n, dtype=np.int64)
    gap = np.zeros(n)
    row_entropy = np.zeros(n)
    if compute_grads:
        grad_h = np.zeros((n, hd))
        grad_w = np.zeros((v, hd))
        grad_b = np.zeros(v) if b is not None else None

    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        hr = h[r0:r1]
        raw = hr @ w.T                                    # (R, V) logits before transforms
        z = transform_logits(raw, b, logit_scale, softcap)
        lse_r, p, ent_r, am_r, gap_r = row_statistics(z)
        tr = t[r0:r1]
        vr = valid[r0:r1]
        rows = np.arange(r1 - r0)
        zt = np.where(vr, z[rows, np.where(vr, tr, 0)], 0.0)
        # cross-entropy against the smoothed target, plus the z-loss term,
        # times the row's class weight
        ce = lse_r - (1.0 - eps) * zt - (eps / v) * z.sum(axis=1)
        row_loss[r0:r1] = np.where(vr, rw[r0:r1] * (ce + zl * lse_r ** 2), 0.0)
        lse[r0:r1] = lse_r
        argmax[r0:r1] = am_r
        gap[r0:r1] = gap_r
        row_entropy[r0:r1] = ent_r
        if compute_grads:
            # d loss_i / d z_ij = p_ij - [j == t_i]  (card: "Algorithm", p - onehot);
            # with the variants (1 + 2 zl lse_i) p_ij - (1 - eps) [j == t_i] - eps / V
            gz = p * (1.0 + 2.0 * zl * lse_r)[:, None] - eps / v
            gz[rows[vr], tr[vr]] -= 1.0 - eps
            gz[~vr] = 0.0
            graw = coef[r0:r1, None] * gz * transform_derivative(z, logit_scale, softcap)
            if b is not None:
                # the bias enters before the scale: d raw / d b_j = 1
                grad_b += graw.sum(axis=0)
            grad_h[r0:r1] = graw @ w                       # (p - onehot) @ weight
            grad_w += graw.T @ hr                          # (p - onehot).T @ hidden

    hit = valid & (argmax == t)
    wsum = float(rw.sum())
    if reduction == "none":
        loss = row_loss.copy()
    elif reduction == "sum":
        loss = float(row_loss[valid].sum())
    else:
        loss = float(row_loss[valid].sum() / wsum) if n_valid > 0 else math.nan
    accuracy = float(hit.sum() / n_valid) if n_valid > 0 else math.nan
    entropy = float(row_entropy[valid].sum() / n_valid) if n_valid > 0 else math.nan

    out = dict(loss=loss, row_loss=row_loss, lse=lse, argmax=argmax, gap=gap, hit=hit,
               row_entropy=row_entropy, n_valid=n_valid, accuracy=accuracy, entropy=entropy)
    if compute_grads:
        out.update(grad_hidden=grad_h, grad_weight=grad_w, grad_bias=grad_b)
    return out


def row_argmax_ids(hidden, weight, bias=None, logit_scale=1.0, softcap=None, row_block=256):
    """First-index argmax of each row's final logits z (after bias, scale and
    soft cap, as in ``transform_logits``); used to build targets that equal
    the row argmax.  Ties resolve to the smallest id (numpy's argmax), the
    same reading as the accuracy metric (card: "Metrics for free")."""
    h = _f64(hidden)
    w = _f64(weight)
    b = _f64(bias)
    out = np.zeros(h.shape[0], dtype=np.int64)
    for r0 in range(0, h.shape[0], row_block):
        z = transform_logits(h[r0:r0 + row_block] @ w.T, b, logit_scale, softcap)
        out[r0:r0 + row_block] = z.argmax(axis=1)
    return out


def gradient_samples(hidden, weight, targets, lse, rows, vocab_ids, bias=None, ignore_index=-100,
                     logit_scale=1.0, softcap=None, reduction="mean", grad_output=None):
    """Selected gradient entries by the definition, given each row's lse.

    grad_hidden[rows] needs the whole logit row of each selected token;
    grad_weight[vocab_ids] and grad_bias[vocab_ids] need the selected logit
    column for every token.  ``lse`` must be the oracle's own per-row
    log-sum-exp (``flce_reference(..., compute_grads=False)["lse"]``).  The
    coefficient of each row is the same as in ``flce_reference``: p - onehot
    (card: "Algorithm"), times the reduction's upstream factor, times
    d z / d raw.
    """
    h = _f64(hidden)
    w = _f64(weight)
    b = _f64(bias)
    t = np.asarray(targets, dtype=np.int64)
    lse = np.asarray(lse, dtype=np.float64)
    n = h.shape[0]
    valid = t != ignore_index
    if np.any(valid & ((t < 0) | (t >= w.shape[0]))):
        raise ValueError("target id outside [0, V) on a non-ignored row")
    n_valid = int(valid.sum())
    if reduction == "none":
        g = np.ones(n) if grad_output is None else np.asarray(grad_output, np.float64).reshape(n)
        coef = np.where(valid, g, 0.0)
    else:
        g = 1.0 if grad_output is None else float(np.asarray(grad_output, np.float64).reshape(()))
        scale = g / n_valid if (reduction == "mean" and n_valid > 0) else (g if reduction == "sum" else 0.0)
        coef = np.where(valid, scale, 0.0)

    rows = np.asarray(rows, dtype=np.int64)
    vocab_ids = np.asarray(vocab_ids, dtype=np.int64)
    # grad_hidden rows: whole logit rows
    z = transform_logits(h[rows] @ w.T, b, logit_scale, softcap)
    gz = np.exp(z - lse[rows, None])
    for k, i in enumerate(rows):
        if valid[i]:
            gz[k, t[i]] -= 1.0
        else:
            gz[k] = 0.0
    graw = coef[rows, None] * gz * transform_derivative(z, logit_scale, softcap)
    grad_h = graw @ w
    # grad_weight / grad_bias entries: selected logit columns for all rows
    zc = transform_logits(h @ w[vocab_ids].T, None if b is None else b[vocab_ids],
                          logit_scale, softcap)
    gzc = np.exp(zc - lse[:, None])
    gzc -= (t[:, None] == vocab_ids[None, :]) & valid[:, None]
    gzc[~valid] = 0.0
    grawc = coef[:, None] * gzc * transform_derivative(zc, logit_scale, softcap)
    grad_w = grawc.T @ h
    grad_b = grawc.sum(axis=0)
    return dict(grad_hidden=grad_h, grad_weight=grad_w, grad_bias=grad_b)


def _lse_merge(m, s, z):
    """Folds a block of logits z (R, B) into each row's running maximum m and
    rescaled sum s = sum_j exp(z_j - m): the online log-sum-exp of the card's
    "Algorithm" (the old sum is rescaled by exp(m_old - m_new))."""
    m_new = np.maximum(m, z.max(axis=1))
    s_new = s * np.exp(m - m_new) + np.exp(z - m_new[:, None]).sum(axis=1)
    return m_new, s_new


def streaming_reference(hidden, weight_rows, vocab, targets, rows=(), vocab_ids=(), bias=None,
                        ignore_index=-100, logit_scale=1.0, softcap=None, reduction="mean",
                        grad_output=None, weight_block=65536, row_block=2048):
    """The loss and selected gradient entries by the definition, in fp64, for
    shapes whose weight is too large to hold in fp64 at once.

    ``weight_rows(r0, r1)`` returns weight rows r0..r1-1 (values exactly
    representable in fp64); ``vocab`` is V.  The weight is visited in blocks
    of ``weight_block`` rows and the tokens in blocks of ``row_block`` rows;
    every logit is formed from its definition (``transform_logits``) and
    nothing of size N x V is held.  Same readings as ``flce_reference``
    (plain cross-entropy; no loss variants).

    Passes:
      1. lse of every row over the whole vocabulary, merged block by block
         (``_lse_merge``), and each row's target logit;
      2. grad_hidden of the selected ``rows``: sum over weight blocks of
         (p - onehot) * coef * dz/draw times the block's rows (card:
         "Algorithm", backward);
      3. grad_weight and grad_bias of the selected ``vocab_ids``: that logit
         column for every token, (p - onehot) * coef * dz/draw, contracted
         with hidden.

    Returns a dict: lse (N,), row_loss (N,), loss, n_valid, grad_hidden
    (len(rows), H), grad_weight (len(vocab_ids), H), grad_bias
    (len(vocab_ids),) or None without a bias.
    """
    if reduction not in ("mean", "sum", "none"):
        raise ValueError(f"unknown reduction {reduction!r}")
    h = _f64(hidden)
    b = _f64(bias)
    t = np.asarray(targets, dtype=np.int64)
    n = h.shape[0]
    v = int(vocab)
    valid = t != ignore_index
    if np.any(valid & ((t < 0) | (t >= v))):
        raise ValueError("target id outside [0, V) on a non-ignored row")
    n_valid = int(valid.sum())
    coef = _reduction_coef(reduction, grad_output, valid.astype(np.float64), n)

    def wblock(r0, r1):
        return np.asarray(weight_rows(r0, r1), dtype=np.float64)

    # pass 1: lse and the target logit of every row
    m = np.full(n, -np.inf)
    s = np.zeros(n)
    zt = np.zeros(n)
    for v0 in range(0, v, weight_block):
        v1 = min(v, v0 + weight_block)
        wb = wblock(v0, v1)
        bb = None if b is None else b[v0:v1]
        for r0 in range(0, n, row_block):
            r1 = min(n, r0 + row_block)
            z = transform_logits(h[r0:r1] @ wb.T, bb, logit_scale, softcap)
            m[r0:r1], s[r0:r1] = _lse_merge(m[r0:r1], s[r0:r1], z)
            tr = t[r0:r1]
            here = valid[r0:r1] & (tr >= v0) & (tr < v1)
            idx = np.nonzero(here)[0]
            zt[r0 + idx] = z[idx, tr[idx] - v0]
    lse = m + np.log(s)
    row_loss = np.where(valid, lse - zt, 0.0)
    if reduction == "none":
        loss = row_loss.copy()
    elif reduction == "sum":
        loss = float(row_loss[valid].sum())
    else:
        loss = float(row_loss[valid].sum() / n_valid) if n_valid > 0 else math.nan

    # pass 2: grad_hidden of the selected rows
    rows = np.asarray(rows, dtype=np.int64)
    grad_h = np.zeros((len(rows), h.shape[1]))
    if len(rows):
        hs = h[rows]
        for v0 in range(0, v, weight_block):
            v1 = min(v, v0 + weight_block)
            wb = wblock(v0, v1)
            z = transform_logits(hs @ wb.T, None if b is None else b[v0:v1], logit_scale, softcap)
            gz = np.exp(z - lse[rows, None])
            for k, i in enumerate(rows):
                if not valid[i]:
                    gz[k] = 0.0
                elif v0 <= t[i] < v1:
                    gz[k, t[i] - v0] -= 1.0
            grad_h += (coef[rows, None] * gz * transform_derivative(z, logit_scale, softcap)) @ wb

    # pass 3: grad_weight / grad_bias of the selected vocabulary ids
    vids = np.asarray(vocab_ids, dtype=np.int64)
    grad_w = np.zeros((len(vids), h.shape[1]))
    grad_b = np.zeros(len(vids)) if b is not None else None
    if len(vids):
        wv = np.concatenate([wblock(int(j), int(j) + 1) for j in vids], axis=0)
        bv = None if b is None else b[vids]
        for r0 in range(0, n, row_block):
            r1 = min(n, r0 + row_block)
            zc = transform_logits(h[r0:r1] @ wv.T, bv, logit_scale, softcap)
            gzc = np.exp(zc - lse[r0:r1, None])
            gzc -= (t[r0:r1, None] == vids[None, :]) & valid[r0:r1, None]
            gzc[~valid[r0:r1]] = 0.0
            graw = coef[r0:r1, None] * gzc * transform_derivative(zc, logit_scale, softcap)
            grad_w += graw.T @ h[r0:r1]
            if grad_b is not None:
                grad_b += graw.sum(axis=0)
    return dict(lse=lse, row_loss=row_loss, loss=loss, n_valid=n_valid, grad_hidden=grad_h,
                grad_weight=grad_w, grad_bias=grad_b)
