"""ORACLE (test infrastructure only): linear cross-entropy with tanh logit softcap, float64.

The loss of the little-lm training step is Liger's fused linear cross-entropy with softcap 15
over the untied LM head [youdonthavefriends cost analysis, "config appendix": loss
LigerFusedLinearCrossEntropyLoss(softcap=15.0)]; the fusion chunks the LM-head matmul inside the
loss so the (B*T, vocab) logits are never materialised [hn.213312.xyz translation, "提升吞吐量 /
Increasing throughput"]. Fusion changes where the arithmetic happens, not its result, so the
oracle is the unfused definition:

    z    = H W^T                     (H [N, D], W [V, D]; all V = 50304 padded columns included)
    c    = s * tanh(z / s)           (s = softcap)
    lse  = log sum_v exp(c[n, v])
    loss = (1 / N_valid) * sum over rows with target != ignore_index of (lse[n] - c[n, y_n])
    dz   = grad_scale / N_valid * (softmax(c) - onehot(y)) * (1 - (c / s)^2)   (0 on ignored rows)
    dH   = dz W,   dW = dz^T H

Readings (the pages are silent): mean over non-ignored rows with ignore_index -100 (the PyTorch
cross-entropy convention); if no row is valid the loss and all gradients are 0; the padded
vocabulary columns are ordinary columns of the softmax. In bf16 mode z is rounded to bf16 (it is
a GEMM output), dz is rounded once where stored, dH is rounded, dW is accumulated exactly and
rounded once.
"""
from __future__ import annotations

import numpy as np

from .model import rounder


def lce_fwd_bwd(hidden, weight, targets, softcap=15.0, ignore_index=-100, grad_scale=1.0,
                mode="bf16", need_grads=True):
    """Returns dict(loss, lse [N], dh [N, D] | None, dw [V, D] | None, n_valid)."""
    R = rounder(mode)
    h = np.asarray(hidden, np.float64)
    w = np.asarray(weight, np.float64)
    y = np.asarray(targets, np.int64)
    N = h.shape[0]
    z = R(h @ w.T)
    c = softcap * np.tanh(z / softcap)
    mx = np.max(c, axis=1, keepdims=True)
    lse = (mx + np.log(np.sum(np.exp(c - mx), axis=1, keepdims=True)))[:, 0]
    valid = y != ignore_index
    n_valid = int(np.sum(valid))
    rows = np.nonzero(valid)[0]
    if n_valid:
        loss = float(np.sum(lse[rows] - c[rows, y[rows]]) / n_valid)
    else:
        loss = 0.0
    out = dict(loss=loss, lse=lse, n_valid=n_valid, dh=None, dw=None)
    if not need_grads:
        return out
    if n_valid:
        p = np.exp(c - lse[:, None])
        p[rows, y[rows]] -= 1.0
        dz = (grad_scale / n_valid) * p * (1.0 - (c / softcap) ** 2)
        dz[~valid] = 0.0
    else:
        dz = np.zeros_like(c)
    dz = R(dz)
    out["dh"] = R(dz @ w)
    out["dw"] = R(dz.T @ h)
    return out
