"""ORACLE (test infrastructure only): the optimizer step of the little-lm training run, float64.

The pages group the parameters [youdonthavefriends cost analysis, "config appendix"; linlog.top
article, 从失败跑开始, the optimizer paragraph]: the matrix parameters (the four weight matrices of every decoder layer) take
Muon with learning rate 0.02, momentum 0.95 and weight decay 0; the token embedding, the LM head,
the value-embedding tables and the scalars take AdamW with per-group learning rates, betas
(0.8, 0.995 | 0.96 | 0.95), eps 1e-10 and weight decays 0.001-0.05. The master weights (and,
read plainly, the optimizer state stored beside them) are bf16 [linlog.top article, 吞吐量优化:
bf16 主权重].

The pages give neither Muon's orthogonalisation coefficients nor its iteration count. Muon is
taken as published by its author (K. Jordan, "Muon: An optimizer for hidden layers in neural
networks", blog post, December 2024):
  * momentum on the raw gradient, buf <- mu buf + g, and Nesterov's look-ahead u = g + mu buf;
  * the update is u orthogonalised by a quintic Newton-Schulz iteration: X_0 = u / (||u||_F + 1e-7),
    taken as its transpose when it has more rows than columns (so that the Gram matrix X X^T is
    the smaller one), then 5 times
        A = X X^T,  B = b A + c A A,  X <- a X + B X,   (a, b, c) = (3.4445, -4.7750, 2.0315),
    which maps every singular value s of X_0 through p(s) = a s + b s^3 + c s^5 and leaves the
    singular vectors alone;
  * W <- W - lr sqrt(max(1, rows / cols)) X_5 (and W <- W (1 - lr wd) first; wd = 0 here).
AdamW is the decoupled-weight-decay Adam of Loshchilov and Hutter with bias correction, as
torch.optim.AdamW computes it: W <- W (1 - lr wd); m <- b1 m + (1 - b1) g;
v <- b2 v + (1 - b2) g^2; W <- W - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).

Rounding contract of bf16 mode (mode="bf16"; the GPU path stores these tensors in bf16, all of its
arithmetic in between is fp32): Muon rounds buf, u, X_0, and each A, B and X of the iteration, and
the new W (its decay and update in one step); the Frobenius norm is exact. AdamW rounds m, v and
the new W, each once (a bf16 parameter with fp32 state rounds only W). mode="fp32" rounds nothing.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_round

NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_STEPS = 5
NS_EPS = 1e-7


def _rounder(mode: str):
    if mode == "bf16":
        return bf16_round
    if mode == "fp32":
        return lambda a: np.asarray(a, dtype=np.float64)
    raise ValueError(mode)


def newton_schulz(u, steps: int = NS_STEPS, mode: str = "fp32", coeffs=NS_COEFFS, eps: float = NS_EPS):
    """The quintic Newton-Schulz orthogonalisation of u [rows, cols] (module docstring)."""
    R = _rounder(mode)
    a, b, c = coeffs
    u = np.asarray(u, np.float64)
    X = R(u / (np.linalg.norm(u) + eps))
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    for _ in range(steps):
        A = R(X @ X.T)
        B = R(b * A + c * (A @ A))
        X = R(a * X + B @ X)
    return X.T if tall else X


def muon_update(w, g, buf, lr: float = 0.02, momentum: float = 0.95, nesterov: bool = True,
                weight_decay: float = 0.0, steps: int = NS_STEPS, mode: str = "fp32"):
    """One Muon step of the matrix w [rows, cols] with gradient g and momentum buffer buf.
    Returns (new w, new buf)."""
    R = _rounder(mode)
    w = np.asarray(w, np.float64)
    g = np.asarray(g, np.float64)
    buf = R(momentum * np.asarray(buf, np.float64) + g)
    u = R(g + momentum * buf) if nesterov else buf
    o = newton_schulz(u, steps, mode)
    scale = np.sqrt(max(1.0, w.shape[0] / w.shape[1]))
    return R(w * (1.0 - lr * weight_decay) - lr * scale * o), buf


def adamw_param_update(p, m, v, step: int, lr: float, beta1: float, beta2: float, eps: float,
                       weight_decay: float, mode: str = "fp32"):
    """The parameter half of one AdamW step, from the step's updated moments m and v:
    p (1 - lr wd) - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps), rounded by mode."""
    R = _rounder(mode)
    p = np.asarray(p, np.float64)
    m = np.asarray(m, np.float64)
    v = np.asarray(v, np.float64)
    bc1 = 1.0 - beta1 ** step
    bc2 = 1.0 - beta2 ** step
    return R(p * (1.0 - lr * weight_decay) - lr * (m / bc1) / (np.sqrt(v / bc2) + eps))


def adamw_update(p, g, m, v, step: int, lr: float, beta1: float, beta2: float, eps: float,
                 weight_decay: float, mode: str = "fp32", state_mode: str | None = None):
    """One AdamW step (module docstring) at step number `step` (1 for the first). mode rounds the
    parameter, state_mode (default: mode) the two moments. Returns (new p, new m, new v)."""
    Rs = _rounder(state_mode or mode)
    g = np.asarray(g, np.float64)
    m = Rs(beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g)
    v = Rs(beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g)
    p = adamw_param_update(p, m, v, step, lr, beta1, beta2, eps, weight_decay, mode)
    return p, m, v


# The parameter groups of the run [youdonthavefriends cost analysis, "config appendix"]. The norm
# gains are read as members of the "scalars" group (the pages name no other group for them).
ADAMW_GROUPS = {
    "embeddings": dict(lr=0.1414, betas=(0.8, 0.995), eps=1e-10, weight_decay=0.001),
    "lm_head": dict(lr=0.002828, betas=(0.8, 0.96), eps=1e-10, weight_decay=0.01),
    "value_embeds": dict(lr=0.0707, betas=(0.8, 0.995), eps=1e-10, weight_decay=0.01),
    "scalars": dict(lr=0.005, betas=(0.8, 0.95), eps=1e-10, weight_decay=0.05),
}
MUON_GROUP = dict(lr=0.02, momentum=0.95, weight_decay=0.0)
