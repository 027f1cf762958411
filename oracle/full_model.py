"""ORACLE (test infrastructure only): the whole little-lm model for one micro-batch, float64.

The model [hn.213312.xyz translation, "设置 / Setup", parameter table: token embeddings, an untied
LM head, 28 decoder layers and 14 value-embedding tables, one on every other layer;
youdonthavefriends cost analysis, "config appendix": loss LigerFusedLinearCrossEntropyLoss with
softcap 15]:

    x_0     = E[ids]                                   (token embedding rows)
    x_{i+1} = layer_i(x_i)                             (oracle.model.layer_fwd; value embedding on
                                                        the layers that carry a table)
    hn      = RMSNorm(x_L) g_final                     (final norm before the head)
    loss    = linear cross-entropy(hn, W_head, targets) (oracle.lce)

and the backward chain: dL/dhn from the loss, the final-norm backward, layer_bwd from the last
layer to the first, and dL/dE[v] = sum of dL/dx_0[n] over the tokens n with ids[n] = v.

Readings (the pages are silent): a final RMSNorm with a learnable gain sits before the head (the
Llama-style block the pages name; its D parameters fit the page's rounded parameter count); the
embedding is not scaled. In bf16 mode hn and dL/dx_L are rounded to bf16 where they are stored;
the embedding gradient is accumulated exactly (fp32 on the GPU).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .lce import lce_fwd_bwd
from .model import (LayerDims, LayerParams, gather_rows, layer_bwd, layer_fwd, rmsnorm, rmsnorm_bwd, rounder,
                    scatter_rows)


@dataclass
class ModelParams:
    embed: np.ndarray                   # [vocab, D]
    layers: list = field(default_factory=list)   # [LayerParams]
    g_final: np.ndarray = None          # [D]
    head: np.ndarray = None             # [vocab, D]


def embedding(table, ids):
    """x[n] = table[ids[n]] (a zero row for an id outside the table)."""
    return gather_rows(table, ids)


def embedding_bwd(dx, ids, rows):
    """dE[v] = sum over n with ids[n] = v of dx[n] (ids outside the table add nothing)."""
    return scatter_rows(dx, ids, rows)


def model_fwd_bwd(p: ModelParams, ids, targets, d: LayerDims, softcap=15.0, ignore_index=-100,
                  grad_scale=1.0):
    """Returns dict(loss, embed [vocab, D], layers [layer_bwd dicts], g_final [D], head [vocab, D],
    hn [N, D])."""
    R = rounder(d.mode)
    x = embedding(p.embed, ids)
    caches = []
    for lp in p.layers:
        x, c = layer_fwd(lp, x, ids, d)
        caches.append(c)
    hn_raw, rf = rmsnorm(x, p.g_final, d.rms_eps)
    hn = R(hn_raw)
    l = lce_fwd_bwd(hn, p.head, targets, softcap, ignore_index, grad_scale, mode=d.mode)
    dx_norm, dg_final = rmsnorm_bwd(l["dh"], x, p.g_final, rf)
    dx = R(dx_norm)
    grads = [None] * len(p.layers)
    for i in range(len(p.layers) - 1, -1, -1):
        dy = dx
        grads[i] = layer_bwd(p.layers[i], caches[i], dy, d)
        # natural magnitudes of the residual-scalar gradients (Cauchy-Schwarz bounds of their sums),
        # for tolerances only
        grads[i]["scale_a_mlp"] = float(np.linalg.norm(dy) * np.linalg.norm(caches[i]["m"]))
        grads[i]["scale_a_attn"] = float(np.linalg.norm(grads[i]["dh"]) * np.linalg.norm(caches[i]["attn_out"]))
        dx = grads[i]["dx"]
    return dict(loss=l["loss"], embed=embedding_bwd(dx, ids, p.embed.shape[0]), layers=grads,
                g_final=dg_final, head=l["dw"], hn=hn)
