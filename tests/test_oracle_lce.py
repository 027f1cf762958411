"""Pins of oracle.lce (softcapped linear cross-entropy) against torch's CPU cross_entropy with
autograd, closed forms (uniform logits, large softcap), ignore_index behaviour and the expected
loss at the LM-head initialisation, plus the parameter table printed on the pages."""
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from oracle import lce as ol
from oracle import model as om
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _torch_lce(h, w, y, s, gscale=1.0, ignore=-100):
    ht = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    z = ht @ wt.T
    c = s * torch.tanh(z / s)
    loss = F.cross_entropy(c, torch.tensor(y, dtype=torch.long), ignore_index=ignore)
    (loss * gscale).backward()
    return loss.item(), ht.grad.numpy(), wt.grad.numpy()


def test_lce_matches_torch_cross_entropy():
    rng = np.random.default_rng(0)
    h = rng.standard_normal((37, 24))
    w = rng.standard_normal((53, 24)) * 0.5
    y = rng.integers(0, 50, 37)
    y[[3, 9]] = -100
    out = ol.lce_fwd_bwd(h, w, y, softcap=15.0, grad_scale=0.25, mode="fp32")
    loss, dh, dw = _torch_lce(h, w, y, 15.0, 0.25)
    assert math.isclose(out["loss"], loss, rel_tol=1e-12)
    np.testing.assert_allclose(out["dh"], dh, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(out["dw"], dw, rtol=1e-10, atol=1e-13)
    assert out["n_valid"] == 35
    assert not np.any(out["dh"][[3, 9]])


def test_lce_uniform_logits_and_large_softcap():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((8, 16))
    out = ol.lce_fwd_bwd(h, np.zeros((100, 16)), rng.integers(0, 100, 8), mode="fp32")
    assert math.isclose(out["loss"], math.log(100), rel_tol=1e-13)
    np.testing.assert_allclose(out["lse"], math.log(100), rtol=1e-13)
    # softcap -> infinity is the plain cross-entropy
    w = rng.standard_normal((30, 16))
    y = rng.integers(0, 30, 8)
    big = ol.lce_fwd_bwd(h, w, y, softcap=1e7, mode="fp32")
    loss = F.cross_entropy(torch.tensor(h @ w.T), torch.tensor(y)).item()
    assert math.isclose(big["loss"], loss, rel_tol=1e-9)


def test_lce_all_ignored_is_zero():
    h = np.ones((4, 8))
    out = ol.lce_fwd_bwd(h, np.ones((16, 8)), np.full(4, -100), mode="fp32")
    assert out["loss"] == 0.0 and not np.any(out["dh"]) and not np.any(out["dw"])


def test_lce_init_loss_closed_form():
    """At the LM-head shape with H ~ N(0,1), W ~ N(0, 0.02^2) and D = 3072, each row's logits are
    ~N(0, 1.2288); softcap 15 barely changes them, so E[loss] ~= ln(V) + 1.2288/2 = 11.44."""
    inp = synth.lce_inputs(256, 3072, 50304, 50257, dtype="bf16", seed=0)
    out = ol.lce_fwd_bwd(inp.hidden, inp.weight, inp.targets, mode="bf16", need_grads=False)
    expected = math.log(50304) + 0.5 * 3072 * 0.02 ** 2
    assert abs(out["loss"] - expected) < 0.25, out["loss"]


def test_parameter_table_reproduced_by_layer_shapes():
    """Shapes of the oracle's layer (two pre-norm gains, gain-free QK-norm, no biases, two
    residual scalars) reproduce the page's parameter table at the 3.8B configuration."""
    gold = {}
    with open(os.path.join(GOLD, "param_table.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, v = line.split()
                gold[k] = float(v)
    s = synth.LAYER_1K
    D, F_, V = s.d_model, s.d_ff, s.vocab
    shapes = om.LayerParams(np.empty((s.qkv_dim, D)), np.empty((D, s.n_q_heads * s.head_dim)),
                            np.empty((F_, D)), np.empty((D, F_)), np.empty(D), np.empty(D), 1.0, 1.0)
    per_layer = sum(np.size(getattr(shapes, k)) for k in ("w_qkv", "w_o", "w_fc", "w_proj", "g_attn", "g_mlp")) + 2
    emb = V * D
    ve = 14 * V * s.n_kv_heads * s.head_dim
    assert round(emb / 1e6, 1) == gold["token_embeddings"] == gold["lm_head_untied"]
    assert round(28 * per_layer / 1e6, 1) == gold["decoder_layers_28"]
    assert round(ve / 1e6, 1) == gold["value_embeddings_14"]
    total = 2 * emb + 28 * per_layer + ve + D          # + final norm gain
    # the page's total is its own row sum truncated to 3 decimals (3.8489...B -> 3.848B)
    assert math.floor(total / 1e6) / 1e3 == gold["total_billions"]
