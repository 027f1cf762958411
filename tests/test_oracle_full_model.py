"""Pins of the whole-model oracle (oracle.full_model) against things other than itself: the
embedding as a one-hot matrix product, finite differences of the model's own loss along random
directions, and the reduction to a plain norm + softcapped cross-entropy computed by torch when
every residual branch is switched off."""
import numpy as np
import torch
import torch.nn.functional as F

import synth
from oracle import full_model as fm
from oracle import model as om

TINY = synth.LayerShape(batch=2, seq=12, d_model=32, n_q_heads=4, n_kv_heads=2, head_dim=8,
                        d_ff=64, vocab=24, real_vocab=21, dtype="fp32", fp8_mlp=False)


def _params(mi) -> fm.ModelParams:
    f = lambda a: np.asarray(a, np.float64)
    return fm.ModelParams(f(mi.embed), [om.params_from_inputs(li) for li in mi.layers], f(mi.g_final), f(mi.head))


def test_embedding_is_one_hot_product():
    rng = np.random.default_rng(1)
    E = rng.standard_normal((9, 5))
    ids = np.array([4, 0, 4, 8, 2, 4])
    onehot = np.eye(9)[ids]
    np.testing.assert_array_equal(fm.embedding(E, ids), onehot @ E)
    dx = rng.standard_normal((6, 5))
    np.testing.assert_allclose(fm.embedding_bwd(dx, ids, 9), onehot.T @ dx, rtol=1e-14, atol=1e-15)
    assert not np.any(fm.embedding_bwd(dx, ids, 9)[[1, 3, 5, 6, 7]])


def test_model_fp32_finite_differences():
    """Directional derivatives of the loss (central differences, h = 1e-6) against the backward
    chain for the embedding, the head, the final gain and a weight, a gain, a residual scalar and a
    value-embedding table of each layer."""
    mi = synth.model_inputs(TINY, n_layers=2, seed=3, perturb=True, w_std=0.2)
    p = _params(mi)
    d = om.dims_from_shape(TINY)
    out = fm.model_fwd_bwd(p, mi.ids, mi.targets, d)
    rng = np.random.default_rng(3)
    eps = 1e-6

    def loss_with(**repl):
        q = fm.ModelParams(repl.get("embed", p.embed), repl.get("layers", p.layers),
                           repl.get("g_final", p.g_final), repl.get("head", p.head))
        return fm.model_fwd_bwd(q, mi.ids, mi.targets, d)["loss"]

    def check(fd, an, what):
        assert abs(fd - an) <= 2e-7 * max(1.0, abs(fd)), (what, fd, an)

    for name in ("embed", "g_final", "head"):
        base = getattr(p, name)
        u = rng.standard_normal(base.shape)
        fd = (loss_with(**{name: base + eps * u}) - loss_with(**{name: base - eps * u})) / (2 * eps)
        grad = out["embed" if name == "embed" else ("g_final" if name == "g_final" else "head")]
        check(fd, float(np.sum(grad * u)), name)
    for li in range(2):
        for name in ("w_qkv", "w_fc", "g_mlp", "a_attn") + (("ve_table",) if li == 0 else ()):
            base = getattr(p.layers[li], name)
            u = rng.standard_normal(np.shape(base))
            def f(sign):
                layers = list(p.layers)
                layers[li] = om.LayerParams(**{**p.layers[li].__dict__, name: base + sign * eps * u})
                return loss_with(layers=layers)
            fd = (f(1) - f(-1)) / (2 * eps)
            check(fd, float(np.sum(np.asarray(out["layers"][li][name]) * u)), f"layer{li}.{name}")


def test_model_without_branches_is_norm_plus_softcapped_ce():
    """With every residual scalar 0 the layers are identities: loss = CE(15 tanh(rms_norm(E[ids]) W^T / 15))
    (torch float64, an independent route), dE and dg_final by torch autograd."""
    mi = synth.model_inputs(TINY, n_layers=2, seed=4, perturb=True, w_std=0.2)
    p = _params(mi)
    for lp in p.layers:
        lp.a_attn = 0.0
        lp.a_mlp = 0.0
    d = om.dims_from_shape(TINY)
    out = fm.model_fwd_bwd(p, mi.ids, mi.targets, d)
    E = torch.tensor(p.embed, requires_grad=True)
    g = torch.tensor(p.g_final, requires_grad=True)
    W = torch.tensor(p.head, requires_grad=True)
    x = E[torch.tensor(mi.ids, dtype=torch.long)]
    hn = F.rms_norm(x, (TINY.d_model,), weight=g, eps=TINY.rms_eps)
    c = 15.0 * torch.tanh((hn @ W.T) / 15.0)
    loss = F.cross_entropy(c, torch.tensor(mi.targets, dtype=torch.long))
    loss.backward()
    np.testing.assert_allclose(out["loss"], loss.item(), rtol=1e-12)
    np.testing.assert_allclose(out["embed"], E.grad.numpy(), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(out["g_final"], g.grad.numpy(), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(out["head"], W.grad.numpy(), rtol=1e-9, atol=1e-12)
    for lg in out["layers"]:
        assert not np.any(lg["w_qkv"]) and not np.any(lg["w_fc"])
