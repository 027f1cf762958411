"""Pins of oracle.model (the decoder layer) against things other than itself:
torch CPU float64 library routines (F.rms_norm, scaled_dot_product_attention with GQA, autograd
as an independent backward), closed forms and identities of RoPE, brute-force softmax on tiny
inputs, central finite differences of the oracle's own forward, and special cases."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import model as om
from oracle import numerics as nu
import synth


def _t(a):
    return torch.tensor(np.asarray(a, np.float64), dtype=torch.float64)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_matches_torch_and_autograd():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 33))
    g = 1 + 0.1 * rng.standard_normal(33)
    d = rng.standard_normal((7, 33))
    y, r = om.rmsnorm(x, g, 1e-6)
    xt, gt = _t(x).requires_grad_(), _t(g).requires_grad_()
    yt = F.rms_norm(xt, (33,), weight=gt, eps=1e-6)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-13, atol=1e-13)
    yt.backward(_t(d))
    dx, dg = om.rmsnorm_bwd(d, x, g, r)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_rmsnorm_scale_invariance():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64))
    g = np.ones(64)
    a, _ = om.rmsnorm(x, g, 0.0)
    b, _ = om.rmsnorm(37.5 * x, g, 0.0)
    np.testing.assert_allclose(a, b, rtol=1e-13)


# ---------------------------------------------------------------- RoPE
def test_rope_identities():
    rng = np.random.default_rng(2)
    B, T, H, Dh = 2, 50, 3, 16
    cos, sin = om.rope_angles(T, Dh, 10000.0)
    x = rng.standard_normal((B, T, H, Dh))
    y = om.rope(x, cos, sin)
    np.testing.assert_array_equal(y[:, 0], x[:, 0])                              # R_0 = I
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    d = rng.standard_normal(x.shape)
    np.testing.assert_allclose(np.sum(y * d), np.sum(x * om.rope_transpose(d, cos, sin)), rtol=1e-12)
    np.testing.assert_allclose(om.rope_transpose(y, cos, sin), x, atol=1e-13)
    # relative-position identity <R_m q, R_n k> = <R_{m-n} q, k>
    q = rng.standard_normal(Dh)
    k = rng.standard_normal(Dh)
    def rot(v, t):
        arr = np.zeros((1, T, 1, Dh)); arr[0, t, 0] = v
        return om.rope(arr, cos, sin)[0, t, 0]
    for m, n in [(10, 3), (40, 39), (7, 7)]:
        np.testing.assert_allclose(rot(q, m) @ rot(k, n), rot(q, m - n) @ k, rtol=1e-10)


def test_rope_complex_form():
    """Rotate-half RoPE = multiply z_i = x_i + 1j x_{i+half} by exp(1j t theta^(-2i/Dh))."""
    rng = np.random.default_rng(3)
    T, Dh, theta = 64, 128, 10000.0
    x = rng.standard_normal((1, T, 2, Dh))
    cos, sin = om.rope_angles(T, Dh, theta)
    y = om.rope(x, cos, sin)
    half = Dh // 2
    z = x[..., :half] + 1j * x[..., half:]
    t = np.arange(T)[None, :, None, None]
    i = np.arange(half)[None, None, None, :]
    zr = z * np.exp(1j * t * theta ** (-2.0 * i / Dh))
    np.testing.assert_allclose(y, np.concatenate([zr.real, zr.imag], -1), atol=1e-12)


# ---------------------------------------------------------------- attention
def _brute_attention(qh, kh, v):
    B, T, Hq, Dh = qh.shape
    g = Hq // kh.shape[2]
    o = np.zeros_like(qh)
    for b in range(B):
        for h in range(Hq):
            for t in range(T):
                s = [float(qh[b, t, h] @ kh[b, j, h // g]) / math.sqrt(Dh) for j in range(t + 1)]
                mx = max(s)
                w = [math.exp(si - mx) for si in s]
                tot = sum(w)
                o[b, t, h] = sum(w[j] / tot * v[b, j, h // g] for j in range(t + 1))
    return o


def test_attention_bruteforce_tiny():
    rng = np.random.default_rng(4)
    qh, kh, v = rng.standard_normal((1, 6, 4, 8)), rng.standard_normal((1, 6, 2, 8)), rng.standard_normal((1, 6, 2, 8))
    o, _ = om.attention(qh, kh, v)
    np.testing.assert_allclose(o, _brute_attention(qh, kh, v), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv", [(6, 2), (4, 4)])
def test_attention_matches_sdpa_and_autograd(Hq, Hkv):
    rng = np.random.default_rng(5)
    B, T, Dh = 2, 37, 16
    qh, kh, v = (rng.standard_normal((B, T, Hq, Dh)), rng.standard_normal((B, T, Hkv, Dh)),
                 rng.standard_normal((B, T, Hkv, Dh)))
    do = rng.standard_normal((B, T, Hq, Dh))
    o, lse = om.attention(qh, kh, v)
    qt, kt, vt = (_t(a).permute(0, 2, 1, 3).requires_grad_() for a in (qh, kh, v))
    ot = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, enable_gqa=(Hq != Hkv))
    np.testing.assert_allclose(o, ot.permute(0, 2, 1, 3).detach().numpy(), rtol=1e-11, atol=1e-12)
    s = torch.einsum("bhtd,bhjd->bhtj", qt, torch.repeat_interleave(kt, Hq // Hkv, 1)) / math.sqrt(Dh)
    s = s.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).detach().numpy(), rtol=1e-12)
    ot.backward(_t(do).permute(0, 2, 1, 3))
    dq, dk, dv = om.attention_bwd(qh, kh, v, do)
    np.testing.assert_allclose(dq, qt.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-11)


def test_attention_special_cases():
    rng = np.random.default_rng(6)
    qh, kh, v = rng.standard_normal((2, 1, 6, 8)), rng.standard_normal((2, 1, 2, 8)), rng.standard_normal((2, 1, 2, 8))
    o, _ = om.attention(qh, kh, v)                      # T = 1: output is v
    np.testing.assert_allclose(o, np.repeat(v, 3, axis=2), rtol=1e-14)
    # causality: changing positions > t leaves o[:t+1] unchanged
    qh, kh, v = rng.standard_normal((1, 20, 6, 8)), rng.standard_normal((1, 20, 2, 8)), rng.standard_normal((1, 20, 2, 8))
    o1, _ = om.attention(qh, kh, v)
    kh2, v2 = kh.copy(), v.copy()
    kh2[:, 11:] += 5.0
    v2[:, 11:] -= 3.0
    o2, _ = om.attention(qh, kh2, v2)
    np.testing.assert_array_equal(o1[:, :11], o2[:, :11])
    # unit-rms q_hat, k_hat bound the scores by sqrt(Dh)
    q = rng.standard_normal((1, 20, 6, 128)); k = rng.standard_normal((1, 20, 2, 128))
    qn, _ = om.qk_norm(q, 0.0); kn, _ = om.qk_norm(k, 0.0)
    s = np.einsum("bthd,bjhd->bhtj", qn, np.repeat(kn, 3, 2)) / math.sqrt(128)
    assert np.max(np.abs(s)) <= math.sqrt(128) * (1 + 1e-12)


def test_qknorm_backward_matches_autograd():
    rng = np.random.default_rng(7)
    x, d = rng.standard_normal((3, 5, 2, 16)), rng.standard_normal((3, 5, 2, 16))
    y, r = om.qk_norm(x, 1e-6)
    xt = _t(x).requires_grad_()
    yt = F.rms_norm(xt, (16,), eps=1e-6)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-13)
    yt.backward(_t(d))
    np.testing.assert_allclose(om.qk_norm_bwd(d, x, r), xt.grad.numpy(), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- the layer
SMALL = synth.LayerShape(batch=2, seq=24, d_model=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
                         d_ff=256, vocab=40, real_vocab=37, dtype="fp32", fp8_mlp=False,
                         value_embed=True)


def _torch_layer(inp, s, ids):
    """Independent float64 torch forward of the layer (library norm and attention, complex
    RoPE), used only through autograd as a second backward."""
    P = {k: _t(getattr(inp, k)).requires_grad_() for k in
         ("w_qkv", "w_o", "w_fc", "w_proj", "g_attn", "g_mlp", "ve_table")}
    P["a_attn"] = _t(float(inp.a_attn)).requires_grad_()
    P["a_mlp"] = _t(float(inp.a_mlp)).requires_grad_()
    x = _t(inp.x).requires_grad_()
    B, T, Hq, Hkv, Dh = s.batch, s.seq, s.n_q_heads, s.n_kv_heads, s.head_dim
    xn = F.rms_norm(x, (s.d_model,), weight=P["g_attn"], eps=s.rms_eps)
    q, k, v = torch.split(xn @ P["w_qkv"].T, [Hq * Dh, Hkv * Dh, Hkv * Dh], dim=1)
    v = v + P["ve_table"][torch.tensor(ids, dtype=torch.long)]
    q = F.rms_norm(q.reshape(B, T, Hq, Dh), (Dh,), eps=s.rms_eps)
    k = F.rms_norm(k.reshape(B, T, Hkv, Dh), (Dh,), eps=s.rms_eps)
    half = Dh // 2
    ang = torch.arange(T, dtype=torch.float64)[:, None] * s.rope_theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / Dh)
    rot = torch.polar(torch.ones_like(ang), ang)[None, :, None, :]
    def rope(a):
        z = torch.complex(a[..., :half], a[..., half:]) * rot
        return torch.cat([z.real, z.imag], -1)
    q, k = rope(q), rope(k)
    o = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2),
                                       v.reshape(B, T, Hkv, Dh).transpose(1, 2),
                                       is_causal=True, enable_gqa=True)
    h = x + P["a_attn"] * (o.transpose(1, 2).reshape(B * T, Hq * Dh) @ P["w_o"].T)
    hn = F.rms_norm(h, (s.d_model,), weight=P["g_mlp"], eps=s.rms_eps)
    y = h + P["a_mlp"] * (torch.relu(hn @ P["w_fc"].T) ** 2 @ P["w_proj"].T)
    return y, x, P


def test_layer_fp32_matches_torch_autograd():
    inp = synth.layer_inputs(SMALL, seed=11, perturb=True, w_std=0.1)
    p, d = om.params_from_inputs(inp), om.dims_from_shape(SMALL)
    y, cache = om.layer_fwd(p, inp.x, inp.ids, d)
    g = om.layer_bwd(p, cache, inp.dy, d)
    yt, xt, P = _torch_layer(inp, SMALL, inp.ids)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-11, atol=1e-11)
    yt.backward(_t(inp.dy))
    np.testing.assert_allclose(g["dx"], xt.grad.numpy(), rtol=1e-9, atol=1e-10)
    for k in ("w_qkv", "w_o", "w_fc", "w_proj", "g_attn", "g_mlp", "ve_table"):
        np.testing.assert_allclose(g[k], P[k].grad.numpy(), rtol=1e-9, atol=1e-10, err_msg=k)
    for k in ("a_attn", "a_mlp"):
        np.testing.assert_allclose(g[k], P[k].grad.item(), rtol=1e-9)


def test_layer_fp32_finite_differences():
    """Directional derivatives of the oracle's own forward vs its backward (central, h=1e-6)."""
    inp = synth.layer_inputs(SMALL, seed=12, perturb=True, w_std=0.1)
    p, d = om.params_from_inputs(inp), om.dims_from_shape(SMALL)
    rng = np.random.default_rng(12)
    dy = np.asarray(inp.dy, np.float64)
    y, cache = om.layer_fwd(p, inp.x, inp.ids, d)
    g = om.layer_bwd(p, cache, dy, d)
    L = lambda yy: float(np.sum(yy * dy))
    eps = 1e-6
    x0 = np.asarray(inp.x, np.float64)
    u = rng.standard_normal(x0.shape)
    fd = (L(om.layer_fwd(p, x0 + eps * u, inp.ids, d)[0]) - L(om.layer_fwd(p, x0 - eps * u, inp.ids, d)[0])) / (2 * eps)
    assert abs(fd - np.sum(g["dx"] * u)) <= 1e-7 * max(1.0, abs(fd))
    for name in ("w_qkv", "w_o", "w_fc", "w_proj", "g_attn", "g_mlp", "ve_table", "a_attn", "a_mlp"):
        base = getattr(p, name)
        u = rng.standard_normal(np.shape(base))
        def f(sign):
            q = om.LayerParams(**{**p.__dict__, name: base + sign * eps * u})
            return L(om.layer_fwd(q, x0, inp.ids, d)[0])
        fd = (f(1) - f(-1)) / (2 * eps)
        an = float(np.sum(np.asarray(g[name]) * u))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), name


def test_layer_zero_residual_scalars():
    inp = synth.layer_inputs(SMALL, seed=13, perturb=True, w_std=0.1)
    p, d = om.params_from_inputs(inp), om.dims_from_shape(SMALL)
    p.a_mlp = 0.0
    y, cache = om.layer_fwd(p, inp.x, inp.ids, d)
    np.testing.assert_array_equal(y, cache["h"])
    g = om.layer_bwd(p, cache, inp.dy, d)
    assert not np.any(g["w_fc"]) and not np.any(g["w_proj"]) and not np.any(g["g_mlp"])
    p.a_attn = 0.0
    y, cache = om.layer_fwd(p, inp.x, inp.ids, d)
    np.testing.assert_array_equal(y, np.asarray(inp.x, np.float64))
    g = om.layer_bwd(p, cache, inp.dy, d)
    np.testing.assert_array_equal(g["dx"], np.asarray(inp.dy, np.float64))
    assert not np.any(g["w_qkv"]) and not np.any(g["ve_table"])


def test_value_embedding_gather_and_scatter():
    rng = np.random.default_rng(14)
    table = rng.standard_normal((10, 6))
    ids = np.array([3, 3, 7, 0, 3, 9])
    onehot = np.eye(10)[ids]
    np.testing.assert_array_equal(table[ids], onehot @ table)
    dv = rng.standard_normal((6, 6))
    acc = np.zeros_like(table)
    np.add.at(acc, ids, dv)
    np.testing.assert_allclose(acc, onehot.T @ dv, rtol=1e-14)
    assert np.allclose(acc[3], dv[0] + dv[1] + dv[4])


# ---------------------------------------------------------------- bf16 / FP8 mode
def test_bf16_mode_stored_tensors_are_bf16():
    s = synth.LayerShape(batch=1, seq=32, d_model=128, n_q_heads=4, n_kv_heads=2, head_dim=32,
                         d_ff=512, vocab=64, real_vocab=60, dtype="bf16", fp8_mlp=True,
                         value_embed=True)
    inp = synth.layer_inputs(s, seed=15, perturb=True)
    p, d = om.params_from_inputs(inp), om.dims_from_shape(s)
    y, c = om.layer_fwd(p, inp.x, inp.ids, d)
    g = om.layer_bwd(p, c, inp.dy, d)
    for a in (y, c["xn"], c["h"], c["hn"], c["u"], c["r"], c["m"], c["o"], c["qh"], g["dx"], g["w_qkv"], g["w_fc"]):
        np.testing.assert_array_equal(a, nu.bf16_round(a))


def test_fp8_mlp_exact_when_operands_representable():
    """If hn and W1 are e4m3 values times a power of two with amax = 448 * 2^k, quantisation is
    exact, so the FP8 first GEMM equals the plain GEMM."""
    rng = np.random.default_rng(16)
    vals = nu.e4m3_decode(np.arange(0, 127))
    hn = rng.choice(np.concatenate([vals, -vals]), size=(16, 64)) * 2.0 ** -5
    hn[0, 0] = 448 * 2.0 ** -5
    w1 = rng.choice(np.concatenate([vals, -vals]), size=(96, 64)) * 2.0 ** -12
    w1[0, 0] = -448 * 2.0 ** -12
    w2 = rng.standard_normal((64, 96)) * 0.02
    R = om.rounder("bf16")
    _, c8 = om.mlp_fwd(hn, w1, w2, True, R)
    _, c16 = om.mlp_fwd(hn, w1, w2, False, R)
    np.testing.assert_array_equal(c8["u"], c16["u"])
    np.testing.assert_array_equal(c8["hn8"] * c8["inv_hn"], hn)


def test_fp8_mlp_close_to_bf16_mlp():
    """e4m3 keeps 4 significant bits: the FP8 MLP stays within a few percent of the bf16 one,
    and its gradients too (a missing dequantisation scale would be off by orders of magnitude)."""
    rng = np.random.default_rng(17)
    hn = nu.bf16_round(rng.standard_normal((128, 256)))
    w1 = nu.bf16_round(rng.standard_normal((1024, 256)) * 0.02)
    w2 = nu.bf16_round(rng.standard_normal((256, 1024)) * 0.02)
    dm = nu.bf16_round(rng.standard_normal((128, 256)))
    R = om.rounder("bf16")
    m8, c8 = om.mlp_fwd(hn, w1, w2, True, R)
    m16, c16 = om.mlp_fwd(hn, w1, w2, False, R)
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(m8, m16) < 0.08
    g8 = om.mlp_bwd(dm, c8, w1, w2, True, R)
    g16 = om.mlp_bwd(dm, c16, w1, w2, False, R)
    for a, b in zip(g8, g16):
        assert rel(a, b) < 0.08


def test_gather_and_scatter_rows_out_of_range_ids():
    """ids outside the table pick zero rows and receive nothing; in-range ids are the one-hot
    products (gather = onehot @ table, scatter = onehot^T @ d)."""
    rng = np.random.default_rng(19)
    table = rng.standard_normal((6, 3))
    ids = np.array([2, -1, 5, 6, 2, 10**6, 0])
    ok = (ids >= 0) & (ids < 6)
    onehot = np.zeros((len(ids), 6))
    onehot[np.arange(len(ids))[ok], ids[ok]] = 1.0
    np.testing.assert_array_equal(om.gather_rows(table, ids), onehot @ table)
    d = rng.standard_normal((len(ids), 3))
    np.testing.assert_allclose(om.scatter_rows(d, ids, 6), onehot.T @ d, rtol=1e-14)


# ---------------------------------------------------------------- SwiGLU variant
def test_swiglu_mlp_matches_torch_autograd():
    """The gated MLP against torch float64 (F.silu, autograd as an independent backward)."""
    rng = np.random.default_rng(20)
    N, D, F = 12, 32, 40
    hn = rng.standard_normal((N, D))
    w_fc = rng.standard_normal((2 * F, D)) * 0.3
    w_proj = rng.standard_normal((D, F)) * 0.3
    dm = rng.standard_normal((N, D))
    R = om.rounder("fp32")
    m, c = om.swiglu_mlp_fwd(hn, w_fc, w_proj, R)
    dhn, dw_fc, dw_proj = om.swiglu_mlp_bwd(dm, c, w_fc, w_proj, R)
    th, t1, t2 = _t(hn).requires_grad_(), _t(w_fc).requires_grad_(), _t(w_proj).requires_grad_()
    gu = th @ t1.T
    mt = (F_silu(gu[:, :F]) * gu[:, F:]) @ t2.T
    np.testing.assert_allclose(m, mt.detach().numpy(), rtol=1e-12, atol=1e-12)
    mt.backward(_t(dm))
    np.testing.assert_allclose(dhn, th.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dw_fc, t1.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dw_proj, t2.grad.numpy(), rtol=1e-10, atol=1e-12)


def F_silu(x):
    return torch.nn.functional.silu(x)


def test_swiglu_layer_finite_differences_and_planted_mistake(monkeypatch):
    """The whole layer with the SwiGLU MLP in fp32 mode: central finite differences along random
    directions of x and both MLP weights; a planted mistake (silu'(g) taken as sigmoid(g)) fails."""
    s = synth.LayerShape(batch=1, seq=12, d_model=32, n_q_heads=4, n_kv_heads=2, head_dim=8, d_ff=24, vocab=40,
                         real_vocab=40, dtype="fp32", fp8_mlp=False, value_embed=False, mlp="swiglu")
    inp = synth.layer_inputs(s, seed=21, perturb=True, w_std=0.2)
    p, d = om.params_from_inputs(inp), om.dims_from_shape(s)
    assert p.w_fc.shape == (48, 32)
    rng = np.random.default_rng(21)
    dy = np.asarray(inp.dy, np.float64)
    y, cache = om.layer_fwd(p, inp.x, inp.ids, d)
    g = om.layer_bwd(p, cache, dy, d)
    L = lambda yy: float(np.sum(yy * dy))
    eps = 1e-6
    x0 = np.asarray(inp.x, np.float64)
    for name in ("x", "w_fc", "w_proj"):
        base = x0 if name == "x" else getattr(p, name)
        u = rng.standard_normal(np.shape(base))
        def f(sign):
            if name == "x":
                return L(om.layer_fwd(p, x0 + sign * eps * u, inp.ids, d)[0])
            q = om.LayerParams(**{**p.__dict__, name: base + sign * eps * u})
            return L(om.layer_fwd(q, x0, inp.ids, d)[0])
        fd = (f(1) - f(-1)) / (2 * eps)
        an = float(np.sum(np.asarray(g["dx" if name == "x" else name]) * u))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), name
    # planted: the gradient through silu without its (1 + g (1 - s)) factor
    real_exp = np.exp
    calls = {"n": 0}
    def planted_bwd(dm, c, w_fc, w_proj, R):
        F_ = w_proj.shape[1]
        gg, uu = c["gu"][:, :F_], c["gu"][:, F_:]
        da = R(dm @ w_proj)
        sg = 1.0 / (1.0 + real_exp(-gg))
        dgu = R(np.concatenate([da * uu * sg, da * gg * sg], axis=1))
        return R(dgu @ w_fc), R(dgu.T @ c["hn"]), R(dm.T @ c["a"])
    monkeypatch.setattr(om, "swiglu_mlp_bwd", planted_bwd)
    gb = om.layer_bwd(p, cache, dy, d)
    u = rng.standard_normal(x0.shape)
    fd = (L(om.layer_fwd(p, x0 + eps * u, inp.ids, d)[0]) - L(om.layer_fwd(p, x0 - eps * u, inp.ids, d)[0])) / (2 * eps)
    assert abs(fd - float(np.sum(gb["dx"] * u))) > 1e-4 * abs(fd)
