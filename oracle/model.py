"""ORACLE (test infrastructure only): one little-lm decoder layer, forward and backward, float64.

The layer [hn.213312.xyz translation, "设置 / Setup"; youdonthavefriends cost analysis, "config
appendix"]: Llama-style pre-norm block with RMSNorm (eps 1e-6), RoPE (theta 10000), GQA with 24
query / 8 key-value heads of dim 128 (group 3), QK-norm, causal softmax attention
(scaled_dot_product_attention with is_causal=True [hn.213312.xyz translation, "不起作用的部分 /
What didn't work"]), a non-gated relu^2 MLP 3072 -> 12288 -> 3072, learnable per-layer residual
scalars (layer_scale: true), and on value-embedding layers a vocab x kv_dim table whose rows,
picked by the input token ids, are added to V (ResFormer-style value embeddings, 14 tables on
alternate layers).

Readings taken where the pages are silent (each listed in the design notes):
  * norm gains on the two pre-norms (init 1), QK-norm without gain, no biases — the only reading
    that reproduces the page's 2,818.7M parameters for 28 layers [hn.213312.xyz translation,
    "设置 / Setup", parameter table];
  * QK-norm uses the same eps as the block norms; RoPE pairs channel i with i + Dh/2
    ("rotate-half"), positions restart at 0 in every row of the batch  (parity unpinned: a
    pairing convention is not fixed by the pages);
  * residual scalars multiply the branch outputs: h = x + a_attn * Attn(RMSNorm(x)),
    y = h + a_mlp * MLP(RMSNorm(h))  (parity unpinned: the pages only say "scalar");
  * value embedding: v <- v + E[ids], no gate, before attention; V is neither normed nor rotated;
  * FP8 (see oracle.numerics) on the three GEMMs of each MLP linear: forward, input-gradient and
    weight-gradient; quantisation is straight-through in the backward.

Rounding contract of bf16 mode (mode="bf16"): every GEMM output is rounded to bf16 before any
epilogue math; every elementwise chain is evaluated exactly and rounded to bf16 once, where the
GPU path stores it (xn, qkv, v+VE, q_hat/k_hat, o, attn_out, h, hn, u, r, m, y, dm, dr, du, dhn,
dh, dattn, do, dq/dk/dv, dxn, dx); reductions (rstd, softmax, amax, dg, da, dE_ve, dW) are not
rounded except the final weight gradients, rounded once to bf16. mode="fp32" rounds nothing.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import bf16_round, quantize_tensorwise


def rounder(mode: str):
    if mode == "bf16":
        return bf16_round
    if mode == "fp32":
        return lambda a: np.asarray(a, dtype=np.float64)
    raise ValueError(mode)


# ----------------------------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------------------------
def rmsnorm(x, g, eps):
    """y = x * r * g with r = (mean over the last axis of x^2 + eps)^(-1/2). Returns (y, r)."""
    x = np.asarray(x, np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    return x * r[..., None] * np.asarray(g, np.float64), r


def rmsnorm_bwd(d, x, g, r):
    """Gradients of y = x*r*g given dL/dy = d: (dL/dx, dL/dg summed over all leading axes).

    dL/dx = r*(g*d) - x*r^3*mean(x*g*d);  dL/dg = sum(d * x * r).
    """
    d = np.asarray(d, np.float64)
    x = np.asarray(x, np.float64)
    g = np.asarray(g, np.float64)
    gd = g * d
    dx = r[..., None] * gd - x * (r ** 3)[..., None] * np.mean(x * gd, axis=-1)[..., None]
    dg = np.sum((d * x * r[..., None]).reshape(-1, x.shape[-1]), axis=0)
    return dx, dg


# ----------------------------------------------------------------------------------------------
# RoPE and QK-norm
# ----------------------------------------------------------------------------------------------
def rope_angles(seq: int, head_dim: int, theta: float):
    """cos, sin of phi[t, i] = t * theta^(-2i/head_dim), t < seq, i < head_dim/2 (float64)."""
    half = head_dim // 2
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / head_dim)
    phi = np.arange(seq, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(phi), np.sin(phi)


def rope(x, cos, sin):
    """Rotate pairs (x_i, x_{i+half}) of x [B, T, H, Dh] by phi[t, i]."""
    half = x.shape[-1] // 2
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def rope_transpose(d, cos, sin):
    """Adjoint of `rope` (rotation by -phi): maps dL/d(rope(x)) to dL/dx."""
    half = d.shape[-1] // 2
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    a, b = d[..., :half], d[..., half:]
    return np.concatenate([a * c + b * s, -a * s + b * c], axis=-1)


def qk_norm(x, eps):
    """Gain-free per-head RMS normalisation over the head dimension. Returns (x*r, r)."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    return x * r[..., None], r


def qk_norm_bwd(d, x, r):
    """Adjoint of qk_norm: r*d - x*r^3*mean(x*d) per head."""
    return r[..., None] * d - x * (r ** 3)[..., None] * np.mean(x * d, axis=-1)[..., None]


# ----------------------------------------------------------------------------------------------
# causal GQA attention
# ----------------------------------------------------------------------------------------------
def _expand_kv(k, n_q_heads):
    g = n_q_heads // k.shape[2]
    return np.repeat(k, g, axis=2)           # q head h reads kv head h // g


def attention_probs(qh, kh):
    """P[b, h, t, j] = softmax_j(q_t . k_j / sqrt(Dh)) over j <= t. Also returns lse[b, h, t]."""
    B, T, Hq, Dh = qh.shape
    k = _expand_kv(kh, Hq)
    s = np.einsum("bthd,bjhd->bhtj", qh, k) / np.sqrt(Dh)
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)       # key j > query t
    s = np.where(mask[None, None], -np.inf, s)
    mx = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - mx)
    tot = np.sum(e, axis=-1, keepdims=True)
    return e / tot, (mx + np.log(tot))[..., 0]


def attention(qh, kh, v):
    """o[b, t, h] = sum_j P[b, h, t, j] v[b, j, h // g]; returns (o [B,T,Hq,Dh], lse [B,Hq,T])."""
    p, lse = attention_probs(qh, kh)
    o = np.einsum("bhtj,bjhd->bthd", p, _expand_kv(v, qh.shape[2]))
    return o, lse


def attention_bwd(qh, kh, v, do):
    """Softmax-attention backward: (dq_hat, dk_hat, dv); kv grads summed over each group."""
    B, T, Hq, Dh = qh.shape
    Hkv = kh.shape[2]
    g = Hq // Hkv
    p, _ = attention_probs(qh, kh)
    kx, vx = _expand_kv(kh, Hq), _expand_kv(v, Hq)
    dvx = np.einsum("bhtj,bthd->bjhd", p, do)
    dp = np.einsum("bthd,bjhd->bhtj", do, vx)
    ds = p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
    sc = 1.0 / np.sqrt(Dh)
    dq = np.einsum("bhtj,bjhd->bthd", ds, kx) * sc
    dkx = np.einsum("bhtj,bthd->bjhd", ds, qh) * sc
    dk = dkx.reshape(B, T, Hkv, g, Dh).sum(axis=3)
    dv = dvx.reshape(B, T, Hkv, g, Dh).sum(axis=3)
    return dq, dk, dv


# ----------------------------------------------------------------------------------------------
# relu^2 MLP, optionally with FP8 GEMMs
# ----------------------------------------------------------------------------------------------
def mlp_fwd(hn, w_fc, w_proj, fp8: bool, R):
    """m = relu(hn W1^T)^2 W2^T. With fp8, each GEMM takes dynamically quantised e4m3 operands
    and is dequantised by the product of the inverse scales. Returns (m, cache)."""
    if fp8:
        _, hn8, _, inv_hn = quantize_tensorwise(hn)
        _, w18, _, inv_w1 = quantize_tensorwise(w_fc)
        u = R((hn8 @ w18.T) * inv_hn * inv_w1)
        r = R(np.maximum(u, 0.0) ** 2)
        _, r8, _, inv_r = quantize_tensorwise(r)
        _, w28, _, inv_w2 = quantize_tensorwise(w_proj)
        m = R((r8 @ w28.T) * inv_r * inv_w2)
        return m, dict(hn=hn, u=u, r=r, m=m, hn8=hn8, inv_hn=inv_hn, w18=w18, inv_w1=inv_w1,
                       r8=r8, inv_r=inv_r, w28=w28, inv_w2=inv_w2)
    u = R(hn @ w_fc.T)
    r = R(np.maximum(u, 0.0) ** 2)
    m = R(r @ w_proj.T)
    return m, dict(hn=hn, u=u, r=r, m=m)


def mlp_bwd(dm, c, w_fc, w_proj, fp8: bool, R):
    """Backward of mlp_fwd given dL/dm (straight-through quantisation): (dhn, dW1, dW2).
    With fp8, dm and du are quantised and every GEMM takes the e4m3 operands of the forward
    (one forward and two backward GEMMs per linear)."""
    if fp8:
        _, dm8, _, inv_dm = quantize_tensorwise(dm)
        dr = R((dm8 @ c["w28"]) * inv_dm * c["inv_w2"])
        dw2 = R((dm8.T @ c["r8"]) * inv_dm * c["inv_r"])
    else:
        dr = R(dm @ w_proj)
        dw2 = R(dm.T @ c["r"])
    du = R(dr * 2.0 * np.maximum(c["u"], 0.0))
    if fp8:
        _, du8, _, inv_du = quantize_tensorwise(du)
        dw1 = R((du8.T @ c["hn8"]) * inv_du * c["inv_hn"])
        dhn = R((du8 @ c["w18"]) * inv_du * c["inv_w1"])
    else:
        dw1 = R(du.T @ c["hn"])
        dhn = R(du @ w_fc)
    return dhn, dw1, dw2


# ----------------------------------------------------------------------------------------------
# SwiGLU MLP (the gated variant the run replaced by relu^2)
# ----------------------------------------------------------------------------------------------
def silu(x):
    """x * sigmoid(x)."""
    return x / (1.0 + np.exp(-x))


def swiglu_mlp_fwd(hn, w_fc, w_proj, R):
    """The gated MLP the pages ablated against relu^2 [linlog.top article, 吞吐量优化: SwiGLU has
    three matmuls where relu^2 has two; manulx summary: intermediate ratio 2.75 for SwiGLU, 4x for
    the non-gated MLP]: with w_fc [2F, D] holding the gate rows then the up rows,
    [g | u] = hn w_fc^T,  a = silu(g) * u,  m = a w_proj^T  (w_proj [D, F]).
    Rounded where the GPU path stores: [g | u], a, m. Returns (m, cache)."""
    F = w_proj.shape[1]
    gu = R(hn @ w_fc.T)
    g, u = gu[:, :F], gu[:, F:]
    a = R(silu(g) * u)
    m = R(a @ w_proj.T)
    return m, dict(hn=hn, gu=gu, a=a, m=m)


def swiglu_mlp_bwd(dm, c, w_fc, w_proj, R):
    """Backward of swiglu_mlp_fwd: da = dm w_proj; dg = da u silu'(g), du = da silu(g) with
    silu'(g) = s (1 + g (1 - s)), s = sigmoid(g); returns (dhn, dW_fc, dW_proj)."""
    F = w_proj.shape[1]
    g, u = c["gu"][:, :F], c["gu"][:, F:]
    da = R(dm @ w_proj)
    sg = 1.0 / (1.0 + np.exp(-g))
    dgu = R(np.concatenate([da * u * sg * (1.0 + g * (1.0 - sg)), da * g * sg], axis=1))
    dw_proj = R(dm.T @ c["a"])
    dw_fc = R(dgu.T @ c["hn"])
    dhn = R(dgu @ w_fc)
    return dhn, dw_fc, dw_proj


# ----------------------------------------------------------------------------------------------
# table rows picked by token ids (value embeddings; the model's token embedding)
# ----------------------------------------------------------------------------------------------
def gather_rows(table, ids):
    """out[n] = table[ids[n]]; an id outside [0, rows) picks a zero row (the library's contract for
    ids it cannot look up; the pages only ever index in range)."""
    table = np.asarray(table, np.float64)
    ids = np.asarray(ids, np.int64)
    ok = (ids >= 0) & (ids < table.shape[0])
    return np.where(ok[:, None], table[np.where(ok, ids, 0)], 0.0)


def scatter_rows(d, ids, rows):
    """dT[v] = sum of d[n] over the n with ids[n] = v (ids outside [0, rows) add nothing)."""
    d = np.asarray(d, np.float64)
    ids = np.asarray(ids, np.int64)
    ok = (ids >= 0) & (ids < rows)
    out = np.zeros((rows, d.shape[1]), np.float64)
    np.add.at(out, ids[ok], d[ok])
    return out


# ----------------------------------------------------------------------------------------------
# the layer
# ----------------------------------------------------------------------------------------------
@dataclass
class LayerParams:
    w_qkv: np.ndarray      # [(Hq + 2 Hkv) * Dh, D]: q rows, then k rows, then v rows, head-major
    w_o: np.ndarray        # [D, Hq * Dh]
    w_fc: np.ndarray       # [F, D] ([2F, D] for SwiGLU: gate rows, then up rows)
    w_proj: np.ndarray     # [D, F]
    g_attn: np.ndarray     # [D]
    g_mlp: np.ndarray      # [D]
    a_attn: float
    a_mlp: float
    ve_table: np.ndarray | None = None    # [vocab, Hkv * Dh] or None


@dataclass
class LayerDims:
    batch: int
    seq: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    fp8_mlp: bool = False
    mode: str = "bf16"
    mlp: str = "relu2"        # "relu2" (the run's MLP) or "swiglu" (the ablated gated variant)


def params_from_inputs(inp) -> LayerParams:
    """Adapter from synth.LayerInputs (plain arrays) to LayerParams."""
    f = lambda a: None if a is None else np.asarray(a, np.float64)
    return LayerParams(f(inp.w_qkv), f(inp.w_o), f(inp.w_fc), f(inp.w_proj), f(inp.g_attn),
                       f(inp.g_mlp), float(inp.a_attn), float(inp.a_mlp), f(inp.ve_table))


def dims_from_shape(s) -> LayerDims:
    return LayerDims(s.batch, s.seq, s.n_q_heads, s.n_kv_heads, s.head_dim, s.rms_eps,
                     s.rope_theta, bool(s.fp8_mlp), s.dtype, getattr(s, "mlp", "relu2"))


def layer_fwd(p: LayerParams, x, ids, d: LayerDims):
    """Forward of one decoder layer on x [B*T, D]. Returns (y [B*T, D], cache for layer_bwd)."""
    R = rounder(d.mode)
    x = np.asarray(x, np.float64)
    N, D = x.shape
    B, T, Hq, Hkv, Dh = d.batch, d.seq, d.n_q_heads, d.n_kv_heads, d.head_dim
    c = {}
    xn_raw, r1 = rmsnorm(x, p.g_attn, d.rms_eps)
    xn = R(xn_raw)
    qkv = R(xn @ p.w_qkv.T)
    q = qkv[:, : Hq * Dh].reshape(B, T, Hq, Dh)
    k = qkv[:, Hq * Dh:(Hq + Hkv) * Dh].reshape(B, T, Hkv, Dh)
    v = qkv[:, (Hq + Hkv) * Dh:]
    if p.ve_table is not None:
        v = R(v + gather_rows(p.ve_table, ids))
    v = v.reshape(B, T, Hkv, Dh)
    cos, sin = rope_angles(T, Dh, d.rope_theta)
    qt, rq = qk_norm(q, d.rms_eps)
    kt, rk = qk_norm(k, d.rms_eps)
    qh, kh = R(rope(qt, cos, sin)), R(rope(kt, cos, sin))
    o4, lse = attention(qh, kh, v)
    o = R(o4.reshape(N, Hq * Dh))
    attn_out = R(o @ p.w_o.T)
    h = R(x + p.a_attn * attn_out)
    hn_raw, r2 = rmsnorm(h, p.g_mlp, d.rms_eps)
    hn = R(hn_raw)
    if d.mlp == "swiglu":
        m, mc = swiglu_mlp_fwd(hn, p.w_fc, p.w_proj, R)
    else:
        m, mc = mlp_fwd(hn, p.w_fc, p.w_proj, d.fp8_mlp, R)
    c.update(mc)
    y = R(h + p.a_mlp * m)
    c.update(x=x, ids=ids, xn=xn, r1=r1, q=q, k=k, v=v, rq=rq, rk=rk, qh=qh, kh=kh, o=o, lse=lse,
             attn_out=attn_out, h=h, hn=hn, r2=r2, cos=cos, sin=sin)
    return y, c


def layer_bwd(p: LayerParams, c: dict, dy, d: LayerDims):
    """Backward of one decoder layer given dL/dy. Returns a dict of gradients:
    dx [N, D]; w_qkv, w_o, w_fc, w_proj (matrix grads); g_attn, g_mlp [D]; a_attn, a_mlp
    (scalars); ve_table [vocab, Hkv*Dh] (or None)."""
    R = rounder(d.mode)
    dy = np.asarray(dy, np.float64)
    N, D = dy.shape
    B, T, Hq, Hkv, Dh = d.batch, d.seq, d.n_q_heads, d.n_kv_heads, d.head_dim
    g = {}
    # MLP residual branch
    g["a_mlp"] = float(np.sum(dy * c["m"]))
    dm = R(p.a_mlp * dy)
    if d.mlp == "swiglu":
        dhn, g["w_fc"], g["w_proj"] = swiglu_mlp_bwd(dm, c, p.w_fc, p.w_proj, R)
    else:
        dhn, g["w_fc"], g["w_proj"] = mlp_bwd(dm, c, p.w_fc, p.w_proj, d.fp8_mlp, R)
    dh_norm, g["g_mlp"] = rmsnorm_bwd(dhn, c["h"], p.g_mlp, c["r2"])
    dh = R(dy + dh_norm)
    # attention residual branch
    g["a_attn"] = float(np.sum(dh * c["attn_out"]))
    dattn = R(p.a_attn * dh)
    do = R(dattn @ p.w_o)
    g["w_o"] = R(dattn.T @ c["o"])
    dqh, dkh, dv = attention_bwd(c["qh"], c["kh"], c["v"], do.reshape(B, T, Hq, Dh))
    dv = R(dv.reshape(N, Hkv * Dh))
    dq = R(qk_norm_bwd(rope_transpose(dqh, c["cos"], c["sin"]), c["q"], c["rq"]))
    dk = R(qk_norm_bwd(rope_transpose(dkh, c["cos"], c["sin"]), c["k"], c["rk"]))
    if p.ve_table is not None:
        g["ve_table"] = scatter_rows(dv, c["ids"], p.ve_table.shape[0])
    else:
        g["ve_table"] = None
    dqkv = np.concatenate([dq.reshape(N, -1), dk.reshape(N, -1), dv], axis=1)
    dxn = R(dqkv @ p.w_qkv)
    g["w_qkv"] = R(dqkv.T @ c["xn"])
    dx_norm, g["g_attn"] = rmsnorm_bwd(dxn, c["x"], p.g_attn, c["r1"])
    g["dx"] = R(dh + dx_norm)
    g["dqkv"] = dqkv
    g["dh"] = dh
    return g
