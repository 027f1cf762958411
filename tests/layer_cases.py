"""Runs one decoder layer (and optionally the loss chained after it) on the GPU through the C ABI
and in the oracle, on the same seeded inputs. Shared by the GPU parity tests and the smoke check."""
from __future__ import annotations

import numpy as np
import torch

import synth
from oracle import lce as olce
from oracle import model as om
from transformer_train_step_amd.ops import FusedLCE, Layer, LayerConfig

GRAD_KEYS = ("w_qkv", "w_o", "w_fc", "w_proj", "g_attn", "g_mlp", "a_attn", "a_mlp", "ve_table")
GPU_NAME = {"g_attn": "attn_norm_w", "g_mlp": "mlp_norm_w", "a_attn": "resid_attn", "a_mlp": "resid_mlp"}


def config_of(s: synth.LayerShape) -> LayerConfig:
    return LayerConfig(batch=s.batch, seq=s.seq, d_model=s.d_model, n_q_heads=s.n_q_heads,
                       n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, d_ff=s.d_ff, dtype=s.dtype,
                       fp8_mlp=s.fp8_mlp, value_embed=s.value_embed, ve_rows=s.vocab,
                       rms_eps=s.rms_eps, rope_theta=s.rope_theta, mlp=s.mlp)


def _dev(a, dt):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return (t.to(torch.bfloat16) if dt == "bf16" else t).cuda()


def _host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def device_params(inp: synth.LayerInputs) -> dict:
    dt = inp.shape.dtype
    p = {"attn_norm_w": torch.from_numpy(inp.g_attn).cuda(), "mlp_norm_w": torch.from_numpy(inp.g_mlp).cuda(),
         "w_qkv": _dev(inp.w_qkv, dt), "w_o": _dev(inp.w_o, dt), "w_fc": _dev(inp.w_fc, dt),
         "w_proj": _dev(inp.w_proj, dt),
         "resid_attn": torch.tensor([float(inp.a_attn)], dtype=torch.float32, device="cuda"),
         "resid_mlp": torch.tensor([float(inp.a_mlp)], dtype=torch.float32, device="cuda")}
    if inp.ve_table is not None:
        p["ve_table"] = _dev(inp.ve_table, dt)
    return p


def run_gpu(inp: synth.LayerInputs, dy=None, lce_head=None):
    """Layer fwd (+ optional LCE on y with lce_head = (weight, targets)) + bwd on the GPU."""
    s = inp.shape
    layer = Layer(config_of(s))
    p = device_params(inp)
    x = _dev(inp.x, s.dtype)
    ids = torch.from_numpy(inp.ids).cuda()
    y = layer.forward(p, x, ids)
    out = {"y": y}
    if lce_head is not None:
        w_head, targets = lce_head
        lce = FusedLCE(s.dtype, s.tokens, s.d_model, w_head.shape[0], token_chunk=0)
        loss, dh, dw = lce(y, _dev(w_head, s.dtype), torch.from_numpy(targets).cuda())
        out.update(loss=loss, d_head=dw)
        dy_dev = dh
    else:
        dy_dev = _dev(inp.dy if dy is None else dy, s.dtype)
    dx, g = layer.backward(p, x, ids, dy_dev)
    torch.cuda.synchronize()
    res = {"y": _host(y), "dx": _host(dx), "dy": _host(dy_dev), "ids": inp.ids}
    for k in GRAD_KEYS:
        name = GPU_NAME.get(k, k)
        if name in g:
            res[k] = _host(g[name]) if name not in ("resid_attn", "resid_mlp") else float(g[name].item())
    if lce_head is not None:
        res["loss"] = float(out["loss"].item())
        res["d_head"] = _host(out["d_head"])
    return res


def run_oracle(inp: synth.LayerInputs, dy=None, lce_head=None):
    s = inp.shape
    p, d = om.params_from_inputs(inp), om.dims_from_shape(s)
    y, cache = om.layer_fwd(p, inp.x, inp.ids, d)
    res = {"y": y}
    if lce_head is not None:
        w_head, targets = lce_head
        o = olce.lce_fwd_bwd(y, w_head, targets, softcap=15.0, mode=s.dtype)
        dy = o["dh"]
        res.update(loss=o["loss"], d_head=o["dw"])
    elif dy is None:
        dy = inp.dy
    g = om.layer_bwd(p, cache, dy, d)
    res["dx"] = g["dx"]
    res["dy"] = np.asarray(dy, np.float64)
    # natural scales of the residual-scalar gradients (Cauchy-Schwarz bounds of the two sums)
    res["scale_a_mlp"] = float(np.linalg.norm(res["dy"]) * np.linalg.norm(cache["m"]))
    res["scale_a_attn"] = float(np.linalg.norm(g["dh"]) * np.linalg.norm(cache["attn_out"]))
    for k in GRAD_KEYS:
        if g.get(k) is not None:
            res[k] = g[k]
    return res
