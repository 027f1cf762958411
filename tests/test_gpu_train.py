"""GPU parity of the rest of the single-GPU training step: gradient accumulation over micro-batches
through ll_model_fwd_bwd (the first call overwrites, the others add), and the optimizer step of
ops.TrainStep (Muon on every layer matrix, AdamW on the embedding, head, value-embedding tables,
gains and residual scalars, bf16 master weights), against oracle.full_model and oracle.optim.

The optimizer is checked on the GPU's own accumulated gradients (AdamW's first step moves each
weight by about lr sign(g), so a gradient element that is zero within rounding could flip the
update on either side; the gradients themselves are checked against the oracle's separately)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from oracle import full_model as fm
from oracle import model as om
from oracle import numerics as nu
from oracle import optim as oo
from tests.gpu_util import assert_close, dev, error_stats, host, need_gpu, rel_err
from tests.layer_cases import GPU_NAME, config_of, device_params
from tests.test_gpu_optim import FLIP_FRAC, _ulp_close, check_muon_w, f32

# Muon on the gradients of a real step. Such gradients are ill-conditioned (their singular values
# span several decades), and the Newton-Schulz polynomial's slope at zero is a = 3.4445, so a
# component at rounding level grows up to a^5 ~ 490x over the five steps before the polynomial
# saturates it near 1: where the GPU's fp32 sums and the oracle's float64 sums round an iterate to
# different bf16 values, those directions of the result differ by a few percent of the update.
# Measured on this model: the updates agree to 2.1-3.4% norm-wise, the worst element of w_new is
# 0.124 x (|update| + rms(update)) beyond one ulp; the bounds leave 2x. (Muon itself is checked on
# well-conditioned inputs to 0.1 in test_gpu_optim.)
TRAIN_MUON_ELEM, TRAIN_MUON_RTOL = 0.25, 7e-2
from transformer_train_step_amd.ops import ADAMW, MATRICES, MUON, Model, TrainStep

pytestmark = pytest.mark.gpu


def _model_inputs(s, n_layers, seed, n_batches):
    mi = synth.model_inputs(s, n_layers, seed=seed, perturb=True)
    batches = [(synth.uniform_ints((s.tokens,), s.real_vocab, seed, 200 + i),
                synth.uniform_ints((s.tokens,), s.real_vocab, seed, 300 + i)) for i in range(n_batches)]
    return mi, batches


def _device_params(mi):
    s = mi.shape
    return {"embed": dev(mi.embed, s.dtype), "layers": [device_params(li) for li in mi.layers],
            "final_norm_w": torch.from_numpy(mi.g_final.copy()).cuda(), "head": dev(mi.head, s.dtype)}


def _oracle_sum(mi, batches, scale):
    """Sum over the micro-batches of the oracle's gradients of scale * loss."""
    f = lambda a: np.asarray(a, np.float64)
    p = fm.ModelParams(f(mi.embed), [om.params_from_inputs(li) for li in mi.layers], f(mi.g_final), f(mi.head))
    tot = None
    for ids, tg in batches:
        r = fm.model_fwd_bwd(p, ids, tg, om.dims_from_shape(mi.shape), grad_scale=scale)
        if tot is None:
            tot = r
            continue
        for k in ("embed", "g_final", "head"):
            tot[k] = tot[k] + r[k]
        for a, b in zip(tot["layers"], r["layers"]):
            for k in ("w_qkv", "w_o", "w_fc", "w_proj", "g_attn", "g_mlp", "a_attn", "a_mlp"):
                a[k] = a[k] + b[k]
            if a.get("ve_table") is not None:
                a["ve_table"] = a["ve_table"] + b["ve_table"]
    return tot


def test_tiny_fp32_model_gradient_accumulation():
    """Two micro-batches (different tokens and targets) into the same gradients, the second with
    accumulate: every gradient equals the oracle's sum (fp32, 1e-5)."""
    need_gpu()
    s = replace(synth.TINY_FP32, value_embed=False)
    mi, batches = _model_inputs(s, 2, 90, 2)
    M = Model(config_of(s), 2, s.vocab, 0)
    params = _device_params(mi)
    g = M.new_grads(params)
    print("tiny fp32 model: two accumulated micro-batches", flush=True)
    for i, (ids, tg) in enumerate(batches):
        M(params, dev(ids), dev(tg), g, grad_scale=0.5, accumulate=i > 0)
    torch.cuda.synchronize()
    ref = _oracle_sum(mi, batches, 0.5)
    assert_close(host(g["embed"]), ref["embed"], 1e-5, "d_embed", elem_rtol=1e-3)
    assert_close(host(g["head"]), ref["head"], 1e-5, "d_head", elem_rtol=1e-3)
    assert_close(host(g["final_norm_w"]), ref["g_final"], 1e-5, "d_final_norm_w", elem_rtol=1e-3)
    for i, (gl, rl) in enumerate(zip(g["layers"], ref["layers"])):
        for k in ("w_qkv", "w_o", "w_fc", "w_proj", "g_attn", "g_mlp", "ve_table"):
            if rl.get(k) is None:
                continue
            assert_close(host(gl[GPU_NAME.get(k, k)]), rl[k], 1e-5, f"layer{i}.{k}", elem_rtol=1e-3)


def test_train_step_bf16_small_model():
    """TrainStep on a bf16 model with the real head width (d 256, 2 q / 1 kv heads of 128, F 1024,
    vocab 512, 2 layers, value embeddings on layer 0, bf16 MLPs) over 2 micro-batches of 2 x 256
    tokens: accumulated gradients against the oracle at 2e-2, then Muon and AdamW on them."""
    need_gpu()
    # 2 x 256 tokens per micro-batch: every weight gradient has full rank (a gradient of rank below
    # its smaller dimension leaves singular directions at rounding-noise level, which the
    # Newton-Schulz polynomial grows ~3.4x per step, so two correct implementations would differ
    # there by far more than their rounding)
    s = synth.LayerShape(batch=2, seq=256, d_model=256, n_q_heads=2, n_kv_heads=1, head_dim=128, d_ff=1024,
                         vocab=512, real_vocab=512, dtype="bf16", fp8_mlp=False)
    mi, batches = _model_inputs(s, 2, 91, 2)
    M = Model(config_of(replace(s, value_embed=False)), 2, s.vocab, 0)
    params = _device_params(mi)
    before = {"embed": host(params["embed"]), "head": host(params["head"]), "final": host(params["final_norm_w"]),
              "layers": [{k: host(v) for k, v in lp.items()} for lp in params["layers"]]}
    ts = TrainStep(M, params, accum=2)
    before_by_ptr = {t.data_ptr(): host(t) for _, t, _, _, _ in ts.adamw}
    print("bf16 small model: TrainStep over 2 micro-batches", flush=True)
    dbatches = [(dev(a), dev(b)) for a, b in batches]
    ts.backward_all(dbatches)
    torch.cuda.synchronize()
    g = ts.g
    grads = {"embed": host(g["embed"]), "head": host(g["head"]), "final": host(g["final_norm_w"]),
             "layers": [{k: host(v) for k, v in gl.items()} for gl in g["layers"]]}
    ts.optimizer_step()
    torch.cuda.synchronize()
    # (a) accumulated gradients against the oracle's sum of the mean-loss gradients
    ref = _oracle_sum(mi, batches, 0.5)
    assert_close(grads["head"], ref["head"], 2e-2, "d_head", elem_rtol=0.25, row_rtol=0.1)
    touched = np.unique(np.concatenate([b[0] for b in batches]))
    assert_close(grads["embed"][touched], ref["embed"][touched], 2e-2, "d_embed", elem_rtol=0.25)
    for i, (gl, rl) in enumerate(zip(grads["layers"], ref["layers"])):
        for k in MATRICES + ("attn_norm_w", "mlp_norm_w"):
            rk = {"attn_norm_w": "g_attn", "mlp_norm_w": "g_mlp"}.get(k, k)
            assert_close(gl[k], rl[rk], 2e-2, f"layer{i}.{k}", elem_rtol=0.25)
    # (b) the optimizer on the GPU's gradients: Muon on every matrix, AdamW on the rest (step 1)
    for i, lp in enumerate(params["layers"]):
        for k in MATRICES:
            w_ref, _ = oo.muon_update(before["layers"][i][k], grads["layers"][i][k], np.zeros_like(grads["layers"][i][k]),
                                      lr=f32(MUON["lr"]), momentum=f32(MUON["momentum"]), nesterov=True,
                                      weight_decay=f32(MUON["weight_decay"]), mode="bf16")
            upd, upd_ref = host(lp[k]) - before["layers"][i][k], w_ref - before["layers"][i][k]
            print(f"layer{i}.{k} Muon update", error_stats(upd, upd_ref), flush=True)
            check_muon_w(host(lp[k]), w_ref, before["layers"][i][k], f"layer{i}.{k} after Muon", elem=TRAIN_MUON_ELEM)
            e = rel_err(upd, upd_ref)        # elementwise: check_muon_w, in ulps of w
            assert e <= TRAIN_MUON_RTOL, f"layer{i}.{k} Muon update: norm-wise {e:.3e} > {TRAIN_MUON_RTOL}"
    # AdamW on every other parameter: the moments from the GPU's gradient, the parameter from the
    # GPU's new moments (each stored value on its own inputs)
    for grp, prm, grd, ea, eas in ts.adamw:
        lr, b1, b2, eps, wd = (f32(x) for x in ADAMW[grp])
        mode = "bf16" if prm.dtype == torch.bfloat16 else "fp32"
        p0, g0 = before_by_ptr[prm.data_ptr()], host(grd)
        _, m_ref, v_ref = oo.adamw_update(p0, g0, 0, 0, 1, lr, b1, b2, eps, wd, mode=mode)
        gm, gv = host(ea), host(eas)
        p_ref = oo.adamw_param_update(p0, gm, gv, 1, lr, b1, b2, eps, wd, mode=mode)
        sc = np.abs(p0) + np.abs(p_ref - p0)
        if mode == "bf16":
            _ulp_close(gm, m_ref, f"{grp} m", frac=FLIP_FRAC, scale=np.abs((1 - b1) * g0))
            _ulp_close(gv, v_ref, f"{grp} v", frac=FLIP_FRAC)
            _ulp_close(host(prm), p_ref, f"{grp} p", frac=FLIP_FRAC, scale=sc)
        else:
            assert np.all(np.abs(host(prm) - p_ref) <= 2.0 ** -20 * sc + 1e-30), grp
