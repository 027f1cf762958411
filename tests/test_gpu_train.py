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
from tests.gpu_util import assert_close, dev, error_stats, host, need_gpu
from tests.layer_cases import GPU_NAME, config_of, device_params
from tests.test_gpu_optim import MUON_ELEM, MUON_ROW, MUON_RTOL, _ulp_close, f32
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
    vocab 512, 2 layers, value embeddings on layer 0, bf16 MLPs) over 2 micro-batches of 2 x 64
    tokens: accumulated gradients against the oracle at 2e-2, then Muon and AdamW on them."""
    need_gpu()
    s = synth.LayerShape(batch=2, seq=64, d_model=256, n_q_heads=2, n_kv_heads=1, head_dim=128, d_ff=1024,
                         vocab=512, real_vocab=512, dtype="bf16", fp8_mlp=False)
    mi, batches = _model_inputs(s, 2, 91, 2)
    M = Model(config_of(replace(s, value_embed=False)), 2, s.vocab, 0)
    params = _device_params(mi)
    before = {"embed": host(params["embed"]), "head": host(params["head"]), "final": host(params["final_norm_w"]),
              "layers": [{k: host(v) for k, v in lp.items()} for lp in params["layers"]]}
    ts = TrainStep(M, params, accum=2)
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
            assert_close(upd, upd_ref, MUON_RTOL, f"layer{i}.{k} Muon update", elem_rtol=MUON_ELEM, row_rtol=MUON_ROW)
        groups = [("scalars", k) for k in ("attn_norm_w", "mlp_norm_w", "resid_attn", "resid_mlp")]
        if "ve_table" in lp:
            groups.append(("value_embeds", "ve_table"))
        for grp, k in groups:
            lr, b1, b2, eps, wd = (f32(x) for x in ADAMW[grp])
            mode = "bf16" if lp[k].dtype == torch.bfloat16 else "fp32"
            p_ref, _, _ = oo.adamw_update(before["layers"][i][k], grads["layers"][i][k], 0, 0, 1, lr, b1, b2, eps, wd,
                                          mode=mode)
            sc = np.abs(before["layers"][i][k]) + np.abs(p_ref - before["layers"][i][k])
            if mode == "bf16":
                _ulp_close(host(lp[k]), p_ref, f"layer{i}.{k}", scale=sc)
            else:
                assert np.all(np.abs(host(lp[k]) - p_ref) <= 2.0 ** -20 * sc + 1e-30), (i, k)
    for name, grp, key in (("embed", "embeddings", "embed"), ("head", "lm_head", "head"),
                           ("final", "scalars", "final_norm_w")):
        lr, b1, b2, eps, wd = (f32(x) for x in ADAMW[grp])
        mode = "bf16" if params[key].dtype == torch.bfloat16 else "fp32"
        p_ref, _, _ = oo.adamw_update(before[name], grads[name], 0, 0, 1, lr, b1, b2, eps, wd, mode=mode)
        sc = np.abs(before[name]) + np.abs(p_ref - before[name])
        if mode == "bf16":
            _ulp_close(host(params[key]), p_ref, name, scale=sc)
        else:
            assert np.all(np.abs(host(params[key]) - p_ref) <= 2.0 ** -20 * sc + 1e-30), name
