"""The layer + loss step captured in a HIP graph (as bench.py --graph times it): every replay, with
eager work and synchronisations between the replays, reproduces the eager step. The library clears
its counters and accumulators with fill kernels (no hipMemsetAsync nodes in the graph)."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import need_gpu
from tests.layer_cases import config_of, device_params
from transformer_train_step_amd.ops import FusedLCE, Layer

pytestmark = pytest.mark.gpu


def test_layer_lce_step_graph_replays_match_eager():
    need_gpu()
    s = synth.LayerShape(batch=2, seq=256)
    inp = synth.layer_inputs(s, seed=60, perturb=True)
    N, D, V = s.tokens, s.d_model, 4096
    layer = Layer(config_of(s))
    p = device_params(inp)
    x = torch.from_numpy(inp.x).to(torch.bfloat16).cuda()
    ids = torch.from_numpy(inp.ids).cuda()
    w_head = torch.from_numpy(synth.normal((V, D), 0.02, 60, synth.K_WHEAD, "bf16")).to(torch.bfloat16).cuda()
    targets = torch.from_numpy(synth.uniform_ints((N,), V, 60, synth.K_TARGETS)).cuda()
    lce = FusedLCE("bf16", N, D, V, token_chunk=256)
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    dh = torch.empty_like(x)
    dw = torch.empty_like(w_head)
    grads = layer.new_grads()

    def step():
        layer.forward(p, x, ids, y)
        lce(y, w_head, targets, d_hidden=dh, d_weight=dw)
        layer.backward(p, x, ids, dh, dx=dx, grads=grads)

    def snapshot():
        out = {"y": y.clone(), "dx": dx.clone(), "dw": dw.clone(), "loss": lce.loss.clone()}
        out.update({k: v.clone() for k, v in grads.items()})
        return out

    print("graph: eager step", flush=True)
    step()
    torch.cuda.synchronize()
    ref = snapshot()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        # eager work between replays that overwrites every output
        for t in (y, dx, dh, dw):
            t.normal_()
        for v in grads.values():
            v.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        print(f"graph: replay {r} checked", flush=True)
        for k, want in ref.items():
            a, b = got[k].float(), want.float()
            if k in ("resid_attn", "resid_mlp", "loss"):
                # sums of fp32 atomics: the order differs between runs
                assert torch.allclose(a, b, rtol=1e-5, atol=1e-6), (r, k, a, b)
            else:
                assert torch.equal(a, b), (r, k, (a - b).abs().max().item())
