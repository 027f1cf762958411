"""Parity at the full workload sizes, in the launch configuration bench.py times, on outputs the
oracle can compute piece by piece:

* the e4m3 quantiser on the layer's [40960, 3072] activation (every code) and on [40960, 12288]
  (sampled rows, with the row holding the global amax so that the oracle's scale is the whole
  tensor's);
* one decoder layer at 40 x 1024 tokens: attention is causal within each sequence, so the oracle
  runs whole sampled sequences and y and dx of those sequences are compared (bf16 MLP: the
  tensorwise FP8 scales depend on every token). The FP8 layer at the same size is compared with
  the bf16 layer (property: FP8 noise only);
* the value-embedding layer at 20 x 2048 tokens on a sampled sequence;
* the fused linear cross-entropy at 40960 x 3072 @ 50304 x 3072, chunk 10240: lse of every row and
  the loss from the oracle run over all rows in chunks, dH of sampled rows, sampled rows of dW
  from the oracle's dz of every token on those vocabulary columns.
Weight gradients of the layer sum over all 40 sequences; the FP8 layer, with every weight gradient,
is compared with the oracle at 4 x 1024 and 2 x 2048 tokens (tests/test_gpu_fp8_layer.py), sizes
that run the same launch configurations as this one."""
import numpy as np
import pytest
import torch

import synth
import transformer_train_step_amd as ll
from oracle import lce as olce
from oracle import model as om
from oracle import numerics as nu
from tests.gpu_util import assert_close, dev, host, need_gpu
from tests.layer_cases import config_of, device_params
from transformer_train_step_amd.ops import FusedLCE, Layer

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def _quant(x_dev, rows, cols):
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    qt = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    inv = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    ll.ll_fp8_quant_tensorwise(ll.LL_BF16, x_dev, rows, cols, cols, q, qt, sc, inv, ws, 64)
    torch.cuda.synchronize()
    return q, qt, sc, inv


def test_quant_full_hidden_bitexact():
    need_gpu()
    print("quant 40960x3072 full", flush=True)
    x = synth.normal((40960, 3072), 1.0, 31, 1, "bf16")
    q, qt, sc, inv = _quant(dev(x, "bf16"), *x.shape)
    codes, _, scale, inv_scale = nu.quantize_tensorwise(x.astype(np.float64))
    assert np.float32(sc.item()) == np.float32(scale) and np.float32(inv.item()) == np.float32(inv_scale)
    got = q.cpu().numpy()
    assert np.array_equal(got, codes), f"{int((got != codes).sum())} codes differ"
    assert np.array_equal(qt.cpu().numpy(), codes.T)


def test_quant_full_mlp_sampled_rows():
    need_gpu()
    print("quant 40960x12288 sampled", flush=True)
    rows, cols = 40960, 12288
    x = synth.normal((rows, cols), 1.0, 32, 1, "bf16")
    q, qt, sc, inv = _quant(dev(x, "bf16"), rows, cols)
    amax_row = int(np.argmax(np.max(np.abs(x), axis=1)))
    pick = np.unique(np.concatenate([synth.rng(32, 2).choice(rows, 63, replace=False), [amax_row]]))
    codes, _, scale, _ = nu.quantize_tensorwise(x[pick].astype(np.float64))
    assert np.float32(sc.item()) == np.float32(scale)
    assert np.array_equal(q.cpu().numpy()[pick], codes)
    assert np.array_equal(qt.cpu().numpy()[:, pick], codes.T)


def _layer_gpu(s, inp):
    layer = Layer(config_of(s))
    p = device_params(inp)
    x, ids = dev(inp.x, "bf16"), dev(inp.ids)
    y = layer.forward(p, x, ids)
    dx, _ = layer.backward(p, x, ids, dev(inp.dy, "bf16"))
    torch.cuda.synchronize()
    return y, dx


def _oracle_sequences(s, inp, seqs):
    """y and dx of whole sequences from the oracle (same weights; attention never crosses
    sequences; no FP8, so nothing depends on other sequences)."""
    T = s.seq
    sub = synth.LayerShape(**{**s.__dict__, "batch": 1})
    out = {}
    for b in seqs:
        r = slice(b * T, (b + 1) * T)
        pi = synth.LayerInputs(sub, inp.x[r], inp.dy[r], inp.w_qkv, inp.w_o, inp.w_fc, inp.w_proj, inp.g_attn,
                               inp.g_mlp, inp.a_attn, inp.a_mlp, inp.ids[r], inp.ve_table)
        p, d = om.params_from_inputs(pi), om.dims_from_shape(sub)
        y, cache = om.layer_fwd(p, pi.x, pi.ids, d)
        g = om.layer_bwd(p, cache, pi.dy, d)
        out[b] = (y, g["dx"])
    return out


@pytest.mark.parametrize("shape,seqs", [(synth.LayerShape(batch=40, seq=1024, fp8_mlp=False), (0, 39)),
                                        (synth.LayerShape(batch=20, seq=2048, fp8_mlp=False, value_embed=True), (7,))])
def test_layer_full_size_sampled_sequences(shape, seqs):
    need_gpu()
    print(f"layer full size {shape.batch}x{shape.seq} ve={shape.value_embed} sequences {seqs}", flush=True)
    inp = synth.layer_inputs(shape, seed=33, perturb=True)
    y, dx = _layer_gpu(shape, inp)
    ref = _oracle_sequences(shape, inp, seqs)
    T = shape.seq
    for b, (yr, dxr) in ref.items():
        r = slice(b * T, (b + 1) * T)
        # bf16 MLP: measured elementwise <= 0.027 of (|ref| + rms), rows <= 0.006, norm-wise 3.4e-3
        assert_close(host(y[r]), yr, 2e-2, f"y[seq {b}]", elem_rtol=0.06, row_rtol=0.015)
        assert_close(host(dx[r]), dxr, 2e-2, f"dx[seq {b}]", elem_rtol=0.06, row_rtol=0.015)


def test_layer_full_size_fp8_vs_bf16():
    """Property at 40 x 1024: the FP8 layer differs from the bf16 layer (same inputs) only by the
    e4m3 quantisation of the MLP GEMM operands (a few percent norm-wise), and is finite."""
    need_gpu()
    print("layer full size fp8 vs bf16", flush=True)
    s8 = synth.LayerShape(batch=40, seq=1024)
    inp = synth.layer_inputs(s8, seed=34, perturb=True)
    y8, dx8 = _layer_gpu(s8, inp)
    y16, dx16 = _layer_gpu(synth.LayerShape(batch=40, seq=1024, fp8_mlp=False), inp)
    for name, a, b in (("y", y8, y16), ("dx", dx8, dx16)):
        a, b = a.float(), b.float()
        assert torch.isfinite(a).all(), name
        rel = (torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b)).item()
        print(f"  {name}: fp8 vs bf16 rel {rel:.3e}", flush=True)
        assert rel < 0.08, (name, rel)


def test_lce_full_size_sampled():
    """The loss at its full size: lse of every row, the loss and sampled rows of dW from the oracle
    run chunk by chunk over all 40960 rows (float64), dH on sampled rows."""
    need_gpu()
    print("lce full size 40960x3072 @ 50304x3072 chunk 10240", flush=True)
    n, d, v = synth.LCE_TOKENS, synth.LCE_DIM, synth.LCE_VOCAB
    li = synth.lce_inputs(n, d, v, synth.LCE_REAL_VOCAB, "bf16", seed=35)
    H, W, y = dev(li.hidden, "bf16"), dev(li.weight, "bf16"), dev(li.targets)
    lse = torch.empty(n, dtype=torch.float32, device="cuda")
    loss, dh, dw = FusedLCE("bf16", n, d, v, token_chunk=10240)(H, W, y, lse=lse)
    torch.cuda.synchronize()
    lse_g, dh_g, dw_g = host(lse), host(dh), host(dw)
    del dh, dw, H, W
    torch.cuda.empty_cache()
    h64, w64 = li.hidden.astype(np.float64), li.weight.astype(np.float64)
    vs = np.sort(synth.rng(35, 10).choice(v, 6, replace=False))
    # the oracle over every row, 2048 rows at a time: lse, the loss terms, and dz on the sampled
    # vocabulary columns (for dW = dz^T H on those rows)
    lse_o = np.empty(n)
    loss_terms = 0.0
    dz_vs = np.empty((n, len(vs)))
    for r0 in range(0, n, 2048):
        r = slice(r0, min(n, r0 + 2048))
        o = olce.lce_fwd_bwd(h64[r], w64, li.targets[r], softcap=15.0, mode="bf16", need_grads=False)
        lse_o[r] = o["lse"]
        loss_terms += o["loss"] * o["n_valid"]
        z = nu.bf16_round(h64[r] @ w64[vs].T)
        c = 15.0 * np.tanh(z / 15.0)
        p = np.exp(c - o["lse"][:, None])
        p[li.targets[r][:, None] == vs[None, :]] -= 1.0
        dz_vs[r] = nu.bf16_round(p * (1.0 - (c / 15.0) ** 2) / n)
        print(f"  oracle rows {r0}..{r.stop}", flush=True)
    assert_close(lse_g, lse_o, 1e-6, "lse (every row)", elem_rtol=1e-5)
    ref_loss = loss_terms / n
    assert abs(loss.item() - ref_loss) <= 1e-5 * abs(ref_loss), (loss.item(), ref_loss)
    dw_ref = nu.bf16_round(dz_vs.T @ h64)
    # measured at 300 rows: elementwise <= 0.007 of (|ref| + rms), rows <= 0.007
    assert_close(dw_g[vs], dw_ref, 2e-2, "dW rows", elem_rtol=0.03, row_rtol=0.02)
    rows = np.sort(synth.rng(35, 9).choice(n, 48, replace=False))
    o = olce.lce_fwd_bwd(h64[rows], w64, li.targets[rows], softcap=15.0, mode="bf16", grad_scale=len(rows) / n)
    assert_close(dh_g[rows], o["dh"], 2e-2, "dH rows", elem_rtol=0.03, row_rtol=0.02)
