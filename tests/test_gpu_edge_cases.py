"""Edge cases of the library's contracts on the GPU: a NaN in a quantised tensor reaches the FP8
GEMMs as the NaN code, and token ids outside a value-embedding table add nothing and receive no
gradient (the oracle reads them the same way, oracle.model.gather_rows / scatter_rows)."""
import numpy as np
import pytest
import torch

import synth
import transformer_train_step_amd as ll
from oracle import numerics as nu
from tests.gpu_util import dev, need_gpu
from tests.layer_cases import run_gpu, run_oracle
from tests.test_gpu_layer import _compare

pytestmark = pytest.mark.gpu


def test_quant_nan_gives_nan_code():
    need_gpu()
    rows, cols = 64, 256
    x = synth.normal((rows, cols), 1.0, 51, 1, "bf16")
    nan_at = [(3, 17), (40, 255), (63, 0)]
    xn = x.copy()
    for r, c in nan_at:
        xn[r, c] = np.nan
    print("quant with NaN elements", flush=True)
    t = torch.from_numpy(xn).to(torch.bfloat16).cuda()
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    qt = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    inv = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    ll.ll_fp8_quant_tensorwise(ll.LL_BF16, t, rows, cols, cols, q, qt, sc, inv, ws, 64)
    torch.cuda.synchronize()
    got = q.cpu().numpy()
    for r, c in nan_at:
        assert got[r, c] == 0x7F and np.isnan(nu.e4m3_decode(np.array([got[r, c]]))[0])
    # the finite elements: the oracle's codes of the tensor without the NaN elements (the amax
    # skips NaN, so the scale is that of the finite elements)
    xz = x.astype(np.float64).copy()
    for r, c in nan_at:
        xz[r, c] = 0.0
    codes, _, scale, _ = nu.quantize_tensorwise(xz)
    mask = np.ones_like(got, bool)
    for r, c in nan_at:
        mask[r, c] = False
    assert np.float32(sc.item()) == np.float32(scale)
    assert np.array_equal(got[mask], codes[mask])
    assert np.array_equal(qt.cpu().numpy(), got.T)


def test_value_embedding_ids_outside_the_table():
    need_gpu()
    s = synth.LayerShape(batch=2, seq=40, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, d_ff=1024,
                         vocab=512, real_vocab=512, dtype="fp32", fp8_mlp=False, value_embed=True)
    inp = synth.layer_inputs(s, seed=52, perturb=True)
    inp.ids[[0, 7, 41, 79]] = np.array([-1, 512, 10**6, -(2**31)], np.int32)
    print("value-embedding layer with out-of-range ids", flush=True)
    gpu = run_gpu(inp)
    ref = run_oracle(inp)
    ok = (inp.ids >= 0) & (inp.ids < s.vocab)
    # rows of ids that are in range get gradient; the rest of the table stays exactly 0
    inp_ids_ok = inp.ids[ok]
    gpu["ids"] = inp_ids_ok
    _compare(gpu, ref, 1e-5, 1e-3)
