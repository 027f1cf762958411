"""The allocation-free quantiser entry point (static device scratch) against the workspace one,
through the C ABI: two calls in a row, the second on a smaller tensor, each compared bit for bit
(codes, transposed codes, scale, inverse scale) with ll_fp8_quant_tensorwise on the same input."""
import numpy as np
import pytest
import torch

import synth
import transformer_train_step_amd as ll
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu


def _buffers(rows, cols):
    return (torch.empty((rows, cols), dtype=torch.uint8, device="cuda"),
            torch.empty((cols, rows), dtype=torch.uint8, device="cuda"),
            torch.empty(1, dtype=torch.float32, device="cuda"), torch.empty(1, dtype=torch.float32, device="cuda"))


def test_noalloc_quant_matches_workspace_quant():
    need_gpu()
    ws = torch.empty(ll.ll_fp8_quant_workspace_bytes(), dtype=torch.uint8, device="cuda")
    # the second tensor is smaller and its amax lower: a scratch left over from the first call
    # (amax not cleared) would give it the first tensor's scale
    for rows, cols, std, seed in ((1000, 3072, 4.0, 61), (136, 512, 0.05, 62)):
        print(f"noalloc quant {rows}x{cols}", flush=True)
        x = torch.from_numpy(synth.normal((rows, cols), std, seed, 1, "bf16")).to(torch.bfloat16).cuda()
        q0, qt0, s0, i0 = _buffers(rows, cols)
        q1, qt1, s1, i1 = _buffers(rows, cols)
        ll.ll_fp8_quant_tensorwise(ll.LL_BF16, x, rows, cols, cols, q0, qt0, s0, i0, ws, ws.numel())
        ll._lib.ll_fp8_quant_tensorwise_noalloc(ll.LL_BF16, x, rows, cols, cols, q1, qt1, s1, i1)
        torch.cuda.synchronize()
        assert s0.item() == s1.item() and i0.item() == i1.item()
        assert torch.equal(q0, q1) and torch.equal(qt0, qt1)
        assert np.isfinite(s1.item()) and s1.item() > 0


def test_noalloc_quant_validates_before_launching():
    need_gpu()
    x = torch.zeros((4, 16), dtype=torch.bfloat16, device="cuda")
    q, qt, s, i = _buffers(4, 16)
    st = ll._lib.ll_fp8_quant_tensorwise_noalloc(ll.LL_BF16, x, 4, 15, 16, q, qt, s, i, raise_on_error=False)
    assert st == ll._lib.LL_ERR_UNSUPPORTED
    st = ll._lib.ll_fp8_quant_tensorwise_noalloc(ll.LL_BF16, x, 4, 16, 16, q, qt, None, i, raise_on_error=False)
    assert st == ll._lib.LL_ERR_INVALID_ARG
