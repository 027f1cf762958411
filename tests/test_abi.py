"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function that
include/*.h declares, and rejects invalid arguments with the documented status codes before any
launch (so these calls are safe without a device)."""
import ctypes
import os
import re

import pytest

import transformer_train_step_amd as ll
from transformer_train_step_amd import _lib as L
from transformer_train_step_amd.ops import LayerConfig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b((?:ll|llt)_[a-z0-9_]+)\s*\(", src))
    return names


def test_library_exports_every_declared_function():
    lib = L.lib()
    declared = _declared()
    assert {"ll_layer_fwd", "ll_layer_bwd", "ll_fused_lce_fwd_bwd", "ll_fp8_quant_tensorwise"} <= declared
    missing = [n for n in sorted(declared) if not hasattr(lib, n)]
    assert not missing, missing
    assert set(L.ENTRY_POINTS) <= declared


def test_status_strings_and_version():
    assert ll.ll_status_string(0) == "LL_OK"
    assert ll.ll_status_string(3) == "LL_ERR_WORKSPACE"
    assert ll.ll_version() >= 100


def _fake(n=1 << 20):
    # a 16-byte aligned host buffer; only its address is used (validation fails before any launch)
    buf = ctypes.create_string_buffer(n + 16)
    a = ctypes.addressof(buf)
    return buf, a + (-a % 16)


def test_quant_validation():
    keep, p = _fake()
    st = ll.ll_fp8_quant_tensorwise(7, p, 4, 16, 16, p, None, p, p, p, 64, stream=0, raise_on_error=False)
    assert st == L.LL_ERR_INVALID_ARG
    st = ll.ll_fp8_quant_tensorwise(1, p, 4, 15, 16, p, None, p, p, p, 64, stream=0, raise_on_error=False)
    assert st == L.LL_ERR_UNSUPPORTED
    st = ll.ll_fp8_quant_tensorwise(1, p, 4, 16, 8, p, None, p, p, p, 64, stream=0, raise_on_error=False)
    assert st == L.LL_ERR_INVALID_ARG and "ld" in ll.ll_last_error()
    st = ll.ll_fp8_quant_tensorwise(1, p, 4, 16, 16, p, None, p, p, p, 4, stream=0, raise_on_error=False)
    assert st == L.LL_ERR_WORKSPACE
    st = ll.ll_fp8_quant_tensorwise(1, p + 2, 4, 16, 16, p, None, p, p, p, 64, stream=0, raise_on_error=False)
    assert st == L.LL_ERR_INVALID_ARG
    st = ll.ll_fp8_quant_tensorwise(1, p, 4, 16, 16, p, None, None, p, p, 64, stream=0, raise_on_error=False)
    assert st == L.LL_ERR_INVALID_ARG


def test_layer_size_queries_and_validation():
    c = LayerConfig(batch=40, seq=1024).c_struct()
    saved, ws = ll.ll_layer_saved_bytes(c), ll.ll_layer_workspace_bytes(c)
    assert saved > 40 * 1024 * 3072 * 2 * 8 and ws > 0
    assert saved + ws < 200 * 2 ** 30                  # fits one MI355X (288 GB) with room to spare
    sw8 = LayerConfig(batch=2, seq=8, mlp="swiglu").c_struct()        # SwiGLU with FP8 GEMMs
    assert ll.ll_layer_saved_bytes(sw8) == 0 and ll.ll_layer_workspace_bytes(sw8) == 0
    sw = LayerConfig(batch=2, seq=8, mlp="swiglu", fp8_mlp=False, d_ff=8448).c_struct()
    assert ll.ll_layer_saved_bytes(sw) > ll.ll_layer_saved_bytes(
        LayerConfig(batch=2, seq=8, fp8_mlp=False, d_ff=8448).c_struct())
    odd = LayerConfig(batch=2, seq=8).c_struct()
    odd.mlp_kind = 7
    assert ll.ll_layer_saved_bytes(odd) == 0
    bad = LayerConfig(batch=2, seq=8, dtype="fp32", fp8_mlp=True, head_dim=64).c_struct()
    assert ll.ll_layer_saved_bytes(bad) == 0
    keep, p = _fake()
    params = L.LayerParams(*([p] * 9))
    st = ll.ll_layer_fwd(bad, params, p, None, p, p, 1 << 20, p, 1 << 20, stream=0, raise_on_error=False)
    assert st == L.LL_ERR_UNSUPPORTED
    c = LayerConfig(batch=2, seq=8).c_struct()
    st = ll.ll_layer_fwd(c, params, p, None, p + 16, p, 16, p, 1 << 20, stream=0, raise_on_error=False)
    assert st == L.LL_ERR_WORKSPACE and "saved" in ll.ll_last_error()
    c = LayerConfig(batch=2, seq=8, head_dim=64).c_struct()
    assert ll.ll_layer_workspace_bytes(c) == 0
    c = LayerConfig(batch=2, seq=8, value_embed=True).c_struct()
    params = L.LayerParams(p, p, p, p, p, p, None, p, p)
    st = ll.ll_layer_fwd(c, params, p, p, p + 16, p, 1 << 40, p, 1 << 40, stream=0, raise_on_error=False)
    assert st == L.LL_ERR_INVALID_ARG and "ve_table" in ll.ll_last_error()
    st = ll.ll_layer_fwd(c, L.LayerParams(*([p] * 9)), p, None, p + 16, p, 1 << 40, p, 1 << 40, stream=0,
                         raise_on_error=False)
    assert st == L.LL_ERR_INVALID_ARG and "token_ids" in ll.ll_last_error()
    st = ll.ll_layer_fwd(c, L.LayerParams(*([p] * 9)), p, p, p, p, 1 << 40, p, 1 << 40, stream=0,
                         raise_on_error=False)
    assert st == L.LL_ERR_INVALID_ARG and "alias" in ll.ll_last_error()


def test_lce_validation():
    keep, p = _fake()
    f = lambda **kw: ll.ll_fused_lce_fwd_bwd(**{**dict(dtype=1, hidden=p, weight=p, targets=p, n=16, d=3072,
                                                         v=50304, softcap=15.0, ignore_index=-100, grad_scale=1.0,
                                                         token_chunk=0, vocab_tile=0, accumulate_dw=0, loss=p,
                                                         lse=None, d_hidden=p, d_weight=p,
                                                         ws=p, ws_bytes=1 << 20, stream=0,
                                                         raise_on_error=False), **kw})
    assert f(d=100) == L.LL_ERR_UNSUPPORTED
    assert f(v=50301) == L.LL_ERR_UNSUPPORTED
    assert f(softcap=0.0) == L.LL_ERR_INVALID_ARG
    assert f(softcap=61.0) == L.LL_ERR_INVALID_ARG and "softcap" in ll.ll_last_error()
    assert f(vocab_tile=64) == L.LL_ERR_UNSUPPORTED
    assert f(accumulate_dw=2) == L.LL_ERR_INVALID_ARG
    assert f(d_weight=None) == L.LL_ERR_INVALID_ARG
    assert f(loss=None) == L.LL_ERR_INVALID_ARG
    assert f() == L.LL_ERR_WORKSPACE
    need = ll.ll_fused_lce_workspace_bytes(1, 40960, 3072, 50304, 8192)
    assert 1e9 < need < 5e9
    # 128-wide vocabulary tiles: twice the partial row sums
    n128 = ll.ll_fused_lce_workspace_bytes(1, 40960, 3072, 50304, 8192, 128)
    assert n128 - need == (8192 * 393 - 8192 * 197) * 4
    assert ll.ll_fused_lce_workspace_bytes(9, 1, 64, 8, 0) == 0
    assert ll.ll_fused_lce_workspace_bytes(1, 1, 64, 8, 0, 192) == 0


def test_flop_accounting_reproduces_pages_b200_rate():
    """bench.py's per-token layer FLOP count reproduces the pages' ~1,047 TFLOP/s per B200 from
    their ~480,000 tokens/s on 8 GPUs at 1024 context over 28 layers (tests/golden)."""
    import bench
    gold = {}
    with open(os.path.join(ROOT, "tests", "golden", "b200_throughput.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, v = line.split()
                gold[k] = float(v)
    per_gpu = gold["tokens_per_s_node"] / gold["gpus"]
    tf = per_gpu * gold["n_layers"] * bench.layer_flops_per_token(int(gold["seq"])) / 1e12
    assert abs(tf - gold["tflops_per_gpu"]) / gold["tflops_per_gpu"] < 0.005, tf
    assert bench.P_MM == 100_663_296
    assert bench.layer_flops_per_token(1024) == 622_872_576
