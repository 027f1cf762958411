"""ctypes binding of libll (include/ll.h, include/ll_testing.h): same names, argument marshalling
only. Tensor arguments may be torch tensors (their data_ptr is passed), plain integer addresses,
or None (NULL). Every computation happens in the HIP library; if libll.so is missing or fails to
load, every call raises — there is no fallback."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libll.so")

LL_OK, LL_ERR_INVALID_ARG, LL_ERR_UNSUPPORTED, LL_ERR_WORKSPACE, LL_ERR_HIP = 0, 1, 2, 3, 4
LL_F32, LL_BF16 = 0, 1
LL_MLP_RELU2, LL_MLP_SWIGLU = 0, 1
LLT_OP_F32, LLT_OP_BF16, LLT_OP_E4M3 = 0, 1, 2

c_void_p, c_int32, c_int64, c_size_t, c_float = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                                  ctypes.c_size_t, ctypes.c_float)


class LLError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


STATUS_NAMES = {0: "LL_OK", 1: "LL_ERR_INVALID_ARG", 2: "LL_ERR_UNSUPPORTED", 3: "LL_ERR_WORKSPACE",
                4: "LL_ERR_HIP"}


class LayerCfg(ctypes.Structure):
    _fields_ = [("dtype", c_int32), ("fp8_mlp", c_int32), ("batch", c_int64), ("seq", c_int64),
                ("d_model", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("d_ff", c_int32), ("rms_eps", c_float),
                ("rope_theta", c_float), ("has_value_embed", c_int32), ("ve_rows", c_int64),
                ("mlp_kind", c_int32)]


class LayerParams(ctypes.Structure):
    _fields_ = [("attn_norm_w", c_void_p), ("w_qkv", c_void_p), ("w_o", c_void_p),
                ("mlp_norm_w", c_void_p), ("w_fc", c_void_p), ("w_proj", c_void_p),
                ("ve_table", c_void_p), ("resid_attn", c_void_p), ("resid_mlp", c_void_p)]


class LayerGrads(ctypes.Structure):
    _fields_ = [("attn_norm_w", c_void_p), ("w_qkv", c_void_p), ("w_o", c_void_p),
                ("mlp_norm_w", c_void_p), ("w_fc", c_void_p), ("w_proj", c_void_p),
                ("ve_table", c_void_p), ("resid_attn", c_void_p), ("resid_mlp", c_void_p),
                ("accumulate", c_int32)]


class ModelParams(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("layers", ctypes.POINTER(LayerParams)), ("final_norm_w", c_void_p),
                ("head", c_void_p)]


class ModelGrads(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("layers", ctypes.POINTER(LayerGrads)), ("final_norm_w", c_void_p),
                ("head", c_void_p), ("accumulate", c_int32)]


_lib = None
_load_error = None

# name -> (restype, argtypes)
_SIGS = {
    "ll_status_string": (ctypes.c_char_p, [c_int32]),
    "ll_last_error": (ctypes.c_char_p, []),
    "ll_version": (c_int32, []),
    "ll_fp8_quant_workspace_bytes": (c_size_t, []),
    "ll_fp8_quant_tensorwise": (c_int32, [c_int32, c_void_p, c_int64, c_int64, c_int64, c_void_p,
                                          c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "ll_layer_saved_bytes": (c_size_t, [ctypes.POINTER(LayerCfg)]),
    "ll_layer_workspace_bytes": (c_size_t, [ctypes.POINTER(LayerCfg)]),
    "ll_layer_fwd": (c_int32, [ctypes.POINTER(LayerCfg), ctypes.POINTER(LayerParams), c_void_p,
                               c_void_p, c_void_p, c_void_p, c_size_t, c_void_p, c_size_t, c_void_p]),
    "ll_layer_bwd": (c_int32, [ctypes.POINTER(LayerCfg), ctypes.POINTER(LayerParams), c_void_p,
                               c_void_p, c_void_p, c_size_t, c_void_p, c_void_p,
                               ctypes.POINTER(LayerGrads), c_void_p, c_size_t, c_void_p]),
    "ll_fused_lce_workspace_bytes": (c_size_t, [c_int32, c_int64, c_int32, c_int64, c_int64, c_int32]),
    "ll_fused_lce_fwd_bwd": (c_int32, [c_int32, c_void_p, c_void_p, c_void_p, c_int64, c_int32,
                                       c_int64, c_float, c_int32, c_float, c_int64, c_int32, c_int32,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "ll_model_saved_bytes": (c_size_t, [ctypes.POINTER(LayerCfg), c_int32, c_int64]),
    "ll_model_workspace_bytes": (c_size_t, [ctypes.POINTER(LayerCfg), c_int32, c_int64, c_int64]),
    "ll_model_fwd_bwd": (c_int32, [ctypes.POINTER(LayerCfg), c_int32, c_int64, ctypes.POINTER(ModelParams),
                                   c_void_p, c_void_p, c_float, c_int32, c_float, c_int64, c_void_p,
                                   ctypes.POINTER(ModelGrads), c_void_p, c_size_t, c_void_p, c_size_t,
                                   c_void_p]),
    "llt_embedding_gather": (c_int32, [c_int32, c_void_p, c_int64, c_int32, c_void_p, c_int64, c_void_p,
                                       c_void_p]),
    "llt_embedding_scatter_add": (c_int32, [c_int32, c_void_p, c_void_p, c_int64, c_int32, c_void_p, c_int64,
                                            c_void_p]),
    "llt_rmsnorm_fwd": (c_int32, [c_int32, c_void_p, c_void_p, c_int64, c_int32, c_float, c_void_p, c_void_p,
                                  c_void_p]),
    "llt_rmsnorm_bwd_workspace_bytes": (c_size_t, [c_int64, c_int32]),
    "llt_rmsnorm_bwd": (c_int32, [c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_void_p,
                                  c_void_p, c_void_p, c_size_t, c_void_p]),
    "llt_gemm": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_int64, c_void_p, c_int64, c_int32,
                           c_int32, c_int32, c_int32, c_void_p, c_int64, c_void_p, c_void_p, c_void_p,
                           c_size_t, c_void_p]),
    "llt_gemm_splitk_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "llt_gemm_splitk": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_int64, c_void_p, c_int64, c_int32,
                                  c_int32, c_int32, c_int32, c_int32, c_void_p, c_int64, c_void_p, c_void_p,
                                  c_void_p, c_size_t, c_void_p]),
    "llt_set_gemm_config": (c_int32, [c_int32]),
    "llt_trace_begin": (c_int32, [c_int32]),
    "llt_trace_end": (c_int32, []),
    "llt_trace_count": (c_int32, []),
    "llt_trace_get": (c_int32, [c_int32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(c_float),
                                ctypes.POINTER(c_int64)]),
    "llt_trace_get_gemm": (c_int32, [c_int32, ctypes.POINTER(c_int32), ctypes.POINTER(c_int32)]),
    "ll_muon_workspace_bytes": (c_size_t, [c_int64, c_int64]),
    "ll_muon_step": (c_int32, [c_int32, c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_float, c_float, c_int32,
                               c_float, c_int32, c_void_p, c_size_t, c_void_p]),
    "ll_adamw_step": (c_int32, [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_float, c_float,
                                c_float, c_float, c_float, c_int64, c_void_p]),
    "llt_layer_buffer": (c_int32, [ctypes.POINTER(LayerCfg), c_int32, ctypes.c_char_p, ctypes.POINTER(c_size_t),
                                   ctypes.POINTER(c_size_t)]),
    "llt_e4m3_cast": (c_int32, [c_void_p, c_int64, c_float, c_void_p, c_void_p]),
}
_SIGS["ll_fp8_quant_tensorwise_noalloc"] = (c_int32, [c_int32, c_void_p, c_int64, c_int64, c_int64, c_void_p,
                                                      c_void_p, c_void_p, c_void_p, c_void_p])

ENTRY_POINTS = tuple(_SIGS)


def lib():
    """The loaded libll (raises if it is not built or cannot be loaded)."""
    global _lib, _load_error
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libll.so not built ({LIB_PATH}); run python -m transformer_train_step_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        if not hasattr(L, name):
            continue
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def stream_handle(stream=None) -> int | None:
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def check(status: int, fn: str):
    if status != LL_OK:
        msg = lib().ll_last_error().decode(errors="replace")
        raise LLError(status, fn, msg)


def _call(name, *args, raise_on_error=True):
    st = getattr(lib(), name)(*args)
    if raise_on_error:
        check(st, name)
    return st


# ---------------------------------------------------------------- same-name wrappers
def ll_status_string(status: int) -> str:
    return lib().ll_status_string(status).decode()


def ll_last_error() -> str:
    return lib().ll_last_error().decode(errors="replace")


def ll_version() -> int:
    return lib().ll_version()


def ll_fp8_quant_workspace_bytes() -> int:
    return lib().ll_fp8_quant_workspace_bytes()


def ll_fp8_quant_tensorwise(in_dtype, x, rows, cols, ld, q, q_t, scale, inv_scale, ws, ws_bytes,
                            stream=None, raise_on_error=True):
    return _call("ll_fp8_quant_tensorwise", in_dtype, ptr(x), rows, cols, ld, ptr(q), ptr(q_t),
                 ptr(scale), ptr(inv_scale), ptr(ws), ws_bytes, stream_handle(stream),
                 raise_on_error=raise_on_error)


def ll_layer_saved_bytes(cfg: LayerCfg) -> int:
    return lib().ll_layer_saved_bytes(ctypes.byref(cfg))


def ll_layer_workspace_bytes(cfg: LayerCfg) -> int:
    return lib().ll_layer_workspace_bytes(ctypes.byref(cfg))


def ll_layer_fwd(cfg, params, x, token_ids, y, saved, saved_bytes, ws, ws_bytes, stream=None,
                 raise_on_error=True):
    return _call("ll_layer_fwd", ctypes.byref(cfg), ctypes.byref(params), ptr(x), ptr(token_ids),
                 ptr(y), ptr(saved), saved_bytes, ptr(ws), ws_bytes, stream_handle(stream),
                 raise_on_error=raise_on_error)


def ll_layer_bwd(cfg, params, x, token_ids, saved, saved_bytes, dy, dx, grads, ws, ws_bytes,
                 stream=None, raise_on_error=True):
    return _call("ll_layer_bwd", ctypes.byref(cfg), ctypes.byref(params), ptr(x), ptr(token_ids),
                 ptr(saved), saved_bytes, ptr(dy), ptr(dx), ctypes.byref(grads), ptr(ws), ws_bytes,
                 stream_handle(stream), raise_on_error=raise_on_error)


def ll_fused_lce_workspace_bytes(dtype, n, d, v, token_chunk, vocab_tile=0) -> int:
    return lib().ll_fused_lce_workspace_bytes(dtype, n, d, v, token_chunk, vocab_tile)


def ll_fused_lce_fwd_bwd(dtype, hidden, weight, targets, n, d, v, softcap, ignore_index, grad_scale,
                         token_chunk, vocab_tile, accumulate_dw, loss, lse, d_hidden, d_weight, ws, ws_bytes,
                         stream=None, raise_on_error=True):
    return _call("ll_fused_lce_fwd_bwd", dtype, ptr(hidden), ptr(weight), ptr(targets), n, d, v,
                 softcap, ignore_index, grad_scale, token_chunk, vocab_tile, int(accumulate_dw), ptr(loss),
                 ptr(lse), ptr(d_hidden), ptr(d_weight), ptr(ws), ws_bytes, stream_handle(stream),
                 raise_on_error=raise_on_error)


def ll_model_saved_bytes(cfg: LayerCfg, n_layers: int, vocab: int) -> int:
    return lib().ll_model_saved_bytes(ctypes.byref(cfg), n_layers, vocab)


def ll_model_workspace_bytes(cfg: LayerCfg, n_layers: int, vocab: int, token_chunk: int) -> int:
    return lib().ll_model_workspace_bytes(ctypes.byref(cfg), n_layers, vocab, token_chunk)


def ll_model_fwd_bwd(cfg, n_layers, vocab, params: ModelParams, token_ids, targets, softcap, ignore_index,
                     grad_scale, token_chunk, loss, grads: ModelGrads, saved, saved_bytes, ws, ws_bytes,
                     stream=None, raise_on_error=True):
    return _call("ll_model_fwd_bwd", ctypes.byref(cfg), n_layers, vocab, ctypes.byref(params), ptr(token_ids),
                 ptr(targets), softcap, ignore_index, grad_scale, token_chunk, ptr(loss), ctypes.byref(grads),
                 ptr(saved), saved_bytes, ptr(ws), ws_bytes, stream_handle(stream), raise_on_error=raise_on_error)


def llt_embedding_gather(dtype, table, rows, d, ids, n, out, stream=None, raise_on_error=True):
    return _call("llt_embedding_gather", dtype, ptr(table), rows, d, ptr(ids), n, ptr(out), stream_handle(stream),
                 raise_on_error=raise_on_error)


def llt_embedding_scatter_add(dtype, d_out, ids, n, d, d_table, rows, stream=None, raise_on_error=True):
    return _call("llt_embedding_scatter_add", dtype, ptr(d_out), ptr(ids), n, d, ptr(d_table), rows,
                 stream_handle(stream), raise_on_error=raise_on_error)


def llt_rmsnorm_fwd(dtype, x, g, n, d, eps, y, rstd, stream=None, raise_on_error=True):
    return _call("llt_rmsnorm_fwd", dtype, ptr(x), ptr(g), n, d, eps, ptr(y), ptr(rstd), stream_handle(stream),
                 raise_on_error=raise_on_error)


def llt_rmsnorm_bwd_workspace_bytes(n: int, d: int) -> int:
    return lib().llt_rmsnorm_bwd_workspace_bytes(n, d)


def llt_rmsnorm_bwd(dtype, dy, x, g, rstd, n, d, dx, dg, ws, ws_bytes, stream=None, raise_on_error=True):
    return _call("llt_rmsnorm_bwd", dtype, ptr(dy), ptr(x), ptr(g), ptr(rstd), n, d, ptr(dx), ptr(dg), ptr(ws),
                 ws_bytes, stream_handle(stream), raise_on_error=raise_on_error)


def llt_gemm(op_dtype, a_kmajor, b_kmajor, A, lda, B, ldb, M, N, K, out_dtype, C, ldc, inv_a=None,
             inv_b=None, ws=None, ws_bytes=0, stream=None, raise_on_error=True):
    return _call("llt_gemm", op_dtype, int(a_kmajor), int(b_kmajor), ptr(A), lda, ptr(B), ldb, M, N, K,
                 out_dtype, ptr(C), ldc, ptr(inv_a), ptr(inv_b), ptr(ws), ws_bytes, stream_handle(stream),
                 raise_on_error=raise_on_error)


def llt_gemm_nt(op_dtype, A, lda, B, ldb, M, N, K, out_dtype, C, ldc, inv_a=None, inv_b=None, stream=None,
                raise_on_error=True):
    """llt_gemm with both operands K-major."""
    return llt_gemm(op_dtype, 1, 1, A, lda, B, ldb, M, N, K, out_dtype, C, ldc, inv_a, inv_b, None, 0, stream,
                    raise_on_error)


def llt_gemm_splitk_workspace_bytes(M, N, slices) -> int:
    return lib().llt_gemm_splitk_workspace_bytes(M, N, slices)


def llt_gemm_splitk(op_dtype, a_kmajor, b_kmajor, A, lda, B, ldb, M, N, K, slices, out_dtype, C, ldc, ws,
                    ws_bytes, inv_a=None, inv_b=None, stream=None, raise_on_error=True):
    return _call("llt_gemm_splitk", op_dtype, int(a_kmajor), int(b_kmajor), ptr(A), lda, ptr(B), ldb, M, N, K,
                 slices, out_dtype, ptr(C), ldc, ptr(inv_a), ptr(inv_b), ptr(ws), ws_bytes, stream_handle(stream),
                 raise_on_error=raise_on_error)


def llt_set_gemm_config(cfg: int):
    return _call("llt_set_gemm_config", cfg)


def llt_trace_begin(capacity: int):
    return _call("llt_trace_begin", capacity)


def llt_trace_end():
    return _call("llt_trace_end")


def llt_trace_count() -> int:
    return lib().llt_trace_count()


def llt_trace_get(i: int):
    tag = ctypes.c_char_p()
    ms = c_float()
    mnk = (c_int64 * 3)()
    _call("llt_trace_get", i, ctypes.byref(tag), ctypes.byref(ms), mnk)
    return tag.value.decode(), ms.value, (mnk[0], mnk[1], mnk[2])


def llt_trace_read() -> list:
    """[(tag, ms, (M, N, K))] of every launch recorded since llt_trace_begin."""
    return [llt_trace_get(i) for i in range(llt_trace_count())]


def llt_trace_get_gemm(i: int):
    """(block configuration, K slices) of GEMM launch i of the trace; (0, 0) for other launches."""
    cfg, sl = c_int32(), c_int32()
    _call("llt_trace_get_gemm", i, ctypes.byref(cfg), ctypes.byref(sl))
    return cfg.value, sl.value


def llt_layer_buffer(cfg: LayerCfg, region: int, name: str):
    """(byte offset, bytes) of a named intermediate inside saved (0), fwd ws (1) or bwd ws (2)."""
    off, nb = c_size_t(), c_size_t()
    _call("llt_layer_buffer", ctypes.byref(cfg), region, name.encode(), ctypes.byref(off), ctypes.byref(nb))
    return off.value, nb.value


def llt_e4m3_cast(x, n: int, scale: float, q, stream=None, raise_on_error=True):
    return _call("llt_e4m3_cast", ptr(x), n, scale, ptr(q), stream_handle(stream), raise_on_error=raise_on_error)


def ll_fp8_quant_tensorwise_noalloc(in_dtype, x, rows, cols, ld, q, q_t, scale, inv_scale, stream=None,
                                    raise_on_error=True):
    return _call("ll_fp8_quant_tensorwise_noalloc", in_dtype, ptr(x), rows, cols, ld, ptr(q), ptr(q_t),
                 ptr(scale), ptr(inv_scale), stream_handle(stream), raise_on_error=raise_on_error)


def ll_muon_workspace_bytes(rows: int, cols: int) -> int:
    return lib().ll_muon_workspace_bytes(rows, cols)


def ll_muon_step(dtype, w, grad, momentum_buf, rows, cols, lr, momentum, nesterov, weight_decay, ns_steps, ws,
                 ws_bytes, stream=None, raise_on_error=True):
    return _call("ll_muon_step", dtype, ptr(w), ptr(grad), ptr(momentum_buf), rows, cols, lr, momentum, int(nesterov),
                 weight_decay, ns_steps, ptr(ws), ws_bytes, stream_handle(stream), raise_on_error=raise_on_error)


def ll_adamw_step(param_dtype, grad_dtype, param, grad, exp_avg, exp_avg_sq, n, lr, beta1, beta2, eps,
                  weight_decay, step, stream=None, raise_on_error=True):
    return _call("ll_adamw_step", param_dtype, grad_dtype, ptr(param), ptr(grad), ptr(exp_avg), ptr(exp_avg_sq), n,
                 lr, beta1, beta2, eps, weight_decay, step, stream_handle(stream), raise_on_error=raise_on_error)
