"""Torch-side convenience around the C ABI: allocates outputs, `saved` and workspace buffers with
torch on the current device and calls libll. No arithmetic happens here."""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib as L


@dataclass
class LayerConfig:
    batch: int
    seq: int
    d_model: int = 3072
    n_q_heads: int = 24
    n_kv_heads: int = 8
    head_dim: int = 128
    d_ff: int = 12288
    dtype: str = "bf16"          # 'bf16' or 'fp32'
    fp8_mlp: bool = True
    value_embed: bool = False
    ve_rows: int = 50304
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    mlp: str = "relu2"           # 'relu2' or 'swiglu' (w_fc [2 d_ff, D]: gate rows, then up rows)

    def c_struct(self) -> L.LayerCfg:
        return L.LayerCfg(dtype=L.LL_BF16 if self.dtype == "bf16" else L.LL_F32, fp8_mlp=int(self.fp8_mlp),
                          batch=self.batch, seq=self.seq, d_model=self.d_model, n_q_heads=self.n_q_heads,
                          n_kv_heads=self.n_kv_heads, head_dim=self.head_dim, d_ff=self.d_ff,
                          rms_eps=self.rms_eps, rope_theta=self.rope_theta,
                          has_value_embed=int(self.value_embed), ve_rows=self.ve_rows if self.value_embed else 0,
                          mlp_kind=L.LL_MLP_SWIGLU if self.mlp == "swiglu" else L.LL_MLP_RELU2)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def qkv_dim(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


PARAM_NAMES = ("attn_norm_w", "w_qkv", "w_o", "mlp_norm_w", "w_fc", "w_proj", "ve_table", "resid_attn", "resid_mlp")


def param_shapes(c: LayerConfig) -> dict:
    D, F = c.d_model, c.d_ff
    s = {"attn_norm_w": (D,), "w_qkv": (c.qkv_dim, D), "w_o": (D, c.n_q_heads * c.head_dim),
         "mlp_norm_w": (D,), "w_fc": ((2 if c.mlp == "swiglu" else 1) * F, D), "w_proj": (D, F),
         "resid_attn": (1,), "resid_mlp": (1,)}
    if c.value_embed:
        s["ve_table"] = (c.ve_rows, c.n_kv_heads * c.head_dim)
    return s


def _is_fp32_param(name: str) -> bool:
    return name in ("attn_norm_w", "mlp_norm_w", "resid_attn", "resid_mlp")


class Layer:
    """One decoder layer bound to a configuration: owns the `saved` and workspace buffers."""

    def __init__(self, cfg: LayerConfig, device="cuda"):
        self.cfg = cfg
        self.c = cfg.c_struct()
        self.saved_bytes = L.ll_layer_saved_bytes(self.c)
        self.ws_bytes = L.ll_layer_workspace_bytes(self.c)
        if self.saved_bytes == 0 or self.ws_bytes == 0:
            raise L.LLError(L.LL_ERR_INVALID_ARG, "ll_layer_*_bytes", "invalid layer configuration")
        self.saved = torch.empty(self.saved_bytes, dtype=torch.uint8, device=device)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.device = device

    def c_params(self, p: dict) -> L.LayerParams:
        return L.LayerParams(**{k: L.ptr(p.get(k)) for k in PARAM_NAMES})

    def new_grads(self) -> dict:
        g = {}
        for k, shp in param_shapes(self.cfg).items():
            dt = torch.float32 if (_is_fp32_param(k) or k == "ve_table") else self.cfg.torch_dtype
            g[k] = (torch.zeros if k == "ve_table" else torch.empty)(shp, dtype=dt, device=self.device)
        return g

    def forward(self, p: dict, x: torch.Tensor, ids: torch.Tensor | None, y: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
        if y is None:
            y = torch.empty_like(x)
        L.ll_layer_fwd(self.c, self.c_params(p), x, ids, y, self.saved, self.saved_bytes, self.ws, self.ws_bytes,
                       stream)
        return y

    def backward(self, p: dict, x, ids, dy, dx=None, grads: dict | None = None, stream=None, accumulate=False):
        if dx is None:
            dx = torch.empty_like(dy)
        if grads is None:
            grads = self.new_grads()
        cg = L.LayerGrads(**{k: L.ptr(grads.get(k)) for k in PARAM_NAMES}, accumulate=int(accumulate))
        L.ll_layer_bwd(self.c, self.c_params(p), x, ids, self.saved, self.saved_bytes, dy, dx, cg, self.ws,
                       self.ws_bytes, stream)
        return dx, grads


class FusedLCE:
    """Fused linear cross-entropy bound to (dtype, n, d, v, token_chunk): owns its workspace."""

    def __init__(self, dtype: str, n: int, d: int, v: int, token_chunk: int = 0, vocab_tile: int = 0, device="cuda"):
        self.dt = L.LL_BF16 if dtype == "bf16" else L.LL_F32
        self.n, self.d, self.v, self.chunk, self.vocab_tile = n, d, v, token_chunk, vocab_tile
        self.ws_bytes = L.ll_fused_lce_workspace_bytes(self.dt, n, d, v, token_chunk, vocab_tile)
        if self.ws_bytes == 0:
            raise L.LLError(L.LL_ERR_INVALID_ARG, "ll_fused_lce_workspace_bytes", "invalid sizes")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.loss = torch.empty(1, dtype=torch.float32, device=device)
        self.device = device

    def __call__(self, hidden, weight, targets, softcap=15.0, ignore_index=-100, grad_scale=1.0, grads=True,
                 lse=None, d_hidden=None, d_weight=None, stream=None, accumulate_dw=False):
        if grads:
            d_hidden = torch.empty_like(hidden) if d_hidden is None else d_hidden
            d_weight = torch.empty_like(weight) if d_weight is None else d_weight
        L.ll_fused_lce_fwd_bwd(self.dt, hidden, weight, targets, self.n, self.d, self.v, softcap, ignore_index,
                               grad_scale, self.chunk, self.vocab_tile, accumulate_dw, self.loss, lse,
                               d_hidden if grads else None, d_weight if grads else None, self.ws, self.ws_bytes,
                               stream)
        return self.loss, d_hidden, d_weight


class Model:
    """The whole model (embedding, n_layers decoder layers, final RMSNorm, untied head + fused
    linear cross-entropy) bound to a per-layer configuration: owns the `saved` and workspace
    buffers of ll_model_fwd_bwd. Layer i is a value-embedding layer iff its parameter dict holds a
    "ve_table" (in the 3.8B model: the even layers)."""

    def __init__(self, cfg: LayerConfig, n_layers: int, vocab: int, token_chunk: int = 0, device="cuda"):
        self.cfg, self.n_layers, self.vocab, self.chunk = cfg, n_layers, vocab, token_chunk
        self.c = cfg.c_struct()
        self.saved_bytes = L.ll_model_saved_bytes(self.c, n_layers, vocab)
        self.ws_bytes = L.ll_model_workspace_bytes(self.c, n_layers, vocab, token_chunk)
        if self.saved_bytes == 0 or self.ws_bytes == 0:
            raise L.LLError(L.LL_ERR_INVALID_ARG, "ll_model_*_bytes", L.ll_last_error())
        self.saved = torch.empty(self.saved_bytes, dtype=torch.uint8, device=device)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.loss = torch.empty(1, dtype=torch.float32, device=device)
        self.device = device

    def layer_shapes(self, value_embed: bool) -> dict:
        c = LayerConfig(**{**self.cfg.__dict__, "value_embed": value_embed, "ve_rows": self.vocab})
        return param_shapes(c)

    def new_grads(self, params: dict) -> dict:
        dt = self.cfg.torch_dtype
        D = self.cfg.d_model
        layers = []
        for lp in params["layers"]:
            g = {}
            for k, shp in self.layer_shapes("ve_table" in lp and lp["ve_table"] is not None).items():
                gdt = torch.float32 if (_is_fp32_param(k) or k == "ve_table") else dt
                g[k] = (torch.zeros if k == "ve_table" else torch.empty)(shp, dtype=gdt, device=self.device)
            layers.append(g)
        return {"embed": torch.empty((self.vocab, D), dtype=torch.float32, device=self.device),
                "layers": layers,
                "final_norm_w": torch.empty(D, dtype=torch.float32, device=self.device),
                "head": torch.empty((self.vocab, D), dtype=dt, device=self.device)}

    def __call__(self, params: dict, token_ids, targets, grads: dict, softcap=15.0, ignore_index=-100,
                 grad_scale=1.0, stream=None, accumulate=False, loss=None):
        lp = (L.LayerParams * self.n_layers)(*[L.LayerParams(**{k: L.ptr(p.get(k)) for k in PARAM_NAMES})
                                               for p in params["layers"]])
        lg = (L.LayerGrads * self.n_layers)(*[L.LayerGrads(**{k: L.ptr(g.get(k)) for k in PARAM_NAMES})
                                              for g in grads["layers"]])
        mp = L.ModelParams(L.ptr(params["embed"]), lp, L.ptr(params["final_norm_w"]), L.ptr(params["head"]))
        mg = L.ModelGrads(L.ptr(grads["embed"]), lg, L.ptr(grads["final_norm_w"]), L.ptr(grads["head"]),
                          int(accumulate))
        loss = self.loss if loss is None else loss
        L.ll_model_fwd_bwd(self.c, self.n_layers, self.vocab, mp, token_ids, targets, softcap, ignore_index,
                           grad_scale, self.chunk, loss, mg, self.saved, self.saved_bytes, self.ws,
                           self.ws_bytes, stream)
        return loss


# The run's optimizer groups [youdonthavefriends cost analysis, "config appendix"]: Muon for the
# layer matrices, AdamW (lr, beta1, beta2, eps, weight decay) per group for the rest; the norm gains
# are read as members of the "scalars" group.
MUON = dict(lr=0.02, momentum=0.95, weight_decay=0.0, nesterov=1, ns_steps=5)
ADAMW = {"embeddings": (0.1414, 0.8, 0.995, 1e-10, 0.001), "lm_head": (0.002828, 0.8, 0.96, 1e-10, 0.01),
         "value_embeds": (0.0707, 0.8, 0.995, 1e-10, 0.01), "scalars": (0.005, 0.8, 0.95, 1e-10, 0.05)}
MATRICES = ("w_qkv", "w_o", "w_fc", "w_proj")


class TrainStep:
    """One optimizer step of the whole model on one GPU: `accum` micro-batches through
    ll_model_fwd_bwd (the first overwrites the gradients, the others add into them; each loss is
    scaled by 1/accum so the gradients are those of the mean loss), then ll_muon_step on every layer
    matrix and ll_adamw_step on the token embedding, the head, the value-embedding tables and the
    gains and residual scalars. Owns the gradients and the optimizer state; the optimizer state
    lives beside the master weights in their dtype (bf16 for bf16 weights)."""

    def __init__(self, model: Model, params: dict, accum: int = 7):
        self.model, self.p, self.accum = model, params, accum
        dev = model.device
        self.g = model.new_grads(params)
        self.t = 0
        self.losses = torch.zeros(accum, dtype=torch.float32, device=dev)
        self.muon = []          # (weight, gradient, momentum buffer)
        self.adamw = []         # (group, param, grad, exp_avg, exp_avg_sq)
        for lp, lg in zip(params["layers"], self.g["layers"]):
            for k in MATRICES:
                self.muon.append((lp[k], lg[k], torch.zeros_like(lp[k])))
            if lp.get("ve_table") is not None:
                self.adamw.append(("value_embeds", lp["ve_table"], lg["ve_table"]))
            for k in ("attn_norm_w", "mlp_norm_w", "resid_attn", "resid_mlp"):
                self.adamw.append(("scalars", lp[k], lg[k]))
        self.adamw += [("embeddings", params["embed"], self.g["embed"]), ("lm_head", params["head"], self.g["head"]),
                       ("scalars", params["final_norm_w"], self.g["final_norm_w"])]
        self.adamw = [(grp, p, g, torch.zeros_like(p), torch.zeros_like(p)) for grp, p, g in self.adamw]
        wsb = max(L.ll_muon_workspace_bytes(*w.shape) for w, _, _ in self.muon)
        self.muon_ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    @staticmethod
    def _dt(t):
        return L.LL_BF16 if t.dtype == torch.bfloat16 else L.LL_F32

    def backward_all(self, batches, stream=None):
        """The accumulated gradients of the micro-batches [(token_ids, targets)]; losses into self.losses."""
        assert len(batches) == self.accum
        for i, (ids, targets) in enumerate(batches):
            self.model(self.p, ids, targets, self.g, grad_scale=1.0 / self.accum, stream=stream,
                       accumulate=i > 0, loss=self.losses[i:i + 1])

    def optimizer_step(self, stream=None):
        self.t += 1
        m = MUON
        for w, g, buf in self.muon:
            L.ll_muon_step(L.LL_BF16, w, g, buf, w.shape[0], w.shape[1], m["lr"], m["momentum"], m["nesterov"],
                           m["weight_decay"], m["ns_steps"], self.muon_ws, self.muon_ws.numel(), stream)
        for grp, p, g, ea, eas in self.adamw:
            lr, b1, b2, eps, wd = ADAMW[grp]
            L.ll_adamw_step(self._dt(p), self._dt(g), p, g, ea, eas, p.numel(), lr, b1, b2, eps, wd, self.t, stream)

    def __call__(self, batches, stream=None):
        self.backward_all(batches, stream)
        self.optimizer_step(stream)
        return self.losses
