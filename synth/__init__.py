"""Seeded synthetic inputs for the little-lm training-step hot path.

This module is shared by the oracle tests, the GPU parity tests and the benchmark.
It draws random tensors and nothing else: it holds none of the training step's
arithmetic (no norm, rotation, attention, MLP, loss or quantisation).

Recipe (one numpy generator per tensor, so every tensor is reproducible on its own):
  * generator  = numpy.random.default_rng([seed, k]) where k is the tensor's fixed
    index below (per-layer tensors of a multi-layer model add 100 * layer);
  * real tensors are drawn in float64, rounded to float32 (numpy's RNE cast) and,
    for bf16 configurations, rounded again to bf16 (round-to-nearest-even on the
    float32 bit pattern);
  * token ids and targets are drawn uniformly in [0, real_vocab).

The distributions are those of the workloads on the pages: activations N(0,1),
weights N(0, 0.02) (GPT-2 style initialisation, mentioned on the
"hn.213312.xyz translation" page, section "What didn't work"), norm gains and
residual scalars at their initial value 1.0; ``perturb=True`` draws gains
1 + N(0, 0.1) and residual scalars U(0.5, 1.5) instead, so that a test cannot pass
with a multiply by the gain or the scalar left out.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# fixed tensor indices (k in default_rng([seed, k]))
K_X, K_DY, K_WQKV, K_WO, K_W1, K_W2, K_VE, K_IDS = 0, 1, 2, 3, 4, 5, 6, 7
K_G1, K_G2, K_AATTN, K_AMLP = 8, 9, 10, 11
K_HIDDEN, K_WHEAD, K_TARGETS, K_EMB, K_GFINAL = 20, 21, 22, 23, 24
K_GENERIC = 50


def rng(seed: int, k: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(k)])


def round_to_bf16_values(a: np.ndarray) -> np.ndarray:
    """float32 array -> float32 array holding the nearest-even bf16 values (input prep)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array of bf16-representable values -> uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def normal(shape, std: float, seed: int, k: int, dtype: str = "bf16", mean: float = 0.0) -> np.ndarray:
    """float32 array of N(mean, std^2) draws, rounded to `dtype` ('fp32' or 'bf16')."""
    v = rng(seed, k).standard_normal(size=shape) * std + mean
    v = v.astype(np.float32)
    return round_to_bf16_values(v) if dtype == "bf16" else v


def uniform_ints(shape, high: int, seed: int, k: int) -> np.ndarray:
    return rng(seed, k).integers(0, high, size=shape, dtype=np.int64).astype(np.int32)


@dataclass
class LayerShape:
    batch: int
    seq: int
    d_model: int = 3072
    n_q_heads: int = 24
    n_kv_heads: int = 8
    head_dim: int = 128
    d_ff: int = 12288
    vocab: int = 50304          # padded vocab (rows of the value-embedding table and LM head)
    real_vocab: int = 50257     # ids/targets are drawn below this
    dtype: str = "bf16"         # 'bf16' or 'fp32'
    fp8_mlp: bool = True
    value_embed: bool = False
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    mlp: str = "relu2"          # "relu2", or "swiglu" (w_fc then holds 2 * d_ff rows: gate, then up)

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def qkv_dim(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim


# the five workloads of the hot path
TINY_FP32 = LayerShape(batch=2, seq=128, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                       d_ff=1024, vocab=512, real_vocab=512, dtype="fp32", fp8_mlp=False,
                       value_embed=True)
LAYER_1K = LayerShape(batch=40, seq=1024)                       # one layer, 40 x 1024 tokens
LAYER_2K_VE = LayerShape(batch=20, seq=2048, value_embed=True)  # value-embedding layer, 20 x 2048
LCE_TOKENS, LCE_DIM, LCE_VOCAB, LCE_REAL_VOCAB = 40960, 3072, 50304, 50257


@dataclass
class LayerInputs:
    shape: LayerShape
    x: np.ndarray
    dy: np.ndarray
    w_qkv: np.ndarray
    w_o: np.ndarray
    w_fc: np.ndarray
    w_proj: np.ndarray
    g_attn: np.ndarray
    g_mlp: np.ndarray
    a_attn: np.float32
    a_mlp: np.float32
    ids: np.ndarray | None = None
    ve_table: np.ndarray | None = None
    extra: dict = field(default_factory=dict)


def layer_inputs(s: LayerShape, seed: int = 0, layer: int = 0, perturb: bool = False,
                 x_std: float = 1.0, dy_std: float = 1.0, w_std: float = 0.02) -> LayerInputs:
    o = 100 * layer
    dt = s.dtype
    N, D = s.tokens, s.d_model
    x = normal((N, D), x_std, seed, K_X + o, dt)
    dy = normal((N, D), dy_std, seed, K_DY + o, dt)
    w_qkv = normal((s.qkv_dim, D), w_std, seed, K_WQKV + o, dt)
    w_o = normal((D, s.n_q_heads * s.head_dim), w_std, seed, K_WO + o, dt)
    w_fc = normal(((2 if s.mlp == "swiglu" else 1) * s.d_ff, D), w_std, seed, K_W1 + o, dt)
    w_proj = normal((D, s.d_ff), w_std, seed, K_W2 + o, dt)
    if perturb:
        g1 = (1.0 + 0.1 * rng(seed, K_G1 + o).standard_normal(D)).astype(np.float32)
        g2 = (1.0 + 0.1 * rng(seed, K_G2 + o).standard_normal(D)).astype(np.float32)
        a1 = np.float32(rng(seed, K_AATTN + o).uniform(0.5, 1.5))
        a2 = np.float32(rng(seed, K_AMLP + o).uniform(0.5, 1.5))
    else:
        g1 = np.ones(D, np.float32)
        g2 = np.ones(D, np.float32)
        a1 = np.float32(1.0)
        a2 = np.float32(1.0)
    ids = uniform_ints((N,), s.real_vocab, seed, K_IDS + o)
    ve = None
    if s.value_embed:
        ve = normal((s.vocab, s.n_kv_heads * s.head_dim), w_std, seed, K_VE + o, dt)
    return LayerInputs(s, x, dy, w_qkv, w_o, w_fc, w_proj, g1, g2, a1, a2, ids, ve)


@dataclass
class LceInputs:
    hidden: np.ndarray
    weight: np.ndarray
    targets: np.ndarray


def lce_inputs(n_tokens: int, d: int, vocab: int, real_vocab: int, dtype: str = "bf16",
               seed: int = 0, h_std: float = 1.0, w_std: float = 0.02,
               n_ignored: int = 0, ignore_index: int = -100) -> LceInputs:
    h = normal((n_tokens, d), h_std, seed, K_HIDDEN, dtype)
    w = normal((vocab, d), w_std, seed, K_WHEAD, dtype)
    t = uniform_ints((n_tokens,), real_vocab, seed, K_TARGETS)
    if n_ignored:
        idx = rng(seed, K_TARGETS + 1).choice(n_tokens, size=n_ignored, replace=False)
        t[idx] = ignore_index
    return LceInputs(h, w, t)


@dataclass
class ModelInputs:
    shape: LayerShape
    n_layers: int
    embed: np.ndarray            # [vocab, D]
    layers: list                 # [LayerInputs]; layer i carries a value-embedding table iff i is even
    g_final: np.ndarray          # [D] fp32
    head: np.ndarray             # [vocab, D]
    ids: np.ndarray              # int32 [N]
    targets: np.ndarray          # int32 [N]


def model_inputs(s: LayerShape, n_layers: int, seed: int = 0, perturb: bool = False,
                 w_std: float = 0.02) -> ModelInputs:
    """Inputs of the whole model: per-layer tensors as in layer_inputs(layer=i) (their x / dy are
    unused), value-embedding tables on the even layers, the token embedding and untied head drawn
    N(0, w_std), the final-norm gain 1 (or 1 + N(0, 0.1) with perturb), token ids from layer 0's
    generator and targets uniform in [0, real_vocab)."""
    from dataclasses import replace
    layers = [layer_inputs(replace(s, value_embed=(i % 2 == 0)), seed, layer=i, perturb=perturb, w_std=w_std)
              for i in range(n_layers)]
    embed = normal((s.vocab, s.d_model), w_std, seed, K_EMB, s.dtype)
    head = normal((s.vocab, s.d_model), w_std, seed, K_WHEAD, s.dtype)
    if perturb:
        g_final = (1.0 + 0.1 * rng(seed, K_GFINAL).standard_normal(s.d_model)).astype(np.float32)
    else:
        g_final = np.ones(s.d_model, np.float32)
    ids = layers[0].ids
    targets = uniform_ints((s.tokens,), s.real_vocab, seed, K_TARGETS)
    return ModelInputs(s, n_layers, embed, layers, g_final, head, ids, targets)
