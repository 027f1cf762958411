"""ORACLE — plain, slow, obviously-correct CPU reference of the little-lm training-step hot path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library (``transformer_train_step_amd``) never
imports it, and this package imports nothing from the product: the two share no code. The only
module both sides use is ``synth`` (seeded random inputs, none of the method's arithmetic).

What it computes, and where the pages state it (citations name the page and the section on it):

* the decoder layer of the little-lm 3.8B model — RMSNorm, RoPE, GQA 24q/8kv heads of dim 128,
  QK-norm, causal attention, non-gated relu^2 MLP at 4x width, learnable per-layer residual
  scalars, ResFormer-style value embeddings on alternate layers
  [hn.213312.xyz translation, "设置 / Setup"; youdonthavefriends cost analysis, "config appendix"];
* FP8 e4m3 dynamic tensorwise scaling of the three GEMMs (one forward, two backward) of each MLP
  linear [hn.213312.xyz translation, "提升吞吐量 / Increasing throughput"; linlog.top article,
  "吞吐量优化"];
* the fused linear cross-entropy with tanh logit softcap 15 over the 50304-padded vocabulary
  [youdonthavefriends cost analysis, "Increasing throughput" and "config appendix"];
* the whole model around the layers — token embedding, final RMSNorm, untied head, and the
  backward chain through them ([hn.213312.xyz translation, "设置 / Setup", parameter table]).

Everything is evaluated in float64 numpy. In bf16 mode the oracle rounds to bf16 exactly where
the GPU path stores a bf16 tensor (the rounding contract in ``oracle.model``), and FP8 operands go
through an exact emulation of the e4m3 tensorwise quantiser (``oracle.numerics``).

Pins (what each function is checked against, other than itself) live in ``tests/test_oracle_*.py``.
Functions without an independent pin say "parity unpinned" in their docstring:
  * ``model.rope`` pairing convention (rotate-half) — the pages give only theta;
  * ``model.layer_fwd``/``layer_bwd`` residual-scalar placement — the pages say only
    "learnable per-layer residual scalars" / ``layer_scale: true``.
"""
from . import numerics, model, lce, full_model  # noqa: F401
