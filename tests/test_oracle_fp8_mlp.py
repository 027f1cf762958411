"""Pin of oracle.model's FP8 MLP (forward and the straight-through backward) against an FP8 MLP
composed from torch CPU routines (tests/torch_fp8.py: float8_e4m3fn casts, torch._scaled_mm, a
searched power-of-two scale), and proof that the pin is sharp: mistakes planted in the oracle
(an operand that skips its quantisation, a bf16 operand where the e4m3 one belongs) fail it.

The two sides differ only in the summation order of the GEMMs (torch._scaled_mm sums in fp32, the
oracle in float64), which flips an occasional bf16 rounding and, through it, an occasional e4m3
code: measured below 3e-5 norm-wise on every output (bound 2e-4). Each planted mistake moves at
least one output by more than 2e-2 (asserted: more than 10x the bound)."""
import functools

import numpy as np
import pytest

from oracle import model as om
from oracle import numerics as nu
from tests import torch_fp8

TOL = 2e-4


def _inputs(seed=17, n=128, d=256, f=1024):
    rng = np.random.default_rng(seed)
    hn = nu.bf16_round(rng.standard_normal((n, d)))
    w1 = nu.bf16_round(rng.standard_normal((f, d)) * 0.02)
    w2 = nu.bf16_round(rng.standard_normal((d, f)) * 0.02)
    dm = nu.bf16_round(rng.standard_normal((n, d)))
    return hn, w1, w2, dm


@functools.lru_cache(maxsize=None)
def _torch_side(seed=17):
    return torch_fp8.mlp_fp8(*_inputs(seed))


def _oracle(hn, w1, w2, dm, cache_edit=None):
    R = om.rounder("bf16")
    m, c = om.mlp_fwd(hn, w1, w2, True, R)
    if cache_edit:
        c = dict(c, **cache_edit(c, w1, w2))
    dhn, dw1, dw2 = om.mlp_bwd(dm, c, w1, w2, True, R)
    return dict(u=c["u"], r=c["r"], m=m, dhn=dhn, dw1=dw1, dw2=dw2)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _errors(o, t):
    return {k: _rel(o[k], t[k]) for k in ("u", "r", "m", "dhn", "dw1", "dw2")}


@pytest.mark.parametrize("seed", [17, 18])
def test_fp8_mlp_matches_torch_scaled_mm_composition(seed):
    hn, w1, w2, dm = _inputs(seed)
    o = _oracle(hn, w1, w2, dm)
    t = _torch_side(seed)
    errs = _errors(o, t)
    assert max(errs.values()) <= TOL, errs


# planted mistakes, each in the oracle's cache between forward and backward
CACHE_MISTAKES = {
    "dW2 takes bf16 r instead of e4m3 r": lambda c, w1, w2: dict(r8=c["r"], inv_r=1.0),
    "dr takes W2 instead of Q(W2)": lambda c, w1, w2: dict(w28=w2, inv_w2=1.0),
    "dhn takes W1 instead of Q(W1)": lambda c, w1, w2: dict(w18=w1, inv_w1=1.0),
    "dW1 takes bf16 hn instead of e4m3 hn": lambda c, w1, w2: dict(hn8=c["hn"], inv_hn=1.0),
    "dW2 dequantised without the scale of r": lambda c, w1, w2: dict(inv_r=1.0),
}


@pytest.mark.parametrize("name", sorted(CACHE_MISTAKES))
def test_pin_catches_planted_operand_mistake(name):
    hn, w1, w2, dm = _inputs()
    t = _torch_side()
    errs = _errors(_oracle(hn, w1, w2, dm, CACHE_MISTAKES[name]), t)
    assert max(errs.values()) > 10 * TOL, (name, errs)


# planted mistakes: the k-th call of the quantiser returns its input unquantised (forward calls:
# hn, W1, r, W2; backward calls: dm, du)
@pytest.mark.parametrize("skip,what", [(0, "hn"), (1, "W1"), (2, "r"), (3, "W2"), (4, "dm"), (5, "du")])
def test_pin_catches_a_skipped_quantisation(monkeypatch, skip, what):
    hn, w1, w2, dm = _inputs()
    t = _torch_side()
    real = om.quantize_tensorwise
    calls = {"n": 0}

    def planted(x):
        k = calls["n"]
        calls["n"] += 1
        if k == skip:
            x = np.asarray(x, np.float64)
            return None, x, 1.0, 1.0
        return real(x)

    monkeypatch.setattr(om, "quantize_tensorwise", planted)
    errs = _errors(_oracle(hn, w1, w2, dm), t)
    assert calls["n"] == 6
    assert max(errs.values()) > 10 * TOL, (what, errs)
