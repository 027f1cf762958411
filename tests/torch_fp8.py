"""An FP8 MLP built from torch CPU library routines only, independent of the oracle's code: the
e4m3 codes from torch's float8_e4m3fn cast, every FP8 GEMM through torch._scaled_mm (the routine
the pages name for the three FP8 GEMMs of each linear [linlog.top article, 吞吐量优化;
hn.213312.xyz translation, 提升吞吐量 / Increasing throughput]) and bf16 rounding by torch's
bfloat16 cast. The scale is found by a search over powers of two, not by exponent arithmetic.
Test infrastructure: it pins oracle.model's FP8 branch."""
from __future__ import annotations

import numpy as np
import torch


def search_scale(amax32: float) -> float:
    """Largest power of two 2^k (integer k in [-160, 160]) that is <= the fp32 quotient
    448 / max(amax, 1e-12), the quotient formed by torch's fp32 division. Powers of two are exact
    in float64, so every comparison is exact."""
    num = torch.tensor(448.0, dtype=torch.float32)
    den = torch.clamp(torch.tensor(amax32, dtype=torch.float32), min=torch.tensor(1e-12, dtype=torch.float32))
    ratio = float(num / den)
    best = None
    for k in range(-160, 161):
        if 2.0 ** k <= ratio:
            best = 2.0 ** k
    assert best is not None and best <= ratio < 2 * best
    return best


def quant(t: torch.Tensor):
    """(codes as float8_e4m3fn, inverse scale) of a float32 tensor: amax by torch's max, the
    codes by torch's cast of the clamped fp32 product x * scale."""
    t = t.to(torch.float32)
    scale = search_scale(float(t.abs().max()) if t.numel() else 0.0)
    q = (t * torch.tensor(scale, dtype=torch.float32)).clamp(-448, 448).to(torch.float8_e4m3fn)
    return q, 1.0 / scale


def smm(a8: torch.Tensor, inv_a: float, b8_kn: torch.Tensor, inv_b: float) -> torch.Tensor:
    """deq(a8 @ b8_kn) by torch._scaled_mm (fp32 out): a8 [M, K], b8_kn [K, N] (any layouts)."""
    a = a8.contiguous()
    b = b8_kn.t().contiguous().t()               # column-major second operand
    return torch._scaled_mm(a, b, scale_a=torch.tensor(inv_a), scale_b=torch.tensor(inv_b),
                            out_dtype=torch.float32)


def bf(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float32)


def mlp_fp8(hn, w_fc, w_proj, dm):
    """Forward and straight-through backward of m = relu(hn W1^T)^2 W2^T with the three GEMMs of each
    linear on tensorwise-quantised e4m3 operands, every stored tensor rounded to bf16. Inputs are
    numpy arrays of bf16 values; returns a dict of float64 numpy arrays."""
    f = lambda a: torch.from_numpy(np.asarray(a, np.float32))
    hn, w1, w2, dm = f(hn), f(w_fc), f(w_proj), f(dm)
    hn8, i_hn = quant(hn)
    w18, i_w1 = quant(w1)
    u = bf(smm(hn8, i_hn, w18.t(), i_w1))                 # [N, F]
    r = bf(torch.relu(u) ** 2)
    r8, i_r = quant(r)
    w28, i_w2 = quant(w2)
    m = bf(smm(r8, i_r, w28.t(), i_w2))                   # [N, D]
    dm8, i_dm = quant(dm)
    dr = bf(smm(dm8, i_dm, w28, i_w2))                    # [N, F] = dm W2
    dw2 = bf(smm(dm8.t(), i_dm, r8, i_r))                 # [D, F] = dm^T r
    du = bf(dr * (2.0 * torch.relu(u)))
    du8, i_du = quant(du)
    dw1 = bf(smm(du8.t(), i_du, hn8, i_hn))               # [F, D] = du^T hn
    dhn = bf(smm(du8, i_du, w18, i_w1))                   # [N, D] = du W1
    out = dict(u=u, r=r, m=m, dr=dr, du=du, dw1=dw1, dw2=dw2, dhn=dhn)
    return {k: v.double().numpy() for k, v in out.items()}
