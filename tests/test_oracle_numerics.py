"""Pins of oracle.numerics (bf16 rounding, e4m3fn format, tensorwise quantiser) against things
other than itself: hand-derived fixtures from the format definitions, torch's CPU casts and
torch._scaled_mm (the routine the pages name for the FP8 GEMMs)."""
import os

import numpy as np
import pytest
import torch

from oracle import numerics as nu
from tests import torch_fp8

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _parse_num(s: str) -> float:
    s = s.strip()
    if "p" in s:
        return float.fromhex(s)
    return float(s)


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),     # subnormal range
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38], np.float32),
    ])
    # exact ties: bf16 value + half a bf16 ulp
    b = rng.standard_normal(20000).astype(np.float32)
    bits = (b.view(np.uint32) & 0xFFFF0000) | 0x8000
    x = np.concatenate([x, bits.view(np.float32)])
    ours = nu.bf16_round(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))


def test_e4m3_value_set():
    vals = nu.e4m3_decode(np.arange(256))
    finite = vals[np.isfinite(vals)]
    assert finite.size == 254
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    assert finite.max() == 448.0 and finite.min() == -448.0
    pos = np.unique(finite[finite > 0])
    assert pos.size == 126 and pos[0] == 2.0 ** -9
    assert np.array_equal(vals[:127], -vals[128:255])
    # matches torch's own decoder of the same bytes
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(t), np.isnan(vals))
    assert np.array_equal(t[np.isfinite(t)], finite)


def test_e4m3_golden_cases():
    rows = []
    with open(os.path.join(GOLD, "e4m3_cases.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    assert len(rows) >= 15
    for inp, rounded, code in rows:
        v = _parse_num(inp)
        r = nu.e4m3_round(np.array([v]))
        assert r[0] == _parse_num(rounded), inp
        assert np.signbit(r[0]) == np.signbit(_parse_num(rounded)), inp
        assert int(nu.e4m3_encode(r)[0]) == int(code, 16), inp


def test_e4m3_round_matches_torch_cast():
    rng = np.random.default_rng(2)
    pos = nu.e4m3_decode(np.arange(0, 127))
    mids = (pos[:-1] + pos[1:]) / 2                          # every tie
    x = np.concatenate([
        mids, -mids,
        np.nextafter(mids.astype(np.float32), np.float32(np.inf)).astype(np.float64),
        np.nextafter(mids.astype(np.float32), np.float32(0)).astype(np.float64),
        rng.uniform(-448, 448, 200000),
        rng.standard_normal(200000) * 0.01,
        rng.standard_normal(200000) * 2.0 ** -8,
    ]).astype(np.float32)
    x = np.clip(x, -448, 448).astype(np.float64)
    ours = nu.e4m3_encode(nu.e4m3_round(x))
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_quantizer_golden_example():
    kv = {}
    with open(os.path.join(GOLD, "fp8_quant_example.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, *v = line.split()
                kv[k] = v
    x = np.array([_parse_num(v) for v in kv["x"]])
    codes, vals, scale, inv = nu.quantize_tensorwise(x)
    assert scale == _parse_num(kv["scale"][0])
    assert inv == _parse_num(kv["inv_scale"][0])
    assert [int(c) for c in codes] == [int(c, 16) for c in kv["codes"]]
    assert np.array_equal(vals, nu.e4m3_decode(codes))


def _torch_quant(x32: np.ndarray):
    q, inv = torch_fp8.quant(torch.from_numpy(x32))
    return q, 1.0 / inv, inv


@pytest.mark.parametrize("std", [1.0, 0.02, 1e-4, 30.0])
def test_quantizer_matches_torch(std):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 96)) * std).astype(np.float32)
    codes, vals, scale, inv = nu.quantize_tensorwise(x.astype(np.float64))
    q, ts, tinv = _torch_quant(x)
    assert np.float32(scale) == np.float32(ts)
    assert np.float32(inv) == np.float32(tinv)
    assert np.array_equal(codes, q.view(torch.uint8).numpy())


def test_quantizer_degenerate_inputs():
    codes, vals, scale, inv = nu.quantize_tensorwise(np.zeros((4, 4)))
    assert np.all(codes == 0)
    assert scale == 2.0 ** 48                        # 448 / 1e-12 = 4.48e14 in [2^48, 2^49)
    # amax a power of two times 448/2^k maps exactly onto +-448; otherwise into [224, 448]
    codes, vals, scale, inv = nu.quantize_tensorwise(np.array([[-3.5, 1.0, 2.0]]))
    assert scale == 128.0 and vals[0, 0] == -448.0
    codes, vals, scale, inv = nu.quantize_tensorwise(np.array([[-3.0, 1.0, 2.0]]))
    assert scale == 128.0 and vals[0, 0] == -384.0 and inv == 1.0 / 128
    for amax in np.geomspace(1e-6, 1e6, 97):
        _, v, sc, iv = nu.quantize_tensorwise(np.array([amax, -amax / 3]))
        assert 224.0 <= v[0] <= 448.0 and sc * iv == 1.0 and np.log2(sc) == np.floor(np.log2(sc))


def test_fp8_gemm_matches_torch_scaled_mm():
    """deq(A8 B8^T) = (sum of exact products) * inv_a * inv_b is what torch._scaled_mm computes."""
    rng = np.random.default_rng(4)
    a = rng.standard_normal((32, 256)).astype(np.float32)
    b = (rng.standard_normal((48, 256)) * 0.02).astype(np.float32)
    _, av, _, ainv = nu.quantize_tensorwise(a.astype(np.float64))
    _, bv, _, binv = nu.quantize_tensorwise(b.astype(np.float64))
    ours = nu.fp8_matmul_nt(av, ainv, bv, binv)
    qa, _, tia = _torch_quant(a)
    qb, _, tib = _torch_quant(b)
    ref = torch._scaled_mm(qa, qb.t(), scale_a=torch.tensor(tia), scale_b=torch.tensor(tib),
                           out_dtype=torch.float32).double().numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())


def test_scale_matches_search_over_amax_sweep():
    """The oracle's scale against the largest power of two below 448 / amax found by search, over
    amax values at, just below and just above binade edges, the 1e-12 floor and beyond."""
    am = [0.0, 1e-30, 1e-12, 1.5e-12, 448.0, 448.0 * 2 ** -20, 3.0e38]
    for k in range(-40, 41):
        edge = 448.0 * 2.0 ** k                   # 448 / amax is a power of two exactly here
        am += [edge, float(np.nextafter(np.float32(edge), np.float32(0))),
               float(np.nextafter(np.float32(edge), np.float32(np.inf))), 0.7 * edge]
    for a in am:
        a32 = float(np.float32(a))
        _, _, scale, inv = nu.quantize_tensorwise(np.array([a32, -a32 / 2]))
        assert scale == torch_fp8.search_scale(a32), a32
        assert inv * scale == 1.0
