"""GPU parity of the individual hot-path kernels against the oracle (bit-exact for the FP8
quantiser, tolerance for the GEMMs), called through the C ABI."""
import numpy as np
import pytest
import torch

import synth
import transformer_train_step_amd as ll
from oracle import numerics as nu
from tests.gpu_util import assert_close, dev, host, need_gpu

pytestmark = pytest.mark.gpu


def _quant_gpu(x_dev, in_dtype, rows, cols, want_t=True):
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    qt = torch.empty((cols, rows), dtype=torch.uint8, device="cuda") if want_t else None
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    inv = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    ll.ll_fp8_quant_tensorwise(in_dtype, x_dev, rows, cols, cols, q, qt, sc, inv, ws, ws.numel())
    torch.cuda.synchronize()
    return q, qt, sc, inv


@pytest.mark.parametrize("rows,cols,dtype,std", [
    (1, 16, "bf16", 1.0), (37, 48, "bf16", 1.0), (300, 3072, "bf16", 0.02), (129, 256, "fp32", 3.0),
    (1000, 12288, "bf16", 1.0), (64, 64, "fp32", 1e-30),
])
def test_fp8_quant_bitexact(rows, cols, dtype, std):
    need_gpu()
    print(f"quant {rows}x{cols} {dtype}", flush=True)
    x = synth.normal((rows, cols), std, seed=1, k=synth.K_GENERIC, dtype=dtype)
    q, qt, sc, inv = _quant_gpu(dev(x, dtype), ll.LL_BF16 if dtype == "bf16" else ll.LL_F32, rows, cols)
    codes, _, scale, inv_scale = nu.quantize_tensorwise(x.astype(np.float64))
    assert np.float32(sc.item()) == np.float32(scale)
    assert np.float32(inv.item()) == np.float32(inv_scale)
    got = q.cpu().numpy()
    assert np.array_equal(got, codes), f"{int((got != codes).sum())} codes differ"
    assert np.array_equal(qt.cpu().numpy(), codes.T)


def test_fp8_quant_empty_and_zero():
    need_gpu()
    q, qt, sc, inv = _quant_gpu(torch.zeros((0, 32), device="cuda", dtype=torch.bfloat16), ll.LL_BF16, 0, 32)
    assert sc.item() == 2.0 ** 48
    q, qt, sc, inv = _quant_gpu(torch.zeros((5, 32), device="cuda", dtype=torch.bfloat16), ll.LL_BF16, 5, 32)
    assert not q.cpu().numpy().any()


def test_e4m3_rounding_sweep():
    """Every fp32 in the binades around the subnormal/normal boundary and at the top of the
    range, plus random fp32 values: with amax = 448 the scale is exactly 1, so the kernel's codes
    are e4m3_RNE(x) and must equal the oracle's."""
    need_gpu()
    parts = []
    for e in (-12, -10, -9, -7, -6, -5, 7, 8):          # exponents of 2
        m = np.arange(0, 1 << 23, 3, dtype=np.uint32)     # every third mantissa
        parts.append(((np.uint32(e + 127) << 23) | m).view(np.float32))
    rng = np.random.default_rng(7)
    parts.append(rng.uniform(-448, 448, 2_000_000).astype(np.float32))
    parts.append(rng.standard_normal(1_000_000).astype(np.float32) * np.float32(0.01))
    x = np.concatenate(parts)
    x = np.concatenate([x, -x])
    x = x[np.abs(x) <= 448]
    x = np.concatenate([np.array([448.0], np.float32), x])
    cols = 4096
    pad = (-x.size) % cols
    x = np.concatenate([x, np.zeros(pad, np.float32)]).reshape(-1, cols)
    q, _, sc, _ = _quant_gpu(dev(x, "fp32"), ll.LL_F32, x.shape[0], cols, want_t=False)
    assert sc.item() == 1.0
    ref = nu.e4m3_encode(nu.e4m3_round(x.astype(np.float64)))
    got = q.cpu().numpy()
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} of {got.size} codes differ"


# ------------------------------------------------------------------ GEMM
@pytest.mark.parametrize("op,M,N,K,out", [
    ("fp32", 200, 136, 64, "fp32"), ("fp32", 256, 512, 256, "fp32"),
    ("bf16", 300, 264, 320, "fp32"), ("bf16", 130, 1032, 3072, "bf16"), ("bf16", 1, 8, 64, "fp32"),
    ("bf16", 4096, 4096, 3072, "bf16"), ("e4m3", 4096, 4096, 1024, "fp32"), ("fp32", 4096, 4096, 64, "fp32"),
    ("e4m3", 257, 200, 384, "fp32"), ("e4m3", 512, 384, 3072, "bf16"),
])
def test_gemm_nt_parity(op, M, N, K, out):
    need_gpu()
    print(f"gemm {op} {M}x{N}x{K} -> {out}", flush=True)
    rng = np.random.default_rng(M * 7 + N)
    if op == "e4m3":
        a_codes = rng.integers(0, 256, (M, K), dtype=np.uint8)
        b_codes = rng.integers(0, 256, (N, K), dtype=np.uint8)
        for c in (a_codes, b_codes):                     # normal finite codes only (no NaN, no
            bad = ((c & 0x7F) == 0x7F) | ((c & 0x78) == 0)   # subnormals: see the test below)
            c[bad] = 0x38
        A = torch.from_numpy(a_codes).cuda()
        B = torch.from_numpy(b_codes).cuda()
        ia = torch.tensor([0.015625], device="cuda")
        ib = torch.tensor([1.0 / 448.0], dtype=torch.float32, device="cuda")
        ref = (nu.e4m3_decode(a_codes) @ nu.e4m3_decode(b_codes).T) * ia.item() * ib.item()
        opd = ll._lib.LLT_OP_E4M3
    else:
        dt = "bf16" if op == "bf16" else "fp32"
        a = synth.normal((M, K), 1.0, 2, 1, dt)
        b = synth.normal((N, K), 0.05, 2, 2, dt)
        A, B = dev(a, dt), dev(b, dt)
        ia = ib = None
        ref = a.astype(np.float64) @ b.astype(np.float64).T
        opd = ll._lib.LLT_OP_BF16 if op == "bf16" else ll._lib.LLT_OP_F32
    C = torch.empty((M, N), dtype=torch.float32 if out == "fp32" else torch.bfloat16, device="cuda")
    ll.llt_gemm_nt(opd, A, K, B, K, M, N, K, ll.LL_F32 if out == "fp32" else ll.LL_BF16, C, N, ia, ib)
    torch.cuda.synchronize()
    got = host(C)
    if out == "bf16":
        ref = nu.bf16_round(ref)
        assert_close(got, ref, 4e-3, f"gemm {op}", elem_rtol=1e-2)
    elif op == "e4m3":
        # the e4m3 MFMA sums each 128-deep product block at reduced precision (see the probe below)
        assert_close(got, ref, 1e-4, f"gemm {op}", elem_rtol=2e-3)
    else:
        assert_close(got, ref, 1e-5, f"gemm {op}", elem_rtol=1e-4)


@pytest.mark.parametrize("ak,bk,M,N,K", [
    (True, False, 300, 264, 320), (False, True, 264, 136, 256), (False, False, 136, 520, 200),
    (False, False, 4096, 4096, 448), (True, False, 4096, 4096, 512), (True, True, 4096, 4104, 256),
    (False, False, 8, 8, 1),
])
def test_gemm_operand_layouts(ak, bk, M, N, K):
    """bf16 GEMM with K-major or MN-major operands (MN-major: A(m, k) = A[k, m]), both block-tile
    configurations (>= 256 tiles -> 256 x 256), ragged M/N, and a K that is not a multiple of the K
    tile for MN-major operands (their K tail reads a zero row)."""
    need_gpu()
    print(f"gemm layouts ak={ak} bk={bk} {M}x{N}x{K}", flush=True)
    a = synth.normal((M, K), 1.0, 3, 1, "bf16")
    b = synth.normal((N, K), 0.05, 3, 2, "bf16")
    ref = a.astype(np.float64) @ b.astype(np.float64).T
    A = dev(a if ak else np.ascontiguousarray(a.T), "bf16")
    B = dev(b if bk else np.ascontiguousarray(b.T), "bf16")
    lda = K if ak else M
    ldb = K if bk else N
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    ll.llt_gemm(ll._lib.LLT_OP_BF16, ak, bk, A, lda, B, ldb, M, N, K, ll.LL_F32, C, N, None, None, ws, 256)
    torch.cuda.synchronize()
    assert_close(host(C), ref, 1e-5, "gemm layouts", elem_rtol=1e-4)


@pytest.mark.parametrize("ak,bk,M,N,K,slices,out", [
    (False, False, 3072, 3072, 40960, 7, "bf16"),   # the attention output projection's weight gradient
    (False, False, 136, 520, 1000, 3, "fp32"),      # ragged M/N; last slice shorter, K tail reads zero rows
    (True, True, 264, 136, 700, 4, "fp32"),         # K-major operands, K padded to 704
    (True, False, 8, 8, 130, 5, "fp32"),            # more slices than 64-element K blocks: 3 slices run
    (False, False, 64, 64, 0, 2, "fp32"),           # empty K: zeros
])
def test_gemm_splitk(ak, bk, M, N, K, slices, out):
    """bf16 GEMM split along K into fp32 partial sums added by a second kernel: every slice boundary
    lies on a 64-element K tile, the last slice is ragged, MN-major tails read the zero row."""
    need_gpu()
    print(f"gemm splitk ak={ak} bk={bk} {M}x{N}x{K} slices={slices} out={out}", flush=True)
    a = synth.normal((M, K), 1.0, 5, 1, "bf16")
    b = synth.normal((N, K), 0.05, 5, 2, "bf16")
    kp = (K + 63) // 64 * 64
    ap = np.zeros((M, kp), dtype=a.dtype)
    bp = np.zeros((N, kp), dtype=b.dtype)
    ap[:, :K] = a
    bp[:, :K] = b
    A = dev(ap if ak else np.ascontiguousarray(a.T), "bf16")
    B = dev(bp if bk else np.ascontiguousarray(b.T), "bf16")
    lda = kp if ak else M
    ldb = kp if bk else N
    C = torch.full((M, N), 7.0, dtype=torch.float32 if out == "fp32" else torch.bfloat16, device="cuda")
    nws = ll.llt_gemm_splitk_workspace_bytes(M, N, slices)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ll.llt_gemm_splitk(ll._lib.LLT_OP_BF16, ak, bk, A, lda, B, ldb, M, N, K, slices,
                       ll.LL_F32 if out == "fp32" else ll.LL_BF16, C, N, ws, nws)
    torch.cuda.synchronize()
    got = host(C.float())
    if K == 0:
        assert np.all(got == 0.0)
        return
    if M * N > 1 << 20:
        # a 3072 x 3072 x 40960 product in float64 is costly on the host: check sampled rows
        rows = np.random.default_rng(0).choice(M, 48, replace=False)
        ref = a[rows].astype(np.float64) @ b.astype(np.float64).T
        got = got[rows]
    else:
        ref = a.astype(np.float64) @ b.astype(np.float64).T
    if out == "fp32":
        assert_close(got, ref, 1e-5, "gemm splitk", elem_rtol=1e-4)
    else:
        assert_close(got, ref, 4e-3, "gemm splitk bf16", elem_rtol=8e-3)


@pytest.mark.parametrize("M,N,K,slices", [
    (3072, 12288, 4096, 4),   # the MLP weight-gradient shape (D x F), 576 output tiles
    (200, 136, 1000, 3),      # ragged M/N, K padded to 1024 with zero codes
])
def test_gemm_splitk_e4m3(M, N, K, slices):
    """e4m3 GEMM split along K, the slices' fp32 partials added and scaled by inv_a * inv_b in the
    reduction kernel, compared with the exact product of the decoded codes."""
    need_gpu()
    print(f"gemm splitk e4m3 {M}x{N}x{K} slices={slices}", flush=True)
    rng = np.random.default_rng(21)
    kp = (K + 127) // 128 * 128
    a_codes = np.zeros((M, kp), np.uint8)
    b_codes = np.zeros((N, kp), np.uint8)
    a_codes[:, :K] = rng.integers(0, 0x7F, (M, K)) | (rng.integers(0, 2, (M, K)) << 7)
    b_codes[:, :K] = rng.integers(0, 0x7F, (N, K)) | (rng.integers(0, 2, (N, K)) << 7)
    a_codes[a_codes == 0xFF] = 0
    b_codes[b_codes == 0xFF] = 0
    ia, ib = 0.03125, 0.75
    inv = torch.tensor([ia, ib], dtype=torch.float32, device="cuda")
    C = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    nws = ll.llt_gemm_splitk_workspace_bytes(M, N, slices)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ll.llt_gemm_splitk(ll._lib.LLT_OP_E4M3, True, True, torch.from_numpy(a_codes).cuda(), kp,
                       torch.from_numpy(b_codes).cuda(), kp, M, N, K, slices, ll.LL_BF16, C, N, ws, nws,
                       inv[0:1], inv[1:2])
    torch.cuda.synchronize()
    got = host(C.float())
    rows = np.random.default_rng(1).choice(M, min(M, 64), replace=False)
    ref = (nu.e4m3_decode(a_codes[rows]) @ nu.e4m3_decode(b_codes).T) * ia * ib
    # bf16 output rounding plus the e4m3 MFMA's reduced-precision 128-deep sums
    assert_close(got[rows], ref, 4e-3, "gemm splitk e4m3", elem_rtol=1e-2)


def test_gemm_e4m3_subnormal_operands():
    """Subnormal e4m3 operands (|v| < 2^-6) take part in the e4m3 MFMA like normal ones: A holds
    only subnormal codes, B only normal codes, and the result equals the exact GEMM to the MFMA's
    summation precision (see the next test)."""
    need_gpu()
    rng = np.random.default_rng(11)
    M, N, K = 64, 64, 256
    a_codes = (rng.integers(1, 8, (M, K)) | (rng.integers(0, 2, (M, K)) << 7)).astype(np.uint8)
    b_codes = rng.integers(0x08, 0x7F, (N, K)).astype(np.uint8)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ll.llt_gemm_nt(ll._lib.LLT_OP_E4M3, torch.from_numpy(a_codes).cuda(), K, torch.from_numpy(b_codes).cuda(), K,
                   M, N, K, ll.LL_F32, C, N)
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    ref = nu.e4m3_decode(a_codes) @ nu.e4m3_decode(b_codes).T
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"e4m3 subnormal operands: relative error {rel:.2e}", flush=True)
    assert rel <= 2e-3


def test_gemm_e4m3_products_and_accumulation_precision():
    """Every product of two finite e4m3 values is exact in the e4m3 MFMA (one product per output:
    A[i, 0] = code i, B[j, 0] = code j). The sum of a 128-deep block is not an fp32 sum: measured
    on gfx950, 2^16 + 127 * 1 gives 65656 (the 7 ones that share an 8-product group with 2^16
    are dropped), so the test bounds the relative deviation by 2^-10 and the GEMM parity tests
    use 1e-4 for e4m3."""
    need_gpu()
    codes = np.arange(256, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    K = 128
    A = np.zeros((256, K), np.uint8)
    A[:, 0] = codes
    C = torch.empty((256, 256), dtype=torch.float32, device="cuda")
    Ad = torch.from_numpy(A).cuda()
    ll.llt_gemm_nt(ll._lib.LLT_OP_E4M3, Ad, K, Ad, K, 256, 256, K, ll.LL_F32, C, 256)
    torch.cuda.synchronize()
    v = nu.e4m3_decode(codes)
    ref = np.outer(v, v)
    got = C.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} of 65536 single products differ"
    A = np.full((16, K), 0x38, np.uint8)             # 1.0
    A[:, 0] = 0x78                                   # 256 = 2^8
    Ad = torch.from_numpy(A).cuda()
    C = torch.empty((16, 16), dtype=torch.float32, device="cuda")
    ll.llt_gemm_nt(ll._lib.LLT_OP_E4M3, Ad, K, Ad, K, 16, 16, K, ll.LL_F32, C, 16)
    torch.cuda.synchronize()
    got = float(C[0, 0].item())
    print(f"e4m3 MFMA: 2^16 + 127 * 1 = {got} (exact 65663)", flush=True)
    assert abs(got - 65663.0) <= 65663.0 * 2.0 ** -10


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15])
@pytest.mark.parametrize("op,ak,bk,K", [
    ("bf16", True, True, 64), ("bf16", True, True, 192), ("bf16", True, True, 320),
    ("bf16", False, False, 200), ("bf16", True, False, 1000), ("bf16", False, True, 96),
    ("fp32", True, True, 96), ("e4m3", True, True, 128), ("e4m3", True, True, 384), ("e4m3", True, True, 640),
    ("e4m3", True, True, 2048),
])
def test_gemm_block_configs(cfg, op, ak, bk, K):
    """Every block-tile / K-tile / LDS-stage configuration on ragged M and N and on K-tile counts
    of 1 to 16, so that each pipeline depth meets its prologue, steady state and drain."""
    need_gpu()
    print(f"gemm cfg{cfg} {op} ak={ak} bk={bk} K={K}", flush=True)
    M, N = 264, 520
    if op == "e4m3":
        rng = np.random.default_rng(K)
        a_codes = rng.integers(0, 256, (M, K), dtype=np.uint8)
        b_codes = rng.integers(0, 256, (N, K), dtype=np.uint8)
        for c in (a_codes, b_codes):
            c[((c & 0x7F) == 0x7F) | ((c & 0x78) == 0)] = 0x38
        a, b = nu.e4m3_decode(a_codes), nu.e4m3_decode(b_codes)
        A, B = torch.from_numpy(a_codes).cuda(), torch.from_numpy(b_codes).cuda()
        opd, tol = ll._lib.LLT_OP_E4M3, (1e-4, 2e-3)
    else:
        a = synth.normal((M, K), 1.0, 4, 1, op)
        b = synth.normal((N, K), 0.05, 4, 2, op)
        A = dev(a if ak else np.ascontiguousarray(a.T), op)
        B = dev(b if bk else np.ascontiguousarray(b.T), op)
        opd, tol = (ll._lib.LLT_OP_BF16 if op == "bf16" else ll._lib.LLT_OP_F32), (1e-5, 1e-4)
    if ak and op != "e4m3":
        A = torch.nn.functional.pad(A, (0, (-K) % 64))      # K-major rows padded to the K tile
    if bk and op != "e4m3":
        B = torch.nn.functional.pad(B, (0, (-K) % 64))
    ref = a.astype(np.float64) @ b.astype(np.float64).T
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    try:
        ll._lib.llt_set_gemm_config(cfg)
        ll.llt_gemm(opd, ak, bk, A, A.shape[1], B, B.shape[1], M, N, K, ll.LL_F32, C, N, None, None, ws, 256)
        torch.cuda.synchronize()
    finally:
        ll._lib.llt_set_gemm_config(0)
    assert_close(host(C), ref, tol[0], f"gemm cfg{cfg}", elem_rtol=tol[1])
