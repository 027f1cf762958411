"""GPU parity of the optimizer step (ll_muon_step, ll_adamw_step) against oracle.optim on seeded
inputs: Muon on wide, tall and square matrices (the Newton-Schulz GEMM chain on bf16 MFMA, the
tall ones transposed into the wide orientation), and AdamW on bf16 parameters with bf16 or fp32
gradients and on fp32 parameters, over three steps with a ragged element count.

Hyperparameters reach the kernels as fp32 values, so the oracle is called with the same fp32
values. Every stored bf16 value is checked against the oracle given the GPU's own inputs to that
step: within one bf16 ulp (plus 2^-20 of the magnitude of the terms summed, which matters only
where they cancel), with at most 5% of the elements one ulp apart. The kernels evaluate each
chain in fp32 and round that to bf16; the oracle rounds the exact value once, and the two roundings
differ in up to ~1.5% of the elements for inputs that are themselves bf16 values (measured; an
fp32 emulation on the host gives the same fraction). The Newton-Schulz output itself (lr 1, no
momentum, w = 0, so that w_new is the orthogonalised matrix exactly) is compared at 2e-2
norm-wise (measured 0.38% after 5 steps). A Muon update w_new - w on realistic weights is smaller
than the weights' bf16 resolution allows to compare norm-wise (one ulp of |w| ~ 0.02 is ~10% of
the update), so w_new is checked in ulps."""
import numpy as np
import pytest
import torch

import synth
import transformer_train_step_amd as ll
from oracle import numerics as nu
from oracle import optim as oo
from tests.gpu_util import assert_close, error_stats, need_gpu

pytestmark = pytest.mark.gpu

# The Newton-Schulz iterates are bf16 on both sides, rounded at the same points; they differ where
# the GPU's fp32 sums and the oracle's float64 sums round to different bf16 values, and the
# iteration's cancellation (a X + B X with a = 3.4 and a result near 0.7) amplifies those flips.
# An fp32-accumulation emulation of the same iteration on the host differs from the float64 one by
# 0.4% norm-wise after 5 steps; the bound leaves 5x room.
MUON_RTOL, MUON_ELEM, MUON_ROW = 2e-2, 0.1, 5e-2
FLIP_FRAC = 0.05          # stored bf16 values one ulp apart (fp32-then-bf16 vs exact-then-bf16)


def check_muon_w(got, ref, w0, name, elem=MUON_ELEM):
    """w_new = round(w - lr s X): each element within one bf16 ulp of the oracle's plus `elem` of
    (|update| + rms(update)) - the orthogonalised matrices X agree to 0.4% norm-wise and their
    elements to ~2% of (|X| + rms(X)) (test_newton_schulz_iterates_vs_oracle), and where w and the
    update cancel that is many ulps of the small result."""
    upd = np.abs(ref - w0)
    rms = np.sqrt(np.mean(upd * upd))
    slack = _ulp(ref) * 1.0001 + elem * (upd + rms)
    bad = np.abs(got - ref) > slack
    worst = float(np.max((np.abs(got - ref) - _ulp(ref)) / (upd + rms)))
    assert not bad.any(), f"{name}: {int(bad.sum())} elements beyond the bound (worst {worst:.3f} of |upd| + rms)"


def _bf(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()


def _h(t):
    return t.float().cpu().numpy().astype(np.float64)


def f32(x):
    """A hyperparameter as the C ABI receives it (an fp32 value)."""
    return float(np.float32(x))


def _ulp(x):
    _, e = np.frexp(np.maximum(np.abs(x), 2.0 ** -126))
    return np.ldexp(1.0, e - 8)


def _ulp_close(got, ref, name, frac=1e-3, scale=None):
    """bf16 values: equal except at most `frac` of the elements, which differ by at most one bf16
    ulp of the reference plus the fp32 rounding the kernel's arithmetic may add, 2^-20 of `scale`
    (the magnitude of the terms summed; it matters only where they cancel)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    diff = got != ref
    if diff.any():
        slack = _ulp(ref[diff]) * 1.0001
        if scale is not None:
            slack = slack + 2.0 ** -20 * np.broadcast_to(np.abs(scale), ref.shape)[diff]
        bad = np.abs(got[diff] - ref[diff]) > slack
        assert not bad.any(), (f"{name}: {int(bad.sum())} differences beyond one ulp; first got "
                               f"{got[diff][bad][0]}, ref {ref[diff][bad][0]}")
    assert diff.mean() <= frac, f"{name}: {diff.mean():.2e} of the elements differ"


@pytest.mark.parametrize("rows,cols,nesterov", [(256, 512, 1), (512, 256, 1), (384, 384, 0), (1024, 4096, 1),
                                                (4096, 1024, 1)])
def test_muon_step_vs_oracle(rows, cols, nesterov):
    need_gpu()
    seed = rows + cols
    w = synth.normal((rows, cols), 0.02, seed, 1, "bf16")
    g = synth.normal((rows, cols), 1e-3, seed, 2, "bf16")
    buf = synth.normal((rows, cols), 1e-3, seed, 3, "bf16")
    lr, mu = f32(0.02), f32(0.95)
    print(f"muon {rows}x{cols} nesterov={nesterov}", flush=True)
    W, G, B = _bf(w), _bf(g), _bf(buf)
    ws = torch.empty(ll._lib.ll_muon_workspace_bytes(rows, cols), dtype=torch.uint8, device="cuda")
    ll._lib.ll_muon_step(ll.LL_BF16, W, G, B, rows, cols, lr, mu, nesterov, 0.0, 5, ws, ws.numel())
    torch.cuda.synchronize()
    w_ref, buf_ref = oo.muon_update(w, g, buf, lr=lr, momentum=mu, nesterov=bool(nesterov), mode="bf16")
    _ulp_close(_h(B), buf_ref, "momentum buffer", frac=FLIP_FRAC, scale=np.abs(mu * buf) + np.abs(g))
    upd, upd_ref = _h(W) - w, w_ref - w
    print("update", error_stats(upd, upd_ref), flush=True)
    check_muon_w(_h(W), w_ref, w, "w")


@pytest.mark.parametrize("steps", [0, 1, 2, 5])
def test_newton_schulz_iterates_vs_oracle(steps):
    """The orthogonalised update after 0, 1, 2 and 5 Newton-Schulz steps (lr 1, no momentum), so
    that any growth of the difference over the iteration shows."""
    need_gpu()
    rows, cols = 512, 1536
    g = synth.normal((rows, cols), 1e-3, 71, 2, "bf16")
    W = torch.zeros((rows, cols), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros_like(W)
    ws = torch.empty(ll._lib.ll_muon_workspace_bytes(rows, cols), dtype=torch.uint8, device="cuda")
    ll._lib.ll_muon_step(ll.LL_BF16, W, _bf(g), B, rows, cols, 1.0, 0.0, 0, 0.0, steps, ws, ws.numel())
    torch.cuda.synchronize()
    ref = oo.newton_schulz(g, steps, mode="bf16")
    st = error_stats(-_h(W), ref)
    print(f"ns steps {steps}", st, flush=True)
    assert_close(-_h(W), ref, MUON_RTOL, f"X_{steps}", elem_rtol=MUON_ELEM, row_rtol=MUON_ROW)


def test_muon_weight_decay_and_zero_steps():
    """ns_steps = 0 applies the normalised momentum itself; weight decay scales w first."""
    need_gpu()
    rows, cols = 128, 192
    w = synth.normal((rows, cols), 0.02, 70, 1, "bf16")
    g = synth.normal((rows, cols), 1e-2, 70, 2, "bf16")
    W, G, B = _bf(w), _bf(g), torch.zeros((rows, cols), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ll._lib.ll_muon_workspace_bytes(rows, cols), dtype=torch.uint8, device="cuda")
    ll._lib.ll_muon_step(ll.LL_BF16, W, G, B, rows, cols, 0.1, 0.9, 1, 0.5, 0, ws, ws.numel())
    torch.cuda.synchronize()
    w_ref, _ = oo.muon_update(w, g, np.zeros_like(w), lr=f32(0.1), momentum=f32(0.9), nesterov=True,
                              weight_decay=f32(0.5), steps=0, mode="bf16")
    assert_close(_h(W), w_ref, 1e-2, "w", elem_rtol=0.05)


def test_muon_validation():
    need_gpu()
    t = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ll._lib.ll_muon_workspace_bytes(64, 64), dtype=torch.uint8, device="cuda")
    st = ll._lib.ll_muon_step(ll.LL_BF16, t, t, t, 64, 60, 0.02, 0.95, 1, 0.0, 5, ws, ws.numel(), raise_on_error=False)
    assert st == ll._lib.LL_ERR_UNSUPPORTED
    st = ll._lib.ll_muon_step(ll.LL_F32, t, t, t, 64, 64, 0.02, 0.95, 1, 0.0, 5, ws, ws.numel(), raise_on_error=False)
    assert st == ll._lib.LL_ERR_UNSUPPORTED
    st = ll._lib.ll_muon_step(ll.LL_BF16, t, t, t, 64, 64, 0.02, 0.95, 1, 0.0, 5, ws, 16, raise_on_error=False)
    assert st == ll._lib.LL_ERR_WORKSPACE


@pytest.mark.parametrize("group,pdt,gdt", [("embeddings", "bf16", "fp32"), ("lm_head", "bf16", "bf16"),
                                           ("value_embeds", "bf16", "fp32"), ("scalars", "fp32", "fp32")])
def test_adamw_step_vs_oracle(group, pdt, gdt):
    need_gpu()
    h = {k: (tuple(f32(b) for b in v) if isinstance(v, tuple) else f32(v)) for k, v in oo.ADAMW_GROUPS[group].items()}
    n = 1_000_003                                   # ragged: n % 4 == 3
    p0 = synth.normal((n,), 0.02, 80, 1, "bf16" if pdt == "bf16" else "fp32")
    print(f"adamw {group} param {pdt} grad {gdt}", flush=True)
    mk = lambda a, dt: (torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16) if dt == "bf16"
                        else torch.from_numpy(np.asarray(a, np.float32))).cuda()
    P = mk(p0, pdt)
    M = torch.zeros_like(P)
    V = torch.zeros_like(P)
    p, m, v = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    pd = ll.LL_BF16 if pdt == "bf16" else ll.LL_F32
    gd = ll.LL_BF16 if gdt == "bf16" else ll.LL_F32
    for step in (1, 2, 3):
        g = synth.normal((n,), 1e-3 * step, 80, 10 + step, "bf16" if gdt == "bf16" else "fp32")
        G = mk(g, gdt)
        ll._lib.ll_adamw_step(pd, gd, P, G, M, V, n, h["lr"], *h["betas"], h["eps"], h["weight_decay"], step)
        torch.cuda.synchronize()
        b1, b2 = h["betas"]
        m_scale = np.abs(b1 * m) + np.abs((1 - b1) * g)
        # the moments from the previous (GPU) state, the parameter from the GPU's new moments, so
        # that each stored value is checked on its own inputs
        _, m_ref, v_ref = oo.adamw_update(p, g, m, v, step, h["lr"], b1, b2, h["eps"], h["weight_decay"], mode=pdt)
        gm, gv, gp = _h(M), _h(V), _h(P)
        p_ref = oo.adamw_param_update(p, gm, gv, step, h["lr"], b1, b2, h["eps"], h["weight_decay"], mode=pdt)
        p_scale = np.abs(p) + np.abs(p_ref - p)
        if pdt == "bf16":
            _ulp_close(gm, m_ref, f"m step {step}", frac=FLIP_FRAC, scale=m_scale)
            _ulp_close(gv, v_ref, f"v step {step}", frac=FLIP_FRAC)
            _ulp_close(gp, p_ref, f"p step {step}", frac=FLIP_FRAC, scale=p_scale)
        else:
            # fp32 state: a few fp32 roundings, relative to the magnitudes of the terms summed
            for name, a, b, sc in (("p", gp, p_ref, p_scale), ("m", gm, m_ref, m_scale), ("v", gv, v_ref, np.abs(v_ref))):
                bad = np.abs(a - b) > 2.0 ** -20 * sc + 1e-30
                assert not bad.any(), (name, step, int(bad.sum()), a[bad][:3], b[bad][:3])
        p, m, v = gp, gm, gv
