"""Pins of oracle.optim (Muon and AdamW) against things other than itself: the singular-value form
of the Newton-Schulz iteration through numpy's SVD, closed forms of the momentum recursion, and
torch.optim.AdamW (float64) as an independent implementation of AdamW. Planted mistakes (swapped
coefficients, a missing normalisation, the momentum without its look-ahead) fail the pins."""
import numpy as np
import pytest
import torch

from oracle import optim as oo


def _svd_form(u, steps, coeffs=oo.NS_COEFFS, eps=oo.NS_EPS):
    """U diag(p^(steps)(s / (||u|| + eps))) V^T with p(x) = a x + b x^3 + c x^5."""
    a, b, c = coeffs
    U, s, Vt = np.linalg.svd(np.asarray(u, np.float64), full_matrices=False)
    x = s / (np.linalg.norm(u) + eps)
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return (U * x) @ Vt


@pytest.mark.parametrize("shape", [(24, 40), (40, 24), (32, 32), (7, 64)])
@pytest.mark.parametrize("steps", [1, 5])
def test_newton_schulz_acts_on_singular_values(shape, steps):
    rng = np.random.default_rng(sum(shape) + steps)
    u = rng.standard_normal(shape) * 0.3
    got = oo.newton_schulz(u, steps, mode="fp32")
    want = _svd_form(u, steps)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_newton_schulz_planted_mistakes_fail_the_pin(monkeypatch):
    rng = np.random.default_rng(5)
    u = rng.standard_normal((24, 40))
    want = _svd_form(u, 5)
    a, b, c = oo.NS_COEFFS
    for coeffs in ((a, c, b), (b, a, c)):
        bad = oo.newton_schulz(u, 5, mode="fp32", coeffs=coeffs)
        assert np.abs(bad - want).max() > 1e-2
    # without the Frobenius normalisation (eps so large that X_0 is u / eps)
    bad = oo.newton_schulz(u, 5, mode="fp32", eps=1e3)
    assert np.abs(bad - want).max() > 1e-2


def test_newton_schulz_orthonormal_rows_closed_form():
    """A matrix q with orthonormal rows (all singular values 1, Frobenius norm sqrt(rows)) maps to
    p^(5)(1 / (sqrt(rows) + eps)) q."""
    rng = np.random.default_rng(6)
    _, _, Vt = np.linalg.svd(rng.standard_normal((32, 64)), full_matrices=False)
    q = Vt[:16]
    x = 1.0 / (4.0 + oo.NS_EPS)
    a, b, c = oo.NS_COEFFS
    for _ in range(5):
        x = a * x + b * x ** 3 + c * x ** 5
    np.testing.assert_allclose(oo.newton_schulz(q, 5), x * q, atol=1e-12)
    np.testing.assert_allclose(oo.newton_schulz(q.T, 5), x * q.T, atol=1e-12)


def test_muon_momentum_closed_form_and_scale():
    """With a constant gradient g: buf_t = g (1 - mu^t) / (1 - mu); the Nesterov input is
    u = g + mu buf_t, and the update is lr sqrt(max(1, rows/cols)) NS(u) in its singular-value form."""
    rng = np.random.default_rng(7)
    mu, lr = 0.95, 0.02
    for shape in ((16, 48), (48, 16)):
        g = rng.standard_normal(shape)
        w = rng.standard_normal(shape)
        buf = np.zeros(shape)
        for t in range(1, 4):
            w_new, buf = oo.muon_update(w, g, buf, lr=lr, momentum=mu, nesterov=True)
            np.testing.assert_allclose(buf, g * (1 - mu ** t) / (1 - mu), rtol=1e-13)
            scale = np.sqrt(max(1.0, shape[0] / shape[1]))
            u = g * (1 + mu * (1 - mu ** t) / (1 - mu))
            np.testing.assert_allclose(w - w_new, lr * scale * _svd_form(u, 5), atol=1e-14)
            w = w_new
    # without the look-ahead the buffer itself is orthogonalised: same direction here, but a
    # different result as soon as the gradient changes
    g2 = rng.standard_normal((16, 48))
    b0 = rng.standard_normal((16, 48))
    w0 = np.zeros((16, 48))
    wn, _ = oo.muon_update(w0, g2, b0, nesterov=True)
    wp, _ = oo.muon_update(w0, g2, b0, nesterov=False)
    np.testing.assert_allclose(-wn / 0.02, _svd_form(g2 + 0.95 * (0.95 * b0 + g2), 5), atol=1e-12)
    np.testing.assert_allclose(-wp / 0.02, _svd_form(0.95 * b0 + g2, 5), atol=1e-12)


@pytest.mark.parametrize("group", sorted(oo.ADAMW_GROUPS))
def test_adamw_matches_torch_adamw(group):
    h = oo.ADAMW_GROUPS[group]
    rng = np.random.default_rng(8)
    p0 = rng.standard_normal(300) * 0.02
    grads = [rng.standard_normal(300) * s for s in (1e-2, 3e-3, 2e-2)]
    t = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([t], lr=h["lr"], betas=h["betas"], eps=h["eps"], weight_decay=h["weight_decay"])
    p, m, v = p0.copy(), np.zeros(300), np.zeros(300)
    for step, g in enumerate(grads, start=1):
        t.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = oo.adamw_update(p, g, m, v, step, h["lr"], *h["betas"], h["eps"], h["weight_decay"])
        np.testing.assert_allclose(p, t.detach().numpy(), rtol=1e-12, atol=1e-15)
        st = opt.state[t]
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-12)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12)


def test_adamw_bf16_mode_rounds_only_stored_tensors():
    rng = np.random.default_rng(9)
    from oracle import numerics as nu
    p = nu.bf16_round(rng.standard_normal(64))
    g = rng.standard_normal(64)
    pb, mb, vb = oo.adamw_update(p, g, 0, 0, 1, 0.1, 0.8, 0.995, 1e-10, 0.001, mode="bf16")
    pf, mf, vf = oo.adamw_update(p, g, 0, 0, 1, 0.1, 0.8, 0.995, 1e-10, 0.001, mode="fp32")
    for a in (pb, mb, vb):
        np.testing.assert_array_equal(a, nu.bf16_round(a))
    np.testing.assert_array_equal(mb, nu.bf16_round(mf))
    np.testing.assert_array_equal(vb, nu.bf16_round(vf))
    pm, mm, vm = oo.adamw_update(p, g, 0, 0, 1, 0.1, 0.8, 0.995, 1e-10, 0.001, mode="bf16", state_mode="fp32")
    np.testing.assert_array_equal(mm, mf)
