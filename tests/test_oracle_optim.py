"""Pins for the fp64 optimiser oracle (oracle/optim.py): each check compares
it with something other than itself -- a library implementation of the same
published method, a closed form, or the singular-value form of the
Newton-Schulz iteration -- so that a dropped term, a wrong coefficient, sign
or exponent, or a transposed product fails at least one of them."""
import math

import numpy as np
import pytest
import torch

from oracle import optim
import synthdata
from synthdata import Config

TINY = Config("optim-micro", 2, 16, 2, 8, 64, 32, 2, 8, "f32", 21)


def _rng(seed=0):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# AdamW
# --------------------------------------------------------------------------
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_adamw_matches_torch(wd):
    """Three steps against torch.optim.AdamW (fp64 on the CPU), the same
    decoupled-decay, bias-corrected definition."""
    rng = _rng(3)
    p0 = rng.standard_normal((5, 7))
    grads = [rng.standard_normal((5, 7)) * s for s in (1.0, 0.1, 3.0)]
    lr, b1, b2, eps = 0.05, 0.8, 0.95, 1e-8
    tp = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for step, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = optim.adamw_update(p, g, m, v, step, lr, b1, b2, eps, wd)
    np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-12, atol=1e-14)
    st = opt.state[tp]
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-12)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12)


def test_adamw_first_step_closed_form():
    """From zero moments the bias-corrected step is lr g / (|g| + eps) after
    the decay p (1 - lr wd)."""
    rng = _rng(4)
    p0, g = rng.standard_normal(50), rng.standard_normal(50)
    lr, wd, eps = 0.01, 0.3, 1e-10
    p, m, v = optim.adamw_update(p0, g, np.zeros(50), np.zeros(50), 1, lr, 0.9, 0.99, eps, wd)
    np.testing.assert_allclose(p, p0 * (1 - lr * wd) - lr * g / (np.abs(g) + eps), rtol=1e-13)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-13)
    np.testing.assert_allclose(v, 0.01 * g * g, rtol=1e-13)


# --------------------------------------------------------------------------
# Newton-Schulz
# --------------------------------------------------------------------------
def _ns_by_svd(G, steps, coeffs, eps):
    """The iteration acts on each singular value alone:
    s <- a s + b s^3 + c s^5 from s = sigma / (||G||_F + eps)."""
    a, b, c = coeffs
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    s = S / (math.sqrt(np.sum(S * S)) + eps)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return (U * s) @ Vt


@pytest.mark.parametrize("shape", [(24, 40), (40, 24), (32, 32)])
def test_newton_schulz_matches_singular_value_form(shape):
    G = _rng(5).standard_normal(shape) * 2.5
    np.testing.assert_allclose(optim.newton_schulz(G), _ns_by_svd(G, 5, optim.NS_COEFFS, optim.NS_EPS),
                               rtol=1e-9, atol=1e-12)


def test_newton_schulz_other_coefficients_and_steps():
    """Same singular-value form for other (a, b, c) and step counts, so the
    coefficients are applied to the right powers."""
    G = _rng(6).standard_normal((12, 20))
    for coeffs, steps in (((2.0, -1.5, 0.5), 3), ((1.5, -0.5, 0.0), 7)):
        np.testing.assert_allclose(optim.newton_schulz(G, steps, coeffs), _ns_by_svd(G, steps, coeffs, optim.NS_EPS),
                                   rtol=1e-9, atol=1e-12)


def test_newton_schulz_output_spectrum():
    """For a well-conditioned input the published coefficients leave every
    singular value near 1 (between about 0.7 and 1.2)."""
    G = _rng(7).standard_normal((64, 256))
    s = np.linalg.svd(optim.newton_schulz(G), compute_uv=False)
    assert s.min() > 0.6 and s.max() < 1.25


def test_newton_schulz_transpose_and_scale():
    G = _rng(8).standard_normal((16, 48))
    X = optim.newton_schulz(G)
    np.testing.assert_allclose(optim.newton_schulz(G.T), X.T, rtol=1e-12, atol=1e-14)
    # only eps breaks scale invariance: a 1e-7 / ||G||_F relative change of
    # the normalised input, amplified up to a^5 ~ 500 by the iteration
    np.testing.assert_allclose(optim.newton_schulz(G * 1e3), X, rtol=1e-5, atol=1e-8)


# --------------------------------------------------------------------------
# Muon
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(8, 24), (24, 8)])
def test_muon_first_step(shape):
    """From a zero buffer the Nesterov direction is (1 + mu) G, which the
    normalisation removes: W1 = W0 - lr sqrt(max(1, r/c)) NS(G); the buffer
    becomes G."""
    rng = _rng(9)
    W0, G = rng.standard_normal(shape), rng.standard_normal(shape)
    lr = 0.02
    W1, buf = optim.muon_update(W0, G, np.zeros(shape), lr, 0.9)
    scale = math.sqrt(max(1.0, shape[0] / shape[1]))
    np.testing.assert_allclose(W1, W0 - lr * scale * _ns_by_svd(G, 5, optim.NS_COEFFS, optim.NS_EPS),
                               rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(buf, G, rtol=0, atol=0)


def test_muon_second_step_direction():
    """Step 2: buf = mu G1 + G2 and the Nesterov direction is
    G2 + mu buf = (1 + mu) G2 + mu^2 G1; without Nesterov it is buf."""
    rng = _rng(10)
    W0, G1, G2 = (rng.standard_normal((10, 14)) for _ in range(3))
    mu, lr = 0.85, 0.03
    for nesterov, direction in ((True, (1 + mu) * G2 + mu * mu * G1), (False, mu * G1 + G2)):
        W1, b1 = optim.muon_update(W0, G1, np.zeros_like(W0), lr, mu, nesterov)
        W2, b2 = optim.muon_update(W1, G2, b1, lr, mu, nesterov)
        np.testing.assert_allclose(b2, mu * G1 + G2, rtol=1e-14)
        np.testing.assert_allclose(W2, W1 - lr * _ns_by_svd(direction, 5, optim.NS_COEFFS, optim.NS_EPS),
                                   rtol=1e-6, atol=1e-9)


# --------------------------------------------------------------------------
# schedule
# --------------------------------------------------------------------------
def test_lr_multiplier_and_momentum_ramp():
    n = 1000
    assert optim.lr_multiplier(0, n) == 1.0
    assert optim.lr_multiplier(799, n) == 1.0
    assert optim.lr_multiplier(800, n) == pytest.approx(1.0)
    assert optim.lr_multiplier(900, n) == pytest.approx(0.5)
    assert optim.lr_multiplier(1000, n) == pytest.approx(0.0, abs=1e-15)
    assert optim.lr_multiplier(950, n, final_frac=0.1) == pytest.approx(0.1 + 0.9 * 0.25)
    assert optim.muon_momentum(0) == pytest.approx(0.85)
    assert optim.muon_momentum(150) == pytest.approx(0.90)
    assert optim.muon_momentum(300) == pytest.approx(0.95)
    assert optim.muon_momentum(5000) == pytest.approx(0.95)


def test_default_hparams_width_scale():
    """AdamW rates scale as 1/sqrt(width): a 4x wider model halves them;
    the matrix rate does not depend on width."""
    h1, h4 = optim.default_hparams(768, 0, 100), optim.default_hparams(3072, 0, 100)
    assert h1["lr_embed"] == pytest.approx(0.2) and h4["lr_embed"] == pytest.approx(0.1)
    assert h1["lr_unembed"] == pytest.approx(0.004) and h4["lr_unembed"] == pytest.approx(0.002)
    assert h1["lr_matrix"] == h4["lr_matrix"] == pytest.approx(0.02)
    hend = optim.default_hparams(768, 95, 100, n_micro=8)
    assert hend["lr_matrix"] == pytest.approx(0.02 * 0.25) and hend["grad_scale"] == 0.125


# --------------------------------------------------------------------------
# the whole step
# --------------------------------------------------------------------------
def _setup(seed=11):
    layout = synthdata.param_layout(TINY)
    n = synthdata.param_count(TINY)
    rng = _rng(seed)
    return layout, rng.standard_normal(n) * 0.1, rng.standard_normal(n)


def test_optimizer_step_routes_each_tensor():
    """E and U move by AdamW with their own rates, every block matrix (q, k
    and v each on its own) by Muon; a zero rate leaves a group unchanged."""
    layout, master, grads = _setup()
    hp = optim.default_hparams(TINY.d_model, 0, 10)
    out, _ = optim.optimizer_step(layout, master, grads, optim.new_state(layout), hp)
    for name, layer, r, c, off in layout:
        p0 = master[off:off + r * c].reshape(r, c)
        g = grads[off:off + r * c].reshape(r, c)
        got = out[off:off + r * c].reshape(r, c)
        if name in ("E", "U"):
            lr = hp["lr_embed"] if name == "E" else hp["lr_unembed"]
            want = p0 - lr * g / (np.abs(g) + hp["eps"])          # first AdamW step, wd = 0
            np.testing.assert_allclose(got, want, rtol=1e-12)
        else:
            scale = math.sqrt(max(1.0, r / c))
            want = p0 - hp["lr_matrix"] * scale * _ns_by_svd(g, 5, optim.NS_COEFFS, optim.NS_EPS)
            np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-9)
    # one Muon step over the stacked [3d, d] block would be a different update
    for name, layer, r, c, off in layout:
        if name == "Wq" and layer == 0:
            qkv = slice(off, off + 3 * r * c)
            fused = master[qkv].reshape(3 * r, c) - hp["lr_matrix"] * math.sqrt(3.0) * _ns_by_svd(
                grads[qkv].reshape(3 * r, c), 5, optim.NS_COEFFS, optim.NS_EPS)
            assert np.abs(out[qkv] - fused.ravel()).max() > 1e-3


def test_optimizer_step_grad_scale_is_a_mean():
    """Accumulated gradients g1 + g2 with grad_scale 1/2 step exactly as
    their mean with grad_scale 1.  Taken as the second step (after one
    with g0), where the moments and the momentum buffer mix the two
    gradients and the step is no longer invariant to their scale."""
    layout, master, g0 = _setup(12)
    g1, g2 = _rng(13).standard_normal(g0.shape), _rng(14).standard_normal(g0.shape)
    h0 = optim.default_hparams(TINY.d_model, 0, 10)
    m1, st1 = optim.optimizer_step(layout, master, g0, optim.new_state(layout), h0)
    h = optim.default_hparams(TINY.d_model, 1, 10, n_micro=2)
    a, _ = optim.optimizer_step(layout, m1, g1 + g2, st1, h)
    b, _ = optim.optimizer_step(layout, m1, (g1 + g2) / 2, st1, dict(h, grad_scale=1.0))
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)
    c, _ = optim.optimizer_step(layout, m1, g1 + g2, st1, dict(h, grad_scale=1.0))
    assert np.abs(c - a).max() > 1e-6
