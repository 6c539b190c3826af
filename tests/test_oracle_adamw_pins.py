"""Pins of the AdamW oracle against results fixed independently of it:
closed forms of the first step, of a constant gradient and of a zero gradient,
and torch.optim.AdamW run on the CPU in float64 as a black box.  Mutants of
the plausible mistakes (no bias correction, L2 decay folded into the gradient,
eps under the square root, decay on the new parameter) fail them."""


import numpy as np
import pytest

from oracle import AdamWHyper, adamw_step

HP = AdamWHyper(lr=3e-3, beta1=0.8, beta2=0.95, eps=1e-10, weight_decay=0.05)


def _rng_arrays(seed, n=257):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(n) * 0.02, rng.standard_normal(n) * 1e-3


def test_first_step_closed_form():
    """m = v = 0: m_hat = g and v_hat = g^2, so the step is lr g / (|g| + eps)."""
    p, g = _rng_arrays(1)
    r = adamw_step(p, g, np.zeros_like(g), np.zeros_like(g), HP, 1)
    expect = p * (1 - HP.lr * HP.weight_decay) - HP.lr * g / (np.abs(g) + HP.eps)
    np.testing.assert_allclose(r.p, expect, rtol=1e-13, atol=0)
    np.testing.assert_allclose(r.m, (1 - HP.beta1) * g, rtol=1e-15, atol=0)
    np.testing.assert_allclose(r.v, (1 - HP.beta2) * g * g, rtol=1e-15, atol=0)


def test_constant_gradient_every_step():
    """A constant gradient from zero moments: m_t = (1 - beta1^t) g and
    v_t = (1 - beta2^t) g^2, so every bias-corrected step is lr g / (|g| + eps)."""
    p, g = _rng_arrays(2, 64)
    m, v = np.zeros_like(g), np.zeros_like(g)
    hp = AdamWHyper(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    for t in range(1, 9):
        r = adamw_step(p, g, m, v, hp, t)
        np.testing.assert_allclose(r.m, (1 - 0.9 ** t) * g, rtol=1e-12, atol=0)
        np.testing.assert_allclose(r.v, (1 - 0.999 ** t) * g * g, rtol=1e-12, atol=0)
        np.testing.assert_allclose(r.p - p, -1e-2 * g / (np.abs(g) + 1e-8), rtol=1e-9, atol=0)
        p, m, v = r.p, r.m, r.v


def test_zero_gradient_only_decays():
    p, _ = _rng_arrays(3)
    z = np.zeros_like(p)
    q = p.copy()
    for t in range(1, 6):
        r = adamw_step(q, z, z, z, HP, t)
        q = r.p
    np.testing.assert_allclose(q, p * (1 - HP.lr * HP.weight_decay) ** 5, rtol=1e-14, atol=0)


def test_matches_torch_adamw_black_box():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    p0 = rng.standard_normal(300) * 0.02
    grads = [rng.standard_normal(300) * 10.0 ** rng.uniform(-4, -1) for _ in range(7)]
    tp = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
    opt = torch.optim.AdamW([tp], lr=HP.lr, betas=(HP.beta1, HP.beta2), eps=HP.eps,
                            weight_decay=HP.weight_decay, foreach=False, fused=False)
    p, m, v = p0.copy(), np.zeros(300), np.zeros(300)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        r = adamw_step(p, g, m, v, HP, t)
        p, m, v = r.p, r.m, r.v
        st = opt.state[tp]
        np.testing.assert_allclose(st["exp_avg"].numpy(), m, rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(st["exp_avg_sq"].numpy(), v, rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(tp.detach().numpy(), p, rtol=1e-12, atol=1e-18)


def test_step_zero_rejected():
    p, g = _rng_arrays(5, 4)
    with pytest.raises(ValueError):
        adamw_step(p, g, g, g * g, HP, 0)


def _mutants():
    def no_bias_correction(p, g, m, v, hp, t):
        m2 = hp.beta1 * m + (1 - hp.beta1) * g
        v2 = hp.beta2 * v + (1 - hp.beta2) * g * g
        return p * (1 - hp.lr * hp.weight_decay) - hp.lr * m2 / (np.sqrt(v2) + hp.eps)

    def l2_in_gradient(p, g, m, v, hp, t):
        g = g + hp.weight_decay * p
        m2 = hp.beta1 * m + (1 - hp.beta1) * g
        v2 = hp.beta2 * v + (1 - hp.beta2) * g * g
        return p - hp.lr * (m2 / (1 - hp.beta1 ** t)) / (np.sqrt(v2 / (1 - hp.beta2 ** t)) + hp.eps)

    def eps_under_sqrt(p, g, m, v, hp, t):
        m2 = hp.beta1 * m + (1 - hp.beta1) * g
        v2 = hp.beta2 * v + (1 - hp.beta2) * g * g
        return p * (1 - hp.lr * hp.weight_decay) - hp.lr * (m2 / (1 - hp.beta1 ** t)) / np.sqrt(
            v2 / (1 - hp.beta2 ** t) + hp.eps)

    def decay_after_update(p, g, m, v, hp, t):
        m2 = hp.beta1 * m + (1 - hp.beta1) * g
        v2 = hp.beta2 * v + (1 - hp.beta2) * g * g
        q = p - hp.lr * (m2 / (1 - hp.beta1 ** t)) / (np.sqrt(v2 / (1 - hp.beta2 ** t)) + hp.eps)
        return q * (1 - hp.lr * hp.weight_decay)

    return [no_bias_correction, l2_in_gradient, eps_under_sqrt, decay_after_update]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_mutants_fail_the_pins(mutant):
    """Each plausible mistake disagrees with the closed forms or with torch's AdamW."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(6)
    p0 = rng.standard_normal(100) * 0.5
    grads = [rng.standard_normal(100) * 1e-3 for _ in range(3)]
    tp = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
    hp = AdamWHyper(lr=0.1, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.5)
    opt = torch.optim.AdamW([tp], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps, weight_decay=hp.weight_decay)
    p, m, v = p0.copy(), np.zeros(100), np.zeros(100)
    worst = 0.0
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        pm = mutant(p, g, m, v, hp, t)
        worst = max(worst, float(np.max(np.abs(pm - tp.detach().numpy()))))
        r = adamw_step(p, g, m, v, hp, t)
        p, m, v = r.p, r.m, r.v
    assert worst > 1e-6
