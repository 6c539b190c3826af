"""Pins for the CPU oracle: each check is fixed by something other than the
oracle's own code (the SVD closed form, a geometric series, constants printed on
the pages, brute force on tiny inputs, an outside library run as a black box).

Closed form used throughout.  With X0 = G / (||G||_F + eps) = U S V^T, one
iteration maps X to U p(S) V^T with p(s) = a s + b s^3 + c s^5, because
X X^T = U S^2 U^T.  After k iterations the result is U phi_k(S) V^T with
phi_k = p o ... o p, a scalar function evaluated here by a plain loop.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import Hyper, muon_step_matrix, newton_schulz
from muon_synth import heavy_tail_grad, lowrank_noise_grad, rng_for

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ns_constants.json")

A, B, C = 3.4445, -4.7750, 2.0315


def phi(s, steps=5, a=A, b=B, c=C):
    """Scalar quintic applied ``steps`` times, element by element, by a Python loop."""
    s = np.atleast_1d(np.asarray(s, dtype=np.float64))
    out = np.empty_like(s)
    for i, v in enumerate(s):
        x = float(v)
        for _ in range(steps):
            x = a * x + b * x ** 3 + c * x ** 5
        out[i] = x
    return out


def svd_closed_form(g, steps=5, eps=1e-7):
    """U phi(S / (||G||_F + eps)) V^T from LAPACK's SVD (thin)."""
    u, s, vt = np.linalg.svd(g, full_matrices=False)
    nu = math.sqrt(float(np.sum(g * g)))
    return (u * phi(s / (nu + eps), steps)) @ vt


def relf(x, y):
    return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300))


def _inputs(kind, r, c, seed):
    rng = rng_for(99, seed, r * 7919 + c, 1)
    if kind == "gauss":
        return rng.standard_normal((r, c)) * 0.02
    if kind == "lowrank":
        return lowrank_noise_grad(rng, r, c)
    return heavy_tail_grad(rng, r, c)


# --------------------------------------------------------------------------
# constants printed on the pages
# --------------------------------------------------------------------------

def test_constants_match_pages():
    gold = json.load(open(GOLDEN))
    co = gold["ns_coefficients"]
    assert (oracle.NS_A, oracle.NS_B, oracle.NS_C) == (co["a"], co["b"], co["c"])
    assert oracle.NS_STEPS == gold["ns_steps"]["value"]
    assert oracle.NS_EPS == gold["eps"]["value"]
    assert oracle.BETA == gold["beta"]["value"]
    h = Hyper()
    assert (h.a, h.b, h.c, h.ns_steps, h.eps, h.beta) == (co["a"], co["b"], co["c"], 5, 1e-7, 0.95)


def test_repeated_application_band_matches_pages():
    """The pages print the band the quintic settles in under repeated application
    as 0.68..1.13; iterate the oracle far past 5 steps on a full-spectrum matrix."""
    gold = json.load(open(GOLDEN))["band_repeated"]
    g = _inputs("heavy", 48, 96, 0)
    x0, _ = oracle.frobenius_normalize(g, 1e-7)
    x = oracle.ns_iterate(x0, 40, A, B, C)
    s = np.linalg.svd(x, compute_uv=False)
    # printed to two decimals: allow half a unit of the last printed digit
    assert s.min() >= gold["lo"] - 0.005
    assert s.max() <= gold["hi"] + 0.005
    # and the iterate does not converge to 1: its spread stays of the printed width
    assert s.max() - s.min() > 0.3


def test_flop_overhead_matches_pages():
    gold = json.load(open(GOLDEN))["flop_overhead"]
    frac = oracle.muon_overhead_fraction(gold["hidden"], gold["tokens_per_batch"], gold["ns_steps"])
    assert frac == pytest.approx(5 * 768 / 524288, rel=1e-15)       # T*m/B
    assert round(frac, 3) == gold["approx_fraction"]                  # "~0.7%"
    # Llama-70B-like exercise on the same page: m = 8192, B = 4M tokens
    assert oracle.muon_overhead_fraction(8192, 4_000_000) == pytest.approx(5 * 8192 / 4e6)
    # dense vs distinct-entry counting on a small shape, by brute enumeration
    m, n = 5, 9
    dense = 5 * (2 * m * m * n + 2 * m * m * m + 2 * m * m * n)
    uniq = 5 * (sum(1 for i in range(m) for j in range(m) if i <= j) * 2 * n
                + sum(1 for i in range(m) for j in range(m) if i <= j) * 2 * m + 2 * m * m * n)
    assert oracle.ns_flops_dense(m, n) == dense == oracle.ns_flops_dense(n, m)
    assert oracle.ns_flops_unique(m, n) == uniq


# --------------------------------------------------------------------------
# momentum: geometric series in closed form
# --------------------------------------------------------------------------

def test_momentum_constant_gradient_closed_form():
    g = np.full((3, 4), 0.5)
    m = np.zeros_like(g)
    for _ in range(10):
        m = oracle.momentum_update(m, g, 0.95)
    factor = (1 - 0.95 ** 10) / (1 - 0.95)
    assert factor == pytest.approx(8.025261215232426, rel=1e-15)
    np.testing.assert_allclose(m, factor * g, rtol=1e-14)
    u = oracle.update_direction(g, m, 0.95, True)
    np.testing.assert_allclose(u, 8.623998154470804 * g, rtol=1e-14)
    np.testing.assert_array_equal(oracle.update_direction(g, m, 0.95, False), m)


def test_momentum_random_sequence_is_discounted_sum():
    rng = np.random.default_rng(5)
    gs = [rng.standard_normal((6, 5)) for _ in range(12)]
    m0 = rng.standard_normal((6, 5))
    m = m0.copy()
    for g in gs:
        m = oracle.momentum_update(m, g, 0.9)
    T = len(gs)
    closed = 0.9 ** T * m0 + sum(0.9 ** (T - 1 - t) * gs[t] for t in range(T))
    np.testing.assert_allclose(m, closed, rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# Newton-Schulz against the SVD closed form
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["gauss", "lowrank", "heavy"])
@pytest.mark.parametrize("shape", [(64, 128), (128, 64), (37, 91), (91, 37), (200, 200), (1, 7), (7, 1), (300, 40)])
def test_ns_matches_svd_closed_form(kind, shape):
    g = _inputs(kind, *shape, seed=1)
    o = newton_schulz(g)
    ref = svd_closed_form(g)
    assert o.shape == g.shape
    assert relf(o, ref) <= 1e-12


@pytest.mark.parametrize("steps", [0, 1, 2, 3, 7])
def test_ns_step_count(steps):
    g = _inputs("gauss", 20, 33, 2)
    assert relf(newton_schulz(g, steps=steps), svd_closed_form(g, steps=steps)) <= 1e-12


def test_ns_five_step_band():
    """After exactly 5 steps every direction with s/nu >= 1.5e-3 lands in
    [0.6798, 1.2024]: the quintic's range over that interval (its local maximum
    p(0.5545) = 1.20237 is reached within 5 steps)."""
    xs = np.logspace(np.log10(1.5e-3), 0, 4001)
    v = phi(xs)
    lo, hi = float(v.min()), float(v.max())
    assert 0.6795 < lo < 0.6800 and 1.2020 < hi < 1.2025
    for kind, shape in (("heavy", (96, 256)), ("lowrank", (128, 300)), ("gauss", (64, 128))):
        g = _inputs(kind, *shape, seed=3)
        o = newton_schulz(g)
        s_in = np.linalg.svd(g, compute_uv=False) / np.linalg.norm(g)
        s_out = np.linalg.svd(o, compute_uv=False)
        # singular values of O are phi(s_in); those in range are equalised
        np.testing.assert_allclose(np.sort(s_out), np.sort(phi(s_in / (1 + 1e-7 / np.linalg.norm(g)))), rtol=1e-9, atol=1e-12)
        keep = s_in >= 1.5e-3
        assert np.all(phi(s_in[keep]) >= lo - 1e-12) and np.all(phi(s_in[keep]) <= hi + 1e-12)
        vals = phi(s_in[keep])
        assert vals.max() / vals.min() <= 1.77


@pytest.mark.parametrize("m,n,expected", [(64, 128, 0.6881398558), (96, 96, None), (32, 512, None)])
def test_orthonormal_rows_scaled_by_phi(m, n, expected):
    rng = np.random.default_rng(m + n)
    q, _ = np.linalg.qr(rng.standard_normal((n, m)))
    q = q.T                                     # m x n, orthonormal rows
    o = newton_schulz(q)
    f = phi(1.0 / (math.sqrt(m) + 1e-7))[0]     # ||Q||_F = sqrt(m)
    np.testing.assert_allclose(o, f * q, rtol=1e-11, atol=1e-13)
    if expected is not None:
        assert phi(1.0 / math.sqrt(m))[0] == pytest.approx(expected, abs=1e-9)


def test_rank_one():
    rng = np.random.default_rng(11)
    u = rng.standard_normal(40)
    u /= np.linalg.norm(u)
    v = rng.standard_normal(70)
    v /= np.linalg.norm(v)
    g = 3.7 * np.outer(u, v)
    o = newton_schulz(g)
    f = phi(3.7 / (3.7 + 1e-7))[0]
    assert phi(1.0)[0] == pytest.approx(0.6964364095, abs=1e-9)
    assert f == pytest.approx(0.6964364095, abs=1e-7)
    np.testing.assert_allclose(o, f * np.outer(u, v), rtol=1e-11, atol=1e-14)


def test_transpose_symmetry_and_push_through():
    g = _inputs("lowrank", 150, 60, 4)
    o = newton_schulz(g)
    assert relf(newton_schulz(g.T), o.T) <= 1e-12
    # iterating on the tall side (the n x n Gram) gives the same matrix:
    # p(X X^T) X = X p(X^T X)
    x0, _ = oracle.frobenius_normalize(g, 1e-7)
    assert relf(oracle.ns_iterate(x0, 5, A, B, C), o) <= 1e-11


def test_scale_invariance():
    g = _inputs("gauss", 40, 70, 5)
    o = newton_schulz(g)
    nu = np.linalg.norm(g)
    for alpha in (1e-3, 7.5, 1e4):
        # the only difference is eps's share of each norm: eps/(alpha nu) vs eps/nu
        assert relf(newton_schulz(alpha * g), o) <= 50 * 1e-7 * (1 / (alpha * nu) + 1 / nu) + 1e-12


def test_zero_input_and_zero_lr():
    z = np.zeros((8, 5))
    np.testing.assert_array_equal(newton_schulz(z), z)
    w = np.random.default_rng(1).standard_normal((8, 5))
    r = muon_step_matrix(w, z, z, Hyper(lr=0.02, weight_decay=0.1))
    np.testing.assert_array_equal(r.o, z)
    np.testing.assert_allclose(r.w, w * (1 - 0.02 * 0.1), rtol=0, atol=0)
    g = np.random.default_rng(2).standard_normal((8, 5))
    r0 = muon_step_matrix(w, g, z, Hyper(lr=0.0, weight_decay=0.1))
    np.testing.assert_array_equal(r0.w, w)


def test_one_by_one_brute_force():
    for gval in (0.3, -2.0, 1e-9):
        o = newton_schulz(np.array([[gval]]))
        assert o[0, 0] == pytest.approx(math.copysign(phi(abs(gval) / (abs(gval) + 1e-7))[0], gval), rel=1e-13)


def _matmul_loops(x, y):
    n, k = len(x), len(x[0])
    m = len(y[0])
    return [[sum(x[i][t] * y[t][j] for t in range(k)) for j in range(m)] for i in range(n)]


def test_tiny_brute_force_loops():
    """2x3 and 3x2 by explicit Python loops over the pages' per-iteration steps."""
    rng = np.random.default_rng(8)
    for shape in ((2, 3), (3, 2), (2, 2)):
        g = rng.standard_normal(shape)
        nu = math.sqrt(sum(v * v for v in g.ravel()))
        x = [[g[i][j] / (nu + 1e-7) for j in range(shape[1])] for i in range(shape[0])]
        tall = shape[0] > shape[1]
        if tall:
            x = [list(r) for r in zip(*x)]
        for _ in range(5):
            xt = [list(r) for r in zip(*x)]
            a_ = _matmul_loops(x, xt)
            aa = _matmul_loops(a_, a_)
            b_ = [[B * a_[i][j] + C * aa[i][j] for j in range(len(a_))] for i in range(len(a_))]
            bx = _matmul_loops(b_, x)
            x = [[A * x[i][j] + bx[i][j] for j in range(len(x[0]))] for i in range(len(x))]
        if tall:
            x = [list(r) for r in zip(*x)]
        np.testing.assert_allclose(newton_schulz(g), np.array(x), rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# the whole step: momentum series + SVD closed form + update formula
# --------------------------------------------------------------------------

@pytest.mark.parametrize("nesterov", [False, True])
@pytest.mark.parametrize("shape", [(48, 80), (120, 50)])
def test_full_step_closed_form(nesterov, shape):
    rng = np.random.default_rng(21)
    beta, lr, wd = 0.95, 0.02, 0.01
    w = rng.standard_normal(shape) * 0.02
    m0 = rng.standard_normal(shape) * 0.02
    gs = [rng.standard_normal(shape) * 0.02 for _ in range(4)]
    hp = Hyper(lr=lr, beta=beta, weight_decay=wd, nesterov=nesterov)
    m, wcur = m0, w
    for t, g in enumerate(gs):
        r = muon_step_matrix(wcur, g, m, hp)
        T = t + 1
        m_closed = beta ** T * m0 + sum(beta ** (T - 1 - i) * gs[i] for i in range(T))
        u_closed = g + beta * m_closed if nesterov else m_closed
        o_closed = svd_closed_form(u_closed)
        s = math.sqrt(max(1.0, shape[0] / shape[1]))
        w_closed = wcur * (1 - lr * wd) - lr * s * o_closed
        assert relf(r.m, m_closed) <= 1e-13
        assert relf(r.o, o_closed) <= 1e-11
        assert relf(r.w - wcur, w_closed - wcur) <= 1e-11
        m, wcur = r.m, r.w


def test_against_torch_optim_muon_black_box():
    """torch.optim.Muon run as a black box (its bf16 iteration limits agreement to
    ~1.5e-2): same momentum form, Nesterov form, decoupled decay and shape scale."""
    torch = pytest.importorskip("torch")
    if not hasattr(torch.optim, "Muon"):
        pytest.skip("torch.optim.Muon not present")
    rng = np.random.default_rng(0)
    for shape in ((64, 128), (128, 64)):
        w = rng.standard_normal(shape) * 0.02
        p = torch.nn.Parameter(torch.tensor(w, dtype=torch.float32))
        opt = torch.optim.Muon([p], lr=0.02, weight_decay=0.01, momentum=0.95, nesterov=True,
                               adjust_lr_fn="original")
        m = np.zeros(shape)
        for _ in range(3):
            g = (rng.standard_normal(shape) * 0.02).astype(np.float32).astype(np.float64)
            p.grad = torch.tensor(g, dtype=torch.float32)
            w0 = p.detach().double().numpy().copy()
            opt.step()
            r = muon_step_matrix(w0, g, m, Hyper(lr=0.02, weight_decay=0.01, nesterov=True))
            m = r.m
            assert relf(p.detach().double().numpy() - w0, r.w - w0) <= 3e-2


# --------------------------------------------------------------------------
# the pins have teeth: plant plausible mistakes in a copy of the iteration
# --------------------------------------------------------------------------

def _mutant_iterations():
    def dropped_c(x, s, a, b, c, coeffs=None):
        for _ in range(s):
            g = x @ x.T
            x = a * x + (b * g) @ x
        return x

    def wrong_sign_b(x, s, a, b, c, coeffs=None):
        for _ in range(s):
            g = x @ x.T
            x = a * x + (-b * g + c * g @ g) @ x
        return x

    def right_multiply(x, s, a, b, c, coeffs=None):
        for _ in range(s):
            g = x @ x.T
            x = a * x + x @ (b * g + c * g @ g)
        return x

    def gram_transposed(x, s, a, b, c, coeffs=None):
        for _ in range(s):
            g = x.T @ x
            x = a * x + (b * g + c * g @ g) @ x
        return x

    def four_steps(x, s, a, b, c, coeffs=None):
        for _ in range(s - 1):
            g = x @ x.T
            x = a * x + (b * g + c * g @ g) @ x
        return x

    def swapped_a_c(x, s, a, b, c, coeffs=None):
        for _ in range(s):
            g = x @ x.T
            x = c * x + (b * g + a * g @ g) @ x
        return x

    return [dropped_c, wrong_sign_b, right_multiply, gram_transposed, four_steps, swapped_a_c]


@pytest.mark.parametrize("mutant", _mutant_iterations(), ids=lambda f: f.__name__)
def test_closed_form_pin_detects_planted_mistakes(monkeypatch, mutant):
    """Each mutant is a plausible slip in the iteration; the SVD pin must reject it.
    Square input so that every mutant is shape-valid."""
    from oracle import muon_oracle
    g = _inputs("lowrank", 56, 56, 6)
    ref = svd_closed_form(g)
    assert relf(newton_schulz(g), ref) <= 1e-12
    monkeypatch.setattr(muon_oracle, "ns_iterate", mutant)
    bad = muon_oracle.newton_schulz(g)
    assert relf(bad, ref) > 1e-6


def test_closed_form_pin_detects_missing_transpose(monkeypatch):
    from oracle import muon_oracle
    g = _inputs("gauss", 30, 12, 7)
    ref = svd_closed_form(g)

    def no_transpose_back(gg, steps=5, eps=1e-7, a=A, b=B, c=C, coeffs=None):
        x, _ = muon_oracle.frobenius_normalize(gg, eps)
        return muon_oracle.ns_iterate(x.T, steps, a, b, c)

    bad = no_transpose_back(g)
    assert bad.shape != ref.shape or relf(bad, ref) > 1e-6


# --------------------------------------------------------------------------
# per-iteration coefficients (a_k, b_k, c_k): the closed form composes the
# scalar quintics in iteration order, phi = p_K o ... o p_1
# --------------------------------------------------------------------------

SCHEDULES = {
    # assorted triples, each p_k(1) in the quintic's usual range
    "mixed": ((3.4445, -4.7750, 2.0315), (2.0, -1.5, 0.5), (1.875, -1.25, 0.375), (3.0, -3.2, 1.2),
              (1.5, -0.5, 0.0)),
    "uniform": ((A, B, C),) * 5,
    "identity": ((1.0, 0.0, 0.0),) * 5,
}


def phi_schedule(s, coeffs):
    """Scalar polynomials p_k(x) = a_k x + b_k x^3 + c_k x^5 applied in order, by a Python loop."""
    s = np.atleast_1d(np.asarray(s, dtype=np.float64))
    out = np.empty_like(s)
    for i, v in enumerate(s):
        x = float(v)
        for ak, bk, ck in coeffs:
            x = ak * x + bk * x ** 3 + ck * x ** 5
        out[i] = x
    return out


@pytest.mark.parametrize("name", ["mixed", "uniform"])
@pytest.mark.parametrize("shape", [(40, 96), (96, 40), (64, 64)])
def test_schedule_matches_composed_closed_form(name, shape):
    coeffs = SCHEDULES[name]
    g = _inputs("lowrank", shape[0], shape[1], 31)
    u, s, vt = np.linalg.svd(g, full_matrices=False)
    nu = math.sqrt(float(np.sum(g * g)))
    expect = (u * phi_schedule(s / (nu + 1e-7), coeffs)) @ vt
    got = newton_schulz(g, 5, 1e-7, coeffs=coeffs)
    assert relf(got, expect) <= 1e-12


def test_schedule_order_matters():
    """The same triples in reverse order give the reversed composition (and a different O)."""
    coeffs = SCHEDULES["mixed"]
    g = _inputs("gauss", 48, 80, 32)
    u, s, vt = np.linalg.svd(g, full_matrices=False)
    x = s / (math.sqrt(float(np.sum(g * g))) + 1e-7)
    fwd = newton_schulz(g, 5, coeffs=coeffs)
    rev = newton_schulz(g, 5, coeffs=tuple(reversed(coeffs)))
    assert relf(rev, (u * phi_schedule(x, tuple(reversed(coeffs)))) @ vt) <= 1e-12
    assert relf(fwd, rev) > 1e-3


def test_uniform_schedule_equals_scalar_coefficients():
    g = _inputs("heavy", 64, 96, 33)
    np.testing.assert_allclose(newton_schulz(g, 5, coeffs=SCHEDULES["uniform"]), newton_schulz(g, 5), rtol=0, atol=0)


def test_identity_schedule_returns_normalised_input():
    """p(x) = x at every iteration: O is the normalised input, transposes undone."""
    for shape in [(30, 50), (50, 30)]:
        g = _inputs("gauss", shape[0], shape[1], 34)
        got = newton_schulz(g, 5, 1e-7, coeffs=SCHEDULES["identity"])
        np.testing.assert_allclose(got, g / (np.linalg.norm(g) + 1e-7), rtol=1e-15, atol=0)


def test_schedule_in_full_step():
    """muon_step_matrix threads the schedule through to the iteration."""
    rng = np.random.default_rng(35)
    w, g = rng.standard_normal((24, 40)) * 0.02, rng.standard_normal((24, 40)) * 0.02
    hp = Hyper(coeffs=SCHEDULES["mixed"])
    r = muon_step_matrix(w, g, np.zeros_like(g), hp)
    u, s, vt = np.linalg.svd(g, full_matrices=False)
    o = (u * phi_schedule(s / (np.linalg.norm(g) + 1e-7), SCHEDULES["mixed"])) @ vt
    assert relf(r.o, o) <= 1e-12
    with pytest.raises(ValueError):
        newton_schulz(g, 5, coeffs=SCHEDULES["mixed"][:3])


# --------------------------------------------------------------------------
# sub-block orthogonalisation: each block is a matrix of its own (norm,
# transpose rule, iteration, shape scale); momentum stays elementwise
# --------------------------------------------------------------------------

def _blocked_closed_form(u, bh, bw):
    """Per-block SVD closed form, with the block slicing written out by index."""
    R, Cc = u.shape
    o = np.zeros_like(u)
    for bi in range(R // bh):
        for bj in range(Cc // bw):
            rows = np.arange(bi * bh, (bi + 1) * bh)
            cols = np.arange(bj * bw, (bj + 1) * bw)
            blk = u[np.ix_(rows, cols)]
            uu, s, vt = np.linalg.svd(blk, full_matrices=False)
            o[np.ix_(rows, cols)] = (uu * phi(s / (np.linalg.norm(blk) + 1e-7))) @ vt
    return o


@pytest.mark.parametrize("shape,block", [((384, 96), (128, 0)),    # 6 heads of 64 rows, pairs of heads
                                         ((96, 384), (0, 128)),    # the same cut along columns
                                         ((192, 160), (64, 80)),   # a 3 x 2 grid of blocks
                                         ((130, 60), (65, 0))])    # ragged block sizes, tall blocks
def test_blocked_step_matches_per_block_closed_form(shape, block):
    rng = np.random.default_rng(41)
    g = _inputs("lowrank", shape[0], shape[1], 41)
    w = rng.standard_normal(shape) * 0.02
    hp = Hyper(lr=0.05, weight_decay=0.1)
    r = oracle.muon_step_matrix_blocked(w, g, np.zeros_like(g), hp, *block)
    bh = shape[0] if block[0] == 0 else block[0]
    bw = shape[1] if block[1] == 0 else block[1]
    o = _blocked_closed_form(g, bh, bw)
    assert relf(r.o, o) <= 1e-12
    s = math.sqrt(max(1.0, bh / bw))        # the block's own shape scale
    assert relf(r.w, w * (1 - 0.05 * 0.1) - 0.05 * s * o) <= 1e-12
    assert r.nu.shape == ((shape[0] // bh) * (shape[1] // bw),)
    assert r.nu[0] == pytest.approx(np.linalg.norm(g[:bh, :bw]), rel=1e-14)


def test_blocked_whole_matrix_equals_plain_step():
    rng = np.random.default_rng(42)
    w, g, m = (rng.standard_normal((48, 80)) for _ in range(3))
    hp = Hyper(nesterov=True, weight_decay=0.01)
    a = muon_step_matrix(w, g, m, hp)
    for blk in [(0, 0), (48, 80), (48, 0), (0, 80)]:
        b = oracle.muon_step_matrix_blocked(w, g, m, hp, *blk)
        np.testing.assert_array_equal(a.o, b.o)
        np.testing.assert_array_equal(a.w, b.w)
        np.testing.assert_array_equal(a.m, b.m)
        assert b.nu.tolist() == [a.nu]


def test_blocked_rows_of_one_are_normalised_rows():
    """A 1 x C block has one singular value, its norm ratio: O's row is phi_5(‖u‖/(‖u‖+eps)) u/‖u‖."""
    g = _inputs("gauss", 7, 33, 43)
    r = oracle.muon_step_matrix_blocked(np.zeros_like(g), g, np.zeros_like(g), Hyper(), 1, 0)
    for i in range(7):
        nrm = math.sqrt(sum(float(v) ** 2 for v in g[i]))
        expect = phi([nrm / (nrm + 1e-7)])[0] * g[i] / nrm
        np.testing.assert_allclose(r.o[i], expect, rtol=1e-12, atol=0)


def test_blocked_columns_of_one_take_their_own_shape_scale():
    """An R x 1 block is tall: transposed, and its shape scale is sqrt(R), not the whole weight's."""
    g = _inputs("gauss", 9, 4, 44)
    lr = 0.1
    r = oracle.muon_step_matrix_blocked(np.zeros_like(g), g, np.zeros_like(g), Hyper(lr=lr), 0, 1)
    for j in range(4):
        col = g[:, j]
        nrm = float(np.linalg.norm(col))
        o = phi([nrm / (nrm + 1e-7)])[0] * col / nrm
        np.testing.assert_allclose(r.o[:, j], o, rtol=1e-12, atol=0)
        np.testing.assert_allclose(r.w[:, j], -lr * 3.0 * o, rtol=1e-12, atol=0)


def test_blocked_norm_is_per_block():
    """Scaling one block's gradient leaves every block's O unchanged (per-block
    normalisation); a whole-matrix normalisation would change the others.
    eps = 0 so that the normalisation is exactly scale invariant."""
    g = _inputs("lowrank", 128, 64, 45)
    hp = Hyper(eps=0.0)
    base = oracle.muon_step_matrix_blocked(np.zeros_like(g), g, np.zeros_like(g), hp, 32, 0)
    g2 = g.copy()
    g2[32:64] *= 1000.0
    scaled = oracle.muon_step_matrix_blocked(np.zeros_like(g), g2, np.zeros_like(g), hp, 32, 0)
    assert relf(scaled.o, base.o) <= 1e-11
    whole = newton_schulz(g2)
    assert relf(whole[:32], newton_schulz(g)[:32]) > 1e-2


def test_blocked_permuting_blocks_permutes_output():
    g = _inputs("heavy", 96, 40, 46)
    perm = [2, 0, 1]
    gp = np.concatenate([g[32 * k:32 * (k + 1)] for k in perm])
    a = oracle.muon_step_matrix_blocked(np.zeros_like(g), g, np.zeros_like(g), Hyper(), 32, 0)
    b = oracle.muon_step_matrix_blocked(np.zeros_like(g), gp, np.zeros_like(g), Hyper(), 32, 0)
    np.testing.assert_array_equal(b.o, np.concatenate([a.o[32 * k:32 * (k + 1)] for k in perm]))


def test_blocked_rejects_sizes_that_do_not_tile():
    g = np.ones((10, 12))
    for blk in [(3, 0), (0, 5), (-1, 0), (20, 0)]:
        with pytest.raises(ValueError):
            oracle.muon_step_matrix_blocked(g, g, g, Hyper(), *blk)


def test_blocked_mutant_with_global_norm_fails_pin():
    """A blocked step that normalises by the whole matrix's norm fails the per-block closed form."""
    g = _inputs("lowrank", 128, 48, 47)

    def global_norm_blocked(u, bh):
        nu = np.linalg.norm(u)
        out = np.empty_like(u)
        for r0 in range(0, u.shape[0], bh):
            x = u[r0:r0 + bh] / (nu + 1e-7)
            tall = x.shape[0] > x.shape[1]
            x = x.T if tall else x
            x = oracle.ns_iterate(x, 5, A, B, C)
            out[r0:r0 + bh] = x.T if tall else x
        return out

    assert relf(global_norm_blocked(g, 64), _blocked_closed_form(g, 64, 48)) > 1e-3
