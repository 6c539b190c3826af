"""Why the master copy of X keeps about 16 significant bits: a CPU model of the
bf16 iteration's arithmetic against the float64 oracle.

The model follows the kernels' description (not their code): bf16 MFMA
operands rounded to nearest even, float32 accumulation, A and B stored in
bf16, and one of three representations of X between iterations:

- "bf16": X itself kept in bf16 (the pages' bfloat16 iteration);
- "fp32": an fp32 master of X, operands its bf16 rounding;
- "hilo8": the bf16 operand copy plus the remainder X - hi in one byte, in
  units of 1/256 of the bf16 spacing at hi (what the library stores).

Inputs: the low-rank-plus-noise gradients of the GPT-2 workloads, 5 steps of
Nesterov momentum.  The bf16-only X misses the 3e-2 parity bar; the fp32
master passes with a wide margin, and the byte remainder matches it.
"""

import numpy as np
import pytest

import oracle
from muon_synth import encode_storage, lowrank_noise_grad, rng_for

BAR = 3e-2


def _bf(x):
    return oracle.decode(encode_storage(np.asarray(x, np.float64), "bf16"))


def _f32(x):
    return np.asarray(x, np.float32).astype(np.float64)


def _lo8(x, hi):
    """The remainder x - hi rounded to units of 1/256 of the bf16 spacing at hi."""
    _, e = np.frexp(hi)                  # hi = f 2^e, 0.5 <= |f| < 1: bf16 spacing 2^(e-8)
    unit = np.ldexp(1.0, e - 16)
    q = np.clip(np.rint((x - hi) / unit), -127, 127)
    return np.where(hi == 0, 0.0, q * unit)


def _ns_model(u, master, steps=5, a=3.4445, b=-4.7750, c=2.0315, eps=1e-7):
    tall = u.shape[0] > u.shape[1]
    if tall:
        u = u.T
    x = _f32(u / (np.sqrt(np.sum(u * u)) + eps))
    for _ in range(steps):
        xo = _bf(x)
        A = _bf(_f32(xo @ xo.T))
        B = _bf(_f32(b * A + c * _f32(A @ A)))
        xm = {"bf16": xo, "fp32": x, "hilo8": None}[master]
        if master == "hilo8":
            xm = xo + _lo8(x, xo)
        x = _f32(a * xm + _f32(B @ xo))
        if master == "bf16":
            x = _bf(x)
    return x.T if tall else x


def _direction(r, c, seed):
    m = np.zeros((r, c))
    g = None
    for t in range(1, 6):
        g = _bf(lowrank_noise_grad(rng_for(seed, t, r, 1), r, c))
        m = 0.95 * m + g
    return _bf(g + 0.95 * m)


@pytest.mark.parametrize("shape", [(256, 768), (768, 256), (384, 1536)])
def test_master_precision_budget(shape):
    u = _direction(*shape, seed=5)
    ref = oracle.newton_schulz(u)
    err = {k: np.linalg.norm(_ns_model(u, k) - ref) / np.linalg.norm(ref) for k in ("bf16", "fp32", "hilo8")}
    print(shape, {k: f"{v:.2e}" for k, v in err.items()})
    assert err["bf16"] > BAR                      # X in bf16 misses the bar (measured 4.1-4.2e-2)
    assert err["fp32"] < BAR / 5                  # an fp32 master passes with margin (2.9-4.0e-3)
    assert abs(err["hilo8"] - err["fp32"]) <= 0.05 * err["fp32"]   # the byte remainder matches it


def test_byte_remainder_holds_fifteen_bits():
    """|x - (hi + lo)| <= half a unit, or one unit where the remainder is
    exactly half a bf16 spacing (128 units, clamped to 127): <= 2^-15 |x|."""
    rng = np.random.default_rng(9)
    x = _f32(rng.standard_normal(100000) * np.exp(rng.uniform(-20, 5, 100000)))
    hi = _bf(x)
    rec = hi + _lo8(x, hi)
    rel = np.abs(rec - x) / np.abs(x)
    assert np.all(rel <= 2.0 ** -15)
    assert np.median(rel) < 2.0 ** -17
    assert np.max(np.abs(x - hi) / np.abs(x)) > 2.0 ** -10    # hi alone does not
