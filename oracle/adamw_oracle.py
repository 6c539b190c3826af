"""CPU float64 oracle for the AdamW step that the hybrid Muon setup runs on
every parameter Muon does not take.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module; the product path
never does, and shares no code with it.

Sources (page title, section): "14 — modded-nanogpt: the Speedrun Community",
section 3 (Muon is for matrix-shaped layers; AdamW is recommended for the other
parameters); the "Where Muon does not apply" list of the Muon page (biases,
norm gains and embeddings stay on AdamW; the canonical setup is the hybrid).
The pages give no AdamW formula and no AdamW hyperparameters.  Reading: the
standard AdamW, Adam (Kingma and Ba, 2015) with decoupled weight decay
(Loshchilov and Hutter, 2019), with bias-corrected moments:

    m' = beta1 m + (1 - beta1) g
    v' = beta2 v + (1 - beta2) g^2
    p' = p (1 - lr wd) - lr (m' / (1 - beta1^t)) / (sqrt(v' / (1 - beta2^t)) + eps)

for the 1-based step count t; the decay acts on the old p.  Every function is
checked against independent results (closed forms, and torch.optim.AdamW run as
a black box) by the ``-m "not gpu"`` tests.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class AdamWHyper:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01


@dataclass
class AdamWResult:
    p: np.ndarray       # new parameter, float64 (not rounded to storage)
    m: np.ndarray       # new first moment
    v: np.ndarray       # new second moment


def adamw_step(p: np.ndarray, g: np.ndarray, m: np.ndarray, v: np.ndarray, hp: AdamWHyper,
               step: int) -> AdamWResult:
    """One AdamW step, step = t >= 1 (the bias corrections use beta^t)."""
    if step < 1:
        raise ValueError("step counts from 1")
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    m_new = hp.beta1 * m + (1.0 - hp.beta1) * g
    v_new = hp.beta2 * v + (1.0 - hp.beta2) * g * g
    m_hat = m_new / (1.0 - hp.beta1 ** step)
    v_hat = v_new / (1.0 - hp.beta2 ** step)
    p_new = p * (1.0 - hp.lr * hp.weight_decay) - hp.lr * m_hat / (np.sqrt(v_hat) + hp.eps)
    return AdamWResult(p_new, m_new, v_new)
