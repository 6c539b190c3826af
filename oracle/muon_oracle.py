"""CPU float64 oracle for one Muon optimizer step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module; the product path
(the HIP library and its Python binding) never does, and shares no code with it.

It is a plain, slow, obviously-correct restatement of what the Muon pages
compute, in NumPy float64, one matrix at a time, with library matrix products
as its only building block.  Sources (page title, section):

* "14 — modded-nanogpt: the Speedrun Community", section 3 "Muon — the optimizer
  that started the modern speedrun era", "The one-line version": momentum
  m <- beta*m + g (beta = 0.95, no dampening), orthogonalise the momentum with
  5 Newton-Schulz iterations, then param -= lr * ortho.
* "NanoGPT Speedrun" (modded-nanogpt README mirror), Muon section, the
  Newton-Schulz routine: X = G / (||G||_F + eps) with eps = 1e-7; transpose when
  rows > cols; per iteration A = X X^T, B = b A + c A A, X = a X + B X with
  (a, b, c) = (3.4445, -4.7750, 2.0315); transpose back.  The same section lists
  Nesterov momentum "inside the update, with orthogonalization applied after
  momentum" and the bfloat16 execution of the iteration.
* Same README, GPT-2 medium track: "standard weight decay" (decoupled reading).

Readings where the pages are silent (each also listed in the design notes):

* Nesterov direction: u = g + beta * m', with m' the undampened momentum.
* Weight decay: decoupled and lr-coupled, W' = W (1 - lr*wd) - lr * s * O,
  applied to the old W.
* Shape scale s = sqrt(max(1, rows/cols)) on the stored shape.
* No bfloat16 cast of the normalised input: the oracle is exact float64.
* Sub-block orthogonalisation (query/key weights in pairs of heads): each block
  is a matrix of its own for the norm, the transpose rule, the iteration and
  the shape scale; momentum stays elementwise over the whole weight.

Every function here is checked against results fixed independently of it (the
SVD closed form, the momentum geometric series, printed constants) by the
``-m "not gpu"`` tests.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

# "NanoGPT Speedrun" page, Muon section, Newton-Schulz routine defaults.
NS_A, NS_B, NS_C = 3.4445, -4.7750, 2.0315
NS_STEPS = 5
NS_EPS = 1e-7
# "14 — modded-nanogpt", section 3, pseudocode default momentum.
BETA = 0.95


@dataclass
class Hyper:
    lr: float = 0.02
    beta: float = BETA
    weight_decay: float = 0.0
    nesterov: bool = False
    ns_steps: int = NS_STEPS
    eps: float = NS_EPS
    a: float = NS_A
    b: float = NS_B
    c: float = NS_C
    # optional per-iteration coefficients ((a_1, b_1, c_1), ...), one triple per
    # iteration, replacing (a, b, c) in that iteration's products
    coeffs: Optional[Tuple[Tuple[float, float, float], ...]] = None


# ----------------------------------------------------------------------------
# storage decode: stored values -> float64, exactly
# ----------------------------------------------------------------------------

def decode(stored: np.ndarray) -> np.ndarray:
    """Exact float64 value of a stored array (float32/float64, or uint16 bf16 bits)."""
    if stored.dtype == np.uint16:
        widened = stored.astype(np.uint32) << np.uint32(16)
        return widened.view(np.float32).astype(np.float64)
    return np.asarray(stored, dtype=np.float64)


# ----------------------------------------------------------------------------
# the step, one piece at a time
# ----------------------------------------------------------------------------

def momentum_update(m: np.ndarray, g: np.ndarray, beta: float) -> np.ndarray:
    """m' = beta * m + g  ("14 — modded-nanogpt", section 3 pseudocode; no (1-beta) factor)."""
    return beta * m + g


def update_direction(g: np.ndarray, m_new: np.ndarray, beta: float, nesterov: bool) -> np.ndarray:
    """The matrix handed to orthogonalisation.

    Plain momentum orthogonalises m'.  With Nesterov ("NanoGPT Speedrun" page,
    Muon section, list of practices) the reading is u = g + beta * m'.
    """
    return g + beta * m_new if nesterov else m_new


def frobenius_normalize(u: np.ndarray, eps: float) -> Tuple[np.ndarray, float]:
    """X0 = u / (||u||_F + eps): eps is added to the norm, not to its square."""
    nu = float(np.sqrt(np.sum(u * u)))
    return u / (nu + eps), nu


def ns_iterate(x: np.ndarray, steps: int, a: float, b: float, c: float,
               coeffs: Optional[Sequence[Tuple[float, float, float]]] = None) -> np.ndarray:
    """Quintic Newton-Schulz iterations on x as given (no transpose, no normalisation).

    Per iteration: A = X X^T; B = b A + c A A; X = a X + B X.  With ``coeffs``,
    iteration k (from 1) uses the k-th triple instead of (a, b, c): the
    per-iteration schedules the record list of the "NanoGPT Speedrun" page
    names (Polar Express); the pages print no schedule, so the triples are
    inputs.
    """
    if coeffs is not None and len(coeffs) < steps:
        raise ValueError("one coefficient triple per iteration")
    for k in range(steps):
        ak, bk, ck = coeffs[k] if coeffs is not None else (a, b, c)
        gram = x @ x.T
        poly = bk * gram + ck * (gram @ gram)
        x = ak * x + poly @ x
    return x


def newton_schulz(g: np.ndarray, steps: int = NS_STEPS, eps: float = NS_EPS,
                  a: float = NS_A, b: float = NS_B, c: float = NS_C,
                  coeffs: Optional[Sequence[Tuple[float, float, float]]] = None) -> np.ndarray:
    """Approximate U V^T of g's SVD ("NanoGPT Speedrun" page, Muon section).

    Normalise by the Frobenius norm, transpose when rows > cols (strictly), run
    the quintic iteration, transpose back.  float64 throughout.
    """
    g = np.asarray(g, dtype=np.float64)
    if g.ndim != 2:
        raise ValueError("Newton-Schulz takes a 2-D matrix")
    x, _ = frobenius_normalize(g, eps)
    tall = g.shape[0] > g.shape[1]
    if tall:
        x = x.T
    x = ns_iterate(x, steps, a, b, c, coeffs)
    if tall:
        x = x.T
    return np.ascontiguousarray(x)


def shape_scale(rows: int, cols: int) -> float:
    """s = sqrt(max(1, rows / cols)) on the stored shape (reading)."""
    return math.sqrt(max(1.0, rows / cols))


def param_update(w: np.ndarray, o: np.ndarray, lr: float, weight_decay: float, scale: float) -> np.ndarray:
    """W' = W (1 - lr*wd) - lr * s * O: decoupled decay on the old W, then the
    update of "14 — modded-nanogpt" section 3 (param -= lr * ortho)."""
    return w * (1.0 - lr * weight_decay) - (lr * scale) * o


@dataclass
class StepResult:
    w: np.ndarray       # new weight, float64 (not rounded to storage)
    m: np.ndarray       # new momentum, float64
    o: np.ndarray       # orthogonalised update, stored orientation, float64
    nu: float           # Frobenius norm of the orthogonalised input


def muon_step_matrix(w: np.ndarray, g: np.ndarray, m: np.ndarray, hp: Hyper) -> StepResult:
    """One Muon step for one 2-D weight, all in float64."""
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    m_new = momentum_update(m, g, hp.beta)
    u = update_direction(g, m_new, hp.beta, hp.nesterov)
    nu = float(np.sqrt(np.sum(u * u)))
    o = newton_schulz(u, hp.ns_steps, hp.eps, hp.a, hp.b, hp.c, hp.coeffs)
    s = shape_scale(*w.shape)
    w_new = param_update(w, o, hp.lr, hp.weight_decay, s)
    return StepResult(w_new, m_new, o, nu)


def block_corners(rows: int, cols: int, block_rows: int, block_cols: int) -> List[Tuple[int, int, int, int]]:
    """(r0, c0, h, w) of every block of a rows x cols matrix cut into
    block_rows x block_cols blocks, row-major; 0 means the whole dimension.
    Each block size must divide its dimension."""
    h = rows if block_rows == 0 else block_rows
    w = cols if block_cols == 0 else block_cols
    if h < 1 or w < 1 or rows % h or cols % w:
        raise ValueError(f"block {block_rows} x {block_cols} does not tile {rows} x {cols}")
    return [(r0, c0, h, w) for r0 in range(0, rows, h) for c0 in range(0, cols, w)]


def muon_step_matrix_blocked(w: np.ndarray, g: np.ndarray, m: np.ndarray, hp: Hyper,
                             block_rows: int, block_cols: int) -> StepResult:
    """One Muon step where the weight is cut into blocks, each orthogonalised
    as a matrix of its own.

    "NanoGPT Speedrun" (modded-nanogpt README mirror), record list: the query
    and key weights are orthogonalised in pairs of heads instead of across all
    heads at once.  Reading: momentum is elementwise, so it is the whole
    matrix's recurrence; normalisation (with its eps), the transpose rule, the
    iteration and the shape scale all act on each block with its own shape.
    ``nu`` holds the blocks' norms in row-major block order.
    """
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    m_new = momentum_update(m, g, hp.beta)
    u = update_direction(g, m_new, hp.beta, hp.nesterov)
    o = np.empty_like(u)
    w_new = np.empty_like(w)
    nus = []
    for r0, c0, bh, bw in block_corners(*w.shape, block_rows, block_cols):
        ub = u[r0:r0 + bh, c0:c0 + bw]
        nus.append(float(np.sqrt(np.sum(ub * ub))))
        ob = newton_schulz(ub, hp.ns_steps, hp.eps, hp.a, hp.b, hp.c, hp.coeffs)
        o[r0:r0 + bh, c0:c0 + bw] = ob
        w_new[r0:r0 + bh, c0:c0 + bw] = param_update(w[r0:r0 + bh, c0:c0 + bw], ob, hp.lr, hp.weight_decay,
                                                     shape_scale(bh, bw))
    return StepResult(w_new, m_new, o, np.array(nus))


def muon_step(ws: Sequence[np.ndarray], gs: Sequence[np.ndarray], ms: Sequence[np.ndarray],
              hp: Hyper) -> List[StepResult]:
    """The step over a list of matrices: each matrix independently."""
    return [muon_step_matrix(w, g, m, hp) for w, g, m in zip(ws, gs, ms)]


# ----------------------------------------------------------------------------
# work accounting
# ----------------------------------------------------------------------------

def ns_flops_dense(rows: int, cols: int, steps: int = NS_STEPS) -> int:
    """Dense multiply-add count x2 of the iteration on an m x n X (m <= n).

    X X^T: 2 m^2 n; A A: 2 m^3; B X: 2 m^2 n; per iteration 4 m^2 n + 2 m^3.
    """
    m, n = min(rows, cols), max(rows, cols)
    return steps * (4 * m * m * n + 2 * m ** 3)


def ns_flops_unique(rows: int, cols: int, steps: int = NS_STEPS) -> int:
    """Flops when the symmetric products (X X^T and A A) form only their
    m(m+1)/2 distinct entries: m(m+1) n + m^2 (m+1) + 2 m^2 n per iteration."""
    m, n = min(rows, cols), max(rows, cols)
    return steps * (m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n)


def muon_overhead_fraction(hidden: int, tokens_per_batch: int, steps: int = NS_STEPS) -> float:
    """Newton-Schulz flops on a square hidden x hidden weight divided by the
    training flops that weight costs per batch (6 * params * tokens)."""
    return ns_flops_dense(hidden, hidden, steps) / (6.0 * hidden * hidden * tokens_per_batch)
