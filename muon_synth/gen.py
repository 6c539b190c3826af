"""Seeded synthetic workloads for the Muon step.

Every array is drawn in float64 from ``numpy.random.default_rng`` seeded by
``SeedSequence([workload_id, step, matrix_index, role])`` and then encoded to
its storage type (float32, or bfloat16 bit patterns with round-to-nearest-even).
The stored values are the inputs for every consumer: the oracle decodes them,
the GPU path uploads them bit for bit.

Workload shapes follow the models the Muon pages train: the GPT-2 small
hidden-matrix set (``14 — modded-nanogpt``, section 3 "Muon", the 124M scale
with 768 hidden; "NanoGPT Speedrun" page, the GPT-2 medium track for the 350M
set), plus two larger stand-ins (a 4096/14336 layer share and an MoE expert
stack).  No dataset is read: gradients are synthetic with the stated spectra.

Roles: 0 = weight init, 1 = gradient, 2 = initial momentum, 3 = expert scale.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Callable, Dict, List, Optional, Tuple

import numpy as np

ROLE_PARAM, ROLE_GRAD, ROLE_MOM, ROLE_SCALE = 0, 1, 2, 3


def rng_for(wid: int, step: int, idx: int, role: int) -> np.random.Generator:
    """The generator for one (workload, step, matrix, role) stream."""
    return np.random.default_rng(np.random.SeedSequence([int(wid), int(step), int(idx), int(role)]))


# ----------------------------------------------------------------------------
# storage encoding (not optimizer arithmetic: it defines the stored inputs)
# ----------------------------------------------------------------------------

def _f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32)
    r = (u >> 16) & np.uint32(1)          # lsb of the kept half (ties go to even)
    r += np.uint32(0x7FFF)
    r += u                                # finite values cannot overflow 32 bits
    r >>= 16
    out = r.astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def encode_storage(x: np.ndarray, storage: str) -> np.ndarray:
    """float64 -> stored representation: float32 array, or uint16 bfloat16 bits.

    bfloat16 goes through float32 first (both steps round to nearest even); the
    result is what both the oracle and the GPU consume, so the exact rounding
    path only defines the input, it is not compared against anything.
    """
    if storage == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if storage == "bf16":
        return _f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    raise ValueError(f"unknown storage {storage!r}")


# ----------------------------------------------------------------------------
# distributions
# ----------------------------------------------------------------------------

def gaussian(rng: np.random.Generator, rows: int, cols: int, std: float) -> np.ndarray:
    return rng.standard_normal((rows, cols)) * std


def _rms(x: np.ndarray) -> float:
    if not x.size:
        return 0.0
    v = x.reshape(-1)
    return float(np.sqrt(np.dot(v, v) / v.size))


def _orthonormal_cols(rng: np.random.Generator, n: int, r: int) -> np.ndarray:
    """n x r matrix with orthonormal columns (QR of a Gaussian draw, signs fixed)."""
    q, rr = np.linalg.qr(rng.standard_normal((n, r)))
    d = np.sign(np.diag(rr))
    d[d == 0] = 1.0
    return q * d


def lowrank_noise_grad(rng: np.random.Generator, rows: int, cols: int, rank: int = 16,
                       noise_std: float = 1e-3, std: float = 0.02) -> np.ndarray:
    """Rank-``rank`` Gaussian factors with singular values 1/k, plus noise.

    L = Qu diag(1/k) Qv^T (Qu, Qv orthonormal from QR of Gaussian draws), scaled
    to element RMS 0.02; Z = L + N(0, noise_std^2); G = std * Z / rms(Z).
    """
    r = max(1, min(rank, rows, cols))
    qu = _orthonormal_cols(rng, rows, r)
    qv = _orthonormal_cols(rng, cols, r)
    sig = 1.0 / np.arange(1, r + 1, dtype=np.float64)
    low = (qu * sig) @ qv.T
    low *= 0.02 / max(_rms(low), 1e-300)
    z = low + noise_std * rng.standard_normal((rows, cols))
    return z * (std / max(_rms(z), 1e-300))


def _pow2_factor(n: int, cap: int) -> int:
    f = 1
    while f * 2 <= cap and n % (f * 2) == 0:
        f *= 2
    return f


def _kron_orthonormal_apply(rng: np.random.Generator, t: int, s: int, m: np.ndarray) -> Optional[np.ndarray]:
    """Return Q @ m for a t x s orthonormal-column Q = A (x) B, or None if t, s do not factor.

    B is a Haar-like f x f orthogonal matrix and A a t/f x s/f orthonormal-column
    matrix; Q = kron(A, B) has orthonormal columns, so the product keeps the
    singular values of ``m`` while spreading every entry.
    """
    f = _pow2_factor(np.gcd(t, s), 128)
    if f < 16:
        return None
    t1, r1 = t // f, s // f
    a = _orthonormal_cols(rng, t1, r1)
    b = _orthonormal_cols(rng, f, f)
    cols = m.shape[1]
    m3 = m.reshape(r1, f, cols)
    t_qic = np.tensordot(b, m3, axes=([1], [1]))          # (f, r1, cols): [q, i, c]
    y = np.tensordot(a, t_qic, axes=([1], [1]))           # (t1, f, cols): [p, q, c]
    return y.reshape(t, cols)


def heavy_tail_grad(rng: np.random.Generator, rows: int, cols: int, alpha: float = 0.7,
                    std: float = 0.02) -> np.ndarray:
    """Full-rank gradient with singular values proportional to k^-alpha, element RMS ``std``.

    G = Qt diag(k^-alpha) Qs^T in the tall orientation; large factor matrices are
    Kronecker products of Haar-like factors (exact spectrum, cheap to apply),
    small ones come from a dense QR.
    """
    t, s = max(rows, cols), min(rows, cols)
    sig = np.arange(1, s + 1, dtype=np.float64) ** (-alpha)
    g_tall = None
    if s >= 1024:
        f = _pow2_factor(s, 64)
        qs = np.kron(_orthonormal_cols(rng, s // f, s // f), _orthonormal_cols(rng, f, f))
        mm = sig[:, None] * qs.T                          # diag(sig) Qs^T, s x s
        g_tall = _kron_orthonormal_apply(rng, t, s, mm)
    if g_tall is None:
        qt = _orthonormal_cols(rng, t, s)
        qs = _orthonormal_cols(rng, s, s)
        g_tall = (qt * sig) @ qs.T
    g = g_tall if rows >= cols else g_tall.T
    return np.ascontiguousarray(g * (std / max(_rms(g), 1e-300)))


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class MatSpec:
    rows: int
    cols: int
    name: str
    group: int = -1            # expert index (per-expert gradient scale), -1 = none


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    mats: Tuple[MatSpec, ...]
    storage: str = "bf16"       # param / grad storage; momentum is always float32
    compute: str = "bf16"       # Newton-Schulz operand precision
    grad_kind: str = "lowrank_noise"
    momentum_init: str = "zero"
    steps: int = 10
    beta: float = 0.95
    nesterov: bool = False
    weight_decay: float = 0.0
    lr: float = 0.02
    ns_steps: int = 5
    eps: float = 1e-7
    a: float = 3.4445
    b: float = -4.7750
    c: float = 2.0315
    coeffs: Optional[Tuple[Tuple[float, float, float], ...]] = None   # per-iteration triples, None = (a, b, c)
    blocks: Optional[Tuple[Tuple[int, int], ...]] = None   # per-matrix (block_rows, block_cols), 0 = whole
    expert_scale_range: Tuple[float, float] = (-4.0, -1.0)
    description: str = ""

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def elements(self) -> int:
        return sum(m.rows * m.cols for m in self.mats)


def _gpt2_set(layers: int, d: int, ff: int) -> Tuple[MatSpec, ...]:
    out: List[MatSpec] = []
    for l in range(layers):
        for nm in ("q", "k", "v", "o"):
            out.append(MatSpec(d, d, f"h{l}.attn.{nm}"))
        out.append(MatSpec(d, ff, f"h{l}.mlp.up"))
        out.append(MatSpec(ff, d, f"h{l}.mlp.down"))
    return tuple(out)


def _qk_pairs(mats: Tuple[MatSpec, ...], rows: int) -> Tuple[Tuple[int, int], ...]:
    """Block sizes: query and key weights cut into `rows`-row blocks, the rest whole."""
    return tuple((rows, 0) if m.name.endswith((".q", ".k")) else (0, 0) for m in mats)


def _large_share() -> Tuple[MatSpec, ...]:
    out: List[MatSpec] = []
    for l in range(4):
        out.append(MatSpec(4096, 4096, f"l{l}.sq"))
        out.append(MatSpec(4096, 14336, f"l{l}.wide"))
        out.append(MatSpec(14336, 4096, f"l{l}.tall"))
    return tuple(out)


def _moe_stack() -> Tuple[MatSpec, ...]:
    out: List[MatSpec] = []
    for e in range(64):
        out.append(MatSpec(2048, 1408, f"e{e}.up", group=e))
        out.append(MatSpec(1408, 2048, f"e{e}.down", group=e))
    for i in range(4):
        out.append(MatSpec(2048, 2048, f"shared.attn{i}"))
    return tuple(out)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in (
        Workload("single-64x128-fp32", 1, (MatSpec(64, 128, "w"),), storage="fp32", compute="fp32",
                 grad_kind="gaussian", momentum_init="gaussian", steps=1,
                 description="one 64x128 float32 matrix, W/G/M ~ N(0, 0.02^2), one step, fp32 mode"),
        Workload("gpt2-124m-hidden", 2, _gpt2_set(12, 768, 3072), steps=10,
                 description="GPT-2 124M hidden matrices: 12 x {4 x 768x768, 768x3072, 3072x768}"),
        Workload("gpt2-124m-hidden-qk-head-pairs", 6, _gpt2_set(12, 768, 3072), steps=10,
                 blocks=_qk_pairs(_gpt2_set(12, 768, 3072), 2 * 64),
                 description="the GPT-2 124M set with every query and key weight orthogonalised in "
                             "pairs of 64-wide heads (6 blocks of 128x768 each)"),
        Workload("gpt2-350m-hidden", 3, _gpt2_set(24, 1024, 4096), steps=10, nesterov=True,
                 weight_decay=0.01,
                 description="GPT-2 350M-style: 24 x {4 x 1024x1024, 1024x4096, 4096x1024}, Nesterov, wd 0.01"),
        Workload("large-layer-share-4096x14336", 4, _large_share(), grad_kind="heavy_tail", steps=5,
                 description="4 layers x {4096x4096, 4096x14336, 14336x4096}, spectrum k^-0.7"),
        Workload("moe-64x-2048x1408", 5, _moe_stack(), grad_kind="lowrank_noise_expert", steps=5,
                 description="64 experts x {2048x1408, 1408x2048} + 4 x 2048x2048, log-uniform expert scale"),
    )
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def make_param(wl: Workload, idx: int) -> np.ndarray:
    m = wl.mats[idx]
    return gaussian(rng_for(wl.wid, 0, idx, ROLE_PARAM), m.rows, m.cols, 0.02)


def make_momentum(wl: Workload, idx: int) -> np.ndarray:
    m = wl.mats[idx]
    if wl.momentum_init == "zero":
        return np.zeros((m.rows, m.cols))
    return gaussian(rng_for(wl.wid, 0, idx, ROLE_MOM), m.rows, m.cols, 0.02)


def expert_scale(wl: Workload, group: int) -> float:
    lo, hi = wl.expert_scale_range
    return float(10.0 ** rng_for(wl.wid, 0, group, ROLE_SCALE).uniform(lo, hi))


def make_grad(wl: Workload, step: int, idx: int) -> np.ndarray:
    m = wl.mats[idx]
    rng = rng_for(wl.wid, step, idx, ROLE_GRAD)
    kind = wl.grad_kind
    if kind == "gaussian":
        return gaussian(rng, m.rows, m.cols, 0.02)
    if kind == "lowrank_noise":
        return lowrank_noise_grad(rng, m.rows, m.cols)
    if kind == "lowrank_noise_expert":
        std = expert_scale(wl, m.group) if m.group >= 0 else 0.02
        return lowrank_noise_grad(rng, m.rows, m.cols, std=std)
    if kind == "heavy_tail":
        return heavy_tail_grad(rng, m.rows, m.cols)
    raise ValueError(f"unknown grad kind {kind!r}")


GradFn = Callable[[Workload, int, int], np.ndarray]


# ---------------------------------------------------------------------------
# AdamW parameter sets: the tensors the hybrid setup keeps off Muon
# (embeddings, output head, norm gains and biases), as flat element counts.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class TensorSpec:
    numel: int
    name: str
    kind: str = "weight"       # "weight" (N(0, 0.02^2)), "gain" (ones), "bias" (zeros)


@dataclass(frozen=True)
class AdamWWorkload:
    name: str
    wid: int
    tensors: Tuple[TensorSpec, ...]
    storage: str = "bf16"       # param / grad storage; both moments are float32
    steps: int = 10
    lr: float = 3e-3
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-10
    weight_decay: float = 0.0
    grad_std_range: Tuple[float, float] = (-5.0, -2.0)   # log10 of the per-tensor gradient std
    description: str = ""

    @property
    def elements(self) -> int:
        return sum(t.numel for t in self.tensors)


def _gpt2_adamw_set(layers: int, d: int, ff: int, vocab: int, ctx: int) -> Tuple[TensorSpec, ...]:
    out: List[TensorSpec] = [TensorSpec(vocab * d, "wte"), TensorSpec(ctx * d, "wpe"),
                             TensorSpec(vocab * d, "lm_head")]
    for l in range(layers):
        out += [TensorSpec(d, f"h{l}.ln1.g", "gain"), TensorSpec(d, f"h{l}.ln1.b", "bias"),
                TensorSpec(3 * d, f"h{l}.attn.qkv.b", "bias"), TensorSpec(d, f"h{l}.attn.o.b", "bias"),
                TensorSpec(d, f"h{l}.ln2.g", "gain"), TensorSpec(d, f"h{l}.ln2.b", "bias"),
                TensorSpec(ff, f"h{l}.mlp.up.b", "bias"), TensorSpec(d, f"h{l}.mlp.down.b", "bias")]
    out += [TensorSpec(d, "ln_f.g", "gain"), TensorSpec(d, "ln_f.b", "bias")]
    return tuple(out)


ADAMW_WORKLOADS: Dict[str, AdamWWorkload] = {
    w.name: w
    for w in (
        AdamWWorkload("gpt2-124m-adamw-params", 20, _gpt2_adamw_set(12, 768, 3072, 50257, 1024),
                      description="GPT-2 124M parameters off Muon: token embedding and untied head "
                                  "(50257 x 768 each), position embedding 1024 x 768, norm gains and "
                                  "biases, linear biases"),
    )
}


def adamw_workload(name: str) -> AdamWWorkload:
    return ADAMW_WORKLOADS[name]


def make_adamw_param(wl: AdamWWorkload, idx: int) -> np.ndarray:
    t = wl.tensors[idx]
    if t.kind == "gain":
        return np.ones(t.numel)
    if t.kind == "bias":
        return np.zeros(t.numel)
    return rng_for(wl.wid, 0, idx, ROLE_PARAM).standard_normal(t.numel) * 0.02


def make_adamw_grad(wl: AdamWWorkload, step: int, idx: int) -> np.ndarray:
    """Gaussian gradient with a per-tensor scale, log-uniform over grad_std_range."""
    lo, hi = wl.grad_std_range
    std = 10.0 ** rng_for(wl.wid, 0, idx, ROLE_SCALE).uniform(lo, hi)
    return rng_for(wl.wid, step, idx, ROLE_GRAD).standard_normal(wl.tensors[idx].numel) * std
