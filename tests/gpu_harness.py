"""Helpers shared by the GPU tests: upload seeded stored inputs, run the HIP
path through the C ABI, read results back, compare with the oracle."""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

import oracle
from muon_synth import Workload, encode_storage, make_grad, make_momentum, make_param

# Parity bars (rel-F = ||x - y||_F / ||y||_F against the float64 oracle).
TOL_O_BF16 = 3e-2        # orthogonalised update, bf16 MFMA mode
TOL_O_FP32 = 1e-5        # orthogonalised update, fp32 validation mode
TOL_MOM = 1e-6           # momentum buffers, fp32 storage
# Local bars on O: every 128 x 128 tile of the stored R x C output (the AXPY
# kernel's output tiles), every row of at least LOCAL_MIN_LINE elements and
# every such column must meet the whole-matrix bar on its own, each measured
# against at least its fair share of the whole norm (sqrt(elements / R C)
# ||O||_F), so a tile whose own norm is tiny is not held to a relative bar it
# cannot meet.  One wrong tile, row or column of a large matrix moves the
# whole-matrix error by only ~1e-2 but its own by ~1.
LOCAL_TILE = 128
LOCAL_MIN_LINE = 64


def relf(x: np.ndarray, y: np.ndarray) -> float:
    d = np.linalg.norm(np.asarray(x, np.float64) - np.asarray(y, np.float64))
    return float(d / max(np.linalg.norm(np.asarray(y, np.float64)), 1e-300))


def local_errors(o: np.ndarray, ref: np.ndarray, tile: int = LOCAL_TILE, min_line: int = LOCAL_MIN_LINE) -> dict:
    """Worst local error ratios of ``o`` against ``ref`` (both R x C):
    ||dO_part||_F / max(||ref_part||_F, sqrt(|part| / RC) ||ref||_F) over the
    tile x tile tiles (clipped at the edges), the rows of at least
    ``min_line`` elements and the columns of at least ``min_line`` elements
    (0.0 where a matrix has no such line)."""
    o = np.asarray(o, np.float64)
    ref = np.asarray(ref, np.float64)
    R, C = ref.shape
    n = float(R * C)
    tot = float(np.linalg.norm(ref))
    d = o - ref
    rt = int(np.ceil(R / tile))
    ct = int(np.ceil(C / tile))
    pad_r, pad_c = rt * tile - R, ct * tile - C
    dp = np.pad(d, ((0, pad_r), (0, pad_c))).reshape(rt, tile, ct, tile)
    rp = np.pad(ref, ((0, pad_r), (0, pad_c))).reshape(rt, tile, ct, tile)
    dn = np.sqrt(np.einsum("iajb,iajb->ij", dp, dp))
    rn = np.sqrt(np.einsum("iajb,iajb->ij", rp, rp))
    hr = np.minimum(tile, R - tile * np.arange(rt))[:, None]
    hc = np.minimum(tile, C - tile * np.arange(ct))[None, :]
    floor = np.sqrt(hr * hc / n) * tot
    out = {"tile": float(np.max(dn / np.maximum(np.maximum(rn, floor), 1e-300))), "row": 0.0, "col": 0.0}
    if C >= min_line:
        fl = np.sqrt(C / n) * tot
        out["row"] = float(np.max(np.linalg.norm(d, axis=1) /
                                  np.maximum(np.maximum(np.linalg.norm(ref, axis=1), fl), 1e-300)))
    if R >= min_line:
        fl = np.sqrt(R / n) * tot
        out["col"] = float(np.max(np.linalg.norm(d, axis=0) /
                                  np.maximum(np.maximum(np.linalg.norm(ref, axis=0), fl), 1e-300)))
    return out


def assert_o_close(o_gpu: np.ndarray, o_ref: np.ndarray, tol: float, what: str) -> dict:
    """Whole-matrix rel-F and every local ratio (tiles, rows, columns) within
    ``tol``; returns the figures."""
    e = {"global": relf(o_gpu, o_ref), **local_errors(o_gpu, o_ref)}
    for k, v in e.items():
        assert v <= tol, f"{what}: O {k} error {v:.3e} > {tol}"
    return e


def to_device(stored: np.ndarray, dev="cuda"):
    import torch
    if stored.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(stored).view(np.int16).copy()).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(stored, dtype=np.float32).copy()).to(dev)


def to_stored(t) -> np.ndarray:
    """Device tensor -> stored numpy representation (uint16 bf16 bits or float32)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().contiguous().cpu().numpy().astype(np.float32)


def bf16_rne_from_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 with one rounding (nearest, ties to even); uint16 bits.
    Used only to state the expected stored weight from float64 values."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    q = np.round(m * 256.0) / 256.0          # 8 significant bits, numpy rounds half to even
    y = np.ldexp(q, e).astype(np.float32)    # exact in float32
    return (y.view(np.uint32) >> 16).astype(np.uint16)


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|ordinal(a) - ordinal(b)| for bf16 bit patterns (sign-magnitude to ordinal)."""
    def ordinal(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordinal(a) - ordinal(b))


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (normal range)."""
    return np.spacing(np.abs(np.asarray(x, np.float64)).astype(np.float32)).astype(np.float64) * 65536.0


def weight_error_ok(w_new_bits: np.ndarray, w_old: np.ndarray, o: np.ndarray, lr: float, wd: float,
                    scale: float) -> np.ndarray:
    """Elementwise: the stored bf16 weight lies within one bf16 ulp of the exact
    float64 update of the GPU's own O, widened by the float32 evaluation error of
    W (1 - lr wd) - lr s O (a few float32 roundings of each term), which matters
    only where the two terms cancel."""
    w_exp = w_old * (1.0 - lr * wd) - lr * scale * o
    got = (w_new_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    slack = 4.0 * 2.0 ** -24 * (np.abs(w_old) + lr * scale * np.abs(o))
    return np.abs(got - w_exp) <= bf16_ulp(w_exp) + slack


def hparams_for(wl: Workload):
    import newton_schulz_matrix_step_amd as nsm
    return nsm.Hparams(lr=wl.lr, beta=wl.beta, weight_decay=wl.weight_decay, eps=wl.eps, a=wl.a, b=wl.b, c=wl.c,
                       nesterov=wl.nesterov, ns_steps=wl.ns_steps, compute=wl.compute, coeffs=wl.coeffs)


def oracle_hyper(wl: Workload) -> oracle.Hyper:
    return oracle.Hyper(lr=wl.lr, beta=wl.beta, weight_decay=wl.weight_decay, nesterov=wl.nesterov,
                        ns_steps=wl.ns_steps, eps=wl.eps, a=wl.a, b=wl.b, c=wl.c,
                        coeffs=wl.coeffs)


def shape_scales(shape, block=(0, 0)) -> np.ndarray:
    """Elementwise shape scale sqrt(max(1, h/w)) of the block each element belongs to."""
    bh = shape[0] if block[0] == 0 else block[0]
    bw = shape[1] if block[1] == 0 else block[1]
    return np.full(shape, math.sqrt(max(1.0, bh / bw)))


@dataclass
class StepRecord:
    w_old: np.ndarray    # stored representation before the step
    w_new: np.ndarray    # stored representation after the step
    m_new: np.ndarray    # float32
    o: np.ndarray        # float32 update_out
    g: np.ndarray        # stored gradient of this step


def run_gpu(wl: Workload, steps: int, check: Sequence[int], handle=None, grad_fn=None) -> Dict[int, List[StepRecord]]:
    """Run ``steps`` Muon steps over every matrix of ``wl`` in one grouped call per
    step; record the matrices listed in ``check``."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    own = handle is None
    h = nsm.muon_init(0) if own else handle
    try:
        n = len(wl.mats)
        params = [to_device(encode_storage(make_param(wl, i), wl.storage)) for i in range(n)]
        moms = [to_device(encode_storage(make_momentum(wl, i), "fp32")) for i in range(n)]
        upd = [torch.empty(m.rows, m.cols, dtype=torch.float32, device="cuda") for m in wl.mats]
        hp = hparams_for(wl)
        rec: Dict[int, List[StepRecord]] = {i: [] for i in check}
        gf = grad_fn or make_grad
        for s in range(1, steps + 1):
            g_stored = [encode_storage(gf(wl, s, i), wl.storage) for i in range(n)]
            grads = [to_device(x) for x in g_stored]
            w_old = {i: to_stored(params[i]) for i in check}
            nsm.muon_step(h, params, grads, moms, hp, update_outs=upd, blocks=wl.blocks)
            torch.cuda.synchronize()
            for i in check:
                rec[i].append(StepRecord(w_old[i], to_stored(params[i]), to_stored(moms[i]), to_stored(upd[i]),
                                         g_stored[i]))
        return rec
    finally:
        if own:
            nsm.muon_destroy(h)


def check_against_oracle(wl: Workload, rec: Dict[int, List[StepRecord]], tol_o: float, tol_w_f32: float = 1e-5,
                         report: Optional[list] = None) -> None:
    """Replay every recorded matrix through the oracle from the same initial state
    and the same stored gradients; assert the parity bars."""
    hp = oracle_hyper(wl)
    for i, steps in rec.items():
        m = oracle.decode(encode_storage(make_momentum(wl, i), "fp32"))
        for s, r in enumerate(steps):
            w_old = oracle.decode(r.w_old)
            g = oracle.decode(r.g)
            blk = wl.blocks[i] if wl.blocks is not None else (0, 0)
            if blk == (0, 0):
                res = oracle.muon_step_matrix(w_old, g, m, hp)
            else:
                res = oracle.muon_step_matrix_blocked(w_old, g, m, hp, *blk)
            e_m = relf(r.m_new, res.m)
            e_o = relf(r.o, res.o)
            loc = local_errors(r.o, res.o)
            if report is not None:
                report.append((i, s + 1, e_m, e_o))
            print(f"  matrix {i} {r.w_old.shape} step {s + 1}: mom {e_m:.2e}  O {e_o:.2e}  (tile {loc['tile']:.2e}, "
                  f"row {loc['row']:.2e}, col {loc['col']:.2e})", flush=True)
            assert e_m <= TOL_MOM, f"matrix {i} step {s + 1}: momentum rel err {e_m:.3e}"
            assert e_o <= tol_o, f"matrix {i} step {s + 1}: O rel err {e_o:.3e} > {tol_o}"
            for k, v in loc.items():
                assert v <= tol_o, f"matrix {i} step {s + 1}: O {k} error {v:.3e} > {tol_o}"
            # the stored weight: float64 update of the GPU's own O, rounded once
            sc = shape_scales(r.w_old.shape, blk)
            w_exp = w_old * (1.0 - wl.lr * wl.weight_decay) - wl.lr * sc * r.o.astype(np.float64)
            if r.w_new.dtype == np.uint16:
                ok = weight_error_ok(r.w_new, w_old, r.o.astype(np.float64), wl.lr, wl.weight_decay, sc)
                assert ok.all(), f"matrix {i} step {s + 1}: {int((~ok).sum())} weights beyond 1 bf16 ulp"
            else:
                dw_gpu = r.w_new.astype(np.float64) - w_old
                e_w = relf(dw_gpu, res.w - w_old)
                assert e_w <= max(tol_w_f32, tol_o), f"matrix {i} step {s + 1}: dW rel err {e_w:.3e}"
            m = res.m  # the oracle keeps its own float64 momentum trajectory
