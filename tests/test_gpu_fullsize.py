"""Parity at the full workload sizes, in the launch configuration the benchmark
times: every matrix of a workload goes through one grouped ``muon_step`` call
per step (same plan, tile sizes and kernels as the timed run).

- every matrix, every element: the new momentum against beta * m + g;
- sampled matrices (one of each shape and the extreme cases): the update O
  against the float64 oracle replayed from the same stored inputs, as a whole
  and tile by tile, row by row and column by column, and every stored weight;
- every step of each workload's stated step count (10 for the 350M-style
  set and the head-pair set, 5 for the MoE stack and the large layer share),
  one test per step.

The oracle cannot produce a single element of O without the whole matrix, so
the Newton-Schulz output is compared on whole sampled matrices.
"""

from __future__ import annotations

import math
import time

import numpy as np
import pytest

import oracle
from muon_synth import encode_storage, expert_scale, make_grad, make_momentum, make_param, workload

from gpu_harness import (TOL_O_BF16, assert_o_close, hparams_for, local_errors, oracle_hyper, relf,
                         shape_scales, to_device, to_stored, weight_error_ok)


def _moe_sample():
    wl = workload("moe-64x-2048x1408")
    scales = [expert_scale(wl, e) for e in range(64)]
    lo, hi = int(np.argmin(scales)), int(np.argmax(scales))
    # 2048x1408 of the smallest-scale expert, 1408x2048 of the largest, a shared 2048x2048
    return (2 * lo, 2 * hi + 1, 128)


# workload -> sampled matrix indices (None: chosen from the expert scales)
SAMPLES = {
    "gpt2-350m-hidden": (0, 4, 5, 143),                   # 1024^2, 1024x4096, 4096x1024, last matrix
    "moe-64x-2048x1408": None,
    # 4096x14336, 14336x4096 (transposed, s = 1.871), 4096^2
    "large-layer-share-4096x14336": (1, 2, 9),
    # query and key in six 128x768 blocks (pairs of heads), value and the MLP whole
    "gpt2-124m-hidden-qk-head-pairs": (0, 1, 2, 4, 5, 66),
}
# every step of every workload's stated step count, one test per step
CASES = [(name, s) for name in SAMPLES for s in range(1, workload(name).steps + 1)]


def _momentum_ok(got: np.ndarray, m_old: np.ndarray, g: np.ndarray, beta: float) -> np.ndarray:
    """m' = beta m + g evaluated in float32: within a few float32 roundings."""
    exp = beta * m_old + g
    return np.abs(got - exp) <= 2.0 ** -22 * (np.abs(m_old) + np.abs(g))


class _FullRun:
    """One workload on the GPU in the benchmark's launch configuration (every
    matrix in one grouped call per step; update_out only for the sampled
    matrices), advanced one step at a time, each step checked as it runs:
    every momentum element; for the sampled matrices O against the float64
    oracle (whole matrix, every tile, row and column) and every stored weight."""

    def __init__(self, name: str):
        import torch
        import newton_schulz_matrix_step_amd as nsm
        self.nsm, self.torch = nsm, torch
        self.name = name
        self.wl = wl = workload(name)
        self.n = n = len(wl.mats)
        self.sample = tuple(SAMPLES[name] if SAMPLES[name] is not None else _moe_sample())
        self.hp = hparams_for(wl)
        self.ohp = oracle_hyper(wl)
        self.h = nsm.muon_init(0)
        self.params = [to_device(encode_storage(make_param(wl, i), wl.storage)) for i in range(n)]
        self.moms = [to_device(encode_storage(make_momentum(wl, i), "fp32")) for i in range(n)]
        self.upd = [torch.empty(s.rows, s.cols, dtype=torch.float32, device="cuda") if i in self.sample else None
                    for i, s in enumerate(wl.mats)]
        self.m_oracle = {i: oracle.decode(encode_storage(make_momentum(wl, i), "fp32")) for i in self.sample}
        self.done = 0
        self.worst = 0.0

    def close(self):
        if self.h:
            self.nsm.muon_destroy(self.h)
            self.h = None
        self.params = self.moms = self.upd = None

    def step(self):
        torch, nsm, wl, name, n = self.torch, self.nsm, self.wl, self.name, self.n
        s = self.done + 1
        t0 = time.perf_counter()
        g_st = [encode_storage(make_grad(wl, s, i), wl.storage) for i in range(n)]
        grads = [to_device(x) for x in g_st]
        m_old = [to_stored(m) for m in self.moms]
        w_old = {i: to_stored(self.params[i]) for i in self.sample}
        print(f"{name} step {s}: inputs ready in {time.perf_counter() - t0:.1f} s", flush=True)
        nsm.muon_step(self.h, self.params, grads, self.moms, self.hp, update_outs=self.upd, blocks=wl.blocks)
        torch.cuda.synchronize()
        for i in range(n):
            got = to_stored(self.moms[i]).astype(np.float64)
            ok = _momentum_ok(got, m_old[i].astype(np.float64), oracle.decode(g_st[i]), wl.beta)
            assert ok.all(), f"{name} matrix {i} step {s}: {int((~ok).sum())} momentum elements off"
        self.done = s   # the GPU state has advanced even if a check below fails
        for i in self.sample:
            t1 = time.perf_counter()
            w0 = oracle.decode(w_old[i])
            blk = wl.blocks[i] if wl.blocks is not None else (0, 0)
            if blk == (0, 0):
                res = oracle.muon_step_matrix(w0, oracle.decode(g_st[i]), self.m_oracle[i], self.ohp)
            else:
                res = oracle.muon_step_matrix_blocked(w0, oracle.decode(g_st[i]), self.m_oracle[i], self.ohp, *blk)
            self.m_oracle[i] = res.m
            o_gpu = to_stored(self.upd[i]).astype(np.float64)
            shape = wl.mats[i].rows, wl.mats[i].cols
            e = {"global": relf(o_gpu, res.o), **local_errors(o_gpu, res.o)}
            self.worst = max(self.worst, *e.values())
            print(f"  matrix {i} {shape} step {s}: O rel err {e['global']:.3e} (tile {e['tile']:.3e}, row "
                  f"{e['row']:.3e}, col {e['col']:.3e}; oracle {time.perf_counter() - t1:.1f} s)", flush=True)
            for k, v in e.items():
                assert v <= TOL_O_BF16, f"{name} matrix {i} step {s}: O {k} error {v:.3e} > {TOL_O_BF16}"
            sc = shape_scales(shape, blk)
            ok = weight_error_ok(to_stored(self.params[i]), w0, o_gpu, wl.lr, wl.weight_decay, sc)
            assert ok.all(), f"{name} matrix {i} step {s}: {int((~ok).sum())} weights beyond 1 bf16 ulp"
        del grads


_RUNS = {}


@pytest.mark.gpu
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,step", CASES, ids=[f"{c[0]}-step{c[1]}" for c in CASES])
def test_full_size_workload(name, step):
    """Step ``step`` of the workload's stated step count, on the state the
    earlier steps left (run first when this case is selected alone)."""
    run = _RUNS.get(name)
    if run is None or run.done >= step:
        if run is not None:
            run.close()
        run = _RUNS[name] = _FullRun(name)
    try:
        while run.done < step:
            run.step()
    except BaseException:
        run.close()
        _RUNS.pop(name, None)
        raise
    if step == run.wl.steps:
        print(f"{name}: worst O error over {step} steps and the sampled matrices: {run.worst:.3e}", flush=True)
        run.close()
        _RUNS.pop(name, None)


@pytest.mark.gpu
def test_extreme_aspect_ratios():
    """Very long K (8 x 131072 Gram products), a single row, tall thin
    matrices, grouped with an ordinary square one."""
    import torch
    import newton_schulz_matrix_step_amd as nsm

    shapes = [(8, 131072), (131072, 8), (1, 65536), (65536, 3), (512, 512)]
    wl = workload("gpt2-124m-hidden")
    from muon_synth.gen import MatSpec
    wl = wl.with_(mats=tuple(MatSpec(r, c, f"x{i}") for i, (r, c) in enumerate(shapes)), steps=1)
    hp = hparams_for(wl)
    ohp = oracle_hyper(wl)
    h = nsm.muon_init(0)
    try:
        n = len(shapes)
        w_st = [encode_storage(make_param(wl, i), "bf16") for i in range(n)]
        g_st = [encode_storage(make_grad(wl, 1, i), "bf16") for i in range(n)]
        params = [to_device(x) for x in w_st]
        grads = [to_device(x) for x in g_st]
        moms = [torch.zeros(r, c, dtype=torch.float32, device="cuda") for r, c in shapes]
        upd = [torch.empty(r, c, dtype=torch.float32, device="cuda") for r, c in shapes]
        nsm.muon_step(h, params, grads, moms, hp, update_outs=upd)
        torch.cuda.synchronize()
        for i, (r, c) in enumerate(shapes):
            w0 = oracle.decode(w_st[i])
            res = oracle.muon_step_matrix(w0, oracle.decode(g_st[i]), np.zeros((r, c)), ohp)
            o_gpu = to_stored(upd[i]).astype(np.float64)
            e = assert_o_close(o_gpu, res.o, TOL_O_BF16, f"{r}x{c}")
            print(f"  {r}x{c}: O errors {e}", flush=True)
            sc = math.sqrt(max(1.0, r / c))
            ok = weight_error_ok(to_stored(params[i]), w0, o_gpu, wl.lr, wl.weight_decay, sc)
            assert ok.all(), f"{r}x{c}: {int((~ok).sum())} weights beyond 1 bf16 ulp"
    finally:
        nsm.muon_destroy(h)


@pytest.mark.gpu
def test_maximum_dimension_vectors():
    """The largest accepted dimension (2^20) as a single row and as a single
    column, grouped in one call, plus the rejection of one more."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    from muon_synth.gen import MatSpec

    big = 1 << 20
    shapes = [(1, big), (big, 1)]
    wl = workload("gpt2-124m-hidden")
    wl = wl.with_(mats=tuple(MatSpec(r, c, f"v{i}") for i, (r, c) in enumerate(shapes)), steps=1, wid=77)
    hp = hparams_for(wl)
    ohp = oracle_hyper(wl)
    h = nsm.muon_init(0)
    try:
        w_st = [encode_storage(make_param(wl, i), "bf16") for i in range(2)]
        g_st = [encode_storage(make_grad(wl, 1, i), "bf16") for i in range(2)]
        params = [to_device(x) for x in w_st]
        grads = [to_device(x) for x in g_st]
        moms = [torch.zeros(r, c, dtype=torch.float32, device="cuda") for r, c in shapes]
        upd = [torch.empty(r, c, dtype=torch.float32, device="cuda") for r, c in shapes]
        nsm.muon_step(h, params, grads, moms, hp, update_outs=upd)
        torch.cuda.synchronize()
        for i, (r, c) in enumerate(shapes):
            w0 = oracle.decode(w_st[i])
            res = oracle.muon_step_matrix(w0, oracle.decode(g_st[i]), np.zeros((r, c)), ohp)
            o_gpu = to_stored(upd[i]).astype(np.float64)
            e = assert_o_close(o_gpu, res.o, TOL_O_BF16, f"{r}x{c}")
            print(f"  {r}x{c}: O errors {e}", flush=True)
            sc = math.sqrt(max(1.0, r / c))
            ok = weight_error_ok(to_stored(params[i]), w0, o_gpu, wl.lr, wl.weight_decay, sc)
            assert ok.all()
        # one more than the largest dimension is rejected before any work
        g = torch.ones(1, big + 1, dtype=torch.bfloat16, device="cuda")
        w = torch.zeros_like(g)
        m = torch.zeros(1, big + 1, device="cuda")
        with pytest.raises(nsm.MuonError) as ei:
            nsm.muon_step(h, [w], [g], [m], hp)
        assert ei.value.status == nsm.MUON_ERR_INVALID_ARG
        torch.cuda.synchronize()
        assert float(w.float().abs().max()) == 0.0 and float(m.abs().max()) == 0.0
    finally:
        nsm.muon_destroy(h)
