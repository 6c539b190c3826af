"""muon_step_noalloc (no device allocation; static per-GPU scratch) against
muon_step through the C ABI: two calls in a row, the second with a smaller
input, each bitwise equal to muon_step on the same inputs (same kernels, same
layout) and within the oracle's bar; a call too large for the scratch is
refused before anything runs."""

import numpy as np
import pytest

import oracle
from gpu_harness import TOL_O_BF16, assert_o_close, to_device, to_stored
from muon_synth import encode_storage, lowrank_noise_grad, rng_for

pytestmark = pytest.mark.gpu


def _inputs(shapes, seed):
    w = [encode_storage(rng_for(seed, 0, i, 0).standard_normal(s) * 0.02, "bf16") for i, s in enumerate(shapes)]
    g = [encode_storage(lowrank_noise_grad(rng_for(seed, 1, i, 1), *s), "bf16") for i, s in enumerate(shapes)]
    m = [rng_for(seed, 0, i, 2).standard_normal(s).astype(np.float32) * 0.01 for i, s in enumerate(shapes)]
    return w, g, m


def _twin_step(nsm, torch, h_plain, h_static, shapes, seed, hp):
    w, g, m = _inputs(shapes, seed)
    ga = [to_device(x) for x in g]
    runs = {}
    for name, h, fn in (("plain", h_plain, nsm.muon_step), ("static", h_static, nsm.muon_step_noalloc)):
        ws = [to_device(x) for x in w]
        ms = [to_device(x) for x in m]
        os_ = [torch.empty(s, device="cuda") for s in shapes]
        fn(h, ws, ga, ms, hp, update_outs=os_)
        torch.cuda.synchronize()
        runs[name] = (ws, ms, os_)
    for i in range(len(shapes)):
        for a, b in zip((runs["plain"][k][i] for k in range(3)), (runs["static"][k][i] for k in range(3))):
            assert torch.equal(a, b), f"{shapes[i]}: no-alloc result differs from muon_step"
    hyper = oracle.Hyper(lr=hp.lr, beta=hp.beta, weight_decay=hp.weight_decay, nesterov=hp.nesterov)
    for i, s in enumerate(shapes):
        ref = oracle.muon_step_matrix(oracle.decode(w[i]), oracle.decode(g[i]), m[i].astype(np.float64), hyper)
        e = assert_o_close(to_stored(runs["static"][2][i]).astype(np.float64), ref.o, TOL_O_BF16, f"{s}")
        print(f"  {s}: O errors {e}", flush=True)


def test_noalloc_matches_muon_step_on_two_calls():
    import torch
    import newton_schulz_matrix_step_amd as nsm
    hp = nsm.Hparams(nesterov=True, weight_decay=0.01)
    h_plain, h_static = nsm.muon_init(0), nsm.muon_init(0)
    try:
        big = [(512, 768), (768, 512), (300, 100), (48, 40), (256, 256)]
        small = [(96, 160), (17, 1)]
        _twin_step(nsm, torch, h_plain, h_static, big, 71, hp)
        print("first call (5 matrices) bitwise equal to muon_step", flush=True)
        _twin_step(nsm, torch, h_plain, h_static, small, 72, hp)
        print("second, smaller call (2 matrices) bitwise equal to muon_step", flush=True)
        assert nsm.muon_workspace_bytes(h_static) == 0   # the no-alloc handle holds no plan
    finally:
        nsm.muon_destroy(h_plain)
        nsm.muon_destroy(h_static)


def test_noalloc_wide_tiles_on_two_calls():
    """Large matrices, whose GRAM and AXPY run on 256-wide tiles, through the
    static scratch: a call of two 1024 x 2048 / 2048 x 1024 matrices, then a
    smaller one, each bitwise equal to muon_step."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    hp = nsm.Hparams()
    h_plain, h_static = nsm.muon_init(0), nsm.muon_init(0)
    try:
        _twin_step(nsm, torch, h_plain, h_static, [(1024, 2048), (2048, 1024)], 73, hp)
        _twin_step(nsm, torch, h_plain, h_static, [(1024, 1024), (300, 100)], 74, hp)
    finally:
        nsm.muon_destroy(h_plain)
        nsm.muon_destroy(h_static)


def test_noalloc_refuses_calls_beyond_the_scratch():
    import torch
    import newton_schulz_matrix_step_amd as nsm
    h = nsm.muon_init(0)
    try:
        # 8192 x 8192 in bf16 needs ~7 bytes an element of workspace: ~450 MiB > 256 MiB
        g = torch.ones(8192, 8192, dtype=torch.bfloat16, device="cuda")
        w = torch.zeros_like(g)
        m = torch.zeros(8192, 8192, device="cuda")
        with pytest.raises(nsm.MuonError) as ei:
            nsm.muon_step_noalloc(h, [w], [g], [m], nsm.Hparams())
        assert ei.value.status == nsm.MUON_ERR_INVALID_ARG
        assert "scratch" in str(ei.value)
        torch.cuda.synchronize()
        assert float(w.float().abs().max()) == 0.0 and float(m.abs().max()) == 0.0
    finally:
        nsm.muon_destroy(h)
