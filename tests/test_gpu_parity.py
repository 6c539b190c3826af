"""GPU parity: the HIP path through the C ABI against the float64 oracle on the
same seeded stored inputs.

Bars: O (update_out) rel-F <= 3e-2 in bf16 mode and <= 1e-5 in fp32 mode on the
64x128 case; momentum rel-F <= 1e-6 at every step; stored bf16 weights within
1 ulp of the float64 update of the GPU's own O rounded once (fp32 weights:
rel-F of the weight change).
"""

import numpy as np
import pytest

from muon_synth import MatSpec, workload
from gpu_harness import (TOL_O_BF16, TOL_O_FP32, assert_o_close, check_against_oracle, relf, run_gpu,
                         to_device, to_stored)
import oracle

pytestmark = pytest.mark.gpu


def _wl(name, shapes, **kw):
    base = workload("gpt2-124m-hidden")
    mats = tuple(MatSpec(r, c, f"m{i}") for i, (r, c) in enumerate(shapes))
    return base.with_(name=name, wid=100 + len(shapes), mats=mats, **kw)


def test_single_64x128_fp32_workload():
    wl = workload("single-64x128-fp32")
    rep = []
    rec = run_gpu(wl, wl.steps, [0])
    check_against_oracle(wl, rec, TOL_O_FP32, report=rep)
    print("64x128 fp32:", rep)


@pytest.mark.parametrize("shape", [(64, 128), (128, 64), (100, 300), (300, 100), (129, 257), (256, 256), (1, 1),
                                   (1, 40), (40, 1), (3, 5)])
def test_fp32_mode_ragged(shape):
    wl = workload("single-64x128-fp32").with_(mats=(MatSpec(*shape, "r"),), wid=200 + shape[0] + 7 * shape[1])
    rep = []
    rec = run_gpu(wl, 2, [0])
    # ragged shapes run the same arithmetic; the folding quintic amplifies fp32
    # rounding with size, so only the 64x128 case carries the 1e-5 bar
    check_against_oracle(wl, rec, 1e-4, tol_w_f32=1e-4, report=rep)
    print(shape, [f"{e:.2e}" for (_, _, _, e) in rep])


@pytest.mark.parametrize("nesterov,wd", [(False, 0.0), (True, 0.01)])
def test_bf16_grouped_mixed_shapes(nesterov, wd):
    shapes = [(300, 100), (100, 300), (256, 256), (129, 515), (515, 129), (64, 64), (1, 17), (17, 1), (200, 199)]
    wl = _wl("mixed", shapes, nesterov=nesterov, weight_decay=wd, steps=3)
    rep = []
    rec = run_gpu(wl, 3, list(range(len(shapes))))
    check_against_oracle(wl, rec, TOL_O_BF16, report=rep)
    worst = max(e for (_, _, _, e) in rep)
    print("mixed worst O rel err", worst)


def test_timed_path_matches_checked_path_bitwise():
    """The benchmark calls muon_step without update_out, so the last
    iteration's epilogue writes the weight only (its own compile-time
    variant); every oracle-checked run passes update_out.  The full GPT-2
    124M set, three steps on two handles, one call with update_out for every
    matrix and one without: weights and momenta must agree bit for bit at every
    step, so the checked path vouches for the timed one."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    from gpu_harness import hparams_for
    from muon_synth import encode_storage, make_grad, make_momentum, make_param
    wl = workload("gpt2-124m-hidden")
    n = len(wl.mats)
    hp = hparams_for(wl)
    w_a = [to_device(encode_storage(make_param(wl, i), wl.storage)) for i in range(n)]
    m_a = [to_device(encode_storage(make_momentum(wl, i), "fp32")) for i in range(n)]
    w_b = [w.clone() for w in w_a]
    m_b = [m.clone() for m in m_a]
    upd = [torch.empty(s.rows, s.cols, device="cuda") for s in wl.mats]
    h_a, h_b = nsm.muon_init(0), nsm.muon_init(0)
    try:
        for s in range(1, 4):
            grads = [to_device(encode_storage(make_grad(wl, s, i), wl.storage)) for i in range(n)]
            nsm.muon_step(h_a, w_a, grads, m_a, hp, update_outs=upd)
            nsm.muon_step(h_b, w_b, grads, m_b, hp)
            torch.cuda.synchronize()
            for i in range(n):
                assert torch.equal(w_a[i], w_b[i]), f"step {s}: weights of matrix {i} differ"
                assert torch.equal(m_a[i], m_b[i]), f"step {s}: momentum of matrix {i} differs"
            print(f"step {s}: {n} weights and momenta bitwise equal", flush=True)
    finally:
        nsm.muon_destroy(h_a)
        nsm.muon_destroy(h_b)


def test_gpt2_124m_hidden_workload_sampled():
    """The 72-matrix GPT-2 small set, all 10 steps, one grouped call per step;
    the oracle replays two matrices of each shape class."""
    wl = workload("gpt2-124m-hidden")
    check = [0, 3, 4, 5, 64, 71]
    rep = []
    rec = run_gpu(wl, wl.steps, check)
    check_against_oracle(wl, rec, TOL_O_BF16, report=rep)
    print("gpt2-124m worst O rel err", max(e for (_, _, _, e) in rep), "worst mom", max(e for (_, _, e, _) in rep))


@pytest.mark.parametrize("ns_steps,nesterov", [(0, False), (1, False), (2, False), (0, True), (1, True)])
def test_ns_step_counts(ns_steps, nesterov):
    wl = _wl("steps", [(96, 160), (160, 96)], ns_steps=ns_steps, steps=2, nesterov=nesterov, weight_decay=0.02)
    rec = run_gpu(wl, 2, [0, 1])
    check_against_oracle(wl, rec, TOL_O_BF16)


def test_zero_gradient_and_zero_lr():
    import torch
    import newton_schulz_matrix_step_amd as nsm
    h = nsm.muon_init(0)
    try:
        w = torch.randn(70, 90, device="cuda").to(torch.bfloat16)
        w0 = w.clone()
        g = torch.zeros_like(w)
        m = torch.zeros(70, 90, device="cuda")
        o = torch.full((70, 90), 7.0, device="cuda")
        nsm.muon_step(h, [w], [g], [m], nsm.Hparams(lr=0.02, weight_decay=0.5), update_outs=[o])
        torch.cuda.synchronize()
        assert torch.count_nonzero(o).item() == 0
        from gpu_harness import weight_error_ok
        w0_64 = (to_stored(w0).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert weight_error_ok(to_stored(w), w0_64, np.zeros_like(w0_64), 0.02, 0.5, 1.0).all()
        g2 = torch.randn(70, 90, device="cuda").to(torch.bfloat16)
        w1 = w.clone()
        nsm.muon_step(h, [w], [g2], [m], nsm.Hparams(lr=0.0, weight_decay=0.5))
        torch.cuda.synchronize()
        assert torch.equal(w, w1)
    finally:
        nsm.muon_destroy(h)


def test_strided_views_and_unaligned_columns():
    """Leading dimensions larger than cols (views into wider buffers) and odd
    column counts (no vector path)."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    rng = np.random.default_rng(3)
    h = nsm.muon_init(0)
    try:
        for (r, c, ld) in ((50, 77, 80), (120, 40, 48), (33, 64, 72)):
            big_w = torch.from_numpy(rng.standard_normal((r, ld)).astype(np.float32) * 0.02).cuda()
            big_g = torch.from_numpy(rng.standard_normal((r, ld)).astype(np.float32) * 0.02).cuda()
            big_m = torch.zeros(r, ld + 8, device="cuda")
            w, g, m = big_w[:, :c], big_g[:, :c], big_m[:, :c]
            w0, g0 = w.double().cpu().numpy(), g.double().cpu().numpy()
            o = torch.empty(r, c, device="cuda")
            hp = nsm.Hparams(compute="fp32", nesterov=True, weight_decay=0.1)
            nsm.muon_step(h, [w], [g], [m], hp, update_outs=[o])
            torch.cuda.synchronize()
            ref = oracle.muon_step_matrix(w0, g0, np.zeros((r, c)), oracle.Hyper(nesterov=True, weight_decay=0.1))
            assert_o_close(o.cpu().numpy(), ref.o, 1e-4, f"{r}x{c} in ld {ld}")
            assert relf(m.cpu().numpy(), ref.m) <= 1e-6
            assert relf(w.double().cpu().numpy() - w0, ref.w - w0) <= 1e-4
            # the columns outside the views are untouched
            assert torch.count_nonzero(big_m[:, c:]).item() == 0
    finally:
        nsm.muon_destroy(h)


@pytest.mark.parametrize("compute,tol", [("bf16", TOL_O_BF16), ("fp32", 1e-4)])
@pytest.mark.parametrize("shape", [(64, 128), (300, 100), (257, 513)])
def test_orthogonalize_entry_point(compute, tol, shape):
    import torch
    import newton_schulz_matrix_step_amd as nsm
    from muon_synth import lowrank_noise_grad, rng_for, encode_storage
    g = lowrank_noise_grad(rng_for(7, 0, shape[0], 1), *shape)
    for storage in ("bf16", "fp32"):
        st = encode_storage(g, storage)
        x = to_device(st)
        out = torch.empty(shape, device="cuda")
        h = nsm.muon_init(0)
        try:
            nsm.muon_orthogonalize(h, x, out, nsm.Hparams(compute=compute))
            torch.cuda.synchronize()
        finally:
            nsm.muon_destroy(h)
        ref = oracle.newton_schulz(oracle.decode(st))
        assert_o_close(out.cpu().numpy(), ref, tol, f"{shape} {storage} input, {compute}")


def test_determinism_bitwise():
    wl = _wl("det", [(300, 100), (128, 384)], steps=2, nesterov=True)
    a = run_gpu(wl, 2, [0, 1])
    b = run_gpu(wl, 2, [0, 1])
    for i in (0, 1):
        for ra, rb in zip(a[i], b[i]):
            assert np.array_equal(ra.o, rb.o) and np.array_equal(ra.w_new, rb.w_new) and np.array_equal(ra.m_new, rb.m_new)


def test_norm_readback():
    import torch
    import newton_schulz_matrix_step_amd as nsm
    h = nsm.muon_init(0)
    try:
        g = torch.randn(40, 60, device="cuda")
        w = torch.zeros_like(g)
        m = torch.zeros_like(g)
        nsm.muon_step(h, [w], [g], [m], nsm.Hparams(compute="fp32"))
        nu = nsm.muon_read_norms(h, 1)
        assert nu[0] == pytest.approx(float(torch.linalg.norm(g.double())), rel=1e-6)
    finally:
        nsm.muon_destroy(h)


# per-iteration coefficient schedules: assorted triples (the first is the
# default quintic, the last a plain cubic step) and the default one repeated
MIXED_SCHEDULE = ((3.4445, -4.7750, 2.0315), (2.0, -1.5, 0.5), (1.875, -1.25, 0.375), (3.0, -3.2, 1.2),
                  (1.5, -0.5, 0.0))


@pytest.mark.parametrize("compute,tol", [("bf16", TOL_O_BF16), ("fp32", 1e-4)])
def test_coefficient_schedule(compute, tol):
    shapes = [(300, 100), (100, 300), (256, 256), (129, 515), (64, 64), (17, 1)]
    wl = _wl("sched", shapes, steps=2, nesterov=True, compute=compute, coeffs=MIXED_SCHEDULE)
    rep = []
    rec = run_gpu(wl, 2, list(range(len(shapes))))
    check_against_oracle(wl, rec, tol, tol_w_f32=tol, report=rep)
    print(compute, "schedule worst O rel err", max(e for (_, _, _, e) in rep))


def test_uniform_schedule_matches_default_bitwise():
    wl = _wl("uni", [(300, 100), (128, 384)], steps=2)
    a = run_gpu(wl, 2, [0, 1])
    b = run_gpu(wl.with_(coeffs=((wl.a, wl.b, wl.c),) * wl.ns_steps), 2, [0, 1])
    for i in (0, 1):
        for ra, rb in zip(a[i], b[i]):
            assert np.array_equal(ra.o, rb.o) and np.array_equal(ra.w_new, rb.w_new)


@pytest.mark.parametrize("bad", [(0.0, -1.0, 0.5), (float("nan"), 1.0, 1.0), (1.0, float("inf"), 0.0)])
def test_invalid_schedule_rejected(bad):
    import torch
    import newton_schulz_matrix_step_amd as nsm
    h = nsm.muon_init(0)
    try:
        g = torch.randn(40, 60, device="cuda")
        w = torch.zeros_like(g)
        m = torch.zeros_like(g)
        sched = [(3.4445, -4.7750, 2.0315)] * 4 + [bad]
        with pytest.raises(nsm.MuonError) as ei:
            nsm.muon_step(h, [w], [g], [m], nsm.Hparams(coeffs=sched))
        assert ei.value.status == nsm.MUON_ERR_INVALID_ARG
        assert float(w.abs().max()) == 0.0 and float(m.abs().max()) == 0.0   # nothing ran
    finally:
        nsm.muon_destroy(h)


# sub-block orthogonalisation: query/key style weights cut into pairs of heads
BLOCK_SHAPES = [(768, 768), (2304, 768), (192, 160), (130, 60), (300, 100)]
BLOCKS = ((128, 0), (128, 0), (64, 80), (65, 0), (0, 0))


@pytest.mark.parametrize("compute,tol", [("bf16", TOL_O_BF16), ("fp32", 1e-4)])
def test_blocked_orthogonalisation(compute, tol):
    wl = _wl("blocked", BLOCK_SHAPES, steps=2, nesterov=True, weight_decay=0.01, compute=compute, blocks=BLOCKS)
    rep = []
    rec = run_gpu(wl, 2, list(range(len(BLOCK_SHAPES))))
    check_against_oracle(wl, rec, tol, tol_w_f32=tol, report=rep)
    print(compute, "blocked worst O rel err", max(e for (_, _, _, e) in rep))


def test_blocked_norms_and_whole_block_bitwise():
    """Norm readback has one entry per block; a block covering the whole matrix
    is the plain step, bit for bit."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    wl = _wl("wholeblk", [(300, 100), (128, 384)], steps=1)
    a = run_gpu(wl, 1, [0, 1])
    b = run_gpu(wl.with_(blocks=((300, 100), (128, 384))), 1, [0, 1])
    for i in (0, 1):
        assert np.array_equal(a[i][0].o, b[i][0].o) and np.array_equal(a[i][0].w_new, b[i][0].w_new)
    h = nsm.muon_init(0)
    try:
        g = torch.randn(256, 96, device="cuda")
        w, m = torch.zeros_like(g), torch.zeros_like(g)
        nsm.muon_step(h, [w, torch.zeros(8, 8, device="cuda")], [g, torch.ones(8, 8, device="cuda")],
                      [m, torch.zeros(8, 8, device="cuda")], nsm.Hparams(compute="fp32"), blocks=[(64, 48), (0, 0)])
        nu = nsm.muon_read_norms(h, 9)
        gd = g.double().cpu()
        expect = [float(torch.linalg.norm(gd[r:r + 64, c:c + 48])) for r in range(0, 256, 64) for c in (0, 48)]
        assert nu[:8] == pytest.approx(expect, rel=1e-6)
        assert nu[8] == pytest.approx(8.0, rel=1e-6)
    finally:
        nsm.muon_destroy(h)


@pytest.mark.parametrize("block", [(3, 0), (0, 5), (-1, 0), (20, 0), (1, 1)])
def test_invalid_block_rejected(block):
    import torch
    import newton_schulz_matrix_step_amd as nsm
    shape = (300, 300) if block == (1, 1) else (10, 12)     # (1, 1) blocks: 90000 entries, over the limit
    h = nsm.muon_init(0)
    try:
        g = torch.randn(*shape, device="cuda")
        w, m = torch.zeros_like(g), torch.zeros_like(g)
        with pytest.raises(nsm.MuonError) as ei:
            nsm.muon_step(h, [w], [g], [m], nsm.Hparams(), blocks=[block])
        assert ei.value.status == nsm.MUON_ERR_INVALID_ARG
        assert float(w.abs().max()) == 0.0 and float(m.abs().max()) == 0.0
    finally:
        nsm.muon_destroy(h)


def test_all_options_together():
    """Blocks, a coefficient schedule, Nesterov, weight decay and float32
    storage in one grouped call with plain matrices."""
    shapes = [(256, 192), (192, 640), (130, 60), (77, 33)]
    blocks = ((64, 0), (0, 128), (65, 0), (0, 0))
    wl = _wl("allopts", shapes, steps=2, nesterov=True, weight_decay=0.05, storage="fp32",
             coeffs=MIXED_SCHEDULE, blocks=blocks)
    rep = []
    rec = run_gpu(wl, 2, list(range(len(shapes))))
    check_against_oracle(wl, rec, TOL_O_BF16, report=rep)
    print("all options worst O rel err", max(e for (_, _, _, e) in rep))


def _phi5_scalar(x, a=3.4445, b=-4.7750, c=2.0315):
    """Five applications of the scalar quintic a x + b x^3 + c x^5 (pure Python)."""
    for _ in range(5):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


@pytest.mark.parametrize("compute", ["fp32", "bf16"])
def test_degenerate_inputs_against_closed_forms(compute):
    """Independent of the oracle.

    Rank one: u v^T comes out as phi_5(s/(s+eps)) u v^T / s (s = |u||v|).  The
    coefficient along u v^T must match (fp32 1e-6, bf16 1e-3 relative); the
    whole matrix carries the rounding noise of the null space, which every
    finite-precision Newton-Schulz amplifies by the quintic's slope at 0
    (3.4445 an iteration, ~486 over five): fp32 bar 5e-4 (measured 1.4e-4),
    bf16 the usual 3e-2 (measured 2.9e-3).
    Orthonormal rows scaled by c (64 x 640 and its transpose): phi_5(c/(c
    sqrt(64) + eps)) times the input over c; full rank, so the usual bars
    (fp32 1e-5, measured 4.7e-7; bf16 3e-2, measured 1.5e-2).
    """
    import torch
    import newton_schulz_matrix_step_amd as nsm
    rng = np.random.default_rng(21)
    fp32 = compute == "fp32"

    def ortho(g):
        gin = torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)).cuda()
        out = torch.empty_like(gin)
        nsm.muon_orthogonalize(h, gin, out, nsm.Hparams(compute=compute))
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64)

    h = nsm.muon_init(0)
    try:
        u, v = rng.standard_normal(256), rng.standard_normal(384)
        g = np.outer(u, v) * 1e-3
        s = np.linalg.norm(g)
        k = _phi5_scalar(s / (s + 1e-7))
        o = ortho(g)
        coef = float(np.sum(o * g) / s)
        err = relf(o, k * g / s)
        print(compute, "rank one: coefficient", coef, "closed form", k, f"matrix rel err {err:.2e}")
        assert abs(coef - k) <= (1e-6 if fp32 else 1e-3) * k
        assert err <= (5e-4 if fp32 else TOL_O_BF16)
        q, _ = np.linalg.qr(rng.standard_normal((640, 64)))
        g = np.ascontiguousarray(q.T) * 0.05
        k = _phi5_scalar(0.05 / (0.05 * 8.0 + 1e-7))
        for gi in (g, np.ascontiguousarray(g.T)):
            err = relf(ortho(gi), k * gi / 0.05)
            print(compute, "orthonormal", gi.shape, f"rel err {err:.2e}")
            assert err <= (TOL_O_FP32 if fp32 else TOL_O_BF16)
    finally:
        nsm.muon_destroy(h)


def test_save_reload_continue_is_bitwise_unbroken():
    """Four steps in one run against two steps, a save of weights and momenta to
    host memory, a reload into fresh buffers on a fresh handle and two more
    steps: the library keeps no state between steps beyond its plan, so the
    two must agree bit for bit."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    from muon_synth import make_grad, make_momentum, make_param, encode_storage
    wl = _wl("resume", [(300, 100), (128, 384), (96, 96)], steps=4, nesterov=True, weight_decay=0.02)
    n = len(wl.mats)
    hp = nsm.Hparams(lr=wl.lr, weight_decay=wl.weight_decay, nesterov=True)
    grads = {s: [to_device(encode_storage(make_grad(wl, s, i), "bf16")) for i in range(n)] for s in range(1, 5)}

    def fresh():
        return ([to_device(encode_storage(make_param(wl, i), "bf16")) for i in range(n)],
                [to_device(encode_storage(make_momentum(wl, i), "fp32")) for i in range(n)])

    def steps(h, ws, ms, s0, s1):
        for s in range(s0, s1 + 1):
            nsm.muon_step(h, ws, grads[s], ms, hp)
        torch.cuda.synchronize()

    h = nsm.muon_init(0)
    try:
        w_a, m_a = fresh()
        steps(h, w_a, m_a, 1, 4)
    finally:
        nsm.muon_destroy(h)
    h = nsm.muon_init(0)
    try:
        w_b, m_b = fresh()
        steps(h, w_b, m_b, 1, 2)
        saved = [(to_stored(w), m.cpu().numpy().copy()) for w, m in zip(w_b, m_b)]
    finally:
        nsm.muon_destroy(h)
    del w_b, m_b
    h = nsm.muon_init(0)
    try:
        w_c = [to_device(w) for w, _ in saved]
        m_c = [to_device(m) for _, m in saved]
        steps(h, w_c, m_c, 3, 4)
    finally:
        nsm.muon_destroy(h)
    for i in range(n):
        assert np.array_equal(to_stored(w_a[i]), to_stored(w_c[i]))
        assert np.array_equal(m_a[i].cpu().numpy(), m_c[i].cpu().numpy())


def test_debug_guard_bands():
    """A handle created with MUON_INIT_DEBUG puts a guard band after every
    workspace buffer and checks all of them after each step: over mixed
    shapes (float32 small entries, bf16 ones, transposed, blocked) and three
    steps no band is touched, and the results equal a plain handle's bit for
    bit (the bands only move buffers apart)."""
    wl = _wl("guards", [(300, 100), (128, 384), (96, 96), (48, 40), (17, 1), (256, 256)], steps=3, nesterov=True,
             weight_decay=0.01, blocks=((0, 0), (64, 0), (0, 0), (0, 0), (0, 0), (128, 128)))
    import newton_schulz_matrix_step_amd as nsm
    h = nsm.muon_init(0, nsm.MUON_INIT_DEBUG)
    try:
        a = run_gpu(wl, 3, list(range(6)), handle=h)
    finally:
        nsm.muon_destroy(h)
    b = run_gpu(wl, 3, list(range(6)))
    for i in range(6):
        for ra, rb in zip(a[i], b[i]):
            assert np.array_equal(ra.o, rb.o) and np.array_equal(ra.w_new, rb.w_new) and np.array_equal(ra.m_new, rb.m_new)


def test_forced_allocation_failure():
    """A handle created with MUON_INIT_FAIL_ALLOC fails every workspace or plan
    allocation: both entry points report MUON_ERR_OOM and change nothing."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    h = nsm.muon_init(0, nsm.MUON_INIT_FAIL_ALLOC)
    try:
        g = torch.randn(64, 96, device="cuda")
        w, m = torch.zeros_like(g), torch.zeros_like(g)
        with pytest.raises(nsm.MuonError) as ei:
            nsm.muon_step(h, [w], [g], [m], nsm.Hparams())
        assert ei.value.status == nsm.MUON_ERR_OOM
        p, gv = torch.zeros(1000, device="cuda"), torch.ones(1000, device="cuda")
        mv, vv = torch.zeros(1000, device="cuda"), torch.zeros(1000, device="cuda")
        with pytest.raises(nsm.MuonError) as ei:
            nsm.muon_adamw_step(h, [p], [gv], [mv], [vv], nsm.AdamWHparams())
        assert ei.value.status == nsm.MUON_ERR_OOM
        torch.cuda.synchronize()
        assert float(w.abs().max()) == 0.0 and float(m.abs().max()) == 0.0
        assert float(p.abs().max()) == 0.0 and float(mv.abs().max()) == 0.0
        assert nsm.muon_workspace_bytes(h) == 0
    finally:
        nsm.muon_destroy(h)


def test_step_captured_in_a_hip_graph():
    """After one eager call (plan built, descriptor table resident), a step
    with the same pointers enqueues kernels only, so it can be captured into
    a HIP graph.  Replays with fresh gradients copied into the captured
    buffers, with eager work and synchronisation between them, match an eager
    twin bit for bit at every step."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    from muon_synth import make_grad, make_param, encode_storage
    wl = _wl("graph", [(300, 100), (128, 384), (96, 96)], steps=5, nesterov=True, weight_decay=0.01)
    n = len(wl.mats)
    hp = nsm.Hparams(lr=wl.lr, weight_decay=wl.weight_decay, nesterov=True)
    grads = {s: [to_device(encode_storage(make_grad(wl, s, i), "bf16")) for i in range(n)] for s in range(1, 6)}
    w0 = [to_device(encode_storage(make_param(wl, i), "bf16")) for i in range(n)]
    h_g, h_e = nsm.muon_init(0), nsm.muon_init(0)
    try:
        # graph side: static buffers
        w_g = [w.clone() for w in w0]
        m_g = [torch.zeros(s.rows, s.cols, device="cuda") for s in wl.mats]
        g_g = [g.clone() for g in grads[1]]
        # eager twin
        w_e = [w.clone() for w in w0]
        m_e = [torch.zeros(s.rows, s.cols, device="cuda") for s in wl.mats]
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            nsm.muon_step(h_g, w_g, g_g, m_g, hp)          # step 1, eager: builds the plan
        torch.cuda.current_stream().wait_stream(stream)
        nsm.muon_step(h_e, w_e, grads[1], m_e, hp)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            nsm.muon_step(h_g, w_g, g_g, m_g, hp)
        torch.cuda.synchronize()
        for s in range(2, 6):
            for i in range(n):
                g_g[i].copy_(grads[s][i])
            graph.replay()
            nsm.muon_step(h_e, w_e, grads[s], m_e, hp)
            junk = torch.randn(1000, device="cuda").sum()   # unrelated eager work between replays
            torch.cuda.synchronize()
            assert torch.isfinite(junk)
            for i in range(n):
                assert torch.equal(w_g[i], w_e[i]), f"replay {s}: weights of matrix {i} differ"
                assert torch.equal(m_g[i], m_e[i]), f"replay {s}: momentum of matrix {i} differs"
    finally:
        nsm.muon_destroy(h_g)
        nsm.muon_destroy(h_e)


def test_profiling_limited_to_chosen_roles():
    import torch
    import newton_schulz_matrix_step_amd as nsm
    g = torch.randn(128, 256, device="cuda")
    for roles, expect in ((["ns_axpy"], {"ns_axpy"}), ([], {"momentum_norm", "norm_finalize", "norm_rescale",
                                                             "ns_gram", "ns_poly", "ns_axpy", "ns_axpy_update"})):
        h = nsm.muon_init(0, nsm.MUON_INIT_PROFILE | nsm.profile_roles(roles))
        try:
            w, m = torch.zeros_like(g), torch.zeros_like(g)
            nsm.muon_step(h, [w], [g], [m], nsm.Hparams())
            torch.cuda.synchronize()
            st = nsm.muon_kernel_stats_read(h)
            assert set(st) == expect, st
            if roles == ["ns_axpy"]:
                assert st["ns_axpy"][0] == 4     # iterations 1-4; the last one is ns_axpy_update
        finally:
            nsm.muon_destroy(h)



def test_thousands_of_tiny_matrices():
    """3000 matrices of 1..48 rows and columns in one grouped call (most of
    them far smaller than one tile), sampled against the oracle."""
    rng = np.random.default_rng(31)
    shapes = [(int(rng.integers(1, 49)), int(rng.integers(1, 49))) for _ in range(3000)]
    wl = _wl("tiny", shapes, steps=2, nesterov=True)
    check = [0, 1, 2, 999, 1500, 2998, 2999] + [i for i, (r, c) in enumerate(shapes) if r == 1 or c == 1][:3]
    rep = []
    rec = run_gpu(wl, 2, check)
    check_against_oracle(wl, rec, TOL_O_BF16, report=rep)
    print("tiny worst O rel err", max(e for (_, _, _, e) in rep))


def test_plan_cache_keeps_every_signature():
    """A handle alternating between two lists of shapes keeps both plans: the
    workspace stops growing after the first sight of each, and every call
    matches a fresh handle running the same list, bit for bit."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    rng = np.random.default_rng(41)
    lists = {"a": [(300, 100), (128, 384)], "b": [(256, 256), (96, 160), (33, 17)]}
    bufs = {}
    for k, shapes in lists.items():
        bufs[k] = ([torch.from_numpy(rng.standard_normal(s).astype(np.float32) * 0.02).cuda().to(torch.bfloat16)
                    for s in shapes],
                   [torch.from_numpy(rng.standard_normal(s).astype(np.float32) * 0.02).cuda().to(torch.bfloat16)
                    for s in shapes])
    hp = nsm.Hparams(nesterov=True, weight_decay=0.01)
    h = nsm.muon_init(0)
    try:
        sizes = []
        state = {k: ([w.clone() for w in bufs[k][0]], [torch.zeros(s, device="cuda") for s in lists[k]])
                 for k in lists}
        twin = {k: ([w.clone() for w in bufs[k][0]], [torch.zeros(s, device="cuda") for s in lists[k]])
                for k in lists}
        for k in ("a", "b", "a", "b", "a"):
            nsm.muon_step(h, state[k][0], bufs[k][1], state[k][1], hp)
            sizes.append(nsm.muon_workspace_bytes(h))
            h2 = nsm.muon_init(0)
            try:
                nsm.muon_step(h2, twin[k][0], bufs[k][1], twin[k][1], hp)
            finally:
                nsm.muon_destroy(h2)
            torch.cuda.synchronize()
            for x, y in zip(state[k][0] + state[k][1], twin[k][0] + twin[k][1]):
                assert torch.equal(x, y)
        print("workspace bytes after each call:", sizes)
        assert sizes[0] > 0 and sizes[1] > sizes[0]
        assert sizes[1:] == [sizes[1]] * 4
    finally:
        nsm.muon_destroy(h)


def _capture(stream, fn):
    """Capture fn() into a HIP graph on ``stream``; returns (graph, fn's exception or None)."""
    import torch
    graph = torch.cuda.CUDAGraph()
    err = None
    side = torch.zeros(4, device="cuda")
    with torch.cuda.graph(graph, stream=stream):
        side.add_(1.0)   # keeps the captured graph non-empty when fn enqueues nothing
        try:
            fn()
        except Exception as e:  # noqa: BLE001 - reported to the caller
            err = e
    return graph, err


def test_capture_refused_without_resident_plan_or_table():
    """Under stream capture a call may only enqueue kernels that read state
    already on the device: a new signature, or known shapes with pointers no
    resident table holds, is refused with MUON_ERR_INVALID_ARG and enqueues
    nothing (the weights stay as they were after replaying the graph)."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    h = nsm.muon_init(0)
    try:
        g = torch.randn(96, 160, device="cuda")
        w, m = torch.zeros_like(g), torch.zeros_like(g)
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        graph, err = _capture(stream, lambda: nsm.muon_step(h, [w], [g], [m], nsm.Hparams(), stream=stream))
        assert isinstance(err, nsm.MuonError) and err.status == nsm.MUON_ERR_INVALID_ARG, err
        graph.replay()
        torch.cuda.synchronize()
        assert float(w.abs().max()) == 0.0 and float(m.abs().max()) == 0.0
        assert nsm.muon_workspace_bytes(h) == 0
        # the plan exists now, but not a table with these new pointers
        with torch.cuda.stream(stream):
            nsm.muon_step(h, [w], [g], [m], nsm.Hparams(), stream=stream)
        torch.cuda.synchronize()
        w2, m2 = torch.zeros_like(g), torch.zeros_like(g)
        graph2, err = _capture(stream, lambda: nsm.muon_step(h, [w2], [g], [m2], nsm.Hparams(), stream=stream))
        assert isinstance(err, nsm.MuonError) and err.status == nsm.MUON_ERR_INVALID_ARG, err
        graph2.replay()
        torch.cuda.synchronize()
        assert float(w2.abs().max()) == 0.0 and float(m2.abs().max()) == 0.0
    finally:
        nsm.muon_destroy(h)


def test_captured_step_keeps_its_buffers():
    """A captured step goes on acting on the buffers it was captured with while
    the handle serves other pointers of the same shapes and other signatures
    in between (each with its own descriptor table and plan, none freed): every
    replay matches an eager twin bit for bit, and the other calls match theirs."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    from muon_synth import encode_storage, make_grad, make_param
    wl = _wl("graph2", [(300, 100), (128, 384)], steps=4, nesterov=True, weight_decay=0.01)
    n = len(wl.mats)
    hp = nsm.Hparams(lr=wl.lr, weight_decay=wl.weight_decay, nesterov=True)
    grads = {s: [to_device(encode_storage(make_grad(wl, s, i), "bf16")) for i in range(n)] for s in range(1, 5)}
    w0 = [to_device(encode_storage(make_param(wl, i), "bf16")) for i in range(n)]
    h, h_twin = nsm.muon_init(0), nsm.muon_init(0)
    try:
        w_g, m_g = [w.clone() for w in w0], [torch.zeros(s.rows, s.cols, device="cuda") for s in wl.mats]
        g_g = [g.clone() for g in grads[1]]
        w_e, m_e = [w.clone() for w in w0], [torch.zeros(s.rows, s.cols, device="cuda") for s in wl.mats]
        w_o, m_o = [w.clone() for w in w0], [torch.zeros(s.rows, s.cols, device="cuda") for s in wl.mats]
        w_ot, m_ot = [w.clone() for w in w0], [torch.zeros(s.rows, s.cols, device="cuda") for s in wl.mats]
        sq = torch.randn(200, 200, device="cuda")
        w_sq, m_sq = torch.zeros_like(sq), torch.zeros_like(sq)
        w_sqt, m_sqt = torch.zeros_like(sq), torch.zeros_like(sq)
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            nsm.muon_step(h, w_g, g_g, m_g, hp, stream=stream)
        nsm.muon_step(h_twin, w_e, grads[1], m_e, hp)
        torch.cuda.synchronize()
        graph, err = _capture(stream, lambda: nsm.muon_step(h, w_g, g_g, m_g, hp, stream=stream))
        assert err is None, err
        for s in range(2, 5):
            # other pointers, same shapes, and another signature, eagerly on the same handle
            with torch.cuda.stream(stream):
                nsm.muon_step(h, w_o, grads[s], m_o, hp, stream=stream)
                nsm.muon_step(h, [w_sq], [sq], [m_sq], nsm.Hparams(), stream=stream)
            stream.synchronize()
            nsm.muon_step(h_twin, w_ot, grads[s], m_ot, hp)
            nsm.muon_step(h_twin, [w_sqt], [sq], [m_sqt], nsm.Hparams())
            for i in range(n):
                g_g[i].copy_(grads[s][i])
            torch.cuda.synchronize()
            graph.replay()
            nsm.muon_step(h_twin, w_e, grads[s], m_e, hp)
            torch.cuda.synchronize()
            for i in range(n):
                assert torch.equal(w_g[i], w_e[i]), f"replay {s}: weights of matrix {i} differ"
                assert torch.equal(m_g[i], m_e[i]), f"replay {s}: momentum of matrix {i} differs"
                assert torch.equal(w_o[i], w_ot[i]) and torch.equal(m_o[i], m_ot[i])
            assert torch.equal(w_sq, w_sqt) and torch.equal(m_sq, m_sqt)
    finally:
        nsm.muon_destroy(h)
        nsm.muon_destroy(h_twin)


@pytest.mark.parametrize("alpha", [1e-20, 1.0, 1e20])
def test_extreme_gradient_scales(alpha):
    """Normalisation at any finite scale: gradients (momentum zero) scaled by
    1e-20 and 1e20, stored in bf16, against the oracle on the same stored
    values.  At 1e20 the sum of squares and the first Gram product leave
    float32's range unless handled; at 1e-20 the norm is far below eps, so the
    oracle's X0 = u / (||u|| + eps) is itself tiny and the iteration is close
    to a^5 X0, whose products underflow float32 unless the operand copy is
    rescaled.  Whole-matrix and local bars as everywhere."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    from muon_synth import encode_storage, lowrank_noise_grad, rng_for
    from gpu_harness import TOL_O_BF16
    shapes = [(300, 100), (100, 300), (256, 256), (48, 40)]
    h = nsm.muon_init(0)
    try:
        g_st = [encode_storage(lowrank_noise_grad(rng_for(61, 1, i, 1), *s) * alpha, "bf16") for i, s in enumerate(shapes)]
        ws = [torch.zeros(s, device="cuda", dtype=torch.bfloat16) for s in shapes]
        ms = [torch.zeros(s, device="cuda") for s in shapes]
        os_ = [torch.empty(s, device="cuda") for s in shapes]
        nsm.muon_step(h, ws, [to_device(g) for g in g_st], ms, nsm.Hparams(), update_outs=os_)
        torch.cuda.synchronize()
        nu = nsm.muon_read_norms(h, len(shapes))
        for i, s in enumerate(shapes):
            ref = oracle.muon_step_matrix(np.zeros(s), oracle.decode(g_st[i]), np.zeros(s), oracle.Hyper())
            assert nu[i] == pytest.approx(ref.nu, rel=1e-6)
            o = to_stored(os_[i]).astype(np.float64)
            assert np.isfinite(o).all()
            e = assert_o_close(o, ref.o, TOL_O_BF16, f"{s} at scale {alpha:g}")
            print(f"{s} alpha {alpha:g}: |O| {np.linalg.norm(ref.o):.3e} errors {e}", flush=True)
    finally:
        nsm.muon_destroy(h)


def test_small_matrices_run_in_float32():
    """Matrices with min(rows, cols) <= 64 run the iteration in float32 in
    bf16 mode too, so they meet the float32-mode bar (1e-4, as for the ragged
    float32 cases), next to bf16 ones in the same call."""
    shapes = [(64, 64), (1, 4096), (4096, 3), (48, 40), (17, 1), (64, 300), (300, 64), (65, 200), (200, 199)]
    wl = _wl("small32", shapes, steps=2, nesterov=True)
    rep = []
    rec = run_gpu(wl, 2, list(range(len(shapes))))
    small = [i for i, (r, c) in enumerate(shapes) if min(r, c) <= 64]
    check_against_oracle(wl, {i: rec[i] for i in small}, 1e-4, report=rep)
    check_against_oracle(wl, {i: rec[i] for i in range(len(shapes)) if i not in small}, TOL_O_BF16)
    print("small matrices worst O rel err", max(e for (_, _, _, e) in rep))


def test_wide_axpy_tiles():
    """Large matrices (both sides at least 1024, padded shape a multiple of
    256) run the GRAM and the AXPY on 256-wide tiles when they hold most of
    the phase's flops.  Their results meet the oracle bars (a ragged
    1000 x 2000 matrix among them, every iteration kind over three steps) and
    equal bitwise those of the 128-wide kernels, which the same matrices take
    when a larger matrix that cannot use wide tiles (1152 padded rows)
    dominates the call: both sum every output element's k in the same order."""
    base = workload("gpt2-124m-hidden")
    shapes = [(1024, 2048), (2048, 1024), (1000, 2000), (1024, 1024), (300, 100)]

    def mk(shp):
        mats = tuple(MatSpec(r, c, f"m{i}") for i, (r, c) in enumerate(shp))
        return base.with_(name="wide", wid=140, mats=mats, nesterov=True, weight_decay=0.01, steps=3)

    wl = mk(shapes)
    rep = []
    rec = run_gpu(wl, 3, list(range(len(shapes))))
    check_against_oracle(wl, rec, TOL_O_BF16, report=rep)
    print("wide tiles worst O rel err", max(e for (_, _, _, e) in rep))
    rec128 = run_gpu(mk(shapes + [(1152, 8000)]), 3, list(range(len(shapes))))
    for i in range(len(shapes)):
        for s, (a, b) in enumerate(zip(rec[i], rec128[i])):
            for what in ("w_new", "m_new", "o"):
                assert np.array_equal(getattr(a, what), getattr(b, what)), f"matrix {i} step {s + 1}: {what} differs"

