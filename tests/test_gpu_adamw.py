"""GPU parity of the AdamW step (the update the hybrid setup runs on the
parameters Muon does not take) through the C ABI, against the float64 oracle
on the same stored inputs, one step at a time (each step starts from the GPU's
own stored parameter and moments, decoded exactly).

Bars, elementwise: moments within 2^-21 of the magnitude of their two terms
(a few float32 roundings); a float32 parameter within 2^-20 of |p (1 - lr wd)|
+ |step| (the evaluation error of the update in float32); a bf16 parameter
within one bf16 ulp of the float64 result plus that slack.
"""

import numpy as np
import pytest

import oracle
from gpu_harness import bf16_ulp, to_device, to_stored
from muon_synth import adamw_workload, encode_storage, make_adamw_grad, make_adamw_param

pytestmark = pytest.mark.gpu


def f32(x):
    return float(np.float32(x))


def _hyper(hp):
    """The oracle takes the float32 hyperparameters the kernel receives."""
    return oracle.AdamWHyper(lr=f32(hp.lr), beta1=f32(hp.beta1), beta2=f32(hp.beta2), eps=f32(hp.eps),
                             weight_decay=f32(hp.weight_decay))


def _check(p_old_st, g_st, m_old, v_old, p_new_st, m_new, v_new, hp, step, what=""):
    h = _hyper(hp)
    p_old = oracle.decode(p_old_st)
    g = oracle.decode(g_st)
    r = oracle.adamw_step(p_old, g, m_old.astype(np.float64), v_old.astype(np.float64), h, step)
    tm = 2.0 ** -21 * (h.beta1 * np.abs(m_old) + (1 - h.beta1) * np.abs(g))
    tv = 2.0 ** -21 * (h.beta2 * np.abs(v_old) + (1 - h.beta2) * g * g)
    bad_m = np.abs(m_new.astype(np.float64) - r.m) > tm
    bad_v = np.abs(v_new.astype(np.float64) - r.v) > tv
    assert not bad_m.any(), f"{what} step {step}: {int(bad_m.sum())} first moments off"
    assert not bad_v.any(), f"{what} step {step}: {int(bad_v.sum())} second moments off"
    upd = np.abs(r.p - p_old * (1 - h.lr * h.weight_decay))
    slack = 2.0 ** -20 * (np.abs(p_old) * abs(1 - h.lr * h.weight_decay) + upd)
    p_new = oracle.decode(p_new_st)
    tol = slack + (bf16_ulp(r.p) if p_new_st.dtype == np.uint16 else 0.0)
    bad_p = np.abs(p_new - r.p) > tol
    assert not bad_p.any(), f"{what} step {step}: {int(bad_p.sum())} parameters off, worst " \
                            f"{float(np.max(np.abs(p_new - r.p) - tol)):.3e} beyond"


def _run_and_check(hnd, ps, gs_steps, storages, hp_kw, steps, views=None):
    """ps: host float64 params; gs_steps[s][i]: host float64 grads; one grouped call a step."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    n = len(ps)
    params, ms, vs = [], [], []
    for i in range(n):
        st = encode_storage(ps[i], storages[i])
        if views is not None and views[i]:
            # a view one element into a larger buffer: unaligned bases, scalar path
            big = to_device(encode_storage(np.concatenate([[0.0], ps[i], [0.0]]), storages[i]))
            params.append(big[1:1 + ps[i].size])
            m_big = torch.zeros(ps[i].size + 2, device="cuda")
            v_big = torch.zeros(ps[i].size + 2, device="cuda")
            ms.append(m_big[1:1 + ps[i].size])
            vs.append(v_big[1:1 + ps[i].size])
        else:
            params.append(to_device(st))
            ms.append(torch.zeros(ps[i].size, device="cuda"))
            vs.append(torch.zeros(ps[i].size, device="cuda"))
    for s in range(1, steps + 1):
        g_st = [encode_storage(gs_steps[s - 1][i], storages[i]) for i in range(n)]
        grads = [to_device(x) for x in g_st]
        p_old = [to_stored(p) for p in params]
        m_old = [m.cpu().numpy().copy() for m in ms]
        v_old = [v.cpu().numpy().copy() for v in vs]
        hp = nsm.AdamWHparams(step=s, **hp_kw)
        nsm.muon_adamw_step(hnd, params, grads, ms, vs, hp)
        torch.cuda.synchronize()
        for i in range(n):
            _check(p_old[i], g_st[i], m_old[i], v_old[i], to_stored(params[i]), ms[i].cpu().numpy(),
                   vs[i].cpu().numpy(), hp, s, what=f"tensor {i} ({ps[i].size}, {storages[i]})")
    return params


HP = dict(lr=3e-3, beta1=0.8, beta2=0.95, eps=1e-10, weight_decay=0.1)


def test_adamw_mixed_sizes_dtypes_and_views():
    import newton_schulz_matrix_step_amd as nsm
    rng = np.random.default_rng(11)
    sizes = [1, 3, 4, 5, 4095, 4096, 4097, 12295, 768, 2304, 100003, 0, 8192]
    storages = ["bf16" if i % 2 == 0 else "fp32" for i in range(len(sizes))]
    views = [i % 3 == 1 for i in range(len(sizes))]
    ps = [rng.standard_normal(n) * 0.02 for n in sizes]
    gs = [[rng.standard_normal(n) * 10.0 ** rng.uniform(-5, -2) for n in sizes] for _ in range(3)]
    h = nsm.muon_init(0)
    try:
        _run_and_check(h, ps, gs, storages, HP, 3, views=views)
    finally:
        nsm.muon_destroy(h)


def test_adamw_gpt2_124m_parameter_set():
    """The full GPT-2 124M AdamW set (78M elements, bf16): two grouped steps."""
    import newton_schulz_matrix_step_amd as nsm
    wl = adamw_workload("gpt2-124m-adamw-params")
    n = len(wl.tensors)
    ps = [make_adamw_param(wl, i) for i in range(n)]
    gs = [[make_adamw_grad(wl, s, i) for i in range(n)] for s in (1, 2)]
    h = nsm.muon_init(0)
    try:
        _run_and_check(h, ps, gs, [wl.storage] * n,
                       dict(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps, weight_decay=wl.weight_decay), 2)
    finally:
        nsm.muon_destroy(h)


def test_adamw_deterministic_and_new_pointers():
    """Bitwise repeatable; a second list of tensors of the same sizes (new
    pointers, same plan) gets its own correct result."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    rng = np.random.default_rng(12)
    sizes = [5000, 4096, 17]
    h = nsm.muon_init(0)
    try:
        outs = []
        for rep in range(2):
            ps = [torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda() for n in sizes]
            gs = [torch.from_numpy(rng.standard_normal(n).astype(np.float32) * 1e-3).cuda() for n in sizes]
            if rep == 1:
                ps = [p.clone() for p in outs[0][0]]
                gs = [g.clone() for g in outs[0][1]]
            ms = [torch.zeros(n, device="cuda") for n in sizes]
            vs = [torch.zeros(n, device="cuda") for n in sizes]
            p0 = [p.clone() for p in ps]
            nsm.muon_adamw_step(h, ps, gs, ms, vs, nsm.AdamWHparams(step=1, **HP))
            torch.cuda.synchronize()
            outs.append((p0, gs, ps, ms, vs))
        for a, b in zip(outs[0][2] + outs[0][3] + outs[0][4], outs[1][2] + outs[1][3] + outs[1][4]):
            assert torch.equal(a, b)
    finally:
        nsm.muon_destroy(h)


@pytest.mark.parametrize("bad", [dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0), dict(lr=float("nan")),
                                 dict(step=0), dict(weight_decay=float("inf"))])
def test_adamw_invalid_hparams_rejected(bad):
    import torch
    import newton_schulz_matrix_step_amd as nsm
    h = nsm.muon_init(0)
    try:
        p = torch.zeros(100, device="cuda")
        g = torch.ones(100, device="cuda")
        m, v = torch.zeros(100, device="cuda"), torch.zeros(100, device="cuda")
        kw = dict(HP)
        kw.update(bad)
        step = kw.pop("step", 1)
        with pytest.raises(nsm.MuonError) as ei:
            nsm.muon_adamw_step(h, [p], [g], [m], [v], nsm.AdamWHparams(step=step, **kw))
        assert ei.value.status == nsm.MUON_ERR_INVALID_ARG
        torch.cuda.synchronize()
        assert float(p.abs().max()) == 0.0 and float(m.abs().max()) == 0.0
    finally:
        nsm.muon_destroy(h)


def test_adamw_bad_tensors_rejected():
    import torch
    import newton_schulz_matrix_step_amd as nsm
    h = nsm.muon_init(0)
    try:
        p = torch.zeros(64, device="cuda")
        g = torch.ones(64, device="cuda", dtype=torch.bfloat16)
        m, v = torch.zeros(64, device="cuda"), torch.zeros(64, device="cuda")
        with pytest.raises(nsm.MuonError) as ei:   # param f32, grad bf16
            nsm.muon_adamw_step(h, [p], [g], [m], [v], nsm.AdamWHparams())
        assert ei.value.status == nsm.MUON_ERR_DTYPE
        with pytest.raises(nsm.MuonError) as ei:   # exp_avg aliases exp_avg_sq
            nsm.muon_adamw_step(h, [p], [g.float()], [m], [m], nsm.AdamWHparams())
        assert ei.value.status == nsm.MUON_ERR_INVALID_ARG
        # an empty list and zero-size tensors are no-ops
        nsm.muon_adamw_step(h, [], [], [], [], nsm.AdamWHparams())
        e = torch.zeros(0, device="cuda")
        nsm.muon_adamw_step(h, [e], [e.clone()], [e.clone()], [e.clone()], nsm.AdamWHparams())
        torch.cuda.synchronize()
        assert float(p.abs().max()) == 0.0
    finally:
        nsm.muon_destroy(h)
