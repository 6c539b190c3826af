"""The seeded input generator: determinism, stated spectra, storage encoding."""

import numpy as np
import pytest

from muon_synth import (WORKLOADS, bf16_bits_to_f32, encode_storage, heavy_tail_grad,
                        lowrank_noise_grad, make_grad, make_momentum, make_param, rng_for, workload)
from muon_synth.gen import expert_scale


def test_workload_shapes():
    w = workload("gpt2-124m-hidden")
    assert len(w.mats) == 72 and w.elements == 12 * (4 * 768 * 768 + 2 * 768 * 3072)
    assert workload("gpt2-350m-hidden").nesterov and workload("gpt2-350m-hidden").weight_decay == 0.01
    assert len(workload("gpt2-350m-hidden").mats) == 144
    assert len(workload("large-layer-share-4096x14336").mats) == 12
    moe = workload("moe-64x-2048x1408")
    assert len(moe.mats) == 132
    assert sum(1 for m in moe.mats if (m.rows, m.cols) == (2048, 1408)) == 64
    s1 = workload("single-64x128-fp32")
    assert s1.storage == "fp32" and s1.compute == "fp32" and s1.steps == 1


def test_determinism():
    w = workload("gpt2-124m-hidden")
    np.testing.assert_array_equal(make_grad(w, 3, 5), make_grad(w, 3, 5))
    assert not np.array_equal(make_grad(w, 3, 5), make_grad(w, 4, 5))
    np.testing.assert_array_equal(make_param(w, 1), make_param(w, 1))
    assert not np.any(make_momentum(w, 0))
    assert np.any(make_momentum(workload("single-64x128-fp32"), 0))


def test_lowrank_spectrum_and_scale():
    g = lowrank_noise_grad(rng_for(1, 1, 1, 1), 300, 500)
    assert np.sqrt(np.mean(g ** 2)) == pytest.approx(0.02, rel=1e-12)
    s = np.linalg.svd(g, compute_uv=False)
    # 16 dominant directions with ratios close to 1/k, then a noise floor
    assert s[15] / s[16] > 3
    np.testing.assert_allclose(s[:4] / s[0], [1, 1 / 2, 1 / 3, 1 / 4], rtol=0.1)


@pytest.mark.parametrize("shape", [(200, 120), (120, 200), (2048, 1024)])
def test_heavy_tail_exact_spectrum(shape):
    g = heavy_tail_grad(rng_for(2, 1, 1, 1), *shape)
    s = np.linalg.svd(g, compute_uv=False)
    k = np.arange(1, min(shape) + 1) ** -0.7
    np.testing.assert_allclose(s / s[0], k, rtol=1e-9, atol=1e-12)
    assert np.sqrt(np.mean(g ** 2)) == pytest.approx(0.02, rel=1e-12)


def test_expert_scale_range():
    w = workload("moe-64x-2048x1408")
    sc = [expert_scale(w, e) for e in range(64)]
    assert min(sc) >= 1e-4 and max(sc) <= 1e-1
    g = make_grad(w, 1, 0)
    assert np.sqrt(np.mean(g ** 2)) == pytest.approx(sc[0], rel=1e-12)


def test_bf16_encoding_against_torch():
    torch = pytest.importorskip("torch")
    x = np.concatenate([np.random.default_rng(0).standard_normal(100000) * 0.02,
                        [0.0, -0.0, 1.0, 3.0e38, -1e-40, 1 + 2 ** -8, 1 + 3 * 2 ** -8]])
    bits = encode_storage(x, "bf16")
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(bits),
                                  torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())
    assert set(WORKLOADS) >= {"gpt2-124m-hidden"}
