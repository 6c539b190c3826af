"""The GPU parity checks themselves, on the CPU: the local (tile, row, column)
bars on O catch a single wrong 128 x 128 tile, row or column of a large matrix
that the whole-matrix rel-F bar lets through, and pass uniform rounding-sized
noise."""

import numpy as np
import pytest

from gpu_harness import TOL_O_BF16, local_errors, relf


def _dense(rng, r, c):
    return rng.standard_normal((r, c)) / np.sqrt(max(r, c))


@pytest.fixture(scope="module")
def ref():
    return _dense(np.random.default_rng(1), 4096, 3072)


def test_uniform_noise_passes(ref):
    rng = np.random.default_rng(2)
    o = ref + 5e-3 * rng.standard_normal(ref.shape) * np.sqrt(np.mean(ref ** 2))
    loc = local_errors(o, ref)
    assert relf(o, ref) < 6e-3
    assert max(loc.values()) < 1e-2, loc


@pytest.mark.parametrize("part", ["tile", "row", "col", "edge_tile"])
def test_one_wrong_part_fails_locally_only(ref, part):
    if part == "edge_tile":   # the ragged corner tile of a ragged matrix (104 x 92 elements)
        ref = _dense(np.random.default_rng(3), 1000, 1500)
    o = ref.copy()
    if part == "tile":
        o[256:384, 512:640] *= 0.5
    elif part == "row":
        o[700, :] *= 0.9
    elif part == "col":
        o[:, 1000] *= 0.9
    else:
        o[896:, 1408:] *= 0.8
    assert relf(o, ref) < TOL_O_BF16          # the whole-matrix bar misses it
    loc = local_errors(o, ref)
    assert loc["tile" if part == "edge_tile" else part] > 0.09, loc   # its own bar does not


def test_small_parts_use_fair_share_floor():
    """A tile whose own norm is tiny is measured against its share of the
    whole norm, so rounding-sized error there does not fail."""
    rng = np.random.default_rng(4)
    ref = _dense(rng, 256, 256)
    ref[:128, :128] *= 1e-6
    o = ref + 1e-3 * rng.standard_normal(ref.shape) / 16.0
    assert local_errors(o, ref)["tile"] < 3e-2


def test_short_lines_are_not_checked():
    ref = np.random.default_rng(5).standard_normal((4096, 3))
    o = ref.copy()
    o[17, 1] *= 1.5        # one element of a 3-element row: only the tile and column see it
    loc = local_errors(o, ref)
    assert loc["row"] == 0.0 and loc["col"] > 0.0 and loc["tile"] > 0.0
