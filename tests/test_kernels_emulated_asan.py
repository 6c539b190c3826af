"""Host-side sanitizer run of the kernels: the library's kernel and host
sources are compiled as plain C++ against a CPU stand-in of HIP
(tests/emu/hip) with AddressSanitizer and UndefinedBehaviorSanitizer, and
muon_step / muon_step_noalloc / muon_adamw_step run on exactly sized host
buffers.  Every global address a kernel forms is checked, and any undefined
behaviour of the host code or the kernels' integer and pointer arithmetic
(signed overflow, bad shifts, misaligned or null accesses) aborts the run;
the stand-in's MFMA does no arithmetic, so values are not checked (the GPU
parity tests check those)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "newton_schulz_matrix_step_amd", "csrc")
EMU = os.path.join(ROOT, "tests", "emu")
CXX = "/opt/rocm/lib/llvm/bin/clang++"

CASES = [
    # shapes, ns_steps, dtype (0 bf16, 1 f32), block rows, leading-dimension pad, misaligned start,
    # gradient value (1e15: every norm beyond 2^30, so the rescale pass runs), no-alloc entry point,
    # debug handle
    ("300x100,100x300,256x256,129x515,515x129,64x64,1x17,17x1,200x199", 3, 0, 0),
    ("300x100,100x300,129x515,515x129,1x17,17x1,200x199", 2, 0, 0, 5, 1),
    ("300x100,100x300,129x515,33x64", 2, 1, 0, 8, 3),
    ("300x100,100x300,256x256,129x515,515x129,64x64,1x17,17x1,200x199", 2, 1, 0),
    ("1x1,1x40,40x1,3x5,64x128,128x64", 2, 1, 0),
    ("1024x3584,3584x1024,1024x1024,1x1,17x1", 2, 0, 0),
    ("100x300,300x100", 0, 0, 0),
    ("768x256,384x96,130x60", 1, 0, 128),
    ("384x96,130x60", 2, 0, 65),
    ("300x100,100x300,129x515,515x129,64x64,1x17,17x1,200x199", 2, 0, 0, 0, 0, 1e15),
    ("300x100,100x300,129x515,33x64", 2, 1, 0, 5, 1, 1e15),
    # the no-allocation entry point: static scratch, a call then a smaller one
    ("300x100,100x300,129x515,515x129,64x64,1x17,17x1", 2, 0, 0, 0, 0, 0, 1),
    ("300x100,33x64", 2, 1, 0, 5, 1, 1e15, 1),
    # a debug handle: guard bands after every workspace buffer, written and checked
    ("300x100,100x300,256x256,129x515,515x129,1x17,17x1", 2, 0, 0, 0, 0, 0, 0, 1),
    ("300x100,129x515,33x64", 2, 1, 64, 3, 1, 1e15, 0, 1),
]


def _build(tmp_path_factory, name, extra):
    if not os.path.exists(CXX):
        pytest.skip("ROCm clang++ not available")
    out = tmp_path_factory.mktemp(name)
    flags = ["-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", f"-I{EMU}",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-Wno-unused-value", *extra]
    objs = []
    for src, lang in (("muon_kernels.hip", ["-x", "c++"]), ("adamw_kernels.hip", ["-x", "c++"]),
                      ("muon_static.hip", ["-x", "c++"]), ("muon_api.cpp", [])):
        obj = str(out / (src + ".o"))
        subprocess.run([CXX, *flags, *lang, os.path.join(CSRC, src), "-c", "-o", obj], check=True)
        objs.append(obj)
    obj = str(out / "driver.o")
    subprocess.run([CXX, *flags, os.path.join(EMU, "emu_driver.cpp"), "-c", "-o", obj], check=True)
    exe = str(out / "emu_driver")
    subprocess.run([CXX, "-fsanitize=address,undefined", *objs, obj, "-o", exe], check=True)
    return exe


@pytest.fixture(scope="module")
def emu_binary(tmp_path_factory):
    return _build(tmp_path_factory, "emu", [])


# The 256-wide kernels, which the library gives only to matrices of at least
# 1024 on both sides, here for smaller ones, so that full, diagonal and ragged
# wide tiles (and the first, middle and last iterations) run in a few seconds.
WIDE_CASES = [
    ("256x512,512x256,768x768,500x700,700x500,1x17,300x100", 3, 0, 0),
    ("256x512,512x256,500x700", 1, 0, 0),
    ("512x256,700x500,100x300", 2, 0, 0, 5, 1),
    ("256x512,500x700,300x100", 2, 0, 0, 0, 0, 0, 1),
    ("512x256,500x700", 2, 0, 0, 0, 0, 0, 0, 1),
    ("256x512,700x500", 2, 0, 0, 3, 1, 1e15),
]


@pytest.fixture(scope="module")
def emu_wide_binary(tmp_path_factory):
    return _build(tmp_path_factory, "emu_wide", ["-DMUON_WIDE_MIN=256"])


def _run(exe, case, expect_kernel=None):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    if expect_kernel:
        env["EMU_VERBOSE"] = "1"
    r = subprocess.run([exe, *[str(v) for v in case]], capture_output=True, text=True, env=env, timeout=900)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    assert "runtime error" not in r.stderr, r.stderr[-3000:]
    assert r.returncode == 0, (r.stdout, r.stderr[-2000:])
    assert "step 0" in r.stdout and "adamw 0" in r.stdout
    if expect_kernel:
        assert f"launch ({expect_kernel}" in r.stderr or f"launch {expect_kernel}" in r.stderr, r.stderr[-2000:]


@pytest.mark.parametrize("case", CASES)
def test_kernels_stay_in_bounds(emu_binary, case):
    _run(emu_binary, case)


@pytest.mark.parametrize("case", WIDE_CASES)
def test_wide_axpy_stays_in_bounds(emu_wide_binary, case):
    _run(emu_wide_binary, case, expect_kernel="ns_gemm_wide")


def test_wide_tiles_only_when_they_carry_most_flops(emu_wide_binary):
    """The planner gives a phase wide tiles only when the matrices that can
    take them carry at least half of its flops: alone, a 256 x 512 matrix
    runs its GRAM and AXPY on wide tiles; beside a dominant 300 x 2000 one
    (padded rows not a multiple of 256) every matrix stays on 128-wide tiles."""
    _run(emu_wide_binary, ("256x512", 2, 0, 0), expect_kernel="ns_gemm_wide")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", EMU_VERBOSE="1")
    r = subprocess.run([emu_wide_binary, "256x512,300x2000", "2", "0", "0"], capture_output=True, text=True, env=env,
                       timeout=900)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "ns_gemm_wide" not in r.stderr and "ns_gemm_bf16" in r.stderr

