"""Host-side sanitizer run of the kernels: the library's kernel and host
sources are compiled as plain C++ against a CPU stand-in of HIP
(tests/emu/hip) with AddressSanitizer, and muon_step / muon_adamw_step run on
exactly sized host buffers.  Every global address a kernel forms is checked;
the stand-in's MFMA does no arithmetic, so values are not (the GPU parity
tests check those)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "newton_schulz_matrix_step_amd", "csrc")
EMU = os.path.join(ROOT, "tests", "emu")
CXX = "/opt/rocm/lib/llvm/bin/clang++"

CASES = [
    # shapes, ns_steps, dtype (0 bf16, 1 f32), block rows, leading-dimension pad, misaligned start
    ("300x100,100x300,256x256,129x515,515x129,64x64,1x17,17x1,200x199", 3, 0, 0),
    ("300x100,100x300,129x515,515x129,1x17,17x1,200x199", 2, 0, 0, 5, 1),
    ("300x100,100x300,129x515,33x64", 2, 1, 0, 8, 3),
    ("300x100,100x300,256x256,129x515,515x129,64x64,1x17,17x1,200x199", 2, 1, 0),
    ("1x1,1x40,40x1,3x5,64x128,128x64", 2, 1, 0),
    ("1024x3584,3584x1024,1024x1024,1x1,17x1", 2, 0, 0),
    ("100x300,300x100", 0, 0, 0),
    ("768x256,384x96,130x60", 1, 0, 128),
    ("384x96,130x60", 2, 0, 65),
]


@pytest.fixture(scope="module")
def emu_binary(tmp_path_factory):
    if not os.path.exists(CXX):
        pytest.skip("ROCm clang++ not available")
    out = tmp_path_factory.mktemp("emu")
    flags = ["-O1", "-g", "-std=c++17", "-fsanitize=address", "-fno-omit-frame-pointer", f"-I{EMU}",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-Wno-unused-value"]
    objs = []
    for src, lang in (("muon_kernels.hip", ["-x", "c++"]), ("adamw_kernels.hip", ["-x", "c++"]),
                      ("muon_api.cpp", [])):
        obj = str(out / (src + ".o"))
        subprocess.run([CXX, *flags, *lang, os.path.join(CSRC, src), "-c", "-o", obj], check=True)
        objs.append(obj)
    obj = str(out / "driver.o")
    subprocess.run([CXX, *flags, os.path.join(EMU, "emu_driver.cpp"), "-c", "-o", obj], check=True)
    exe = str(out / "emu_driver")
    subprocess.run([CXX, "-fsanitize=address", *objs, obj, "-o", exe], check=True)
    return exe


@pytest.mark.parametrize("case", CASES)
def test_kernels_stay_in_bounds(emu_binary, case):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([emu_binary, *[str(v) for v in case]], capture_output=True, text=True, env=env, timeout=600)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    assert r.returncode == 0, (r.stdout, r.stderr[-2000:])
    assert "step 0" in r.stdout and "adamw 0" in r.stdout
