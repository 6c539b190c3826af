"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point its header declares, agrees with the header on struct
layouts, and reports a missing device instead of touching one."""

import ctypes
import os
import re
import subprocess

import pytest

import newton_schulz_matrix_step_amd as nsm
from newton_schulz_matrix_step_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_abi.LIB_PATH):
        pytest.fail("HIP library not built: run __graft_entry__.build() first")
    return nsm.load()


def test_every_declared_symbol_is_exported(lib):
    declared = _declared_functions()
    assert "muon_step" in declared and "muon_init" in declared
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in muon.h but not exported"
    assert sorted(declared) == sorted(_abi.EXPORTED_SYMBOLS)


def test_only_the_c_abi_is_exported(lib):
    """Every exported muon_* function is declared in the header, and no
    internal (C++ namespace) symbol of the library leaks out."""
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout.split("\n")
    names = [l.split()[-1] for l in out if len(l.split()) == 3 and l.split()[1] in ("T", "W")]
    assert sorted(n for n in names if n.startswith("muon_")) == _declared_functions()
    assert not [n for n in names if "4muon" in n and not n.startswith("_ZNSt")]


def test_abi_version(lib):
    text = open(HEADER).read()
    ver = int(re.search(r"#define MUON_ABI_VERSION (\d+)", text).group(1))
    assert nsm.muon_abi_version() == ver


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "muon.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu %zu %zu %zu %zu\\n\", sizeof(muon_matrix), sizeof(muon_hparams),"
        " sizeof(muon_kernel_stats), offsetof(muon_matrix, dtype), offsetof(muon_hparams, ns_steps),"
        " offsetof(muon_matrix, ld_update), offsetof(muon_hparams, coeffs), offsetof(muon_matrix, block_rows),"
        " offsetof(muon_matrix, block_cols)); return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert out == [ctypes.sizeof(_abi.muon_matrix), ctypes.sizeof(_abi.muon_hparams),
                   ctypes.sizeof(_abi.muon_kernel_stats), _abi.muon_matrix.dtype.offset,
                   _abi.muon_hparams.ns_steps.offset, _abi.muon_matrix.ld_update.offset,
                   _abi.muon_hparams.coeffs.offset, _abi.muon_matrix.block_rows.offset,
                   _abi.muon_matrix.block_cols.offset]


def test_status_strings(lib):
    for code, name in ((0, "MUON_OK"), (1, "MUON_ERR_INVALID_ARG"), (2, "MUON_ERR_DTYPE"),
                       (3, "MUON_ERR_NO_DEVICE"), (4, "MUON_ERR_OOM"), (5, "MUON_ERR_HIP")):
        assert nsm.muon_status_str(code) == name


def test_null_handle_and_args(lib):
    hp = nsm.Hparams().to_c()
    assert lib.muon_step(None, None, 0, ctypes.byref(hp), None) == nsm.MUON_ERR_INVALID_ARG
    assert lib.muon_orthogonalize(None, None, None, 1, 1, 1, 1, 0, ctypes.byref(hp), None) == nsm.MUON_ERR_INVALID_ARG
    assert lib.muon_init(None, 0, 0) == nsm.MUON_ERR_INVALID_ARG
    assert lib.muon_destroy(None) == nsm.MUON_OK
    assert lib.muon_last_error(None) == b""
    assert lib.muon_workspace_bytes(None) == 0
    assert lib.muon_kernel_stats_read(None, None, 0) == 0


def test_init_without_gpu_reports_no_device(lib):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p()
    assert lib.muon_init(ctypes.byref(h), 0, 0) == nsm.MUON_ERR_NO_DEVICE
    assert h.value is None
    with pytest.raises(nsm.MuonError) as ei:
        nsm.muon_init(0)
    assert ei.value.status == nsm.MUON_ERR_NO_DEVICE
    assert lib.muon_init(ctypes.byref(h), 0, 0x80) == nsm.MUON_ERR_INVALID_ARG   # unknown flag bits


def test_hparams_marshalling():
    c = nsm.Hparams(lr=0.5, nesterov=True, ns_steps=3, compute="fp32").to_c()
    assert (c.lr, c.nesterov, c.ns_steps, c.compute) == (0.5, 1, 3, nsm.MUON_COMPUTE_FP32)
    assert nsm.Hparams(compute="fp16").to_c().compute == -1


def test_hparams_coeffs_marshalling():
    sched = [(3.0, -3.2, 1.2), (2.5, -2.0, 0.6), (1.5, -0.5, 0.0)]
    c = nsm.Hparams(ns_steps=3, coeffs=sched).to_c()
    got = [c.coeffs[i] for i in range(9)]
    assert got == pytest.approx([v for t in sched for v in t], rel=1e-7)
    assert not nsm.Hparams().to_c().coeffs               # NULL: the default triple every iteration
    with pytest.raises(ValueError):
        nsm.Hparams(ns_steps=3, coeffs=sched[:2]).to_c()  # fewer triples than iterations
    with pytest.raises(ValueError):
        nsm.Hparams(ns_steps=1, coeffs=[(1.0, 2.0)]).to_c()


def test_adamw_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout_adamw.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "muon.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu\\n\", sizeof(muon_adamw_tensor), sizeof(muon_adamw_hparams),"
        " offsetof(muon_adamw_tensor, numel), offsetof(muon_adamw_tensor, dtype), offsetof(muon_adamw_hparams, step));"
        " return 0;}\n")
    exe = tmp_path / "layout_adamw"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert out == [ctypes.sizeof(_abi.muon_adamw_tensor), ctypes.sizeof(_abi.muon_adamw_hparams),
                   _abi.muon_adamw_tensor.numel.offset, _abi.muon_adamw_tensor.dtype.offset,
                   _abi.muon_adamw_hparams.step.offset]


def test_adamw_hparams_marshalling():
    c = nsm.AdamWHparams(lr=0.25, beta1=0.5, beta2=0.75, eps=1e-6, weight_decay=0.125, step=7).to_c()
    assert (c.lr, c.beta1, c.beta2, c.weight_decay, c.step) == (0.25, 0.5, 0.75, 0.125, 7)
    assert c.eps == pytest.approx(1e-6, rel=1e-7)


def test_profile_role_flags(lib):
    assert nsm.profile_roles(["ns_axpy"]) == 1 << (16 + 4)
    assert nsm.profile_roles(["momentum_norm", "adamw"]) == (1 | 1 << 8) << 16
    assert nsm.profile_roles(["norm_rescale"]) == 1 << (16 + 9)
    h = ctypes.c_void_p()
    # role bits beyond the last role are unknown flag bits: rejected before any device query
    assert lib.muon_init(ctypes.byref(h), 0, nsm.MUON_INIT_PROFILE | (1 << (16 + 10))) == nsm.MUON_ERR_INVALID_ARG


def test_binding_checks_shapes_dtypes_and_devices():
    """The C ABI sees only pointers and sizes, so the binding rejects tensors
    whose sizes or dtypes the kernels would read or write past (a smaller or
    bf16 momentum, a mismatched update_out), and tensors off the GPU, before
    anything reaches the library."""
    import torch
    w = torch.zeros(8, 12, dtype=torch.bfloat16)
    g = torch.zeros(8, 12, dtype=torch.bfloat16)
    m = torch.zeros(8, 12)
    bad = [
        ((w, g, torch.zeros(8, 12, dtype=torch.bfloat16)), "float32"),   # bf16 momentum
        ((w, g, torch.zeros(8, 11)), "shape"),                           # smaller momentum
        ((w, torch.zeros(12, 8, dtype=torch.bfloat16), m), "shape"),     # transposed grad
        ((w, g, m, torch.zeros(8, 12, dtype=torch.bfloat16)), "float32"),  # bf16 update_out
        ((w, g, m, torch.zeros(4, 12)), "shape"),                        # smaller update_out
        ((torch.zeros(96, dtype=torch.bfloat16), g, m), "2-D"),
        ((w, g, m), "GPU"),                                              # all on the host
    ]
    for args, what in bad:
        with pytest.raises(ValueError, match=what):
            nsm.make_matrix(*args)
    with pytest.raises(ValueError, match="shape"):
        nsm.muon_orthogonalize(0, g, torch.zeros(12, 8), nsm.Hparams())
    with pytest.raises(ValueError, match="float32"):
        nsm.muon_orthogonalize(0, g, torch.zeros(8, 12, dtype=torch.bfloat16), nsm.Hparams())
    with pytest.raises(ValueError, match="GPU"):
        nsm.muon_orthogonalize(0, g, torch.zeros(8, 12), nsm.Hparams())
    z = torch.zeros(100)
    with pytest.raises(ValueError, match="GPU"):
        nsm.make_adamw_tensor(z, z.clone(), z.clone(), z.clone())
    with pytest.raises(ValueError, match="float32"):
        nsm.make_adamw_tensor(z, z.clone(), z.clone().double(), z.clone())
