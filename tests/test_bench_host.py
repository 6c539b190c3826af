"""bench.py's host logic, on the CPU: the algorithmic work its roofline is
priced with, the counter summaries, the rule that recorded counter figures
apply only to the kernel sources they were taken on, and the one-GPU limit."""

import os
import subprocess
import sys

import pytest

import bench
from muon_synth import workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Per-step totals worked out by hand from each workload's shapes (5 iterations;
# NS flops with the upper-triangle counts m(m+1)n + m^2(m+1) + 2m^2 n, the dense
# convention 4m^2 n + 2m^3, momentum bytes 12 per element, 16 in fp32 mode).
# For the GPT-2 124M set every matrix has m = 768, and the n of its 72 entries
# sum to 48 * 768 + 24 * 3072 = 110592: per iteration GRAM 768 * 769 * 110592,
# POLY 72 * 768^2 * 769, AXPY 2 * 768^2 * 110592, together 228.43 GFLOP.
TOTALS = {
    # name: (NS GFLOP, dense-equivalent GFLOP, momentum GB, elements)
    "single-64x128-fp32": (0.00924, 0.0131, 0.000131, 8192),
    "gpt2-124m-hidden": (1142.2, 1630.7, 1.019, 84934656),
    "gpt2-350m-hidden": (5413.9, 7730.9, 3.624, 301989888),
    "large-layer-share-4096x14336": (37112, 52227, 6.442, 536870912),
    "moe-64x-2048x1408": (10272, 14997, 4.631, 385875968),
}


@pytest.mark.parametrize("name", sorted(TOTALS))
def test_algorithmic_work_matches_hand_totals(name):
    ns, dense, mom, elems = TOTALS[name]
    w = bench.algorithmic_work(workload(name))
    assert w["elements"] == elems
    assert w["ns_flops_per_step"] / 1e9 == pytest.approx(ns, rel=1e-3)
    assert w["ns_dense_flops_per_step"] / 1e9 == pytest.approx(dense, rel=1e-3)
    assert w["momentum_bytes"] / 1e9 == pytest.approx(mom, rel=1e-3)
    # one AXPY launch does 2 m^2 n; GRAM + POLY + AXPY make one iteration
    f = w["flops"]
    assert 5 * (f["ns_gram"] + f["ns_poly"] + f["ns_axpy"]) == w["ns_flops_per_step"]
    assert f["ns_axpy_update"] == f["ns_axpy"]


def test_gpt2_124m_iteration_by_hand():
    f = bench.algorithmic_work(workload("gpt2-124m-hidden"))["flops"]
    assert f["ns_gram"] == 768 * 769 * 110592
    assert f["ns_poly"] == 72 * 768 ** 2 * 769
    assert f["ns_axpy"] == 2 * 768 ** 2 * 110592


def test_head_pair_blocks_count_per_block():
    """Query and key weights in 128 x 768 blocks: each block is its own m = 128
    entry, so the Gram products shrink while the element count stays."""
    plain = bench.algorithmic_work(workload("gpt2-124m-hidden"))
    pairs = bench.algorithmic_work(workload("gpt2-124m-hidden-qk-head-pairs"))
    assert pairs["elements"] == plain["elements"]
    assert pairs["ns_flops_per_step"] < plain["ns_flops_per_step"]
    # 24 matrices of 768 x 768 become 144 blocks of 128 x 768 (m = 128, n = 768)
    d_gram = 24 * 768 * 769 * 768 - 144 * 128 * 129 * 768
    assert plain["flops"]["ns_gram"] - pairs["flops"]["ns_gram"] == d_gram


def test_summarize_counters_sums_rows_of_a_dispatch(tmp_path):
    p = tmp_path / "run_counter_collection.csv"
    p.write_text(
        "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n"
        "1,k,FETCH_SIZE,10,100,300\n"
        "1,k,FETCH_SIZE,30,100,300\n"
        "2,k,FETCH_SIZE,20,400,500\n"
        "3,j,FETCH_SIZE,7,0,50\n")
    rows = {r["kernel"]: r for r in bench.summarize_counters([str(p)])}
    assert rows["k"]["dispatches"] == 2
    assert rows["k"]["mean_per_dispatch"] == pytest.approx(30.0)   # (10 + 30 + 20) / 2
    assert rows["k"]["mean_dispatch_ns"] == pytest.approx(150.0)   # (200 + 100) / 2
    assert rows["j"]["dispatches"] == 1 and rows["j"]["mean_per_dispatch"] == 7


def test_recorded_figures_need_the_current_sources(tmp_path, monkeypatch):
    """A traffic summary is used only while the kernel and planner sources hash
    to the value it records."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    body = "- `kernel_source_sha256`: `{h}`\n- `fetch_bytes_per_launch`: `123`\n- `write_bytes_per_launch`: `45`\n"
    (prof / "traffic_ns_axpy_w.md").write_text(body.format(h=bench.kernel_source_hash()))
    (prof / "traffic_ns_gram_w.md").write_text(body.format(h="0" * 64))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # the hash itself still reads the repository's sources
    for rel in bench.KERNEL_SOURCES:
        os.makedirs(os.path.dirname(tmp_path / rel), exist_ok=True)
        os.symlink(os.path.join(ROOT, rel), tmp_path / rel)
    assert bench.recorded_traffic("ns_axpy", "w") == {"fetch": 123.0, "write": 45.0}
    assert bench.recorded_traffic("ns_gram", "w") is None
    assert bench.recorded_traffic("ns_poly", "w") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
