#!/usr/bin/env python3
"""Muon step throughput on one MI355X.

One step = the whole hot path over one batch of synthetic input: momentum
update, Frobenius norm, 5 quintic Newton-Schulz iterations and the parameter
update, for every matrix of the workload, through the C ABI (``muon_step``).
Inputs (weights, momenta, every step's gradients) are resident in HBM before
the timed region starts.

Prints ONE JSON line (rank 0): steps/s as ``value``, plus the Newton-Schulz
TFLOP/s, a roofline entry for the dominant kernel (HIP-event timed launches)
and the CPU float64 oracle timed on a bounded sample of the same workload.

``--workload gpt2-124m-adamw-params`` measures the AdamW step of the hybrid
setup's other parameters instead (``muon_adamw_step``), against HBM.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_CLOCK_GHZ = 2.4           # MI355X peak engine clock, which the MFMA peaks assume

METRIC = "Muon steps/sec + NS TFLOP/s (% bf16 MFMA peak), GPT-2-124M matrix set, 1 GPU"
DEFAULT_WORKLOAD = "gpt2-124m-hidden"

GEMM_ROLES = ("ns_gram", "ns_poly", "ns_axpy", "ns_axpy_update")


def block_of(wl, i):
    """(block_rows, block_cols) of matrix i; (0, 0) = the whole matrix."""
    return tuple(wl.blocks[i]) if wl.blocks is not None else (0, 0)


def block_shapes(wl, i):
    """Shapes of the separately orthogonalised blocks of matrix i."""
    s = wl.mats[i]
    br, bc = block_of(wl, i)
    h, w = (br or s.rows), (bc or s.cols)
    return [(h, w)] * ((s.rows // h) * (s.cols // w))


def algorithmic_work(wl):
    """Per-launch algorithmic flops and bytes of each Newton-Schulz role and
    bytes of the momentum pass, summed over the workload's matrices.

    Flops: GRAM m(m+1) n (the m(m+1)/2 distinct entries of X X^T, 2n flops
    each); POLY m^2 (m+1) (distinct entries of A A); AXPY 2 m^2 n.
    Bytes (each input read once, each output written once, as the kernels
    store them; e = 2 bytes per bf16 operand element and a 1-byte remainder of
    the master X, e = 4 and no remainder for float32 entries):
      GRAM  read X (e RC), write A (e m^2);  POLY read A, write B (2 e m^2);
      AXPY, first iteration: read the copy of u (e RC), m' (4 RC), with
        Nesterov g too, and B (e m^2); write X' (copy + remainder);
      AXPY, middle iterations: read and write X (copy + remainder), read B;
      AXPY, last iteration: read X and B, read and write W.
    ``ns_axpy`` averages the first and the middle iterations (the launches
    that role covers); ``ns_axpy_update`` is the last one.
    Momentum pass: read g (2 B bf16 / 4 B fp32) and m (4 B), write m' (4 B)
    and the operand copy of u (2 B bf16 / 4 B fp32).
    """
    gb = 2 if wl.storage == "bf16" else 4
    ub = 2 if wl.compute == "bf16" else 4
    gram = poly = axpy = dense = 0
    b_gram = b_poly = b_first = b_mid = b_last = 0
    elems = 0
    for i, s in enumerate(wl.mats):
        for (r, c) in block_shapes(wl, i):
            m, n = min(r, c), max(r, c)
            gram += m * (m + 1) * n
            poly += m * m * (m + 1)
            axpy += 2 * m * m * n
            dense += 4 * m * m * n + 2 * m ** 3
            f32 = wl.compute == "fp32" or m <= 64
            e, lo = (4, 0) if f32 else (2, 1)
            rc = r * c
            b_gram += e * rc + e * m * m
            b_poly += 2 * e * m * m
            b_first += e * rc + 4 * rc + (gb * rc if wl.nesterov else 0) + e * m * m + (e + lo) * rc
            b_mid += 2 * (e + lo) * rc + e * m * m
            b_last += (e + lo) * rc + e * m * m + 2 * gb * rc
        elems += s.rows * s.cols
    n_axpy = max(wl.ns_steps - 1, 1)
    b_axpy = (b_first + max(wl.ns_steps - 2, 0) * b_mid) / n_axpy
    return {
        "flops": {"ns_gram": gram, "ns_poly": poly, "ns_axpy": axpy, "ns_axpy_update": axpy},
        "bytes": {"ns_gram": b_gram, "ns_poly": b_poly, "ns_axpy": b_axpy, "ns_axpy_update": b_last},
        "ns_flops_per_step": wl.ns_steps * (gram + poly + axpy),
        "ns_dense_flops_per_step": wl.ns_steps * dense,   # the pages' convention, 4 m^2 n + 2 m^3 an iteration
        "momentum_bytes": elems * (gb + 4 + 4 + ub),
        "elements": elems,
    }


KERNEL_SOURCES = ("newton_schulz_matrix_step_amd/csrc/muon_kernels.hip",
                  "newton_schulz_matrix_step_amd/csrc/adamw_kernels.hip",
                  "newton_schulz_matrix_step_amd/csrc/muon_api.cpp",
                  "newton_schulz_matrix_step_amd/csrc/muon_internal.hpp")


def kernel_source_hash() -> str:
    """sha256 over the kernel and planner sources: a recorded HBM-traffic figure
    is reported only while the code it was measured on is unchanged."""
    import hashlib
    hsh = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            hsh.update(f.read())
    return hsh.hexdigest()


def _recorded_values(name: str):
    """The "- `key`: `value`" lines of profiles/<name>.md, or None when the file
    is missing or the kernel sources changed since its counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{name}.md")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                rec[k.strip("`")] = v.strip().strip("`")
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec


def recorded_traffic(role: str, workload_name: str):
    """HBM bytes per launch of ``role`` on ``workload_name`` from the counter
    summary under profiles/ (rocprofv3 FETCH_SIZE and WRITE_SIZE passes, scaled
    by the same counters' reading for a plain copy of known size), or None when
    there is no summary or the kernel sources changed since it was taken."""
    rec = _recorded_values(f"traffic_{role}_{workload_name}")
    try:
        return {"fetch": float(rec["fetch_bytes_per_launch"]), "write": float(rec["write_bytes_per_launch"])}
    except (TypeError, KeyError, ValueError):
        return None


def recorded_clock(role: str, workload_name: str):
    """Mean shader clock (GHz) during launches of ``role`` on ``workload_name``:
    rocprofv3's GRBM_COUNT (cycles, summed over the XCDs) over the dispatch's
    duration, from profiles/clock_<workload>.md; None as for recorded_traffic."""
    rec = _recorded_values(f"clock_{workload_name}")
    try:
        return float(rec[f"clock_ghz_{role}"])
    except (TypeError, KeyError, ValueError):
        return None


def summarize_counters(paths):
    """Mean per dispatch of every counter, per kernel, from rocprofv3
    ``*_counter_collection.csv`` files (rows of one dispatch are summed), with
    the mean duration of those dispatches (their start and end timestamps)."""
    import csv
    from collections import defaultdict
    tot = defaultdict(float)
    disp = defaultdict(dict)
    for p in paths:
        with open(p) as f:
            for r in csv.DictReader(f):
                key = (r["Kernel_Name"], r["Counter_Name"])
                tot[key] += float(r["Counter_Value"])
                disp[key][(p, r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    rows = []
    for (kname, cname), v in sorted(tot.items()):
        d = disp[(kname, cname)]
        nd = len(d)
        rows.append({"kernel": kname, "counter": cname, "dispatches": nd, "mean_per_dispatch": v / nd,
                     "mean_dispatch_ns": sum(d.values()) / nd})
    return rows


def copy_calibration(mib: int, reps: int = 5):
    """A plain device-to-device copy of ``mib`` MiB, ``reps`` times: the known
    byte count against which FETCH_SIZE / WRITE_SIZE readings are scaled."""
    import torch
    dev = torch.device("cuda:0")
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_bytes": n * 4, "reps": reps, "ms_per_copy": round(ms, 4),
                      "read_plus_write_gbs": round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)}), flush=True)


def host_cpu_model() -> str:
    """The host CPU's model name (as lscpu prints it), from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def yardstick(wl, reps: int = 20):
    """The library GEMM as a yardstick: torch.matmul (hipBLASLt, bf16, dense)
    on each distinct product shape of one Newton-Schulz iteration of the
    workload (X X^T as m x n by n x m, A A as m x m by m x m, B X as m x m by
    m x n), one product per shape, timed with events; dense flops 2 m k n."""
    import torch
    dev = torch.device("cuda:0")
    shapes = sorted({(min(r, c), max(r, c)) for i in range(len(wl.mats)) for (r, c) in block_shapes(wl, i)})
    out = []
    for m, n in shapes:
        for what, (a, b) in (("X X^T", ((m, n), (n, m))), ("A A", ((m, m), (m, m))), ("B X", ((m, m), (m, n)))):
            x = torch.randn(*a, device=dev, dtype=torch.bfloat16)
            y = torch.randn(*b, device=dev, dtype=torch.bfloat16)
            for _ in range(3):
                torch.matmul(x, y)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                torch.matmul(x, y)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            fl = 2.0 * a[0] * a[1] * b[1]
            out.append({"product": what, "m": a[0], "k": a[1], "n": b[1], "us": round(ms * 1e3, 2),
                        "tflops": round(fl / (ms * 1e-3) / 1e12, 1)})
    return out


def cpu_baseline(wl, grads_host, budget_s: float):
    """The oracle, as it stands, on the host cores: whole matrices of the first
    step until ``budget_s`` seconds of work, extrapolated to one full step."""
    import oracle
    from muon_synth import make_momentum, make_param

    try:
        from threadpoolctl import threadpool_info
        cores = max((d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    hp = oracle.Hyper(lr=wl.lr, beta=wl.beta, weight_decay=wl.weight_decay, nesterov=wl.nesterov,
                      ns_steps=wl.ns_steps, eps=wl.eps, a=wl.a, b=wl.b, c=wl.c, coeffs=wl.coeffs)
    weights = [sum(min(r, c) ** 2 * (2 * max(r, c) + min(r, c)) for (r, c) in block_shapes(wl, i))
               for i in range(len(wl.mats))]
    total = sum(s.rows * s.cols for s in wl.mats)

    def run(budget):
        # whole passes over the matrix list (step 1's inputs) while the budget
        # lasts; a pass that alone exceeds it stops early and is extrapolated
        done_elems, t_used, k, passes, done_flops = 0, 0.0, 0, 0, 0
        while t_used < budget:
            w = oracle.decode(grads_host["param"][k])
            g = oracle.decode(grads_host["grad0"][k])
            m = np.asarray(make_momentum(wl, k), dtype=np.float64)
            t0 = time.perf_counter()
            if block_of(wl, k) == (0, 0):
                oracle.muon_step_matrix(w, g, m, hp)
            else:
                oracle.muon_step_matrix_blocked(w, g, m, hp, *block_of(wl, k))
            t_used += time.perf_counter() - t0
            done_elems += wl.mats[k].rows * wl.mats[k].cols
            done_flops += weights[k]
            k += 1
            if k == len(wl.mats):
                k = 0
                passes += 1
        # extrapolate by Newton-Schulz flops (the oracle's cost is its dgemms)
        est_step_s = t_used * sum(weights) / max(done_flops, 1)
        if passes:
            what = f"{passes} full step(s) over all {len(wl.mats)} matrices"
            if k:
                what += f" plus {k} matrices"
        else:
            what = f"{k} of {len(wl.mats)} matrices of one step ({done_elems}/{total} elements)"
        return est_step_s, f"{what} with step 1's inputs, {t_used:.1f} s of float64 NumPy/OpenBLAS"

    est, what = run(budget_s)
    out = {
        "value": 1.0 / est,
        "unit": "steps/s",
        "cores": int(cores),
        "cpu_model": host_cpu_model(),
        "kind": "oracle",
        "sample": what + "; steps/s = Newton-Schulz flops of one step / flops done per second",
    }
    try:   # the same oracle on one thread, over a shorter sample
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            est1, what1 = run(min(4.0, budget_s))
        out["one_thread"] = {"value": 1.0 / est1, "cores": 1, "sample": what1}
    except Exception as e:  # pragma: no cover
        out["one_thread"] = {"value": None, "error": str(e)}
    return out


def adamw_bench(args):
    """AdamW over the workload's tensors: one grouped launch a step, inputs
    resident in HBM; bytes per element: read p, g, m, v and write p, m, v."""
    import torch
    import newton_schulz_matrix_step_amd as nsm
    from muon_synth import adamw_workload, encode_storage, make_adamw_grad, make_adamw_param

    wl = adamw_workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n = len(wl.tensors)
    n_sets = args.grad_sets or 2

    def upload(stored):
        if stored.dtype == np.uint16:
            return torch.from_numpy(stored.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(stored, dtype=np.float32)).to(dev)

    t_gen = time.perf_counter()
    host_p = [encode_storage(make_adamw_param(wl, i), wl.storage) for i in range(n)]
    params = [upload(x) for x in host_p]
    ms = [torch.zeros(t.numel, device=dev) for t in wl.tensors]
    vs = [torch.zeros(t.numel, device=dev) for t in wl.tensors]
    host_g0 = None
    grad_sets = []
    for s in range(1, n_sets + 1):
        st = [encode_storage(make_adamw_grad(wl, s, i), wl.storage) for i in range(n)]
        if s == 1:
            host_g0 = st
        grad_sets.append([upload(x) for x in st])
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen

    arrays = []
    for gs in grad_sets:
        arr = (nsm.muon_adamw_tensor * n)()
        for i in range(n):
            arr[i] = nsm.make_adamw_tensor(params[i], gs[i], ms[i], vs[i])
        arrays.append(arr)
    sptr = int(torch.cuda.current_stream(dev).cuda_stream)
    step_no = [0]

    def run_steps(h, k):
        for _ in range(k):
            step_no[0] += 1
            hp = nsm.AdamWHparams(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                                  weight_decay=wl.weight_decay, step=step_no[0]).to_c()
            st = nsm.muon_adamw_step_raw(h, arrays[step_no[0] % n_sets], n, hp, sptr)
            if st != 0:
                raise nsm.MuonError(st, nsm.muon_last_error(h))

    h = nsm.muon_init(0, nsm.MUON_INIT_PROFILE)
    run_steps(h, args.warmup)
    torch.cuda.synchronize()
    nsm.muon_kernel_stats_reset(h)
    t0 = time.perf_counter()
    run_steps(h, args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stats = nsm.muon_kernel_stats_read(h)
    nsm.muon_destroy(h)
    ms_per_step = elapsed * 1e3 / args.steps
    launches, total_ms = stats["adamw"]
    avg_s = total_ms * 1e-3 / launches
    eb = (2 + 2 + 4 + 4 + 2 + 4 + 4) if wl.storage == "bf16" else (4 + 4 + 4 + 4 + 4 + 4 + 4)
    bytes_per_launch = wl.elements * eb
    achieved = bytes_per_launch / avg_s / 1e9
    out = {
        "metric": "AdamW steps/sec, GPT-2-124M non-matrix parameter set, 1 GPU",
        "value": round(1e3 / ms_per_step, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "tensors": n, "elements": wl.elements, "storage": wl.storage,
                   "grad_sets": n_sets},
        "roofline": {"kernel": "adamw_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": None, "algorithmic_bytes": bytes_per_launch, "bytes_per_element": eb},
        "kernels": {"adamw": {"launches": launches, "avg_us": round(avg_s * 1e6, 2)}},
        "input_gen_s": round(gen_s, 1),
    }
    tr = recorded_traffic("adamw", wl.name)
    if tr is not None:
        out["roofline"]["traffic"] = round(tr["fetch"] + tr["write"])
        out["roofline"]["traffic_fetch"] = round(tr["fetch"])
        out["roofline"]["traffic_write"] = round(tr["write"])
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            cores = max((d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"),
                        default=1)
        except Exception:  # pragma: no cover
            cores = 1
        hyper = oracle.AdamWHyper(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                                  weight_decay=wl.weight_decay)
        done, t_used, k = 0, 0.0, 0
        while t_used < args.cpu_budget and k < n:
            p = oracle.decode(host_p[k])
            g = oracle.decode(host_g0[k])
            z = np.zeros_like(p)
            t1 = time.perf_counter()
            oracle.adamw_step(p, g, z, z, hyper, 1)
            t_used += time.perf_counter() - t1
            done += wl.tensors[k].numel
            k += 1
        out["cpu_baseline"] = {"value": round(1.0 / (t_used * wl.elements / max(done, 1)), 4), "unit": "steps/s",
                               "cores": int(cores), "cpu_model": host_cpu_model(), "kind": "oracle",
                               "sample": f"{k} of {n} tensors of step 1 ({done}/{wl.elements} elements), "
                                         f"{t_used:.1f} s of float64 NumPy, extrapolated by elements"}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--grad-sets", type=int, default=0,
                    help="distinct seeded gradient sets resident in HBM (default: the workload's step count)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--yardstick", action="store_true",
                    help="only time torch.matmul (hipBLASLt) on the workload's product shapes and exit")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration) and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="only print per-kernel means of rocprofv3 counter CSV files and exit")
    args = ap.parse_args()

    if args.summarize_counters:
        for r in summarize_counters(args.summarize_counters):
            print(json.dumps(r))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (every matrix's step is "
              "independent and the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return

    if args.yardstick:
        from muon_synth import workload as _wl
        print(json.dumps({"yardstick": "torch.matmul bf16", "workload": args.workload,
                          "products": yardstick(_wl(args.workload))}), flush=True)
        return

    from muon_synth import ADAMW_WORKLOADS
    if args.workload in ADAMW_WORKLOADS:
        adamw_bench(args)
        return

    import torch
    import newton_schulz_matrix_step_amd as nsm
    from muon_synth import encode_storage, make_grad, make_momentum, make_param, workload

    wl = workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n = len(wl.mats)
    n_sets = args.grad_sets or wl.steps

    def upload(stored):
        if stored.dtype == np.uint16:
            return torch.from_numpy(stored.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(stored).to(dev)

    t_gen = time.perf_counter()
    host = {"param": [encode_storage(make_param(wl, i), wl.storage) for i in range(n)]}
    params = [upload(x) for x in host["param"]]
    moms = [upload(encode_storage(make_momentum(wl, i), "fp32")) for i in range(n)]
    grad_sets = []
    for s in range(1, n_sets + 1):
        st = [encode_storage(make_grad(wl, s, i), wl.storage) for i in range(n)]
        if s == 1:
            host["grad0"] = st
        grad_sets.append([upload(x) for x in st])
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen

    hp_c = nsm.Hparams(lr=wl.lr, beta=wl.beta, weight_decay=wl.weight_decay, eps=wl.eps, a=wl.a, b=wl.b, c=wl.c,
                       nesterov=wl.nesterov, ns_steps=wl.ns_steps, compute=wl.compute, coeffs=wl.coeffs).to_c()
    arrays = []
    for gs in grad_sets:
        arr = (nsm.muon_matrix * n)()
        for i in range(n):
            arr[i] = nsm.make_matrix(params[i], gs[i], moms[i], block=block_of(wl, i))
        arrays.append(arr)
    stream = torch.cuda.current_stream(dev)
    sptr = int(stream.cuda_stream)

    def run_steps(h, k, start):
        for j in range(k):
            st = nsm.muon_step_raw(h, arrays[(start + j) % n_sets], n, hp_c, sptr)
            if st != 0:
                raise nsm.MuonError(st, nsm.muon_last_error(h))

    work = algorithmic_work(wl)

    # ---- per-kernel table: an untimed pass of the same steps on a handle
    # that brackets every launch with HIP events ----
    h = nsm.muon_init(0, nsm.MUON_INIT_PROFILE)
    run_steps(h, args.warmup, 0)
    torch.cuda.synchronize()
    nsm.muon_kernel_stats_reset(h)
    run_steps(h, args.steps, args.warmup)
    torch.cuda.synchronize()
    stats = nsm.muon_kernel_stats_read(h)
    ws_bytes = nsm.muon_workspace_bytes(h)
    nsm.muon_destroy(h)
    dom = max((r for r in GEMM_ROLES if r in stats), key=lambda r: stats[r][1])

    # ---- timed region: only the dominant kernel's launches carry HIP events
    # (on the launch stream), so its average duration comes from the very
    # steps that are timed, at the cost of events on 1 launch in 3 or 4 ----
    h = nsm.muon_init(0, nsm.MUON_INIT_PROFILE | nsm.profile_roles([dom]))
    run_steps(h, args.warmup, 0)
    torch.cuda.synchronize()
    nsm.muon_kernel_stats_reset(h)
    t0 = time.perf_counter()
    run_steps(h, args.steps, args.warmup)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_stats = nsm.muon_kernel_stats_read(h)[dom]
    nsm.muon_destroy(h)
    ms_per_step = elapsed * 1e3 / args.steps

    # ---- the same steps on a plain handle (no per-kernel events), for
    # comparison, each step bracketed by events on the launch stream for the
    # distribution of step times ----
    h = nsm.muon_init(0)
    run_steps(h, args.warmup, 0)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for j in range(args.steps):
        run_steps(h, 1, args.warmup + j)
        evs[j + 1].record(stream)
    torch.cuda.synchronize()
    plain_ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    step_ms = np.array([evs[j].elapsed_time(evs[j + 1]) for j in range(args.steps)])

    # ---- the step captured once into a HIP graph and replayed (one gradient
    # set; after a call with the same pointers a step enqueues kernels only) ----
    graph_ms = None
    if not args.no_graph:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        side_ptr = int(side.cuda_stream)
        st = nsm.muon_step_raw(h, arrays[0], n, hp_c, side_ptr)
        if st != 0:
            raise nsm.MuonError(st, nsm.muon_last_error(h))
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            st = nsm.muon_step_raw(h, arrays[0], n, hp_c, side_ptr)
        if st != 0:
            raise nsm.MuonError(st, nsm.muon_last_error(h))
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps
        del graph
    nsm.muon_destroy(h)

    kernels = {}
    for name, (launches, total_ms) in stats.items():
        avg_us = total_ms * 1e3 / max(launches, 1)
        ent = {"launches": launches, "avg_us": round(avg_us, 2), "ms_per_step": round(total_ms / args.steps, 4)}
        if name in work["flops"]:
            ent["tflops"] = round(work["flops"][name] / (avg_us * 1e-6) / 1e12, 2)
            ent["gbs"] = round(work["bytes"][name] / (avg_us * 1e-6) / 1e9, 1)
        if name == "momentum_norm":
            ent["gbs"] = round(work["momentum_bytes"] / (avg_us * 1e-6) / 1e9, 1)
        kernels[name] = ent
    ns_ms = sum(stats[r][1] for r in GEMM_ROLES if r in stats) / args.steps
    ns_tflops = work["ns_flops_per_step"] / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else 0.0
    peak = PEAK_BF16_TFLOPS if wl.compute == "bf16" else PEAK_FP32_TFLOPS

    dom_avg_s = dom_stats[1] * 1e-3 / dom_stats[0]
    # the kernel's roofline: algorithmic flops against the MFMA peak and
    # algorithmic bytes against HBM; the one that takes longer at its peak
    # bounds the kernel and is the one reported
    flops, nbytes = work["flops"][dom], work["bytes"][dom]
    t_mfma, t_hbm = flops / (peak * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)
    mfma_frac = t_mfma / dom_avg_s
    hbm_frac = t_hbm / dom_avg_s
    # the phase's launches: 128-wide tiles, and 256-wide ones for large matrices
    kname = f"ns_gemm_bf16 / ns_gemm_wide ({dom})" if wl.compute == "bf16" else f"ns_gemm_kernel ({dom})"
    if t_mfma >= t_hbm:
        roofline = {"kernel": kname, "bound": "mfma", "achieved": round(flops / dom_avg_s / 1e12, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(mfma_frac, 4)}
    else:
        roofline = {"kernel": kname, "bound": "hbm", "achieved": round(nbytes / dom_avg_s / 1e9, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(hbm_frac, 4)}
    roofline.update({
        "traffic": None,
        "algorithmic_flops": int(flops),
        "algorithmic_bytes": int(nbytes),
        "flop_per_byte": round(flops / nbytes, 1),
        "ridge_flop_per_byte": round(peak * 1e12 / (PEAK_HBM_GBS * 1e9), 1),
        "mfma_frac": round(mfma_frac, 4),
        "hbm_frac": round(hbm_frac, 4),
        "avg_launch_us": round(dom_avg_s * 1e6, 2),
    })
    tr = recorded_traffic(dom, wl.name)
    if tr is not None:
        roofline["traffic"] = round(tr["fetch"] + tr["write"])
        roofline["traffic_fetch"] = round(tr["fetch"])
        roofline["traffic_write"] = round(tr["write"])
    # the published MFMA peak assumes the 2.4 GHz peak engine clock; under a
    # sustained matrix load the chip runs slower, so the fraction of the peak
    # at the clock the kernel actually ran at is reported beside it
    clk = recorded_clock(dom, wl.name)
    roofline["clock_ghz"] = clk
    if clk is not None:
        roofline["mfma_peak_at_clock"] = round(peak * clk / PEAK_CLOCK_GHZ, 1)
        roofline["mfma_frac_at_clock"] = round(mfma_frac * PEAK_CLOCK_GHZ / clk, 4)
    mom = kernels.get("momentum_norm", {})

    out = {
        "metric": METRIC,
        "value": round(args.steps / elapsed, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_no_events": round(plain_ms_per_step, 4),
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 4) for q in (10, 50, 90)],
        "ms_per_step_hip_graph": round(graph_ms, 4) if graph_ms is not None else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.compute,
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "matrices": n,
            "plan_entries": sum(len(block_shapes(wl, i)) for i in range(n)),
            "elements": work["elements"],
            "ns_steps": wl.ns_steps,
            "storage": wl.storage,
            "grad_sets": n_sets,
            "nesterov": wl.nesterov,
            "weight_decay": wl.weight_decay,
        },
        "ns_tflops": round(ns_tflops, 2),
        "ns_tflops_dense_equiv": round(work["ns_dense_flops_per_step"] / (ns_ms * 1e-3) / 1e12, 2) if ns_ms > 0 else 0.0,
        "ns_frac_peak": round(ns_tflops / peak, 4),
        "ns_ms_per_step": round(ns_ms, 4),
        "momentum_hbm_frac": round(mom.get("gbs", 0.0) / PEAK_HBM_GBS, 4) if mom else None,
        "roofline": roofline,
        "kernels": kernels,
        "kernels_note": "per-kernel figures from an untimed pass of the same steps with events on every "
                        "launch; the roofline kernel is timed inside the timed region",
        "workspace_gb": round(ws_bytes / 1e9, 3),
        "input_gen_s": round(gen_s, 1),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, host, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
