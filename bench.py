"""Benchmark of the exact attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]
    python bench.py --sweep {c1,c2,c4,c5,bwd} > sweep.jsonl (per-case timing, see below)
    python bench.py --summarize-sweep sweep.jsonl           (markdown table of those lines)

Workload (default): B=1, H=8, Sq=Sk=8192, d=128, Q/K/V i.i.d. N(0,1) rounded to bf16,
scale 1/sqrt(d).  One step is one forward pass of the whole path over that batch in
both mask modes: non-causal, then causal (two launches of the same kernel).  Inputs
are resident in device memory before the timed region.  Throughput counts
4*B*H*Sq*Sk*d FLOPs per non-causal pass and half of that per causal pass.

Prints one JSON line.  Besides the headline throughput it carries
  roofline      the dominant kernel's (the non-causal launch's) achieved TFLOP/s from
                HIP events around each of its launches in the timed region, against
                the bf16 dense MFMA peak; `traffic` is its HBM bytes per launch
                measured by rocprofv3 counters (profiles/), or null when that
                measurement does not match the current kernel source;
  cpu_baseline  the fp64 CPU oracle timed on this host on a bounded sample;
  clock         the shader clock under the dominant kernel (sampled through amdsmi while
                it runs back to back, outside the timed region), with the roofline
                fraction also against the peak at that clock;
  environment   GPU name / arch / CUs, ROCm, hipcc and torch versions, CPU model, host
                cores, NumPy and its BLAS.
Before the warm-up, attn_tune picks and stores the launch plan of each mask for the
workload's shape (--no-tune: the fixed rule); config.plans records them.
With the CPU leg, a few sampled rows of two heads are also checked against the oracle's
outputs (outside the timed region).

--sweep times the other workloads case by case (one JSON line per case and mask): every
call timed alone with HIP events on its stream after a 512 MiB device read that evicts
the inputs from L2 and the 256 MB last-level cache, medians over the reps.  c1 (fp32
B=1,H=2,S=128,d=64) reports microseconds; c2 and the 36 c4 cases (d in 64/128/256, S in
512/1000/2048, B in 1/8, H=16, bf16 with 1 % of query rows scaled by 30) report TFLOP/s
against min(bf16 MFMA peak, intensity x 8 TB/s); c5 (fp8 B=1,H=8,Sq=128,Sk=32768,d=128)
times attn_fwd_splitkv and attn_merge apart for n = 1, 4, 16 and reports the algorithmic
bytes (Q, K, V read once, O and lse written once) per second against 8 TB/s.  bwd times
attn_bwd (three launches: prologue, dK/dV, dQ) at the c3 and c2 shapes and at B=1, H=16,
S=2048, d=256, with inputs
resident (repeated calls), counting 10*B*H*Sq*Sk*d FLOPs (2.5x the forward's: the five
products S, dP, dV, dK, dQ; half causal) against the bf16 MFMA peak, and times the fp64
oracle's backward on one head beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "exact_attention_82_amd", "csrc", "attn_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_attn_fwd_bf16_d128_B1_H8_S8192.txt")

WORKLOADS = {
    # name: (B, H, S, d, seed)
    "c3": (1, 8, 8192, 128, 3),
    "c2": (8, 32, 2048, 64, 2),
}


def kernel_source_digest() -> str:
    """Hash of the forward kernels' source: the kernel file up to its backward section (so
    that a change to the backward kernels does not invalidate the forward's counters)."""
    with open(KERNEL_SOURCE, "rb") as f:
        text = f.read()
    cut = text.find(b"// " + b"=" * 66 + b" backward")
    return hashlib.sha256(text[:cut] if cut > 0 else text).hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from the committed counter summary, if it matches the source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_digest():
        return None
    if ROOFLINE_KERNEL not in kv.get("kernel", ""):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _csv_rows(d: str, suffix: str):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, f"*{suffix}"))):
        rows.extend(csv.DictReader(open(f)))
    return rows


def summarize_stats(d: str) -> str:
    """Markdown table of a `rocprofv3 --kernel-trace --stats` output directory."""
    out = ["| kernel | calls | avg ns | min ns | max ns | % time |", "|---|---|---|---|---|---|"]
    for r in _csv_rows(d, "_kernel_stats.csv"):
        out.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                   f"{r['MaxNs']} | {r['Percentage']} |")
    return "\n".join(out)


# The kernel instance the roofline describes: the non-causal forward of the workload,
# which takes most of a step's time (the causal pass runs the tile-pair kernel).
ROOFLINE_KERNEL = "attn_fwd_kernel<1, 128, 32, 0>"


def summarize_traffic(fetch_dir: str, write_dir: str, probe_mib: int, workload: str = "c3",
                      kernel: str = ROOFLINE_KERNEL) -> str:
    """HBM bytes per launch of one attention kernel instance from two `rocprofv3 --pmc`
    runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the plain device copy of `probe_mib` MiB that `--copy-probe-mib`
    runs."""
    B, H, S, d, _ = WORKLOADS[workload]
    vals = {}
    for name, dd in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _csv_rows(dd, "_counter_collection.csv") if r["Counter_Name"] == name]
        kern = [float(r["Counter_Value"]) for r in rows if kernel in r["Kernel_Name"]]
        copies = sorted(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        probe = float(np.median(copies[-3:]))
        vals[name] = (float(np.mean(kern)), len(kern), probe, probe_mib * 1024.0 / probe)
        kname = next(r["Kernel_Name"] for r in rows if kernel in r["Kernel_Name"])
    rd = vals["FETCH_SIZE"][0] * vals["FETCH_SIZE"][3] * 1024
    wr = vals["WRITE_SIZE"][0] * vals["WRITE_SIZE"][3] * 1024
    alg = 3 * B * H * S * d * 2 + B * H * S * d * 4 + B * H * S * 4  # per non-causal launch
    return "\n".join([
        f"kernel: {kname}",
        f"kernel_source_sha256_16: {kernel_source_digest()}",
        f"launches_measured: {vals['FETCH_SIZE'][1]}",
        f"FETCH_SIZE_KiB_per_launch_raw: {vals['FETCH_SIZE'][0]:.1f}",
        f"WRITE_SIZE_KiB_per_launch_raw: {vals['WRITE_SIZE'][0]:.1f}",
        f"copy_probe_FETCH_SIZE_KiB_raw: {vals['FETCH_SIZE'][2]:.1f}",
        f"copy_probe_WRITE_SIZE_KiB_raw: {vals['WRITE_SIZE'][2]:.1f}",
        f"fetch_calibration_factor: {vals['FETCH_SIZE'][3]:.4f}",
        f"write_calibration_factor: {vals['WRITE_SIZE'][3]:.4f}",
        f"hbm_read_bytes_per_launch: {rd:.0f}",
        f"hbm_write_bytes_per_launch: {wr:.0f}",
        f"hbm_bytes_per_launch: {rd + wr:.0f}",
        f"algorithmic_bytes_per_launch: {alg}",
        f"traffic_over_algorithmic: {(rd + wr) / alg:.4f}",
    ])


def _kernel_key(r) -> str:
    """Short name of an attention kernel instance plus its workgroup count (one kernel
    instance serves several grid sizes, e.g. split counts)."""
    k = r["Kernel_Name"].replace("void attn::(anonymous namespace)::", "").split("(attn::")[0]
    grid = int(float(r.get("Grid_Size") or r.get("Grid_Size_X") or 0))
    wg = int(float(r.get("Workgroup_Size") or r.get("Workgroup_Size_X") or 0))
    return f"{k} [{grid // wg} wg]" if grid and wg else k


def summarize_traffic_grid(fetch_dir: str, write_dir: str, probe_mib: int) -> str:
    """HBM bytes per launch of every attention kernel instance and grid in two `rocprofv3
    --pmc` runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch, summed over instances),
    each scaled by what the same counter reads for the plain device copy of `probe_mib`
    MiB that the run's --copy-probe-mib performs."""
    res = {}
    factors = {}
    for name, dd in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per, copies = {}, []
        for r in _csv_rows(dd, "_counter_collection.csv"):
            if r["Counter_Name"] != name:
                continue
            if "copyBuffer" in r["Kernel_Name"]:
                copies.append(float(r["Counter_Value"]))
            elif "attn_" in r["Kernel_Name"]:
                key = (_kernel_key(r), r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        probe = float(np.median(sorted(copies)[-3:]))
        factors[name] = (probe, probe_mib * 1024.0 / probe)
        for (k, _), v in per.items():
            res.setdefault((k, name), []).append(v)
    out = [f"copy probe {probe_mib} MiB: FETCH_SIZE {factors['FETCH_SIZE'][0]:.1f} KiB "
           f"(factor {factors['FETCH_SIZE'][1]:.4f}), WRITE_SIZE {factors['WRITE_SIZE'][0]:.1f} KiB "
           f"(factor {factors['WRITE_SIZE'][1]:.4f})", "",
           "| kernel [workgroups] | launches | HBM read MB / launch | HBM write MB / launch |",
           "|---|---|---|---|"]
    for k in sorted({k for (k, _) in res}):
        rd = np.mean(res.get((k, "FETCH_SIZE"), [np.nan])) * factors["FETCH_SIZE"][1] * 1024 / 1e6
        wr = np.mean(res.get((k, "WRITE_SIZE"), [np.nan])) * factors["WRITE_SIZE"][1] * 1024 / 1e6
        out.append(f"| {k} | {len(res.get((k, 'FETCH_SIZE'), []))} | {rd:.2f} | {wr:.2f} |")
    return "\n".join(out)


def summarize_pmc(dirs) -> str:
    """Markdown table of `rocprofv3 --pmc` counter runs (one directory per pass): the mean
    per dispatch of every counter, for each attention kernel instance and grid seen."""
    acc = {}
    for d in dirs:
        per = {}
        for r in _csv_rows(d, "_counter_collection.csv"):
            if "attn_" not in r["Kernel_Name"]:
                continue
            key = (_kernel_key(r), r["Counter_Name"], r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])  # sum over instances
        for (k, c, _), v in per.items():
            acc.setdefault((k, c), []).append(v)
    dur = {}
    for d in dirs:
        for r in _csv_rows(d, "_kernel_trace.csv"):
            if "attn_" in r["Kernel_Name"]:
                dur.setdefault(_kernel_key(r), []).append(
                    (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-3)
    out = ["| kernel | counter | dispatches | mean per dispatch |", "|---|---|---|---|"]
    for k, us in sorted(dur.items()):
        out.append(f"| {k} | duration (us, counter runs) | {len(us)} | {np.mean(us):.1f} |")
    for (k, c), vs in sorted(acc.items()):
        out.append(f"| {k} | {c} | {len(vs)} | {np.mean(vs):.6g} |")
    return "\n".join(out)


def _gfx_clock_sampler():
    """A function returning (shader clock in MHz, graphics activity in %) of the GPU, read
    through amdsmi from the SMU's metrics table (mean over the XCDs' clocks), and a
    description of the source; (None, reason) if amdsmi cannot be used here.  Read-only
    queries."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
    except Exception as e:  # noqa: BLE001
        return None, f"amdsmi unavailable: {type(e).__name__}"
    if not handles:
        return None, "amdsmi lists no GPU"
    vis = os.environ.get("HIP_VISIBLE_DEVICES") or os.environ.get("ROCR_VISIBLE_DEVICES") or "0"
    idx = int(vis.split(",")[0]) if vis.split(",")[0].isdigit() else 0
    h = handles[idx if idx < len(handles) else 0]

    def num(x):
        return float(x) if isinstance(x, (int, float)) and 0 < x < 10000 else None

    def read():
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        except Exception:  # noqa: BLE001
            return None, None
        xs = [num(x) for x in (m.get("current_gfxclks") or [])]
        xs = [x for x in xs if x is not None]
        clk = float(np.mean(xs)) if xs else num(m.get("current_gfxclk"))
        act = m.get("average_gfx_activity")
        return clk, (float(act) if isinstance(act, (int, float)) else None)
    return read, "amdsmi gpu_metrics current_gfxclks (mean over the XCDs)"


def measure_clock(launch, torch, seconds: float = 2.5):
    """The shader clock under the dominant kernel, taken outside the timed region: the
    kernel is launched back to back for `seconds` while a host thread samples the SMU's
    metrics table (refreshed about once a second); samples taken while the graphics
    activity reads >= 50 % count.  Returns {"mhz": median, "samples": n, "source": ...}."""
    import threading
    read, src = _gfx_clock_sampler()
    if read is None:
        return {"mhz": None, "samples": 0, "source": src}
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            clk, act = read()
            if clk is not None and act is not None and act >= 50.0:
                samples.append(clk)
            time.sleep(0.02)
    launch()
    torch.cuda.synchronize()
    th = threading.Thread(target=poll, daemon=True)
    t_end = time.perf_counter() + seconds
    th.start()
    while time.perf_counter() < t_end:
        for _ in range(20):
            launch()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    return {"mhz": round(float(np.median(samples)), 1) if samples else None,
            "samples": len(samples), "source": src}


def environment(torch, dev) -> dict:
    """Versions and hardware the measurement ran on (recorded beside the numbers)."""
    import platform
    env = {}
    try:
        pr = torch.cuda.get_device_properties(dev)
        env["gpu"] = pr.name
        env["gpu_arch"] = getattr(pr, "gcnArchName", None)
        env["gpu_cus"] = pr.multi_processor_count
    except Exception as e:  # noqa: BLE001
        env["gpu"] = f"unknown ({type(e).__name__})"
    env["torch"] = torch.__version__
    env["torch_hip"] = getattr(torch.version, "hip", None)
    try:
        env["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        env["rocm"] = None
    # the HIP compiler's version from the installed header, not by running hipcc: this
    # process has initialised the GPU, and its children must not replace themselves
    try:
        hv = {}
        for line in open("/opt/rocm/include/hip/hip_version.h"):
            parts = line.split()
            if len(parts) == 3 and parts[0] == "#define" and parts[1].startswith("HIP_VERSION_"):
                hv[parts[1]] = parts[2].strip('"')
        env["hipcc"] = (f"HIP version: {hv['HIP_VERSION_MAJOR']}.{hv['HIP_VERSION_MINOR']}."
                        f"{hv['HIP_VERSION_PATCH']}-{hv.get('HIP_VERSION_GITHASH', '')}")
    except (OSError, KeyError):
        env["hipcc"] = None
    cpu = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    env["cpu"] = cpu or platform.processor()
    env["host_cores"] = len(os.sched_getaffinity(0))
    env["numpy"] = np.__version__
    try:
        cfg = np.show_config(mode="dicts")
        blas = cfg.get("Build Dependencies", {}).get("blas", {})
        env["blas"] = f"{blas.get('name')} {blas.get('version')}".strip()
    except Exception:  # noqa: BLE001
        env["blas"] = None
    return env


def cpu_baseline(inp, scale, budget_s: float, gpu_out):
    """The CPU leg: time the fp64 oracle on whole heads of the same workload, both masks,
    head after head (cycling through the heads), until the time budget is used; and, with
    the oracle's outputs, check sampled rows of the GPU outputs (two heads, both masks).
    Returns (baseline record, max |dO| over the checked rows)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    B, H, S, d = inp.B, inp.H, inp.Sq, inp.d
    q = inp.q64.reshape(B * H, S, d)
    k = inp.k64.reshape(B * H, S, d)
    v = inp.v64.reshape(B * H, S, d)
    rows = np.array([0, 1, 127, 128, S // 2, S - 129, S - 1])
    worst = 0.0
    flops = 0.0
    heads = 0
    t0 = time.perf_counter()
    while True:
        h = heads % (B * H)
        for causal in (False, True):
            ro, _ = oracle.attention(q[h], k[h], v[h], scale, causal)
            flops += oracle.flops(1, 1, S, S, d, causal)
            if heads < B * H and h in (0, B * H - 1):
                worst = max(worst, float(np.abs(gpu_out[causal][h][rows] - ro[rows]).max()))
        heads += 1
        if time.perf_counter() - t0 >= budget_s and heads >= B * H:
            break
    dt = time.perf_counter() - t0
    rec = {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
           "sample": f"{heads} (batch, head) pass(es) over the {B * H} heads of B={B},H={H},S={S},"
                     f"d={d} bf16 inputs (cycling), non-causal and causal each, fp64 NumPy "
                     f"oracle materialising the full score matrix, {dt:.1f} s"}
    return rec, worst


def _alg_bytes(B, H, Sq, Sk, d, in_bytes):
    """Q, K, V read once at their storage width, O and lse (fp32) written once."""
    return (B * H * Sq * d + 2 * B * H * Sk * d) * in_bytes + B * H * Sq * (d + 1) * 4


def _timed_calls(fn, reps, flush):
    """Per-call HIP-event durations (us) on the current stream, each call after a cache
    flush outside the event window: a read of a 512 MiB buffer, which leaves the caches
    full of clean lines (a write would leave dirty lines whose write-back lands inside
    the next timed call)."""
    import torch
    out = []
    for _ in range(reps):
        flush.sum()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3)
    return np.array(out)


def _stats(us):
    return {"median_us": round(float(np.median(us)), 2), "p10_us": round(float(np.percentile(us, 10)), 2),
            "p90_us": round(float(np.percentile(us, 90)), 2), "min_us": round(float(us.min()), 2)}


def sweep(name: str, reps: int, warmup: int, splits=None, seqs=None, masks=(False, True),
          copy_probe_mib: int = 0):
    """Per-case timing of the parity workloads; prints one JSON line per case.  splits
    (c5), seqs (c4) and masks (c1, c2, c4) restrict the cases; copy_probe_mib runs the
    plain device copy that calibrates rocprofv3's FETCH_SIZE / WRITE_SIZE counters
    first."""
    import torch
    import exact_attention_82_amd as ea
    import synthetic_inputs as si

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = torch.zeros(128 << 20, dtype=torch.float32, device=dev)  # 512 MiB
    if copy_probe_mib:
        src = torch.ones(copy_probe_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def to_dev(inp):
        if inp.dtype == "bf16":
            return tuple(torch.from_numpy(t.view(np.int16)).view(torch.bfloat16).to(dev)
                         for t in (inp.q, inp.k, inp.v))
        return tuple(torch.from_numpy(np.ascontiguousarray(t)).to(dev) for t in (inp.q, inp.k, inp.v))

    def emit(rec):
        print(json.dumps(rec), flush=True)

    if name in ("c1", "c2", "c4"):
        if name == "c1":
            cases = [(1, 2, 128, 64, 1, "f32", 0.0)]
        elif name == "c2":
            cases = [(8, 32, 2048, 64, 2, "bf16", 0.0)]
        else:
            cases = [(B, 16, S, d, 400 + (d // 64) * 100 + S // 100 + B, "bf16", 0.01)
                     for d in (64, 128, 256) for S in (512, 1000, 2048) for B in (1, 8)
                     if not seqs or S in seqs]
        for (B, H, S, d, seed, dt, hot) in cases:
            inp = si.make_attention_inputs(B, H, S, S, d, seed=seed, dtype=dt, hot_row_frac=hot)
            q, k, v = to_dev(inp)
            del inp
            scale = float(np.float32(1.0 / np.sqrt(d)))
            o = torch.empty((B, H, S, d), dtype=torch.float32, device=dev)
            lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
            in_bytes = 4 if dt == "f32" else 2
            for causal in masks:
                fn = lambda: ea.attn_fwd(q, k, v, scale=scale, causal=causal, out=o, lse=lse)
                for _ in range(warmup):
                    fn()
                torch.cuda.synchronize()
                us = _timed_calls(fn, reps, flush)
                fl = 4.0 * B * H * S * S * d / (2.0 if causal else 1.0)
                ab = _alg_bytes(B, H, S, S, d, in_bytes)
                rec = {"workload": name, "B": B, "H": H, "Sq": S, "Sk": S, "d": d, "dtype": dt,
                       "causal": causal, "kernel": ea.attn_kernel_name(B, H, S, S, d, int(causal),
                                                                       ea.dtype_code(q)),
                       "reps": reps, **_stats(us)}
                if dt != "f32":
                    tf = fl / (float(np.median(us)) * 1e-6) / 1e12
                    bound = min(PEAK_BF16_TFLOPS, fl / ab * PEAK_HBM_GBS / 1e3)
                    rec.update({"tflops": round(tf, 2), "flop_per_byte": round(fl / ab, 1),
                                "bound_tflops": round(bound, 1),
                                "bound": "mfma" if bound >= PEAK_BF16_TFLOPS else "hbm",
                                "pct_of_bound": round(100.0 * tf / bound, 2)})
                emit(rec)
            del q, k, v, o, lse
            torch.cuda.empty_cache()
        return
    if name == "out16":
        # O written as bf16 (attn_fwd_ex) against fp32 O (attn_fwd): c3, c2 and the
        # HBM-bound c4 shapes at S=512, where O is most of the bytes.
        for (B, H, S, d, seed) in ((1, 8, 8192, 128, 3), (8, 32, 2048, 64, 2), (8, 16, 512, 128, 441),
                                   (8, 16, 512, 64, 341)):
            inp = si.make_attention_inputs(B, H, S, S, d, seed=seed, dtype="bf16")
            q, k, v = to_dev(inp)
            del inp
            scale = float(np.float32(1.0 / np.sqrt(d)))
            o32 = torch.empty((B, H, S, d), dtype=torch.float32, device=dev)
            o16 = torch.empty((B, H, S, d), dtype=torch.bfloat16, device=dev)
            lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
            for causal in (False, True):
                f32 = lambda: ea.attn_fwd(q, k, v, scale=scale, causal=causal, out=o32, lse=lse)
                f16 = lambda: ea.attn_fwd_ex(q, k, v, scale=scale, causal=causal, out_dtype=torch.bfloat16,
                                             out=o16, lse=lse)
                for _ in range(warmup):
                    f32()
                    f16()
                torch.cuda.synchronize()
                u32 = _timed_calls(f32, reps, flush)
                u16 = _timed_calls(f16, reps, flush)
                fl = 4.0 * B * H * S * S * d / (2.0 if causal else 1.0)
                emit({"workload": "out16", "B": B, "H": H, "Sq": S, "Sk": S, "d": d, "dtype": "bf16",
                      "causal": causal, "kernel": ea.attn_kernel_name(B, H, S, S, d, int(causal), ea.ATTN_BF16),
                      "reps": reps, "fp32_out": _stats(u32), "bf16_out": _stats(u16),
                      "tflops_fp32_out": round(fl / (float(np.median(u32)) * 1e-6) / 1e12, 2),
                      "tflops_bf16_out": round(fl / (float(np.median(u16)) * 1e-6) / 1e12, 2)})
            del q, k, v, o32, o16, lse
            torch.cuda.empty_cache()
        return
    if name == "varlen":
        # ragged batches: 16 sequences of 256..4096 tokens (uniform, seeded), H=16, bf16;
        # useful FLOPs = sum over sequences of 4*H*l^2*d (half causal).  The same batch
        # padded to its longest sequence and run through attn_fwd is timed beside it.
        for d, seed in ((64, 31), (128, 32)):
            H = 16
            lens = si.varlen_lengths(16, 256, 4096, seed=seed)
            inp, cu_q, cu_k = si.make_varlen_inputs(lens, lens, H, d, seed=seed + 100, dtype="bf16")
            q, k, v = (t[0] for t in to_dev(inp))
            del inp
            cq, ck = torch.from_numpy(cu_q).to(dev), torch.from_numpy(cu_k).to(dev)
            T, M, B = int(cu_q[-1]), int(lens.max()), len(lens)
            o = torch.empty((H, T, d), dtype=torch.float32, device=dev)
            lse = torch.empty((H, T), dtype=torch.float32, device=dev)
            pad = si.make_attention_inputs(B, H, M, M, d, seed=seed + 200, dtype="bf16")
            pq, pk, pv = to_dev(pad)
            del pad
            po = torch.empty((B, H, M, d), dtype=torch.float32, device=dev)
            pl = torch.empty((B, H, M), dtype=torch.float32, device=dev)
            scale = float(np.float32(1.0 / np.sqrt(d)))
            for causal in (False, True):
                fn = lambda: ea.attn_fwd_varlen(q, k, v, cq, ck, M, M, scale=scale, causal=causal,
                                                out=o, lse=lse)
                fp = lambda: ea.attn_fwd(pq, pk, pv, scale=scale, causal=causal, out=po, lse=pl)
                for _ in range(warmup):
                    fn()
                    fp()
                torch.cuda.synchronize()
                us = _timed_calls(fn, reps, flush)
                pus = _timed_calls(fp, reps, flush)
                fl = float(sum(4.0 * H * int(l) * int(l) * d for l in lens)) / (2.0 if causal else 1.0)
                tf = fl / (float(np.median(us)) * 1e-6) / 1e12
                emit({"workload": "varlen", "B": B, "H": H, "d": d, "dtype": "bf16", "causal": causal,
                      "lengths": [int(l) for l in lens], "total": T, "max_len": M,
                      "kernel": ea.attn_kernel_name(1, H, M, M, d, 0, ea.ATTN_BF16), "reps": reps,
                      **_stats(us), "tflops": round(tf, 2),
                      "pct_of_bound": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
                      "padded_dense": {**_stats(pus),
                                       "tflops_useful": round(fl / (float(np.median(pus)) * 1e-6) / 1e12, 2)}})
            del q, k, v, o, lse, pq, pk, pv, po, pl
            torch.cuda.empty_cache()
        return
    if name == "bwd":
        import oracle
        for (B, H, S, d, seed) in ((1, 8, 8192, 128, 3), (8, 32, 2048, 64, 2), (1, 16, 2048, 256, 421)):
            inp = si.make_attention_inputs(B, H, S, S, d, seed=seed, dtype="bf16")
            q, k, v = to_dev(inp)
            rng = np.random.default_rng(seed + 1000)
            do = torch.from_numpy(rng.standard_normal((B, H, S, d), dtype=np.float32)).to(dev)
            scale = float(np.float32(1.0 / np.sqrt(d)))
            ws = torch.empty(ea.attn_bwd_workspace_bytes(B, H, S, S, d, True), dtype=torch.uint8, device=dev)
            dq = torch.empty((B, H, S, d), dtype=torch.float32, device=dev)
            dk, dv = torch.empty_like(dq), torch.empty_like(dq)
            for causal in (False, True):
                o, lse = ea.attn_fwd(q, k, v, scale=scale, causal=causal)
                fn = lambda: ea.attn_bwd(q, k, v, o, lse, do, scale=scale, causal=causal,
                                         dq=dq, dk=dk, dv=dv, ws=ws)
                for _ in range(warmup):
                    fn()
                torch.cuda.synchronize()
                us = []
                for _ in range(reps):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    fn()
                    e1.record()
                    torch.cuda.synchronize()
                    us.append(e0.elapsed_time(e1) * 1e3)
                us = np.array(us)
                fl = 10.0 * B * H * S * S * d / (2.0 if causal else 1.0)
                tf = fl / (float(np.median(us)) * 1e-6) / 1e12
                rec = {"workload": "bwd", "B": B, "H": H, "Sq": S, "Sk": S, "d": d, "dtype": "bf16",
                       "causal": causal, "kernel": " + ".join(ea.attn_bwd_kernel_name(d, ea.ATTN_BF16, w)
                                                             for w in range(3)),
                       "reps": reps, **_stats(us), "tflops": round(tf, 2),
                       "flop_per_byte": None, "bound_tflops": PEAK_BF16_TFLOPS, "bound": "mfma",
                       "pct_of_bound": round(100.0 * tf / PEAK_BF16_TFLOPS, 2)}
                if B == 1:
                    # the oracle's backward on one head of the same inputs, timed on the host
                    h0 = time.perf_counter()
                    oracle.attention_bwd(inp.q64[0, 0], inp.k64[0, 0], inp.v64[0, 0],
                                         do[0, 0].cpu().numpy(), scale, causal)
                    dt = time.perf_counter() - h0
                    rec["cpu_baseline"] = {"value": round(10.0 * S * S * d / (2.0 if causal else 1.0) / dt / 1e12, 4),
                                           "unit": "TFLOPS", "kind": "oracle",
                                           "sample": f"one head (S={S}, d={d}), fp64 NumPy, {dt:.2f} s"}
                emit(rec)
            del q, k, v, do, ws, dq, dk, dv
            torch.cuda.empty_cache()
        return
    if name == "c5":
        B, H, Sq, Sk, d = 1, 8, 128, 32768, 128
        inp = si.make_attention_inputs(B, H, Sq, Sk, d, seed=5, dtype="fp8")
        q, k, v = to_dev(inp)
        scale = float(np.float32(1.0 / np.sqrt(d)))
        ab = _alg_bytes(B, H, Sq, Sk, d, 1)
        o = torch.empty((B, H, Sq, d), dtype=torch.float32, device=dev)
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
        auto_n = ea.attn_splitkv_num_splits(B, H, Sq, Sk, d, ea.ATTN_FP8_E4M3)
        for n in splits or (1, 4, 16, 32, 64):
            ws = torch.empty(ea.attn_splitkv_workspace_bytes(B, H, Sq, d, n), dtype=torch.uint8, device=dev)
            f1 = lambda: ea.attn_fwd_splitkv(q, k, v, n, scale=scale, descales=inp.scales, ws=ws)
            f2 = lambda: ea.attn_merge(ws, n, B, H, Sq, d, out=o, lse=lse)
            for _ in range(warmup):
                f1()
                f2()
            torch.cuda.synchronize()
            u1 = _timed_calls(f1, reps, flush)
            u2 = _timed_calls(f2, reps, flush)
            wsb = n * B * H * Sq * (d + 2) * 4
            t = float(np.median(u1)) + float(np.median(u2))
            emit({"workload": "c5", "B": B, "H": H, "Sq": Sq, "Sk": Sk, "d": d, "dtype": "fp8",
                  "num_splits": n, "picked_by_attn_splitkv_num_splits": n == auto_n, "kernel": ea.attn_kernel_name(B, H, Sq, Sk, d, 0, ea.ATTN_FP8_E4M3, n),
                  "reps": reps, "splitkv": _stats(u1), "merge": _stats(u2),
                  "total_us": round(t, 2), "alg_bytes": ab, "workspace_bytes_rw": 2 * wsb,
                  "alg_gbs": round(ab / (t * 1e-6) / 1e9, 1),
                  "with_ws_gbs": round((ab + 2 * wsb) / (t * 1e-6) / 1e9, 1),
                  "pct_of_hbm": round(100.0 * ab / (t * 1e-6) / 1e9 / PEAK_HBM_GBS, 2)})
        return
    raise ValueError(name)


def summarize_sweep(path: str) -> str:
    """Markdown table of the JSON lines written by --sweep."""
    recs = [json.loads(l) for l in open(path) if l.strip().startswith("{")]
    out = []
    if recs and recs[0]["workload"] == "out16":
        out += ["| B | H | S | d | mask | kernel | fp32 O median us | bf16 O median us | fp32 O TFLOP/s | bf16 O TFLOP/s |",
                "|---|---|---|---|---|---|---|---|---|---|"]
        for r in recs:
            out.append(f"| {r['B']} | {r['H']} | {r['Sq']} | {r['d']} | {'causal' if r['causal'] else 'full'} | "
                       f"{r['kernel']} | {r['fp32_out']['median_us']} | {r['bf16_out']['median_us']} | "
                       f"{r['tflops_fp32_out']} | {r['tflops_bf16_out']} |")
        return "\n".join(out)
    if recs and recs[0]["workload"] == "varlen":
        out += ["| sequences | H | d | tokens | longest | mask | kernel | median us | TFLOP/s | % of 2500 | padded dense median us | padded dense TFLOP/s (useful) |",
                "|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for r in recs:
            pd = r["padded_dense"]
            out.append(f"| {r['B']} | {r['H']} | {r['d']} | {r['total']} | {r['max_len']} | "
                       f"{'causal' if r['causal'] else 'full'} | {r['kernel']} | {r['median_us']} | "
                       f"{r['tflops']} | {r['pct_of_bound']} | {pd['median_us']} | {pd['tflops_useful']} |")
        out.append("\nlengths: " + "; ".join(f"d={r['d']}: {r['lengths']}" for r in recs if not r["causal"]))
        return "\n".join(out)
    if recs and recs[0]["workload"] == "c5":
        out += ["| n | kernel | splitkv median us | merge median us | total us | GB/s (alg.) | GB/s (with ws) | % of 8 TB/s |",
                "|---|---|---|---|---|---|---|---|"]
        for r in recs:
            pick = " (attn_splitkv_num_splits)" if r.get("picked_by_attn_splitkv_num_splits") else ""
            out.append(f"| {r['num_splits']}{pick} | {r['kernel']} | {r['splitkv']['median_us']} | "
                       f"{r['merge']['median_us']} | {r['total_us']} | {r['alg_gbs']} | "
                       f"{r['with_ws_gbs']} | {r['pct_of_hbm']} |")
        return "\n".join(out)
    out += ["| B | H | S | d | mask | kernel | median us | p10 / p90 us | TFLOP/s | FLOP/B | bound TFLOP/s | % of bound |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in recs:
        out.append(f"| {r['B']} | {r['H']} | {r['Sq']} | {r['d']} | {'causal' if r['causal'] else 'full'} | "
                   f"{r['kernel']} | {r['median_us']} | {r['p10_us']} / {r['p90_us']} | "
                   f"{r.get('tflops', '-')} | {r.get('flop_per_byte', '-')} | "
                   f"{r.get('bound_tflops', '-')} ({r.get('bound', '-')}) | {r.get('pct_of_bound', '-')} |")
    for r in recs:
        if "cpu_baseline" in r:
            cb = r["cpu_baseline"]
            out.append(f"\ncpu_baseline ({'causal' if r['causal'] else 'full'}): {cb['value']} "
                       f"{cb['unit']}, {cb['kind']}, {cb['sample']}")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tune", action="store_true",
                    help="use the fixed launch-plan rule instead of attn_tune's choice")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--sweep", choices=("c1", "c2", "c4", "c5", "bwd", "varlen", "out16"),
                    help="per-case timing of a parity workload (JSON lines)")
    ap.add_argument("--sweep-reps", type=int, default=30)
    ap.add_argument("--splits", default="", help="c5 sweep: comma-separated split counts")
    ap.add_argument("--seqs", default="", help="c4 sweep: comma-separated sequence lengths")
    ap.add_argument("--masks", default="both", choices=("both", "full", "causal"),
                    help="c1/c2/c4 sweeps: which masks to run")
    ap.add_argument("--summarize-sweep", metavar="JSONL")
    ap.add_argument("--summarize-stats", metavar="DIR",
                    help="print a table of a rocprofv3 --stats output directory and exit")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="print per-kernel means of rocprofv3 --pmc counter runs and exit")
    ap.add_argument("--summarize-traffic-grid", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print HBM bytes per launch of every attention kernel and grid and exit")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print HBM bytes per launch from two rocprofv3 --pmc runs and exit")
    args = ap.parse_args()
    if args.summarize_stats:
        print(summarize_stats(args.summarize_stats))
        return
    if args.summarize_sweep:
        print(summarize_sweep(args.summarize_sweep))
        return
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return
    if args.summarize_traffic_grid:
        print(summarize_traffic_grid(*args.summarize_traffic_grid, probe_mib=args.copy_probe_mib or 512))
        return
    if args.summarize_traffic:
        print(summarize_traffic(*args.summarize_traffic, probe_mib=args.copy_probe_mib or 512,
                                workload=args.workload))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        ints = lambda t: [int(x) for x in t.split(",") if x.strip()]
        masks = {"both": (False, True), "full": (False,), "causal": (True,)}[args.masks]
        sweep(args.sweep, args.sweep_reps, args.warmup, splits=ints(args.splits),
              seqs=ints(args.seqs), masks=masks, copy_probe_mib=args.copy_probe_mib)
        return

    import torch
    import exact_attention_82_amd as ea
    import synthetic_inputs as si

    B, H, S, d, seed = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = si.make_attention_inputs(B, H, S, S, d, seed=seed, dtype="bf16")
    q, k, v = (torch.from_numpy(t.view(np.int16)).view(torch.bfloat16).to(dev)
               for t in (inp.q, inp.k, inp.v))
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o = torch.empty((B, H, S, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    modes = (False, True)
    flops = {c: 4.0 * B * H * S * S * d / (2.0 if c else 1.0) for c in modes}

    def step(events=None):
        for i, c in enumerate(modes):
            if events is not None:
                events[i][0].record()
            ea.attn_fwd(q, k, v, scale=scale, causal=c, out=o, lse=lse)
            if events is not None:
                events[i][1].record()

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # shape-keyed tuning (synchronous, before the warm-up and the timed region): the plans
    # attn_tune keeps for this shape are the ones the timed calls use
    plans = {}
    for c in modes:
        name = "causal" if c else "non_causal"
        plan = (ea.attn_tune(q, k, v, scale=scale, causal=c, reps=10, out=o, lse=lse)
                if not args.no_tune else ea.attn_plan_get(B, H, S, S, d, c, ea.ATTN_BF16))
        sched, group = ea.plan_parts(plan)
        plans[name] = {"plan": plan, "schedule": sched, "head_group": group, "tuned": not args.no_tune}

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in modes] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_mode_ms = {c: [ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]
                   for i, c in enumerate(modes)}
    ms_step = wall * 1e3 / args.steps
    total_flops = sum(flops.values())
    value = total_flops * args.steps / wall / 1e12
    # roofline of the dominant kernel: the non-causal launch (mean duration, timed region)
    kern_ms = float(np.mean(per_mode_ms[False]))
    achieved = flops[False] / (kern_ms * 1e-3) / 1e12

    # shader clock under the dominant kernel and the software / hardware it ran on, both
    # outside the timed region
    clock = measure_clock(lambda: ea.attn_fwd(q, k, v, scale=scale, causal=False, out=o, lse=lse),
                          torch)
    env = environment(torch, dev)

    # outputs of both masks for the CPU leg's check, copied outside the timed region
    gpu_out = {}
    for c in modes:
        ea.attn_fwd(q, k, v, scale=scale, causal=c, out=o, lse=lse)
        gpu_out[c] = o.cpu().numpy().reshape(B * H, S, d)

    traffic = read_traffic() if args.workload == "c3" else None
    result = {
        "metric": "attention fwd TFLOPS (bf16, causal/non-causal) and % of MI355X MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: B={B}, H={H}, Sq=Sk={S}, d={d}, bf16 N(0,1) inputs, "
                        "fp32 O + lse; one step = non-causal + causal forward",
            "B": B, "H": H, "Sq": S, "Sk": S, "d": d, "masks": ["non-causal", "causal"],
            "kernels": {m: ea.attn_kernel_name(B, H, S, S, d, c, ea.ATTN_BF16) for m, c in (("non_causal", 0), ("causal", 1))},
            "plans": plans,
        },
        "modes": {
            ("causal" if c else "non_causal"): {
                "tflops": round(flops[c] / (np.median(per_mode_ms[c]) * 1e-3) / 1e12, 2),
                "median_us": round(float(np.median(per_mode_ms[c])) * 1e3, 2),
                "p10_us": round(float(np.percentile(per_mode_ms[c], 10)) * 1e3, 2),
                "p90_us": round(float(np.percentile(per_mode_ms[c], 90)) * 1e3, 2),
                "min_us": round(float(np.min(per_mode_ms[c])) * 1e3, 2),
                "pct_bf16_peak": round(100.0 * flops[c] / (np.median(per_mode_ms[c]) * 1e-3)
                                       / 1e12 / PEAK_BF16_TFLOPS, 2),
            } for c in modes
        },
        "roofline": {
            "kernel": ea.attn_kernel_name(B, H, S, S, d, 0, ea.ATTN_BF16),
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
        "clock": clock,
        "environment": env,
    }
    if clock.get("mhz"):
        # frac = (clock / 2.4 GHz) x (MFMA busy fraction at that clock): the peak assumes
        # 256 CUs x 4096 bf16 FLOP per clock at 2.4 GHz
        cus = env.get("gpu_cus") or 256
        at_clock = cus * 4096 * clock["mhz"] * 1e6 / 1e12
        result["roofline"]["peak_at_measured_clock"] = round(at_clock, 1)
        result["roofline"]["frac_at_measured_clock"] = round(achieved / at_clock, 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"], worst = cpu_baseline(inp, scale, args.cpu_budget, gpu_out)
        result["numerics_max_abs_err_sampled"] = worst
        if worst > 1e-2:
            print(json.dumps(result), flush=True)
            print(f"numerics check failed: max|dO| = {worst}", file=sys.stderr)
            sys.exit(1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
