"""Benchmark of the causal self-attention layer on one MI355X.

A step is one forward of the whole layer (c_attn GEMM -> fused causal
attention -> c_proj GEMM) over one batch of the GPT-2 124M attention layer
workload: B=12, T=1024, C=768, 12 heads, bf16 with fp32 accumulation, seeded
synthetic inputs (x ~ N(0,1), weights at the GPT-2 initialisation).  The
inputs of 8 rotating sets (x, weights, y: 8 x 42.5 MB, larger than the 256 MB
Infinity Cache) are resident in HBM before timing starts.

Reported (one JSON line): layer TFLOP/s with the causal FLOP count
F = 8*B*T*C^2 + 2*B*T*(T+1)*C, tokens/s, fraction of the 2.5166 PFLOP/s dense
bf16 MFMA peak (all from K steps with nothing but the layer's kernels on the
stream), per-kernel times from HIP events recorded by the library on the
launch stream in a second run of the same K steps (the event records
lengthen a step, so the step rate does not include them), the roofline of
the dominant kernel, the training step
(forward + backward) time of the same workload, and the CPU oracle timed on a
bounded sample of the same workload on the host cores.

HBM traffic of the dominant kernel comes from two rocprofv3 counter passes
over `--pmc-run` (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same
counter reads for a plain device copy of known size launched in the same
run; `--write-traffic FETCH_DIR WRITE_DIR` turns the two passes into the
summary under profiles/, which the benchmark reports while the kernel sources
it was taken from are unchanged (else null); the forward kernels then also
carry `hbm_gbs`, those bytes over the kernel's event time.  MFMA, LDS and VALU
utilisation per kernel come from one more counter pass over `--pmc-run-all`
(forward, training and MLP steps), summarised by `--write-util PMC_DIR`.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0
METRIC = ("attention-layer TFLOP/s + tokens/s at B=12,T=1024,C=768,H=12 bf16; "
          "% of MFMA peak")
N_SETS = 8
COPY_BYTES = 1 << 30          # calibration copy: 1 GiB read + 1 GiB written
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_kernels_gpt2_124m_B12_T1024.md")
KERNEL_KEYS = {"c_attn": ("gemm2_kernel", "Epi2QKV"), "attention": ("attn_fwd2_bf16_kernel",),
               "c_proj": ("gemm3_kernel", "gpt_attn::Epi2RowMajor>")}


def layer_flops(B, T, C):
    """Causal algorithmic FLOPs of one forward: the two projections
    (2*B*T*C*3C + 2*B*T*C*C) plus QK^T and PV over the B*T*(T+1)/2 visible
    (query, key) pairs per head (2*hs FLOPs each, twice, summed over heads)."""
    return 8 * B * T * C * C + 2 * B * T * (T + 1) * C


def stage_flops(B, T, C):
    return {"c_attn": 6 * B * T * C * C, "attention": 2 * B * T * (T + 1) * C,
            "c_proj": 2 * B * T * C * C}


def stage_bytes(B, T, C, H, es=2, lse=False):
    """Algorithmic HBM bytes per launch: every tensor read or written once."""
    BT = B * T
    return {"c_attn": (BT * C + 3 * C * C + 3 * C + 3 * BT * C) * es,
            "attention": (3 * BT * C + BT * C) * es + (B * H * T * 4 if lse else 0),
            "c_proj": (BT * C + C * C + C + BT * C) * es}


class HipEvents:
    """hipEvent_t handles through the HIP runtime (timing on the library's
    launch stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                          ctypes.c_void_p(b))
        assert rc == 0, rc
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def cpu_model():
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(workload_index, n_seq, min_seconds=10.0):
    """The fp64 oracle, as it stands, on the first n_seq sequences of the
    same workload (sequences are independent, so throughput scales), run
    repeatedly until about min_seconds of CPU time have elapsed."""
    import oracle
    from gpt_causal_self_amd.inputs import workload_inputs
    inp = workload_inputs(workload_index, B=n_seq)
    threads = oracle.default_threads()
    oracle.load()
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(inp.x, inp.W_attn, inp.b_attn, inp.W_proj, inp.b_proj, inp.n_head,
                       nthreads=threads)
        runs += 1
        if time.perf_counter() - t0 >= min_seconds or runs >= 50:
            break
    dt = (time.perf_counter() - t0) / runs
    B, T, C = inp.x.shape
    return {"value": layer_flops(B, T, C) / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "cpu_model": cpu_model(), "kind": "oracle", "tokens_per_s": B * T / dt,
            "seconds_per_run": dt, "runs": runs,
            "sample": f"{n_seq} of 12 sequences (B={n_seq}, T=1024, C=768, H=12), fp64 "
                      f"forward on the same seeded inputs, mean of {runs} runs"}


def sources_digest():
    """sha256 over the HIP sources and header the kernels are built from."""
    import hashlib
    h = hashlib.sha256()
    for d in (os.path.join(ROOT, "gpt_causal_self_amd", "csrc"), os.path.join(ROOT, "include")):
        for f in sorted(os.listdir(d)):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def newest_counter_file(run_dir):
    """The counter file of the latest rocprofv3 run under run_dir (each run
    writes one <pid>_counter_collection.csv; a directory that collected
    several runs must not mix them: dispatch ids repeat across runs)."""
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    return [max(files, key=os.path.getmtime)]


def _counter_means(run_dir, counter):
    """Mean per-dispatch value of one counter, per kernel group and for the
    calibration copy, from a rocprofv3 -f csv output directory."""
    import csv
    import glob
    files = newest_counter_file(run_dir)
    sums, counts = {}, {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = None
            for k, parts in KERNEL_KEYS.items():
                if all(p in name for p in parts):
                    key = k
            if key is None and "copybuffer" in name.lower():
                key = "copy"
            if key is None:
                continue
            d = r.get("Dispatch_Id", r.get("Correlation_Id"))
            sums.setdefault(key, {}).setdefault(d, 0.0)
            sums[key][d] += float(r["Counter_Value"])
    out = {}
    for k, per in sums.items():
        vals = list(per.values())
        if k == "copy":
            vals = [max(vals)]            # the 1 GiB calibration copy
        out[k] = sum(vals) / len(vals)
    return out


def write_traffic(fetch_dir, write_dir):
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    ff = COPY_BYTES / 1024.0 / fetch["copy"]
    fw = COPY_BYTES / 1024.0 / write["copy"]
    from gpt_causal_self_amd.inputs import WORKLOADS
    w = WORKLOADS[2]
    sb = stage_bytes(w.B, w.T, w.C, w.H)
    rec = {"digest": sources_digest(), "factor_fetch": ff, "factor_write": fw,
           "copy_fetch_kib": fetch["copy"], "copy_write_kib": write["copy"], "kernels": {}}
    lines = ["# HBM traffic per launch: GPT-2 124M attention layer forward "
             "(B12 T1024 C768 H12 bf16)", "",
             "Commands (from /tmp with TMPDIR=/tmp on one MI355X; repository at $R, profiler output under $OUT):", "", "```",
             "timeout -s KILL 60 rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/pmc_fetch "
             "-- python3 $R/bench.py --pmc-run",
             "timeout -s KILL 60 rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/pmc_write "
             "-- python3 $R/bench.py --pmc-run",
             "python3 $R/bench.py --write-traffic $OUT/pmc_fetch $OUT/pmc_write",
             "```", "",
             f"Calibration: a device copy of {COPY_BYTES} bytes reads FETCH_SIZE "
             f"{fetch['copy']:.1f} KiB and WRITE_SIZE {write['copy']:.1f} KiB, so each kernel's "
             f"counters are scaled by {ff:.4f} (reads) and {fw:.4f} (writes).", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled MB read | scaled MB written | "
             "algorithmic MB | traffic / algorithmic |", "|---|---|---|---|---|---|---|"]
    for k in ("c_attn", "attention", "c_proj"):
        if k not in fetch or k not in write:
            continue
        rb, wb = fetch[k] * 1024 * ff, write[k] * 1024 * fw
        rec["kernels"][k] = {"fetch_kib": fetch[k], "write_kib": write[k],
                             "bytes": rb + wb, "algorithmic_bytes": sb[k]}
        lines.append(f"| {k} | {fetch[k]:.1f} | {write[k]:.1f} | {rb / 1e6:.2f} | "
                     f"{wb / 1e6:.2f} | {sb[k] / 1e6:.2f} | {(rb + wb) / sb[k]:.3f} |")
    lines += ["", "Machine-readable record (sources digest = sha256 of the HIP sources and "
              "header the counters were taken with):", "", "```",
              "TRAFFIC " + json.dumps(rec, sort_keys=True), "```", ""]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


UTIL_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT "
                 "SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_VALU_MFMA_COEXEC_CYCLES GRBM_GUI_ACTIVE")
UTIL_FILE = os.path.join(ROOT, "profiles", "mfma_lds_util_kernels_gpt2_124m_B12_T1024.md")
SIMD_NUM, CU_NUM, XCD_NUM = 1024, 256, 8   # MI355X: 8 XCDs x 32 CUs x 4 SIMDs


def write_util(run_dir):
    """Per-kernel MFMA / LDS / VALU utilisation from one rocprofv3 --pmc pass
    over `--pmc-run-all` (forward, training step and MLP at the GPT-2 124M
    shape).  rocprofv3 reports each counter once per dispatch, summed over
    the chip; GRBM_GUI_ACTIVE is then the sum of the 8 XCDs' active cycles,
    so one XCD's (the kernel's duration in cycles) is that sum / 8.  The
    ratios follow rocprofv3's derived MfmaUtil / LdsUtil / LdsBankConflict
    / VALUBusy metrics."""
    import csv
    import glob
    import re
    files = newest_counter_file(run_dir)
    per = {}   # kernel -> dispatch -> counter -> [sum, max]
    for f in files:
        for r in csv.DictReader(open(f)):
            name = re.sub(r"\(.*", "", r["Kernel_Name"]).replace("void ", "")
            name = name.replace("gpt_attn::", "").replace("unsigned short", "bf16")
            if "rocclr" in name or "at::native" in name:
                continue
            d = r.get("Dispatch_Id", r.get("Correlation_Id"))
            v = float(r["Counter_Value"])
            c = per.setdefault(name, {}).setdefault(d, {}).setdefault(r["Counter_Name"], [0.0, 0.0])
            c[0] += v
            c[1] = max(c[1], v)
    lines = ["# MFMA, LDS and VALU utilisation per kernel: GPT-2 124M attention layer "
             "(B12 T1024 C768 H12 bf16), forward, training step and MLP", "",
             "Commands (from /tmp with TMPDIR=/tmp on one MI355X; repository at $R, profiler output under $OUT):", "", "```",
             f"timeout -s KILL 60 rocprofv3 --pmc {UTIL_COUNTERS} -f csv -d $OUT/pmc_util "
             "-- python3 $R/bench.py --pmc-run-all",
             "python3 $R/bench.py --write-util $OUT/pmc_util", "```", "",
             f"Sources digest: {sources_digest()}", "",
             "Per dispatch, averaged over dispatches, with A = GRBM_GUI_ACTIVE / "
             f"{XCD_NUM} (the counter sums the XCDs' active cycles): MFMA util = "
             f"SQ_VALU_MFMA_BUSY_CYCLES / (A x {SIMD_NUM} SIMDs); LDS active and bank-conflict = "
             f"100 x counter / (A x {CU_NUM} CUs); VALU busy = 100 x SQ_ACTIVE_INST_VALU / "
             f"{CU_NUM} / A; MFMA+VALU co-issue = 100 x SQ_VALU_MFMA_COEXEC_CYCLES / "
             f"(A x {SIMD_NUM}); MFMA/VALU instructions are "
             "wave-level counts per dispatch (a 32x32x16 bf16 MFMA is 32768 FLOP).  Counter "
             "collection serialises the kernels, so active cycles cover each kernel alone.", "",
             "| kernel | dispatches | MFMA util % | MFMA instr | VALU instr | VALU busy % | "
             "MFMA+VALU co-issue % | LDS active % | LDS bank-conflict % |",
             "|---|---|---|---|---|---|---|---|---|"]
    rows = []
    for name, ds in per.items():
        acc = {}
        for d in ds.values():
            for cn, (sm, mx) in d.items():
                a = acc.setdefault(cn, [0.0, 0.0, 0])
                a[0] += sm
                a[1] += mx
                a[2] += 1
        mean = {cn: (a[0] / a[2], a[1] / a[2]) for cn, a in acc.items()}
        if "GRBM_GUI_ACTIVE" not in mean or "SQ_VALU_MFMA_BUSY_CYCLES" not in mean:
            continue
        gui = mean["GRBM_GUI_ACTIVE"][0] / XCD_NUM
        g = lambda cn: mean.get(cn, (0.0, 0.0))[0]
        rows.append((gui * len(ds), name, len(ds),
                     100.0 * g("SQ_VALU_MFMA_BUSY_CYCLES") / (gui * SIMD_NUM),
                     g("SQ_INSTS_MFMA"), g("SQ_INSTS_VALU"),
                     100.0 * g("SQ_ACTIVE_INST_VALU") / CU_NUM / gui,
                     100.0 * g("SQ_VALU_MFMA_COEXEC_CYCLES") / (gui * SIMD_NUM),
                     100.0 * g("SQ_LDS_IDX_ACTIVE") / (gui * CU_NUM),
                     100.0 * g("SQ_LDS_BANK_CONFLICT") / (gui * CU_NUM)))
    for r in sorted(rows, reverse=True):
        lines.append(f"| `{r[1]}` | {r[2]} | {r[3]:.1f} | {r[4]:.0f} | {r[5]:.0f} | {r[6]:.1f} | "
                     f"{r[7]:.1f} | {r[8]:.1f} | {r[9]:.1f} |")
    with open(UTIL_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def write_kernel_stats(stats_dir, out_md):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run."""
    import csv
    import glob
    import re
    files = glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {stats_dir}")
    rows = list(csv.DictReader(open(files[0])))

    def short(n):
        n = re.sub(r"\(.*", "", n)
        return n.replace("void gpt_attn::", "").replace("unsigned short", "bf16")
    lines = ["# Kernel trace: GPT-2 124M attention layer (B12 T1024 C768 H12 bf16), "
             "bench.py forward + training step", "",
             "Command (from /tmp with TMPDIR=/tmp on one MI355X; repository at $R, profiler output under $OUT):", "", "```",
             "timeout -k 10 300 rocprofv3 --kernel-trace --stats -f csv -d "
             "$OUT/ktrace -o run -- python3 $R/bench.py --steps 20 --warmup 5 --no-cpu",
             f"python3 $R/bench.py --write-kernel-stats $OUT/ktrace {os.path.basename(out_md)}",
             "```", "", f"Sources digest: {sources_digest()}", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f} |")
    # The table above is rocprofv3's per-name summary over the whole run, in
    # which the other configurations (other shapes, same kernels) mix in.
    # The forward kernels at this workload, from the per-dispatch trace,
    # selected by name and grid (work-items):
    traces = glob.glob(os.path.join(stats_dir, "**", "*kernel_trace.csv"), recursive=True)
    if traces:
        B, T, C, H = 12, 1024, 768, 12
        M = B * T
        want = {"c_attn": ("Epi2QKV", (M // 256) * (3 * C // 256) * 1024, 1),
                "attention": ("attn_fwd2_bf16_kernel<64, 2, false>", B * H * 256, T // 128),
                "c_proj": ("gemm3_kernel<96, 384, 32, 4, true, false, 1, 6, "
                           "gpt_attn::Epi2RowMajor>", ((M + 95) // 96) * (C // 384) * 512, 1)}
        durs = {k: [] for k in want}
        for r in csv.DictReader(open(traces[0])):
            for k, (name, gx, gy) in want.items():
                if (name in r["Kernel_Name"] and int(r["Grid_Size_X"]) == gx
                        and int(r["Grid_Size_Y"]) == gy):
                    durs[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines += ["", "Forward kernels at this workload (B=12 T=1024 C=768 H=12), from the "
                  "per-dispatch trace (`*kernel_trace.csv`), selected by kernel and grid size:", "",
                  "| stage | grid (work-items) | dispatches | avg us | min us | max us |",
                  "|---|---|---|---|---|---|"]
        for k, (name, gx, gy) in want.items():
            d = durs[k]
            if d:
                lines.append(f"| {k} | {gx} x {gy} | {len(d)} | {sum(d) / len(d):.1f} | "
                             f"{min(d):.1f} | {max(d):.1f} |")
    with open(os.path.join(ROOT, "profiles", os.path.basename(out_md)), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def load_traffic():
    """The counter-derived traffic record, or None if absent or taken with
    other kernel sources."""
    try:
        for line in open(TRAFFIC_FILE):
            if line.startswith("TRAFFIC "):
                rec = json.loads(line[len("TRAFFIC "):])
                return rec if rec.get("digest") == sources_digest() else None
    except OSError:
        pass
    return None


def pmc_run(steps):
    """Short run for the counter passes: forward steps of the workload, then
    the calibration copy."""
    import torch
    from gpt_causal_self_amd import gpt_attn as ga
    from gpt_causal_self_amd.inputs import WORKLOADS, make_inputs, to_torch
    w = WORKLOADS[2]
    B, T, C, H = w.B, w.T, w.C, w.H
    dev = torch.device("cuda", 0)
    inp = make_inputs(B, T, C, H, bias=True, dtype="bf16", seed=125, w_std=w.w_std,
                      b_attn_std=w.b_attn_std, proj_std=w.proj_std, b_proj_std=w.b_proj_std)
    t = {k: to_torch(getattr(inp, k), "bf16", dev)
         for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj")}
    y = torch.empty_like(t["x"])
    layer = ga.Layer(C, H, B, T, "bf16")
    for _ in range(steps):
        ga.gpt_attn_forward(layer.h, t["x"], t["W_attn"], t["b_attn"], t["W_proj"],
                            t["b_proj"], H, y)
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    layer.close()
    print(f"pmc run: {steps} forward steps, copy of {COPY_BYTES} bytes", flush=True)


def pmc_run_all(steps):
    """Short run for the utilisation counter pass: forward steps, training
    steps (forward with saved state + backward) and MLP forwards at the
    GPT-2 124M shape."""
    import torch
    from gpt_causal_self_amd import gpt_attn as ga
    from gpt_causal_self_amd.inputs import WORKLOADS, make_inputs, to_torch
    w = WORKLOADS[2]
    B, T, C, H = w.B, w.T, w.C, w.H
    dev = torch.device("cuda", 0)
    inp = make_inputs(B, T, C, H, bias=True, dtype="bf16", seed=125, w_std=w.w_std,
                      b_attn_std=w.b_attn_std, proj_std=w.proj_std, b_proj_std=w.b_proj_std)
    t = {k: to_torch(getattr(inp, k), "bf16", dev)
         for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj")}
    y = torch.empty_like(t["x"])
    dY = torch.randn(y.shape, device=dev).to(torch.bfloat16)
    g = {k: torch.empty_like(t[src]) for k, src in
         (("dx", "x"), ("dWa", "W_attn"), ("dba", "b_attn"), ("dWp", "W_proj"), ("dbp", "b_proj"))}
    layer = ga.Layer(C, H, B, T, "bf16")
    for _ in range(steps):
        ga.gpt_attn_forward(layer.h, t["x"], t["W_attn"], t["b_attn"], t["W_proj"],
                            t["b_proj"], H, y)
    for _ in range(steps):
        ga.gpt_attn_forward(layer.h, t["x"], t["W_attn"], t["b_attn"], t["W_proj"],
                            t["b_proj"], H, y, save_for_backward=True)
        ga.gpt_attn_backward(layer.h, t["x"], t["W_attn"], t["W_proj"], dY, g["dx"], g["dWa"],
                             g["dba"], g["dWp"], g["dbp"])
    M, F = B * T, 4 * C
    wfc = (torch.randn(C, F, device=dev) * 0.02).to(torch.bfloat16)
    bfc = (torch.randn(F, device=dev) * 0.02).to(torch.bfloat16)
    wp2 = (torch.randn(F, C, device=dev) * 0.02).to(torch.bfloat16)
    hbuf = torch.empty(M, F, device=dev, dtype=torch.bfloat16)
    for _ in range(steps):
        ga.gpt_mlp_forward(t["x"], wfc, bfc, wp2, t["b_proj"], hbuf, y, residual=t["x"])
    torch.cuda.synchronize()
    layer.close()
    print(f"pmc run: {steps} forward, {steps} training and {steps} MLP steps", flush=True)


def _read_sclk(path):
    """Current shader clock in MHz from an amdgpu pp_dpm_sclk file (the line
    marked with '*' is the level in use; its value is the measured clock)."""
    import re
    with open(path) as f:
        for line in f:
            if line.rstrip().endswith("*"):
                m = re.search(r"(\d+)\s*mhz", line, re.IGNORECASE)
                return int(m.group(1)) if m else None
    return None


def sample_sclk(step, seconds=0.5, period=0.005):
    """Shader clock while the workload runs: a thread reads the driver's
    pp_dpm_sclk every `period` s while the caller's thread keeps issuing
    step(i) for `seconds` (outside the timed regions).  Needs exactly one
    amdgpu card in sysfs (else the clock cannot be tied to the device)."""
    import glob
    import statistics
    import threading
    import torch
    files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if len(files) != 1:
        return {"error": f"{len(files)} pp_dpm_sclk files; cannot tell which is this device"}
    path, vals, stop = files[0], [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                v = _read_sclk(path)
            except OSError:
                v = None
            if v:
                vals.append(v)
            time.sleep(period)

    th = threading.Thread(target=sampler, daemon=True)
    for i in range(20):
        step(i)
    th.start()
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        step(i)
        i += 1
        if i % 200 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stop.set()
    th.join()
    if not vals:
        return {"error": "no readable samples", "source": path}
    return {"median": statistics.median(vals), "min": min(vals), "max": max(vals),
            "samples": len(vals), "source": path,
            "window": f"{i} forward steps over {seconds} s after the timed regions"}


def time_calls(fn, n, warm=3):
    """Mean milliseconds per call of fn (launches on the current stream),
    from torch events around n back-to-back calls."""
    import torch
    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def other_configs(n=30):
    """Forward throughput of the layer at the other parity configurations:
    the tiny fp32 character model (B=8, T=64, C=128, 4 heads), the
    gpt2-medium shape (B=8, T=1024, C=1024, 16 heads, bf16) and the gpt2-xl
    shape without biases (B=4, C=1600, 25 heads, bf16) over its ragged
    sequence lengths.  Each is timed with events around n back-to-back
    forwards on one input set (inputs resident in HBM)."""
    import torch
    from gpt_causal_self_amd import gpt_attn as ga
    from gpt_causal_self_amd.inputs import WORKLOADS, make_inputs, to_torch
    res = {}
    cases = [(1, WORKLOADS[1].T), (3, WORKLOADS[3].T)]
    cases += [(4, t) for t in WORKLOADS[4].ragged_T]
    for idx, T in cases:
        w = WORKLOADS[idx]
        B, C, H = w.B, w.C, w.H
        inp = make_inputs(B, T, C, H, bias=w.bias, dtype=w.dtype, seed=124 + idx,
                          w_std=w.w_std, b_attn_std=w.b_attn_std, proj_std=w.proj_std,
                          b_proj_std=w.b_proj_std)
        t = {k: to_torch(getattr(inp, k), w.dtype, "cuda")
             for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj")}
        y = torch.empty_like(t["x"])
        layer = ga.Layer(C, H, B, T, w.dtype)
        ms = time_calls(lambda: ga.gpt_attn_forward(layer.h, t["x"], t["W_attn"], t["b_attn"],
                                                    t["W_proj"], t["b_proj"], H, y), n)
        layer.close()
        F = layer_flops(B, T, C)
        key = f"cfg{idx}" if idx != 4 else f"cfg4_T{T}"
        res[key] = {"workload": f"B={B} T={T} C={C} H={H} {w.dtype}" +
                    ("" if w.bias else " no bias"),
                    "ms": round(ms, 5), "tflops": round(F / (ms * 1e-3) / 1e12, 3),
                    "tokens_per_s": round(B * T / (ms * 1e-3), 1),
                    "frac_of_peak": round(F / (ms * 1e-3) / 1e12 /
                                          (PEAK_BF16_TFLOPS if w.dtype == "bf16" else 157.3), 4)}
    return res


def next_rows(n=50):
    """Timings of the pieces around the layer at the GPT-2 124M shape (B=12,
    T=1024, C=768, 12 heads, MLP width 3072): LayerNorm, the Pre-LN attention
    half-block, dropout (forward and training step), one-token decode
    against a full KV cache, and the MLP sublayer with its residual add."""
    import torch
    from gpt_causal_self_amd import gpt_attn as ga
    from gpt_causal_self_amd.inputs import (WORKLOADS, make_inputs, make_ln_params,
                                            make_mlp_inputs, to_torch)
    w = WORKLOADS[2]
    B, T, C, H = w.B, w.T, w.C, w.H
    M, F = B * T, 4 * C
    dev = "cuda"
    inp = make_inputs(B, T, C, H, bias=True, dtype="bf16", seed=125, w_std=w.w_std,
                      b_attn_std=w.b_attn_std, proj_std=w.proj_std, b_proj_std=w.b_proj_std)
    t = {k: to_torch(getattr(inp, k), "bf16", dev)
         for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj")}
    lw, lb = (to_torch(a, "bf16", dev) for a in make_ln_params(C, seed=126))
    out = torch.empty_like(t["x"])
    layer = ga.Layer(C, H, B, T, "bf16")
    res = {}
    ms = time_calls(lambda: ga.gpt_layernorm(t["x"], lw, lb, out), n)
    ln_bytes = 2 * M * C * 2 + 2 * C * 2
    res["layernorm"] = {"workload": f"M={M} C={C} bf16", "ms": round(ms, 5),
                        "gbs": round(ln_bytes / (ms * 1e-3) / 1e9, 1),
                        "roofline": {"bound": "hbm", "achieved": round(ln_bytes / (ms * 1e-3) / 1e9, 1),
                                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                     "frac": round(ln_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                     "algorithmic_bytes": ln_bytes}}
    ms = time_calls(lambda: ga.gpt_attn_block_forward(layer.h, t["x"], lw, lb, t["W_attn"],
                                                      t["b_attn"], t["W_proj"], t["b_proj"], H,
                                                      out), n)
    F_blk = layer_flops(B, T, C)
    res["block_attn_half"] = {"workload": f"x + attn(ln_1(x)), B={B} T={T} C={C} H={H} bf16",
                              "ms": round(ms, 5),
                              "tflops": round(F_blk / (ms * 1e-3) / 1e12, 2),
                              "tokens_per_s": round(M / (ms * 1e-3), 1)}
    # training-time dropout (p = 0.1): forward, and forward + backward
    y = torch.empty_like(t["x"])
    dY = torch.randn_like(t["x"].float()).to(torch.bfloat16)
    grads = [torch.empty_like(t["x"]), torch.empty_like(t["W_attn"]), torch.empty_like(t["b_attn"]),
             torch.empty_like(t["W_proj"]), torch.empty_like(t["b_proj"])]
    ga.gpt_attn_set_dropout(layer.h, 0.1, 1234)
    ms_f = time_calls(lambda: ga.gpt_attn_forward(layer.h, t["x"], t["W_attn"], t["b_attn"],
                                                  t["W_proj"], t["b_proj"], H, y), n)

    def drop_step():
        ga.gpt_attn_forward(layer.h, t["x"], t["W_attn"], t["b_attn"], t["W_proj"],
                            t["b_proj"], H, y, save_for_backward=True)
        ga.gpt_attn_backward(layer.h, t["x"], t["W_attn"], t["W_proj"], dY, *grads)
    ms_t = time_calls(drop_step, max(5, n // 5))
    ga.gpt_attn_set_dropout(layer.h, 0.0, 0)
    res["dropout"] = {"workload": f"dropout p=0.1 on the attention weights and the c_proj "
                                  f"output, B={B} T={T} C={C} H={H} bf16",
                      "forward_ms": round(ms_f, 5),
                      "forward_tflops": round(F_blk / (ms_f * 1e-3) / 1e12, 2),
                      "train_step_ms": round(ms_t, 5),
                      "train_step_tflops": round(3 * F_blk / (ms_t * 1e-3) / 1e12, 2)}
    # one-token decode at the last position of a full 1024-token cache
    hs = C // H
    kc = torch.randn((B, H, T, hs), device=dev).to(torch.bfloat16)
    vc = torch.randn((B, H, T, hs), device=dev).to(torch.bfloat16)
    xt = t["x"][:, T - 1].contiguous()
    yt = torch.empty_like(xt)
    ms = time_calls(lambda: ga.gpt_attn_decode(layer.h, xt, t["W_attn"], t["b_attn"],
                                               t["W_proj"], t["b_proj"], H, kc, vc, yt, T - 1), n)
    dec_bytes = 2 * B * H * T * hs * 2 + (4 * C * C + 4 * C) * 2 + 4 * B * C * 2
    res["decode"] = {"workload": f"one token per sequence at pos={T - 1}, B={B} C={C} H={H}, "
                                 f"bf16 KV cache of {T} positions",
                     "ms": round(ms, 5), "tokens_per_s": round(B / (ms * 1e-3), 1),
                     "roofline": {"bound": "hbm",
                                  "achieved": round(dec_bytes / (ms * 1e-3) / 1e9, 1),
                                  "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": round(dec_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                  "algorithmic_bytes": dec_bytes}}
    layer.close()
    m = make_mlp_inputs(M, C, F, seed=127, with_residual=True)
    d = {k: to_torch(getattr(m, k), "bf16", dev)
         for k in ("x", "W_fc", "b_fc", "W_proj", "b_proj", "residual")}
    hbuf = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, C), dtype=torch.bfloat16, device=dev)
    ms = time_calls(lambda: ga.gpt_mlp_forward(d["x"], d["W_fc"], d["b_fc"], d["W_proj"],
                                               d["b_proj"], hbuf, y, residual=d["residual"]), n)
    F_mlp = 4 * M * C * F
    res["mlp"] = {"workload": f"x + mlp(x), M={M} C={C} F={F} bf16", "ms": round(ms, 5),
                  "tflops": round(F_mlp / (ms * 1e-3) / 1e12, 2),
                  "roofline": {"bound": "mfma", "achieved": round(F_mlp / (ms * 1e-3) / 1e12, 2),
                               "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(F_mlp / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                               "flop_per_launch": F_mlp}}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-train", action="store_true", help="skip the fwd+bwd measurement")
    ap.add_argument("--cpu-seqs", type=int, default=12)
    ap.add_argument("--no-next", action="store_true",
                    help="skip the Block-piece timings (LayerNorm, half-block, MLP)")
    ap.add_argument("--pmc-run-all", action="store_true",
                    help="forward, training and MLP steps only (for the utilisation counter pass)")
    ap.add_argument("--write-util", metavar="PMC_DIR",
                    help="summarise the utilisation counter pass under profiles/")
    ap.add_argument("--pmc-run", action="store_true",
                    help="short forward-only run plus the calibration copy, for counter passes")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 counter passes into the traffic record")
    ap.add_argument("--write-kernel-stats", nargs=2, metavar=("STATS_DIR", "NAME"),
                    help="summarise a rocprofv3 --kernel-trace --stats run under profiles/")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.write_kernel_stats:
        write_kernel_stats(*args.write_kernel_stats)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer runs on a single device)", file=sys.stderr)
        sys.exit(2)

    if args.pmc_run_all:
        pmc_run_all(min(args.steps, 5))
        return
    if args.write_util:
        write_util(args.write_util)
        return
    if args.pmc_run:
        pmc_run(min(args.steps, 10))
        return

    import torch
    from gpt_causal_self_amd import gpt_attn as ga
    from gpt_causal_self_amd.inputs import WORKLOADS, make_inputs, to_torch

    w = WORKLOADS[2]
    B, T, C, H = w.B, w.T, w.C, w.H
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    sets = []
    for s in range(N_SETS):
        inp = make_inputs(B, T, C, H, bias=True, dtype="bf16", seed=125 + 1000 * s,
                          w_std=w.w_std, b_attn_std=w.b_attn_std, proj_std=w.proj_std,
                          b_proj_std=w.b_proj_std, with_dY=(s == 0))
        t = {k: to_torch(getattr(inp, k), "bf16", dev)
             for k in ("x", "W_attn", "b_attn", "W_proj", "b_proj")}
        t["y"] = torch.empty_like(t["x"])
        if s == 0:
            t["dY"] = to_torch(inp.dY, "bf16", dev)
        sets.append(t)
    layer = ga.Layer(C, H, B, T, "bf16")
    stream = torch.cuda.current_stream()

    def step(i):
        t = sets[i % N_SETS]
        ga.gpt_attn_forward(layer.h, t["x"], t["W_attn"], t["b_attn"], t["W_proj"],
                            t["b_proj"], H, t["y"], stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: K steps, nothing but the layer's kernels on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # ---- second timed region for the per-kernel durations: the same K steps
    # with the library recording 4 events per step on the launch stream
    # (before c_attn, after c_attn, after attention, after c_proj).  The
    # event records themselves lengthen a step by ~10 %, so the step rate
    # above is taken without them.
    ev = HipEvents()
    events = [ev.create(4) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ga.gpt_attn_set_stage_events(layer.h, events[i])
        step(i)
    torch.cuda.synchronize()
    wall_events = time.perf_counter() - t0
    ga.gpt_attn_set_stage_events(layer.h, None)

    per = {"c_attn": [], "attention": [], "c_proj": [], "layer": []}
    for e in events:
        per["c_attn"].append(ev.elapsed_ms(e[0], e[1]))
        per["attention"].append(ev.elapsed_ms(e[1], e[2]))
        per["c_proj"].append(ev.elapsed_ms(e[2], e[3]))
        per["layer"].append(ev.elapsed_ms(e[0], e[3]))
    for e in events:
        ev.destroy(e)
    mean = {k: sum(v) / len(v) for k, v in per.items()}
    ms_per_step = wall * 1e3 / args.steps

    F = layer_flops(B, T, C)
    tflops = F / (ms_per_step * 1e-3) / 1e12
    sf = stage_flops(B, T, C)
    sb = stage_bytes(B, T, C, H)
    kernels = {}
    rec = load_traffic()
    for k in ("c_attn", "attention", "c_proj"):
        kernels[k] = {"ms": round(mean[k], 5),
                      "tflops": round(sf[k] / (mean[k] * 1e-3) / 1e12, 2),
                      "gbs": round(sb[k] / (mean[k] * 1e-3) / 1e9, 1),
                      "flop_per_launch": sf[k], "bytes_per_launch": sb[k]}
        if rec and k in rec["kernels"]:
            kernels[k]["hbm_gbs"] = round(rec["kernels"][k]["bytes"] / (mean[k] * 1e-3) / 1e9, 1)
    dom = max(("c_attn", "attention", "c_proj"), key=lambda k: mean[k])
    achieved = sf[dom] / (mean[dom] * 1e-3) / 1e12
    traffic = None
    if rec and dom in rec["kernels"]:
        traffic = round(rec["kernels"][dom]["bytes"])
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                "copy-calibrated)" if traffic else None,
                "algorithmic_bytes": sb[dom], "flop_per_launch": sf[dom]}

    out = {"metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "gpt2-124M causal self-attention layer forward, "
                                  "B=12 T=1024 C=768 H=12 hs=64 bias bf16/fp32-acc",
                      "B": B, "T": T, "C": C, "n_head": H, "bias": True, "global_batch": B,
                      "seq_len": T, "parallelism": "single GPU"},
           "tokens_per_s": round(B * T / (ms_per_step * 1e-3), 1),
           "frac_of_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
           "flop_per_step": F, "flop_count": "causal: 8BTC^2 + 2BT(T+1)C",
           "dense_convention_tflops": round((8 * B * T * C * C + 4 * B * T * T * C)
                                            / (ms_per_step * 1e-3) / 1e12, 2),
           "event_layer_ms": round(mean["layer"], 5),
           "ms_per_step_with_stage_events": round(wall_events * 1e3 / args.steps, 5),
           "kernels": kernels, "roofline": roofline}
    try:
        out["sclk_mhz"] = sample_sclk(step)
    except Exception as e:  # the clock is context; its absence is no failure
        out["sclk_mhz"] = {"error": str(e)}

    if not args.no_train:
        try:
            t = sets[0]
            g = {"dx": torch.empty_like(t["x"]), "dWa": torch.empty_like(t["W_attn"]),
                 "dba": torch.empty_like(t["b_attn"]), "dWp": torch.empty_like(t["W_proj"]),
                 "dbp": torch.empty_like(t["b_proj"])}

            def train_step():
                ga.gpt_attn_forward(layer.h, t["x"], t["W_attn"], t["b_attn"], t["W_proj"],
                                    t["b_proj"], H, t["y"], stream=stream,
                                    save_for_backward=True)
                ga.gpt_attn_backward(layer.h, t["x"], t["W_attn"], t["W_proj"], t["dY"],
                                     g["dx"], g["dWa"], g["dba"], g["dWp"], g["dbp"],
                                     stream=stream)
            for _ in range(5):
                train_step()
            torch.cuda.synchronize()
            n = max(10, args.steps // 4)
            t0 = time.perf_counter()
            for _ in range(n):
                train_step()
            torch.cuda.synchronize()
            tms = (time.perf_counter() - t0) * 1e3 / n
            out["train_step"] = {"workload": "gpt2-124M fwd+bwd B=12 T=1024 C=768 H=12 bf16",
                                 "ms": round(tms, 5),
                                 "tflops": round(3 * F / (tms * 1e-3) / 1e12, 2),
                                 "flop_count": "3 x forward causal count"}
        except ga.GptAttnError as e:
            out["train_step"] = {"error": str(e)}

    if not args.no_next:
        out["next_rows"] = next_rows()
        out["other_configs"] = other_configs()

    if not args.no_cpu:
        cb = cpu_baseline(2, args.cpu_seqs)
        out["cpu_baseline"] = {k: (round(v, 6) if isinstance(v, float) else v)
                               for k, v in cb.items()}
        if cb.get("value"):
            # the same workload's rate on the GPU over the oracle's on the host
            out["cpu_baseline"]["gpu_over_cpu"] = round(out["value"] / cb["value"], 1)
    layer.close()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
