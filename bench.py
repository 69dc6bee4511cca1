"""Benchmark of the GEAR hot path on one MI355X.

Headline step (the `value`): one pass of the whole path over one 7B-shaped
attention layer (batch 8, 32 heads, 4096 tokens, head_dim 128; K and V, fp16 =
536,870,912 B):
  gear_compress    outlier top-k + CSR, 4-bit group quantization, rank-4 fit
                   (3 power iterations) of all 512 K/V matrices
  gear_decompress  reconstruction of all 512 matrices to fp16
  gear_append_decode_attn
                   one new token per sequence into the streaming cache (its
                   buffer is compressed every 64 steps) and decode attention of
                   one query per head over the compressed 4096+ tokens, in one
                   call (the token is written by the attention launch)
Inputs are synthetic, seeded, already resident in HBM.  `value` is fp16 KV
bytes per step / step time (GB/s).  Prints one JSON line.

The K timed steps run uninstrumented; K further steps then run with the
library's per-kernel HIP events on (gear_timing_*) and per-phase events, which
give `phases_ms`, `kernels_ms`, `roofline` (the kernel with the largest share
of a step, its launch time measured live on the launch stream) and
`compress_phase` (the three compress launches as one unit).  Measured HBM
bytes and SQ counters come from the committed rocprofv3 summaries under
profiles/ while they were taken from the current kernel sources (else null);
the counters also name the binding resource (`bound`).

Beside the headline, the same line carries (all timed in this run):
  configs            compress / decompress (and one decode step) of the other
                     workloads: tiny, 2-bit, long context in 512-token chunks,
                     and GEAR-L (no outliers) at the 7B-layer and 2-bit shapes
  stream_gqa_decode  the streaming GQA workload (batch 64, 32 query / 8 KV
                     heads, 2048-token prompt, 256 append + decode steps)
  cpu_baseline       the CPU oracle on a bounded sample of the headline layer

    python bench.py [--gpus 1] [--steps 20] [--warmup 30] [--no-cpu-baseline]
                    [--no-stream] [--no-configs] [--workload 7b_layer]
    python bench.py --make-profiles OUTDIR [--workload W]   (rocprofv3 passes
                    and every summary table under OUTDIR; runs on the GPU machine)
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import hashlib
import json
import os
import platform
import re
import subprocess
import sys
import time
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# 256 CUs x 4 SIMDs x 16 lanes per cycle (a wave64 VALU instruction takes 4
# cycles) x 2.4 GHz: ordinary (non-packed) VALU lane-operations per second
VALU_PEAK_TLANE_OPS = 256 * 64 * 2.4e9 / 1e12
SIMDS = 1024
XCDS = 8
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "kv_cache_compression_gear_amd", "csrc")
COPY_BYTES = 256 << 20          # plain copy used to calibrate the byte counters
COPY_KERNEL = "copyBuffer"      # the runtime's blit kernel behind torch's device copy
COPY_GRID = str(COPY_BYTES // 2048)   # its grid for the 256 MiB calibration copy
METRIC = "GEAR compress+decompress GB/s (fp16 KV in) & decode tok/s; % of HBM peak"

# kernel (name used by gear_timing_read, plus attn_prompt) -> source file
KERNEL_SOURCE = {"select": "gear_compress.hip", "compress": "gear_compress.hip",
                 "lowrank_a": "gear_compress.hip", "decompress": "gear_decompress.hip",
                 "attn_prompt": "gear_attn.hip", "attn_gqa": "gear_attn.hip",
                 "attn_split": "gear_attn.hip", "attn_combine": "gear_attn.hip", "buffer_append": "gear_attn.hip"}
# device symbol of each kernel ("attn_prompt", "attn_gqa" and "attn_split" are
# timed together by the library, as "attn_split": the decode attention over all splits)
KERNEL_SYMBOL = {"select": "select_kernel", "compress": "compress_kernel",
                 "lowrank_a": "lowrank_a_kernel", "decompress": "decompress_kernel",
                 "attn_prompt": "attn_prompt_kernel", "attn_gqa": "attn_gqa_kernel",
                 "attn_split": "attn_split_kernel",
                 "attn_combine": "attn_combine_kernel", "buffer_append": "buffer_append_kernel"}
# further device symbols of a kernel key: the decompress launch is
# decompress_mm_kernel with a low-rank term, decompress_kernel without
KERNEL_ALIASES = {"decompress": ("decompress_mm_kernel",)}
SQ_PASSES = [
    ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_WAVE_CYCLES",
     "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
    ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_WAIT_ANY", "SQ_WAVES",
     "SQ_INSTS_VMEM_RD", "SQ_INSTS_BRANCH", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS",
     "GRBM_GUI_ACTIVE"],
]


# --------------------------------------------------------------------------
# Profile summaries (rocprofv3 output -> the text files under profiles/)
# --------------------------------------------------------------------------

def source_digest(kernel: str) -> str:
    """sha256 (first 16 hex digits) over the code of the kernel's source and of
    the shared header, comments and whitespace removed (so that an edit of a
    comment does not mark the counters stale)."""
    h = hashlib.sha256()
    for name in (KERNEL_SOURCE[kernel], "gear_internal.h"):
        with open(os.path.join(CSRC, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _kernel_key(name: str):
    # the symbol as a whole identifier: compress_kernel is not decompress_kernel
    for k, sym in KERNEL_SYMBOL.items():
        for s_ in (sym,) + KERNEL_ALIASES.get(k, ()):
            if re.search(r"(?<![A-Za-z0-9_])" + s_ + r"(?![A-Za-z0-9_])", name):
                return k
    return None


def summarize_pmc(path: str):
    """Per-kernel mean of each counter in a rocprofv3 counter_collection.csv;
    the 256 MiB calibration copy is listed as 'copy'."""
    vals = defaultdict(lambda: defaultdict(list))
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            key = _kernel_key(name)
            if key is None and COPY_KERNEL in name and row.get("Grid_Size") == COPY_GRID:
                key = "copy"
            if key is None:
                continue
            vals[key][row["Counter_Name"]].append(float(row["Counter_Value"]))
    return {k: {c: (sum(v) / len(v), len(v)) for c, v in d.items()} for k, d in vals.items()}


def _trace_rows(path: str):
    rows = []
    with open(path) as f:
        for row in csv.DictReader(f):
            s = row.get("Start_Timestamp") or row.get("Start") or row.get("BeginNs")
            e = row.get("End_Timestamp") or row.get("End") or row.get("EndNs")
            rows.append((row["Kernel_Name"], int(s), int(e)))
    rows.sort(key=lambda r: r[1])
    return rows


def _short(name: str) -> str:
    m = re.search(r"(\w+_kernel)(<[^()]*>)?", name)
    if not m:
        return name[:48]
    return (m.group(1) + (m.group(2) or "")).replace(" ", "")


def kernel_stats_table(trace_csv: str, last: int, bench_json: dict | None, header: str) -> str:
    """Per kernel instantiation: calls, mean / min / max duration over the
    whole run and the mean of its last `last` launches (the instrumented pass
    of the headline step, which comes last in the run), beside the HIP-event
    means the run's own JSON line reported."""
    per = defaultdict(list)
    for name, s, e in _trace_rows(trace_csv):
        if _kernel_key(name) is not None:      # this library's kernels only
            per[_short(name)].append((e - s) / 1e3)
    bench_k = (bench_json or {}).get("kernels_ms", {})
    # the library's timing covers the instantiation the headline step runs
    # most (the fill compression of the streaming cache is another one)
    main_inst = {}
    for k, d in per.items():
        key = _kernel_key(k)
        if key not in main_inst or len(d) > len(per[main_inst[key]]):
            main_inst[key] = k
    lines = [header.rstrip("\n"), "# Times in microseconds.",
             f"{'kernel':44s} {'calls':>6s} {'avg_us':>8s} {'min_us':>8s} {'max_us':>8s} "
             f"{'last' + str(last) + '_us':>9s} {'bench_us':>9s}"]
    for k, d in sorted(per.items(), key=lambda kv: -sum(kv[1][-last:])):
        key = _kernel_key(k)
        b = bench_k.get(key) if main_inst.get(key) == k else None
        lines.append(f"{k:44s} {len(d):6d} {sum(d) / len(d):8.1f} {min(d):8.1f} {max(d):8.1f} "
                     f"{sum(d[-last:]) / len(d[-last:]):9.1f} {'' if b is None else f'{b * 1e3:9.1f}'}")
    if bench_json:
        lines.append(f"# same run: value {bench_json['value']} GB/s, ms_per_step "
                     f"{bench_json['ms_per_step']}, roofline {bench_json['roofline']['kernel']} "
                     f"launch {bench_json['roofline']['launch_ms']} ms")
    lines.append("# (bench_us: attn_prompt_kernel, attn_gqa_kernel and attn_split_kernel are timed together as "
                 "attn_split by the library)")
    return "\n".join(lines) + "\n"


def hbm_table(fetch_csv: str, write_csv: str, header: str) -> str:
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of every kernel, each
    divided by what the same counter reads per byte of the plain calibration
    copy; with each kernel's source digest (bench.py uses the bytes only while
    the digest matches the current sources)."""
    f, w = summarize_pmc(fetch_csv), summarize_pmc(write_csv)
    kib = COPY_BYTES / 1024
    ff = f["copy"]["FETCH_SIZE"][0] / kib
    wf = w["copy"]["WRITE_SIZE"][0] / kib
    lines = [header.rstrip("\n"),
             f"# calibration: plain copy of {COPY_BYTES} bytes reads FETCH_SIZE "
             f"{f['copy']['FETCH_SIZE'][0]:.1f} KiB (fetch_factor {ff:.5f}), WRITE_SIZE "
             f"{w['copy']['WRITE_SIZE'][0]:.1f} KiB (write_factor {wf:.5f}); bytes = KiB x 1024 / factor",
             f"{'kernel':16s} {'FETCH_KiB':>12s} {'WRITE_KiB':>12s} {'read_B':>12s} {'write_B':>12s} "
             f"{'total_B':>12s} {'dispatches':>10s}  source_sha256"]
    for k in KERNEL_SYMBOL:
        if k not in f or k not in w:
            continue
        fk, nf = f[k]["FETCH_SIZE"]
        wk, _ = w[k]["WRITE_SIZE"]
        rb, wb = fk * 1024 / ff, wk * 1024 / wf
        lines.append(f"{k:16s} {fk:12.1f} {wk:12.1f} {rb:12.0f} {wb:12.0f} {rb + wb:12.0f} "
                     f"{nf:10d}  {source_digest(k)}")
    return "\n".join(lines) + "\n"


def sq_table(p1_csv: str, p2_csv: str, entries: dict, header: str) -> str:
    """SQ counters per dispatch (means) and derived columns: valu% = VALU
    instructions x 4 cycles over the dispatch's SIMD-cycles (1024 SIMDs x
    GRBM_GUI_ACTIVE / 8 XCDs); mfma% = SQ_VALU_MFMA_BUSY_CYCLES over the same;
    coexec% = MFMA cycles with VALU issuing too; lane_ops/entry = VALU
    instructions x 64 / matrix entries the launch covers."""
    a, b = summarize_pmc(p1_csv), summarize_pmc(p2_csv)
    cols = SQ_PASSES[0][:-1] + SQ_PASSES[1][:-1] + ["GRBM_GUI_ACTIVE"]
    lines = [header.rstrip("\n"),
             f"{'kernel':14s} " + " ".join(f"{c.replace('SQ_', ''):>14s}" for c in cols)]
    derived = [f"{'kernel':14s} {'valu%':>7s} {'mfma%':>7s} {'coexec%':>8s} {'lane_ops/entry':>15s} "
               f"{'lds_confl/inst':>15s}  source_sha256"]
    for k in KERNEL_SYMBOL:
        if k not in a or k not in b:
            continue
        v = {**{c: a[k][c][0] for c in a[k]}, **{c: b[k][c][0] for c in b[k] if c != "GRBM_GUI_ACTIVE"}}
        lines.append(f"{k:14s} " + " ".join(f"{v.get(c, float('nan')):14.4g}" for c in cols))
        simd_cycles = SIMDS * v["GRBM_GUI_ACTIVE"] / XCDS
        valu = 100 * v["SQ_INSTS_VALU"] * 4 / simd_cycles
        mfma = 100 * v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / simd_cycles
        co = (100 * v.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0) / v["SQ_VALU_MFMA_BUSY_CYCLES"]
              if v.get("SQ_VALU_MFMA_BUSY_CYCLES") else 0.0)
        ent = entries.get(k)
        lpe = f"{v['SQ_INSTS_VALU'] * 64 / ent:15.2f}" if ent else f"{'':15s}"
        lds = v.get("SQ_LDS_BANK_CONFLICT", 0) / max(v.get("SQ_INSTS_LDS", 1), 1)
        derived.append(f"{k:14s} {valu:7.1f} {mfma:7.1f} {co:8.1f} {lpe} {lds:15.2f}  {source_digest(k)}")
    return "\n".join(lines + [""] + derived) + "\n"


def read_profile_row(kind: str, workload: str, kernel: str):
    """The row of `kernel` in profiles/gear_kernels_<workload>_<kind>.txt as a
    dict of floats, or None if absent or taken from other kernel sources."""
    path = os.path.join(PROFILES, f"gear_kernels_{workload}_{kind}.txt")
    if not os.path.exists(path):
        return None
    hdr = None
    with open(path) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            if parts[0] == "kernel":
                # only the tables that carry each row's source digest
                hdr = parts if parts[-1] == "source_sha256" else None
                continue
            if hdr and parts[0] == kernel and len(parts) == len(hdr):
                if parts[-1] != source_digest(kernel):
                    return None
                out = {}
                for h, p in zip(hdr[1:-1], parts[1:-1]):
                    try:
                        out[h] = float(p)
                    except ValueError:
                        pass
                return out
    return None


def _entries_of(workload: str) -> dict:
    """Matrix entries one launch of each kernel covers, in the headline step
    of `workload` (for lane-ops per entry)."""
    from kv_cache_compression_gear_amd.synth import WORKLOADS
    w = WORKLOADS[workload]
    n = 2 * w.batch * w.heads * w.seq * w.head_dim
    return {"select": n, "compress": n, "lowrank_a": n, "decompress": n, "attn_prompt": n,
            "attn_gqa": n}


def make_profiles(outdir: str, workload: str, keep_raw: bool = False) -> int:
    """rocprofv3 passes over the headline step of `workload` (kernel trace,
    FETCH_SIZE, WRITE_SIZE, two SQ counter sets), then the summary tables,
    written to OUTDIR/profiles/.  This process never touches the GPU: each
    pass is a child process, rocprofv3 with the program after `--`."""
    os.makedirs(os.path.join(outdir, "profiles"), exist_ok=True)
    me = os.path.abspath(__file__)
    step = ["python3", me, "--workload", workload, "--no-cpu-baseline", "--no-stream",
            "--no-configs"]
    short = step + ["--steps", "3", "--warmup", "1"]
    env = dict(os.environ, TMPDIR="/tmp")
    passes = [("kt", ["--kernel-trace", "--stats"], step, 300),
              ("pf", ["--pmc", "FETCH_SIZE"], short + ["--copy-calibration"], 120),
              ("pw", ["--pmc", "WRITE_SIZE"], short + ["--copy-calibration"], 120),
              ("p1", ["--pmc", *SQ_PASSES[0]], short, 120),
              ("p2", ["--pmc", *SQ_PASSES[1]], short, 120)]
    cmds = {}
    for tag, opts, prog, limit in passes:
        d = os.path.join(outdir, tag)
        cmd = ["timeout", "-s", "KILL", str(limit), "rocprofv3", *opts, "-d", d, "-o", "run",
               "--output-format", "csv", "--", *prog]
        cmds[tag] = " ".join(cmd).replace(outdir, "<out>").replace(os.path.dirname(me), "<repo>")
        print(f"[make-profiles] {tag}: {cmds[tag]}", flush=True)
        with open(os.path.join(outdir, f"{tag}.log"), "w") as log:
            r = subprocess.run(cmd, cwd="/tmp", env=env, stdout=log, stderr=subprocess.STDOUT)
        print(f"[make-profiles] {tag}: exit {r.returncode}", flush=True)
        if r.returncode != 0:
            # rocprofv3 can end with a segmentation fault after a complete run
            # (results written); anything else stops here
            if not (r.returncode in (139, -11) and _csv(d, "kernel_trace" if tag == "kt"
                                                        else "counter_collection")):
                return r.returncode
    bench_json = None
    with open(os.path.join(outdir, "kt.log")) as f:
        for line in f:
            if line.startswith("{\"metric\""):
                bench_json = json.loads(line)
    mk = f"python3 <repo>/bench.py --make-profiles <out> --workload {workload}"
    common = (f"# One MI355X (gfx950), ROCm 7.2; workload {workload} (the headline step of "
              f"bench.py --workload {workload}).\n# Made by `{mk}` (committed code), which ran, "
              f"from /tmp with TMPDIR=/tmp:\n")
    out = os.path.join(outdir, "profiles")
    with open(os.path.join(out, f"gear_kernels_{workload}_kernel_stats.txt"), "w") as f:
        f.write(kernel_stats_table(_csv(os.path.join(outdir, "kt"), "kernel_trace"),
                                   bench_json["steps"] if bench_json else 20, bench_json,
                                   common + f"#   {cmds['kt']}\n"))
    with open(os.path.join(out, f"gear_kernels_{workload}_hbm_bytes.txt"), "w") as f:
        f.write(hbm_table(_csv(os.path.join(outdir, "pf"), "counter_collection"),
                          _csv(os.path.join(outdir, "pw"), "counter_collection"),
                          common + f"#   {cmds['pf']}\n#   {cmds['pw']}\n"))
    with open(os.path.join(out, f"gear_kernels_{workload}_sq_counters.txt"), "w") as f:
        f.write(sq_table(_csv(os.path.join(outdir, "p1"), "counter_collection"),
                         _csv(os.path.join(outdir, "p2"), "counter_collection"),
                         _entries_of(workload),
                         common + f"#   {cmds['p1']}\n#   {cmds['p2']}\n"
                         "# Means per dispatch over the run's dispatches of each kernel.\n"))
    if not keep_raw:   # raw traces and counter files: large, and summarised above
        import shutil
        for tag, *_ in passes:
            shutil.rmtree(os.path.join(outdir, tag), ignore_errors=True)
    print(f"[make-profiles] summaries in {out}", flush=True)
    return 0


def _csv(d: str, kind: str):
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith(f"{kind}.csv"):
                return os.path.join(root, fn)
    return None


# --------------------------------------------------------------------------
# Timed parts
# --------------------------------------------------------------------------

def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _cpu_baseline(w, x_sample, p, n_mats_total):
    """The C oracle (as it stands) on a bounded sample of the same workload:
    compress + reconstruct of a number of the layer's matrices, one host thread
    per matrix, on at most 16 threads (one GPU's share of a GPU host)."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as orc

    op = orc.Params(p.bits, p.group, p.outlier_ppm, p.rank, p.power_iters, p.chunk_tokens, p.seed)
    mats = [x_sample[i] for i in range(x_sample.shape[0])]
    host_cpus = len(os.sched_getaffinity(0))
    threads = max(1, min(len(mats), host_cpus, 16))
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda m: orc.compress_matrix(m, op), mats))
    dt = time.perf_counter() - t0
    nbytes = sum(m.nbytes for m in mats)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "host_cpus": host_cpus, "cpu_model": _cpu_model(),
            "sample": f"{len(mats)} of the {n_mats_total} K/V matrices ({w.seq}x{w.head_dim} fp16): "
                      f"compress + reconstruct (no decode attention), {dt:.2f} s wall on "
                      f"{threads} host threads"}


def _packed_bytes(pk) -> int:
    return sum(s.numel() * s.element_size() for s in pk.sections())


def _median(v):
    v = sorted(v)
    return v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])


def _codec_config(gear, torch, w, p, label, reps=10, decode=False, role=0):
    """Compress and decompress of one whole workload (inputs resident), median
    of `reps` timed calls after 3 warm-up calls, per-kernel means from a second
    pass with the library's HIP events; optionally one decode step (append +
    attention) over a cache holding the same compressed prompt."""
    B, H, n, d = w.batch, w.heads, w.seq, w.head_dim
    syn = w.kv_synth("cuda")
    k, v = syn.prompt(n)
    x = torch.cat([k.reshape(B * H, n, d), v.reshape(B * H, n, d)]).contiguous()
    M = x.shape[0]
    L = gear.packed_layout(p, M, n, d, role)
    packed = gear.Packed(torch.empty(L.total_bytes, dtype=torch.uint8, device="cuda"), p, M, n, d, L, role)
    ws = torch.empty(gear.compress_workspace_bytes(p, M, n, d, role), dtype=torch.uint8, device="cuda")
    xhat = torch.empty_like(x)
    for _ in range(3):
        gear.compress(x, p, out=packed, workspace=ws, role=role)
        gear.decompress(packed, out=xhat)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in ev:
        e[0].record()
        gear.compress(x, p, out=packed, workspace=ws, role=role)
        e[1].record()
        gear.decompress(packed, out=xhat)
        e[2].record()
    torch.cuda.synchronize()
    c_ms = _median([e[0].elapsed_time(e[1]) for e in ev])
    d_ms = _median([e[1].elapsed_time(e[2]) for e in ev])
    gear.timing_enable(True)
    for _ in range(reps):
        gear.compress(x, p, out=packed, workspace=ws, role=role)
        gear.decompress(packed, out=xhat)
    torch.cuda.synchronize()
    kt = gear.timing_read()
    gear.timing_enable(False)
    fp16 = x.numel() * 2
    pb = _packed_bytes(packed)
    algo = fp16 + pb
    rec = {"workload": label, "matrices": M * (n // (p.chunk_tokens or n)),
           "compress_ms": round(c_ms, 4), "decompress_ms": round(d_ms, 4),
           "compress_GBps_fp16": round(fp16 / (c_ms * 1e-3) / 1e9, 1),
           "decompress_GBps_fp16": round(fp16 / (d_ms * 1e-3) / 1e9, 1),
           "algorithmic_bytes": algo,
           "compress_hbm_frac": round(algo / (c_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "decompress_hbm_frac": round(algo / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "kernels_ms": {k2: round(t / c, 4) for k2, (c, t) in kt.items()}}
    del xhat, ws
    if decode:
        Hq = w.q_heads or H
        fp = gear.Params(p.bits, p.group, p.outlier_ppm, min(p.rank, w.fill_rank), p.power_iters,
                         quant=p.quant)
        cache = gear.Cache(B, H, d, p, fp, n, buf_tokens=w.buf_tokens, max_new_tokens=1, q_heads=Hq)
        cache.load_prompt(k.contiguous(), v.contiguous())
        kn, vn = syn.step()
        q = syn.queries(Hq)
        cache.append(kn, vn)
        out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
        for _ in range(3):
            cache.decode_attn(q, out=out)
        torch.cuda.synchronize()
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        e0[0].record()
        for i in range(reps):
            cache.decode_attn(q, out=out)
            e0[i + 1].record()
        torch.cuda.synchronize()
        a_ms = _median([e0[i].elapsed_time(e0[i + 1]) for i in range(reps)])
        cb = _packed_bytes(cache.prompt_packed()) + B * H * 2 * d * 2 + q.numel() * 2 + out.numel() * 4
        rec.update({"decode_attn_ms": round(a_ms, 4), "decode_tok_s": round(B / (a_ms * 1e-3), 1),
                    "decode_algorithmic_bytes": cb,
                    "decode_hbm_frac": round(cb / (a_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)})
        del cache
    del x, k, v, packed
    torch.cuda.synchronize()
    return rec


def _configs(gear, torch, WORKLOADS):
    out = {}
    # (key, workload, bits, group, outlier_ppm, quant, role, decode step)
    runs = [("tiny", "tiny", None, None, None, 0, 0, True),
            ("2bit", "2bit", None, None, None, 0, 0, True),
            ("long_ctx", "long_ctx", None, None, None, 0, 0, True),
            ("7b_layer_gear_l", "7b_layer", None, None, 0, 0, 0, True),
            ("2bit_gear_l", "2bit", None, None, 0, 0, 0, False),
            # the backbones at the 7B-layer shape: KIVI 2-bit keys per channel
            # in groups of 64 tokens (values per token), low rank, no outliers;
            # ZipCache 4-bit tokenwise with 2% outliers
            ("7b_layer_kivi_2bit_gear_l", "7b_layer", 2, 64, 0, 1, 2, True),
            ("7b_layer_zipcache", "7b_layer", 4, 128, None, 2, 0, True)]
    names = {0: "", 1: " KIVI", 2: " ZipCache"}
    for key, wname, bits, group, ppm, quant, role, decode in runs:
        w = WORKLOADS[wname]
        bits = w.bits if bits is None else bits
        group = w.group if group is None else group
        ppm = w.outlier_ppm if ppm is None else ppm
        p = gear.Params(bits, group, ppm, w.rank, w.power_iters, w.chunk_tokens, quant=quant)
        label = (f"{wname}{names[quant]}{' GEAR-L' if ppm == 0 else ''}: batch {w.batch}, {w.heads} heads, "
                 f"{w.seq} tokens, head_dim {w.head_dim}, b={bits} g={group} s={ppm / 1e4:g}% r={w.rank} "
                 f"t={w.power_iters}" + (f", chunks of {w.chunk_tokens}" if w.chunk_tokens else ""))
        print(f"[bench] config {key}", file=sys.stderr, flush=True)
        out[key] = _codec_config(gear, torch, w, p, label, decode=decode, role=role)
    return out


def _stream_decode(gear, WORKLOADS, torch):
    """Streaming GQA decode: append + decode attention for 256 steps, timed
    uninstrumented; the same steps on a second cache (same prompt) give the
    per-kernel breakdown and the attention's bytes per step."""
    w = WORKLOADS["stream_gqa"]
    B, H, n, d, Hq = w.batch, w.heads, w.seq, w.head_dim, w.q_heads
    p = gear.Params(w.bits, w.group, w.outlier_ppm, w.rank, w.power_iters)
    fp = gear.Params(w.bits, w.group, w.outlier_ppm, w.fill_rank, w.power_iters)
    syn = w.kv_synth("cuda")
    k, v = syn.prompt(n)
    caches = []
    for _ in range(2):
        c = gear.Cache(B, H, d, p, fp, n, buf_tokens=w.buf_tokens, max_new_tokens=w.decode_steps,
                       q_heads=Hq)
        c.load_prompt(k.contiguous(), v.contiguous())
        caches.append(c)
    del k, v
    steps = w.decode_steps
    nk = torch.empty((steps, B, H, d), dtype=torch.float16, device="cuda")
    nv = torch.empty_like(nk)
    qs = torch.empty((steps, B, Hq, d), dtype=torch.float16, device="cuda")
    for i in range(steps):
        nk[i], nv[i] = syn.step()
        qs[i] = syn.queries(Hq)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    # one warm-up launch of each kernel on a throw-away cache of the same shape
    warm = gear.Cache(B, H, d, p, fp, 0, buf_tokens=w.buf_tokens, max_new_tokens=w.buf_tokens,
                      q_heads=Hq)
    warm.load_prompt(nk[0], nv[0])
    for i in range(w.buf_tokens):
        warm.append(nk[i], nv[i])
    warm.decode_attn(qs[0], out=out)
    torch.cuda.synchronize()
    del warm
    t0 = time.perf_counter()
    for i in range(steps):
        caches[0].append_decode_attn(nk[i], nv[i], qs[i], out=out)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    gear.timing_enable(True)
    for i in range(steps):
        caches[1].append_decode_attn(nk[i], nv[i], qs[i], out=out)
    torch.cuda.synchronize()
    kt = gear.timing_read()
    gear.timing_enable(False)
    attn_ms = sum(kt.get(k2, (0, 0.0))[1] for k2 in ("attn_split", "attn_combine"))
    # what the attention reads and writes over the run: the packed prompt every
    # step, the fills compressed so far, the fp16 buffer rows, q and out
    prompt_b = _packed_bytes(caches[1].prompt_packed())
    fill_b = _packed_bytes(caches[1].fill_packed(0))
    row_b = B * H * 2 * d * 2
    total_b = 0
    for s in range(1, steps + 1):
        total_b += prompt_b + (s // w.buf_tokens) * fill_b + (s % w.buf_tokens) * row_b
        total_b += qs[0].numel() * 2 + out.numel() * 4
    rec = {"workload": f"stream_gqa: batch {B}, {Hq} query / {H} KV heads, prompt {n} tokens, "
                       f"{steps} decode steps, fp16 buffer {w.buf_tokens} tokens compressed "
                       f"on fill at rank {w.fill_rank}",
           "tok_s": round(B * steps / dt, 1),
           "attn_only_tok_s": round(B * steps / (attn_ms * 1e-3), 1) if attn_ms > 0 else None,
           "ms_total": round(dt * 1e3, 3),
           "attn_algorithmic_bytes_per_step": round(total_b / steps),
           "attn_hbm_frac": round(total_b / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4) if attn_ms else None,
           "kernels_ms": {k2: round(v2[1] / v2[0], 4) for k2, v2 in kt.items()}}
    del caches
    torch.cuda.synchronize()
    return rec


# The memory/throughput study of the GEAR pages (app.cochat.ai, "Cites" list,
# Method sentence quoted under the KIVI entry: the batch size is raised until
# the memory runs out, and peak memory and throughput are compared between
# FP16 KV caches and 2-bit KIVI, GEAR and GEAR-L), on one GPU and KV caches
# only: a 7B-shaped model's 32 layers of 32 heads x 128, each layer a streaming
# cache of this library; one decode step appends one token per sequence to
# every layer and runs decode attention in every layer.  FP16 is a cache whose
# fp16 buffer holds every token (no compression; the same attention kernels).
SWEEP_CONFIGS = [
    # name, bits, group, outlier_ppm, rank, power_iters, quant (None: fp16)
    ("fp16", None, None, None, None, None, None),
    ("gear_4bit", 4, 128, 20000, 4, 3, 0),
    ("gear_l_4bit", 4, 128, 0, 4, 3, 0),
    ("gear_2bit", 2, 64, 20000, 4, 3, 0),
    ("gear_l_2bit", 2, 64, 0, 4, 3, 0),
    ("kivi_2bit", 2, 64, 0, 0, 0, 1),
    ("kivi_gear_l_2bit", 2, 64, 0, 4, 3, 1),
]


def _sweep(gear, torch, layers, heads, d, prompt, new, steps, warm):
    """Largest batch each cache kind fits in free HBM (from the library's own
    arena and workspace sizes, plus one layer's fp16 prompt while it is
    compressed), decode throughput at doubling batch sizes up to it, peak
    memory at each."""
    pool_b = 4                      # distinct synthetic sequences, tiled over the batch
    from kv_cache_compression_gear_amd.synth import KVSynth
    syn = KVSynth(pool_b, heads, d, 4, seed=0, device="cuda")
    kp, vp = syn.prompt(prompt)
    steps_k = torch.stack([syn.step()[0] for _ in range(4)])   # [4, pool_b, H, d]
    steps_v = torch.stack([syn.step()[1] for _ in range(4)])
    qpool = syn.queries(heads)
    torch.cuda.synchronize()
    out = {}
    for name, bits, group, ppm, rank, iters, quant in SWEEP_CONFIGS:
        if bits is None:   # fp16: everything stays in the buffer
            pp = fp = gear.Params(4, 128, 0, 0, 0)
            n_prompt, buf, max_new = 0, prompt + new + 1, prompt + new
        else:
            pp = gear.Params(bits, group, ppm, rank, iters, quant=quant)
            fp = gear.Params(bits, group, ppm, min(rank, 2), iters, quant=quant)
            n_prompt, buf, max_new = prompt, 64, new

        def per_seq(B):
            c = gear._CacheConfig(pp._c(), fp._c(), B, heads, d, n_prompt, buf, max_new)
            return (gear.lib().gear_cache_arena_bytes(ctypes.byref(c)),
                    gear.lib().gear_cache_workspace_bytes(ctypes.byref(c), heads))
        a64, w64 = per_seq(64)
        # per sequence: every layer's arena and workspace, and the fp16 prompt
        # (K and V) the layers are loaded from
        seq_bytes = layers * (a64 + w64) / 64 + 2 * heads * prompt * d * 2
        torch.cuda.empty_cache()
        free, total = torch.cuda.mem_get_info()
        bmax = int((free * 0.92 - (2 << 30)) // seq_bytes)
        batches = sorted({b for b in (8, 16, 32, 64, 128, 256, 512, 1024) if b < bmax} | {bmax})
        rec = {"cache_bytes_per_sequence": round(layers * a64 / 64), "max_batch": bmax, "runs": []}
        for B in batches:
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats()
            caches = []
            try:
                reps = (B + pool_b - 1) // pool_b
                k = kp.repeat(reps, 1, 1, 1)[:B].contiguous()
                v = vp.repeat(reps, 1, 1, 1)[:B].contiguous()
                for _ in range(layers):
                    c = gear.Cache(B, heads, d, pp, fp, n_prompt, buf_tokens=buf, max_new_tokens=max_new,
                                   q_heads=heads)
                    if n_prompt:
                        c.load_prompt(k, v)
                    else:
                        c.append(k, v)
                    caches.append(c)
                del k, v
                kn = steps_k.repeat(1, reps, 1, 1)[:, :B].contiguous()
                vn = steps_v.repeat(1, reps, 1, 1)[:, :B].contiguous()
                q = qpool.repeat(reps, 1, 1)[:B].contiguous()
                o = torch.empty((B, heads, d), dtype=torch.float32, device="cuda")
                torch.cuda.synchronize()
                t0 = None
                for s_ in range(warm + steps):
                    if s_ == warm:
                        torch.cuda.synchronize()
                        t0 = time.perf_counter()
                    for c in caches:
                        c.append(kn[s_ % 4], vn[s_ % 4])
                        c.decode_attn(q, out=o)
                torch.cuda.synchronize()
                dt = time.perf_counter() - t0
                rec["runs"].append({"batch": B, "tok_s": round(B * steps / dt, 1),
                                    "ms_per_step": round(dt * 1e3 / steps, 3),
                                    "peak_GB": round(torch.cuda.max_memory_allocated() / 1e9, 2)})
                print(f"[sweep] {name} B={B}: {B * steps / dt:.0f} tok/s, peak "
                      f"{torch.cuda.max_memory_allocated() / 1e9:.1f} GB", file=sys.stderr, flush=True)
            except torch.cuda.OutOfMemoryError:
                rec["runs"].append({"batch": B, "oom": True})
                print(f"[sweep] {name} B={B}: out of memory", file=sys.stderr, flush=True)
            del caches
            torch.cuda.synchronize()
        done = [r for r in rec["runs"] if "tok_s" in r]
        rec["peak_tok_s"] = max((r["tok_s"] for r in done), default=None)
        out[name] = rec
    base = out["fp16"]
    for name, rec in out.items():
        if base["peak_tok_s"] and rec["peak_tok_s"]:
            rec["throughput_vs_fp16"] = round(rec["peak_tok_s"] / base["peak_tok_s"], 2)
        rec["max_batch_vs_fp16"] = round(rec["max_batch"] / max(base["max_batch"], 1), 2)
        same = [r for r in rec["runs"] if r.get("batch") == 64 and "peak_GB" in r]
        fb = [r for r in base["runs"] if r.get("batch") == 64 and "peak_GB" in r]
        if same and fb:
            rec["peak_memory_vs_fp16_at_batch_64"] = round(fb[0]["peak_GB"] / same[0]["peak_GB"], 2)
    return out


def sweep_table(path: str) -> str:
    """The text table of a --sweep JSON line (profiles/ summary)."""
    with open(path) as f:
        d = json.loads([l for l in f if l.startswith("{")][-1])
    lines = [f"# {d['metric']}", f"# {d['model']}; {d['data']}; wall {d['wall_s']} s",
             f"{'cache':18s} {'MB/seq':>8s} {'max_batch':>9s} {'peak_tok_s':>10s} {'tok/s vs fp16':>13s} "
             f"{'batch vs fp16':>13s} {'mem vs fp16 @64':>15s}"]
    for k, v in d["configs"].items():
        lines.append(f"{k:18s} {v['cache_bytes_per_sequence'] / 1e6:8.1f} {v['max_batch']:9d} "
                     f"{v['peak_tok_s'] or 0:10.1f} {v.get('throughput_vs_fp16', 0):13.2f} "
                     f"{v['max_batch_vs_fp16']:13.2f} {v.get('peak_memory_vs_fp16_at_batch_64', 0):15.2f}")
    lines.append("# per batch: (batch, tok/s, peak GB)")
    for k, v in d["configs"].items():
        lines.append(f"{k:18s} " + " ".join(f"({r['batch']}, {r.get('tok_s', 'oom')}, {r.get('peak_GB', '-')})"
                                             for r in v["runs"]))
    return "\n".join(lines) + "\n"


def _bound_from_counters(kernel: str, workload: str, launch_ms: float, algo_bytes: float):
    """The binding resource of `kernel` from the committed counters: VALU
    issue (instructions x 4 cycles over the launch's SIMD-cycles, as measured)
    against HBM (measured bytes over the launch time at 8 TB/s)."""
    sq = read_profile_row("sq_counters", workload, kernel)
    hb = read_profile_row("hbm_bytes", workload, kernel)
    if sq is None:
        return None
    lane_ops = None
    p = os.path.join(PROFILES, f"gear_kernels_{workload}_sq_counters.txt")
    with open(p) as f:
        txt = f.read()
    m = re.search(rf"^{kernel}\s+((?:[-\d.e+]+\s+)+)", txt, flags=re.M)
    if m:
        lane_ops = float(m.group(1).split()[0]) * 64       # first column: SQ_INSTS_VALU
    valu_frac = sq.get("valu%", 0.0) / 100.0
    hbm_frac = (hb["total_B"] / (launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS) if hb else None
    return {"valu_busy_frac": round(valu_frac, 4),
            "hbm_busy_frac": None if hbm_frac is None else round(hbm_frac, 4),
            "lane_ops_per_launch": lane_ops,
            "lane_ops_per_entry": sq.get("lane_ops/entry"),
            "traffic": None if hb is None else hb["total_B"],
            "bound": "alu" if hbm_frac is None or valu_frac > hbm_frac else "hbm"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="7b_layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=256)
    ap.add_argument("--no-stream", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--make-profiles", metavar="OUTDIR",
                    help="run the rocprofv3 passes and write the summary tables under OUTDIR")
    ap.add_argument("--keep-raw", action="store_true",
                    help="with --make-profiles: keep the raw rocprofv3 output")
    ap.add_argument("--sweep", action="store_true",
                    help="KV-only decode sweep (batch until HBM is full, 32 layers, FP16 / GEAR / "
                         "GEAR-L / KIVI) instead of the benchmark step")
    ap.add_argument("--sweep-layers", type=int, default=32)
    ap.add_argument("--sweep-prompt", type=int, default=2048)
    ap.add_argument("--sweep-new", type=int, default=64)
    ap.add_argument("--sweep-steps", type=int, default=8)
    ap.add_argument("--sweep-table", metavar="JSON", help="print the table of a --sweep output")
    args = ap.parse_args()
    if args.sweep_table:
        print(sweep_table(args.sweep_table), end="")
        return
    if args.make_profiles:
        sys.exit(make_profiles(os.path.abspath(args.make_profiles), args.workload, args.keep_raw))
    if args.sweep:
        if args.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        import torch

        import kv_cache_compression_gear_amd as gear
        torch.cuda.set_device(0)
        t0 = time.perf_counter()
        res = _sweep(gear, torch, args.sweep_layers, 32, 128, args.sweep_prompt, args.sweep_new,
                     args.sweep_steps, 2)
        print(json.dumps({"metric": "KV-only decode sweep: tok/s and peak HBM, batch raised until HBM is full",
                          "model": f"7B-shaped KV caches: {args.sweep_layers} layers x 32 heads x 128, "
                                   f"prompt {args.sweep_prompt} + {args.sweep_new} new tokens "
                                   f"({args.sweep_steps} timed decode steps)",
                          "data": "synthetic (seeded, tiled over the batch)",
                          "wall_s": round(time.perf_counter() - t0, 1), "configs": res}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the GEAR path has no cross-GPU step and this "
              f"build measures one GPU (--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_compression_gear_amd as gear
    from kv_cache_compression_gear_amd.synth import WORKLOADS

    torch.cuda.set_device(0)
    # the other workloads first, so that the headline step's instrumented pass
    # is the last launch of each of its kernels in a profiler trace
    configs = None if args.no_configs else _configs(gear, torch, WORKLOADS)
    stream = None if args.no_stream else _stream_decode(gear, WORKLOADS, torch)

    w = WORKLOADS[args.workload]
    B, H, n, d = w.batch, w.heads, w.seq, w.head_dim
    Hq = w.q_heads or H
    p = gear.Params(w.bits, w.group, w.outlier_ppm, w.rank, w.power_iters, w.chunk_tokens)
    fp = gear.Params(w.bits, w.group, w.outlier_ppm, w.fill_rank, w.power_iters)
    syn = w.kv_synth("cuda")
    k, v = syn.prompt(n)
    x = torch.cat([k.reshape(B * H, n, d), v.reshape(B * H, n, d)]).contiguous()
    M = x.shape[0]
    # warm-up steps, the timed steps, then as many steps again with per-kernel
    # and per-phase events recorded (kept out of the timed region)
    total = args.warmup + 2 * args.steps
    new_k = torch.empty((total, B, H, d), dtype=torch.float16, device="cuda")
    new_v = torch.empty_like(new_k)
    qs = torch.empty((total, B, Hq, d), dtype=torch.float16, device="cuda")
    for i in range(total):
        new_k[i], new_v[i] = syn.step()
        qs[i] = syn.queries(Hq)

    L = gear.packed_layout(p, M, n, d)
    packed = gear.Packed(torch.empty(L.total_bytes, dtype=torch.uint8, device="cuda"), p, M, n, d, L)
    ws = torch.empty(gear.compress_workspace_bytes(p, M, n, d), dtype=torch.uint8, device="cuda")
    xhat = torch.empty_like(x)
    cache = gear.Cache(B, H, d, p, fp, n, buf_tokens=w.buf_tokens, max_new_tokens=total, q_heads=Hq)
    cache.load_prompt(k.contiguous(), v.contiguous())
    del k, v
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(total)]

    def step(i, marks=False):
        e = ev[i]
        if marks:
            e[0].record()
        gear.compress(x, p, out=packed, workspace=ws)
        if marks:
            e[1].record()
        gear.decompress(packed, out=xhat)
        if marks:
            e[2].record()
        cache.append_decode_attn(new_k[i], new_v[i], qs[i], out=out)
        if marks:
            e[3].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, args.warmup + args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # the same steps again, instrumented: per-phase events and the library's
    # per-kernel HIP events on the launch stream
    gear.timing_enable(True)
    for i in range(args.warmup + args.steps, total):
        step(i, marks=True)
    torch.cuda.synchronize()
    ktimes = gear.timing_read()
    gear.timing_enable(False)

    ms_step = (t1 - t0) * 1e3 / args.steps
    timed = ev[args.warmup + args.steps:]
    comp_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in timed]))
    decomp_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in timed]))
    dec_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in timed]))
    fp16_bytes = x.numel() * 2
    packed_bytes = _packed_bytes(packed)
    value = fp16_bytes / (ms_step * 1e-3) / 1e9

    # algorithmic bytes per launch of each kernel: what it must read and write
    sec = {nme: s.numel() * s.element_size() for nme, s in
           zip(["codes", "scale", "zero", "row_ptr", "col", "val", "A", "B"], packed.sections())}
    prompt_cache = _packed_bytes(cache.prompt_packed())
    algo = {
        "select": fp16_bytes,
        "compress": fp16_bytes + sec["codes"] + sec["scale"] + sec["zero"] + sec["row_ptr"]
                    + sec["col"] + sec["val"] + sec["B"],
        "lowrank_a": fp16_bytes + sec["codes"] + sec["scale"] + sec["zero"] + sec["A"],
        "decompress": packed_bytes + fp16_bytes,
        # the compressed prompt dominates what one decode step reads
        "attn_split": prompt_cache + qs[0].numel() * 2,
    }
    kern = {k2: (n2, ms2 / n2) for k2, (n2, ms2) in ktimes.items()}
    dom = max(((k2, n2 * t2) for k2, (n2, t2) in kern.items() if k2 in algo), key=lambda z: z[1])[0]
    launch_ms = kern[dom][1]
    achieved = algo[dom] / (launch_ms * 1e-3) / 1e9
    cnt = _bound_from_counters(dom, args.workload, launch_ms, algo[dom])
    entries = M * n * d
    if cnt and cnt["bound"] == "alu" and cnt["lane_ops_per_launch"]:
        ach = cnt["lane_ops_per_launch"] / (launch_ms * 1e-3) / 1e12
        roofline = {"kernel": KERNEL_SYMBOL[dom], "bound": "alu", "achieved": round(ach, 2),
                    "peak": round(VALU_PEAK_TLANE_OPS, 2), "unit": "Tlane-op/s",
                    "frac": round(ach / VALU_PEAK_TLANE_OPS, 4), "traffic": cnt["traffic"],
                    "basis": "VALU lane-ops issued per launch (SQ_INSTS_VALU x 64, committed counters) "
                             "/ live launch time",
                    "lane_ops_per_entry": cnt["lane_ops_per_entry"],
                    "hbm_achieved": round(achieved, 1), "hbm_peak": HBM_PEAK_GBPS,
                    "hbm_frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "algorithmic_bytes": algo[dom], "launch_ms": round(launch_ms, 4)}
    else:
        roofline = {"kernel": KERNEL_SYMBOL[dom], "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": None if cnt is None else cnt["traffic"],
                    "valu_busy_frac": None if cnt is None else cnt["valu_busy_frac"],
                    "algorithmic_bytes": algo[dom], "launch_ms": round(launch_ms, 4)}

    # the compress phase as one unit: fp16 in + packed out, over its three launches
    phase_algo = fp16_bytes + packed_bytes
    ph_traffic, ph_ops, ph_ok = 0.0, 0.0, True
    for k2 in ("select", "compress", "lowrank_a"):
        if k2 not in kern:
            continue
        hb = read_profile_row("hbm_bytes", args.workload, k2)
        sq = read_profile_row("sq_counters", args.workload, k2)
        if hb is None or sq is None or sq.get("lane_ops/entry") is None:
            ph_ok = False
            continue
        ph_traffic += hb["total_B"]
        ph_ops += sq["lane_ops/entry"]
    compress_phase = {"kernels": [KERNEL_SYMBOL[k2] for k2 in ("select", "compress", "lowrank_a")
                                  if k2 in kern],
                      "algorithmic_bytes": phase_algo, "ms": round(comp_ms, 4),
                      "achieved": round(phase_algo / (comp_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                      "unit": "GB/s", "frac": round(phase_algo / (comp_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                      "traffic": round(ph_traffic) if ph_ok else None,
                      "traffic_ratio": round(ph_traffic / phase_algo, 3) if ph_ok else None,
                      "lane_ops_per_entry": round(ph_ops, 2) if ph_ok else None,
                      "valu_lane_op_budget_per_entry_at_60pct_hbm":
                          round(VALU_PEAK_TLANE_OPS * 1e12 / (0.6 * HBM_PEAK_GBPS * 1e9 / (phase_algo / entries)), 2)}

    cpu = None
    if not args.no_cpu_baseline:
        sample = x[: min(args.cpu_sample, M)].cpu().numpy().view(np.uint16)
        cpu = _cpu_baseline(w, sample, p, M)

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded K/V shaped like a 7B-class attention layer)",
        "config": {"workload": f"{w.name}: batch {B}, {H} heads, {n} tokens, head_dim {d}, "
                               f"b={w.bits} g={w.group} s={w.outlier_ppm / 1e4:g}% r={w.rank} "
                               f"t={w.power_iters}; per step: compress + decompress of all "
                               f"{M} K/V matrices, 1-token append and decode attention"},
        "phases_ms": {"compress": round(comp_ms, 4), "decompress": round(decomp_ms, 4),
                      "append+decode_attn": round(dec_ms, 4)},
        "kernels_ms": {k2: round(t2, 4) for k2, (n2, t2) in kern.items()},
        "compress_GBps_fp16": round(fp16_bytes / (comp_ms * 1e-3) / 1e9, 1),
        "decompress_GBps_fp16": round(fp16_bytes / (decomp_ms * 1e-3) / 1e9, 1),
        "decompress_hbm_frac": round((packed_bytes + fp16_bytes) / (decomp_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "decode_tok_s": round(B / (dec_ms * 1e-3), 1),
        "roofline": roofline,
        "compress_phase": compress_phase,
        "cpu_baseline": cpu,
        "configs": configs,
        "stream_gqa_decode": stream,
    }
    del cache, packed, xhat, ws, x
    torch.cuda.synchronize()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
