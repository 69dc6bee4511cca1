"""Benchmark of the GEAR hot path on one MI355X.

One step = one pass of the whole path over one 7B-shaped attention layer
(batch 8, 32 heads, 4096 tokens, head_dim 128; K and V, fp16 = 536,870,912 B):
  gear_compress    outlier top-k + CSR, 4-bit group quantization, rank-4 fit
                   (3 power iterations) of all 512 K/V matrices
  gear_decompress  reconstruction of all 512 matrices to fp16
  gear_append_tokens + gear_decode_attn
                   one new token per sequence into the streaming cache (its
                   buffer is compressed every 64 steps) and decode attention of
                   one query per head over the compressed 4096+ tokens
Inputs are synthetic, seeded, already resident in HBM.  `value` is fp16 KV
bytes per step / step time (GB/s).  Prints one JSON line.

The K timed steps run uninstrumented; K further steps then run with the
library's per-kernel HIP events on (gear_timing_*) and per-phase events, which
give `phases_ms`, `kernels_ms` and the `roofline` object: the kernel with the
largest share of a step, its launch time measured live on the launch stream.
`traffic` is its measured HBM bytes per launch from
the committed rocprofv3 counter summary under profiles/, when that summary was
taken from the current kernel sources (else null).  Next to it, the CPU
oracle is timed on a bounded sample of the same workload (`cpu_baseline`).
A second block times the streaming GQA decode workload (batch 64, 32 query /
8 KV heads, 2048-token prompt, 256 decode steps).

    python bench.py [--gpus 1] [--steps 20] [--warmup 30] [--no-cpu-baseline]
                    [--no-stream] [--copy-calibration]
    python bench.py --summarize-pmc counter_collection.csv   (profile helper)
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "kv_cache_compression_gear_amd", "csrc")
COPY_BYTES = 256 << 20          # plain copy used to calibrate the byte counters
# kernel -> source file it is built from
KERNEL_SOURCE = {"select": "gear_compress.hip", "compress": "gear_compress.hip",
                 "lowrank_a": "gear_compress.hip", "decompress": "gear_decompress.hip",
                 "attn_prompt": "gear_attn.hip", "attn_split": "gear_attn.hip",
                 "attn_combine": "gear_attn.hip", "buffer_append": "gear_attn.hip"}
# device symbol of each kernel (for rocprofv3 summaries)
# ("attn_prompt" and "attn_split" are timed together by the library, as
# "attn_split": the decode attention over all splits)
KERNEL_SYMBOL = {"select": "select_kernel", "compress": "compress_kernel",
                 "lowrank_a": "lowrank_a_kernel", "decompress": "decompress_kernel",
                 "attn_prompt": "attn_prompt_kernel", "attn_split": "attn_split_kernel",
                 "attn_combine": "attn_combine_kernel", "buffer_append": "buffer_append_kernel"}


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


def read_traffic(kernel: str, workload: str):
    """Measured HBM bytes per launch from profiles/<symbol>_<workload>_traffic.txt,
    or None if absent or taken from other kernel sources."""
    path = os.path.join(PROFILES, f"{KERNEL_SYMBOL[kernel]}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


COPY_KERNEL = "copyBuffer"      # the runtime's blit kernel behind torch's device copy
COPY_GRID = str(COPY_BYTES // 2048)   # its grid for the 256 MiB calibration copy


def summarize_pmc(path: str):
    """Per-kernel mean of each counter in a rocprofv3 counter_collection.csv;
    the 256 MiB calibration copy of --copy-calibration is listed as 'copy'."""
    vals = defaultdict(lambda: defaultdict(list))
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            key = None
            for k, sym in KERNEL_SYMBOL.items():
                if sym in name:
                    key = k
            if key is None and COPY_KERNEL in name and row["Grid_Size"] == COPY_GRID:
                key = "copy"
            if key is None:
                continue
            vals[key][row["Counter_Name"]].append(float(row["Counter_Value"]))
    return {k: {c: (sum(v) / len(v), len(v)) for c, v in d.items()} for k, d in vals.items()}


def traffic_summary(fetch_csv: str, write_csv: str, kernel: str, workload: str) -> str:
    """The traffic file read by read_traffic(): FETCH_SIZE and WRITE_SIZE (KiB
    per dispatch) of `kernel`, each divided by what the same counter reads per
    byte of the plain calibration copy."""
    f = summarize_pmc(fetch_csv)
    w = summarize_pmc(write_csv)
    kib = COPY_BYTES / 1024
    ff = f["copy"]["FETCH_SIZE"][0] / kib
    wf = w["copy"]["WRITE_SIZE"][0] / kib
    fk, nf = f[kernel]["FETCH_SIZE"]
    wk, nw = w[kernel]["WRITE_SIZE"]
    fetch_b = fk * 1024 / ff
    write_b = wk * 1024 / wf
    return "\n".join([
        f"# HBM traffic per launch of {KERNEL_SYMBOL[kernel]}, workload {workload}",
        f"kernel: {KERNEL_SYMBOL[kernel]}",
        f"fetch_size_kib_per_dispatch: {fk:.1f}   ({nf} dispatches)",
        f"write_size_kib_per_dispatch: {wk:.1f}   ({nw} dispatches)",
        f"copy_fetch_size_kib: {f['copy']['FETCH_SIZE'][0]:.1f}   (plain copy of {COPY_BYTES} bytes)",
        f"copy_write_size_kib: {w['copy']['WRITE_SIZE'][0]:.1f}",
        f"fetch_factor: {ff:.5f}",
        f"write_factor: {wf:.5f}",
        f"hbm_fetch_bytes_per_launch: {fetch_b:.0f}",
        f"hbm_write_bytes_per_launch: {write_b:.0f}",
        f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"source_sha256: {source_digest(kernel)}",
    ]) + "\n"


def _cpu_baseline(w, x_sample, p, n_mats_total):
    """The C oracle (as it stands) on a bounded sample of the same workload:
    compress + reconstruct of a number of the layer's matrices, one host thread
    per matrix."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as orc

    op = orc.Params(p.bits, p.group, p.outlier_ppm, p.rank, p.power_iters, p.chunk_tokens, p.seed)
    mats = [x_sample[i] for i in range(x_sample.shape[0])]
    threads = max(1, min(len(mats), len(os.sched_getaffinity(0)), 16))
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda m: orc.compress_matrix(m, op), mats))
    dt = time.perf_counter() - t0
    nbytes = sum(m.nbytes for m in mats)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(mats)} of the {n_mats_total} K/V matrices ({w.seq}x{w.head_dim} fp16): "
                      f"compress + reconstruct (no decode attention), {dt:.2f} s wall on "
                      f"{threads} host threads"}


def _packed_bytes(pk) -> int:
    return sum(s.numel() * s.element_size() for s in pk.sections())


def _stream_decode(gear, WORKLOADS, torch):
    """Streaming GQA decode: append + decode attention for 256 steps, timed
    uninstrumented; the same steps on a second cache (same prompt) give the
    per-kernel breakdown."""
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
        caches[0].append(nk[i], nv[i])
        caches[0].decode_attn(qs[i], out=out)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    gear.timing_enable(True)
    for i in range(steps):
        caches[1].append(nk[i], nv[i])
        caches[1].decode_attn(qs[i], out=out)
    torch.cuda.synchronize()
    kt = gear.timing_read()
    gear.timing_enable(False)
    attn_ms = sum(kt.get(k2, (0, 0.0))[1] for k2 in ("attn_split", "attn_combine"))
    return {"workload": f"stream_gqa: batch {B}, {Hq} query / {H} KV heads, prompt {n} tokens, "
                        f"{steps} decode steps, fp16 buffer {w.buf_tokens} tokens compressed "
                        f"on fill at rank {w.fill_rank}",
            "tok_s": round(B * steps / dt, 1),
            "attn_only_tok_s": round(B * steps / (attn_ms * 1e-3), 1) if attn_ms > 0 else None,
            "ms_total": round(dt * 1e3, 3),
            "kernels_ms": {k2: round(v2[1] / v2[0], 4) for k2, v2 in kt.items()}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="7b_layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=256)
    ap.add_argument("--no-stream", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--summarize-pmc", metavar="CSV",
                    help="print per-kernel counter means of a rocprofv3 counter_collection.csv")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the traffic file of --kernel from FETCH_SIZE / WRITE_SIZE runs")
    ap.add_argument("--kernel", default="compress")
    args = ap.parse_args()
    if args.traffic_summary:
        print(traffic_summary(*args.traffic_summary, args.kernel, args.workload), end="")
        return
    if args.summarize_pmc:
        for k, d in sorted(summarize_pmc(args.summarize_pmc).items()):
            for c, (mean, cnt) in sorted(d.items()):
                print(f"{k:16s} {c:12s} dispatches={cnt:4d} mean={mean:.6g}")
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the GEAR path has no cross-GPU step "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_compression_gear_amd as gear
    from kv_cache_compression_gear_amd.synth import WORKLOADS

    torch.cuda.set_device(0)
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
        cache.append(new_k[i], new_v[i])
        cache.decode_attn(qs[i], out=out)
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
    traffic = read_traffic(dom, args.workload)

    cpu = None
    if not args.no_cpu_baseline:
        sample = x[: min(args.cpu_sample, M)].cpu().numpy().view(np.uint16)
        cpu = _cpu_baseline(w, sample, p, M)

    stream = None if args.no_stream else _stream_decode(gear, WORKLOADS, torch)

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    rec = {
        "metric": "GEAR compress+decompress GB/s (fp16 KV in) & decode tok/s; % of HBM peak",
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
        "roofline": {"kernel": KERNEL_SYMBOL[dom], "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "algorithmic_bytes": algo[dom], "launch_ms": round(launch_ms, 4)},
        "cpu_baseline": cpu,
        "stream_gqa_decode": stream,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
