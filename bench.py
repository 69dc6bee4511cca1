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

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def _cpu_baseline(w, x_cpu_sample, p, seconds_hint: float):
    """The C oracle (as it stands) on a bounded sample of the same workload:
    compress + reconstruct of a few matrices, one host thread per matrix."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as orc

    op = orc.Params(p.bits, p.group, p.outlier_ppm, p.rank, p.power_iters, p.chunk_tokens, p.seed)
    mats = [x_cpu_sample[i] for i in range(x_cpu_sample.shape[0])]
    threads = max(1, min(len(mats), len(os.sched_getaffinity(0)), 16))
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda m: orc.compress_matrix(m, op), mats))
    dt = time.perf_counter() - t0
    nbytes = sum(m.nbytes for m in mats)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(mats)} of the {w.num_matrices} K/V matrices ({w.seq}x{w.head_dim} fp16), "
                      f"compress + reconstruct, {dt:.1f} s wall on {threads} host threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="7b_layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=48)
    args = ap.parse_args()
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
    total = args.warmup + args.steps
    new_k = torch.empty((total, B, H, d), dtype=torch.float16, device="cuda")
    new_v = torch.empty_like(new_k)
    qs = torch.empty((total, B, Hq, d), dtype=torch.float16, device="cuda")
    for i in range(total):
        new_k[i], new_v[i] = syn.step()
        qs[i] = syn.queries(Hq)

    L = gear.packed_layout(p, M, n, d)
    packed = gear.Packed(torch.empty(L.total_bytes, dtype=torch.uint8, device="cuda"), p, M, n, d, L)
    ws = torch.empty(max(gear.compress_workspace_bytes(p, M, n, d), 256), dtype=torch.uint8, device="cuda")
    xhat = torch.empty_like(x)
    cache = gear.Cache(B, H, d, p, fp, n, buf_tokens=w.buf_tokens, max_new_tokens=total, q_heads=Hq)
    cache.load_prompt(k.contiguous(), v.contiguous())
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(total)]

    def step(i):
        e = ev[i]
        e[0].record()
        gear.compress(x, p, out=packed, workspace=ws)
        e[1].record()
        gear.decompress(packed, out=xhat)
        e[2].record()
        cache.append(new_k[i], new_v[i])
        cache.decode_attn(qs[i], out=out)
        e[3].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, total):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_step = (t1 - t0) * 1e3 / args.steps
    timed = ev[args.warmup:]
    comp_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in timed]))
    decomp_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in timed]))
    dec_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in timed]))
    fp16_bytes = x.numel() * 2
    packed_bytes = sum(s.numel() * s.element_size() for s in packed.sections())
    algo_bytes = fp16_bytes + packed_bytes          # compress: read X, write Q, S, A, B
    value = fp16_bytes / (ms_step * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        sample = x[: min(args.cpu_sample, M)].cpu().numpy().view(np.uint16)
        cpu = _cpu_baseline(w, sample, p, 20.0)

    achieved = algo_bytes / (comp_ms * 1e-3) / 1e9
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
        "dtype": "fp16 in, u8 codes, f32",
        "data": "synthetic (seeded K/V shaped like a 7B-class layer)",
        "config": {"workload": f"{w.name}: batch {B}, {H} heads, {n} tokens, head_dim {d}, "
                               f"b={w.bits} g={w.group} s={w.outlier_ppm / 1e4:g}% r={w.rank} "
                               f"t={w.power_iters}; +1 token append and decode attention per step",
                   "global_batch": B, "seq_len": n, "parallelism": "none (1 GPU)"},
        "phases_ms": {"compress": round(comp_ms, 4), "decompress": round(decomp_ms, 4),
                      "append+decode_attn": round(dec_ms, 4)},
        "compress_GBps_fp16": round(fp16_bytes / (comp_ms * 1e-3) / 1e9, 1),
        "decompress_GBps_fp16": round(fp16_bytes / (decomp_ms * 1e-3) / 1e9, 1),
        "decompress_hbm_frac": round((packed_bytes + fp16_bytes) / (decomp_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "decode_tok_s": round(B / (dec_ms * 1e-3), 1),
        "roofline": {"kernel": "compress_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
