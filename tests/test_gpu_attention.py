"""GPU parity of the streaming cache (gear_append_tokens) and of decode
attention over it (gear_decode_attn) against the oracle's cache model."""
import numpy as np
import pytest
import torch

import kv_cache_compression_gear_amd as gear
from kv_cache_compression_gear_amd.synth import KVSynth, WORKLOADS
from oracle import oracle as orc
from parity import REL_TOL, Report, check_matrix, to_orc_params

pytestmark = pytest.mark.gpu
P = gear.Params


def _say(msg):
    print(msg, flush=True)


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _attn_check(out_gpu, out_orc, batches=None, what=""):
    g = out_gpu.cpu().numpy().astype(np.float64)
    if batches is not None:
        g = g[batches]
        out_orc = out_orc[batches]
    e = _rel(g, out_orc)
    _say(f"    attention {what}: rel err {e:.2e}")
    assert e <= REL_TOL, f"decode attention relative error {e:.3e} {what}"


def _new_cache(B, Hkv, Hq, d, pp, fp, n_prompt, nb, max_new):
    return gear.Cache(B, Hkv, d, pp, fp, n_prompt, buf_tokens=nb, max_new_tokens=max_new,
                      q_heads=Hq)


@pytest.mark.parametrize("name,B,Hkv,Hq,d,n,pp", [
    ("tiny_mha", 1, 4, 4, 64, 256, P(4, 64, 20000, 4, 3)),
    ("gqa4_prompt_ragged", 2, 2, 8, 128, 700, P(4, 128, 20000, 4, 3)),
    ("gqa8_chunked", 1, 2, 16, 128, 1024, P(4, 128, 10000, 4, 3, chunk_tokens=512)),
    ("gqa2_2bit", 2, 2, 4, 128, 300, P(2, 64, 50000, 8, 4)),
    # whole 256-token prompt splits: two groups per token, rank 8, 2-bit codes
    ("whole_splits_2bit_r8", 1, 2, 4, 128, 512, P(2, 64, 50000, 8, 4)),
    # more outliers in a split than the prompt kernel stages in LDS
    ("whole_splits_dense_outliers", 1, 2, 2, 128, 512, P(4, 128, 100000, 4, 2)),
    # head_dim 64, two groups per token, no low-rank term
    ("whole_splits_d64_r0", 2, 2, 2, 64, 768, P(4, 32, 20000, 0, 0)),
    # the matrix-core kernel (2, 4 or 8 query heads per KV head, whole
    # 256-token splits) at every code width and group count it is built for
    ("gqa2_whole_4bit", 1, 2, 4, 128, 512, P(4, 128, 20000, 4, 3)),
    ("gqa2_whole_4bit_g64_r2", 1, 2, 4, 128, 512, P(4, 64, 20000, 2, 2)),
    ("gqa4_whole_2bit_r8", 1, 2, 8, 128, 512, P(2, 128, 20000, 8, 3)),
    ("gqa4_whole_2bit_g64", 1, 2, 8, 128, 768, P(2, 64, 20000, 4, 3)),
    ("gqa4_whole_4bit_r3", 2, 2, 8, 128, 512, P(4, 128, 20000, 3, 3)),
    # no low-rank term and no outliers: the A, B, column and value arrays are
    # replaced by stand-in addresses
    ("gqa4_whole_r0_no_outliers", 1, 2, 8, 128, 512, P(4, 64, 0, 0, 0)),
    ("gqa8_whole_2bit_g64_r1", 1, 2, 16, 128, 512, P(2, 64, 20000, 1, 2)),
    ("gqa8_whole_2bit_s0_r8", 1, 2, 16, 128, 512, P(2, 128, 0, 8, 3)),
    # more outliers in a split than the kernel stages in LDS (read from HBM)
    ("gqa8_whole_dense_outliers", 1, 2, 16, 128, 512, P(4, 64, 100000, 4, 2)),
])
def test_decode_attention_over_compressed_prompt(name, B, Hkv, Hq, d, n, pp):
    _say(f"[attention] {name}")
    syn = KVSynth(B, Hkv, d, 4 if d == 128 else 2, seed=1)
    k, v = syn.prompt(n)
    q = syn.queries(Hq)
    fp = P(pp.bits, pp.group, pp.outlier_ppm, 2, 3)
    cache = _new_cache(B, Hkv, Hq, d, pp, fp, n, 64, 64)
    cache.load_prompt(k.cuda().contiguous(), v.cuda().contiguous())
    out = cache.decode_attn(q.cuda())
    torch.cuda.synchronize()
    oc = orc.OracleCache(B, Hkv, d, to_orc_params(pp), to_orc_params(fp), 64)
    oc.load_prompt(k.numpy(), v.numpy())
    _attn_check(out, oc.decode_attention(q.numpy()), what=name)


@pytest.mark.parametrize("name,Hkv,Hq,d", [
    # the tail's workgroup merges the pair's splits for all of its query
    # heads: G*d columns over 256 threads
    ("fused_merge_mha_d64", 2, 2, 64),      # 64 columns, 4 threads per column
    ("fused_merge_gqa2_d64", 2, 4, 64),     # 128 columns, 2 threads per column
    ("fused_merge_gqa2_d128", 2, 4, 128),   # 256 columns, one per thread
    ("fused_merge_gqa8_d128", 1, 8, 128),   # 1024 columns, 4 per thread
])
def test_tail_merge_every_column_mapping(name, Hkv, Hq, d):
    B, n0 = 2, 512
    _say(f"[attention] {name}: prompt {n0} + 3 buffer tokens, merged by the tail")
    g = 64 if d == 64 else 128
    pp = P(4, g, 20000, 4, 3)
    fp = P(4, g, 20000, 2, 3)
    syn = KVSynth(B, Hkv, d, 4 if d == 128 else 2, seed=7)
    k, v = syn.prompt(n0)
    q = syn.queries(Hq)
    cache = _new_cache(B, Hkv, Hq, d, pp, fp, n0, 64, 8)
    cache.load_prompt(k.cuda().contiguous(), v.cuda().contiguous())
    oc = orc.OracleCache(B, Hkv, d, to_orc_params(pp), to_orc_params(fp), 64)
    oc.load_prompt(k.numpy(), v.numpy())
    for _ in range(3):
        kn, vn = syn.step()
        cache.append(kn.cuda(), vn.cuda())
        oc.append(kn.numpy(), vn.numpy())
    out = cache.decode_attn(q.cuda())
    torch.cuda.synchronize()
    _attn_check(out, oc.decode_attention(q.numpy()), what=name)


def _buffer_rows(cache, B, Hkv, d):
    """The used rows of a cache's fp16 buffer: [2, B, Hkv, buf_len, d]."""
    inf = cache.info()
    cap = cache.cfg.buf_tokens
    buf = cache._view(inf.buffer_f16, 2 * B * Hkv * cap * d * 2).view(torch.float16)
    return buf.view(2, B, Hkv, cap, d)[:, :, :, :inf.buf_len]


@pytest.mark.parametrize("name,Hkv,Hq,d,n0", [
    ("fused_step_gqa4", 2, 8, 128, 256),
    ("fused_step_mha", 2, 2, 128, 512),
    ("fused_step_gqa8", 1, 8, 128, 256),     # buffer rows read per batch, not at the start
    ("fused_step_d64", 2, 4, 64, 256),
    ("fused_step_no_prompt", 2, 4, 128, 0),
])
def test_append_decode_attn_matches_separate_calls(name, Hkv, Hq, d, n0):
    """gear_append_decode_attn (the token written by the attention launch)
    against gear_append_tokens + gear_decode_attn on a twin cache, over 140
    steps (two buffer fills, taken by the two-call path): identical outputs,
    counters, buffer rows and fills."""
    B, steps = 2, 140
    _say(f"[attention] {name}: {steps} fused steps vs separate calls")
    g = 64 if d == 64 else 128
    pp = P(4, g, 20000, 4, 3)
    fp = P(4, g, 20000, 2, 3)
    syn = KVSynth(B, Hkv, d, 4 if d == 128 else 2, seed=11)
    c1 = _new_cache(B, Hkv, Hq, d, pp, fp, n0, 64, steps)
    c2 = _new_cache(B, Hkv, Hq, d, pp, fp, n0, 64, steps)
    if n0:
        k, v = syn.prompt(n0)
        k, v = k.cuda().contiguous(), v.cuda().contiguous()
    else:
        k = v = torch.empty(0, dtype=torch.float16, device="cuda")
    c1.load_prompt(k, v)
    c2.load_prompt(k, v)
    for s in range(1, steps + 1):
        kn, vn = syn.step()
        kn, vn = kn.cuda().contiguous(), vn.cuda().contiguous()
        q = syn.queries(Hq).cuda().contiguous()
        c1.append(kn, vn)
        o1 = c1.decode_attn(q)
        o2 = c2.append_decode_attn(kn, vn, q)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), f"step {s}: max diff {(o1 - o2).abs().max().item()}"
        i1, i2 = c1.info(), c2.info()
        assert (i1.tokens, i1.buf_len, i1.num_fills) == (i2.tokens, i2.buf_len, i2.num_fills)
        assert torch.equal(_buffer_rows(c1, B, Hkv, d), _buffer_rows(c2, B, Hkv, d)), f"step {s}"
    assert c2.info().num_fills == 2
    for f in range(2):
        for a, b in zip(c1.fill_packed(f).sections(), c2.fill_packed(f).sections()):
            assert torch.equal(a, b), f"fill {f}"


def test_streaming_cache_against_oracle():
    B, Hkv, Hq, d, n0, steps = 2, 2, 8, 128, 256, 140
    _say(f"[stream] B={B} Hkv={Hkv} Hq={Hq} prompt={n0} steps={steps}")
    pp = P(4, 128, 20000, 4, 3)
    fp = P(4, 128, 20000, 2, 3)
    syn = KVSynth(B, Hkv, d, 4, seed=2)
    k, v = syn.prompt(n0)
    cache = _new_cache(B, Hkv, Hq, d, pp, fp, n0, 64, steps)
    cache.load_prompt(k.cuda().contiguous(), v.cuda().contiguous())
    oc = orc.OracleCache(B, Hkv, d, to_orc_params(pp), to_orc_params(fp), 64)
    oc.load_prompt(k.numpy(), v.numpy())
    check_at = {1, 2, 63, 64, 65, 127, 128, 129, 140}
    for s in range(1, steps + 1):
        kn, vn = syn.step()
        q = syn.queries(Hq)
        cache.append(kn.cuda(), vn.cuda())
        oc.append(kn.numpy(), vn.numpy())
        out = cache.decode_attn(q.cuda())
        if s in check_at:
            torch.cuda.synchronize()
            inf = cache.info()
            assert inf.tokens == n0 + s and inf.buf_len == s % 64 and inf.num_fills == s // 64
            _attn_check(out, oc.decode_attention(q.numpy()), what=f"step {s}")
    # the compressed fills match the oracle's bulk compression of the same tokens
    rep = Report()
    for f, segs in enumerate(oc.fills):
        packed = cache.fill_packed(f)
        xh = gear.decompress(packed).float().cpu().numpy()
        for m, ref in enumerate(segs):
            x16 = np.ascontiguousarray(oc.fill_inputs[f][m])
            check_matrix(x16, packed, m, ref, fp, rep, xh[m])
    _say(f"    fills: {rep.summary()}")


def test_bulk_append_equals_single_appends():
    B, Hkv, Hq, d, n0 = 1, 2, 4, 64, 128
    _say("[stream] bulk append of 70 tokens vs 70 single appends")
    pp = P(4, 64, 20000, 4, 3)
    fp = P(4, 64, 20000, 2, 3)
    syn = KVSynth(B, Hkv, d, 2, seed=4)
    k, v = syn.prompt(n0)
    kn, vn = syn.prompt(70)
    q = syn.queries(Hq).cuda()
    c1 = _new_cache(B, Hkv, Hq, d, pp, fp, n0, 64, 80)
    c2 = _new_cache(B, Hkv, Hq, d, pp, fp, n0, 64, 80)
    for c in (c1, c2):
        c.load_prompt(k.cuda().contiguous(), v.cuda().contiguous())
    c1.append(kn.cuda().contiguous(), vn.cuda().contiguous())
    for t in range(70):
        c2.append(kn[:, :, t].cuda().contiguous(), vn[:, :, t].cuda().contiguous())
    o1, o2 = c1.decode_attn(q), c2.decode_attn(q)
    torch.cuda.synchronize()
    for sa, sb in zip(c1.fill_packed(0).sections(), c2.fill_packed(0).sections()):
        assert torch.equal(sa.view(torch.uint8), sb.view(torch.uint8))
    assert torch.equal(o1, o2)


def test_buffer_only_and_empty_cache():
    B, Hkv, Hq, d = 2, 2, 4, 128
    _say("[attention] empty cache, then buffer-only tokens (exact fp16 attention)")
    pp = P(4, 128, 20000, 4, 3)
    fp = P(4, 128, 20000, 2, 3)
    syn = KVSynth(B, Hkv, d, 4, seed=5)
    cache = _new_cache(B, Hkv, Hq, d, pp, fp, 0, 64, 10)
    cache.load_prompt(torch.empty(0, dtype=torch.float16, device="cuda"),
                      torch.empty(0, dtype=torch.float16, device="cuda"))
    q = syn.queries(Hq)
    out = cache.decode_attn(q.cuda())
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
    oc = orc.OracleCache(B, Hkv, d, to_orc_params(pp), to_orc_params(fp), 64)
    for s in range(1, 6):
        kn, vn = syn.step()
        cache.append(kn.cuda(), vn.cuda())
        oc.append(kn.numpy(), vn.numpy())
        out = cache.decode_attn(q.cuda())
        torch.cuda.synchronize()
        if s == 1:   # one token: out = v exactly (up to fp32 rounding)
            vv = vn.float().numpy()
            exp = np.repeat(vv, Hq // Hkv, axis=1)
            assert np.allclose(out.cpu().numpy(), exp, rtol=1e-6, atol=1e-6)
        _attn_check(out, oc.decode_attention(q.numpy()), what=f"buffer-only step {s}")


def test_streaming_full_gqa_workload_sampled():
    """The 64 x (32q / 8kv) x 2048-token streaming workload, 256 decode steps,
    checked against the oracle on batches {0, 63} at steps {1, 64, 65, 256}."""
    w = WORKLOADS["stream_gqa"]
    B, Hkv, Hq, d, n0 = w.batch, w.heads, w.q_heads, w.head_dim, w.seq
    _say(f"[stream full] B={B} Hkv={Hkv} Hq={Hq} prompt={n0} steps={w.decode_steps}")
    pp = P(w.bits, w.group, w.outlier_ppm, w.rank, w.power_iters)
    fp = P(w.bits, w.group, w.outlier_ppm, w.fill_rank, w.power_iters)
    syn = w.kv_synth("cuda")
    k, v = syn.prompt(n0)
    cache = _new_cache(B, Hkv, Hq, d, pp, fp, n0, w.buf_tokens, w.decode_steps)
    cache.load_prompt(k, v)
    sel = [0, B - 1]
    oc = orc.OracleCache(len(sel), Hkv, d, to_orc_params(pp), to_orc_params(fp), w.buf_tokens)
    oc.load_prompt(k[sel].cpu().numpy(), v[sel].cpu().numpy())
    for s in range(1, w.decode_steps + 1):
        kn, vn = syn.step()
        q = syn.queries(Hq)
        cache.append(kn, vn)
        oc.append(kn[sel].cpu().numpy(), vn[sel].cpu().numpy())
        out = cache.decode_attn(q)
        if s in (1, 64, 65, 256):
            torch.cuda.synchronize()
            ref = oc.decode_attention(q[sel].cpu().numpy())
            _attn_check(out[sel], ref, what=f"step {s}")


def _full_decode_sampled(name, bsel, hsel):
    """One decode step of a full-size workload (the whole compressed prompt,
    one appended token, one query per head, MHA), sampled batches x heads
    against the oracle (heads attend independently at one query head per KV
    head)."""
    w = WORKLOADS[name]
    B, H, n, d = w.batch, w.heads, w.seq, w.head_dim
    Hq = w.q_heads or H
    assert Hq == H
    _say(f"[attention full] {name} B={B} H={H} prompt={n} chunk={w.chunk_tokens} b={w.bits} "
         f"g={w.group} r={w.rank}")
    pp = P(w.bits, w.group, w.outlier_ppm, w.rank, w.power_iters, w.chunk_tokens)
    fp = P(w.bits, w.group, w.outlier_ppm, w.fill_rank, w.power_iters)
    syn = w.kv_synth("cuda")
    k, v = syn.prompt(n)
    cache = _new_cache(B, H, Hq, d, pp, fp, n, w.buf_tokens, 1)
    cache.load_prompt(k, v)
    kn, vn = syn.step()
    q = syn.queries(Hq)
    cache.append(kn, vn)
    out = cache.decode_attn(q)
    torch.cuda.synchronize()
    oc = orc.OracleCache(len(bsel), len(hsel), d, to_orc_params(pp), to_orc_params(fp),
                         w.buf_tokens)
    oc.load_prompt(k[bsel][:, hsel].cpu().numpy(), v[bsel][:, hsel].cpu().numpy())
    oc.append(kn[bsel][:, hsel].cpu().numpy(), vn[bsel][:, hsel].cpu().numpy())
    ref = oc.decode_attention(q[bsel][:, hsel].cpu().numpy())
    _attn_check(out[bsel][:, hsel], ref, what=f"{name} sampled")


def test_decode_attention_full_7b_layer_sampled():
    """8 x 32 heads, 4096-token prompt (whole-split prompt kernel at one query
    head per KV head with staged outliers, plus the buffer tail)."""
    _full_decode_sampled("7b_layer", [0, 7], [0, 1, 2, 3])


def test_decode_attention_full_2bit_sampled():
    """16 x 32 heads, 2048-token prompt, 2-bit codes, two groups of 64 per
    token, rank 8, one query head per KV head: the prompt kernel's 2-bit MHA
    variant."""
    _full_decode_sampled("2bit", [0, 15], [0, 17, 31])


def test_decode_attention_full_long_ctx_sampled():
    """1 x 32 heads, 32,768-token prompt compressed in 64 chunks of 512
    tokens: 128 prompt splits per head merged by log-sum-exp."""
    _full_decode_sampled("long_ctx", [0], [0, 31])
