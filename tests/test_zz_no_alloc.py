"""gear_compress_noalloc (static device scratch, no workspace) against
gear_compress (caller's workspace): identical packed bytes on two calls in a
row, the second with a smaller input of another shape, so that scratch
contents left by the first call would show."""
import ctypes

import numpy as np
import pytest
import torch

import kv_cache_compression_gear_amd as gear
from kv_cache_compression_gear_amd.synth import KVSynth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _stack(B, H, n, d, k_ch, seed):
    syn = KVSynth(B, H, d, k_ch, seed=seed)
    k, v = syn.prompt(n)
    return torch.cat([k.reshape(B * H, n, d), v.reshape(B * H, n, d)]).to("cuda").contiguous()


def _noalloc(x, p):
    M, n, d = x.shape
    L = gear.packed_layout(p, M, n, d)
    out = gear.Packed(torch.full((L.total_bytes,), 0xAB, dtype=torch.uint8, device="cuda"), p, M, n,
                      d, L)
    st = gear.lib().gear_compress_noalloc(ctypes.byref(p._c()), ctypes.byref(gear._shape(M, n, d)),
                                          ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.buf.data_ptr()),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, gear.lib().gear_last_error()
    return out


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_compress_matches_workspace_compress(order):
    cases = [
        ("16 x 1024 x 128, b4 g128 s2% r4 t3", _stack(2, 4, 1024, 128, 4, 5), gear.Params(4, 128, 20000, 4, 3)),
        ("6 x 300 x 64, b2 g32 s3% r2 t2", _stack(1, 3, 300, 64, 2, 6), gear.Params(2, 32, 30000, 2, 2)),
    ]
    for name, x, p in cases:
        _say(f"[noalloc] {name}")
        ref = gear.compress(x, p)
        got = _noalloc(x, p)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref.sections(), got.sections())):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"section {i} differs ({name})"
        xa = gear.decompress(ref).float()
        xb = gear.decompress(got).float()
        torch.cuda.synchronize()
        assert torch.equal(xa, xb)


def test_noalloc_compress_and_decompress_under_graph_capture():
    """The callers the allocation-free entry point is for: compress (no
    workspace) and decompress captured into one HIP graph and replayed three
    times, the program's own eager work and synchronisations in between; every
    replay gives the eager call's packed bytes and reconstruction exactly."""
    p = gear.Params(4, 128, 20000, 4, 3)
    x = _stack(2, 4, 1024, 128, 4, 7)
    M, n, d = x.shape
    L = gear.packed_layout(p, M, n, d)
    ref = gear.compress(x, p)
    ref_x = gear.decompress(ref)
    pk = gear.Packed(torch.empty(L.total_bytes, dtype=torch.uint8, device="cuda"), p, M, n, d, L)
    xh = torch.empty_like(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # first calls (the scratch address lookup) outside the capture
        gear.compress_noalloc(x, p, out=pk)
        gear.decompress(pk, out=xh)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gear.compress_noalloc(x, p, out=pk)
        gear.decompress(pk, out=xh)
    torch.cuda.synchronize()
    for rep in range(3):
        _say(f"[noalloc graph] replay {rep}")
        pk.buf.fill_(0xAB)
        xh.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref.sections(), pk.sections())):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"section {i} differs (replay {rep})"
        assert torch.equal(xh.view(torch.int16), ref_x.view(torch.int16)), f"reconstruction differs (replay {rep})"
