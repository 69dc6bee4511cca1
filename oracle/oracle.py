"""Python face of the CPU oracle for the GEAR compression path.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  The arithmetic lives
in ``gear_oracle.c`` (plain C, fp64 except the fp32 quantizer); this module
only marshals numpy arrays and holds the plain bookkeeping of the streaming
cache (which segments exist, what the buffer holds).

Sources: the GEAR pages -- "GEAR: Efficient KV Cache Compression for LLM
Inference" (allpcb.com Q&A, section Q3) and the app.cochat.ai page for "GEAR:
An Efficient KV Cache Compression Recipe for Near-Lossless Generative Inference
of LLM" (its "Cites" list of quoted paper sentences).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gear_oracle.c")
_LIB = os.path.join(_HERE, "libgear_oracle.so")

_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile gear_oracle.c with gcc into libgear_oracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, u64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64
        L.orc_half_to_double.restype = ctypes.c_double
        L.orc_half_to_double.argtypes = [ctypes.c_uint16]
        L.orc_num_outliers.restype = i64
        L.orc_num_outliers.argtypes = [i64, i64, i32]
        L.orc_select_outliers.argtypes = [P, i64, i64, i64, P]
        L.orc_build_csr.argtypes = [P, P, i64, i64, P, P, P]
        L.orc_quantize.argtypes = [P, i64, i64, ctypes.c_int, ctypes.c_int, P, P, P]
        L.orc_pack_codes.argtypes = [P, i64, i64, ctypes.c_int, P]
        L.orc_dequantize.argtypes = [P, P, P, i64, i64, ctypes.c_int, P]
        L.orc_splitmix64.restype = u64
        L.orc_splitmix64.argtypes = [u64, u64]
        L.orc_init_b0.argtypes = [i64, ctypes.c_int, u64, P]
        L.orc_mgs.argtypes = [P, i64, ctypes.c_int]
        L.orc_power_iteration.argtypes = [P, i64, i64, ctypes.c_int, ctypes.c_int, P, P, P]
        L.orc_low_rank_product.argtypes = [P, P, i64, i64, ctypes.c_int, P]
        L.orc_compress_matrix.argtypes = [P, i64, i64, ctypes.c_int, ctypes.c_int, i32,
                                          ctypes.c_int, ctypes.c_int, u64,
                                          P, P, P, P, P, P, P, P, P, P]
        L.orc_attention.argtypes = [P, P, i64, i64, P, ctypes.c_double, P]
        L.orc_quantize_channel.argtypes = [P, i64, i64, ctypes.c_int, ctypes.c_int, P, P, P]
        L.orc_dequantize_channel.argtypes = [P, P, P, i64, i64, ctypes.c_int, P]
        L.orc_compress_matrix_mode.argtypes = [P, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               i32, ctypes.c_int, ctypes.c_int, u64,
                                               P, P, P, P, P, P, P, P, P, P]
        L.orc_channel_exponents.argtypes = [P, i64, i64, P]
        L.orc_double_to_half.restype = ctypes.c_uint16
        L.orc_double_to_half.argtypes = [ctypes.c_double]
        L.orc_channel_normalize.argtypes = [P, i64, i64, P, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _bits16(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    assert x.dtype == np.uint16
    return np.ascontiguousarray(x)


# --------------------------------------------------------------------------
# Single steps (exposed for the pins)
# --------------------------------------------------------------------------

def num_outliers(n: int, d: int, ppm: int) -> int:
    return int(lib().orc_num_outliers(n, d, ppm))


def select_outliers(x, k: int) -> np.ndarray:
    """Boolean mask of the k selected outlier entries of x (n x d fp16)."""
    xb = _bits16(x)
    n, d = xb.shape
    mask = np.zeros((n, d), np.uint8)
    lib().orc_select_outliers(_p(xb), n, d, k, _p(mask))
    return mask.astype(bool)


def quantize(D: np.ndarray, bits: int, group: int):
    """Group quantization of an fp32 matrix: (codes uint8 [n,d], scale, zero)."""
    D = np.ascontiguousarray(D, dtype=np.float32)
    n, d = D.shape
    code = np.zeros((n, d), np.uint8)
    scale = np.zeros((n, d // group), np.float32)
    zero = np.zeros((n, d // group), np.float32)
    lib().orc_quantize(_p(D), n, d, bits, group, _p(code), _p(scale), _p(zero))
    return code, scale, zero


def pack_codes(code: np.ndarray, bits: int) -> np.ndarray:
    code = np.ascontiguousarray(code, dtype=np.uint8)
    n, d = code.shape
    out = np.zeros((n, d * bits // 8), np.uint8)
    lib().orc_pack_codes(_p(code), n, d, bits, _p(out))
    return out


def quantize_channel(D: np.ndarray, bits: int, group: int):
    """Per-channel quantization (groups of `group` tokens of one column):
    (codes uint8 [n,d], scale [n/group, d], zero [n/group, d])."""
    D = np.ascontiguousarray(D, dtype=np.float32)
    n, d = D.shape
    code = np.zeros((n, d), np.uint8)
    scale = np.zeros((n // group, d), np.float32)
    zero = np.zeros((n // group, d), np.float32)
    lib().orc_quantize_channel(_p(D), n, d, bits, group, _p(code), _p(scale), _p(zero))
    return code, scale, zero


def dequantize_channel(code, scale, zero, group: int) -> np.ndarray:
    code = np.ascontiguousarray(code, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    zero = np.ascontiguousarray(zero, dtype=np.float32)
    n, d = code.shape
    out = np.zeros((n, d), np.float64)
    lib().orc_dequantize_channel(_p(code), _p(scale), _p(zero), n, d, group, _p(out))
    return out


def channel_exponents(x) -> np.ndarray:
    """e_j: the smallest power of two not below channel j's largest |x|."""
    xb = _bits16(x)
    n, d = xb.shape
    e = np.zeros(d, np.int32)
    lib().orc_channel_exponents(_p(xb), n, d, _p(e))
    return e


def double_to_half(v: float) -> int:
    return int(lib().orc_double_to_half(float(v)))


def channel_normalize(x, e) -> np.ndarray:
    """fl16(x * 2^-e_j) as fp16 bits."""
    xb = _bits16(x)
    n, d = xb.shape
    e = np.ascontiguousarray(e, dtype=np.int32)
    out = np.zeros((n, d), np.uint16)
    lib().orc_channel_normalize(_p(xb), n, d, _p(e), _p(out))
    return out


def dequantize(code, scale, zero, group: int) -> np.ndarray:
    code = np.ascontiguousarray(code, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    zero = np.ascontiguousarray(zero, dtype=np.float32)
    n, d = code.shape
    out = np.zeros((n, d), np.float64)
    lib().orc_dequantize(_p(code), _p(scale), _p(zero), n, d, group, _p(out))
    return out


def splitmix64(seed: int, i: int) -> int:
    return int(lib().orc_splitmix64(seed, i))


def init_b0(d: int, r: int, seed: int) -> np.ndarray:
    out = np.zeros((d, r), np.float64)
    lib().orc_init_b0(d, r, seed, _p(out))
    return out


def mgs(P: np.ndarray) -> np.ndarray:
    A = np.array(P, dtype=np.float64, order="C", copy=True)
    lib().orc_mgs(_p(A), A.shape[0], A.shape[1])
    return A


def power_iteration(R: np.ndarray, r: int, iters: int, B0: np.ndarray):
    """(A, B) after `iters` PowerSGD steps on R from B0."""
    R = np.ascontiguousarray(R, dtype=np.float64)
    B0 = np.ascontiguousarray(B0, dtype=np.float64)
    n, d = R.shape
    A = np.zeros((n, r), np.float64)
    B = np.zeros((d, r), np.float64)
    lib().orc_power_iteration(_p(R), n, d, r, iters, _p(B0), _p(A), _p(B))
    return A, B


def low_rank_product(A, B) -> np.ndarray:
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    n, r = A.shape
    d = B.shape[0]
    L = np.zeros((n, d), np.float64)
    lib().orc_low_rank_product(_p(A), _p(B), n, d, r, _p(L))
    return L


def attention(K: np.ndarray, V: np.ndarray, q: np.ndarray, scale: float) -> np.ndarray:
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    q = np.ascontiguousarray(q, dtype=np.float64)
    ntok, d = K.shape
    out = np.zeros(d, np.float64)
    lib().orc_attention(_p(K), _p(V), ntok, d, _p(q), float(scale), _p(out))
    return out


# --------------------------------------------------------------------------
# Whole-matrix compression
# --------------------------------------------------------------------------

QUANT_GROUP, QUANT_KIVI, QUANT_ZIPCACHE = 0, 1, 2
ROLE_KEYS, ROLE_VALUES = 0, 1


@dataclass(frozen=True)
class Params:
    """GEAR settings: b-bit codes, group size g, outlier share in parts per
    million, rank r, power iterations t, chunking, B0 seed, and the
    quantization backbone: GEAR's own (groups of g head_dim columns of a
    token), KIVI (keys: groups of g tokens of a channel; values as GEAR's) or
    ZipCache (channels separated out by powers of two, then one group per
    token)."""
    bits: int = 4
    group: int = 128
    outlier_ppm: int = 20000
    rank: int = 4
    power_iters: int = 3
    chunk_tokens: int = 0
    seed: int = 0
    quant: int = QUANT_GROUP


@dataclass
class Compressed:
    """One compressed matrix (n x d)."""
    packed: np.ndarray   # uint8 [n, d*bits/8]
    scale: np.ndarray    # float32 [n, d/g]
    zero: np.ndarray     # float32 [n, d/g]
    row_ptr: np.ndarray  # int32 [n+1]
    col: np.ndarray      # uint16 [k]
    val: np.ndarray      # uint16 [k] (fp16 bits)
    A: np.ndarray        # float64 [n, r]
    B: np.ndarray        # float64 [d, r]
    L: np.ndarray        # float64 [n, d]
    xhat: np.ndarray     # float64 [n, d]
    chan: np.ndarray | None = None   # ZipCache: float32 [d] channel factors 2^e_j


def compress_matrix(x, p: Params, role: int = ROLE_KEYS) -> Compressed:
    """One n x d matrix.  role says whether it holds keys or values (only
    the KIVI backbone treats them differently)."""
    xb = _bits16(x)
    n, d = xb.shape
    if p.quant == QUANT_ZIPCACHE:
        # the channels separated out, GEAR with one group per token on the rest
        assert p.group == d, "ZipCache's quantization is tokenwise: group = head_dim"
        e = channel_exponents(xb)
        xt = channel_normalize(xb, e)
        c = compress_matrix(xt, Params(**{**p.__dict__, "quant": QUANT_GROUP}), role)
        f = np.ldexp(1.0, e)
        c.chan = f.astype(np.float32)
        c.xhat = c.xhat * f[None, :]
        return c
    mode = 1 if (p.quant == QUANT_KIVI and role == ROLE_KEYS) else 0
    if mode == 1:
        assert n % p.group == 0, "KIVI keys: tokens per matrix must be a multiple of the group"
    k = num_outliers(n, d, p.outlier_ppm)
    r = p.rank
    pshape = (n // p.group, d) if mode == 1 else (n, d // p.group)
    out = Compressed(
        packed=np.zeros((n, d * p.bits // 8), np.uint8),
        scale=np.zeros(pshape, np.float32),
        zero=np.zeros(pshape, np.float32),
        row_ptr=np.zeros(n + 1, np.int32),
        col=np.zeros(max(k, 1), np.uint16),
        val=np.zeros(max(k, 1), np.uint16),
        A=np.zeros((n, max(r, 1)), np.float64),
        B=np.zeros((d, max(r, 1)), np.float64),
        L=np.zeros((n, d), np.float64),
        xhat=np.zeros((n, d), np.float64),
    )
    lib().orc_compress_matrix_mode(
        _p(xb), n, d, p.bits, p.group, mode, p.outlier_ppm, r, p.power_iters, p.seed,
        _p(out.packed), _p(out.scale), _p(out.zero), _p(out.row_ptr),
        _p(out.col), _p(out.val), _p(out.A), _p(out.B), _p(out.L), _p(out.xhat))
    out.col, out.val = out.col[:k], out.val[:k]
    out.A, out.B = out.A[:, :r], out.B[:, :r]
    return out


def compress(x, p: Params, role: int = ROLE_KEYS, roles=None) -> list:
    """Compress a stack of matrices x [M, n, d].  With chunk_tokens > 0 each
    matrix is cut into n/chunk_tokens row chunks, compressed independently;
    the result is ordered matrix-major, chunk-minor.  roles (optional) gives
    each matrix's role, else every matrix has `role`."""
    xb = _bits16(x)
    M, n, d = xb.shape
    ct = p.chunk_tokens or n
    assert n % ct == 0
    res = []
    for m in range(M):
        rm = role if roles is None else roles[m]
        for c in range(n // ct):
            res.append(compress_matrix(xb[m, c * ct:(c + 1) * ct], p, rm))
    return res


# --------------------------------------------------------------------------
# Streaming cache and decode attention
# --------------------------------------------------------------------------
# [QA] Q3 "Streaming strategy": new tokens' KV first go to a small buffer and
# compression runs when the buffer fills.  [CITES] (ZeroQuant entry, Method):
# rank 2 for each group of n_b new tokens.
# readings: the buffer holds n_b tokens of exact fp16; on the append that
# fills it the n_b tokens are compressed as one new segment (same b, g, s as
# configured for decode chunks) and the buffer empties; segments are never
# merged or recompressed; a query sees every cached token (no mask); query
# head h reads KV head floor(h / (Hq/Hkv)).

def half_to_float64(x) -> np.ndarray:
    return np.asarray(x).view(np.float16).astype(np.float64) if np.asarray(x).dtype == np.uint16 \
        else np.asarray(x, dtype=np.float16).astype(np.float64)


class OracleCache:
    """Reference model of the compressed KV cache of one layer.

    Holds, per (b, kv-head), the fp64 reconstructions of every compressed
    segment in token order plus the exact fp16 buffer rows.
    """

    def __init__(self, batch: int, kv_heads: int, head_dim: int, prompt: Params,
                 fill: Params, buf_tokens: int = 64):
        self.B, self.H, self.d = batch, kv_heads, head_dim
        self.prompt_p, self.fill_p, self.nb = prompt, fill, buf_tokens
        self.K = [[[] for _ in range(kv_heads)] for _ in range(batch)]
        self.V = [[[] for _ in range(kv_heads)] for _ in range(batch)]
        self.buf_k = np.zeros((batch, kv_heads, buf_tokens, head_dim), np.uint16)
        self.buf_v = np.zeros((batch, kv_heads, buf_tokens, head_dim), np.uint16)
        self.buf_len = 0
        self.fills = []          # list of per-fill Compressed lists (K then V)
        self.fill_inputs = []    # the fp16 inputs of each fill, [2*B*H, n_b, d]

    def load_prompt(self, k, v):
        """k, v: fp16 [B, H, n, d]; compressed with the prompt settings."""
        kb, vb = _bits16(k), _bits16(v)
        B, H, n, d = kb.shape
        x = np.concatenate([kb.reshape(B * H, n, d), vb.reshape(B * H, n, d)])
        segs = compress(x, self.prompt_p, roles=[ROLE_KEYS] * (B * H) + [ROLE_VALUES] * (B * H))
        C = len(segs) // (2 * B * H)
        for t in range(2):
            for b in range(B):
                for h in range(H):
                    m = (t * B + b) * H + h
                    for c in range(C):
                        (self.K if t == 0 else self.V)[b][h].append(segs[m * C + c].xhat)
        return segs

    def append(self, k_new, v_new):
        """k_new, v_new: fp16 [B, H, d] -- one new token per sequence."""
        self.buf_k[:, :, self.buf_len] = _bits16(k_new)
        self.buf_v[:, :, self.buf_len] = _bits16(v_new)
        self.buf_len += 1
        if self.buf_len == self.nb:
            B, H, nb, d = self.buf_k.shape
            x = np.concatenate([self.buf_k.reshape(B * H, nb, d),
                                self.buf_v.reshape(B * H, nb, d)])
            segs = compress(x, Params(**{**self.fill_p.__dict__, "chunk_tokens": 0}),
                            roles=[ROLE_KEYS] * (B * H) + [ROLE_VALUES] * (B * H))
            self.fill_inputs.append(x)
            for t in range(2):
                for b in range(B):
                    for h in range(H):
                        (self.K if t == 0 else self.V)[b][h].append(segs[(t * B + b) * H + h].xhat)
            self.fills.append(segs)
            self.buf_len = 0

    def kv(self, b: int, h: int):
        """Full K^, V^ of (b, h) in token order, fp64."""
        ks = self.K[b][h] + [half_to_float64(self.buf_k[b, h, :self.buf_len])]
        vs = self.V[b][h] + [half_to_float64(self.buf_v[b, h, :self.buf_len])]
        return np.concatenate(ks), np.concatenate(vs)

    def decode_attention(self, q, scale: float | None = None, batches=None) -> np.ndarray:
        """q: fp16 [B, Hq, d] -> out float64 [B, Hq, d] (rows of batches not
        listed in `batches` are left as zero)."""
        qf = half_to_float64(_bits16(q))
        B, Hq, d = qf.shape
        grp = Hq // self.H
        scale = 1.0 / np.sqrt(d) if scale is None else scale
        out = np.zeros((B, Hq, d), np.float64)
        for b in (range(B) if batches is None else batches):
            for h in range(self.H):
                K, V = self.kv(b, h)
                for hq in range(h * grp, (h + 1) * grp):
                    out[b, hq] = attention(K, V, qf[b, hq], scale)
        return out
