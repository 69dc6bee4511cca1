"""Comparison of the HIP path against the CPU oracle (test helper).

Bars (per compressed matrix):
  outlier CSR (row_ptr, col, val), scale, zero ........ bit-exact
  packed codes ......................................... bit-exact, except
      entries whose oracle quotient (x - min)/scale lies within 1e-5 of a
      half-integer (a rounding-boundary tie); those are counted and must stay
      <= 1e-6 of all entries
  L = A B^T ............... ||L_gpu - L_orc||_F <= 1e-3 ||L_orc||_F
                            (if L_orc = 0: ||L_gpu||_F <= 1e-6 ||X||_F)
  X^ (decompress) ......... ||X^_gpu - X^_orc||_F <= 1e-3 ||X^_orc||_F
  decode attention ........ ||out_gpu - out_orc||_F <= 1e-3 ||out_orc||_F
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle as orc

REL_TOL = 1e-3


def to_orc_params(p) -> orc.Params:
    return orc.Params(bits=p.bits, group=p.group, outlier_ppm=p.outlier_ppm, rank=p.rank,
                      power_iters=p.power_iters, chunk_tokens=p.chunk_tokens, seed=p.seed,
                      quant=p.quant)


def channel_keys(p, role: int) -> bool:
    """Whether a matrix of this role is quantized per channel (KIVI keys)."""
    return p.quant == orc.QUANT_KIVI and role == orc.ROLE_KEYS


def unpack_codes(packed_rows: np.ndarray, d: int, bits: int) -> np.ndarray:
    n = packed_rows.shape[0]
    out = np.zeros((n, d), np.uint8)
    per = 8 // bits
    for j in range(d):
        out[:, j] = (packed_rows[:, j // per] >> ((j % per) * bits)) & ((1 << bits) - 1)
    return out


def tie_quotients(x16: np.ndarray, ref: orc.Compressed, p, role: int = 0) -> np.ndarray:
    """fp64 distance of the oracle quotient to the nearest half-integer."""
    n, d = x16.shape
    if p.quant == orc.QUANT_ZIPCACHE:   # the quotients are of the normalized matrix
        x16 = orc.channel_normalize(x16, orc.channel_exponents(x16))
    xs = x16.view(np.float16).astype(np.float64)
    mask = np.zeros((n, d), bool)
    for t in range(n):
        for e in range(ref.row_ptr[t], ref.row_ptr[t + 1]):
            mask[t, ref.col[e]] = True
    D = np.where(mask, 0.0, xs)
    axis = 0 if channel_keys(p, role) else 1
    sc = np.repeat(ref.scale.astype(np.float64), p.group, axis=axis)
    zr = np.repeat(ref.zero.astype(np.float64), p.group, axis=axis)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(sc > 0, (D - zr) / sc, 0.0)
    return np.abs(v - np.floor(v) - 0.5)


class Report:
    def __init__(self):
        self.l_err, self.x_err, self.ties, self.entries = [], [], 0, 0

    def summary(self) -> str:
        le = np.array(self.l_err or [0.0])
        xe = np.array(self.x_err or [0.0])
        return (f"L rel err max {le.max():.2e} median {np.median(le):.2e}; "
                f"X^ rel err max {xe.max():.2e} median {np.median(xe):.2e}; "
                f"ties {self.ties} of {self.entries}")


def check_matrix(x16: np.ndarray, packed, m: int, ref: orc.Compressed, p, rep: Report,
                 xhat_gpu: np.ndarray | None = None, role: int = 0):
    """Compare compressed matrix m of `packed` (GPU) with the oracle's `ref`
    (role: what matrix m holds, keys or values)."""
    n, d = x16.shape
    k = packed.k
    # CSR of the outliers: exact
    rp = packed.row_ptr()[m].cpu().numpy()
    assert np.array_equal(rp, ref.row_ptr), f"row_ptr differs (matrix {m})"
    col = packed.col()[m].cpu().numpy().astype(np.int64) & 0xFFFF
    assert np.array_equal(col, ref.col.astype(np.int64)), f"outlier columns differ (matrix {m})"
    val = packed.val()[m].cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(val, ref.val), f"outlier values differ (matrix {m})"
    assert k == len(ref.col)
    # scale, zero: exact (the per-channel layout of KIVI keys holds as many)
    assert np.array_equal(packed.scale()[m].cpu().numpy().reshape(-1).view(np.uint32),
                          ref.scale.reshape(-1).view(np.uint32)), f"scale differs (matrix {m})"
    assert np.array_equal(packed.zero()[m].cpu().numpy().reshape(-1).view(np.uint32),
                          ref.zero.reshape(-1).view(np.uint32)), f"zero differs (matrix {m})"
    if p.quant == orc.QUANT_ZIPCACHE:
        assert np.array_equal(packed.chan()[m].cpu().numpy().view(np.uint32),
                              ref.chan.view(np.uint32)), f"channel factors differ (matrix {m})"
    # codes: exact up to counted rounding-boundary ties
    gc = packed.codes()[m].cpu().numpy()
    if not np.array_equal(gc, ref.packed):
        cg = unpack_codes(gc, d, p.bits)
        co = unpack_codes(ref.packed, d, p.bits)
        bad = cg != co
        dist = tie_quotients(x16, ref, p, role)
        assert np.all(dist[bad] < 1e-5), f"code mismatch away from a rounding tie (matrix {m})"
        rep.ties += int(bad.sum())
    rep.entries += n * d
    # L = A B^T
    if p.rank > 0:
        A = packed.A()[m].cpu().numpy().astype(np.float64)
        B = packed.B()[m].cpu().numpy().astype(np.float64)
        Lg = A @ B.T
        nref = np.linalg.norm(ref.L)
        if nref == 0:
            xs = np.linalg.norm(x16.view(np.float16).astype(np.float64))
            assert np.linalg.norm(Lg) <= 1e-6 * xs, f"nonzero L for a zero residual (matrix {m})"
            rep.l_err.append(0.0)
        else:
            e = np.linalg.norm(Lg - ref.L) / nref
            rep.l_err.append(e)
            assert e <= REL_TOL, f"L relative error {e:.3e} (matrix {m})"
    if xhat_gpu is not None:
        xr = np.linalg.norm(ref.xhat)
        e = np.linalg.norm(xhat_gpu.astype(np.float64) - ref.xhat) / max(xr, 1e-300)
        rep.x_err.append(e)
        assert e <= REL_TOL, f"X^ relative error {e:.3e} (matrix {m})"
