"""kv_cache_compression_gear_amd -- GEAR KV-cache compression on AMD MI355X.

Thin Python binding of libgear.so (see include/gear.h).  Every step of the
compression path runs in the library's HIP kernels; this module only marshals
arguments, and uses PyTorch for device memory and the current stream.  It
raises if the library is missing: there is no CPU fallback.

    import kv_cache_compression_gear_amd as gear
    p = gear.Params(bits=4, group=128, outlier_ppm=20000, rank=4, power_iters=3)
    packed = gear.compress(x, p)          # x: fp16 [M, n, d] on the GPU
    xhat = gear.decompress(packed)        # fp16 [M, n, d]
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgear.so")

GEAR_OK = 0
_STATUS = {0: "GEAR_OK", 1: "GEAR_ERR_INVALID_ARG", 2: "GEAR_ERR_UNSUPPORTED",
           3: "GEAR_ERR_CAPACITY", 4: "GEAR_ERR_HIP", 5: "GEAR_ERR_WORKSPACE"}


class GearError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status


# quantization backbones (gear_quant) and roles of a stack (gear_role)
QUANT_GROUP, QUANT_KIVI, QUANT_ZIPCACHE = 0, 1, 2
ROLE_KEYS, ROLE_VALUES, ROLE_KEYS_THEN_VALUES = 0, 1, 2


class _Params(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("outlier_ppm", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("power_iters", ctypes.c_int32), ("chunk_tokens", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("quant", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class _Shape(ctypes.Structure):
    _fields_ = [("num_mats", ctypes.c_int64), ("n_tokens", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("role", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class _Layout(ctypes.Structure):
    _fields_ = [("num_compressed", ctypes.c_int64), ("rows", ctypes.c_int32), ("k", ctypes.c_int32),
                ("off_codes", ctypes.c_size_t), ("off_scale", ctypes.c_size_t),
                ("off_zero", ctypes.c_size_t), ("off_row_ptr", ctypes.c_size_t),
                ("off_col", ctypes.c_size_t), ("off_val", ctypes.c_size_t),
                ("off_a", ctypes.c_size_t), ("off_b", ctypes.c_size_t), ("off_chan", ctypes.c_size_t),
                ("total_bytes", ctypes.c_size_t)]


class _CacheConfig(ctypes.Structure):
    _fields_ = [("prompt", _Params), ("fill", _Params), ("batch", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("prompt_tokens", ctypes.c_int32), ("buf_tokens", ctypes.c_int32),
                ("max_new_tokens", ctypes.c_int32)]


class _CacheInfo(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("buf_len", ctypes.c_int32),
                ("num_fills", ctypes.c_int32), ("prompt_packed", ctypes.c_void_p),
                ("fill_packed", ctypes.c_void_p), ("fill_stride", ctypes.c_size_t),
                ("buffer_f16", ctypes.c_void_p)]


# Every symbol include/gear.h declares (checked by the tests).
EXPORTS = ["gear_packed_layout", "gear_packed_bytes", "gear_compress_workspace_bytes",
           "gear_compress", "gear_compress_noalloc", "gear_decompress",
           "gear_cache_arena_bytes", "gear_cache_workspace_bytes", "gear_cache_create",
           "gear_cache_destroy", "gear_cache_load_prompt", "gear_append_tokens",
           "gear_decode_attn", "gear_append_decode_attn", "gear_cache_get_info", "gear_timing_enable", "gear_timing_read",
           "gear_status_str", "gear_last_error"]

# Kernel names accepted by gear_timing_read.
KERNELS = ["select", "compress", "lowrank_a", "decompress", "attn_split", "attn_combine",
           "buffer_append", "channel"]

_lib = None


def lib():
    """The loaded libgear.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m kv_cache_compression_gear_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, S, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_size_t
        pp, ps = ctypes.POINTER(_Params), ctypes.POINTER(_Shape)
        pc = ctypes.POINTER(_CacheConfig)
        L.gear_packed_layout.restype = S
        L.gear_packed_layout.argtypes = [pp, ps, ctypes.POINTER(_Layout)]
        L.gear_packed_bytes.restype = sz
        L.gear_packed_bytes.argtypes = [pp, ps]
        L.gear_compress_workspace_bytes.restype = sz
        L.gear_compress_workspace_bytes.argtypes = [pp, ps]
        L.gear_compress.restype = S
        L.gear_compress.argtypes = [pp, ps, P, P, P, sz, P]
        L.gear_compress_noalloc.restype = S
        L.gear_compress_noalloc.argtypes = [pp, ps, P, P, P]
        L.gear_decompress.restype = S
        L.gear_decompress.argtypes = [pp, ps, P, P, P]
        L.gear_cache_arena_bytes.restype = sz
        L.gear_cache_arena_bytes.argtypes = [pc]
        L.gear_cache_workspace_bytes.restype = sz
        L.gear_cache_workspace_bytes.argtypes = [pc, i32]
        L.gear_cache_create.restype = S
        L.gear_cache_create.argtypes = [pc, P, sz, ctypes.POINTER(P)]
        L.gear_cache_destroy.restype = None
        L.gear_cache_destroy.argtypes = [P]
        L.gear_cache_load_prompt.restype = S
        L.gear_cache_load_prompt.argtypes = [P, P, P, P, sz, P]
        L.gear_append_tokens.restype = S
        L.gear_append_tokens.argtypes = [P, P, P, i32, P, sz, P]
        L.gear_decode_attn.restype = S
        L.gear_decode_attn.argtypes = [P, P, i32, ctypes.c_float, P, P, sz, P]
        L.gear_append_decode_attn.restype = S
        L.gear_append_decode_attn.argtypes = [P, P, P, P, i32, ctypes.c_float, P, P, sz, P]
        L.gear_cache_get_info.restype = S
        L.gear_cache_get_info.argtypes = [P, ctypes.POINTER(_CacheInfo)]
        L.gear_timing_enable.restype = S
        L.gear_timing_enable.argtypes = [S]
        L.gear_timing_read.restype = S
        L.gear_timing_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_double)]
        L.gear_status_str.restype = ctypes.c_char_p
        L.gear_status_str.argtypes = [S]
        L.gear_last_error.restype = ctypes.c_char_p
        L.gear_last_error.argtypes = []
        _lib = L
    return _lib


def _check(status: int):
    if status != GEAR_OK:
        raise GearError(status, lib().gear_last_error().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


@dataclass(frozen=True)
class Params:
    """GEAR settings (bits b, group g, outlier share in ppm, rank r,
    power-iteration steps t, optional token chunking, B0 seed, quantization
    backbone: QUANT_GROUP (GEAR's own), QUANT_KIVI, QUANT_ZIPCACHE)."""
    bits: int = 4
    group: int = 128
    outlier_ppm: int = 20000
    rank: int = 4
    power_iters: int = 3
    chunk_tokens: int = 0
    seed: int = 0
    quant: int = QUANT_GROUP

    def _c(self) -> _Params:
        return _Params(self.bits, self.group, self.outlier_ppm, self.rank, self.power_iters,
                       self.chunk_tokens, self.seed, self.quant, 0)


def _shape(num_mats: int, n: int, d: int, role: int = ROLE_KEYS) -> _Shape:
    return _Shape(num_mats, n, d, role, 0)


def packed_layout(p: Params, num_mats: int, n_tokens: int, head_dim: int,
                  role: int = ROLE_KEYS) -> _Layout:
    L = _Layout()
    _check(lib().gear_packed_layout(ctypes.byref(p._c()),
                                    ctypes.byref(_shape(num_mats, n_tokens, head_dim, role)), ctypes.byref(L)))
    return L


def compress_workspace_bytes(p: Params, num_mats: int, n_tokens: int, head_dim: int,
                             role: int = ROLE_KEYS) -> int:
    n = lib().gear_compress_workspace_bytes(ctypes.byref(p._c()),
                                            ctypes.byref(_shape(num_mats, n_tokens, head_dim, role)))
    if n == 0:
        _check(1)
    return n


class Packed:
    """A compressed stack: one uint8 device buffer plus typed section views.
    role: which matrices hold keys (only the KIVI backbone cares)."""

    def __init__(self, buf: torch.Tensor, p: Params, num_mats: int, n_tokens: int, head_dim: int,
                 layout: _Layout, role: int = ROLE_KEYS):
        self.buf, self.params = buf, p
        self.num_mats, self.n_tokens, self.head_dim = num_mats, n_tokens, head_dim
        self.layout = layout
        self.role = role

    def sections(self):
        """The sections, in layout order (alignment padding excluded)."""
        out = [self.codes(), self.scale(), self.zero(), self.row_ptr(), self.col(), self.val(),
               self.A(), self.B()]
        if self.params.quant == QUANT_ZIPCACHE:
            out.append(self.chan())
        return out

    def chan(self):
        """ZipCache channel factors [M, d] (float32)."""
        return self._sec(self.layout.off_chan, self.M * self.head_dim, torch.float32).view(self.M, self.head_dim)

    def _sec(self, off: int, count: int, dtype: torch.dtype) -> torch.Tensor:
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        return self.buf[off:off + nbytes].view(dtype)

    @property
    def M(self) -> int:
        return self.layout.num_compressed

    @property
    def rows(self) -> int:
        return self.layout.rows

    @property
    def k(self) -> int:
        return self.layout.k

    def codes(self):
        L, d = self.layout, self.head_dim
        return self._sec(L.off_codes, self.M * self.rows * d * self.params.bits // 8,
                         torch.uint8).view(self.M, self.rows, d * self.params.bits // 8)

    def scale(self):
        ng = self.head_dim // self.params.group
        return self._sec(self.layout.off_scale, self.M * self.rows * ng, torch.float32).view(self.M, self.rows, ng)

    def zero(self):
        ng = self.head_dim // self.params.group
        return self._sec(self.layout.off_zero, self.M * self.rows * ng, torch.float32).view(self.M, self.rows, ng)

    def row_ptr(self):
        return self._sec(self.layout.off_row_ptr, self.M * (self.rows + 1), torch.int32).view(self.M, self.rows + 1)

    def col(self):
        return self._sec(self.layout.off_col, self.M * self.k, torch.int16).view(self.M, self.k)

    def val(self):
        return self._sec(self.layout.off_val, self.M * self.k, torch.float16).view(self.M, self.k)

    def A(self):
        r = self.params.rank
        return self._sec(self.layout.off_a, self.M * self.rows * r, torch.float32).view(self.M, self.rows, r)

    def B(self):
        r = self.params.rank
        return self._sec(self.layout.off_b, self.M * self.head_dim * r, torch.float32).view(self.M, self.head_dim, r)


def _check_input(x: torch.Tensor):
    if not (x.is_cuda and x.dtype == torch.float16 and x.is_contiguous()):
        raise ValueError("expected a contiguous fp16 CUDA tensor")


def compress(x: torch.Tensor, p: Params, out: Packed | None = None,
             workspace: torch.Tensor | None = None, role: int = ROLE_KEYS) -> Packed:
    """x: fp16 [M, n, d] (or [..., n, d]) on the GPU -> Packed."""
    _check_input(x)
    n, d = x.shape[-2], x.shape[-1]
    M = x.numel() // (n * d)
    L = packed_layout(p, M, n, d, role)
    if out is None:
        out = Packed(torch.empty(L.total_bytes, dtype=torch.uint8, device=x.device), p, M, n, d, L, role)
    if workspace is None:
        workspace = torch.empty(max(compress_workspace_bytes(p, M, n, d, role), 256), dtype=torch.uint8,
                                device=x.device)
    _check(lib().gear_compress(ctypes.byref(p._c()), ctypes.byref(_shape(M, n, d, role)), _ptr(x),
                               _ptr(out.buf), _ptr(workspace), workspace.numel(), _stream()))
    return out


def compress_noalloc(x: torch.Tensor, p: Params, out: Packed) -> Packed:
    """gear_compress_noalloc: like compress(), into a caller-provided Packed,
    with the library's static device scratch instead of a workspace."""
    _check_input(x)
    n, d = x.shape[-2], x.shape[-1]
    M = x.numel() // (n * d)
    _check(lib().gear_compress_noalloc(ctypes.byref(p._c()), ctypes.byref(_shape(M, n, d, out.role)),
                                       _ptr(x), _ptr(out.buf), _stream()))
    return out


def timing_enable(on: bool = True):
    """Start (or stop and drop) per-kernel HIP-event timing inside the library."""
    _check(lib().gear_timing_enable(1 if on else 0))


def timing_read() -> dict:
    """{kernel: (launches, total_ms)} since timing_enable(True); waits for the events."""
    out = {}
    for name in KERNELS:
        n, ms = ctypes.c_int64(), ctypes.c_double()
        _check(lib().gear_timing_read(name.encode(), ctypes.byref(n), ctypes.byref(ms)))
        if n.value:
            out[name] = (n.value, ms.value)
    return out


def decompress(packed: Packed, out: torch.Tensor | None = None) -> torch.Tensor:
    M, n, d = packed.num_mats, packed.n_tokens, packed.head_dim
    if out is None:
        out = torch.empty((M, n, d), dtype=torch.float16, device=packed.buf.device)
    _check_input(out)
    _check(lib().gear_decompress(ctypes.byref(packed.params._c()), ctypes.byref(_shape(M, n, d, packed.role)),
                                 _ptr(packed.buf), _ptr(out), _stream()))
    return out


class Cache:
    """Streaming GEAR cache of one attention layer (device arena owned here)."""

    def __init__(self, batch: int, kv_heads: int, head_dim: int, prompt: Params, fill: Params,
                 prompt_tokens: int, buf_tokens: int = 64, max_new_tokens: int = 256,
                 q_heads: int | None = None, device: str = "cuda"):
        self.cfg = _CacheConfig(prompt._c(), fill._c(), batch, kv_heads, head_dim, prompt_tokens,
                                buf_tokens, max_new_tokens)
        self.batch, self.kv_heads, self.head_dim = batch, kv_heads, head_dim
        self.prompt_params, self.fill_params = prompt, fill
        self.q_heads = q_heads or kv_heads
        L = lib()
        nbytes = L.gear_cache_arena_bytes(ctypes.byref(self.cfg))
        if nbytes == 0:
            _check(1)
        wbytes = L.gear_cache_workspace_bytes(ctypes.byref(self.cfg), self.q_heads)
        if wbytes == 0:
            _check(1)
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.workspace = torch.empty(wbytes, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        _check(L.gear_cache_create(ctypes.byref(self.cfg), _ptr(self.arena), nbytes, ctypes.byref(h)))
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.gear_cache_destroy(h)
            self._h = None

    def load_prompt(self, k: torch.Tensor, v: torch.Tensor):
        _check_input(k)
        _check_input(v)
        _check(lib().gear_cache_load_prompt(self._h, _ptr(k), _ptr(v), _ptr(self.workspace),
                                            self.workspace.numel(), _stream()))

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor):
        """k_new, v_new: fp16 [B, Hkv, n_new, d] (or [B, Hkv, d] for one token)."""
        _check_input(k_new)
        _check_input(v_new)
        n_new = 1 if k_new.dim() == 3 else k_new.shape[2]
        _check(lib().gear_append_tokens(self._h, _ptr(k_new), _ptr(v_new), n_new,
                                        _ptr(self.workspace), self.workspace.numel(), _stream()))

    def decode_attn(self, q: torch.Tensor, sm_scale: float | None = None,
                    out: torch.Tensor | None = None) -> torch.Tensor:
        _check_input(q)
        B, Hq, d = q.shape
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        scale = 1.0 / (d ** 0.5) if sm_scale is None else sm_scale
        _check(lib().gear_decode_attn(self._h, _ptr(q), Hq, ctypes.c_float(scale), _ptr(out),
                                      _ptr(self.workspace), self.workspace.numel(), _stream()))
        return out

    def append_decode_attn(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                           sm_scale: float | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
        """One decode step: append one token per sequence (k_new, v_new fp16
        [B, Hkv, d]) and take decode attention of q (fp16 [B, Hq, d]) over the
        cache including it; the same as append() then decode_attn()."""
        _check_input(k_new)
        _check_input(v_new)
        _check_input(q)
        if k_new.dim() != 3 or v_new.shape != k_new.shape:
            raise ValueError("k_new, v_new must be [B, Hkv, d] (one token per sequence)")
        B, Hq, d = q.shape
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        scale = 1.0 / (d ** 0.5) if sm_scale is None else sm_scale
        _check(lib().gear_append_decode_attn(self._h, _ptr(k_new), _ptr(v_new), _ptr(q), Hq,
                                             ctypes.c_float(scale), _ptr(out), _ptr(self.workspace),
                                             self.workspace.numel(), _stream()))
        return out

    def info(self) -> _CacheInfo:
        inf = _CacheInfo()
        _check(lib().gear_cache_get_info(self._h, ctypes.byref(inf)))
        return inf

    def _view(self, ptr: int, nbytes: int) -> torch.Tensor:
        off = ptr - self.arena.data_ptr()
        return self.arena[off:off + nbytes]

    def prompt_packed(self) -> Packed:
        c = self.cfg
        M = 2 * c.batch * c.kv_heads
        L = packed_layout(self.prompt_params, M, c.prompt_tokens, c.head_dim, ROLE_KEYS_THEN_VALUES)
        return Packed(self._view(self.info().prompt_packed, L.total_bytes), self.prompt_params, M,
                      c.prompt_tokens, c.head_dim, L, ROLE_KEYS_THEN_VALUES)

    def fill_packed(self, f: int) -> Packed:
        c, inf = self.cfg, self.info()
        M = 2 * c.batch * c.kv_heads
        fp = Params(**{**self.fill_params.__dict__, "chunk_tokens": 0})
        L = packed_layout(fp, M, c.buf_tokens, c.head_dim, ROLE_KEYS_THEN_VALUES)
        return Packed(self._view(inf.fill_packed + f * inf.fill_stride, L.total_bytes), fp, M,
                      c.buf_tokens, c.head_dim, L, ROLE_KEYS_THEN_VALUES)
