"""ctypes wrapper over the plain CPU reference in nosa_oracle.c.

TEST INFRASTRUCTURE ONLY: imported by the test-suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product package.  All arrays
are numpy; bf16 values travel as their uint16 bit patterns.  Layouts are the
ones documented at the top of nosa_oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nosa_oracle.c")
_LIB = os.path.join(_HERE, "libnosa_oracle.so")

GCC_CMD = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-o", _LIB, _SRC, "-lm"]


def build() -> str:
    """Compile the reference with gcc (plain C99 + OpenMP); returns the .so path."""
    subprocess.run(GCC_CMD, check=True, cwd=_HERE)
    return _LIB


class _Params(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int), ("num_kv_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("block_size", ctypes.c_int),
                ("kernel", ctypes.c_int), ("stride", ctypes.c_int), ("topk", ctypes.c_int),
                ("window", ctypes.c_int), ("scale", ctypes.c_double),
                ("locality", ctypes.c_double)]


@dataclass(frozen=True)
class Params:
    num_q_heads: int = 16
    num_kv_heads: int = 2
    head_dim: int = 128
    block_size: int = 64
    kernel: int = 32
    stride: int = 16
    topk: int = 64
    window: int = 1024
    scale: float = 0.0  # <= 0 means 1/sqrt(head_dim)
    locality: float = 0.0  # gamma_0: share of topk given to the blocks nearest the window

    def c(self) -> _Params:
        return _Params(self.num_q_heads, self.num_kv_heads, self.head_dim, self.block_size,
                       self.kernel, self.stride, self.topk, self.window, float(self.scale),
                       float(self.locality))

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def window_blocks(self) -> int:
        return self.window // self.block_size


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.POINTER
        vp = ctypes.c_void_p
        i = ctypes.c_int
        L.nosa_ref_num_keys.argtypes = [i, i, i]
        L.nosa_ref_num_keys.restype = i
        L.nosa_ref_bf16_round.argtypes = [ctypes.c_double]
        L.nosa_ref_bf16_round.restype = ctypes.c_uint16
        L.nosa_ref_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.nosa_ref_bf16_to_double.restype = ctypes.c_double
        L.nosa_ref_num_threads.argtypes = []
        L.nosa_ref_num_threads.restype = i
        L.nosa_ref_check_params.argtypes = [P(_Params)]
        L.nosa_ref_compress_keys.argtypes = [P(_Params), vp, vp, i, i, vp]
        L.nosa_ref_append_keys.argtypes = [P(_Params), vp, vp, vp, i, i, vp]
        L.nosa_ref_set_num_threads.argtypes = [i]
        L.nosa_ref_set_num_threads.restype = None
        L.nosa_ref_block_scores.argtypes = [P(_Params), vp, vp, vp, i, vp, i, i, i, vp]
        L.nosa_ref_select_blocks.argtypes = [P(_Params), vp, vp, vp, i, i, i, i, vp, vp]
        L.nosa_ref_sparse_attend.argtypes = [P(_Params), vp, vp, vp, vp, vp, i, vp, vp, i, i,
                                             vp, vp]
        L.nosa_ref_qkv_rope.argtypes = [P(_Params), i, ctypes.c_double, vp, vp, vp, vp, i, vp,
                                        vp, vp]
        for f in ("nosa_ref_compress_keys", "nosa_ref_append_keys", "nosa_ref_block_scores",
                  "nosa_ref_select_blocks",
                  "nosa_ref_sparse_attend", "nosa_ref_check_params", "nosa_ref_qkv_rope"):
            getattr(L, f).restype = i
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def num_keys(L: int, p: Params) -> int:
    return lib().nosa_ref_num_keys(int(L), p.kernel, p.stride)


def bf16_round(x: float) -> int:
    return int(lib().nosa_ref_bf16_round(float(x)))


def bf16_to_float(bits: int) -> float:
    return float(lib().nosa_ref_bf16_to_double(int(bits)))


def num_threads() -> int:
    return int(lib().nosa_ref_num_threads())


def lengths(cu):
    cu = np.asarray(cu)
    return cu[1:] - cu[:-1]


def shapes(p: Params, cu_k, cu_q=None):
    """(max_nc, max_qblk, max_nb, max_sel) for a batch."""
    Lk = lengths(cu_k)
    Lq = np.ones_like(Lk) if cu_q is None else lengths(cu_q)
    max_nc = max(1, max(num_keys(int(L), p) for L in Lk))
    max_qblk = max(1, int(((Lq + p.block_size - 1) // p.block_size).max()))
    max_nb = max(1, int(((Lk + p.block_size - 1) // p.block_size).max()))
    max_sel = p.topk + p.window_blocks
    return max_nc, max_qblk, max_nb, max_sel


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def qkv_rope(p: Params, x, w, pos, theta=10000.0, inv_freq=None):
    """Front end of one decode token per sequence: (q [B][Hq][d], k and v
    [B][Hkv][d]) as bf16 bits from x [B][hidden] and w [(Hq+2Hkv) d][hidden]
    (bf16 bits) at positions pos [B]."""
    x = _u16(x)
    w = _u16(w)
    pos = _i32(pos)
    B, hidden = x.shape
    d = p.head_dim
    q = np.zeros((B, p.num_q_heads, d), dtype=np.uint16)
    k = np.zeros((B, p.num_kv_heads, d), dtype=np.uint16)
    v = np.zeros((B, p.num_kv_heads, d), dtype=np.uint16)
    f = None if inv_freq is None else np.ascontiguousarray(inv_freq, dtype=np.float64)
    _check(lib().nosa_ref_qkv_rope(ctypes.byref(p.c()), hidden, float(theta),
                                   None if f is None else _ptr(f), _ptr(x), _ptr(w), _ptr(pos), B,
                                   _ptr(q), _ptr(k), _ptr(v)), "qkv_rope")
    return q, k, v


def compress_keys(p: Params, k, cu_k, max_nc=None):
    k = _u16(k)
    cu_k = _i32(cu_k)
    B = len(cu_k) - 1
    if max_nc is None:
        max_nc = shapes(p, cu_k)[0]
    kc = np.zeros((B, p.num_kv_heads, max_nc, p.head_dim), dtype=np.uint16)
    _check(lib().nosa_ref_compress_keys(ctypes.byref(p.c()), _ptr(k), _ptr(cu_k), B, max_nc,
                                        _ptr(kc)), "compress_keys")
    return kc


def set_num_threads(n: int) -> None:
    lib().nosa_ref_set_num_threads(int(n))


def append_keys(p: Params, k, cu_k, valid_len, kc):
    """Pooled keys of a grown cache, in place: for each sequence the keys of
    tokens past valid_len[s] (kc [B][Hkv][max_nc][d] holds the earlier ones)."""
    k = _u16(k)
    cu_k = _i32(cu_k)
    valid_len = _i32(valid_len)
    assert kc.dtype == np.uint16 and kc.flags.c_contiguous
    B = len(cu_k) - 1
    _check(lib().nosa_ref_append_keys(ctypes.byref(p.c()), _ptr(k), _ptr(cu_k), _ptr(valid_len),
                                      B, kc.shape[2], _ptr(kc)), "append_keys")
    return kc


def block_scores(p: Params, q, cu_q, kc, cu_k, max_qblk=None, max_nb=None):
    q = _u16(q)
    kc = _u16(kc)
    cu_k = _i32(cu_k)
    cu_q = _i32(cu_q)
    B = len(cu_k) - 1
    _, mq, mn, _ = shapes(p, cu_k, cu_q)
    max_qblk = max_qblk or mq
    max_nb = max_nb or mn
    scores = np.empty((B, max_qblk, p.num_kv_heads, max_nb), dtype=np.float64)
    _check(lib().nosa_ref_block_scores(ctypes.byref(p.c()), _ptr(q), _ptr(cu_q), _ptr(kc),
                                       kc.shape[2], _ptr(cu_k), B, max_qblk, max_nb,
                                       _ptr(scores)), "block_scores")
    return scores


def select_blocks(p: Params, scores, cu_q, cu_k):
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    cu_k = _i32(cu_k)
    cu_q = _i32(cu_q)
    B, max_qblk, _, max_nb = scores.shape
    max_sel = p.topk + p.window_blocks
    sel = np.empty((B, max_qblk, p.num_kv_heads, max_sel), dtype=np.int32)
    cnt = np.empty((B, max_qblk, p.num_kv_heads), dtype=np.int32)
    _check(lib().nosa_ref_select_blocks(ctypes.byref(p.c()), _ptr(scores), _ptr(cu_q),
                                        _ptr(cu_k), B, max_qblk, max_nb, max_sel, _ptr(sel),
                                        _ptr(cnt)), "select_blocks")
    return sel, cnt


def sparse_attend(p: Params, q, cu_q, k, v, cu_k, sel, cnt):
    q, k, v = _u16(q), _u16(k), _u16(v)
    cu_k = _i32(cu_k)
    cu_q = _i32(cu_q)
    sel = _i32(sel)
    cnt = _i32(cnt)
    B = len(cu_k) - 1
    max_qblk, max_sel = sel.shape[1], sel.shape[3]
    total_q = q.shape[0]
    out = np.empty((total_q, p.num_q_heads, p.head_dim), dtype=np.float64)
    lse = np.empty((total_q, p.num_q_heads), dtype=np.float64)
    _check(lib().nosa_ref_sparse_attend(ctypes.byref(p.c()), _ptr(q), _ptr(cu_q), _ptr(k),
                                        _ptr(v), _ptr(cu_k), B, _ptr(sel), _ptr(cnt), max_qblk,
                                        max_sel, _ptr(out), _ptr(lse)), "sparse_attend")
    return out, lse


def forward(p: Params, q, cu_q, k, v, cu_k):
    """The whole step in the pages' order; returns every intermediate."""
    kc = compress_keys(p, k, cu_k)
    scores = block_scores(p, q, cu_q, kc, cu_k)
    sel, cnt = select_blocks(p, scores, cu_q, cu_k)
    out, lse = sparse_attend(p, q, cu_q, k, v, cu_k, sel, cnt)
    return dict(kc=kc, scores=scores, sel=sel, cnt=cnt, out=out, lse=lse)
