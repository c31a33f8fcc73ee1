"""Thin Python binding of libnosa.so (the C ABI in include/nosa.h).

Argument marshalling only: every function takes torch tensors (device memory,
allocated by the caller), passes their pointers to the entry point of the same
name and raises NosaError on a non-zero status.  Nothing here computes any
part of the method, and there is no fallback: if the HIP library is not built
the import of the library fails loudly.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnosa.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "nosa.h")

STATUS = {0: "NOSA_OK", 1: "NOSA_ERR_NULL", 2: "NOSA_ERR_INVALID", 3: "NOSA_ERR_UNSUPPORTED",
          4: "NOSA_ERR_WORKSPACE", 5: "NOSA_ERR_HIP"}


class NosaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


class nosa_params(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("kernel", ctypes.c_int32), ("stride", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("window", ctypes.c_int32), ("scale", ctypes.c_float),
                ("locality", ctypes.c_float)]


class nosa_paged_kv(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("kc_pool", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("max_blocks_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


class nosa_offload_kv(ctypes.Structure):
    _fields_ = [("k_host", ctypes.c_void_p), ("v_host", ctypes.c_void_p),
                ("kc_pool", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("max_blocks_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("k_recent", ctypes.c_void_p), ("v_recent", ctypes.c_void_p),
                ("recent_blocks", ctypes.c_int32), ("cache_blocks", ctypes.c_int32),
                ("cache_k", ctypes.c_void_p), ("cache_v", ctypes.c_void_p),
                ("cache_map", ctypes.c_void_p), ("cache_used", ctypes.c_void_p)]


class nosa_front_params(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("inv_freq", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_sparse_attention_nosa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P, KV = ctypes.POINTER(nosa_params), ctypes.POINTER(nosa_paged_kv)
        L.nosa_abi_version.restype = ctypes.c_int
        L.nosa_abi_version.argtypes = []
        L.nosa_status_string.restype = ctypes.c_char_p
        L.nosa_status_string.argtypes = [ctypes.c_int]
        sigs = {
            "nosa_workspace_size": [P, i32, i32, i32, ctypes.POINTER(sz)],
            "nosa_compress_keys": [P, KV, vp, vp, i32, i32, vp],
            "nosa_block_scores": [P, KV, vp, vp, vp, i32, i32, i32, vp, vp, sz, vp],
            "nosa_select_blocks": [P, vp, vp, vp, i32, i32, i32, vp, vp, vp],
            "nosa_sparse_attend": [P, KV, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp],
            "nosa_decode_step": [P, KV, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp],
            "nosa_decode_step_static": [P, KV, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp],
            "nosa_prefill_sparse_workspace_size": [P, i32, i32, i32, ctypes.POINTER(sz)],
            "nosa_prefill_sparse": [P, KV, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp],
            "nosa_offload_workspace_size": [P, i32, i32, i32, ctypes.POINTER(sz)],
            "nosa_pack_qkv_weights": [P, i32, vp, vp, vp],
            "nosa_qkv_rope_append": [P, ctypes.POINTER(nosa_front_params), KV, vp, vp, vp, i32,
                                     i32, vp, vp],
            "nosa_layer_decode_step": [P, ctypes.POINTER(nosa_front_params), KV, vp, vp, vp, i32,
                                       i32, vp, vp, vp, vp, vp, vp, sz, vp],
            "nosa_offload_decode_step": [P, ctypes.POINTER(nosa_offload_kv), vp, vp, i32, i32, vp,
                                         vp, vp, vp, vp, vp, sz, vp],
            "nosa_check_inputs": [P, KV, vp, vp, i32, i32, i32, vp, vp],
        }
        for name, argtypes in sigs.items():
            f = getattr(L, name)
            f.argtypes = argtypes
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions declared in include/nosa.h."""
    txt = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^(?:nosa_status|int|const char\*)\s+(nosa_\w+)\s*\(", txt,
                                 flags=re.M)))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != 0:
        raise NosaError(fn, status, lib().nosa_status_string(status).decode())


def params(num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=64, kernel=32, stride=16,
           topk=64, window=1024, scale=0.0, locality=0.0) -> nosa_params:
    return nosa_params(num_q_heads, num_kv_heads, head_dim, block_size, kernel, stride, topk,
                       window, scale, locality)


def paged_kv(k_pool, v_pool, kc_pool, block_table, max_blocks_per_seq=None,
             num_pages=None) -> nosa_paged_kv:
    """Struct over the paged pools (the tensors must outlive every call using it)."""
    if max_blocks_per_seq is None:
        max_blocks_per_seq = block_table.shape[1]
    if num_pages is None:
        num_pages = k_pool.shape[0]
    return nosa_paged_kv(_ptr(k_pool), _ptr(v_pool), _ptr(kc_pool), _ptr(block_table),
                         int(max_blocks_per_seq), int(num_pages))


def abi_version() -> int:
    return int(lib().nosa_abi_version())


def status_string(status: int) -> str:
    return lib().nosa_status_string(int(status)).decode()


def nosa_workspace_size(p: nosa_params, batch: int, max_seqlen_q: int, max_seqlen_k: int) -> int:
    out = ctypes.c_size_t(0)
    _check("nosa_workspace_size", lib().nosa_workspace_size(
        ctypes.byref(p), batch, max_seqlen_q, max_seqlen_k, ctypes.byref(out)))
    return int(out.value)


def nosa_compress_keys(p, kv, cu_seqlens_k, kc_valid_len, batch, max_seqlen_k, stream=None):
    _check("nosa_compress_keys", lib().nosa_compress_keys(
        ctypes.byref(p), ctypes.byref(kv), _ptr(cu_seqlens_k), _ptr(kc_valid_len), batch,
        max_seqlen_k, _stream(stream)))


def nosa_block_scores(p, kv, q, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k,
                      block_scores, workspace, stream=None):
    _check("nosa_block_scores", lib().nosa_block_scores(
        ctypes.byref(p), ctypes.byref(kv), _ptr(q), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
        batch, max_seqlen_q, max_seqlen_k, _ptr(block_scores), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream)))


def nosa_select_blocks(p, block_scores, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q,
                       max_seqlen_k, sel_idx, sel_count, stream=None):
    _check("nosa_select_blocks", lib().nosa_select_blocks(
        ctypes.byref(p), _ptr(block_scores), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch,
        max_seqlen_q, max_seqlen_k, _ptr(sel_idx), _ptr(sel_count), _stream(stream)))


def nosa_check_inputs(p, kv, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k,
                      flags, stream=None):
    _check("nosa_check_inputs", lib().nosa_check_inputs(
        ctypes.byref(p), ctypes.byref(kv), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch,
        max_seqlen_q, max_seqlen_k, _ptr(flags), _stream(stream)))


def nosa_sparse_attend(p, kv, q, cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k,
                       sel_idx, sel_count, out, lse, workspace, stream=None):
    _check("nosa_sparse_attend", lib().nosa_sparse_attend(
        ctypes.byref(p), ctypes.byref(kv), _ptr(q), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
        batch, max_seqlen_q, max_seqlen_k, _ptr(sel_idx), _ptr(sel_count), _ptr(out), _ptr(lse),
        _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream)))


def nosa_decode_step(p, kv, q, cu_seqlens_k, batch, max_seqlen_k, out, lse, workspace,
                     sel_idx=None, sel_count=None, block_scores=None, stream=None):
    _check("nosa_decode_step", lib().nosa_decode_step(
        ctypes.byref(p), ctypes.byref(kv), _ptr(q), _ptr(cu_seqlens_k), batch, max_seqlen_k,
        _ptr(out), _ptr(lse), _ptr(sel_idx), _ptr(sel_count), _ptr(block_scores),
        _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream)))


STATIC_SCRATCH_BYTES = 32 << 20  # NOSA_STATIC_SCRATCH_BYTES


def nosa_decode_step_static(p, kv, q, cu_seqlens_k, batch, max_seqlen_k, out, lse, sel_idx=None,
                            sel_count=None, block_scores=None, stream=None):
    _check("nosa_decode_step_static", lib().nosa_decode_step_static(
        ctypes.byref(p), ctypes.byref(kv), _ptr(q), _ptr(cu_seqlens_k), batch, max_seqlen_k,
        _ptr(out), _ptr(lse), _ptr(sel_idx), _ptr(sel_count), _ptr(block_scores),
        _stream(stream)))


def nosa_prefill_sparse_workspace_size(p: nosa_params, batch: int, max_seqlen: int,
                                       chunk: int) -> int:
    out = ctypes.c_size_t(0)
    _check("nosa_prefill_sparse_workspace_size", lib().nosa_prefill_sparse_workspace_size(
        ctypes.byref(p), batch, max_seqlen, chunk, ctypes.byref(out)))
    return int(out.value)


def nosa_prefill_sparse(p, kv, q, cu_seqlens, batch, max_seqlen, chunk, out, lse, workspace,
                        stream=None):
    _check("nosa_prefill_sparse", lib().nosa_prefill_sparse(
        ctypes.byref(p), ctypes.byref(kv), _ptr(q), _ptr(cu_seqlens), batch, max_seqlen, chunk,
        _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream)))


def offload_kv(k_host, v_host, kc_pool, block_table, k_recent, v_recent, cache_k, cache_v,
               cache_map, cache_used, max_blocks_per_seq=None, num_pages=None) -> nosa_offload_kv:
    """Struct over an offloaded KV cache (the tensors must outlive every call
    using it).  k_host / v_host: pinned CPU tensors [pages][Hkv][64 * 128];
    k_recent / v_recent: [batch][recent][Hkv][64 * 128]; cache_k / cache_v:
    [batch][Hkv][slots][64 * 128]; cache_map, cache_used: int32
    [batch][Hkv][slots]."""
    if max_blocks_per_seq is None:
        max_blocks_per_seq = block_table.shape[1]
    if num_pages is None:
        num_pages = k_host.shape[0]
    return nosa_offload_kv(_ptr(k_host), _ptr(v_host), _ptr(kc_pool), _ptr(block_table),
                           int(max_blocks_per_seq), int(num_pages), _ptr(k_recent),
                           _ptr(v_recent), int(k_recent.shape[1]), int(cache_map.shape[-1]),
                           _ptr(cache_k), _ptr(cache_v), _ptr(cache_map), _ptr(cache_used))


def nosa_offload_workspace_size(p: nosa_params, batch: int, max_seqlen_k: int,
                                cache_blocks: int) -> int:
    out = ctypes.c_size_t(0)
    _check("nosa_offload_workspace_size", lib().nosa_offload_workspace_size(
        ctypes.byref(p), batch, max_seqlen_k, cache_blocks, ctypes.byref(out)))
    return int(out.value)


def nosa_offload_decode_step(p, okv, q, cu_seqlens_k, batch, max_seqlen_k, out, lse, workspace,
                             sel_idx=None, sel_count=None, fetch_count=None, stream=None):
    _check("nosa_offload_decode_step", lib().nosa_offload_decode_step(
        ctypes.byref(p), ctypes.byref(okv), _ptr(q), _ptr(cu_seqlens_k), batch, max_seqlen_k,
        _ptr(out), _ptr(lse), _ptr(sel_idx), _ptr(sel_count), _ptr(fetch_count), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream)))


def front_params(hidden: int, rope_theta: float = 10000.0, inv_freq=None) -> nosa_front_params:
    """Front-end parameters (inv_freq: optional device float32 tensor [64])."""
    return nosa_front_params(int(hidden), float(rope_theta), _ptr(inv_freq))


def nosa_pack_qkv_weights(p, hidden, w, packed, stream=None):
    _check("nosa_pack_qkv_weights", lib().nosa_pack_qkv_weights(
        ctypes.byref(p), hidden, _ptr(w), _ptr(packed), _stream(stream)))


def nosa_qkv_rope_append(p, front, kv, x, w_packed, cu_seqlens_k, batch, max_seqlen_k, q_out,
                         stream=None):
    _check("nosa_qkv_rope_append", lib().nosa_qkv_rope_append(
        ctypes.byref(p), ctypes.byref(front), ctypes.byref(kv), _ptr(x), _ptr(w_packed),
        _ptr(cu_seqlens_k), batch, max_seqlen_k, _ptr(q_out), _stream(stream)))


def nosa_layer_decode_step(p, front, kv, x, w_packed, cu_seqlens_k, batch, max_seqlen_k, q_out,
                           out, lse, workspace, sel_idx=None, sel_count=None, stream=None):
    _check("nosa_layer_decode_step", lib().nosa_layer_decode_step(
        ctypes.byref(p), ctypes.byref(front), ctypes.byref(kv), _ptr(x), _ptr(w_packed),
        _ptr(cu_seqlens_k), batch, max_seqlen_k, _ptr(q_out), _ptr(out), _ptr(lse), _ptr(sel_idx),
        _ptr(sel_count), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream)))
