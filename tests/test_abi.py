"""The C ABI without a GPU: the library loads, exports every function that
include/nosa.h declares, and rejects bad arguments on the host before anything
is enqueued (so none of these calls launches a kernel)."""
import ctypes
import os

import pytest

from block_sparse_attention_nosa_amd import nosa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nosa.LIB_PATH):
        from block_sparse_attention_nosa_amd import build
        build.build()
    return nosa.lib()


def test_exports_every_declared_function(L):
    names = nosa.header_functions()
    assert set(names) >= {"nosa_abi_version", "nosa_status_string", "nosa_workspace_size",
                          "nosa_compress_keys", "nosa_block_scores", "nosa_select_blocks",
                          "nosa_sparse_attend", "nosa_decode_step", "nosa_prefill_sparse",
                          "nosa_prefill_sparse_workspace_size", "nosa_offload_decode_step",
                          "nosa_offload_workspace_size", "nosa_pack_qkv_weights",
                          "nosa_qkv_rope_append", "nosa_layer_decode_step",
                          "nosa_decode_step_static"}
    for n in names:
        assert hasattr(L, n), n


def test_timeline_build_is_a_library_of_its_own(L):
    """The stamped build of the decode kernels exports the ABI and its
    readout; the library itself has no readout."""
    from block_sparse_attention_nosa_amd import build
    if not os.path.exists(build.TIMELINE_LIB):
        build.build()
    T = ctypes.CDLL(build.TIMELINE_LIB)
    for n in ("nosa_timeline_read", "nosa_timeline_clear", "nosa_timeline_clock_khz"):
        assert hasattr(T, n), n
        assert not hasattr(L, n), n
    for n in nosa.header_functions():
        assert hasattr(T, n), n


def test_version_and_status_strings(L):
    assert nosa.abi_version() == 5
    for s in range(6):
        assert nosa.status_string(s)
    assert nosa.status_string(0) == "ok"
    assert nosa.status_string(99) == "unknown status"


def test_header_is_plain_c():
    """Signatures use only C scalar types, plain pointers and the header's own
    structs: no torch, HIP or C++ types cross the boundary."""
    import re
    txt = open(os.path.join(ROOT, "include", "nosa.h")).read()
    code = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    for bad in ("torch", "at::", "Tensor", "hipStream_t", "std::", "template", "&"):
        assert bad not in code, bad


def _ws(p, B, q, k):
    return nosa.nosa_workspace_size(p, B, q, k)


def test_workspace_size_for_the_workloads(L):
    assert _ws(nosa.params(topk=16), 1, 1, 4096) > 0
    assert _ws(nosa.params(topk=64), 8, 1, 16640) > 0
    assert _ws(nosa.params(topk=64), 32, 1, 32768) > 0
    assert _ws(nosa.params(num_q_heads=32, num_kv_heads=8, topk=96), 16, 1, 65536) > 0
    # monotone in the batch and the length
    p = nosa.params()
    assert _ws(p, 8, 1, 16384) <= _ws(p, 16, 1, 16384) <= _ws(p, 16, 1, 32768)
    assert _ws(p, 0, 0, 0) >= 0


@pytest.mark.parametrize("field,value,status", [
    ("num_q_heads", 0, 2), ("num_kv_heads", 3, 2), ("window", 1000, 2),
    ("topk", -1, 2), ("head_dim", 64, 3), ("block_size", 32, 3), ("kernel", 16, 3),
    ("stride", 8, 3), ("block_size", 48, 2), ("locality", -0.1, 2), ("locality", 1.5, 2),
    ("locality", float("nan"), 2)])
def test_parameter_errors(L, field, value, status):
    p = nosa.params()
    setattr(p, field, value)
    with pytest.raises(nosa.NosaError) as e:
        nosa.nosa_workspace_size(p, 8, 1, 16384)
    assert e.value.status == status


def test_locality_window_limit(L):
    # window 8192 tokens (128 blocks) leaves no room for local blocks
    p = nosa.params(window=8192, topk=64, locality=0.5)
    with pytest.raises(nosa.NosaError) as e:
        nosa.nosa_workspace_size(p, 1, 1, 16384)
    assert e.value.status == 3
    assert nosa.nosa_workspace_size(nosa.params(window=1024, topk=64, locality=0.75), 8, 1, 16640) > 0


def test_group_too_large_is_unsupported(L):
    p = nosa.params(num_q_heads=32, num_kv_heads=1)
    with pytest.raises(nosa.NosaError) as e:
        nosa.nosa_workspace_size(p, 1, 1, 4096)
    assert e.value.status == 3


def test_null_and_size_errors(L):
    f = L.nosa_workspace_size
    out = ctypes.c_size_t()
    assert f(None, 1, 1, 4096, ctypes.byref(out)) == 1
    p = nosa.params()
    assert f(ctypes.byref(p), 1, 1, 4096, None) == 1
    assert f(ctypes.byref(p), -1, 1, 4096, ctypes.byref(out)) == 2
    assert f(ctypes.byref(p), 1, 1, 0, ctypes.byref(out)) == 2
    assert f(ctypes.byref(p), 1, 1, 8192 * 64 + 1, ctypes.byref(out)) == 3
    assert f(ctypes.byref(p), 1, 64, 4096, ctypes.byref(out)) == 0   # a 64-query chunk
    assert out.value > 0
    assert f(ctypes.byref(p), 1, 8192, 4096, ctypes.byref(out)) == 2  # more queries than keys


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _kv(max_blocks=256, pages=16):
    return nosa.nosa_paged_kv(FAKE, FAKE, FAKE, FAKE, max_blocks, pages)


def test_decode_step_host_errors(L):
    p = nosa.params()
    kv = _kv()
    call = lambda **kw: L.nosa_decode_step(
        ctypes.byref(kw.get("p", p)), ctypes.byref(kw.get("kv", kv)) if kw.get("kv", kv) else None,
        kw.get("q", FAKE), kw.get("cu", FAKE), kw.get("B", 8), kw.get("Lk", 16384),
        kw.get("out", FAKE), None, kw.get("sel", None), kw.get("cnt", None), None,
        kw.get("ws", FAKE), kw.get("wsb", 0), None)
    assert call(q=None) == 1
    assert call(out=None) == 1
    assert call(cu=None) == 1
    assert call(kv=None) == 1
    assert call(sel=FAKE) == 1                     # sel without count
    assert call(kv=_kv(max_blocks=100)) == 2       # table cannot reach max_seqlen_k
    assert call(kv=_kv(pages=0)) == 2
    assert call(ws=None, wsb=1 << 40) == 4
    assert call(wsb=100) == 4                      # too small
    assert call(B=0) == 0                          # empty batch: nothing to do
    bad = nosa.params(window=100)
    assert call(p=bad) == 2


def test_decode_step_static_host_errors(L):
    """The entry point without a workspace: the same argument checks, and a
    step whose partials would not fit the static scratch array is rejected
    with NOSA_ERR_WORKSPACE before anything is enqueued."""
    p = nosa.params()
    call = lambda **kw: L.nosa_decode_step_static(
        ctypes.byref(kw.get("p", p)), ctypes.byref(kw.get("kv", _kv(max_blocks=kw.get("mb", 256)))),
        kw.get("q", FAKE), kw.get("cu", FAKE), kw.get("B", 8), kw.get("Lk", 16384),
        kw.get("out", FAKE), None, kw.get("sel", None), kw.get("cnt", None), None, None)
    assert call(q=None) == 1
    assert call(out=None) == 1
    assert call(sel=FAKE) == 1
    assert call(mb=100) == 2
    assert call(B=0) == 0
    assert call(p=nosa.params(window=100)) == 2
    # the largest step that fits and the first that does not
    need = lambda B: nosa.nosa_workspace_size(p, B, 1, 16384)
    B = 8
    while need(B * 2) <= nosa.STATIC_SCRATCH_BYTES:
        B *= 2
    assert need(B) <= nosa.STATIC_SCRATCH_BYTES < need(B * 2)
    assert call(B=B * 2) == 4
    assert call(B=4096, Lk=65536, mb=1024) == 4
    import re
    m = re.search(r"#define NOSA_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)",
                  open(os.path.join(ROOT, "include", "nosa.h")).read())
    assert int(m.group(1)) << int(m.group(2)) == nosa.STATIC_SCRATCH_BYTES


def test_other_entry_points_host_errors(L):
    p = nosa.params()
    kv = _kv()
    assert L.nosa_compress_keys(ctypes.byref(p), ctypes.byref(kv), None, None, 8, 16384,
                                None) == 1
    assert L.nosa_compress_keys(ctypes.byref(p), None, FAKE, None, 8, 16384, None) == 1
    assert L.nosa_compress_keys(ctypes.byref(p), ctypes.byref(kv), FAKE, None, 0, 16384,
                                None) == 0
    assert L.nosa_block_scores(ctypes.byref(p), ctypes.byref(kv), FAKE, None, FAKE, 8, 1, 16384,
                               None, FAKE, 1 << 30, None) == 1
    assert L.nosa_block_scores(ctypes.byref(p), ctypes.byref(kv), FAKE, FAKE, FAKE, 8, 64, 16384,
                               FAKE, FAKE, 16, None) == 4             # chunk: workspace too small
    assert L.nosa_block_scores(ctypes.byref(p), ctypes.byref(kv), FAKE, None, FAKE, 8, 64, 16384,
                               FAKE, FAKE, 1 << 30, None) == 2        # 64 queries need cu_seqlens_q
    assert L.nosa_block_scores(ctypes.byref(p), ctypes.byref(kv), FAKE, None, FAKE, 8, 1, 16384,
                               FAKE, FAKE, 16, None) == 4
    assert L.nosa_select_blocks(ctypes.byref(p), None, None, FAKE, 8, 1, 16384, FAKE, FAKE,
                                None) == 1
    assert L.nosa_sparse_attend(ctypes.byref(p), ctypes.byref(kv), FAKE, None, FAKE, 8, 1, 16384,
                                FAKE, FAKE, FAKE, None, FAKE, 8, None) == 4
    assert L.nosa_sparse_attend(ctypes.byref(p), ctypes.byref(kv), FAKE, None, FAKE, 8, 1, 16384,
                                None, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1


def test_prompt_prefill_host_errors(L):
    p = nosa.params()
    kv = _kv()
    size = lambda ch, B=2, Lm=5000: nosa.nosa_prefill_sparse_workspace_size(p, B, Lm, ch)
    assert size(512) > 0
    assert size(8192) == size(5056)                # capped by the longest prompt (whole blocks)
    for bad in (0, -64, 100):
        with pytest.raises(nosa.NosaError) as e:
            size(bad)
        assert e.value.status == 2
    call = lambda **kw: L.nosa_prefill_sparse(
        ctypes.byref(p), ctypes.byref(kv), kw.get("q", FAKE), kw.get("cu", FAKE), kw.get("B", 2),
        kw.get("Lm", 5000), kw.get("ch", 512), kw.get("out", FAKE), None, kw.get("ws", FAKE),
        kw.get("wsb", 0), None)
    assert call(q=None) == 1
    assert call(cu=None) == 1
    assert call(out=None) == 1
    assert call(ch=96) == 2
    assert call(Lm=16385) == 2                     # the table cannot reach it
    assert call(wsb=100) == 4
    assert call(B=0) == 0


def test_offload_host_errors(L):
    p = nosa.params(topk=64)
    size = lambda cap, **kw: nosa.nosa_offload_workspace_size(kw.get("p", p), 8, 16640, cap)
    assert size(64) > nosa.nosa_workspace_size(p, 8, 1, 16640)
    assert size(128) > size(64)
    for cap, status in ((63, 2), (0, 2), (257, 3)):
        with pytest.raises(nosa.NosaError) as e:
            size(cap)
        assert e.value.status == status
    with pytest.raises(nosa.NosaError) as e:      # a window of no block
        size(64, p=nosa.params(topk=64, window=0))
    assert e.value.status == 3
    loc = nosa.params(topk=64, locality=0.5)      # the local half needs no cache slot
    assert nosa.nosa_offload_workspace_size(loc, 8, 16640, 32) > 0
    okv = nosa.nosa_offload_kv(FAKE, FAKE, FAKE, FAKE, 512, 16, FAKE, FAKE, 16, 64, FAKE, FAKE,
                               FAKE, FAKE)
    call = lambda o, **kw: L.nosa_offload_decode_step(
        ctypes.byref(kw.get("p", p)), ctypes.byref(o) if o is not None else None, FAKE, FAKE,
        kw.get("B", 8), 16640, FAKE, None, None, None, None, FAKE, kw.get("wsb", 0), None)
    assert call(None) == 1
    for f in ("k_host", "v_host", "kc_pool", "block_table", "k_recent", "v_recent", "cache_k",
              "cache_v", "cache_map", "cache_used"):
        bad = nosa.nosa_offload_kv(*[getattr(okv, n) for n, _ in okv._fields_])
        setattr(bad, f, None)
        assert call(bad) == 1, f
    small = nosa.nosa_offload_kv(*[getattr(okv, n) for n, _ in okv._fields_])
    small.recent_blocks = 15                      # the 16 window blocks do not fit
    assert call(small) == 2
    small.recent_blocks = 16
    small.cache_blocks = 60                       # fewer slots than picks
    assert call(small) == 2
    assert call(okv, wsb=100) == 4
    assert call(okv, B=0) == 0


def test_front_host_errors(L):
    p = nosa.params()
    kv = _kv()
    f = nosa.front_params(2048)
    assert L.nosa_pack_qkv_weights(ctypes.byref(p), 2048, None, FAKE, None) == 1
    assert L.nosa_pack_qkv_weights(ctypes.byref(p), 100, FAKE, FAKE, None) == 2
    assert L.nosa_pack_qkv_weights(ctypes.byref(nosa.params(head_dim=64)), 2048, FAKE, FAKE,
                                   None) == 3
    call = lambda **kw: L.nosa_qkv_rope_append(
        ctypes.byref(p), ctypes.byref(kw.get("f", f)) if kw.get("f", f) else None,
        ctypes.byref(kv), kw.get("x", FAKE), FAKE, FAKE, kw.get("B", 8), 16384,
        kw.get("q", FAKE), None)
    assert call(f=None) == 1
    assert call(x=None) == 1
    assert call(q=None) == 1
    assert call(f=nosa.front_params(1000)) == 2
    assert call(f=nosa.front_params(0)) == 2
    assert call(B=0) == 0
    step = lambda **kw: L.nosa_layer_decode_step(
        ctypes.byref(p), ctypes.byref(f), ctypes.byref(kv), FAKE, FAKE, FAKE, 8, 16384, FAKE,
        kw.get("out", FAKE), None, kw.get("sel", None), None, FAKE, kw.get("wsb", 0), None)
    assert step(out=None) == 1
    assert step(sel=FAKE) == 1
    assert step(wsb=100) == 4
