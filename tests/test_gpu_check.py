"""GPU test of nosa_check_inputs: the device-side checks of the inputs the
other entry points take on trust (monotone cu_seqlens, lengths within their
host bounds, block-table entries of the blocks in use inside the pool).
Valid decode and prefill batches give 0; each planted violation sets its own
bit and no other; table entries past a sequence's blocks are not checked.
The planted values are only ever read by the checker (it reads the length
arrays and the table entries of the blocks it checks, never a page)."""
import pytest
import torch

from block_sparse_attention_nosa_amd import nosa

from helpers import log

CU_K, LEN_K, TABLE, CU_Q = 1, 2, 4, 8
MAX_BLOCKS, NUM_PAGES = 64, 512


def _run(lens_cu_k, table, max_seqlen_k, cu_q=None, max_seqlen_q=1):
    p = nosa.params()
    B = len(lens_cu_k) - 1
    tb = torch.as_tensor(table, dtype=torch.int32, device="cuda")
    kv = nosa.paged_kv(None, None, None, tb, num_pages=NUM_PAGES)
    cu_k = torch.as_tensor(lens_cu_k, dtype=torch.int32, device="cuda")
    cq = None if cu_q is None else torch.as_tensor(cu_q, dtype=torch.int32, device="cuda")
    flags = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    nosa.nosa_check_inputs(p, kv, cq, cu_k, B, max_seqlen_q, max_seqlen_k, flags)
    torch.cuda.synchronize()
    return int(flags.item())


def _table(B, fill=None):
    t = [[(s * MAX_BLOCKS + b) % NUM_PAGES for b in range(MAX_BLOCKS)] for s in range(B)]
    return t if fill is None else [[fill] * MAX_BLOCKS for _ in range(B)]


def _cu(lens):
    out = [0]
    for L in lens:
        out.append(out[-1] + L)
    return out


@pytest.mark.gpu
def test_check_inputs_valid_batches():
    log("case: nosa_check_inputs on valid batches")
    lens = [4096, 1, 64, 65, 3000]
    assert _run(_cu(lens), _table(5), 4096) == 0
    # a prefill chunk: the last Lq_s positions of each context
    assert _run(_cu(lens), _table(5), 4096, cu_q=_cu([64, 1, 64, 0, 2048]), max_seqlen_q=2048) == 0
    # entries past a sequence's blocks may hold anything
    t = _table(5)
    t[1][5] = -3
    t[2][1] = NUM_PAGES + 7
    assert _run(_cu(lens), t, 4096) == 0


@pytest.mark.gpu
def test_check_inputs_each_violation_sets_its_bit():
    log("case: nosa_check_inputs planted violations")
    lens = [1000, 2000, 500]
    cu = _cu(lens)
    # cu_seqlens_k not starting at 0 (lengths themselves fine)
    assert _run([5] + [c + 5 for c in cu[1:]], _table(3), 2048) == CU_K
    # a decreasing entry: the negative length is also out of range
    bad = list(cu)
    bad[2] = bad[1] - 10
    assert _run(bad, _table(3), 2048) & CU_K
    # a length above max_seqlen_k, or zero
    assert _run(cu, _table(3), 1500) == LEN_K
    assert _run(_cu([1000, 0, 500]), _table(3), 2048) == LEN_K
    # a table entry of a block in use outside the pool: negative, or num_pages
    for v in (-1, NUM_PAGES):
        t = _table(3)
        t[1][31] = v  # block 31 holds tokens 1984 .. 1999 of the 2000-token sequence
        assert _run(cu, t, 2048) == TABLE, v
    # the same entry one block past the sequence is not checked
    t = _table(3)
    t[1][32] = -1
    assert _run(cu, t, 2048) == 0
    # cu_seqlens_q: not starting at 0, decreasing, a chunk longer than its
    # context or than max_seqlen_q
    assert _run(cu, _table(3), 2048, cu_q=[1, 65, 129, 193], max_seqlen_q=64) == CU_Q
    assert _run(cu, _table(3), 2048, cu_q=[0, 64, 32, 96], max_seqlen_q=64) == CU_Q
    assert _run(cu, _table(3), 2048, cu_q=_cu([64, 64, 501]), max_seqlen_q=512) == CU_Q
    assert _run(cu, _table(3), 2048, cu_q=_cu([64, 128, 64]), max_seqlen_q=64) == CU_Q
    # several at once
    t = _table(3)
    t[0][0] = NUM_PAGES + 1
    assert _run(cu, t, 1500, cu_q=_cu([64, 64, 600]), max_seqlen_q=512) == LEN_K | TABLE | CU_Q


@pytest.mark.gpu
def test_check_inputs_empty_batch_clears_flags():
    log("case: nosa_check_inputs, batch 0")
    assert _run([0], [[0] * MAX_BLOCKS], 64) == 0
