"""Host-side checks of the stored page orders (no GPU): each is a bijection
onto the logical page, and the 1 KB runs hold what one matrix-core step of
a wave loads."""
import torch

from block_sparse_attention_nosa_amd import synth


def test_page_index_is_a_permutation():
    for kind, n in (("k", 64 * 128), ("v", 64 * 128), ("kc", 4 * 128)):
        idx = synth.page_index(kind)
        assert idx.numel() == n
        assert torch.equal(torch.sort(idx).values, torch.arange(n)), kind


def test_k_runs_cover_token_groups_and_channel_steps():
    # run (t, st) holds 16 tokens x 32 channels: the tokens of tile t and the
    # channels of k-step st, each token with channels 32st .. 32st + 31
    idx = synth.page_index("k").view(16, 64, 8)
    for t in range(4):
        for st in range(4):
            run = idx[4 * t + st]
            tok, ch = run // 128, run % 128
            assert set(ch.flatten().tolist()) == set(range(32 * st, 32 * st + 32))
            toks = sorted(set(tok.flatten().tolist()))
            # tiles 2v and 2v + 1 together cover the 32 tokens of k-step v
            assert len(toks) == 16 and all(32 * (t // 2) <= x < 32 * (t // 2) + 32 for x in toks)


def test_v_runs_are_channel_tile_by_token_half():
    idx = synth.page_index("v").view(16, 64, 8)
    for u in range(2):
        for nt in range(8):
            run = idx[8 * u + nt]
            tok, ch = run // 128, run % 128
            assert set(ch.flatten().tolist()) == set(range(16 * nt, 16 * nt + 16))
            assert set(tok.flatten().tolist()) == set(range(32 * u, 32 * u + 32))
            # 8 consecutive elements are 8 consecutive tokens of one channel
            assert torch.equal(tok[:, 1:] - tok[:, :-1], torch.ones(64, 7, dtype=tok.dtype))


def test_kc_order_is_chunk_major():
    idx = synth.page_index("kc")
    slot, ch = idx // 128, idx % 128
    assert torch.equal(slot.view(16, 4, 8)[0, :, 0], torch.arange(4))
    assert torch.equal(ch.view(16, 4, 8)[:, 0, 0], torch.arange(0, 128, 8))
