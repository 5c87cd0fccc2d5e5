"""Host logic of per-request residency: pipeline.ResidencyTracker against the oracle's
reclaimable_pages / is_fully_resident on random tables, and its per-row inputs."""

import numpy as np

import oracle
from sparse_attention_kv_amd.pipeline import ResidencyTracker


def test_tracker_matches_oracle_through_releases():
    rng = np.random.default_rng(6)
    for trial in range(20):
        B, W, bs = 7, 12, 16
        seq = rng.integers(1, W * bs + 1, size=B)
        bt = rng.permutation(B * W).reshape(B, W).astype(np.int32)
        bt[rng.random((B, W)) < 0.1] = -1
        t = ResidencyTracker(bt, seq, bs)
        for _ in range(4):
            assert t.reclaimable_pages() == oracle.reclaimable_pages(t.block_table, seq, bs)
            assert np.array_equal(t.fully_resident(), oracle.is_fully_resident(t.block_table, seq, bs))
            pages = t.reclaimable_pages()
            if not pages:
                break
            b, p = pages[rng.integers(len(pages))]
            blk = int(t.block_table[b, p])
            t.release_resident_page(b, p)
            assert t.block_table[b, p] == -1 and t.free_blocks[-1] == blk


def test_row_inputs_split_rows_by_their_request():
    bt = np.array([[0, 1], [2, -1], [4, 5]], dtype=np.int32)
    t = ResidencyTracker(bt, np.array([20, 20, 20]), 16)   # request 1 lost page 1
    req = np.array([0, 1, 2, 0, 1, 2, -1])
    a, b, sel = (x.numpy() for x in t.row_inputs(req, "cpu"))
    assert a.tolist() == [0, -1, 2, 0, -1, 2, -1]
    assert b.tolist() == [-1, 1, -1, -1, 1, -1, -1]
    assert sel.tolist() == [0, 1, 0, 0, 1, 0, 1]


def test_reclaim_matches_oracle_selection_and_releases():
    """ResidencyTracker.reclaim picks the oracle's pages (P3 reclaim_resident_blocks reading)
    and releases exactly those; requests that gave pages stop being fully resident."""
    rng = np.random.default_rng(17)
    for trial in range(30):
        B, W, bs = 7, 12, 16
        seq = rng.integers(1, W * bs + 1, size=B)
        bt = rng.permutation(B * W).reshape(B, W).astype(np.int32)
        t = ResidencyTracker(bt, seq, bs)
        for _ in range(3):
            prio = rng.integers(0, 4, size=B)
            hot = rng.random((B, W)) < 0.25
            d = int(rng.integers(0, 9))
            want = oracle.select_reclaim_pages(t.block_table, seq, bs, d, prio, hot)
            before = t.block_table.copy()
            got = t.reclaim(d, prio, hot)
            assert got == want
            for b, p in got:
                assert t.block_table[b, p] == -1 and before[b, p] in t.free_blocks
            changed = np.argwhere(t.block_table != before)
            assert sorted(map(tuple, changed.tolist())) == sorted(got)
            assert np.array_equal(t.fully_resident(), oracle.is_fully_resident(t.block_table, seq, bs))
