"""Pins of the oracle's per-request residency pieces: mixed-source attention, reclaimable
pages and the fully-resident test.

Mixed attention is checked against single-source attention over the two caches laid end
to end (an independent formulation); the residency rules against a hand-worked example
of the pages' description (P3 reclaim_resident_blocks: never the last two blocks).
"""

import numpy as np

import oracle


def _raw_bf16(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_mixed_equals_attention_over_concatenated_caches():
    rng = np.random.default_rng(2)
    rows, H, D, DV, K = 6, 4, 64, 48, 20
    q = _raw_bf16(rng, (rows, H, D))
    kv_a = _raw_bf16(rng, (50, D))
    kv_b = _raw_bf16(rng, (30, D))
    idx_a = rng.integers(-2, 55, size=(rows, K))   # some past kv_a's end
    idx_b = rng.integers(-2, 35, size=(rows, K))   # some past kv_b's end
    sel = np.array([0, 1, 1, 0, 1, 0])
    out, lse = oracle.sparse_decode_attn_mixed(q, kv_a, idx_a, kv_b, idx_b, sel, 0.125, DV)
    cat = np.concatenate([kv_a, kv_b])
    a_ok = np.where((idx_a >= 0) & (idx_a < 50), idx_a, -1)
    b_ok = np.where((idx_b >= 0) & (idx_b < 30), idx_b + 50, -1)
    idx = np.where(sel[:, None] != 0, b_ok, a_ok)
    ref, rlse = oracle.sparse_decode_attn(q, cat, idx, 0.125, DV)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, rlse, rtol=1e-12, atol=1e-12)


def test_mixed_with_one_source_is_plain_attention():
    rng = np.random.default_rng(8)
    q = _raw_bf16(rng, (3, 2, 32))
    kv_a, kv_b = _raw_bf16(rng, (20, 32)), _raw_bf16(rng, (25, 32))
    idx = rng.integers(-1, 20, size=(3, 7))
    for sel, kv in ((np.zeros(3, int), kv_a), (np.ones(3, int), kv_b)):
        out, lse = oracle.sparse_decode_attn_mixed(q, kv_a, idx, kv_b, idx, sel, 0.2, 16)
        ref, rlse = oracle.sparse_decode_attn(q, kv, idx, 0.2, 16)
        assert np.array_equal(out, ref) and np.array_equal(lse, rlse)


def test_residency_rules_hand_worked():
    # block size 4.  Request 0: 18 tokens -> pages 0..4 used, page 2 reclaimed already.
    # Request 1: 8 tokens -> pages 0..1 (only the last two: nothing reclaimable).
    # Request 2: 13 tokens -> pages 0..3 used; page 5 mapped but unused.
    bt = np.array([[3, 8, -1, 4, 9, -1, -1],
                   [5, 6, -1, -1, -1, -1, -1],
                   [0, 1, 2, 7, -1, 11, -1]])
    seq = np.array([18, 8, 13])
    assert oracle.reclaimable_pages(bt, seq, 4) == [(0, 0), (0, 1), (2, 0), (2, 1)]
    assert oracle.is_fully_resident(bt, seq, 4).tolist() == [False, True, True]


def test_fully_resident_needs_every_used_page_inside_the_table_row():
    """A request whose token count needs more pages than its table row has cannot be fully
    resident, even when every entry the row does have is mapped.  Block size 4: 9 tokens use
    pages 0, 1 and 2, but the table rows are 2 wide; 8 tokens fit; 0 tokens need no page."""
    bt = np.array([[3, 5], [1, 2], [-1, -1]])
    seq = np.array([9, 8, 0])
    assert oracle.is_fully_resident(bt, seq, 4).tolist() == [False, True, True]


def test_reclaim_selection_hand_worked():
    """Worked by hand (block size 4).  Request 0: 18 tokens, pages 0-4 used, reclaimable
    pages 0, 1, 2 (never the last two).  Request 1: 20 tokens, pages 0-4 used, reclaimable
    0, 1, 2.  Request 2: 8 tokens, pages 0-1: nothing reclaimable.  Priorities 5, 1, 0:
    request 1 gives first (lowest priority among those with candidates), oldest page first;
    request 0 after it.  Page 1 of request 1 is hot: screened out."""
    bt = np.array([[10, 11, 12, 13, 14, -1],
                   [20, 21, 22, 23, 24, -1],
                   [30, 31, -1, -1, -1, -1]])
    seq = np.array([18, 20, 8])
    prio = np.array([5, 1, 0])
    hot = np.zeros(bt.shape, dtype=bool)
    hot[1, 1] = True
    sel = oracle.select_reclaim_pages
    assert sel(bt, seq, 4, 2, prio, hot) == [(1, 0), (1, 2)]
    assert sel(bt, seq, 4, 3, prio, hot) == [(1, 0), (1, 2), (0, 0)]
    assert sel(bt, seq, 4, 9, prio, hot) == [(1, 0), (1, 2), (0, 0), (0, 1), (0, 2)]
    assert sel(bt, seq, 4, 0, prio, hot) == []
    # no priorities and no hot pages: oldest page index first across requests, then request
    assert sel(bt, seq, 4, 4) == [(0, 0), (1, 0), (0, 1), (1, 1)]


def test_reclaim_selection_respects_the_budget_and_the_last_two_pages():
    """Random tables: the selection is at most the deficit, only reclaimable cold pages, in
    (priority, page, request) order, and it is a prefix of the same ordering with a larger
    deficit."""
    rng = np.random.default_rng(21)
    for trial in range(40):
        B, W, bs = 6, 10, 8
        seq = rng.integers(1, W * bs + 1, size=B)
        bt = rng.permutation(B * W).reshape(B, W)
        bt[rng.random((B, W)) < 0.15] = -1
        prio = rng.integers(0, 3, size=B)
        hot = rng.random((B, W)) < 0.2
        d = int(rng.integers(0, 12))
        got = oracle.select_reclaim_pages(bt, seq, bs, d, prio, hot)
        assert len(got) <= d
        ok = set(oracle.reclaimable_pages(bt, seq, bs))
        assert all(bp in ok and not hot[bp] for bp in got)
        keys = [(prio[b], p, b) for b, p in got]
        assert keys == sorted(keys)
        assert got == oracle.select_reclaim_pages(bt, seq, bs, d + 5, prio, hot)[:len(got)]
        if len(got) < d:  # everything eligible was taken
            assert len(got) == sum(1 for bp in ok if not hot[bp])
