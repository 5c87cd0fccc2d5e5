"""Pins for the oracle's resolve_topk (CPU only).

The mapping is checked against an independent construction: a simulated paged
writer that appends each request's tokens, in order, into the rows of the pages
its block table lists (P3 "数据 back up": block ``p`` spans rows
``p*block_size + offset``), and tags every row with (request, position).
Resolving a position must land on the row tagged with it.
"""

import numpy as np
import pytest

from oracle import resolve_topk
from workloads import generate, spec


def _tag_pool(block_table, seq_len, block_size, num_pages):
    """Tag every physical row with the (request, position) a sequential writer puts there."""
    tag_req = np.full(num_pages * block_size, -1, dtype=np.int64)
    tag_pos = np.full(num_pages * block_size, -1, dtype=np.int64)
    for b in range(len(seq_len)):
        written = 0
        for page in block_table[b]:
            if page < 0 or written >= seq_len[b]:
                break
            for row in range(page * block_size, page * block_size + block_size):
                if written >= seq_len[b]:
                    break
                tag_req[row], tag_pos[row] = b, written
                written += 1
        assert written == seq_len[b]
    return tag_req, tag_pos


@pytest.mark.parametrize("name,over", [("tiny", {}), ("tiny", {"seq_rule": ("fixed", [10, 70])}),
                                       ("resident", {"num_reqs": 3}),
                                       ("mixed_finalize", {"num_reqs": 5, "vocab": 64})])
def test_resolve_matches_sequential_writer(name, over):
    s = spec(name, **over)
    w = generate(s)
    slots, valid = resolve_topk(w.topk_pos, w.req_id, w.causal_limit, w.block_table,
                                s.block_size, s.block_size, s.num_reqs)
    tag_req, tag_pos = _tag_pool(w.block_table, w.seq_len, s.block_size, w.num_pages)
    t = w.topk_pos
    inlim = (t >= 0) & (t < w.causal_limit[:, None])
    # -1 exactly where the position is padding or past the causal limit
    assert np.array_equal(slots >= 0, inlim)
    assert np.array_equal(valid, inlim.sum(1))
    r, j = np.nonzero(inlim)
    assert (tag_req[slots[r, j]] == w.req_id[r]).all()
    assert (tag_pos[slots[r, j]] == t[r, j]).all()


def test_resolve_tiny_exhaustive_injective():
    s = spec("tiny")
    w = generate(s)
    seen = {}
    for b in range(s.num_reqs):
        pos = np.arange(int(w.seq_len[b]), dtype=np.int32)[None, :]
        out, v = resolve_topk(pos, np.array([b], np.int32), np.array([w.seq_len[b]], np.int32),
                              w.block_table, s.block_size, s.block_size, s.num_reqs)
        assert v[0] == w.seq_len[b]
        for t, row in enumerate(out[0]):
            assert row not in seen, "two (request, position) pairs share a physical row"
            seen[int(row)] = (b, t)
    assert len(seen) == int(w.seq_len.sum())


def test_resolve_fail_closed_cases():
    bt = np.array([[3, -1, 1], [0, 2, -1]], dtype=np.int32)
    pos = np.array([[0, 5, 9, 4, -1, 12, 100, -7],
                    [0, 5, 9, 4, -1, 12, 100, -7],
                    [1, 2, 3, 4, 5, 6, 7, 8]], dtype=np.int32)
    req = np.array([0, 1, 7], dtype=np.int32)          # request 7 does not exist
    lim = np.array([13, 9, 100], dtype=np.int32)
    out, v = resolve_topk(pos, req, lim, bt, 4, 4, 2)
    # req 0, pages [3, -1, 1]: 0 -> row 12; 5 and 4 fall in table slot 1 (no page);
    # 9 -> page 1 offset 1 = row 5; 12 is past the 3-entry table row; 100 past the limit
    assert out[0].tolist() == [12, -1, 5, -1, -1, -1, -1, -1]
    # req 1 (limit 9): 0 -> page 0; 5 -> page 2 offset 1; 9 past limit; 4 -> page 2 offset 0
    assert out[1].tolist() == [0, 9, -1, 8, -1, -1, -1, -1]
    assert out[2].tolist() == [-1] * 8
    assert v.tolist() == [2, 3, 0]


def test_resolve_physical_block_stride():
    # a stride larger than the block size leaves gaps between pages (packed layouts)
    bt = np.array([[2, 0]], dtype=np.int32)
    pos = np.array([[0, 1, 2, 3]], dtype=np.int32)
    out, _ = resolve_topk(pos, np.array([0], np.int32), np.array([4], np.int32), bt, 2, 8, 1)
    assert out[0].tolist() == [16, 17, 0, 1]


def test_resolve_masks_position_at_causal_limit():
    # the limit is exclusive: a query row at position p may see positions <= p only
    bt = np.array([[0, 1, 2]], dtype=np.int32)
    pos = np.array([[8, 9, 10]], dtype=np.int32)
    out, v = resolve_topk(pos, np.array([0], np.int32), np.array([9], np.int32), bt, 4, 4, 1)
    assert out[0].tolist() == [8, -1, -1] and v.tolist() == [1]
