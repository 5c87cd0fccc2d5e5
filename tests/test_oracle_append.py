"""Pins of the oracle's append_accepted (draft-model context KV grows by the accepted
prefix): the P2 worked example, and properties that hold for any input."""

import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def test_worked_example_first_verify_step():
    g = json.load(open(GOLDEN))
    d, names = g["dflash_context"], g["token_names"]
    rows = [names[t] for t in g["verify_rows"]]         # a0, b1, b2, b3 (one request)
    new_rows = np.array([[v, v] for v in rows], dtype=np.uint16)
    cache = np.zeros((12, 2), dtype=np.uint16)
    bt = np.array([d["block_table"]])
    out, lens = oracle.append_accepted(cache, bt, np.array([d["context_len_before"]]), new_rows,
                                       np.array([g["expected"]["accept_len"]]),
                                       len(rows), d["block_size"], d["block_size"])
    assert lens.tolist() == [d["context_len_after"]]
    written = np.nonzero(out[:, 0])[0].tolist()
    assert written == d["appended_cache_rows"]
    assert out[written, 0].tolist() == [names[t] for t in d["appended_rows"]]


def test_two_appends_continue_where_the_first_stopped():
    """A second append continues after the first one's last position; nothing else is
    written."""
    rng = np.random.default_rng(1)
    B, R, bs, W = 4, 4, 8, 10
    bt = rng.permutation(B * W).reshape(B, W)
    bt[1, 3] = -1                      # an unmapped page: its positions are skipped
    cache = rng.integers(0, 2 ** 16, size=(B * W * bs, 3), dtype=np.uint16)
    lens0 = np.array([5, 17, 30, 0])
    rows1 = rng.integers(0, 2 ** 16, size=(B * R, 3), dtype=np.uint16)
    rows2 = rng.integers(0, 2 ** 16, size=(B * R, 3), dtype=np.uint16)
    acc1, acc2 = np.array([1, 3, 0, 2]), np.array([3, 0, 7, -2])  # clamped to [0, R-1]
    c1, l1 = oracle.append_accepted(cache, bt, lens0, rows1, acc1, R, bs, bs)
    c2, l2 = oracle.append_accepted(c1, bt, l1, rows2, acc2, R, bs, bs)
    L1, L2 = np.clip(acc1, 0, R - 1), np.clip(acc2, 0, R - 1)
    assert l2.tolist() == (lens0 + L1 + 1 + L2 + 1).tolist()
    expect = cache.copy()
    for b in range(B):
        seq = [rows1[r * B + b] for r in range(L1[b] + 1)] + [rows2[r * B + b] for r in range(L2[b] + 1)]
        for k, v in enumerate(seq):
            pos = lens0[b] + k
            page = bt[b, pos // bs]
            if page >= 0:
                expect[page * bs + pos % bs] = v
    assert np.array_equal(c2, expect)
