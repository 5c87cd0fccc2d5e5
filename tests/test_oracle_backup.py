"""Pins of the oracle's device -> host backup (plan_backup_rows, backup_rows).

The golden example (tests/golden/backup_example.json) was worked out by hand from P3's
"数据 back up" address formulas; the properties below hold for any input.
"""

import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "backup_example.json")


def _golden():
    return json.load(open(GOLDEN))


def test_plan_matches_hand_worked_example():
    g = _golden()["plan"]
    transfers = [oracle.PageTransfer(tuple(t["source_block_ids"]), t["destination_block_id"],
                                     t["destination_page_offset"]) for t in g["transfers"]]
    src, dst = oracle.plan_backup_rows(transfers, g["kernel_block_size"], g["blocks_per_kv_block"],
                                       g["num_caches"])
    assert src.tolist() == g["expected_src"]
    assert dst.tolist() == g["expected_dst"]


def test_copy_matches_hand_worked_example():
    g = _golden()["copy"]
    L, R, H = g["layers"], g["dev_rows"], g["host_rows"]
    dev = np.zeros((L, R, 2), dtype=np.uint16)
    for layer in range(L):
        for r in range(R):
            dev[layer, r, :] = 100 * layer + r
    host = np.full((L, H, 2), g["fill"], dtype=np.uint16)
    out = oracle.backup_rows(dev, host, np.array(g["src_slots"]), np.array(g["dst_rows"]),
                             g["src_block_size"], g["src_block_stride"])
    assert out[:, :, 0].tolist() == g["expected_host_markers"]
    assert np.array_equal(out[:, :, 0], out[:, :, 1])
    assert (host == g["fill"]).all()  # the input is not modified


def test_shared_list_equals_per_layer_copies_of_it():
    rng = np.random.default_rng(3)
    L, R, H, E, n = 3, 40, 30, 6, 25
    dev = rng.integers(0, 2 ** 16, size=(L, R, E), dtype=np.uint16)
    host = rng.integers(0, 2 ** 16, size=(L, H, E), dtype=np.uint16)
    src = rng.integers(-3, 45, size=n)
    dst = rng.permutation(H + 5)[:n] - 2
    a = oracle.backup_rows(dev, host, src, dst, 5, 7)
    b = oracle.backup_rows(dev, host, np.tile(src, (L, 1)), dst, 5, 7)
    assert np.array_equal(a, b)


def test_every_copied_row_is_its_source_and_nothing_else_changes():
    """Brute-force check against the definition with distinct destinations."""
    rng = np.random.default_rng(11)
    L, R, H, E, n = 2, 64, 50, 8, 40
    bs, stride = 8, 10
    dev = rng.integers(0, 2 ** 16, size=(L, R, E), dtype=np.uint16)
    host = rng.integers(0, 2 ** 16, size=(L, H, E), dtype=np.uint16)
    src = rng.integers(-2, 60, size=(L, n))
    dst = rng.permutation(np.arange(-5, H + 5))[:n]
    out = oracle.backup_rows(dev, host, src, dst, bs, stride)
    written = np.zeros((L, H), dtype=bool)
    for layer in range(L):
        for i in range(n):
            s, d = int(src[layer, i]), int(dst[i])
            p = (s // bs) * stride + s % bs
            if s >= 0 and 0 <= d < H and p < R:
                assert np.array_equal(out[layer, d], dev[layer, p])
                written[layer, d] = True
    assert np.array_equal(out[~written], host[~written])


def test_plan_then_copy_moves_each_page_to_its_host_page():
    """Planning and copying compose: host page (block * per + page) ends up holding the
    device block's rows, for every cache."""
    rng = np.random.default_rng(5)
    kbs, per, C = 16, 4, 3
    dev_blocks, host_blocks = 12, 5
    dev = rng.integers(0, 2 ** 16, size=(C, dev_blocks * kbs, 4), dtype=np.uint16)
    host = np.zeros((C, host_blocks * per * kbs, 4), dtype=np.uint16)
    transfers = [oracle.PageTransfer(tuple(int(x) for x in rng.integers(0, dev_blocks, size=C)),
                                     int(hb), int(po))
                 for hb, po in [(0, 3), (4, 0), (2, 2)]]
    src, dst = oracle.plan_backup_rows(transfers, kbs, per, C)
    out = oracle.backup_rows(dev, host, src, dst)
    for tr in transfers:
        hp = tr.destination_block_id * per + tr.destination_page_offset
        for c in range(C):
            sb = tr.source_block_ids[c]
            assert np.array_equal(out[c, hp * kbs:(hp + 1) * kbs], dev[c, sb * kbs:(sb + 1) * kbs])
