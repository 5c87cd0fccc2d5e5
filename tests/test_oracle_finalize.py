"""Pins for the oracle's greedy accept and accepted-prefix finalize (CPU only).

The main pin is the pages' worked example (tests/golden/worked_example.json):
5 prompt tokens, verify rows [a0, b1, b2, b3], b1 accepted, b2 replaced by c2.
"""

import json
import os

import numpy as np
import torch

from oracle import HotState, build_hot_state, finalize_accepted, greedy_accept, resolve_topk
from tests.helpers import check_state_invariants, raw

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))


def _logits_with_choices(choices, vocab, seed=0):
    g = torch.Generator().manual_seed(seed)
    lg = torch.randn(len(choices), vocab, generator=g).to(torch.bfloat16)
    for i, c in enumerate(choices):
        lg[i, c] = 8.0
    return raw(lg)


def _worked_example_state():
    """One request, prompt of 5 plus 4 verify positions, one 16-token page, 8 hot slots."""
    names = GOLD["token_names"]
    R = len(GOLD["verify_rows"])
    P = GOLD["prompt_len"]
    seq = np.array([P + R], np.int32)
    bt = np.array([[2, -1]], np.int32)           # the request's tokens live on page 2
    bs = 16
    rng = np.random.default_rng(0)
    pool = rng.standard_normal((3 * bs, 6)).astype(np.float32)
    # all 9 positions resident (prompt + the 4 verify rows' temporary KV), stamps 0..8
    init_pos = np.full((1, 12), -1, np.int32)
    init_stamp = np.full((1, 12), -1, np.int32)
    init_pos[0, :9] = np.arange(9)
    init_stamp[0, :9] = np.arange(9)
    st = build_hot_state(init_pos, init_stamp, seq, bt, bs, pool)
    choices = [names[c] for c in GOLD["target_greedy_choice_per_row"]]
    logits = _logits_with_choices(choices, 64)
    draft = np.array([names[r] for r in GOLD["verify_rows"]], np.int32)
    return seq, bt, bs, pool, st, logits, draft, R


def test_worked_example_accept():
    seq, bt, bs, pool, st, logits, draft, R = _worked_example_state()
    acc, nxt, am = greedy_accept(logits, draft, 1, R)
    exp = GOLD["expected"]
    assert acc[0] == exp["accept_len"]
    assert nxt[0] == GOLD["token_names"][exp["next_token"]]
    # confirmed sequence = prompt + accepted rows + the replacement token
    assert GOLD["prompt_len"] + acc[0] + 1 + 1 == exp["confirmed_sequence_len"]


def test_worked_example_finalize_keeps_exact_prefix():
    seq, bt, bs, pool, st, logits, draft, R = _worked_example_state()
    exp = GOLD["expected"]
    acc, _, _ = greedy_accept(logits, draft, 1, R)
    rng = np.random.default_rng(9)
    new_kv = rng.standard_normal((R, 6)).astype(np.float32)
    pool_before = pool.copy()
    committed = finalize_accepted(st, pool, new_kv, acc, seq, bt, bs, R, tick=100)
    assert committed[0] == exp["committed_len"] == exp["next_anchor_position"]
    row_of = {t: 2 * bs + t for t in range(9)}
    kept = sorted(int(st.slot_loc[0, s]) - 2 * bs for s in range(12) if st.slot_loc[0, s] >= 0)
    assert kept == exp["kept_kv_positions"]
    for t in exp["dropped_positions"]:
        assert st.loc_to_hot[row_of[t]] == -1
        assert np.array_equal(pool[row_of[t]], pool_before[row_of[t]])   # host row untouched
    # the accepted rows' new KV reached host pool and hot buffer; prompt rows unchanged
    for r, t in enumerate(GOLD["verify_positions"][: acc[0] + 1]):
        assert np.array_equal(pool[row_of[t]], new_kv[r])
        assert np.array_equal(st.hot_kv[st.loc_to_hot[row_of[t]]], new_kv[r])
        assert st.slot_stamp[0, st.loc_to_hot[row_of[t]]] == 100
    for t in range(GOLD["prompt_len"]):
        assert np.array_equal(pool[row_of[t]], pool_before[row_of[t]])
    check_state_invariants(st, pool)
    # next round: the anchor sits at the committed length, drafts right after it
    assert [int(committed[0]) + 1 + i for i in range(GOLD["drafts_per_round"])] == exp["next_draft_positions"]


def test_accept_all_and_none():
    V = 32
    # 2 requests x 4 rows, wave-major rows
    choices = [5, 6, 7, 8, 9, 10, 11, 12]          # am[row]
    logits = _logits_with_choices(choices, V, seed=1)
    B = 2
    draft = np.zeros(8, np.int32)
    # request 0: every draft equals the previous row's choice -> accept all 3
    draft[1 * B + 0], draft[2 * B + 0], draft[3 * B + 0] = choices[0], choices[2], choices[4]
    # request 1: first draft already wrong -> accept 0
    draft[1 * B + 1], draft[2 * B + 1], draft[3 * B + 1] = 31, choices[3], choices[5]
    acc, nxt, am = greedy_accept(logits, draft, B, 4)
    assert am.tolist() == choices
    assert acc.tolist() == [3, 0]
    assert nxt.tolist() == [choices[6], choices[1]]      # bonus from the last row; else row 0's pick


def test_argmax_tie_takes_lowest_index_like_numpy():
    rng = np.random.default_rng(5)
    lg = torch.from_numpy(rng.standard_normal((50, 40)).astype(np.float32)).to(torch.bfloat16)
    for i in range(50):
        a, b = rng.choice(40, 2, replace=False)
        lg[i, a] = lg[i, b] = 9.0
    r = raw(lg)
    _, _, am = greedy_accept(r, np.zeros(50, np.int32), 50, 1)
    assert am.tolist() == np.argmax(lg.float().numpy(), axis=1).tolist()


def test_finalize_installs_misses_with_lru_rule():
    """Kept rows not in the hot buffer evict the least-recently-used unpinned slots."""
    bs, cap = 4, 6
    seq = np.array([10], np.int32)
    bt = np.array([[1, 0, 3]], np.int32)
    pool = np.arange(16 * 2, dtype=np.float32).reshape(16, 2)
    # resident positions 0..5 with stamps 10..15 -> slot s holds position s
    init_pos = np.arange(6, dtype=np.int32)[None]
    init_stamp = (10 + np.arange(6, dtype=np.int32))[None]
    st = build_hot_state(init_pos, init_stamp, seq, bt, bs, pool)
    new_kv = -np.arange(3 * 2, dtype=np.float32).reshape(3, 2) - 1
    # R=3 rows at positions 7, 8, 9; all accepted (L=2)
    committed = finalize_accepted(st, pool, new_kv, np.array([2]), seq, bt, bs, 3, tick=50)
    assert committed.tolist() == [10]
    # positions 7, 8, 9 -> rows: 7 -> page 0 (row 0*4+3=3); 8 -> page 3 row 12; 9 -> row 13
    rows, _ = resolve_topk(np.array([[7, 8, 9]], np.int32), np.array([0], np.int32),
                           np.array([10], np.int32), bt, bs, bs, 1)
    assert rows.tolist() == [[3, 12, 13]]
    # victims: the three oldest slots 0, 1, 2 (stamps 10, 11, 12), paired in row order
    assert st.slot_loc[0].tolist()[:3] == [3, 12, 13]
    assert st.slot_stamp[0].tolist() == [50, 50, 50, 13, 14, 15]
    check_state_invariants(st, pool)


def test_finalize_pins_kept_hits_when_tick_is_not_newest():
    """Worked by hand.  Block size 4, table [1, 0]: verify positions 6 and 7 (R = 2) live in
    host rows 2 and 3.  Slot 0 holds row 2 (stamp 10); slots 1-3 hold rows 8, 9, 10 (stamps
    11-13).  Both rows are kept (L = 1) with tick 5, below every stamp.  Row 2 hits slot 0:
    overwritten and restamped 5, and pinned, so although its stamp is now the lowest the miss
    of row 3 must evict slot 1 (stamp 11), not slot 0."""
    bs = 4
    seq = np.array([8], np.int32)
    bt = np.array([[1, 0]], np.int32)
    pool = np.arange(16 * 2, dtype=np.float32).reshape(16, 2)
    st = HotState(4, np.array([[2, 8, 9, 10]], np.int32), np.array([[10, 11, 12, 13]], np.int32),
                  np.full(16, -1, np.int32), pool[[2, 8, 9, 10]].copy())
    st.loc_to_hot[[2, 8, 9, 10]] = [0, 1, 2, 3]
    rows, _ = resolve_topk(np.array([[6, 7]], np.int32), np.array([0], np.int32), seq, bt, bs, bs, 1)
    assert rows.tolist() == [[2, 3]]
    new_kv = np.array([[-1.0, -2.0], [-3.0, -4.0]], np.float32)
    committed = finalize_accepted(st, pool, new_kv, np.array([1]), seq, bt, bs, 2, tick=5)
    assert committed.tolist() == [8]
    assert st.slot_loc[0].tolist() == [2, 3, 9, 10]
    assert st.slot_stamp[0].tolist() == [5, 5, 12, 13]
    assert st.loc_to_hot[2] == 0 and st.loc_to_hot[3] == 1 and st.loc_to_hot[8] == -1
    assert np.array_equal(st.hot_kv[[0, 1]], new_kv)
    assert np.array_equal(pool[[2, 3]], new_kv)
    check_state_invariants(st, pool)


def test_finalize_keeps_every_kept_row_resident_at_any_tick():
    """Random states and ticks (including ticks below existing stamps): after finalize every
    kept row is resident and holds its new KV, every dropped position is not, and the maps
    stay mutually inverse."""
    rng = np.random.default_rng(11)
    for trial in range(60):
        bs, cap, R = 4, int(rng.integers(4, 10)), int(rng.integers(1, 4))
        npages = 8
        seq = np.array([int(rng.integers(R, npages * bs + 1))], np.int32)
        bt = rng.permutation(npages).astype(np.int32)[None]
        pool = rng.standard_normal((npages * bs, 3)).astype(np.float32)
        n_res = int(rng.integers(0, min(cap, int(seq[0])) + 1))
        init_pos = np.full((1, cap), -1, np.int32)
        init_stamp = np.full((1, cap), -1, np.int32)
        where = rng.choice(cap, n_res, replace=False)
        init_pos[0, where] = rng.choice(int(seq[0]), n_res, replace=False)
        init_stamp[0, where] = rng.integers(0, 20, size=n_res)
        st = build_hot_state(init_pos, init_stamp, seq, bt, bs, pool)
        new_kv = rng.standard_normal((R, 3)).astype(np.float32)
        L = int(rng.integers(0, R))
        tick = int(rng.integers(0, 25))
        finalize_accepted(st, pool, new_kv, np.array([L]), seq, bt, bs, R, tick=tick)
        rows, _ = resolve_topk((seq[0] - R + np.arange(R, dtype=np.int32))[None], np.array([0], np.int32),
                               seq, bt, bs, bs, 1)
        for r in range(R):
            g = st.loc_to_hot[rows[0, r]]
            if r <= L:
                assert g >= 0, (trial, r)
                assert np.array_equal(st.hot_kv[g], new_kv[r]) and st.slot_stamp[0, g] == tick
            else:
                assert g == -1, (trial, r)
        check_state_invariants(st, pool)


def test_argmax_ignores_nan_like_numpy_nanargmax():
    """NaN never wins: on rows that hold NaNs next to finite values the argmax is numpy's
    nanargmax (lowest index of the largest non-NaN value).  A row of only NaN and -inf
    has no winner and keeps the lowest index, 0."""
    rng = np.random.default_rng(12)
    lg = rng.standard_normal((40, 33)).astype(np.float32)
    for i in range(40):
        lg[i, rng.choice(33, int(rng.integers(1, 10)), replace=False)] = np.nan
    lg[3, :] = np.nan
    lg[3, 5] = -np.inf
    t = torch.from_numpy(lg).to(torch.bfloat16)
    _, _, am = greedy_accept(raw(t), np.zeros(40, np.int32), 40, 1)
    f = t.float().numpy()
    for i in range(40):
        if i == 3:
            assert am[i] == 0
        else:
            assert am[i] == np.nanargmax(f[i]), i


def test_finalize_eviction_keeps_the_map_of_a_live_copy():
    """Worked by hand.  Slot 1 holds a stale copy of row 9 (the map names slot 0).  The one
    verify row (position 7: page index 1 -> table entry 0 -> host row 3) is kept and missing,
    so it evicts the least-recent slot, slot 1 (stamp 0).  loc_to_hot[9] keeps naming slot 0."""
    bs = 4
    seq = np.array([8], np.int32)
    bt = np.array([[1, 0]], np.int32)
    pool = np.arange(16 * 2, dtype=np.float32).reshape(16, 2)
    st = HotState(4, np.array([[9, 9, 10, 11]], np.int32), np.array([[1, 0, 5, 6]], np.int32),
                  np.full(16, -1, np.int32), pool[[9, 9, 10, 11]].copy())
    st.loc_to_hot[[9, 10, 11]] = [0, 2, 3]
    new_kv = np.array([[-5.0, -6.0]], np.float32)
    finalize_accepted(st, pool, new_kv, np.array([0]), seq, bt, bs, 1, tick=20)
    assert st.slot_loc[0].tolist() == [9, 3, 10, 11]
    assert st.slot_stamp[0].tolist() == [1, 20, 5, 6]
    assert st.loc_to_hot[9] == 0 and st.loc_to_hot[3] == 1
    assert np.array_equal(st.hot_kv[1], new_kv[0]) and np.array_equal(pool[3], new_kv[0])
