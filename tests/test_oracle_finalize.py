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
