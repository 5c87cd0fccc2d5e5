"""Pins for the oracle's swap_in (hit/miss split + LRU hot buffer), CPU only."""

from collections import OrderedDict

import numpy as np
import pytest

from oracle import HotState, build_hot_state, resolve_topk, swap_in
from tests.helpers import check_state_invariants, check_state_weak, raw, with_duplicates
from workloads import generate, spec


def _setup(name, **over):
    s = spec(name, **over)
    w = generate(s)
    pool = raw(w.kv_pool)
    st = build_hot_state(w.init_pos, w.init_stamp, w.seq_len, w.block_table, s.block_size, pool)
    slots, _ = resolve_topk(w.topk_pos, w.req_id, w.causal_limit, w.block_table,
                            s.block_size, s.block_size, s.num_reqs)
    return s, w, pool, st, slots


@pytest.mark.parametrize("name,over", [("tiny", {}), ("tiny", {"seq_rule": ("fixed", [10, 70])}),
                                       ("mtp_swap", {"num_reqs": 3, "seq_rule": ("const", 6000),
                                                     "capacity": 1024, "topk": 256}),
                                       ("mixed_finalize", {"num_reqs": 4, "vocab": 64, "topk": 128,
                                                           "capacity": 512})])
def test_swap_invariants_over_waves(name, over):
    s, w, pool, st, slots = _setup(name, **over)
    check_state_invariants(st, pool)
    B = s.num_reqs
    for r in range(s.rows_per_req):
        wave = slots[r * B:(r + 1) * B]
        before = st.copy()
        hot_idx, mc, mp = swap_in(st, wave, s.tick0 + r, pool)
        check_state_invariants(st, pool)
        valid = wave >= 0
        # every valid entry is resident afterwards, and hot_idx names the slot holding it
        flat = st.slot_loc.reshape(-1)
        assert (flat[hot_idx[valid]] == wave[valid]).all()
        assert (hot_idx[~valid] == -1).all()
        # hot_idx stays inside the request's own slot range
        b_of = np.repeat(np.arange(B), s.topk).reshape(B, s.topk)
        assert ((hot_idx[valid] // s.capacity) == b_of[valid]).all()
        # hits + misses = valid; misses are exactly the entries absent before the call
        was_hit = valid & (before.loc_to_hot[np.where(valid, wave, 0)] >= 0)
        assert np.array_equal(mc, (valid & ~was_hit).sum(1))
        for b in range(B):
            assert mp[b, :mc[b]].tolist() == np.nonzero(valid[b] & ~was_hit[b])[0].tolist()
            assert (mp[b, mc[b]:] == -1).all()
        # hit entries keep their slot; touched slots carry the tick
        assert (hot_idx[was_hit] == before.loc_to_hot[wave[was_hit]]).all()
        assert (st.slot_stamp.reshape(-1)[hot_idx[valid]] == s.tick0 + r).all()
        # slots not touched by this wave keep their stamps unless they were evicted to host a miss
        untouched = np.ones(B * s.capacity, dtype=bool)
        untouched[hot_idx[valid]] = False
        assert (st.slot_stamp.reshape(-1)[untouched] == before.slot_stamp.reshape(-1)[untouched]).all()


def _empty_state(B, cap, host_rows, d):
    return HotState(cap, np.full((B, cap), -1, np.int32), np.full((B, cap), -1, np.int32),
                    np.full(host_rows, -1, np.int32), np.zeros((B * cap, d), np.float32))


def test_swap_empty_buffer_misses_fill_slots_in_order():
    rng = np.random.default_rng(0)
    pool = rng.standard_normal((200, 8)).astype(np.float32)
    st = _empty_state(2, 10, 200, 8)
    wave = np.array([[50, -1, 3, 77, 12, -1], [150, 151, 199, -1, -1, 160]], np.int32)
    hot_idx, mc, mp = swap_in(st, wave, 5, pool)
    assert mc.tolist() == [4, 4]
    assert hot_idx.tolist() == [[0, -1, 1, 2, 3, -1], [10, 11, 12, -1, -1, 13]]
    assert mp.tolist() == [[0, 2, 3, 4, -1, -1], [0, 1, 2, 5, -1, -1]]
    assert np.array_equal(st.hot_kv[[0, 1, 2, 3]], pool[[50, 3, 77, 12]])
    check_state_invariants(st, pool)


def test_swap_all_resident_only_stamps_change():
    s, w, pool, st, slots = _setup("tiny")
    B = s.num_reqs
    # make a wave of rows the buffer already holds
    wave = np.full((B, s.topk), -1, np.int32)
    for b in range(B):
        held = st.slot_loc[b][st.slot_loc[b] >= 0][: s.topk]
        wave[b, :len(held)] = held
    before = st.copy()
    hot_idx, mc, _ = swap_in(st, wave, 77, pool)
    assert (mc == 0).all()
    assert np.array_equal(st.slot_loc, before.slot_loc)
    assert np.array_equal(st.loc_to_hot, before.loc_to_hot)
    assert np.array_equal(st.hot_kv, before.hot_kv)
    touched = np.zeros(B * s.capacity, dtype=bool)
    touched[hot_idx[wave >= 0]] = True
    assert (st.slot_stamp.reshape(-1)[touched] == 77).all()
    assert np.array_equal(st.slot_stamp.reshape(-1)[~touched], before.slot_stamp.reshape(-1)[~touched])


def test_swap_victim_set_matches_textbook_lru():
    """With distinct stamps, the evicted set equals an OrderedDict LRU's evictions."""
    rng = np.random.default_rng(3)
    for trial in range(40):
        cap, host_rows, K = 12, 60, 8
        pool = rng.standard_normal((host_rows, 4)).astype(np.float32)
        st = _empty_state(1, cap, host_rows, 4)
        n_occ = int(rng.integers(0, cap + 1))
        rows_held = rng.choice(host_rows, n_occ, replace=False)
        slots_used = rng.choice(cap, n_occ, replace=False)
        stamps = rng.permutation(100)[:n_occ]                 # distinct
        lru = OrderedDict()
        for i in np.argsort(stamps):                          # oldest first
            st.slot_loc[0, slots_used[i]] = rows_held[i]
            st.slot_stamp[0, slots_used[i]] = stamps[i]
            st.loc_to_hot[rows_held[i]] = slots_used[i]
            st.hot_kv[slots_used[i]] = pool[rows_held[i]]
            lru[int(rows_held[i])] = True
        wave = rng.choice(host_rows, K, replace=False).astype(np.int32)[None, :]
        # textbook LRU: hits are protected, then misses evict from the cold end;
        # free capacity is used before anything is evicted
        hits = [int(x) for x in wave[0] if int(x) in lru]
        misses = [int(x) for x in wave[0] if int(x) not in lru]
        free = cap - len(lru)
        n_evict = max(0, len(misses) - free)
        evicted = [k for k in lru if k not in hits][:n_evict]
        before = set(int(x) for x in st.slot_loc[0] if x >= 0)
        swap_in(st, wave, 1000, pool)
        after = set(int(x) for x in st.slot_loc[0] if x >= 0)
        assert before - after == set(evicted), trial
        assert after == (before - set(evicted)) | set(misses)


def test_swap_pairs_misses_with_victims_in_slot_order():
    """Misses (in entry order) take the victims in ascending slot order, not LRU order."""
    pool = np.arange(100 * 2, dtype=np.float32).reshape(100, 2)
    st = _empty_state(1, 4, 100, 2)
    # slot s holds host row 10+s; stamps make LRU order slot 2 (1), slot 1 (2), slot 0 (5), slot 3 (9)
    for s, stamp in enumerate([5, 2, 1, 9]):
        st.slot_loc[0, s], st.slot_stamp[0, s] = 10 + s, stamp
        st.loc_to_hot[10 + s] = s
        st.hot_kv[s] = pool[10 + s]
    wave = np.array([[60, 13, 70]], np.int32)       # 13 hits slot 3; 60 and 70 miss
    hot_idx, mc, mp = swap_in(st, wave, 20, pool)
    assert mc.tolist() == [2] and mp[0, :2].tolist() == [0, 2]
    # victims {2, 1}; ascending slot order pairs 60 -> slot 1 and 70 -> slot 2
    assert hot_idx.tolist() == [[1, 3, 2]]
    assert st.slot_loc[0].tolist() == [10, 60, 70, 13]
    assert st.slot_stamp[0].tolist() == [5, 20, 20, 20]
    assert st.loc_to_hot[11] == -1 and st.loc_to_hot[12] == -1


DUP_CASE = ("mtp_swap", {"num_reqs": 3, "seq_rule": ("const", 6000), "capacity": 1024, "topk": 256})


def test_swap_duplicate_rows_in_a_request():
    """Top-k sets never repeat a row, but the call defines what a repeat does: copies of a hit
    share its slot; every copy of a miss is a miss of its own and takes its own victim under
    the pairing rule, so each entry's hot index names a slot holding its row.  From a state
    without repeats the map names the slot of the last copy; later waves keep the weaker
    invariants (a row may sit in several slots, the map names one of them or none)."""
    _duplicate_waves(*DUP_CASE)


def test_swap_duplicate_rows_evicting_stale_copies():
    """A small buffer: copies the map no longer names get evicted while their row is installed
    again in the same wave."""
    _duplicate_waves("tiny", {})


def _duplicate_waves(name, over):
    s, w, pool, st, slots = _setup(name, **over)
    B = s.num_reqs
    seen_hit_dup = seen_miss_dup = 0
    # wave 0 comes back after every other wave, so rows return while stale copies remain
    sched = [r for k in range(s.rows_per_req) for r in (k, 0)]
    for t, r in enumerate(sched):
        wave = with_duplicates(slots[r * B:(r + 1) * B])
        before = st.copy()
        hot_idx, mc, mp = swap_in(st, wave, s.tick0 + t, pool)
        check_state_weak(st, pool)
        valid = wave >= 0
        assert (st.slot_loc.reshape(-1)[hot_idx[valid]] == wave[valid]).all()
        assert np.array_equal(st.hot_kv[hot_idx[valid]], pool[wave[valid]])
        was_hit = valid & (before.loc_to_hot[np.where(valid, wave, 0)] >= 0)
        assert np.array_equal(mc, (valid & ~was_hit).sum(1))
        for b in range(B):
            miss_slots = hot_idx[b, valid[b] & ~was_hit[b]]
            assert len(np.unique(miss_slots)) == len(miss_slots), "two misses share a victim"
            assert not np.isin(miss_slots, hot_idx[b, was_hit[b]]).any()
            for row in np.unique(wave[b, valid[b]]):
                js = np.nonzero(wave[b] == row)[0]
                if len(js) < 2:
                    continue
                if was_hit[b, js[0]]:
                    seen_hit_dup += 1
                    assert (hot_idx[b, js] == before.loc_to_hot[row]).all()
                else:
                    seen_miss_dup += 1
                    assert len(np.unique(hot_idx[b, js])) == len(js)
                    # the map names the copy installed last (the highest victim slot)
                    assert st.loc_to_hot[row] == hot_idx[b, js[-1]]
            # no eviction of a stale copy unmaps a row this wave selected
            assert (st.loc_to_hot[wave[b, valid[b]]] >= 0).all()
    assert seen_hit_dup > 0 and seen_miss_dup > 0


def test_swap_map_rule_for_repeats_and_stale_copies_hand_worked():
    """Worked by hand.  Slot 2 holds a stale copy of row 10 (the map names slot 0 for it);
    the wave selects row 20 twice and row 11 once.  Row 11 hits slot 1 (pinned).  Victims:
    the two least-recent unpinned slots by (stamp, slot) are slot 3 (empty, -1) and slot 2
    (stamp 0); in ascending slot order miss 0 -> slot 2, miss 1 -> slot 3.  Evicting slot 2
    leaves loc_to_hot[10] alone (it names slot 0), and the map names slot 3, the copy of
    row 20 installed last."""
    pool = np.arange(100 * 2, dtype=np.float32).reshape(100, 2)
    st = _empty_state(1, 4, 100, 2)
    for slot, row, stamp in ((0, 10, 1), (1, 11, 2), (2, 10, 0)):
        st.slot_loc[0, slot], st.slot_stamp[0, slot] = row, stamp
        st.hot_kv[slot] = pool[row]
    st.loc_to_hot[10], st.loc_to_hot[11] = 0, 1
    hot_idx, mc, mp = swap_in(st, np.array([[20, 20, 11]], np.int32), 5, pool)
    assert hot_idx.tolist() == [[2, 3, 1]]
    assert mc.tolist() == [2] and mp.tolist() == [[0, 1, -1]]
    assert st.slot_loc[0].tolist() == [10, 11, 20, 20]
    assert st.slot_stamp[0].tolist() == [1, 5, 5, 5]
    assert st.loc_to_hot[10] == 0 and st.loc_to_hot[11] == 1 and st.loc_to_hot[20] == 3
    assert np.array_equal(st.hot_kv[[2, 3]], pool[[20, 20]])


def test_swap_rejects_a_row_owned_by_another_request():
    """Host rows belong to one request: request 0 selecting a row that request 1's slot
    holds is a caller error, and nothing is written."""
    pool = np.zeros((50, 2), np.float32)
    st = _empty_state(2, 4, 50, 2)
    st.slot_loc[1, 2], st.slot_stamp[1, 2], st.loc_to_hot[7] = 7, 3, 4 + 2
    before = st.copy()
    with pytest.raises(ValueError):
        swap_in(st, np.array([[7, 8], [-1, -1]], np.int32), 9, pool)
    assert np.array_equal(st.slot_loc, before.slot_loc)
    assert np.array_equal(st.loc_to_hot, before.loc_to_hot)
