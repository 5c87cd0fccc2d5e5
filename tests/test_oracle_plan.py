"""Pins of the oracle's apply_plan (a follower cache applies the leader's swap plan).

Hand-worked example, and the equivalence the plan exists for: a follower that applies the
leader's plan ends with exactly the hot buffer it would have had by swapping its own host
pool under the same state (oracle.swap_in, pinned separately).
"""

import numpy as np

import oracle


def test_hand_worked_example():
    # one request, 4 slots; entries 0 and 2 missed into slots 1 and 0, entry 1 hit slot 3
    wave_rows = np.array([[5, 2, 9]])
    hot_idx = np.array([[1, 3, 0]])
    miss_count = np.array([2])
    miss_pos = np.array([[0, 2, -1]])
    host = np.zeros((2, 12, 3), dtype=np.uint16)
    for c in range(2):
        for r in range(12):
            host[c, r] = 1000 * (c + 1) + r
    hot = np.full((2, 4, 3), 7, dtype=np.uint16)
    out = oracle.apply_plan(hot, host, wave_rows, hot_idx, miss_count, miss_pos)
    assert out[:, :, 0].tolist() == [[1009, 1005, 7, 7], [2009, 2005, 7, 7]]
    assert (hot == 7).all()


def _state(rng, B, cap, host_rows, E):
    """Request b owns the host rows r with r % B == b (each host row belongs to one request)."""
    st = oracle.HotState(cap, np.full((B, cap), -1, dtype=np.int64), np.full((B, cap), -1, dtype=np.int64),
                         np.full(host_rows, -1, dtype=np.int64), np.zeros((B * cap, E), dtype=np.uint16))
    for b in range(B):
        own = rng.permutation(np.arange(b, host_rows, B))
        k = 0
        for s in range(cap):
            if rng.random() < 0.7:
                st.slot_loc[b, s] = own[k]
                st.loc_to_hot[own[k]] = b * cap + s
                st.slot_stamp[b, s] = int(rng.integers(0, 50))
                k += 1
    return st


def _wave(rng, st, B, K, host_rows):
    rows = np.full((B, K), -1, dtype=np.int64)
    for b in range(B):
        held = st.slot_loc[b][st.slot_loc[b] >= 0]
        own = np.arange(b, host_rows, B)
        pick = np.concatenate([rng.choice(held, K // 2, replace=False),
                               rng.choice(np.setdiff1d(own, held), K - K // 2, replace=False)])
        rows[b] = rng.permutation(pick)
    rows[0, 3] = -1
    return rows


def test_apply_plan_equals_follower_swapping_itself():
    rng = np.random.default_rng(4)
    B, cap, K, host_rows, E, C = 3, 40, 24, 400, 8, 2
    st = _state(rng, B, cap, host_rows, E)
    pools = rng.integers(0, 2 ** 16, size=(C + 1, host_rows, E), dtype=np.uint16)
    # every cache's hot buffer is consistent with the shared state
    hots = np.zeros((C + 1, B * cap, E), dtype=np.uint16)
    for c in range(C + 1):
        for g in range(B * cap):
            r = st.slot_loc.reshape(-1)[g]
            hots[c, g] = pools[c, r] if r >= 0 else rng.integers(0, 2 ** 16, size=E)
    for wave in range(3):
        wave_rows = _wave(rng, st, B, K, host_rows)
        followers_self = []
        for c in range(1, C + 1):  # each follower swapping on its own, from the same state
            fst = st.copy()
            fst.hot_kv = hots[c].copy()
            oracle.swap_in(fst, wave_rows, 100 + wave, pools[c])
            followers_self.append(fst.hot_kv)
        st.hot_kv = hots[0].copy()
        hot_idx, miss_count, miss_pos = oracle.swap_in(st, wave_rows, 100 + wave, pools[0])
        assert miss_count.sum() > 0
        applied = oracle.apply_plan(hots[1:], pools[1:], wave_rows, hot_idx, miss_count, miss_pos)
        for c in range(C):
            assert np.array_equal(applied[c], followers_self[c])
        hots = np.concatenate([st.hot_kv[None], applied])
        # invariant of every cache: occupied slots hold their host row
        for c in range(C + 1):
            occ = np.nonzero(st.slot_loc.reshape(-1) >= 0)[0]
            assert np.array_equal(hots[c][occ], pools[c][st.slot_loc.reshape(-1)[occ]])
