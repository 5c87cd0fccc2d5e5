"""GPU parity of hs_finalize_accepted on the pages' worked example and on edge cases,
and cross-path identity of attention (resident pool vs swapped-in hot buffer)."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import dev, gpu_inputs, log, make, oracle_resolve, to_dev
from tests.helpers import check_state_invariants, raw

pytestmark = pytest.mark.gpu
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))


def _pinned(a: np.ndarray) -> torch.Tensor:
    t = torch.empty(a.shape, dtype=torch.float32, pin_memory=True)
    t.copy_(torch.from_numpy(a))
    return t


def _run_finalize(B, R, cap, seq, bt, bs, pool, init_pos, init_stamp, logits, draft, new_kv, tick):
    """Run GPU and oracle finalize on the same inputs; return both results."""
    import sparse_attention_kv_amd as hs
    from sparse_attention_kv_amd.pipeline import build_hot_state
    ost = oracle.build_hot_state(init_pos, init_stamp, seq, bt, bs, pool.copy())
    opool = pool.copy()
    acc, nxt, am = oracle.greedy_accept(raw(logits), draft, B, R)
    committed = oracle.finalize_accepted(ost, opool, new_kv, acc, seq, bt, bs, R, tick)
    hpool = _pinned(pool)
    gst = build_hot_state(torch.from_numpy(init_pos), torch.from_numpy(init_stamp), to_dev(seq),
                          to_dev(bt), bs, hpool, dev())
    g_am = torch.empty((B * R,), dtype=torch.int32, device=dev())
    g_acc = torch.empty((B,), dtype=torch.int32, device=dev())
    g_nxt = torch.empty((B,), dtype=torch.int32, device=dev())
    log(f"finalize B={B} R={R} cap={cap} vocab={logits.shape[1]}")
    hs.hs_finalize_accepted(gst, logits.to(dev()), to_dev(draft), torch.from_numpy(new_kv).to(dev()),
                            R, to_dev(seq), to_dev(bt), bs, tick, g_am, g_acc, g_nxt)
    torch.cuda.synchronize()
    assert np.array_equal(g_am.cpu().numpy(), am)
    assert np.array_equal(g_acc.cpu().numpy(), acc)
    assert np.array_equal(g_nxt.cpu().numpy(), nxt)
    assert np.array_equal(gst.slot_loc.cpu().numpy(), ost.slot_loc)
    assert np.array_equal(gst.slot_stamp.cpu().numpy(), ost.slot_stamp)
    assert np.array_equal(gst.loc_to_hot.cpu().numpy(), ost.loc_to_hot)
    occ = np.nonzero(ost.slot_loc.reshape(-1) >= 0)[0]
    assert np.array_equal(gst.hot_kv.cpu().numpy()[occ], ost.hot_kv[occ])
    assert np.array_equal(hpool.numpy(), opool)
    check_state_invariants(ost, opool)
    return acc, nxt, committed, ost, opool


def test_worked_example_on_gpu():
    names = GOLD["token_names"]
    R, P = len(GOLD["verify_rows"]), GOLD["prompt_len"]
    seq = np.array([P + R], np.int32)
    bt = np.array([[2, -1]], np.int32)
    bs, cap = 16, 12
    rng = np.random.default_rng(0)
    pool = rng.standard_normal((3 * bs, 8)).astype(np.float32)
    init_pos = np.full((1, cap), -1, np.int32)
    init_stamp = np.full((1, cap), -1, np.int32)
    init_pos[0, :9] = np.arange(9)
    init_stamp[0, :9] = np.arange(9)
    gen = torch.Generator().manual_seed(0)
    logits = torch.randn(R, 64, generator=gen).to(torch.bfloat16)
    for i, c in enumerate(GOLD["target_greedy_choice_per_row"]):
        logits[i, names[c]] = 8.0
    draft = np.array([names[r] for r in GOLD["verify_rows"]], np.int32)
    new_kv = rng.standard_normal((R, 8)).astype(np.float32)
    acc, nxt, committed, ost, _ = _run_finalize(1, R, cap, seq, bt, bs, pool, init_pos, init_stamp,
                                                logits, draft, new_kv, tick=100)
    exp = GOLD["expected"]
    assert acc[0] == exp["accept_len"] and nxt[0] == names[exp["next_token"]]
    assert committed[0] == exp["committed_len"]
    kept = sorted(int(x) - 2 * bs for x in ost.slot_loc[0] if x >= 0)
    assert kept == exp["kept_kv_positions"]


@pytest.mark.parametrize("vocab", [61, 1000, 129280])
def test_finalize_random_requests(vocab):
    """Several requests: mixed accept lengths, ties, misses installed with the LRU rule."""
    rng = np.random.default_rng(vocab)
    B, R, cap, bs, width = 9, 4, 40, 8, 12
    bt = rng.permutation(B * width).astype(np.int32).reshape(B, width)
    seq = rng.integers(R + 1, width * bs, size=B).astype(np.int32)
    pool = rng.standard_normal((B * width * bs, 16)).astype(np.float32)
    init_pos = np.full((B, cap), -1, np.int32)
    init_stamp = np.full((B, cap), -1, np.int32)
    for b in range(B):
        cnt = int(rng.integers(0, min(cap, seq[b]) + 1))
        pos = rng.choice(int(seq[b]), cnt, replace=False)
        sl = rng.permutation(cap)[:cnt]
        init_pos[b, sl] = pos
        init_stamp[b, sl] = rng.integers(0, 4, size=cnt)
    gen = torch.Generator().manual_seed(vocab)
    logits = torch.randn(B * R, vocab, generator=gen).to(torch.bfloat16)
    plant = rng.integers(0, vocab, size=B * R)
    logits[torch.arange(B * R), torch.from_numpy(plant)] = 9.0
    for i in range(0, B * R, 3):                 # ties: a second maximum in some rows
        logits[i, int(rng.integers(0, vocab))] = 9.0
    draft = rng.integers(0, vocab, size=B * R).astype(np.int32)
    for r in range(1, R):
        for b in range(B):
            if rng.random() < 0.75:
                draft[r * B + b] = plant[(r - 1) * B + b]
    new_kv = rng.standard_normal((B * R, 16)).astype(np.float32)
    acc, *_ = _run_finalize(B, R, cap, seq, bt, bs, pool, init_pos, init_stamp, logits, draft,
                            new_kv, tick=50)
    log(f"accept lengths {acc.tolist()}")




@pytest.mark.parametrize("accept", [63, 40, 0])
def test_finalize_sixty_four_verify_rows(accept):
    """The most verify rows a request may have (64): the acceptance ballot spans a whole
    wave, and up to 64 kept rows miss and are installed with the LRU rule."""
    rng = np.random.default_rng(6400 + accept)
    B, R, cap, bs, width = 3, 64, 96, 16, 12
    bt = rng.permutation(B * width).astype(np.int32).reshape(B, width)
    seq = np.full(B, width * bs - 3, np.int32)
    pool = rng.standard_normal((B * width * bs, 16)).astype(np.float32)
    init_pos = np.full((B, cap), -1, np.int32)
    init_stamp = np.full((B, cap), -1, np.int32)
    for b in range(B):  # full buffers: committed positions plus a few verify positions
        pos = rng.choice(int(seq[b]) - R, cap - 5, replace=False)
        init_pos[b, :cap - 5] = pos
        init_pos[b, cap - 5:] = seq[b] - R + np.array([0, 3, 17, 40, 63])
        init_stamp[b] = rng.integers(0, 30, size=cap)
    vocab = 300
    gen = torch.Generator().manual_seed(accept)
    logits = torch.randn(B * R, vocab, generator=gen).to(torch.bfloat16)
    plant = rng.integers(0, vocab, size=B * R)
    logits[torch.arange(B * R), torch.from_numpy(plant)] = 9.0
    draft = rng.integers(0, vocab, size=B * R).astype(np.int32)
    for b in range(B):
        for r in range(1, accept + 1):
            draft[r * B + b] = plant[(r - 1) * B + b]
        if accept + 1 < R:  # the first rejected draft differs from the argmax
            draft[(accept + 1) * B + b] = (plant[accept * B + b] + 1) % vocab
    new_kv = rng.standard_normal((B * R, 16)).astype(np.float32)
    acc, *_ = _run_finalize(B, R, cap, seq, bt, bs, pool, init_pos, init_stamp, logits, draft,
                            new_kv, tick=40)
    assert acc.tolist() == [accept] * B

@pytest.mark.parametrize("accept", [3, 1, 0])
def test_finalize_large_capacity_with_resident_and_dropped_rows(accept):
    """4608 hot slots per request, beyond the 4096 (stamp, slot) keys the kernel keeps in
    registers, with verify rows already resident: kept ones are pinned, dropped ones are
    emptied in memory first, and the victim search then reads those emptied slots (the
    preferred victims) from memory.  Nearly full buffers with stamps from a small range
    (many ties, broken by slot)."""
    rng = np.random.default_rng(4608 + accept)
    B, R, cap, bs, width = 3, 4, 4608, 64, 80
    bt = rng.permutation(B * width).astype(np.int32).reshape(B, width)
    seq = np.full(B, width * bs - 3, np.int32)
    pool = rng.standard_normal((B * width * bs, 16)).astype(np.float32)
    init_pos = np.full((B, cap), -1, np.int32)
    init_stamp = np.full((B, cap), -1, np.int32)
    for b in range(B):
        sl = rng.permutation(cap)
        pos = rng.choice(int(seq[b]) - R, cap - 8, replace=False)
        init_pos[b, sl[:cap - 8]] = pos
        init_stamp[b, sl[:cap - 8]] = rng.integers(0, 30, size=cap - 8)
        hits = seq[b] - R + np.array([0, 2, 3]) if b != 1 else seq[b] - R + np.array([1])
        init_pos[b, sl[cap - 8:cap - 8 + len(hits)]] = hits  # resident verify rows
        init_stamp[b, sl[cap - 8:cap - 8 + len(hits)]] = rng.integers(0, 30, size=len(hits))
    vocab = 300
    gen = torch.Generator().manual_seed(4608 + accept)
    logits = torch.randn(B * R, vocab, generator=gen).to(torch.bfloat16)
    plant = rng.integers(0, vocab, size=B * R)
    logits[torch.arange(B * R), torch.from_numpy(plant)] = 9.0
    draft = rng.integers(0, vocab, size=B * R).astype(np.int32)
    for b in range(B):
        for r in range(1, accept + 1):
            draft[r * B + b] = plant[(r - 1) * B + b]
        if accept + 1 < R:
            draft[(accept + 1) * B + b] = (plant[accept * B + b] + 1) % vocab
    new_kv = rng.standard_normal((B * R, 16)).astype(np.float32)
    acc, *_ = _run_finalize(B, R, cap, seq, bt, bs, pool, init_pos, init_stamp, logits, draft,
                            new_kv, tick=31)
    assert acc.tolist() == [accept] * B


@pytest.mark.parametrize("vocab", [129280, 129281, 8, 9])
def test_argmax_special_values(vocab):
    """Argmax rows with NaN, -inf, all-NaN and all -inf rows, the maximum in the first or
    the last element, and ties between the first and a later pass of the kernel's loads:
    the lowest index of the maximum, NaN never winning (an all-NaN row gives 0)."""
    B, R, cap, bs, width = 4, 3, 16, 8, 4
    rows = B * R
    gen = torch.Generator().manual_seed(vocab)
    logits = torch.randn(rows, vocab, generator=gen).to(torch.bfloat16)
    nan, inf = float("nan"), float("inf")
    logits[0, :] = -inf                                   # all -inf: index 0
    logits[1, :] = nan                                    # all NaN: index 0
    logits[2, 0] = nan; logits[2, vocab - 1] = 50.0       # maximum in the last element
    logits[3, 0] = 50.0; logits[3, 1:] = nan              # maximum first, NaN after
    logits[4, :] = -inf; logits[4, vocab // 2] = nan      # NaN among -inf: index 0
    if vocab > 9000:                                      # equal maxima 8704 apart, and at
        logits[5, 8704 + 3] = 40.0; logits[5, 3] = 40.0  # the start of a later pass
        logits[6, vocab - 2] = 40.0; logits[6, 4096 * 8 + 1] = 40.0
    logits[7, :] = 0.0; logits[7, 5:] = -0.0              # +0 and -0 compare equal: index 0
    seq = np.full(B, width * bs - 2, np.int32)
    bt = np.arange(B * width, dtype=np.int32).reshape(B, width)
    rng = np.random.default_rng(vocab)
    pool = rng.standard_normal((B * width * bs, 8)).astype(np.float32)
    init_pos = np.full((B, cap), -1, np.int32)
    init_stamp = np.full((B, cap), -1, np.int32)
    draft = rng.integers(0, vocab, size=rows).astype(np.int32)
    new_kv = rng.standard_normal((rows, 8)).astype(np.float32)
    _run_finalize(B, R, cap, seq, bt, bs, pool, init_pos, init_stamp, logits, draft, new_kv,
                  tick=7)


def test_finalize_capacity_beyond_register_keys():
    """More than 4096 hot slots per request: the victim search reads the stamps from
    memory instead of registers; nearly full buffers so every miss evicts."""
    rng = np.random.default_rng(4099)
    B, R, cap, bs, width = 3, 4, 4500, 64, 80
    bt = rng.permutation(B * width).astype(np.int32).reshape(B, width)
    seq = rng.integers(4600, width * bs, size=B).astype(np.int32)
    pool = rng.standard_normal((B * width * bs, 8)).astype(np.float32)
    init_pos = np.full((B, cap), -1, np.int32)
    init_stamp = np.full((B, cap), -1, np.int32)
    for b in range(B):
        pos = rng.choice(int(seq[b]) - R, cap, replace=False)   # full; no verify row resident
        init_pos[b] = pos
        init_stamp[b] = rng.integers(0, 50, size=cap)
        if b == 1:                                               # two verify rows resident
            init_pos[b, 17] = seq[b] - R
            init_pos[b, 4400] = seq[b] - 1
    vocab = 1000
    gen = torch.Generator().manual_seed(1)
    logits = torch.randn(B * R, vocab, generator=gen).to(torch.bfloat16)
    plant = rng.integers(0, vocab, size=B * R)
    logits[torch.arange(B * R), torch.from_numpy(plant)] = 9.0
    draft = rng.integers(0, vocab, size=B * R).astype(np.int32)
    for b in range(B):                                           # accept lengths 3, 1, 2
        for r in range(1, [4, 2, 3][b]):
            draft[r * B + b] = plant[(r - 1) * B + b]
    new_kv = rng.standard_normal((B * R, 8)).astype(np.float32)
    acc, *_ = _run_finalize(B, R, cap, seq, bt, bs, pool, init_pos, init_stamp, logits, draft,
                            new_kv, tick=60)
    assert acc.tolist() == [3, 1, 2]

def test_finalize_tick_below_stamps_keeps_kept_hits_pinned():
    """Full buffers whose stamps are all above the finalize tick: a kept row that hits is
    restamped to the tick, the lowest stamp in its request, and must stay pinned while the
    request's kept misses pick their victims (the LRU rule would otherwise evict it)."""
    rng = np.random.default_rng(515)
    B, R, cap, bs, width = 12, 4, 16, 8, 12
    bt = rng.permutation(B * width).astype(np.int32).reshape(B, width)
    seq = rng.integers(cap + R + 1, width * bs, size=B).astype(np.int32)
    pool = rng.standard_normal((B * width * bs, 8)).astype(np.float32)
    init_pos = np.full((B, cap), -1, np.int32)
    init_stamp = np.full((B, cap), -1, np.int32)
    for b in range(B):
        verify = seq[b] - R + np.arange(R)
        hit = verify[rng.random(R) < 0.5]                 # some verify rows already resident
        others = rng.choice(int(seq[b]) - R, cap - len(hit), replace=False)
        init_pos[b] = rng.permutation(np.concatenate([hit, others]))
        init_stamp[b] = rng.integers(10, 40, size=cap)
    vocab = 300
    gen = torch.Generator().manual_seed(515)
    logits = torch.randn(B * R, vocab, generator=gen).to(torch.bfloat16)
    plant = rng.integers(0, vocab, size=B * R)
    logits[torch.arange(B * R), torch.from_numpy(plant)] = 9.0
    draft = rng.integers(0, vocab, size=B * R).astype(np.int32)
    for r in range(1, R):
        for b in range(B):
            if rng.random() < 0.8:
                draft[r * B + b] = plant[(r - 1) * B + b]
    new_kv = rng.standard_normal((B * R, 8)).astype(np.float32)
    acc, _, _, ost, _ = _run_finalize(B, R, cap, seq, bt, bs, pool, init_pos, init_stamp, logits,
                                      draft, new_kv, tick=5)
    # the case is reached: some request keeps a resident row and installs a missing one
    reached = 0
    for b in range(B):
        kept = seq[b] - R + np.arange(acc[b] + 1)
        was = np.isin(kept, init_pos[b])
        reached += bool(was.any() and (~was).any())
    log(f"finalize low tick: {reached} requests keep a hit and install a miss")
    assert reached > 0


def test_finalize_eviction_of_a_stale_copy():
    """Slot 1 holds a stale copy of host row 9 (the map names slot 0); the kept verify row
    misses and evicts slot 1, the least recent: row 9 stays mapped to slot 0 (worked by hand
    in the oracle's pins; here the kernel must give the same state)."""
    import sparse_attention_kv_amd as hs
    bs, cap, R = 4, 4, 1
    seq = np.array([8], np.int32)
    bt = np.array([[1, 0]], np.int32)
    pool = np.arange(16 * 8, dtype=np.float32).reshape(16, 8)
    slot_loc = np.array([[9, 9, 10, 11]], np.int32)
    stamps = np.array([[1, 0, 5, 6]], np.int32)
    l2h = np.full(16, -1, np.int32)
    l2h[[9, 10, 11]] = [0, 2, 3]
    ost = oracle.HotState(cap, slot_loc.copy(), stamps.copy(), l2h.copy(), pool[[9, 9, 10, 11]].copy())
    opool = pool.copy()
    new_kv = -np.arange(8, dtype=np.float32)[None] - 1
    logits = torch.zeros((1, 16), dtype=torch.bfloat16)
    oracle.finalize_accepted(ost, opool, new_kv, np.array([0]), seq, bt, bs, R, 20)
    hpool = _pinned(pool)
    gst = hs.HotState(to_dev(slot_loc), to_dev(stamps), to_dev(l2h),
                      torch.from_numpy(pool[[9, 9, 10, 11]].copy()).to(dev()), hpool)
    am = torch.empty((1,), dtype=torch.int32, device=dev())
    acc = torch.empty((1,), dtype=torch.int32, device=dev())
    nxt = torch.empty((1,), dtype=torch.int32, device=dev())
    hs.hs_finalize_accepted(gst, logits.to(dev()), to_dev(np.zeros(1, np.int32)),
                            torch.from_numpy(new_kv).to(dev()), R, to_dev(seq), to_dev(bt), bs, 20,
                            am, acc, nxt)
    torch.cuda.synchronize()
    assert ost.slot_loc.tolist() == [[9, 3, 10, 11]] and ost.loc_to_hot[9] == 0
    assert np.array_equal(gst.slot_loc.cpu().numpy(), ost.slot_loc)
    assert np.array_equal(gst.slot_stamp.cpu().numpy(), ost.slot_stamp)
    assert np.array_equal(gst.loc_to_hot.cpu().numpy(), ost.loc_to_hot)
    assert np.array_equal(gst.hot_kv.cpu().numpy(), ost.hot_kv)
    assert np.array_equal(hpool.numpy(), opool)


@pytest.mark.parametrize("vocab", [9, 129280])
def test_greedy_argmax_alone_then_finalize_from_it(vocab):
    """hs_greedy_argmax gives the oracle's argmax (special values included), and
    hs_finalize_accepted with logits=None, reading that argmax, leaves the same state,
    host rows and outputs as the one-call form."""
    import sparse_attention_kv_amd as hs
    from sparse_attention_kv_amd.pipeline import build_hot_state
    rng = np.random.default_rng(vocab + 5)
    B, R, cap, bs, width = 6, 3, 24, 8, 10
    bt = rng.permutation(B * width).astype(np.int32).reshape(B, width)
    seq = rng.integers(cap + R, width * bs, size=B).astype(np.int32)
    pool = rng.standard_normal((B * width * bs, 8)).astype(np.float32)
    init_pos = np.full((B, cap), -1, np.int32)
    init_stamp = np.full((B, cap), -1, np.int32)
    for b in range(B):
        init_pos[b] = rng.choice(int(seq[b]), cap, replace=False)
        init_stamp[b] = rng.integers(0, 30, size=cap)
    gen = torch.Generator().manual_seed(vocab)
    logits = torch.randn(B * R, vocab, generator=gen).to(torch.bfloat16)
    logits[0, :] = float("nan"); logits[1, :] = -float("inf"); logits[2, vocab - 1] = 60.0
    plant = rng.integers(0, vocab, size=B * R)
    logits[torch.arange(3, B * R), torch.from_numpy(plant[3:])] = 40.0
    draft = rng.integers(0, vocab, size=B * R).astype(np.int32)
    for r in range(1, R):
        for b in range(B):
            if rng.random() < 0.7:
                draft[r * B + b] = plant[(r - 1) * B + b]
    new_kv = rng.standard_normal((B * R, 8)).astype(np.float32)
    _, _, am = oracle.greedy_accept(raw(logits), draft, B, R)
    results = []
    for split in (False, True):
        hpool = _pinned(pool)
        gst = build_hot_state(torch.from_numpy(init_pos), torch.from_numpy(init_stamp), to_dev(seq),
                              to_dev(bt), bs, hpool, dev())
        g_am = torch.full((B * R,), -5, dtype=torch.int32, device=dev())
        g_acc = torch.empty((B,), dtype=torch.int32, device=dev())
        g_nxt = torch.empty((B,), dtype=torch.int32, device=dev())
        lg = logits.to(dev())
        log(f"finalize split={split} vocab={vocab}")
        if split:
            hs.hs_greedy_argmax(lg, g_am)
            torch.cuda.synchronize()
            assert np.array_equal(g_am.cpu().numpy(), am), "hs_greedy_argmax"
            hs.hs_finalize_accepted(gst, None, to_dev(draft), torch.from_numpy(new_kv).to(dev()), R,
                                    to_dev(seq), to_dev(bt), bs, 50, g_am, g_acc, g_nxt)
        else:
            hs.hs_finalize_accepted(gst, lg, to_dev(draft), torch.from_numpy(new_kv).to(dev()), R,
                                    to_dev(seq), to_dev(bt), bs, 50, g_am, g_acc, g_nxt)
        torch.cuda.synchronize()
        results.append([t.cpu().clone() for t in (g_am, g_acc, g_nxt, gst.slot_loc, gst.slot_stamp,
                                                  gst.loc_to_hot, gst.hot_kv)] + [hpool.clone()])
    for i, (a, b_) in enumerate(zip(*results)):
        assert torch.equal(a, b_), f"output {i} differs between the one-call and split forms"


def test_attention_identical_on_resident_and_swap_paths():
    """Same rows, same index order, same launch: the paged pool and the hot buffer give
    equal bits."""
    import sparse_attention_kv_amd as hs
    from sparse_attention_kv_amd.pipeline import DecodeStep
    for name, over in (("tiny", {}), ("mtp_swap", dict(num_reqs=4, seq_rule=("const", 5000)))):
        s, w = make(name, **over)
        g = gpu_inputs(s, w)
        from tests.test_gpu_swap import _both_states
        ost, gst, pool = _both_states(s, w, g)
        step = DecodeStep(num_reqs=s.num_reqs, rows_per_req=s.rows_per_req, topk=s.topk,
                          num_heads=s.num_heads, d_qk=s.d_qk, d_v=s.d_v, dtype=w.q.dtype,
                          capacity=s.capacity, device=dev())
        # waves followed by another swap-in run the attention sized for the CUs it leaves
        overlap = step.overlaps(gst, s.tick0)
        log(f"cross-path {name}: swap path")
        step.run_swap(gst, g["topk_pos"], g["req_id"], g["causal_limit"], g["block_table"],
                      s.block_size, g["q"], s.scale, s.tick0)
        torch.cuda.synchronize()
        dev_pool = w.kv_pool.to(dev())
        res = DecodeStep(num_reqs=s.num_reqs, rows_per_req=s.rows_per_req, topk=s.topk,
                         num_heads=s.num_heads, d_qk=s.d_qk, d_v=s.d_v, dtype=w.q.dtype, device=dev())
        # the resident path runs all rows at once; run it per wave so the split plan matches
        B = s.num_reqs
        log(f"cross-path {name}: resident path")
        res.run_resident(g["topk_pos"], g["req_id"], g["causal_limit"], g["block_table"],
                         s.block_size, g["q"], dev_pool, s.scale)
        out_wave = torch.empty_like(res.buf.out)
        for r in range(s.rows_per_req):
            lo, hi = r * B, (r + 1) * B
            ws_b = hs.hs_attn_workspace_bytes(B, s.num_heads, s.d_qk, s.d_v, s.topk, w.q.dtype)
            ws = torch.empty((max(ws_b, 16),), dtype=torch.uint8, device=dev()) if ws_b else None
            cus = step.cus_beside_swap if (overlap and r + 1 < s.rows_per_req) else 256
            hs.hs_sparse_decode_attn_cus(g["q"][lo:hi], dev_pool, res.buf.slots[lo:hi], s.scale,
                                         s.d_v, out_wave[lo:hi], None, ws, cus)
        torch.cuda.synchronize()
        assert torch.equal(out_wave, step.buf.out), name
