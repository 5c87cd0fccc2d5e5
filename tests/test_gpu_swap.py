"""GPU parity of hs_swap_in and of a whole swap-path decode step against the oracle.

Bit-exact: hot indices, miss counts and positions, slot_loc, slot_stamp, loc_to_hot and
the hot-buffer rows of every occupied slot, after every wave.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import (BF16_TOL, F32_TOL, assert_close, dev, gpu_inputs, log, make,
                             oracle_resolve, out_f64, to_dev)
from tests.helpers import check_state_invariants, raw

pytestmark = pytest.mark.gpu


def _both_states(s, w, g):
    from sparse_attention_kv_amd.pipeline import build_hot_state
    pool = raw(w.kv_pool)
    ost = oracle.build_hot_state(w.init_pos, w.init_stamp, w.seq_len, w.block_table, s.block_size, pool)
    gst = build_hot_state(torch.from_numpy(w.init_pos), torch.from_numpy(w.init_stamp), g["seq_len"],
                          g["block_table"], s.block_size, w.kv_pool, dev())
    torch.cuda.synchronize()
    return ost, gst, pool


def _compare_state(ost, gst, what, with_kv=True):
    assert np.array_equal(gst.slot_loc.cpu().numpy(), ost.slot_loc), what + " slot_loc"
    assert np.array_equal(gst.slot_stamp.cpu().numpy(), ost.slot_stamp), what + " slot_stamp"
    assert np.array_equal(gst.loc_to_hot.cpu().numpy(), ost.loc_to_hot), what + " loc_to_hot"
    if with_kv:
        occ = np.nonzero(ost.slot_loc.reshape(-1) >= 0)[0]
        got = raw(gst.hot_kv.cpu())
        assert np.array_equal(got[occ], ost.hot_kv[occ]), what + " hot_kv"


@pytest.mark.parametrize("name", ["tiny", "mtp_swap", "long", "mixed_finalize"])
def test_swap_waves_bit_exact(name):
    _swap_waves(name)


@pytest.mark.parametrize("over", [
    # the library's limits: 16384 slots (16 per thread), top-k 4096 (4 entries per thread)
    dict(num_reqs=3, capacity=16384, topk=4096, seq_rule=("const", 30000)),
    # sizes that are no multiple of the workgroup: 5 slots and 3 entries per thread, the
    # last threads partly empty
    dict(num_reqs=5, capacity=5000, topk=3000, seq_rule=("uniform", 6000, 9000)),
], ids=["max_capacity_and_topk", "ragged_capacity_and_topk"])
def test_swap_waves_bit_exact_at_size_limits(over):
    """Full hot buffers, so every miss evicts an LRU victim."""
    _swap_waves("mtp_swap", **over)


def _swap_waves(name, **over):
    import sparse_attention_kv_amd as hs
    s, w = make(name, **over)
    g = gpu_inputs(s, w)
    ost, gst, pool = _both_states(s, w, g)
    _compare_state(ost, gst, f"{name} initial state")
    slots, _ = oracle_resolve(s, w)
    B, K = s.num_reqs, s.topk
    for r in range(s.rows_per_req):
        wave = slots[r * B:(r + 1) * B]
        hot = torch.full((B, K), 7, dtype=torch.int32, device=dev())
        mc = torch.full((B,), 7, dtype=torch.int32, device=dev())
        mp = torch.full((B, K), 7, dtype=torch.int32, device=dev())
        log(f"swap {name} wave {r}")
        hs.hs_swap_in(gst, to_dev(wave), s.tick0 + r, hot, mc, mp)
        torch.cuda.synchronize()
        oh, omc, omp = oracle.swap_in(ost, wave, s.tick0 + r, pool)
        assert np.array_equal(hot.cpu().numpy(), oh), f"{name} wave {r} hot_idx"
        assert np.array_equal(mc.cpu().numpy(), omc), f"{name} wave {r} miss_count"
        assert np.array_equal(mp.cpu().numpy(), omp), f"{name} wave {r} miss_pos"
        # hot-buffer bytes after every wave on tiny and the MTP workload, after the last
        # wave on the larger ones
        _compare_state(ost, gst, f"{name} wave {r}",
                       with_kv=(r == s.rows_per_req - 1 or name in ("tiny", "mtp_swap")))
        log(f"swap {name} wave {r}: misses/row {omc.mean():.1f} hit rate "
            f"{1 - omc.sum() / max(1, (wave >= 0).sum()):.3f}")
    check_state_invariants(ost, pool)


def test_swap_capacity_error_leaves_state():
    import sparse_attention_kv_amd as hs
    s, w = make("tiny")
    g = gpu_inputs(s, w)
    ost, gst, pool = _both_states(s, w, g)
    before = [t.clone() for t in (gst.slot_loc, gst.slot_stamp, gst.loc_to_hot, gst.hot_kv)]
    wide = torch.zeros((s.num_reqs, s.capacity + 1), dtype=torch.int32, device=dev())
    out = torch.empty_like(wide)
    mc = torch.empty((s.num_reqs,), dtype=torch.int32, device=dev())
    with pytest.raises(hs.HsError) as e:
        hs.hs_swap_in(gst, wide, 5, out, mc)
    assert e.value.status == hs.HS_ERR_CAPACITY
    torch.cuda.synchronize()
    after = (gst.slot_loc, gst.slot_stamp, gst.loc_to_hot, gst.hot_kv)
    assert all(torch.equal(a, b) for a, b in zip(before, after))


def test_swap_rejects_pageable_host_pool():
    import sparse_attention_kv_amd as hs
    s, w = make("tiny")
    g = gpu_inputs(s, w)
    _, gst, _ = _both_states(s, w, g)
    gst.host_pool = w.kv_pool.clone()     # ordinary (pageable) host memory
    assert not gst.host_pool.is_pinned()
    out = torch.empty((s.num_reqs, s.topk), dtype=torch.int32, device=dev())
    mc = torch.empty((s.num_reqs,), dtype=torch.int32, device=dev())
    with pytest.raises(hs.HsError) as e:
        hs.hs_swap_in(gst, torch.zeros_like(out), 5, out, mc)
    assert e.value.status == hs.HS_ERR_INVALID_ARG


def _pipeline_case(name, sample_rows_per_wave=6, **over):
    """Whole step through DecodeStep.run_swap (copy stream overlapped with attention)."""
    from sparse_attention_kv_amd.pipeline import DecodeStep
    s, w = make(name, **over)
    g = gpu_inputs(s, w)
    ost, gst, pool = _both_states(s, w, g)
    B, R = s.num_reqs, s.rows_per_req
    fin = None
    snap = None
    if s.finalize:
        # host rows the finalize step may overwrite: the verify rows' positions
        locs = np.concatenate([oracle.resolve_topk(
            (w.seq_len[b] - R + np.arange(R, dtype=np.int32))[None, :], np.array([b], np.int32),
            np.array([w.seq_len[b]], np.int32), w.block_table, s.block_size, s.block_size, B)[0][0]
            for b in range(B)])
        locs = locs[locs >= 0]
        snap = (locs, w.kv_pool[torch.from_numpy(locs).long()].clone())
        fin = dict(logits=w.logits.to(dev()), draft_ids=to_dev(w.draft_ids),
                   new_kv=w.new_kv.to(dev()), seq_len=g["seq_len"])
        # the draft model's context cache takes the accepted prefix too (its own rows)
        crng = np.random.default_rng(77)
        cbs, cpages = 16, 8
        ctx = dict(bt=crng.permutation(B * cpages).reshape(B, cpages).astype(np.int32),
                   len=crng.integers(0, cpages * cbs - R, size=B).astype(np.int32),
                   rows=raw(w.new_kv)[crng.permutation(B * R)],
                   cache=raw(w.new_kv)[crng.integers(0, B * R, size=B * cpages * cbs)])
        tdt = w.new_kv.dtype

        def _t(a):
            t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
            return (t.view(tdt) if a.dtype == np.uint16 else t).to(dev())
        fin["dflash"] = dict(ctx_cache=_t(ctx["cache"]), ctx_block_table=to_dev(ctx["bt"]),
                             ctx_len=to_dev(ctx["len"]), ctx_rows=_t(ctx["rows"]), block_size=cbs)
    step = DecodeStep(num_reqs=B, rows_per_req=R, topk=s.topk, num_heads=s.num_heads, d_qk=s.d_qk,
                      d_v=s.d_v, dtype=w.q.dtype, capacity=s.capacity, finalize=s.finalize,
                      want_miss_pos=True, device=dev())
    log(f"pipeline {name}: run_swap")
    step.run_swap(gst, g["topk_pos"], g["req_id"], g["causal_limit"], g["block_table"],
                  s.block_size, g["q"], s.scale, s.tick0, finalize=fin)
    torch.cuda.synchronize()
    log(f"pipeline {name}: oracle")
    gpu_fin_rows = None
    if snap is not None:
        locs, orig = snap
        gpu_fin_rows = w.kv_pool[torch.from_numpy(locs).long()].clone()
        w.kv_pool[torch.from_numpy(locs).long()] = orig        # oracle starts from the original rows
    slots, valid = oracle_resolve(s, w)
    assert np.array_equal(step.buf.slots.cpu().numpy(), slots)
    assert np.array_equal(step.buf.valid.cpu().numpy(), valid)
    hot_all = np.empty_like(slots)
    for r in range(R):
        oh, omc, omp = oracle.swap_in(ost, slots[r * B:(r + 1) * B], s.tick0 + r, pool)
        hot_all[r * B:(r + 1) * B] = oh
        assert np.array_equal(step.buf.miss_count[r].cpu().numpy(), omc)
        assert np.array_equal(step.buf.miss_pos[r * B:(r + 1) * B].cpu().numpy(), omp)
    assert np.array_equal(step.buf.hot_idx.cpu().numpy(), hot_all)
    # attention against the oracle over the host pool: every row of the first wave (it runs
    # while the second wave's swap is in flight), sampled rows of the others
    rng = np.random.default_rng(0)
    q_raw = raw(w.q)
    sample = np.concatenate([np.arange(B)] + [r * B + rng.choice(B, min(B, sample_rows_per_wave), replace=False)
                                              for r in range(1, R)])
    ref, rlse = oracle.sparse_decode_attn(q_raw[sample], pool, slots[sample], s.scale, s.d_v)
    tol = F32_TOL if s.dtype == "f32" else BF16_TOL
    assert_close(out_f64(step.buf.out[torch.from_numpy(sample).to(dev())]), ref, tol, f"{name} attention")
    if s.finalize:
        acc, nxt, am = oracle.greedy_accept(raw(w.logits), w.draft_ids, B, R)
        assert np.array_equal(step.buf.argmax.cpu().numpy(), am)
        assert np.array_equal(step.buf.accept_len.cpu().numpy(), acc)
        assert np.array_equal(step.buf.next_token.cpu().numpy(), nxt)
        oracle.finalize_accepted(ost, pool, raw(w.new_kv), acc, w.seq_len, w.block_table,
                                 s.block_size, R, s.tick0 + R)
        locs, _ = snap
        assert np.array_equal(raw(gpu_fin_rows), pool[locs]), "host rows after finalize"
        d = fin["dflash"]
        ref_cache, ref_len = oracle.append_accepted(ctx["cache"], ctx["bt"], ctx["len"], ctx["rows"],
                                                    acc, R, cbs, cbs)
        got_cache = d["ctx_cache"].cpu()
        got_cache = raw(got_cache) if got_cache.dtype == torch.bfloat16 else got_cache.numpy()
        assert np.array_equal(got_cache, ref_cache), "draft-model context cache"
        assert np.array_equal(d["ctx_len"].cpu().numpy(), ref_len), "draft-model context length"
        log(f"finalize {name}: accept-length histogram {np.bincount(acc, minlength=R).tolist()}")
    _compare_state(ost, gst, f"{name} after step")
    check_state_invariants(ost, pool)


@pytest.mark.parametrize("name", ["tiny", "mtp_swap", "long"])
def test_pipeline_step(name):
    _pipeline_case(name)


def test_pipeline_step_with_finalize_full():
    _pipeline_case("mixed_finalize", sample_rows_per_wave=4)


# The finalize step at other shapes: other batch sizes, verify-row counts, top-k and seeds;
# hot buffers of at least 2 x top-k (waves overlapped, the attention beside each swap-in
# planned for the CUs it leaves free) and of less (waves serialised).
@pytest.mark.parametrize("over", [
    dict(index=10, num_reqs=12, rows_per_req=4, topk=512, capacity=1024, bt_stride=256,
         seq_rule=("uniform", 600, 16000), vocab=1000),
    dict(index=11, num_reqs=24, rows_per_req=2, topk=300, capacity=500, bt_stride=128,
         seq_rule=("loguniform", 200, 8000), vocab=4000),
    dict(index=12, num_reqs=40, rows_per_req=3, topk=2048, capacity=4096, bt_stride=512,
         seq_rule=("loguniform", 1024, 32768), vocab=2000),
], ids=["12x4-k512", "24x2-k300-serial", "40x3-k2048"])
def test_pipeline_step_with_finalize_varied(over):
    _pipeline_case("mixed_finalize", sample_rows_per_wave=8, **over)


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("mtp_swap", {"num_reqs": 3, "seq_rule": ("const", 6000), "capacity": 1024, "topk": 256}),
], ids=["tiny", "mtp_small"])
def test_swap_duplicate_rows_in_a_request(name, over):
    """Rows repeated within a request (top-k sets never do this; the call still defines it):
    each copy of a miss takes its own victim, an eviction clears a map entry only while it
    names the evicted slot, and the map names a repeated row's last install.  Hot indices,
    miss lists, slot_loc, stamps, loc_to_hot and the hot rows match the oracle bit for bit
    after every call, with no state carried over from the device."""
    import sparse_attention_kv_amd as hs
    from tests.helpers import check_state_weak, with_duplicates
    s, w = make(name, **over)
    g = gpu_inputs(s, w)
    ost, gst, pool = _both_states(s, w, g)
    slots, _ = oracle_resolve(s, w)
    B, K = s.num_reqs, s.topk
    stale_evictions = 0
    # wave 0 comes back after every other wave: rows then sit in slots the map no longer
    # names, and evicting such a slot must leave the row's live mapping alone
    sched = [r for k in range(s.rows_per_req) for r in (k, 0)]
    for t, r in enumerate(sched):
        wave = with_duplicates(slots[r * B:(r + 1) * B])
        before = ost.copy()
        hot = torch.full((B, K), 7, dtype=torch.int32, device=dev())
        mc = torch.full((B,), 7, dtype=torch.int32, device=dev())
        mp = torch.full((B, K), 7, dtype=torch.int32, device=dev())
        log(f"swap duplicates {name} call {t} (wave {r})")
        hs.hs_swap_in(gst, to_dev(wave), s.tick0 + t, hot, mc, mp)
        torch.cuda.synchronize()
        oh, omc, omp = oracle.swap_in(ost, wave, s.tick0 + t, pool)
        assert np.array_equal(hot.cpu().numpy(), oh), f"{name} call {t} hot_idx"
        assert np.array_equal(mc.cpu().numpy(), omc), f"{name} call {t} miss_count"
        assert np.array_equal(mp.cpu().numpy(), omp), f"{name} call {t} miss_pos"
        _compare_state(ost, gst, f"{name} call {t}")
        check_state_weak(ost, pool)
        # evicted slots whose old row the map named elsewhere (stale copies)
        held = before.slot_loc.reshape(-1)
        for b in range(B):
            for m in range(omc[b]):
                gslot = int(oh[b, omp[b, m]])
                old = int(held[gslot])
                if old >= 0 and before.loc_to_hot[old] != gslot:
                    stale_evictions += 1
    log(f"swap duplicates {name}: {stale_evictions} evictions of stale copies")
    if name == "tiny":
        assert stale_evictions > 0


def _next_step_positions(w, s, rng, keep_frac=0.5):
    """Top-k positions of a following step: per row, a random half of this step's set plus
    fresh distinct positions below the same causal limit (top-k sets stay distinct)."""
    out = np.full_like(w.topk_pos, -1)
    K = s.topk
    for i in range(out.shape[0]):
        c = int(w.causal_limit[i])
        prev = w.topk_pos[i][w.topk_pos[i] >= 0]
        keep = rng.choice(prev, min(len(prev), int(K * keep_frac)), replace=False)
        rest = np.setdiff1d(np.arange(c), keep)
        fresh = rng.choice(rest, min(K - len(keep), len(rest)), replace=False)
        row = rng.permutation(np.concatenate([keep, fresh]))
        out[i, :len(row)] = row
    return out.astype(np.int32)


@pytest.mark.parametrize("second_tick", ["after", "stale"])
def test_pipeline_two_consecutive_steps(second_tick):
    """Two decode steps on one hot state.  With the second step's first tick above every
    stamp of the first ("after": tick0 + R + 1) the pipeline overlaps each wave's swap with
    the previous wave's attention; with a tick reused ("stale": tick0 again) it must fall
    back to waiting for the previous wave, since victims may then be that wave's slots.
    Both steps are compared with the oracle: hot indices, miss lists, state, hot-buffer
    bytes, and attention on every row."""
    from sparse_attention_kv_amd.pipeline import DecodeStep
    s, w = make("mtp_swap", num_reqs=8)
    g = gpu_inputs(s, w)
    ost, gst, pool = _both_states(s, w, g)
    B, R = s.num_reqs, s.rows_per_req
    step = DecodeStep(num_reqs=B, rows_per_req=R, topk=s.topk, num_heads=s.num_heads, d_qk=s.d_qk,
                      d_v=s.d_v, dtype=w.q.dtype, capacity=s.capacity, want_miss_pos=True,
                      device=dev())
    rng = np.random.default_rng(31)
    pos2 = _next_step_positions(w, s, rng)
    tick2 = s.tick0 + R + 1 if second_tick == "after" else s.tick0
    for t, (pos, tick) in enumerate(((w.topk_pos, s.tick0), (pos2, tick2))):
        expect_overlap = t == 0 or second_tick == "after"
        assert step.overlaps(gst, tick) == expect_overlap
        log(f"two steps ({second_tick}): step {t} tick {tick} overlap {expect_overlap}")
        step.run_swap(gst, to_dev(pos), g["req_id"], g["causal_limit"], g["block_table"],
                      s.block_size, g["q"], s.scale, tick)
        torch.cuda.synchronize()
        assert gst.max_stamp == tick + R - 1
        slots, _ = oracle.resolve_topk(pos, w.req_id, w.causal_limit, w.block_table, s.block_size,
                                       s.block_size, B)
        assert np.array_equal(step.buf.slots.cpu().numpy(), slots)
        for r in range(R):
            oh, omc, omp = oracle.swap_in(ost, slots[r * B:(r + 1) * B], tick + r, pool)
            assert np.array_equal(step.buf.hot_idx[r * B:(r + 1) * B].cpu().numpy(), oh), (t, r)
            assert np.array_equal(step.buf.miss_count[r].cpu().numpy(), omc), (t, r)
            assert np.array_equal(step.buf.miss_pos[r * B:(r + 1) * B].cpu().numpy(), omp), (t, r)
        _compare_state(ost, gst, f"two steps ({second_tick}) after step {t}")
        ref, _ = oracle.sparse_decode_attn(raw(w.q), pool, slots, s.scale, s.d_v)
        assert_close(out_f64(step.buf.out), ref, BF16_TOL, f"two steps ({second_tick}) step {t}")
        check_state_invariants(ost, pool)
