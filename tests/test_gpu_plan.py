"""GPU parity of hs_apply_plan: follower caches filled from the leader's swap plan.

Bit-exact against oracle.apply_plan on the GPU leader's plan (itself checked against
oracle.swap_in), and the invariant the plan exists for: every follower's occupied slots
hold their host rows after every wave.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import dev, gpu_inputs, log, make, oracle_resolve, to_dev
from tests.helpers import raw

pytestmark = pytest.mark.gpu


def _follower_pools(pool: np.ndarray, C: int, seed: int) -> np.ndarray:
    """C host pools of the leader's shape with different contents (other layers)."""
    rng = np.random.default_rng(seed)
    if pool.dtype == np.uint16:
        return rng.integers(0, 2 ** 16, size=(C,) + pool.shape, dtype=np.uint16)
    return rng.standard_normal((C,) + pool.shape).astype(np.float32)


def _to_torch_raw(a: np.ndarray, dtype, pinned: bool):
    t = torch.empty(a.shape, dtype=dtype, pin_memory=pinned)
    if dtype == torch.bfloat16:
        t.view(torch.int16).numpy()[...] = a.view(np.int16)
    else:
        t.numpy()[...] = a
    return t


@pytest.mark.parametrize("name,over", [("tiny", {}),
                                        ("mtp_swap", {"seq_rule": ("uniform", 4096, 6144)})])
def test_followers_apply_leader_plan(name, over):
    import sparse_attention_kv_amd as hs
    from sparse_attention_kv_amd.pipeline import build_hot_state
    s, w = make(name, **over)
    g = gpu_inputs(s, w)
    pool = raw(w.kv_pool)
    ost = oracle.build_hot_state(w.init_pos, w.init_stamp, w.seq_len, w.block_table, s.block_size, pool)
    gst = build_hot_state(torch.from_numpy(w.init_pos), torch.from_numpy(w.init_stamp), g["seq_len"],
                          g["block_table"], s.block_size, w.kv_pool, dev())
    torch.cuda.synchronize()
    C = 2
    fpools = _follower_pools(pool, C, seed=5)
    occ0 = np.nonzero(ost.slot_loc.reshape(-1) >= 0)[0]
    fhot = np.zeros((C,) + ost.hot_kv.shape, dtype=pool.dtype)
    for c in range(C):
        fhot[c][occ0] = fpools[c][ost.slot_loc.reshape(-1)[occ0]]
    tdt = torch.bfloat16 if pool.dtype == np.uint16 else torch.float32
    fhot_gpu = _to_torch_raw(fhot, tdt, False).to(dev())
    fpool_pinned = _to_torch_raw(fpools, tdt, True)
    slots, _ = oracle_resolve(s, w)
    B, K = s.num_reqs, s.topk
    for r in range(s.rows_per_req):
        wave = slots[r * B:(r + 1) * B]
        hot = torch.empty((B, K), dtype=torch.int32, device=dev())
        mc = torch.empty((B,), dtype=torch.int32, device=dev())
        mp = torch.empty((B, K), dtype=torch.int32, device=dev())
        wave_d = to_dev(wave)
        log(f"plan {name} wave {r}")
        hs.hs_swap_in(gst, wave_d, s.tick0 + r, hot, mc, mp)
        hs.hs_apply_plan(fhot_gpu, fpool_pinned, wave_d, hot, mc, mp, s.capacity)
        torch.cuda.synchronize()
        oh, omc, omp = oracle.swap_in(ost, wave, s.tick0 + r, pool)
        assert np.array_equal(hot.cpu().numpy(), oh)
        assert np.array_equal(mc.cpu().numpy(), omc)
        assert np.array_equal(mp.cpu().numpy(), omp)
        fhot = oracle.apply_plan(fhot, fpools, wave, oh, omc, omp)
        got = raw(fhot_gpu.cpu()) if tdt == torch.bfloat16 else fhot_gpu.cpu().numpy()
        assert np.array_equal(got.view(np.uint8), fhot.view(np.uint8)), f"{name} wave {r}"
        occ = np.nonzero(ost.slot_loc.reshape(-1) >= 0)[0]
        for c in range(C):
            assert np.array_equal(fhot[c][occ], fpools[c][ost.slot_loc.reshape(-1)[occ]])
        log(f"plan {name} wave {r}: {int(omc.sum())} misses applied to {C} followers")


def test_apply_plan_rejects_bad_arguments():
    import sparse_attention_kv_amd as hs
    hot = torch.zeros((2, 8, 64), dtype=torch.float32, device=dev())
    idx = torch.zeros((2, 4), dtype=torch.int32, device=dev())
    mc = torch.zeros((2,), dtype=torch.int32, device=dev())
    with pytest.raises(ValueError):  # pageable pool
        hs.hs_apply_plan(hot, torch.zeros((2, 16, 64)), idx, idx, mc, idx, 4)
    with pytest.raises(ValueError):  # wrong hot-buffer row count for num_reqs * capacity
        hs.hs_apply_plan(hot, torch.zeros((2, 16, 64), pin_memory=True), idx, idx, mc, idx, 3)
    st = hs._lib.hs_apply_plan(hot.data_ptr(), 0, 16, 2, 2, 4, 256, idx.data_ptr(), 4,
                               idx.data_ptr(), mc.data_ptr(), idx.data_ptr(), None)
    assert st == hs.HS_ERR_INVALID_ARG  # null pool
