"""GPU parity of per-request residency: hs_sparse_decode_attn_mixed against the oracle on
every kernel path, and a whole mixed step (DecodeStep.run_mixed) against the oracle.

Tolerances as in test_gpu_attn: bf16 |gpu - ref| <= 2e-2 + 1e-2 |ref|; LSE 1e-3 + 1e-4 |ref|.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import BF16_TOL, assert_close, dev, gpu_inputs, log, make, oracle_resolve, out_f64, to_dev
from tests.helpers import raw

pytestmark = pytest.mark.gpu
LSE_TOL = (1e-3, 1e-4)


def _rand_bf16(shape, seed):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(shape, generator=gen).to(torch.bfloat16).to(dev())


def _mixed(q, kv_a, ia, kv_b, ib, sel, scale=1 / 24, max_cus=None):
    import sparse_attention_kv_amd as hs
    rows, H, D = q.shape
    out = torch.full((rows, H, 512), float("nan"), dtype=q.dtype, device=dev())
    lse = torch.full((rows, H), float("nan"), dtype=torch.float32, device=dev())
    wsb = hs.hs_attn_workspace_bytes(rows, H, D, 512, ia.shape[1], q.dtype)
    ws = torch.empty((wsb,), dtype=torch.uint8, device=dev()) if wsb else None
    hs.hs_sparse_decode_attn_mixed(q, kv_a, ia, kv_b, ib, sel, scale, 512, out, lse, ws,
                                   max_cus=max_cus)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("rows,topk,sample,cus", [(8, 2048, None, None), (40, 700, None, None),
                                                  (256, 600, [0, 1, 2, 3, 100, 255], None),
                                                  (8, 2048, None, 64), (128, 900, None, 128)])
def test_mixed_attention_matches_oracle(rows, topk, sample, cus):
    """8 rows take the 32-head kernel, 40 the 64-head one, 256 the 128-head one; with `cus`
    the call is planned for that many compute units (8 rows: the 64-head kernel, 4 splits;
    128 rows: the 128-head kernel, one split)."""
    import sparse_attention_kv_amd as hs
    H = 128
    if cus is None:
        assert hs.hs_attn_plan_info(rows, H, 576, 512, topk, torch.bfloat16)[0] == {8: 32, 40: 64, 256: 128}[rows]
    else:
        assert hs.hs_attn_plan_info_cus(rows, H, 576, 512, topk, torch.bfloat16, cus) == {64: (64, 4), 128: (128, 1)}[cus]
    rng = np.random.default_rng(rows)
    q = _rand_bf16((rows, H, 576), rows)
    kv_a = _rand_bf16((3000, 576), rows + 1)
    kv_b = _rand_bf16((2500, 576), rows + 2)
    ia = np.stack([rng.choice(3000, topk, replace=False) for _ in range(rows)]).astype(np.int32)
    ib = np.stack([rng.choice(2500, topk, replace=False) for _ in range(rows)]).astype(np.int32)
    ia[1, : topk // 3] = -1
    ib[2, rng.random(topk) < 0.2] = 2500 + 5  # past kv_b end
    sel = (rng.random(rows) < 0.5).astype(np.int32)
    sel[:4] = [0, 1, 1, 0]
    log(f"mixed attention rows={rows} topk={topk} cus={cus}")
    out, lse = _mixed(q, kv_a, to_dev(ia), kv_b, to_dev(ib), to_dev(sel), max_cus=cus)
    rs = list(range(rows)) if sample is None else sample
    ref, rlse = oracle.sparse_decode_attn_mixed(raw(q.cpu()[rs]), raw(kv_a.cpu()), ia[rs],
                                                raw(kv_b.cpu()), ib[rs], sel[rs], 1 / 24, 512)
    assert_close(out_f64(out[rs]), ref, BF16_TOL, "mixed attention")
    g = lse[rs].cpu().double().numpy()
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(g), fin)
    assert_close(g[fin], rlse[fin], LSE_TOL, "mixed lse")


def test_mixed_step_matches_oracle():
    """Requests with a reclaimed page swap in; the rest read a device copy of the pool.
    Every row must equal attention over the host pool (same rows either way), and the hot
    state must follow the oracle's swaps of the non-resident requests only."""
    import sparse_attention_kv_amd as hs
    from sparse_attention_kv_amd.pipeline import DecodeStep, ResidencyTracker, build_hot_state
    s, w = make("mtp_swap", num_reqs=8, seq_rule=("uniform", 3000, 5000))
    g = gpu_inputs(s, w)
    pool = raw(w.kv_pool)
    ost = oracle.build_hot_state(w.init_pos, w.init_stamp, w.seq_len, w.block_table, s.block_size, pool)
    gst = build_hot_state(torch.from_numpy(w.init_pos), torch.from_numpy(w.init_stamp), g["seq_len"],
                          g["block_table"], s.block_size, w.kv_pool, dev())
    dev_pool = w.kv_pool.to(dev())  # the resident pool: same rows as the host pool
    tracker = ResidencyTracker(w.block_table, w.seq_len, s.block_size)
    for b in (1, 4, 6):  # reclaim one old page of three requests
        page = [p for (bb, p) in tracker.reclaimable_pages() if bb == b][0]
        tracker.release_resident_page(b, page)
    resident = tracker.fully_resident()
    assert resident.tolist().count(False) == 3
    req_res, req_swap, sel = tracker.row_inputs(w.req_id, dev())
    step = DecodeStep(num_reqs=s.num_reqs, rows_per_req=s.rows_per_req, topk=s.topk,
                      num_heads=s.num_heads, d_qk=s.d_qk, d_v=s.d_v, dtype=torch.bfloat16,
                      capacity=s.capacity, mixed=True, device=dev())
    q = w.q.to(dev())
    log("mixed step")
    step.run_mixed(gst, g["topk_pos"], req_res, req_swap, sel, g["causal_limit"],
                   tracker.table(dev()), g["block_table"], s.block_size, q, dev_pool, s.scale,
                   s.tick0)
    torch.cuda.synchronize()
    slots, _ = oracle_resolve(s, w)
    ref, rlse = oracle.sparse_decode_attn(raw(q.cpu()), pool, slots, s.scale, 512)
    assert_close(out_f64(step.buf.out), ref, BF16_TOL, "mixed step")
    B = s.num_reqs
    for r in range(s.rows_per_req):
        wave = slots[r * B:(r + 1) * B].copy()
        wave[resident] = -1  # resident requests do not swap
        oracle.swap_in(ost, wave, s.tick0 + r, pool)
    assert np.array_equal(gst.slot_loc.cpu().numpy(), ost.slot_loc)
    assert np.array_equal(gst.slot_stamp.cpu().numpy(), ost.slot_stamp)
    assert np.array_equal(gst.loc_to_hot.cpu().numpy(), ost.loc_to_hot)
    mc = step.buf.miss_count.cpu().numpy()
    assert (mc[:, resident] == 0).all() and mc[:, ~resident].sum() > 0


def test_mixed_rejects_fp32():
    import sparse_attention_kv_amd as hs
    q = torch.zeros((2, 4, 64), dtype=torch.float32, device=dev())
    kv = torch.zeros((8, 64), dtype=torch.float32, device=dev())
    idx = torch.zeros((2, 4), dtype=torch.int32, device=dev())
    sel = torch.zeros((2,), dtype=torch.int32, device=dev())
    out = torch.zeros((2, 4, 48), dtype=torch.float32, device=dev())
    with pytest.raises(hs.HsError) as e:
        hs.hs_sparse_decode_attn_mixed(q, kv, idx, kv, idx, sel, 0.1, 48, out)
    assert e.value.status == hs.HS_ERR_UNSUPPORTED
