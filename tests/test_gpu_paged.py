"""GPU parity of hs_sparse_decode_attn_paged (resolve + attention in one call) against the
oracle's resolve_topk followed by sparse_decode_attn, and against the two-call GPU path.

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


def _paged(q, kv, pos, req, lim, bt, block_size, scale, d_v=512):
    import sparse_attention_kv_amd as hs
    rows, H, D = q.shape
    out = torch.full((rows, H, d_v), float("nan"), dtype=q.dtype, device=dev())
    lse = torch.full((rows, H), float("nan"), dtype=torch.float32, device=dev())
    wsb = hs.hs_attn_workspace_bytes(rows, H, D, d_v, pos.shape[1], q.dtype)
    ws = torch.empty((wsb,), dtype=torch.uint8, device=dev()) if wsb else None
    hs.hs_sparse_decode_attn_paged(q, kv, pos, req, lim, bt, block_size, block_size, scale, d_v,
                                   out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def _two_call(q, kv, pos, req, lim, bt, block_size, scale, d_v=512):
    import sparse_attention_kv_amd as hs
    rows, H, D = q.shape
    slots = torch.empty_like(pos)
    hs.hs_resolve_topk(pos, req, lim, bt, block_size, block_size, slots)
    out = torch.empty((rows, H, d_v), dtype=q.dtype, device=dev())
    lse = torch.empty((rows, H), dtype=torch.float32, device=dev())
    wsb = hs.hs_attn_workspace_bytes(rows, H, D, d_v, pos.shape[1], q.dtype)
    ws = torch.empty((wsb,), dtype=torch.uint8, device=dev()) if wsb else None
    hs.hs_sparse_decode_attn(q, kv, slots, scale, d_v, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def _check_vs_oracle(out, lse, q, kv, slots, scale, what):
    ref, rlse = oracle.sparse_decode_attn(raw(q.cpu()), raw(kv.cpu()), slots, scale, 512)
    assert_close(out_f64(out), ref, BF16_TOL, what)
    g = lse.cpu().double().numpy()
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(g), fin), what + " lse finiteness"
    assert_close(g[fin], rlse[fin], LSE_TOL, what + " lse")


def test_paged_resident_full_matches_oracle_and_two_calls():
    """The resident decode workload at full size (8 rows x 128 heads x top-k 2048)."""
    s, w = make("resident")
    g = gpu_inputs(s, w)
    log("paged attention, resident full size")
    out, lse = _paged(g["q"], w.kv_pool, g["topk_pos"], g["req_id"], g["causal_limit"],
                      g["block_table"], s.block_size, s.scale)
    slots, _ = oracle_resolve(s, w)
    _check_vs_oracle(out, lse, g["q"], w.kv_pool, slots, s.scale, "paged resident")
    out2, lse2 = _two_call(g["q"], w.kv_pool, g["topk_pos"], g["req_id"], g["causal_limit"],
                           g["block_table"], s.block_size, s.scale)
    assert torch.equal(out, out2)
    assert torch.equal(lse, lse2)


@pytest.mark.parametrize("num_reqs,topk", [(3, 300), (8, 2048), (40, 777)])
def test_paged_fail_closed_cases(num_reqs, topk):
    """Positions past the causal limit or negative, an out-of-range request id, unmapped
    pages and a short block-table row select nothing; 40 requests take the 64-head kernel."""
    import sparse_attention_kv_amd as hs
    s, w = make("resident", num_reqs=num_reqs, topk=topk, seq_rule=("uniform", 900, 1500))
    assert hs.hs_attn_plan_info(s.rows, s.num_heads, 576, 512, topk, torch.bfloat16)[0] == \
        (64 if num_reqs == 40 else 32)
    rng = np.random.default_rng(num_reqs * 1000 + topk)
    pos = w.topk_pos.copy()
    lim = w.causal_limit.copy()
    req = w.req_id.copy()
    bt = w.block_table.copy()
    rows = pos.shape[0]
    # scatter bad positions: negative, at the limit, far past it
    m = rng.random(pos.shape) < 0.05
    pos[m] = rng.choice([-1, -7, 10 ** 6], size=int(m.sum()))
    pos[0, : topk // 2] = lim[0]                 # exactly at the (exclusive) limit
    lim[1] = lim[1] // 3                          # shorter causal limit
    req[2 % rows] = num_reqs + 5                  # request id out of range: empty row
    bt[0, 1::3] = -1                              # unmapped pages of request 0
    args = [to_dev(a) for a in (pos, req, lim, bt)]
    q = w.q.to(dev())
    log(f"paged attention fail-closed: {num_reqs} requests, top-k {topk}")
    out, lse = _paged(q, w.kv_pool, *args, s.block_size, s.scale)
    slots, _ = oracle.resolve_topk(pos, req, lim, bt, s.block_size, s.block_size, num_reqs)
    assert (slots[2 % rows] == -1).all()
    _check_vs_oracle(out, lse, q, w.kv_pool, slots, s.scale, f"paged fail-closed {num_reqs}x{topk}")
    out2, lse2 = _two_call(q, w.kv_pool, *args, s.block_size, s.scale)
    assert torch.equal(out, out2)
    assert torch.equal(lse, lse2)


def test_prepared_call_matches_plain_call_and_follows_input_changes():
    """PagedAttnCall forwards the same arguments: bit-identical to the plain call, and a
    change to the inputs in place is seen by the next call."""
    import sparse_attention_kv_amd as hs
    s, w = make("resident", num_reqs=3, topk=500, seq_rule=("uniform", 900, 1500))
    g = gpu_inputs(s, w)
    q = g["q"]
    rows, H, D = q.shape
    wsb = hs.hs_attn_workspace_bytes(rows, H, D, 512, g["topk_pos"].shape[1], q.dtype)
    ws = torch.empty((wsb,), dtype=torch.uint8, device=dev()) if wsb else None
    out = torch.empty((rows, H, 512), dtype=q.dtype, device=dev())
    lse = torch.empty((rows, H), dtype=torch.float32, device=dev())
    call = hs.PagedAttnCall(q, w.kv_pool, g["topk_pos"], g["req_id"], g["causal_limit"],
                            g["block_table"], s.block_size, s.block_size, s.scale, 512, out, lse, ws)
    log("prepared paged call")
    for step in range(2):
        call()
        torch.cuda.synchronize()
        ref_out, ref_lse = _paged(q, w.kv_pool, g["topk_pos"], g["req_id"], g["causal_limit"],
                                  g["block_table"], s.block_size, s.scale)
        assert torch.equal(out, ref_out), step
        assert torch.equal(lse, ref_lse), step
        q.mul_(-0.5)  # new query values at the same address


def test_paged_rejects_fp32_and_bad_sizes():
    import sparse_attention_kv_amd as hs
    q = torch.zeros((2, 4, 64), dtype=torch.float32, device=dev())
    kv = torch.zeros((32, 64), dtype=torch.float32, device=dev())
    pos = torch.zeros((2, 8), dtype=torch.int32, device=dev())
    req = torch.zeros((2,), dtype=torch.int32, device=dev())
    lim = torch.full((2,), 8, dtype=torch.int32, device=dev())
    bt = torch.zeros((1, 2), dtype=torch.int32, device=dev())
    out = torch.zeros((2, 4, 48), dtype=torch.float32, device=dev())
    with pytest.raises(hs.HsError) as e:
        hs.hs_sparse_decode_attn_paged(q, kv, pos, req, lim, bt, 16, 16, 0.125, 48, out)
    assert e.value.status == hs.HS_ERR_UNSUPPORTED
    with pytest.raises(hs.HsError) as e:
        hs.hs_sparse_decode_attn_paged(q, kv, pos, req, lim, bt, 0, 16, 0.125, 48, out)
    assert e.value.status == hs.HS_ERR_INVALID_ARG
