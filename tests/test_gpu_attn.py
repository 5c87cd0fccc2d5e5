"""GPU parity of hs_sparse_decode_attn against the oracle (float64).

bf16 path: |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise; fp32 path: 1e-5 + 1e-5 |ref|.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import (BF16_TOL, F32_TOL, assert_close, dev, gpu_inputs, log, make,
                             oracle_resolve, out_f64, to_dev)
from tests.helpers import raw

pytestmark = pytest.mark.gpu
LSE_TOL = (1e-3, 1e-4)


def _attn(q, kv, idx, scale, d_v, lse=True):
    import sparse_attention_kv_amd as hs
    rows, H, _ = q.shape
    out = torch.full((rows, H, d_v), float("nan"), dtype=q.dtype, device=dev())
    l = torch.full((rows, H), float("nan"), dtype=torch.float32, device=dev()) if lse else None
    ws_bytes = hs.hs_attn_workspace_bytes(rows, H, q.shape[2], d_v, idx.shape[1], q.dtype)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev()) if ws_bytes else None
    hs.hs_sparse_decode_attn(q, kv, idx, scale, d_v, out, l, ws)
    torch.cuda.synchronize()
    return out, l


def _check(q, kv, idx, scale, d_v, tol, what, lse_check=True):
    log(f"attn {what}: rows={q.shape[0]} H={q.shape[1]} topk={idx.shape[1]} kv_rows={kv.shape[0]}")
    out, lse = _attn(q, kv, idx, scale, d_v)
    ref, rlse = oracle.sparse_decode_attn(raw(q.cpu()), raw(kv.cpu()), idx.cpu().numpy(), scale, d_v)
    assert_close(out_f64(out), ref, tol, what)
    if lse_check:
        g = lse.cpu().double().numpy()
        fin = np.isfinite(rlse)
        assert np.array_equal(np.isfinite(g), fin), what
        assert_close(g[fin], rlse[fin], LSE_TOL, what + " lse")
    return out, lse


def test_attn_tiny_f32():
    s, w = make("tiny")
    g = gpu_inputs(s, w)
    ref_slots, _ = oracle_resolve(s, w)
    kv = w.kv_pool.to(dev())
    _check(g["q"], kv, to_dev(ref_slots), s.scale, s.d_v, F32_TOL, "tiny f32")


def test_attn_resident_full_bf16():
    """The resident decode workload at full size: 8 rows x 128 heads x top-k 2048."""
    s, w = make("resident")
    g = gpu_inputs(s, w)
    ref_slots, _ = oracle_resolve(s, w)
    _check(g["q"], w.kv_pool, to_dev(ref_slots), s.scale, s.d_v, BF16_TOL, "resident full")


def _kernel(rows, H, topk):
    """Heads per workgroup of the bf16 kernel the planner picks for these sizes."""
    import sparse_attention_kv_amd as hs
    return hs.hs_attn_plan_info(rows, H, 576, 512, topk, torch.bfloat16)[0]


def _rand_bf16(shape, seed):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn(shape, generator=gen).to(torch.bfloat16).to(dev())


@pytest.mark.parametrize("topk", [1, 16, 63, 64, 65, 200, 2047, 2048, 3000, 4500])
def test_attn_bf16_ragged_topk(topk):
    rows, H, kv_rows = 3, 32, 5000
    rng = np.random.default_rng(topk)
    q = _rand_bf16((rows, H, 576), topk)
    kv = _rand_bf16((kv_rows, 576), topk + 1)
    idx = np.stack([rng.choice(kv_rows, topk, replace=False) for _ in range(rows)]).astype(np.int32)
    # scatter some padding and out-of-range entries through the rows
    idx[1, rng.random(topk) < 0.3] = -1
    idx[2, rng.random(topk) < 0.2] = kv_rows + 7
    _check(q, kv, to_dev(idx), 1 / 24, 512, BF16_TOL, f"ragged topk={topk}")


def test_attn_bf16_empty_single_duplicate_and_zero_query():
    rows, H, kv_rows, topk = 5, 64, 300, 96
    q = _rand_bf16((rows, H, 576), 11)
    kv = _rand_bf16((kv_rows, 576), 12)
    idx = np.full((rows, topk), -1, np.int32)
    idx[1, 50] = 17                       # a single selected key
    idx[2, :40] = np.arange(40)           # 40 keys listed twice: duplicates count twice
    idx[2, 40:80] = np.arange(40)
    idx[3, :96] = np.arange(100, 196)
    q[4] = 0                              # zero query: uniform weights
    idx[4, :90] = np.arange(200, 290)
    out, lse = _check(q, kv, to_dev(idx), 1 / 24, 512, BF16_TOL, "edge rows")
    o = out.cpu()
    assert (o[0] == 0).all() and torch.isneginf(lse[0].cpu()).all()        # empty row
    assert torch.equal(o[1], kv[17, :512].cpu().expand(H, 512))           # p = 1 exactly
    mean = kv[200:290, :512].double().mean(0).cpu()
    assert_close(o[4].double().numpy(), mean.expand(H, 512).numpy(), BF16_TOL, "zero query mean")


def test_attn_split_and_unsplit_agree():
    """One row alone (key-split + combine) vs the same row in a large batch (no split)."""
    import sparse_attention_kv_amd as hs
    H, kv_rows, topk, big_rows = 128, 20000, 2048, 256
    assert hs.hs_attn_workspace_bytes(1, H, 576, 512, topk, torch.bfloat16) > 0
    assert hs.hs_attn_workspace_bytes(big_rows, H, 576, 512, topk, torch.bfloat16) == 0
    q = _rand_bf16((big_rows, H, 576), 21)
    kv = _rand_bf16((kv_rows, 576), 22)
    rng = np.random.default_rng(5)
    idx = to_dev(np.stack([rng.choice(kv_rows, topk, replace=False) for _ in range(big_rows)]).astype(np.int32))
    log("attn split vs unsplit")
    big, big_lse = _attn(q, kv, idx, 1 / 24, 512)
    for r in (0, 33, 255):
        one, one_lse = _attn(q[r:r + 1].contiguous(), kv, idx[r:r + 1].contiguous(), 1 / 24, 512)
        assert_close(out_f64(one[0]), out_f64(big[r]), (1e-2, 1e-2), "split vs unsplit")
        assert_close(one_lse[0].cpu().double().numpy(), big_lse[r].cpu().double().numpy(), LSE_TOL, "lse")


def test_attn_many_splits_with_empty_leading_splits():
    """Long top-k on few rows: many key splits, combined in several chunks; row 0 has
    only padding in its first 6000 entries (empty splits), row 1 keeps one valid key."""
    import sparse_attention_kv_amd as hs
    rows, H, kv_rows, topk = 2, 128, 30000, 8192
    assert hs.hs_attn_workspace_bytes(rows, H, 576, 512, topk, torch.bfloat16) > 0
    q = _rand_bf16((rows, H, 576), 31)
    kv = _rand_bf16((kv_rows, 576), 32)
    rng = np.random.default_rng(9)
    idx = np.stack([rng.choice(kv_rows, topk, replace=False) for _ in range(rows)]).astype(np.int32)
    idx[0, :6000] = -1
    idx[1, :] = -1
    idx[1, 5000] = 17
    _check(q, kv, to_dev(idx), 1 / 24, 512, BF16_TOL, "many splits")


# Shapes with >= 64 (row, 64-head) groups take the 64-head kernel; the cases above take the
# 32-head one.  These repeat the ragged / padded / empty cases on the 64-head path.
@pytest.mark.parametrize("topk", [1, 65, 2047, 4500])
def test_attn_bf16_64head_path_ragged_topk(topk):
    rows, H, kv_rows = 32, 128, 6000
    assert _kernel(rows, H, topk) == 64
    rng = np.random.default_rng(100 + topk)
    q = _rand_bf16((rows, H, 576), 200 + topk)
    kv = _rand_bf16((kv_rows, 576), 300 + topk)
    idx = np.stack([rng.choice(kv_rows, topk, replace=False) for _ in range(rows)]).astype(np.int32)
    idx[1, rng.random(topk) < 0.3] = -1
    idx[2, rng.random(topk) < 0.2] = kv_rows + 7
    idx[3, :] = -1
    if topk > 1:
        idx[4, :] = idx[4, 0]  # one key repeated
    _check(q, kv, to_dev(idx), 1 / 24, 512, BF16_TOL, f"64-head ragged topk={topk}")


def test_attn_bf16_64head_path_zero_query_and_large_scores():
    rows, H, kv_rows, topk = 64, 64, 3000, 300
    assert _kernel(rows, H, topk) == 64
    rng = np.random.default_rng(77)
    q = _rand_bf16((rows, H, 576), 78)
    q[0] = 0  # uniform softmax
    q[1] *= 8  # large scores: the reference maximum moves several times
    kv = _rand_bf16((kv_rows, 576), 79)
    idx = np.stack([rng.choice(kv_rows, topk, replace=False) for _ in range(rows)]).astype(np.int32)
    _check(q, kv, to_dev(idx), 1 / 24, 512, BF16_TOL, "64-head zero query / large scores")


# >= 256 (row, 128-head) groups take the 128-head kernel: the same cases on that path.  The
# kernel runs on all 256 rows; the oracle checks all of them, or for the longest index
# lists a sample that holds every special row.
_SAMPLE128 = [0, 1, 2, 3, 4, 5, 6, 7, 100, 199, 255]


def _check_sampled(q, kv, idx, scale, d_v, what, sample):
    log(f"attn {what}: rows={q.shape[0]} H={q.shape[1]} topk={idx.shape[1]} sampled {len(sample)}")
    out, lse = _attn(q, kv, idx, scale, d_v)
    sel = torch.as_tensor(sample)
    ref, rlse = oracle.sparse_decode_attn(raw(q.cpu()[sel]), raw(kv.cpu()), idx.cpu().numpy()[sample], scale, d_v)
    assert_close(out_f64(out[sel.to(out.device)]), ref, BF16_TOL, what)
    g = lse[sel.to(lse.device)].cpu().double().numpy()
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(g), fin), what
    assert_close(g[fin], rlse[fin], LSE_TOL, what + " lse")
    assert torch.isfinite(out).all(), what + " non-finite output"


@pytest.mark.parametrize("topk", [1, 65, 2047, 4500])
def test_attn_bf16_128head_path_ragged_topk(topk):
    import sparse_attention_kv_amd as hs
    rows, H, kv_rows = 256, 128, 6000
    assert _kernel(rows, H, topk) == 128
    if topk <= 2048:  # one split holds at most 2048 keys; longer lists always split
        assert hs.hs_attn_workspace_bytes(rows, H, 576, 512, topk, torch.bfloat16) == 0
    rng = np.random.default_rng(500 + topk)
    q = _rand_bf16((rows, H, 576), 600 + topk)
    kv = _rand_bf16((kv_rows, 576), 700 + topk)
    idx = np.stack([rng.choice(kv_rows, topk, replace=False) for _ in range(rows)]).astype(np.int32)
    idx[1, rng.random(topk) < 0.3] = -1
    idx[2, rng.random(topk) < 0.2] = kv_rows + 7
    idx[3, :] = -1
    if topk > 1:
        idx[4, :] = idx[4, 0]  # one key repeated
    idx[199, : topk // 2] = -1  # leading padding
    # at 65 and 2047 keys every row is compared; the long lists sample the special rows
    sample = list(range(rows)) if topk in (65, 2047) else _SAMPLE128
    _check_sampled(q, kv, to_dev(idx), 1 / 24, 512, f"128-head ragged topk={topk}", sample)


def test_attn_bf16_128head_path_zero_query_and_large_scores():
    rows, H, kv_rows, topk = 256, 128, 3000, 700
    assert _kernel(rows, H, topk) == 128
    rng = np.random.default_rng(88)
    q = _rand_bf16((rows, H, 576), 89)
    q[0] = 0   # uniform softmax
    q[1] *= 8  # large scores: the reference maximum moves several times
    q[2] *= 32
    q[255] *= 16
    kv = _rand_bf16((kv_rows, 576), 90)
    idx = np.stack([rng.choice(kv_rows, topk, replace=False) for _ in range(rows)]).astype(np.int32)
    _check_sampled(q, kv, to_dev(idx), 1 / 24, 512, "128-head zero query / large scores",
                   list(range(rows)))



@pytest.mark.parametrize("rows", [8, 128, 256])
def test_attn_reference_moves_at_later_keys(rows):
    """Forces every kernel's rare path (8 rows: 32-head, 128: 64-head, 256: 128-head).  In
    the special rows all heads share one query direction, and keys along it are planted at
    later positions with scores (log2 domain) near 100, 200, 300 and 400, each beyond the
    reference slack, so the reference moves and O is rescaled after the first block, more
    than once, and last at the final block."""
    H, kv_rows, topk = 128, 9000, 2048
    assert _kernel(rows, H, topk) == {8: 32, 128: 64, 256: 128}[rows]
    rng = np.random.default_rng(4400 + rows)
    q = _rand_bf16((rows, H, 576), 4500 + rows).cpu()
    kv = _rand_bf16((kv_rows, 576), 4600 + rows).cpu()
    idx = np.stack([rng.choice(kv_rows - 64, topk, replace=False) for _ in range(rows)]).astype(np.int32)
    special = [0, 1, rows // 2, rows - 1]
    for j, r in enumerate(special):
        base = torch.randn((576,), generator=torch.Generator().manual_seed(4700 + j))
        q[r] = (base[None, :] + 0.1 * torch.randn((H, 576), generator=torch.Generator().manual_seed(4800 + j))).to(torch.bfloat16)
        # |base|^2 ~ 576: score(c * base) ~ c * 24 (natural) ~ c * 34.6 (log2)
        for c, pos in zip((3.0, 6.0, 9.0, 12.0), (40 + j, 300 + 7 * j, 1100 + j, topk - 1 - j)):
            row = kv_rows - 64 + 16 * j + int(c)
            kv[row] = (c * base).to(torch.bfloat16)
            idx[r, pos] = row
        # the condition the test is for: each planted key's score exceeds the maximum over
        # the row's first 32 keys by more than the kernels' 64 (log2) slack, in every head
        qf, kf = raw(q[r]).astype(np.uint32), raw(kv).astype(np.uint32)
        qv = (qf << 16).view(np.float32).astype(np.float64)
        kvv = (kf << 16).view(np.float32).astype(np.float64)
        s2 = (qv @ kvv[idx[r]].T) / 24 * np.log2(np.e)          # [H, topk], log2 domain
        first = s2[:, :32].max(axis=1)
        for pos in (300 + 7 * j, 1100 + j, topk - 1 - j):
            assert (s2[:, pos] > first + 64).all() and (s2[:, pos] >= s2[:, :pos].max(axis=1) + 64).all()
    sample = sorted(set(special + [2, rows // 3]))
    _check_sampled(q.to(dev()), kv.to(dev()), to_dev(idx), 1 / 24, 512,
                   f"reference moves, {rows} rows", sample)

def test_attn_deterministic_and_index_order_invariant():
    s, w = make("resident", num_reqs=4)
    g = gpu_inputs(s, w)
    ref_slots, _ = oracle_resolve(s, w)
    idx = to_dev(ref_slots)
    log("attn determinism")
    a, _ = _attn(g["q"], w.kv_pool, idx, s.scale, s.d_v)
    b, _ = _attn(g["q"], w.kv_pool, idx, s.scale, s.d_v)
    assert torch.equal(a, b)
    perm = torch.randperm(idx.shape[1], generator=torch.Generator().manual_seed(0)).to(dev())
    c, _ = _attn(g["q"], w.kv_pool, idx[:, perm].contiguous(), s.scale, s.d_v)
    assert_close(out_f64(c), out_f64(a), (1e-2, 1e-2), "permuted indices")


# Head counts other than 128 reach the kernels through other planner choices: 32 and 96
# heads only the 32-head kernel, 192 the 64-head one from 64 (row, 64-head) groups, 256
# the 128-head one from 256 (row, 128-head) groups.  The oracle checks sampled rows.
@pytest.mark.parametrize("H,rows", [(32, 5), (96, 7), (96, 40), (192, 3), (192, 24), (256, 128)])
def test_attn_head_counts(H, rows):
    rng = np.random.default_rng(H * 1000 + rows)
    kv_rows, topk = 5000, 900
    assert _kernel(rows, H, topk) == {32: 32, 96: 32, 192: 32 if rows < 16 else 64, 256: 128}[H]
    q = _rand_bf16((rows, H, 576), H + rows)
    kv = _rand_bf16((kv_rows, 576), H + rows + 1)
    idx = np.stack([rng.choice(kv_rows, topk, replace=False) for _ in range(rows)]).astype(np.int32)
    idx[0, rng.random(topk) < 0.25] = -1
    log(f"attn head count H={H} rows={rows}")
    out, lse = _attn(q, kv, to_dev(idx), 1 / 24, 512)
    sample = sorted(set([0, 1, rows // 2, rows - 1]))
    ref, rlse = oracle.sparse_decode_attn(raw(q.cpu()[sample]), raw(kv.cpu()), idx[sample], 1 / 24, 512)
    assert_close(out_f64(out[sample]), ref, BF16_TOL, f"H={H} rows={rows}")
    g = lse[sample].cpu().double().numpy()
    assert_close(g, rlse, LSE_TOL, f"H={H} rows={rows} lse")


@pytest.mark.parametrize("rows,cus,topk", [(128, 128, 2048), (32, 224, 2048), (8, 64, 777),
                                           (20, 192, 2048), (3, 16, 4500)])
def test_attn_cus_matches_oracle_and_plain_call(rows, cus, topk):
    """hs_sparse_decode_attn_cus: the launch sized for `cus` compute units (another kernel,
    or none, in the others) gives the oracle's result on every row, with the plain call's
    workspace size, and the plain call's result up to fp32 summation order."""
    import sparse_attention_kv_amd as hs
    H, kv_rows = 128, 9000
    hpw, splits = hs.hs_attn_plan_info_cus(rows, H, 576, 512, topk, torch.bfloat16, cus)
    if rows * (H // hpw) * -(-topk // 2048) <= cus:
        assert rows * (H // hpw) * splits <= cus
    rng = np.random.default_rng(rows * 1000 + cus)
    q = _rand_bf16((rows, H, 576), 900 + rows)
    kv = _rand_bf16((kv_rows, 576), 901 + rows)
    idx = np.stack([rng.choice(kv_rows, topk, replace=False) for _ in range(rows)]).astype(np.int32)
    idx[1, rng.random(topk) < 0.3] = -1
    idx[2, :] = -1
    idx = to_dev(idx)
    ws_bytes = hs.hs_attn_workspace_bytes(rows, H, 576, 512, topk, torch.bfloat16)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev()) if ws_bytes else None
    out = torch.full((rows, H, 512), float("nan"), dtype=torch.bfloat16, device=dev())
    lse = torch.full((rows, H), float("nan"), dtype=torch.float32, device=dev())
    log(f"attn cus: rows={rows} cus={cus} topk={topk} plan=({hpw}, {splits})")
    hs.hs_sparse_decode_attn_cus(q, kv, idx, 1 / 24, 512, out, lse, ws, cus)
    torch.cuda.synchronize()
    ref, rlse = oracle.sparse_decode_attn(raw(q.cpu()), raw(kv.cpu()), idx.cpu().numpy(), 1 / 24, 512)
    assert_close(out_f64(out), ref, BF16_TOL, f"cus {cus}")
    g = lse.cpu().double().numpy()
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(g), fin)
    assert_close(g[fin], rlse[fin], LSE_TOL, f"cus {cus} lse")
    plain, plain_lse = _attn(q, kv, idx, 1 / 24, 512)
    assert_close(out_f64(out), out_f64(plain), BF16_TOL, f"cus {cus} vs plain")
    with pytest.raises(hs.HsError):
        hs.hs_sparse_decode_attn_cus(q, kv, idx, 1 / 24, 512, out, lse, ws, 0)


# Plans with key-split counts that are not powers of two (the splits fill the CUs in one
# round), on all three kernels; the last split of a row is shorter than the others.
@pytest.mark.parametrize("rows,H,topk,plan", [(5, 128, 2048, (32, 11)), (9, 128, 2048, (32, 7)),
                                              (5, 64, 3100, (32, 17)), (12, 256, 2048, (64, 5)),
                                              (20, 256, 1000, (64, 3)), (72, 256, 3100, (128, 2))])
def test_attn_uneven_split_counts(rows, H, topk, plan):
    import sparse_attention_kv_amd as hs
    assert hs.hs_attn_plan_info(rows, H, 576, 512, topk, torch.bfloat16) == plan
    kv_rows = 7000
    rng = np.random.default_rng(rows * 7 + H + topk)
    q = _rand_bf16((rows, H, 576), 1000 + rows + H)
    kv = _rand_bf16((kv_rows, 576), 1001 + rows + H)
    idx = np.stack([rng.choice(kv_rows, topk, replace=False) for _ in range(rows)]).astype(np.int32)
    idx[1, rng.random(topk) < 0.4] = -1
    idx[2, topk // 3:] = -1  # only the leading splits hold keys
    sample = sorted({0, 1, 2, rows // 2, rows - 1})
    _check_sampled(q, kv, to_dev(idx), 1 / 24, 512, f"splits {plan}", sample)
