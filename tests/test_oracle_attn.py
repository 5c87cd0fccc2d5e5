"""Pins for the oracle's sparse_decode_attn (CPU only).

Checked against PyTorch's scaled_dot_product_attention (a library routine) run
densely over the whole KV pool with a boolean mask in float64, closed forms
(one selected key; zero query), and invariances.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

from oracle import as_f64, resolve_topk, sparse_decode_attn
from tests.helpers import raw
from workloads import generate, spec


def _dense_masked(qf, kvf, indices, scale, d_v):
    rows, H, D = qf.shape
    out = np.zeros((rows, H, d_v))
    for i in range(rows):
        mask = np.zeros(kvf.shape[0], dtype=bool)
        sel = indices[i][indices[i] >= 0]
        mask[sel] = True
        q = torch.from_numpy(qf[i])[None]                       # [1, H, D]
        k = torch.from_numpy(kvf)[None, None].expand(1, H, -1, -1)
        v = torch.from_numpy(kvf[:, :d_v])[None, None].expand(1, H, -1, -1)
        m = torch.from_numpy(mask)[None, None, None].expand(1, H, 1, -1)
        o = F.scaled_dot_product_attention(q[:, :, None, :], k, v, attn_mask=m, scale=scale)
        out[i] = o[0, :, 0].numpy()
    return out


@pytest.mark.parametrize("name,over", [("tiny", {}), ("tiny", {"seq_rule": ("fixed", [10, 70])}),
                                       ("resident", {"num_reqs": 2, "topk": 64, "num_heads": 8,
                                                     "seq_rule": ("uniform", 100, 300)})])
def test_attn_equals_dense_masked_sdpa(name, over):
    s = spec(name, **over)
    w = generate(s)
    slots, _ = resolve_topk(w.topk_pos, w.req_id, w.causal_limit, w.block_table,
                            s.block_size, s.block_size, s.num_reqs)
    q, kv = raw(w.q), raw(w.kv_pool)
    out, lse = sparse_decode_attn(q, kv, slots, s.scale, s.d_v)
    ref = _dense_masked(as_f64(q), as_f64(kv), slots, s.scale, s.d_v)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # lse = log-sum-exp of the selected scores
    for i in range(s.rows):
        sel = slots[i][slots[i] >= 0]
        sc = s.scale * as_f64(q[i]) @ as_f64(kv[sel]).T
        np.testing.assert_allclose(lse[i], logsumexp(sc, axis=1), rtol=1e-12)


def test_attn_single_key_returns_value_row():
    rng = np.random.default_rng(1)
    kv = rng.standard_normal((50, 16)).astype(np.float32)
    q = rng.standard_normal((3, 4, 16)).astype(np.float32)
    idx = np.full((3, 8), -1, np.int32)
    idx[0, 5] = 7
    idx[1, 0] = 49
    idx[2, 7] = 0
    out, _ = sparse_decode_attn(q, kv, idx, 0.3, 12)
    for i, j in enumerate([7, 49, 0]):
        assert np.array_equal(out[i], np.broadcast_to(kv[j, :12].astype(np.float64), (4, 12)))


def test_attn_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    kv = rng.standard_normal((40, 10)).astype(np.float32)
    q = np.zeros((1, 2, 10), np.float32)
    sel = np.array([3, 9, 17, 33, 2], np.int32)
    idx = np.concatenate([sel, [-1, -1]])[None]
    out, lse = sparse_decode_attn(q, kv, idx, 1.0, 6)
    np.testing.assert_allclose(out[0], np.broadcast_to(kv[sel, :6].astype(np.float64).mean(0), (2, 6)),
                               rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse[0], np.log(5.0))


def test_attn_permutation_invariant_and_empty_row():
    rng = np.random.default_rng(4)
    kv = rng.standard_normal((64, 12)).astype(np.float32)
    q = rng.standard_normal((2, 3, 12)).astype(np.float32)
    idx = np.stack([rng.permutation(64)[:20], np.full(20, -1)]).astype(np.int32)
    out1, lse1 = sparse_decode_attn(q, kv, idx, 0.5, 12)
    out2, lse2 = sparse_decode_attn(q, kv, idx[:, rng.permutation(20)], 0.5, 12)
    np.testing.assert_allclose(out1, out2, rtol=1e-13, atol=1e-14)
    assert (out1[1] == 0).all() and np.isneginf(lse1[1]).all()


def test_attn_bf16_upcast_is_exact():
    t = torch.randn(1000).to(torch.bfloat16)
    assert np.array_equal(as_f64(raw(t)), t.double().numpy())
