"""GPU parity of hs_resolve_topk against the oracle: bit-exact slots and valid counts."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import dev, gpu_inputs, log, make, oracle_resolve, to_dev

pytestmark = pytest.mark.gpu


def _run(topk_pos, req_id, lim, bt, bs, stride):
    import sparse_attention_kv_amd as hs
    rows, k = topk_pos.shape
    out = torch.full((rows, k), 7, dtype=torch.int32, device=dev())
    valid = torch.full((rows,), 7, dtype=torch.int32, device=dev())
    hs.hs_resolve_topk(to_dev(topk_pos), to_dev(req_id), to_dev(lim), to_dev(bt), bs, stride,
                       out, valid)
    torch.cuda.synchronize()
    return out.cpu().numpy(), valid.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "resident", "mtp_swap", "long", "mixed_finalize"])
def test_resolve_parity_full_size(name):
    s, w = make(name, tensors=False)
    log(f"resolve {name}: rows={s.rows} topk={s.topk}")
    got, gv = _run(w.topk_pos, w.req_id, w.causal_limit, w.block_table, s.block_size, s.block_size)
    ref, rv = oracle_resolve(s, w)
    assert np.array_equal(got, ref)
    assert np.array_equal(gv, rv)


def test_resolve_fail_closed_and_stride():
    bt = np.array([[3, -1, 1], [0, 2, -1]], dtype=np.int32)
    pos = np.array([[0, 5, 9, 4, -1, 12, 100, -7],
                    [0, 5, 9, 4, -1, 12, 100, -7],
                    [1, 2, 3, 4, 5, 6, 7, 8],
                    [8, 9, 10, 11, 0, 1, 2, 3]], dtype=np.int32)
    req = np.array([0, 1, 7, -1], dtype=np.int32)
    lim = np.array([13, 9, 100, 100], dtype=np.int32)
    for stride in (4, 8, 5):
        log(f"resolve fail-closed stride={stride}")
        got, gv = _run(pos, req, lim, bt, 4, stride)
        ref, rv = oracle.resolve_topk(pos, req, lim, bt, 4, stride, 2)
        assert np.array_equal(got, ref) and np.array_equal(gv, rv)


@pytest.mark.parametrize("topk", [1, 3, 255, 257, 1025, 4096])
def test_resolve_ragged_topk(topk):
    rng = np.random.default_rng(topk)
    B, bs, width = 3, 16, 300
    bt = rng.permutation(B * width).astype(np.int32).reshape(B, width)
    bt[1, 200:] = -1
    rows = 7
    req = rng.integers(-1, B + 1, size=rows).astype(np.int32)
    lim = rng.integers(0, width * bs + 50, size=rows).astype(np.int32)
    pos = rng.integers(-3, width * bs + 100, size=(rows, topk)).astype(np.int32)
    log(f"resolve ragged topk={topk}")
    got, gv = _run(pos, req, lim, bt, bs, bs)
    ref, rv = oracle.resolve_topk(pos, req, lim, bt, bs, bs, B)
    assert np.array_equal(got, ref) and np.array_equal(gv, rv)


def test_resolve_zero_rows_is_noop():
    import sparse_attention_kv_amd as hs
    out = torch.empty((0, 16), dtype=torch.int32, device=dev())
    e = torch.empty((0,), dtype=torch.int32, device=dev())
    bt = torch.zeros((1, 4), dtype=torch.int32, device=dev())
    hs.hs_resolve_topk(torch.empty((0, 16), dtype=torch.int32, device=dev()), e, e, bt, 16, 16, out)
    torch.cuda.synchronize()
