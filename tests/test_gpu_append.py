"""GPU parity of hs_append_accepted (draft-model context KV grows by the accepted prefix)
against oracle.append_accepted: bit-exact cache rows and context lengths."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import dev, log, to_dev
from tests.helpers import raw


pytestmark = pytest.mark.gpu


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev())


def test_append_steps_match_oracle():
    """The verify shape of the mixed workload (128 requests x 3 rows, 576-wide bf16 rows),
    three decode steps, with unmapped pages and out-of-range accept lengths."""
    import sparse_attention_kv_amd as hs
    rng = np.random.default_rng(12)
    B, R, E, bs, W = 128, 3, 576, 64, 40
    bt = rng.permutation(B * W).reshape(B, W).astype(np.int32)
    bt[rng.random((B, W)) < 0.05] = -1
    cache = rng.integers(0, 2 ** 16, size=(B * W * bs, E), dtype=np.uint16)
    lens = rng.integers(0, W * bs - 20, size=B).astype(np.int32)
    g_cache, g_bt, g_len = _bf16(cache), to_dev(bt), to_dev(lens)
    for rnd in range(3):
        rows = rng.integers(0, 2 ** 16, size=(B * R, E), dtype=np.uint16)
        acc = rng.integers(-1, R + 1, size=B).astype(np.int32)
        log(f"append step {rnd}")
        hs.hs_append_accepted(g_cache, g_bt, g_len, _bf16(rows), to_dev(acc), bs, bs, R)
        torch.cuda.synchronize()
        cache, lens64 = oracle.append_accepted(cache, bt, lens, rows, acc, R, bs, bs)
        lens = lens64.astype(np.int32)
        assert np.array_equal(g_len.cpu().numpy(), lens), rnd
        assert np.array_equal(raw(g_cache.cpu()), cache), rnd


def test_append_unmapped_and_full_acceptance():
    import sparse_attention_kv_amd as hs
    rng = np.random.default_rng(3)
    B, R, E, bs = 4, 4, 64, 16
    bt = np.full((B, 2), -1, dtype=np.int32)  # nothing mapped: no row is written
    cache = np.zeros((64, E), dtype=np.float32)
    rows = rng.standard_normal((B * R, E)).astype(np.float32)
    g_cache = torch.from_numpy(cache).to(dev())
    g_len = to_dev(np.array([0, 3, 15, 31], dtype=np.int32))
    hs.hs_append_accepted(g_cache, to_dev(bt), g_len, torch.from_numpy(rows).to(dev()),
                          to_dev(np.full(B, R - 1, dtype=np.int32)), bs, bs, R)
    torch.cuda.synchronize()
    assert (g_cache.cpu().numpy() == 0).all()
    assert g_len.cpu().tolist() == [4, 7, 19, 35]  # lengths still advance by L + 1


def test_append_rejects_bad_arguments():
    import sparse_attention_kv_amd as hs
    c = torch.zeros((8, 6), dtype=torch.bfloat16, device=dev())  # 12-byte rows
    bt = torch.zeros((1, 1), dtype=torch.int32, device=dev())
    ln = torch.zeros((1,), dtype=torch.int32, device=dev())
    with pytest.raises(hs.HsError) as e:
        hs.hs_append_accepted(c, bt, ln, torch.zeros((2, 6), dtype=torch.bfloat16, device=dev()),
                              ln, 4, 4, 2)
    assert e.value.status == hs.HS_ERR_INVALID_ARG
