"""hs_sparse_decode_attn_noalloc (the attention entry point that allocates nothing: its
key-split partials live in the library's fixed per-GPU scratch array) against
hs_sparse_decode_attn with a caller workspace: the same kernels and launch plan, so the
outputs must be bit-identical.  Two calls in a row, the second with a smaller input, then
a shape whose workspace exceeds the scratch, which must be refused before any launch."""

import numpy as np
import pytest
import torch

from tests.gpu_cases import dev, log

pytestmark = pytest.mark.gpu


def _case(rows, heads, topk, kv_rows, seed):
    g = torch.Generator(device=dev()).manual_seed(seed)
    q = torch.randn((rows, heads, 576), generator=g, device=dev()).to(torch.bfloat16)
    kv = torch.randn((kv_rows, 576), generator=g, device=dev()).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(kv_rows, topk, replace=False) for _ in range(rows)]).astype(np.int32)
    idx[0, rng.random(topk) < 0.3] = -1          # padding in one row
    return q, kv, torch.as_tensor(idx, device=dev())


def _both(q, kv, idx):
    import sparse_attention_kv_amd as hs
    rows, heads, _ = q.shape
    wsb = hs.hs_attn_workspace_bytes(rows, heads, 576, 512, idx.shape[1], torch.bfloat16)
    assert 0 < wsb <= hs.NOALLOC_SCRATCH_BYTES   # the call uses the scratch
    ws = torch.empty((wsb,), dtype=torch.uint8, device=dev())
    ref = torch.empty((rows, heads, 512), dtype=torch.bfloat16, device=dev())
    ref_lse = torch.empty((rows, heads), dtype=torch.float32, device=dev())
    hs.hs_sparse_decode_attn(q, kv, idx, 1 / 24, 512, ref, ref_lse, ws)
    out = torch.full_like(ref, 7.0)
    lse = torch.full_like(ref_lse, 7.0)
    hs.hs_sparse_decode_attn_noalloc(q, kv, idx, 1 / 24, 512, out, lse)
    torch.cuda.synchronize()
    return out, lse, ref, ref_lse, wsb


def test_noalloc_matches_workspace_call_twice_then_refuses_oversize():
    import sparse_attention_kv_amd as hs
    first = _case(8, 128, 2048, 40000, 1)       # 32-head kernel, 8 key splits
    second = _case(3, 64, 700, 9000, 2)         # smaller: fewer rows, heads and keys
    for n, (q, kv, idx) in enumerate((first, second)):
        out, lse, ref, ref_lse, wsb = _both(q, kv, idx)
        log(f"noalloc call {n}: rows {q.shape[0]} heads {q.shape[1]} topk {idx.shape[1]} "
            f"workspace {wsb} B")
        assert torch.equal(out, ref), f"call {n} output"
        assert torch.equal(lse, ref_lse), f"call {n} lse"
    # a shape whose split partials exceed the scratch is refused before any launch
    rows, heads, topk = 256, 256, 4096
    assert hs.hs_attn_workspace_bytes(rows, heads, 576, 512, topk, torch.bfloat16) > hs.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((rows, heads, 576), dtype=torch.bfloat16, device=dev())
    kv = torch.zeros((16, 576), dtype=torch.bfloat16, device=dev())
    idx = torch.full((rows, topk), -1, dtype=torch.int32, device=dev())
    out = torch.full((rows, heads, 512), 3.0, dtype=torch.bfloat16, device=dev())
    with pytest.raises(hs.HsError) as e:
        hs.hs_sparse_decode_attn_noalloc(q, kv, idx, 1 / 24, 512, out)
    assert e.value.status == hs.HS_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "a refused call wrote its output"
