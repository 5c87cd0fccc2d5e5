"""GPU parity of hs_backup_rows (device -> pinned host row copy) against the oracle.

Bit-exact: the host cache after the call must equal oracle.backup_rows on the same input.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import dev, log
from tests.helpers import raw

pytestmark = pytest.mark.gpu


def _pinned_like(a: np.ndarray, dtype) -> torch.Tensor:
    t = torch.empty(a.shape, dtype=dtype, pin_memory=True)
    if dtype == torch.bfloat16:
        t.view(torch.int16).numpy()[...] = a.view(np.int16)
    else:
        t.numpy()[...] = a
    return t


def _case(L, dev_rows, host_rows, elems, n, dtype, per_layer, bs, stride, seed, frac_bad=0.1):
    rng = np.random.default_rng(seed)
    np_dt = np.uint16 if dtype == torch.bfloat16 else np.float32
    if np_dt == np.uint16:
        dev_np = rng.integers(0, 2 ** 16, size=(L, dev_rows, elems), dtype=np.uint16)
        host_np = rng.integers(0, 2 ** 16, size=(L, host_rows, elems), dtype=np.uint16)
    else:
        dev_np = rng.standard_normal((L, dev_rows, elems)).astype(np.float32)
        host_np = rng.standard_normal((L, host_rows, elems)).astype(np.float32)
    max_slot = (dev_rows // stride + 1) * bs
    shape = (L, n) if per_layer else (n,)
    src = rng.integers(0, max_slot, size=shape).astype(np.int32)
    src[rng.random(shape) < frac_bad] = -1
    dst = rng.permutation(host_rows)[:n].astype(np.int32)
    dst[rng.random(n) < frac_bad] = -1
    if n > 2:
        dst[1] = host_rows + 3  # out of range: skipped
    return dev_np, host_np, src, dst


def _run(dev_np, host_np, src, dst, dtype, bs, stride):
    import sparse_attention_kv_amd as hs
    dev_t = torch.from_numpy(dev_np.view(np.int16) if dev_np.dtype == np.uint16 else dev_np)
    dev_t = dev_t.view(dtype).to(dev()) if dtype == torch.bfloat16 else dev_t.to(dev())
    host_t = _pinned_like(host_np, dtype)
    hs.hs_backup_rows(dev_t, host_t, torch.from_numpy(src).to(dev()),
                      torch.from_numpy(dst).to(dev()), bs, stride)
    ev = torch.cuda.Event()
    ev.record()
    ev.synchronize()
    got = raw(host_t) if dtype == torch.bfloat16 else host_t.numpy()
    return got


@pytest.mark.parametrize("per_layer", [True, False])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_backup_matches_oracle(per_layer, dtype):
    L, dev_rows, host_rows, n = 3, 3000, 2500, 1999
    elems = 576 if dtype == torch.bfloat16 else 64
    bs, stride = 64, 80
    dev_np, host_np, src, dst = _case(L, dev_rows, host_rows, elems, n, dtype, per_layer, bs,
                                      stride, seed=7 + per_layer)
    log(f"backup L={L} n={n} dtype={dtype} per_layer={per_layer}")
    got = _run(dev_np, host_np, src, dst, dtype, bs, stride)
    ref = oracle.backup_rows(dev_np, host_np, src, dst, bs, stride)
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))


def test_backup_empty_all_invalid_and_single_row():
    dtype = torch.bfloat16
    dev_np, host_np, src, dst = _case(2, 100, 80, 576, 5, dtype, True, 1, 1, seed=3)
    log("backup edge cases")
    for s, d in [(src[:, :0], dst[:0]),                       # nothing to copy
                 (np.full_like(src, -1), dst),               # no valid source
                 (src, np.full_like(dst, -1)),               # no valid destination
                 (src[:, :1], dst[:1])]:                     # one row
        got = _run(dev_np, host_np, np.ascontiguousarray(s), np.ascontiguousarray(d), dtype, 1, 1)
        ref = oracle.backup_rows(dev_np, host_np, s, d, 1, 1)
        assert np.array_equal(got, ref)


def test_backup_duplicate_destination_parts_come_from_its_sources():
    """Distinct destinations are the caller's contract; with a duplicate, each 16-byte part
    of the row comes from one of its sources, and every other row is exact."""
    dtype = torch.bfloat16
    dev_np, host_np, src, dst = _case(1, 500, 300, 576, 200, dtype, True, 1, 1, seed=9, frac_bad=0)
    dst[10:20] = 42  # ten entries write host row 42
    got = _run(dev_np, host_np, src, dst, dtype, 1, 1)
    parts = got[0, 42].reshape(-1, 8)  # 16-byte parts of bf16
    cands = np.stack([dev_np[0, src[0, i]].reshape(-1, 8) for i in np.flatnonzero(dst == 42)])
    assert all(any(np.array_equal(parts[k], c[k]) for c in cands) for k in range(parts.shape[0]))
    keep = dst != 42
    ref = oracle.backup_rows(dev_np, host_np, src[:, keep], dst[keep], 1, 1)
    rows = np.ones(300, dtype=bool)
    rows[42] = False
    assert np.array_equal(got[0, rows], ref[0, rows])


def test_backup_full_size_prefill_staging():
    """The staging workload's size: 4 layers x 16384 rows of 1152 B (75 MB)."""
    dtype = torch.bfloat16
    dev_np, host_np, src, dst = _case(4, 16384, 16384, 576, 16384, dtype, False, 64, 64, seed=21,
                                      frac_bad=0.02)
    log("backup full size")
    got = _run(dev_np, host_np, src, dst, dtype, 64, 64)
    ref = oracle.backup_rows(dev_np, host_np, src, dst, 64, 64)
    assert np.array_equal(got, ref)


def test_backup_event_marks_completion():
    """An event recorded after the call fires only once the host rows hold the copies."""
    import sparse_attention_kv_amd as hs
    rows, elems = 8192, 576
    src_dev = torch.randn((rows, elems), device=dev()).to(torch.bfloat16)
    host = torch.zeros((rows, elems), dtype=torch.bfloat16, pin_memory=True)
    idx = torch.arange(rows, dtype=torch.int32, device=dev())
    torch.cuda.synchronize()
    torch.cuda._sleep(2_000_000)  # keep the stream busy so the event is still pending
    hs.hs_backup_rows(src_dev, host, idx, idx)
    ev = torch.cuda.Event()
    ev.record()
    polls = 0
    while not ev.query():
        polls += 1
    assert torch.equal(host, src_dev.cpu())
    log(f"event polled {polls} times")


def test_backup_rejects_bad_arguments():
    import sparse_attention_kv_amd as hs
    d = torch.zeros((4, 576), dtype=torch.bfloat16, device=dev())
    idx = torch.zeros((2,), dtype=torch.int32, device=dev())
    with pytest.raises(ValueError):  # pageable host memory
        hs.hs_backup_rows(d, torch.zeros((4, 576), dtype=torch.bfloat16), idx, idx)
    with pytest.raises(hs.HsError) as e:  # 12-byte rows
        hs.hs_backup_rows(torch.zeros((4, 6), dtype=torch.bfloat16, device=dev()),
                          torch.zeros((4, 6), dtype=torch.bfloat16, pin_memory=True), idx, idx)
    assert e.value.status == hs.HS_ERR_INVALID_ARG
    with pytest.raises(hs.HsError) as e:  # device memory as the destination
        lib = hs._lib
        st = lib.hs_backup_rows(d.data_ptr(), 4, d.data_ptr(), 4, 1, 1152, idx.data_ptr(), 0,
                                idx.data_ptr(), 2, 1, 1, None)
        hs._check("hs_backup_rows", st)
    assert e.value.status == hs.HS_ERR_INVALID_ARG


def test_stager_pages_match_oracle_plan_and_copy():
    """BackupStager (host planning, pinned staging, async index copies, backup kernel,
    event) against the oracle's plan_backup_rows + backup_rows, over three enqueues so the
    two staging buffers are reused."""
    from sparse_attention_kv_amd.pipeline import BackupStager, PageTransfer
    rng = np.random.default_rng(17)
    L, kbs, per, dev_blocks, host_blocks = 3, 64, 4, 40, 10
    dev_np = rng.integers(0, 2 ** 16, size=(L, dev_blocks * kbs, 576), dtype=np.uint16)
    host_np = rng.integers(0, 2 ** 16, size=(L, host_blocks * per * kbs, 576), dtype=np.uint16)
    dev_t = torch.from_numpy(dev_np.view(np.int16)).view(torch.bfloat16).to(dev())
    host_t = _pinned_like(host_np, torch.bfloat16)
    stager = BackupStager(dev_t, host_t, kbs, per, max_pages=8)
    pages = [(hb, po) for hb in range(host_blocks) for po in range(per)]
    order = rng.permutation(len(pages))
    ref = host_np
    events = []
    for call in range(3):
        chosen = [pages[k] for k in order[call * 6:(call + 1) * 6]]
        trs = [PageTransfer(tuple(int(x) for x in rng.integers(0, dev_blocks, size=L)), hb, po)
               for hb, po in chosen]
        events.append(stager.enqueue(trs))
        otr = [oracle.PageTransfer(tuple(t.source_block_ids), t.destination_block_id,
                                   t.destination_page_offset) for t in trs]
        src, dst = oracle.plan_backup_rows(otr, kbs, per, L)
        ref = oracle.backup_rows(dev_np, ref, src, dst)
    log("backup stager")
    while not BackupStager.ready(events[-1]):
        pass
    assert all(BackupStager.ready(e) for e in events)
    assert np.array_equal(raw(host_t), ref)
