"""The C-ABI library loads and exports every symbol include/hisparse.h declares; its host
validation rejects bad arguments before any HIP call (runs without a GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hisparse.h")
LIB = os.path.join(ROOT, "sparse_attention_kv_amd", "libhisparse.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libhisparse.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hs_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("hs_resolve_topk", "hs_swap_in", "hs_sparse_decode_attn", "hs_finalize_accepted"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_exports_match_header():
    import sparse_attention_kv_amd as hs
    assert sorted(hs.EXPORTED) == _declared()
    assert hs.version().startswith("hisparse-gfx950")
    assert hs.status_string(hs.HS_ERR_CAPACITY) == "top-k exceeds hot-buffer capacity"


def _lib():
    import sparse_attention_kv_amd as hs
    return hs, hs._lib


def test_resolve_validation():
    hs, lib = _lib()
    p = ctypes.c_void_p(16)
    # num_rows == 0 is a no-op
    assert lib.hs_resolve_topk(None, 0, 16, None, None, 1, None, 4, 16, 16, None, None, None) == hs.HS_OK
    assert lib.hs_resolve_topk(p, -1, 16, p, p, 1, p, 4, 16, 16, p, None, None) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_resolve_topk(p, 2, 0, p, p, 1, p, 4, 16, 16, p, None, None) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_resolve_topk(p, 2, 16, p, p, 1, p, 4, 0, 16, p, None, None) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_resolve_topk(None, 2, 16, p, p, 1, p, 4, 16, 16, p, None, None) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_resolve_topk(p, 2, 16, p, p, 1, p, 4, 16, 16, None, None, None) == hs.HS_ERR_INVALID_ARG


def _state(hs, **kw):
    d = dict(num_reqs=2, capacity=24, slot_loc=16, slot_stamp=32, loc_to_hot=48, host_rows=256,
             row_elems=64, dtype=hs.HS_F32, hot_kv=64, host_pool=128)
    d.update(kw)
    return hs.HsHotState(**d)


def test_swap_validation():
    hs, lib = _lib()
    p = ctypes.c_void_p(16)
    st = _state(hs)
    # top-k beyond the hot-buffer capacity -> capacity error, nothing touched
    assert lib.hs_swap_in(ctypes.byref(st), p, 25, 1, p, p, None, None) == hs.HS_ERR_CAPACITY
    assert lib.hs_swap_in(None, p, 16, 1, p, p, None, None) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_swap_in(ctypes.byref(st), None, 16, 1, p, p, None, None) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_swap_in(ctypes.byref(st), p, 0, 1, p, p, None, None) == hs.HS_ERR_INVALID_ARG
    bad = _state(hs, row_elems=6)         # 24-byte rows are not a multiple of 16
    assert lib.hs_swap_in(ctypes.byref(bad), p, 16, 1, p, p, None, None) == hs.HS_ERR_INVALID_ARG
    bad = _state(hs, hot_kv=72)           # misaligned hot buffer
    assert lib.hs_swap_in(ctypes.byref(bad), p, 16, 1, p, p, None, None) == hs.HS_ERR_INVALID_ARG
    bad = _state(hs, dtype=7)
    assert lib.hs_swap_in(ctypes.byref(bad), p, 16, 1, p, p, None, None) == hs.HS_ERR_INVALID_ARG
    big = _state(hs, capacity=20000)
    assert lib.hs_swap_in(ctypes.byref(big), p, 16, 1, p, p, None, None) == hs.HS_ERR_UNSUPPORTED
    wide = _state(hs, capacity=8192)
    assert lib.hs_swap_in(ctypes.byref(wide), p, 5000, 1, p, p, None, None) == hs.HS_ERR_UNSUPPORTED


def test_attn_validation_and_workspace():
    hs, lib = _lib()
    p = ctypes.c_void_p(16)
    assert lib.hs_sparse_decode_attn(p, p, 10, p, 0, 128, 576, 512, 2048, 1.0, hs.HS_BF16, p, None,
                                      None, 0, None) == hs.HS_OK
    # unsupported shapes of the bf16 MFMA path
    assert lib.hs_sparse_decode_attn(p, p, 10, p, 2, 128, 512, 512, 2048, 1.0, hs.HS_BF16, p, None,
                                      None, 0, None) == hs.HS_ERR_UNSUPPORTED
    assert lib.hs_sparse_decode_attn(p, p, 10, p, 2, 100, 576, 512, 2048, 1.0, hs.HS_BF16, p, None,
                                      None, 0, None) == hs.HS_ERR_UNSUPPORTED
    assert lib.hs_sparse_decode_attn(p, p, 10, p, 2, 4, 2048, 48, 16, 1.0, hs.HS_F32, p, None,
                                      None, 0, None) == hs.HS_ERR_UNSUPPORTED
    assert lib.hs_sparse_decode_attn(p, p, 10, p, 2, 4, 64, 48, 16, 1.0, 9, p, None,
                                      None, 0, None) == hs.HS_ERR_INVALID_ARG
    # split-KV shapes need the workspace the library asks for
    ws = lib.hs_attn_workspace_bytes(8, 128, 576, 512, 2048, hs.HS_BF16)
    assert ws > 0
    assert lib.hs_sparse_decode_attn(p, p, 10, p, 8, 128, 576, 512, 2048, 1.0, hs.HS_BF16, p, None,
                                      None, 0, None) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_sparse_decode_attn(p, p, 10, p, 8, 128, 576, 512, 2048, 1.0, hs.HS_BF16, p, None,
                                      p, ws - 16, None) == hs.HS_ERR_INVALID_ARG
    # large batches need no split and no workspace
    assert lib.hs_attn_workspace_bytes(256, 128, 576, 512, 2048, hs.HS_BF16) == 0
    assert lib.hs_attn_workspace_bytes(4, 4, 64, 48, 16, hs.HS_F32) == 0


def test_finalize_validation():
    hs, lib = _lib()
    p = ctypes.c_void_p(16)
    st = _state(hs)
    args = lambda **k: [ctypes.byref(k.get("st", st)), p, k.get("vocab", 100), p, p,
                        k.get("R", 3), p, p, 4, 16, 1, p, p, p, None]
    assert lib.hs_finalize_accepted(*args(vocab=0)) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_finalize_accepted(*args(R=0)) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_finalize_accepted(*args(R=25)) == hs.HS_ERR_INVALID_ARG   # > capacity
    big = _state(hs, capacity=200)
    assert lib.hs_finalize_accepted(*args(st=big, R=65)) == hs.HS_ERR_UNSUPPORTED


def test_backup_validation():
    hs, lib = _lib()
    f = lib.hs_backup_rows
    P = 4096  # fake non-null, 16-byte aligned pointers (never dereferenced on these paths)
    ok = dict(dev=P, dev_rows=10, host=P, host_rows=10, layers=1, row_bytes=1152, src=P,
              per_layer=0, dst=P, n=4, bs=1, stride=1)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["dev"], a["dev_rows"], a["host"], a["host_rows"], a["layers"], a["row_bytes"],
                 a["src"], a["per_layer"], a["dst"], a["n"], a["bs"], a["stride"], None)

    assert call(n=0) == hs.HS_OK  # nothing to copy: returns before any HIP call
    bad = hs.HS_ERR_INVALID_ARG
    assert call(n=-1) == bad
    assert call(layers=0) == bad
    assert call(row_bytes=12) == bad
    assert call(row_bytes=0) == bad
    assert call(dev_rows=0) == bad
    assert call(host_rows=0) == bad
    assert call(bs=0) == bad
    assert call(stride=0) == bad
    assert call(dev=None) == bad
    assert call(host=None) == bad
    assert call(src=None) == bad
    assert call(dst=None) == bad
    assert call(dev_rows=1 << 31) == bad
    assert call(dev=P + 8) == bad  # misaligned


def test_apply_plan_validation():
    hs, lib = _lib()
    f = lib.hs_apply_plan
    P = 4096
    ok = dict(hot=P, pool=P, host_rows=100, caches=1, reqs=2, cap=8, row_bytes=1152, rows=P,
              topk=4, idx=P, mc=P, mp=P)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["hot"], a["pool"], a["host_rows"], a["caches"], a["reqs"], a["cap"],
                 a["row_bytes"], a["rows"], a["topk"], a["idx"], a["mc"], a["mp"], None)

    bad = hs.HS_ERR_INVALID_ARG
    for kw in (dict(host_rows=0), dict(caches=0), dict(reqs=0), dict(cap=0), dict(row_bytes=24),
               dict(topk=0), dict(hot=None), dict(pool=None), dict(rows=None), dict(idx=None),
               dict(mc=None), dict(mp=None), dict(host_rows=1 << 31), dict(hot=P + 4)):
        assert call(**kw) == bad, kw


def test_append_validation():
    hs, lib = _lib()
    f = lib.hs_append_accepted
    P = 4096
    ok = dict(cache=P, rows=100, rb=1152, bt=P, bts=4, bs=16, ps=16, ln=P, new=P, acc=P, B=2, R=3)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["cache"], a["rows"], a["rb"], a["bt"], a["bts"], a["bs"], a["ps"], a["ln"],
                 a["new"], a["acc"], a["B"], a["R"], None)

    for kw in (dict(rows=0), dict(rb=8), dict(bts=0), dict(bs=0), dict(ps=0), dict(B=0), dict(R=0),
               dict(cache=None), dict(bt=None), dict(ln=None), dict(new=None), dict(acc=None),
               dict(rows=1 << 31), dict(new=P + 8)):
        assert call(**kw) == hs.HS_ERR_INVALID_ARG, kw


def test_attn_plan_info():
    """The launch the attention calls make, without a GPU: kernel by batch, and key splits."""
    import torch
    hs, lib = _lib()
    plan = lambda rows, heads=128, topk=2048: hs.hs_attn_plan_info(rows, heads, 576, 512, topk,
                                                                   torch.bfloat16)
    assert plan(8) == (32, 8)        # 32 workgroups of (row, 32 heads) -> 8 key splits
    # splits fill the 256 CUs in one round of workgroups, each split at least two tiles
    assert plan(1) == (32, 16) and plan(12) == (32, 5) and plan(20) == (32, 3)
    assert plan(40) == (64, 3) and plan(96) == (64, 1)
    for rows in range(1, 256):
        hpw, splits = plan(rows)
        groups = rows * (128 // hpw)
        assert groups * splits <= 256 if groups <= 256 else splits == 1, rows
    assert plan(20)[0] == 32 and plan(24)[0] == 64 and plan(128)[0] == 64 and plan(129)[0] == 128
    assert plan(128) == (64, 1) and plan(256) == (128, 1) and plan(192) == (128, 1)
    assert plan(8, topk=4500)[1] >= 3  # one split holds at most 2048 keys
    assert plan(40, heads=96)[0] == 32  # 96 heads: only the 32-head kernel
    assert hs.hs_attn_plan_info(4, 4, 64, 48, 16, torch.float32) == (1, 1)
    h, s = ctypes.c_int32(0), ctypes.c_int32(0)
    assert lib.hs_attn_plan_info(0, 128, 576, 512, 2048, hs.HS_BF16, ctypes.byref(h), ctypes.byref(s)) == hs.HS_ERR_INVALID_ARG
    assert lib.hs_attn_plan_info(8, 100, 576, 512, 2048, hs.HS_BF16, None, None) == hs.HS_ERR_UNSUPPORTED
    assert lib.hs_attn_plan_info(8, 128, 576, 512, 2048, 9, None, None) == hs.HS_ERR_INVALID_ARG


def test_attn_plan_info_cus():
    """The launch sized for part of the GPU: at most max_cus workgroups when the chosen
    kernel's (row, head-group) units fit in them with the fewest splits top-k needs, never
    more key splits than the whole-GPU plan (its workspace is enough), and the whole-GPU
    plan at 256 or more."""
    import torch
    hs, lib = _lib()
    plan = lambda rows, heads=128, topk=2048: hs.hs_attn_plan_info(rows, heads, 576, 512, topk,
                                                                   torch.bfloat16)
    cus = lambda rows, c, heads=128, topk=2048: hs.hs_attn_plan_info_cus(
        rows, heads, 576, 512, topk, torch.bfloat16, c)
    assert cus(128, 128) == (128, 1)  # 128 workgroups: the other 128 CUs stay free
    assert cus(64, 192) == (64, 1) and cus(32, 224) == (64, 3)
    for heads in (32, 64, 128, 256):
        for topk in (1, 65, 2048, 4500):
            for rows in (1, 2, 3, 8, 12, 20, 24, 32, 40, 64, 100, 128, 129, 200, 256, 300):
                whole = plan(rows, heads, topk)
                assert cus(rows, 256, heads, topk) == whole and cus(rows, 999, heads, topk) == whole
                for c in (1, 32, 64, 128, 192, 255):
                    hpw, splits = cus(rows, c, heads, topk)
                    units = rows * (heads // hpw)
                    assert splits <= whole[1], (rows, heads, topk, c)
                    if units * -(-topk // 2048) <= c:  # a split holds at most 2048 keys
                        assert units * splits <= c, (rows, heads, topk, c)
    h = ctypes.c_int32(0)
    assert lib.hs_attn_plan_info_cus(8, 128, 576, 512, 2048, hs.HS_BF16, 0, ctypes.byref(h), None) == hs.HS_ERR_INVALID_ARG


def test_binding_rejects_mis_sized_tensors_before_any_call():
    """The Python binding checks that argument shapes agree before it checks devices or calls
    the library, so a mis-sized buffer never reaches a kernel (no GPU needed: the tensors
    here are CPU tensors; correctly sized ones fail the device check instead)."""
    import torch
    hs, _ = _lib()
    i32 = dict(dtype=torch.int32)
    z = lambda *sh, **kw: torch.zeros(sh, **(kw or i32))  # noqa: E731

    def shape_error(fn, *a):
        with pytest.raises(ValueError, match="shape mismatch"):
            fn(*a)

    def device_error(fn, *a):
        with pytest.raises(ValueError, match="device tensor"):
            fn(*a)

    # resolve: per-row vectors and the output must match the position array
    device_error(hs.hs_resolve_topk, z(4, 16), z(4), z(4), z(2, 8), 16, 16, z(4, 16), z(4))
    shape_error(hs.hs_resolve_topk, z(4, 16), z(3), z(4), z(2, 8), 16, 16, z(4, 16))
    shape_error(hs.hs_resolve_topk, z(4, 16), z(4), z(4), z(2, 8), 16, 16, z(4, 15))
    shape_error(hs.hs_resolve_topk, z(4, 16), z(4), z(4), z(2, 8), 16, 16, z(4, 16), z(5))
    # hot state: stamps, reverse map and hot buffer sized from slot_loc and the host pool
    f32 = dict(dtype=torch.float32)

    def state(**kw):
        d = dict(slot_loc=z(2, 24), slot_stamp=z(2, 24), loc_to_hot=z(256),
                 hot_kv=z(48, 64, **f32), host_pool=z(256, 64, **f32))
        d.update(kw)
        return hs.HotState(**d)
    device_error(hs.hs_swap_in, state(), z(2, 16), 5, z(2, 16), z(2))
    shape_error(hs.hs_swap_in, state(slot_stamp=z(2, 23)), z(2, 16), 5, z(2, 16), z(2))
    shape_error(hs.hs_swap_in, state(loc_to_hot=z(255)), z(2, 16), 5, z(2, 16), z(2))
    shape_error(hs.hs_swap_in, state(hot_kv=z(47, 64, **f32)), z(2, 16), 5, z(2, 16), z(2))
    shape_error(hs.hs_swap_in, state(), z(3, 16), 5, z(3, 16), z(3))
    shape_error(hs.hs_swap_in, state(), z(2, 16), 5, z(2, 17), z(2))
    shape_error(hs.hs_swap_in, state(), z(2, 16), 5, z(2, 16), z(3))
    shape_error(hs.hs_swap_in, state(), z(2, 16), 5, z(2, 16), z(2), z(2, 15))
    # attention: kv width, index rows, output and lse shapes
    q = z(3, 4, 64, **f32)
    device_error(hs.hs_sparse_decode_attn, q, z(10, 64, **f32), z(3, 8), 0.1, 48, z(3, 4, 48, **f32), z(3, 4, **f32))
    shape_error(hs.hs_sparse_decode_attn, q, z(10, 32, **f32), z(3, 8), 0.1, 48, z(3, 4, 48, **f32))
    shape_error(hs.hs_sparse_decode_attn, q, z(10, 64, **f32), z(2, 8), 0.1, 48, z(3, 4, 48, **f32))
    shape_error(hs.hs_sparse_decode_attn, q, z(10, 64, **f32), z(3, 8), 0.1, 48, z(3, 4, 47, **f32))
    shape_error(hs.hs_sparse_decode_attn, q, z(10, 64, **f32), z(3, 8), 0.1, 48, z(3, 4, 48, **f32), z(3, 5, **f32))
    shape_error(hs.hs_sparse_decode_attn_paged, q, z(10, 64, **f32), z(3, 8), z(2), z(3), z(2, 4), 16, 16,
                0.1, 48, z(3, 4, 48, **f32))
    shape_error(hs.hs_sparse_decode_attn_mixed, q, z(10, 64, **f32), z(3, 8), z(10, 63, **f32), z(3, 8), z(3),
                0.1, 48, z(3, 4, 48, **f32))
    # finalize: logits, drafts and new rows are num_reqs * rows_per_req long
    fin = lambda st, logits, draft, new_kv, seq: hs.hs_finalize_accepted(  # noqa: E731
        st, logits, draft, new_kv, 3, seq, z(2, 8), 16, 9, z(6), z(2), z(2))
    device_error(fin, state(), z(6, 100, dtype=torch.bfloat16), z(6), z(6, 64, **f32), z(2))
    shape_error(fin, state(), z(5, 100, dtype=torch.bfloat16), z(6), z(6, 64, **f32), z(2))
    shape_error(fin, state(), z(6, 100, dtype=torch.bfloat16), z(7), z(6, 64, **f32), z(2))
    shape_error(fin, state(), z(6, 100, dtype=torch.bfloat16), z(6), z(6, 32, **f32), z(2))
    shape_error(fin, state(), z(6, 100, dtype=torch.bfloat16), z(6), z(6, 64, **f32), z(3))
