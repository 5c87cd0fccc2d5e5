"""Shared test helpers: raw numpy views of generated workloads, state invariants."""

from __future__ import annotations

import numpy as np
import torch


def raw(t: torch.Tensor) -> np.ndarray:
    """Raw elements of a CPU tensor: uint16 bit patterns for bf16, float32 as is."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def check_state_invariants(st, host_pool_raw: np.ndarray):
    """Hot-buffer invariants that hold after every swap-in / finalize call."""
    B, cap = st.slot_loc.shape
    occ = st.slot_loc >= 0
    # slot_loc and loc_to_hot are mutually inverse on occupied slots
    bs, ss = np.nonzero(occ)
    rows = st.slot_loc[bs, ss]
    assert len(np.unique(rows)) == len(rows), "a host row is held by two slots"
    assert (st.loc_to_hot[rows] == bs * cap + ss).all()
    mapped = np.nonzero(st.loc_to_hot >= 0)[0]
    assert len(mapped) == occ.sum()
    g = st.loc_to_hot[mapped]
    assert (st.slot_loc.reshape(-1)[g] == mapped).all()
    # empty slots carry stamp -1; occupied slots a real tick
    assert (st.slot_stamp[~occ] == -1).all()
    assert (st.slot_stamp[occ] >= 0).all()
    # the device buffer holds exactly the host rows it claims to
    flat = st.slot_loc.reshape(-1)
    o = np.nonzero(flat >= 0)[0]
    assert np.array_equal(st.hot_kv[o], host_pool_raw[flat[o]])


def with_duplicates(wave: np.ndarray) -> np.ndarray:
    """A copy of a swap wave in which rows repeat within each request: entry 4i+1 repeats entry
    4i and entry 4i+3 repeats entry 4i (three copies)."""
    out = wave.copy()
    n1 = len(out[:, 1::4][0])
    out[:, 1::4] = wave[:, 0::4][:, :n1]
    n3 = len(out[:, 3::4][0])
    out[:, 3::4] = wave[:, 0::4][:, :n3]
    return out


def check_state_weak(st, host_pool_raw: np.ndarray):
    """What holds after waves that repeat a row within a request: a row may sit in several
    slots of its request and the map names at most one of them, but a mapped row's slot holds
    that row, and every occupied slot holds the bytes of the row it names."""
    B, cap = st.slot_loc.shape
    flat = st.slot_loc.reshape(-1)
    mapped = np.nonzero(st.loc_to_hot >= 0)[0]
    g = st.loc_to_hot[mapped]
    assert (g < B * cap).all()
    assert (flat[g] == mapped).all(), "a mapped row's slot holds another row"
    occ = st.slot_loc >= 0
    assert (st.slot_stamp[~occ] == -1).all()
    assert (st.slot_stamp[occ] >= 0).all()
    o = np.nonzero(flat >= 0)[0]
    assert np.array_equal(st.hot_kv[o], host_pool_raw[flat[o]])
