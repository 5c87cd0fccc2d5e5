"""Reference (oracle) implementation of the HiSparse decode calls and the host backup.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the benchmark's
CPU-baseline leg.  numpy only; float64 for every floating-point step.

Conventions shared with the caller (not with the GPU code):

* Query rows are wave-major: row ``r * num_reqs + b`` is row ``r`` (0 = the
  decode anchor, 1.. = draft rows being verified) of request ``b``.
* KV rows are stored raw: ``uint16`` bit patterns for bf16, ``float32`` for f32.
  Copies move raw elements (bit-exact); arithmetic upcasts exactly to float64.
* Parity status: every function here is pinned (see ``tests/test_oracle_*.py``).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def as_f64(raw: np.ndarray) -> np.ndarray:
    """Exact float64 value of raw KV/query/logit elements (uint16 = bf16 bits, or float32)."""
    if raw.dtype == np.uint16:
        return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if raw.dtype == np.float32:
        return raw.astype(np.float64)
    raise TypeError(f"unsupported raw dtype {raw.dtype}")


# --------------------------------------------------------------------------------------
# 1. resolve_topk
# --------------------------------------------------------------------------------------
def resolve_topk(topk_pos: np.ndarray, req_id: np.ndarray, causal_limit: np.ndarray,
                 block_table: np.ndarray, block_size: int, physical_block_stride: int,
                 num_reqs: int):
    """Request-local top-k token positions -> physical KV rows.

    P3, ``HiSparseCacheHandle.resolve_topk`` listing: in the fully-resident branch the
    per-row top-k indices are converted to global cache slots through the request's
    block table (block size and physical block stride given), optionally with a
    per-row count of valid entries.  P3 "数据 back up": the rows of physical block
    ``p`` are ``p * block_size + offset`` for ``offset`` in ``[0, block_size)``.

    Reading (the converter's body is not printed): position ``t`` of row ``i`` is valid
    iff ``0 <= t < causal_limit[i]``, its page index ``t // block_size`` is inside the
    table row and the table entry is a page (>= 0), and the row's request id is in
    range.  A valid entry maps to ``page * physical_block_stride + t % block_size``;
    anything else becomes -1 in place (no compaction).  ``valid[i]`` counts the
    non-negative outputs.
    """
    rows, K = topk_pos.shape
    bt_stride = block_table.shape[1]
    slots = np.full((rows, K), -1, dtype=np.int64)
    valid = np.zeros(rows, dtype=np.int32)
    for i in range(rows):
        b = int(req_id[i])
        if b < 0 or b >= num_reqs:
            continue
        t = topk_pos[i].astype(np.int64)
        ok = (t >= 0) & (t < int(causal_limit[i]))
        page_idx = np.where(ok, t // block_size, 0)
        ok &= page_idx < bt_stride
        page = np.where(ok, block_table[b, np.minimum(page_idx, bt_stride - 1)], -1).astype(np.int64)
        ok &= page >= 0
        slots[i] = np.where(ok, page * physical_block_stride + t % block_size, -1)
        valid[i] = int(ok.sum())
    assert slots.max(initial=-1) < 2 ** 31
    return slots.astype(np.int32), valid


# --------------------------------------------------------------------------------------
# 2. hot-buffer state and swap_in
# --------------------------------------------------------------------------------------
@dataclass
class HotState:
    """Per-request HiSparse hot buffer (P1 "1. 启动阶段", core-state list).

    ``slot_loc[b, s]``   host row held by slot ``s`` of request ``b`` (-1: empty) -- the
                         slot -> physical KV loc map;
    ``slot_stamp[b, s]`` LRU tick of the slot's last use (-1: empty) -- "LRU slots";
    ``loc_to_hot[row]``  ``b * capacity + s`` holding host row ``row``, or -1 -- the
                         logical loc -> physical HiSparse slot map;
    ``hot_kv[b*cap+s]``  the KV row held in that slot (the device buffer).
    Slot range of request ``b`` is ``[b*cap, (b+1)*cap)`` (req -> physical slots); its
    size is fixed per request as in P3's ``HiSparseHotSpec`` (blocks_per_request).
    """
    capacity: int
    slot_loc: np.ndarray
    slot_stamp: np.ndarray
    loc_to_hot: np.ndarray
    hot_kv: np.ndarray

    def copy(self) -> "HotState":
        return HotState(self.capacity, self.slot_loc.copy(), self.slot_stamp.copy(),
                        self.loc_to_hot.copy(), self.hot_kv.copy())


def build_hot_state(init_pos: np.ndarray, init_stamp: np.ndarray, seq_len: np.ndarray,
                    block_table: np.ndarray, block_size: int, host_pool: np.ndarray) -> HotState:
    """Hot-buffer state from a position-level description (slot -> token position)."""
    B, cap = init_pos.shape
    rows, _ = resolve_topk(init_pos, np.arange(B, dtype=np.int32), seq_len.astype(np.int32),
                           block_table, block_size, block_size, B)
    loc_to_hot = np.full(host_pool.shape[0], -1, dtype=np.int32)
    hot_kv = np.zeros((B * cap, host_pool.shape[1]), dtype=host_pool.dtype)
    for b in range(B):
        for s in range(cap):
            if rows[b, s] >= 0:
                loc_to_hot[rows[b, s]] = b * cap + s
                hot_kv[b * cap + s] = host_pool[rows[b, s]]
    stamps = np.where(rows >= 0, init_stamp, -1).astype(np.int32)
    return HotState(cap, rows.astype(np.int32), stamps, loc_to_hot, hot_kv)


def _lru_victims(stamps: np.ndarray, pinned: np.ndarray, count: int) -> np.ndarray:
    """The ``count`` least-recently-used unpinned slots, returned in ascending slot order.

    Recency order is (stamp ascending, slot ascending); empty slots carry stamp -1 and
    so are taken first.
    """
    cand = np.nonzero(~pinned)[0]
    if len(cand) < count:
        raise ValueError("hot buffer capacity exceeded")
    order = np.lexsort((cand, stamps[cand]))
    return np.sort(cand[order[:count]])


def swap_in(st: HotState, wave_rows: np.ndarray, tick: int, host_pool: np.ndarray):
    """One wave of swap-in: row ``b`` of ``wave_rows`` holds request ``b``'s resolved host rows.

    P3 ``resolve_topk`` listing: when the batch is not fully resident, the selected
    KV is brought into the hot cache (``runtime.swap_in``) and indices into that cache
    are returned.  P1 startup: the coordinator keeps a device buffer, a host pool and
    LRU slots per request.  The swap algorithm itself is not printed; the reading:

    1. entry ``j`` is valid iff ``0 <= L[j] < host_rows``; it hits iff
       ``loc_to_hot[L[j]] >= 0``; misses are listed in ascending ``j``;
    2. hit slots are pinned for this wave; the victims are the ``#misses``
       least-recently-used unpinned slots (stamp, then slot, ascending);
    3. miss ``m`` goes to the ``m``-th victim in ascending slot order, applied in that
       order: the evicted row's map entry is cleared if it names the evicted slot, the
       new row is mapped to its slot, its KV copied bitwise;
    4. every valid entry's slot gets stamp ``tick``; ``hot_idx = b*cap + slot``.

    A host row belongs to one request (no shared prefix pages): a row of request ``b``
    mapped into another request's slots is a caller error (``ValueError``).  Rows
    repeated within a request (top-k sets never repeat) follow from the order in 3:
    each copy of a miss takes its own victim and the map names the last one installed.

    Mutates ``st``.  Returns ``(hot_idx [B,K], miss_count [B], miss_pos [B,K])``
    (``miss_pos`` is -1 past ``miss_count``).
    """
    B, K = wave_rows.shape
    cap = st.capacity
    host_rows = host_pool.shape[0]
    hot_idx = np.full((B, K), -1, dtype=np.int32)
    miss_count = np.zeros(B, dtype=np.int32)
    miss_pos = np.full((B, K), -1, dtype=np.int32)
    for b in range(B):
        L = wave_rows[b].astype(np.int64)
        valid = (L >= 0) & (L < host_rows)
        hotg = np.full(K, -1, dtype=np.int64)
        hotg[valid] = st.loc_to_hot[L[valid]]
        hit = valid & (hotg >= 0)
        miss = valid & (hotg < 0)
        if ((hotg[hit] < b * cap) | (hotg[hit] >= (b + 1) * cap)).any():
            raise ValueError(f"request {b} selects a host row mapped into another request's slots")
        M = np.nonzero(miss)[0]
        slot = np.full(K, -1, dtype=np.int64)
        slot[hit] = hotg[hit] - b * cap
        pinned = np.zeros(cap, dtype=bool)
        pinned[slot[hit]] = True
        V = _lru_victims(st.slot_stamp[b], pinned, len(M))
        for m in range(len(M)):
            v, j = int(V[m]), int(M[m])
            old = int(st.slot_loc[b, v])
            if old >= 0 and st.loc_to_hot[old] == b * cap + v:
                st.loc_to_hot[old] = -1
            st.slot_loc[b, v] = L[j]
            st.loc_to_hot[L[j]] = b * cap + v
            st.hot_kv[b * cap + v] = host_pool[L[j]]
            slot[j] = v
        st.slot_stamp[b, slot[valid]] = tick
        hot_idx[b, valid] = b * cap + slot[valid]
        miss_count[b] = len(M)
        miss_pos[b, :len(M)] = M
    return hot_idx, miss_count, miss_pos


def apply_plan(hot_kv: np.ndarray, host_pool: np.ndarray, wave_rows: np.ndarray,
               hot_idx: np.ndarray, miss_count: np.ndarray, miss_pos: np.ndarray):
    """A follower cache applies the leader's swap plan; returns its new hot buffers.

    P3 ``resolve_topk`` listing: a runtime with a leader returns ``apply_plan(...)``
    instead of swapping itself; the leader's ``swap_in`` produces the plan for its
    followers (and with ``prefetch_followers`` fills them).  Reading: the plan of one wave
    is the leader's ``(hot_idx, miss_count, miss_pos)``; a follower shares the slot
    assignment but has its own hot buffer and host pool, so for every cache ``c``, request
    ``b`` and ``m < miss_count[b]``, with ``e = miss_pos[b, m]``, row ``wave_rows[b, e]``
    of ``host_pool[c]`` is copied bitwise to row ``hot_idx[b, e]`` of ``hot_kv[c]``.
    Entries out of range are skipped.

    ``hot_kv`` [C, B*cap, E] raw (not modified), ``host_pool`` [C, host_rows, E] raw.
    """
    out = hot_kv.copy()
    C, hot_rows = hot_kv.shape[0], hot_kv.shape[1]
    host_rows = host_pool.shape[1]
    B, K = wave_rows.shape
    for c in range(C):
        for b in range(B):
            for m in range(min(max(int(miss_count[b]), 0), K)):
                e = int(miss_pos[b, m])
                if e < 0 or e >= K:
                    continue
                row, g = int(wave_rows[b, e]), int(hot_idx[b, e])
                if 0 <= row < host_rows and 0 <= g < hot_rows:
                    out[c, g] = host_pool[c, row]
    return out


# --------------------------------------------------------------------------------------
# 3. sparse decode attention
# --------------------------------------------------------------------------------------
def sparse_decode_attn(q: np.ndarray, kv: np.ndarray, indices: np.ndarray, scale: float,
                       d_v: int):
    """Attention of each query row over only its selected KV rows.

    P1 startup: the DSA attention backend reads KV through HiSparse; P3
    ``resolve_topk``: attention receives the cache plus per-row indices (-1 padded).
    Reading: per row ``i`` and head ``h``, over ``S_i = {j : 0 <= idx[i,j] < kv_rows}``
    (duplicates count as separate terms), ``s_j = scale * <q[i,h,:], kv[idx_j, :]>``,
    ``p = softmax(s)`` (max-subtracted), ``o = sum_j p_j * kv[idx_j, :d_v]`` (the value
    is the leading ``d_v`` entries of the same latent row); ``lse = log sum_j exp(s_j)``.
    An empty set gives ``o = 0``, ``lse = -inf``.  float64 throughout.

    ``q``: raw [rows, H, D]; ``kv``: raw [kv_rows, D].  Returns float64
    ``(out [rows, H, d_v], lse [rows, H])``.
    """
    rows, H, D = q.shape
    kv_rows = kv.shape[0]
    out = np.zeros((rows, H, d_v), dtype=np.float64)
    lse = np.full((rows, H), -np.inf, dtype=np.float64)
    for i in range(rows):
        idx = indices[i].astype(np.int64)
        sel = idx[(idx >= 0) & (idx < kv_rows)]
        if len(sel) == 0:
            continue
        keys = as_f64(kv[sel])                          # [n, D]
        s = scale * (as_f64(q[i]) @ keys.T)             # [H, n]
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        out[i] = (p @ keys[:, :d_v]) / l
        lse[i] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def sparse_decode_attn_mixed(q: np.ndarray, kv_a: np.ndarray, idx_a: np.ndarray,
                             kv_b: np.ndarray, idx_b: np.ndarray, row_sel: np.ndarray,
                             scale: float, d_v: int):
    """Attention of a batch whose rows read one of two caches.

    P3 resolve_topk listing: a fully resident batch reads the resident cache, any other
    batch the hot cache after swap-in; P3 reclaim_resident_blocks: a request whose resident
    pages were reclaimed is no longer fully resident.  Reading (per-request residency): row
    ``i`` is attended exactly as ``sparse_decode_attn`` over ``(kv_b, idx_b[i])`` when
    ``row_sel[i] != 0``, else over ``(kv_a, idx_a[i])``.  Returns ``(out, lse)`` float64.
    """
    rows, H, _ = q.shape
    out = np.zeros((rows, H, d_v), dtype=np.float64)
    lse = np.full((rows, H), -np.inf, dtype=np.float64)
    for i in range(rows):
        kv, idx = (kv_b, idx_b) if row_sel[i] != 0 else (kv_a, idx_a)
        o, l = sparse_decode_attn(q[i:i + 1], kv, idx[i:i + 1], scale, d_v)
        out[i], lse[i] = o[0], l[0]
    return out, lse


def reclaimable_pages(block_table: np.ndarray, seq_len: np.ndarray, block_size: int):
    """Resident pages the coordinator may reclaim: P3 reclaim_resident_blocks, where the
    resident manager scans every request and offers its older blocks, never the last two.

    Reading: request ``b`` uses pages ``0 .. ceil(seq_len[b] / block_size) - 1``; the mapped
    ones (table entry >= 0) below index ``used - 2`` are offered, as ``(b, page_index)``
    in request then page order."""
    out = []
    for b in range(block_table.shape[0]):
        used = -(-int(seq_len[b]) // block_size)
        for p in range(max(0, used - 2)):
            if block_table[b, p] >= 0:
                out.append((b, p))
    return out


def select_reclaim_pages(block_table: np.ndarray, seq_len: np.ndarray, block_size: int,
                         deficit: int, priority=None, hot_pages=None):
    """The resident pages to give back when the cache manager is ``deficit`` blocks short.

    P3 reclaim_resident_blocks: allocation fails for lack of blocks; the coordinator is asked
    to reclaim that many; the resident manager offers every request's older pages (never
    the last two); the coordinator screens them by priority, hot pages and budget and
    releases the chosen ones (the table entry becomes null, the block returns to the pool);
    allocation then checks its capacity again.

    Reading (the screening is not printed): the candidates are ``reclaimable_pages``; a page
    marked in ``hot_pages`` ([num_reqs, bt_stride] bool, e.g. pages the latest top-k
    selections touched) is screened out; the rest are taken in the order (request priority
    ascending -- ``priority[b]``, default 0, the larger the longer a request keeps its pages
    --, page index ascending, i.e. oldest first, then request id), and the budget is the
    deficit: the first ``min(deficit, #candidates)`` are returned as ``(b, page_index)``.
    Fewer than ``deficit`` means the allocation still fails; that is the caller's concern.
    """
    nreq = block_table.shape[0]
    prio = np.zeros(nreq, dtype=np.int64) if priority is None else np.asarray(priority, np.int64)
    cand = [(int(prio[b]), p, b) for (b, p) in reclaimable_pages(block_table, seq_len, block_size)
            if hot_pages is None or not hot_pages[b, p]]
    cand.sort()
    return [(b, p) for (_, p, b) in cand[:max(0, int(deficit))]]


def is_fully_resident(block_table: np.ndarray, seq_len: np.ndarray, block_size: int) -> np.ndarray:
    """Per request: every page that holds one of its tokens is still mapped in the resident
    pool (P3: once any of a request's resident KV is reclaimed, fully_resident is false;
    are_requests_fully_resident asks it of every request of a batch)."""
    res = np.zeros(block_table.shape[0], dtype=bool)
    for b in range(block_table.shape[0]):
        used = -(-int(seq_len[b]) // block_size)
        res[b] = used <= block_table.shape[1] and bool((block_table[b, :used] >= 0).all())
    return res


# --------------------------------------------------------------------------------------
# 4. greedy accept + accepted-prefix finalize
# --------------------------------------------------------------------------------------
def greedy_accept(logits: np.ndarray, draft_ids: np.ndarray, num_reqs: int, rows_per_req: int):
    """Greedy verification of the draft rows.

    P2 ④ (target verify): the target runs the anchor and the drafts in one causal
    pass; the logits of row ``r`` judge draft ``r+1``; a draft is kept while it equals
    the target's greedy choice, the first mismatch is replaced by the target's token
    and everything after it is dropped; if every draft passes, the last row's logits
    give one extra token.

    Reading: ``am[i]`` = lowest index of the row maximum (NaN never wins);
    ``L_b`` = longest ``l <= R-1`` with ``draft[row(b,k)] == am[row(b,k-1)]`` for
    ``1 <= k <= l``; ``next_token[b] = am[row(b, L_b)]``.
    Returns ``(accept_len [B], next_token [B], argmax [rows])``.
    """
    vals = as_f64(logits)
    vals = np.where(np.isnan(vals), -np.inf, vals)
    rows = vals.shape[0]
    am = np.empty(rows, dtype=np.int32)
    for i in range(rows):
        m = vals[i].max()
        am[i] = int(np.nonzero(vals[i] == m)[0][0])
    B, R = num_reqs, rows_per_req
    acc = np.zeros(B, dtype=np.int32)
    nxt = np.zeros(B, dtype=np.int32)
    for b in range(B):
        L = 0
        while L < R - 1 and int(draft_ids[(L + 1) * B + b]) == int(am[L * B + b]):
            L += 1
        acc[b] = L
        nxt[b] = am[L * B + b]
    return acc, nxt, am


def finalize_accepted(st: HotState, host_pool: np.ndarray, new_kv: np.ndarray,
                      accept_len: np.ndarray, seq_len: np.ndarray, block_table: np.ndarray,
                      block_size: int, rows_per_req: int, tick: int) -> np.ndarray:
    """Keep exactly the target-verified prefix's KV.

    P2 ④: although KV was computed for every verify row, only the accepted prefix
    (anchor plus accepted drafts) stays in the target cache; the replacement token has
    no KV yet.  P2 ⑥ and the timeline table: the next anchor sits right after the kept
    prefix.  P1 summary: accepted-KV finalize is the last stage of the main line.

    Reading: request ``b`` has ``n = seq_len[b] - R`` committed positions; verify row
    ``r`` sits at position ``n + r``.  Rows ``r > L_b`` are discarded: a hot slot holding
    that position is emptied (map cleared, stamp -1); its host row is left alone.  Rows
    ``r <= L_b`` are kept: ``new_kv`` is written to the position's host row and to the
    hot buffer (overwrite if resident, else install with the swap-in victim rule, the
    slots of this request's resident kept rows pinned, an evicted row's map entry
    cleared if it names the evicted slot), stamp ``tick``.  Rejected rows are processed
    before kept rows.  As in ``swap_in``, a row mapped into another request's slots is a
    caller error.  Returns ``committed = n + L_b + 1`` per request.
    Mutates ``st`` and ``host_pool``.
    """
    B, R, cap = len(seq_len), rows_per_req, st.capacity
    committed = np.zeros(B, dtype=np.int64)
    for b in range(B):
        n = int(seq_len[b]) - R
        L = int(accept_len[b])
        pos = np.array([n + r for r in range(R)], dtype=np.int32)
        locs, _ = resolve_topk(pos[None, :], np.array([b], np.int32),
                               np.array([seq_len[b]], np.int32), block_table,
                               block_size, block_size, B)
        locs = locs[0]
        for r in range(L + 1, R):
            loc = int(locs[r])
            if loc >= 0 and st.loc_to_hot[loc] >= 0:
                if not b * cap <= st.loc_to_hot[loc] < (b + 1) * cap:
                    raise ValueError(f"request {b} drops a host row mapped into another "
                                     "request's slots")
                s = int(st.loc_to_hot[loc]) - b * cap
                st.slot_loc[b, s] = -1
                st.slot_stamp[b, s] = -1
                st.loc_to_hot[loc] = -1
        kept = [r for r in range(L + 1) if locs[r] >= 0]
        pinned = np.zeros(cap, dtype=bool)
        miss_rows = []
        for r in kept:
            loc = int(locs[r])
            host_pool[loc] = new_kv[r * B + b]
            g = int(st.loc_to_hot[loc])
            if g >= 0 and not b * cap <= g < (b + 1) * cap:
                raise ValueError(f"request {b} keeps a host row mapped into another request's slots")
            if g >= 0:
                pinned[g - b * cap] = True
                st.hot_kv[g] = new_kv[r * B + b]
                st.slot_stamp[b, g - b * cap] = tick
            else:
                miss_rows.append(r)
        V = _lru_victims(st.slot_stamp[b], pinned, len(miss_rows))
        for m, r in enumerate(miss_rows):
            v, loc = int(V[m]), int(locs[r])
            old = int(st.slot_loc[b, v])
            if old >= 0 and st.loc_to_hot[old] == b * cap + v:
                st.loc_to_hot[old] = -1
            st.slot_loc[b, v] = loc
            st.loc_to_hot[loc] = b * cap + v
            st.hot_kv[b * cap + v] = new_kv[r * B + b]
            st.slot_stamp[b, v] = tick
        committed[b] = n + L + 1
    return committed


# --------------------------------------------------------------------------------------
# 5. device -> host backup (prefill staging, page spills)
# --------------------------------------------------------------------------------------
@dataclass
class PageTransfer:
    """One page spill as P3's ``SparseKVPageTransfer``: the source block of every cache
    (``source_block_ids``), the destination host block and the page inside it."""
    source_block_ids: tuple
    destination_block_id: int
    destination_page_offset: int


def plan_backup_rows(transfers, kernel_block_size: int, blocks_per_kv_block: int,
                     num_caches: int):
    """Page transfers -> row lists, as P3 "数据 back up" (``HiSparseWorker._enqueue_transfers``)
    fills its staging arrays.

    Transfer ``t`` owns entries ``[t*kbs, (t+1)*kbs)``.  For cache ``c`` the source rows
    are ``source_block_ids[c] * kbs + offset``; the host page is
    ``destination_block_id * blocks_per_kv_block + destination_page_offset`` and the
    destination rows are ``host_page * kbs + offset``, for ``offset`` in ``[0, kbs)``.
    Returns ``(src [num_caches, n], dst [n])`` as int64.
    """
    kbs = kernel_block_size
    n = len(transfers) * kbs
    src = np.zeros((num_caches, n), dtype=np.int64)
    dst = np.zeros(n, dtype=np.int64)
    for t, tr in enumerate(transfers):
        for off in range(kbs):
            e = t * kbs + off
            for c in range(num_caches):
                src[c, e] = tr.source_block_ids[c] * kbs + off
            host_page = tr.destination_block_id * blocks_per_kv_block + tr.destination_page_offset
            dst[e] = host_page * kbs + off
    return src, dst


def backup_rows(dev_cache: np.ndarray, host_cache: np.ndarray, src_slots: np.ndarray,
                dst_rows: np.ndarray, src_block_size: int = 1, src_block_stride: int = 1):
    """Copy the listed device rows into the host cache, every layer; returns the new host cache.

    P3 "数据 back up": the backup op copies, for each cache (layer), the rows named by the
    source slot list into the host cache rows named by the destination list; the slot of
    block ``b`` at offset ``o`` lives at physical row ``b * block_stride + o`` of the device
    cache (the op takes the source block size and stride).  P1 "3. HiSparse staging": this
    is how prefill KV reaches the host pool.

    ``dev_cache`` [L, dev_rows, E] raw, ``host_cache`` [L, host_rows, E] raw (not modified),
    ``src_slots`` [L, n] or [n] (shared by all layers), ``dst_rows`` [n].  Reading: an entry
    whose slot or destination is negative or out of range is skipped; rows are copied bit
    for bit; entries are applied in order (a repeated destination keeps the last source).
    """
    out = host_cache.copy()
    L, dev_rows = dev_cache.shape[0], dev_cache.shape[1]
    host_rows = host_cache.shape[1]
    n = len(dst_rows)
    per_layer = src_slots.ndim == 2
    for layer in range(L):
        for i in range(n):
            s = int(src_slots[layer, i] if per_layer else src_slots[i])
            d = int(dst_rows[i])
            if s < 0 or d < 0 or d >= host_rows:
                continue
            p = (s // src_block_size) * src_block_stride + s % src_block_size
            if p >= dev_rows:
                continue
            out[layer, d] = dev_cache[layer, p]
    return out


# --------------------------------------------------------------------------------------
# 6. draft-model context KV append
# --------------------------------------------------------------------------------------
def append_accepted(ctx_cache: np.ndarray, ctx_block_table: np.ndarray, ctx_len: np.ndarray,
                    new_rows: np.ndarray, accept_len: np.ndarray, rows_per_req: int,
                    block_size: int, physical_block_stride: int):
    """The draft model's context cache grows by each request's accepted prefix.

    P2 ⑤: after target verification, only the accepted prefix's target features go
    through the draft model's context K/V branch and are appended to its context cache
    (``KV_D(P) -> KV_D(P + [a0, b1])``); the KV of the draft round is not used.  ⑥ and the
    timeline table: the context then covers the confirmed positions except the newest
    token.  Reading: verify rows are wave-major (row ``r * B + b``); with
    ``L = clamp(accept_len[b], 0, rows_per_req - 1)``, rows ``r = 0 .. L`` go to positions
    ``ctx_len[b] + r`` through the block table (row ``page * stride + pos % block_size``);
    unmapped positions are skipped; ``ctx_len[b]`` advances by ``L + 1``.
    Returns ``(new ctx_cache, new ctx_len)``; the inputs are not modified.
    """
    cache = ctx_cache.copy()
    lens = np.array(ctx_len, dtype=np.int64, copy=True)
    B = len(ctx_len)
    for b in range(B):
        L = min(max(int(accept_len[b]), 0), rows_per_req - 1)
        for r in range(L + 1):
            pos = int(ctx_len[b]) + r
            pidx = pos // block_size
            if pos < 0 or pidx >= ctx_block_table.shape[1]:
                continue
            page = int(ctx_block_table[b, pidx])
            if page < 0:
                continue
            row = page * physical_block_stride + pos % block_size
            if row < cache.shape[0]:
                cache[row] = new_rows[r * B + b]
        lens[b] = int(ctx_len[b]) + L + 1
    return cache, lens
