"""Decode-step driver over the C ABI: buffers, streams and events for one step.

Per step (P1 "hiSparse-MTP" summary: decode, then MTP verify, then accepted-KV
finalize; P3 "vllm 分析（十二）——Hisparse下篇" resolve_topk listing: the fully
resident batch reads the paged device cache directly, otherwise KV is swapped in):

  resident batch:  hs_resolve_topk(all rows) -> hs_sparse_decode_attn(paged pool)
  swap batch:      hs_resolve_topk(all rows) on the main stream, then for each wave r
                   (row r of every request): hs_swap_in on the copy stream, attention
                   of wave r on the main stream once that swap has landed; the swap of
                   wave r+1 overlaps the attention of wave r, which is then sized for
                   the CUs that swap leaves free (hs_sparse_decode_attn_cus).
                   hs_finalize_accepted closes the step when draft rows are verified.

The copy stream waits for the attention of wave r-2 before swapping wave r.  That is safe
when capacity >= 2*topk and tick0 is above every stamp already in the state: wave r-1's
slots then carry the newest stamp, and at least #misses unpinned slots are older, so none
of them is a victim of wave r.  The state's host-side record (HotState.max_stamp, set by
build_hot_state and advanced by every wrapper call) decides it; with a smaller hot buffer,
a tick0 not above that record, or no record, the copy stream waits for wave r-1 instead.
Both streams run at the default priority.

Mixed batch (P3 reclaim_resident_blocks, build_offload_command): ResidencyTracker keeps
the resident block table and tells which requests are still fully resident; run_mixed lets
those read the resident pool while the rest swap in, instead of one switch per batch.

Backup (P1 "3. HiSparse staging", P3 "数据 back up"): BackupStager turns page transfers
into row lists in pinned staging buffers, copies them to the device without blocking,
launches hs_backup_rows and records an event that `ready` polls.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

from . import (HotState, hs_append_accepted, hs_attn_workspace_bytes, hs_backup_rows,
               hs_finalize_accepted, hs_greedy_argmax,
               hs_resolve_topk, hs_sparse_decode_attn, hs_sparse_decode_attn_cus,
               hs_sparse_decode_attn_mixed, hs_sparse_decode_attn_paged, hs_swap_in)


def build_hot_state(init_pos: torch.Tensor, init_stamp: torch.Tensor, seq_len: torch.Tensor,
                    block_table: torch.Tensor, block_size: int, host_pool: torch.Tensor,
                    device: torch.device) -> HotState:
    """Hot buffer from a slot -> token-position description (a request admitted with
    some of its KV already resident).  Positions are mapped to host rows with
    hs_resolve_topk; the reverse map and the resident rows are filled with plain torch
    indexing (setup, not part of a step)."""
    B, cap = init_pos.shape
    pos = init_pos.to(device=device, dtype=torch.int32).contiguous()
    req = torch.arange(B, dtype=torch.int32, device=device)
    slot_loc = torch.empty((B, cap), dtype=torch.int32, device=device)
    hs_resolve_topk(pos, req, seq_len.to(device=device, dtype=torch.int32).contiguous(),
                    block_table, block_size, block_size, slot_loc)
    stamps = torch.where(slot_loc >= 0, init_stamp.to(device=device, dtype=torch.int32),
                         torch.full_like(slot_loc, -1)).contiguous()
    max_stamp = int(stamps.max().item()) if stamps.numel() else -1
    host_rows = host_pool.shape[0]
    loc_to_hot = torch.full((host_rows,), -1, dtype=torch.int32, device=device)
    flat = slot_loc.view(-1)
    occ = flat >= 0
    gidx = torch.arange(B * cap, dtype=torch.int32, device=device)
    loc_to_hot[flat[occ].long()] = gidx[occ]
    hot_kv = torch.zeros((B * cap, host_pool.shape[1]), dtype=host_pool.dtype, device=device)
    rows_cpu = flat[occ].long().cpu()
    if rows_cpu.numel():
        hot_kv[occ] = host_pool.index_select(0, rows_cpu).to(device)
    return HotState(slot_loc, stamps, loc_to_hot, hot_kv, host_pool, max_stamp=max_stamp)


@dataclass
class StepBuffers:
    slots: torch.Tensor          # [rows, topk] int32
    valid: torch.Tensor          # [rows] int32
    hot_idx: Optional[torch.Tensor]
    miss_count: Optional[torch.Tensor]  # [R, B]
    miss_pos: Optional[torch.Tensor]
    out: torch.Tensor            # [rows, H, d_v]
    lse: torch.Tensor            # [rows, H] fp32
    workspace: Optional[torch.Tensor]
    argmax: Optional[torch.Tensor] = None
    accept_len: Optional[torch.Tensor] = None
    next_token: Optional[torch.Tensor] = None
    slots_res: Optional[torch.Tensor] = None  # [rows, topk] resident-pool rows (mixed batch)


class DecodeStep:
    """Preallocated buffers + streams for repeated decode steps of one shape."""

    def __init__(self, *, num_reqs: int, rows_per_req: int, topk: int, num_heads: int,
                 d_qk: int, d_v: int, dtype: torch.dtype, capacity: int = 0,
                 finalize: bool = False, want_miss_pos: bool = False, mixed: bool = False,
                 device: torch.device = torch.device("cuda")):
        self.B, self.R, self.K = num_reqs, rows_per_req, topk
        self.H, self.d_qk, self.d_v, self.dtype = num_heads, d_qk, d_v, dtype
        self.capacity, self.device = capacity, device
        rows = num_reqs * rows_per_req
        i32 = dict(dtype=torch.int32, device=device)
        swap = capacity > 0
        # attention runs per wave on the swap path, over all rows on the resident path
        attn_rows = num_reqs if swap else rows
        ws = hs_attn_workspace_bytes(attn_rows, num_heads, d_qk, d_v, topk, dtype)
        self.buf = StepBuffers(
            slots=torch.empty((rows, topk), **i32),
            valid=torch.empty((rows,), **i32),
            hot_idx=torch.empty((rows, topk), **i32) if swap else None,
            miss_count=torch.empty((rows_per_req, num_reqs), **i32) if swap else None,
            miss_pos=torch.empty((rows, topk), **i32) if (swap and want_miss_pos) else None,
            out=torch.empty((rows, num_heads, d_v), dtype=dtype, device=device),
            lse=torch.empty((rows, num_heads), dtype=torch.float32, device=device),
            workspace=torch.empty((max(ws, 16),), dtype=torch.uint8, device=device) if ws else None,
            argmax=torch.empty((rows,), **i32) if finalize else None,
            accept_len=torch.empty((num_reqs,), **i32) if finalize else None,
            next_token=torch.empty((num_reqs,), **i32) if finalize else None,
            slots_res=torch.empty((rows, topk), **i32) if (swap and mixed) else None,
        )
        self.copy_stream = torch.cuda.Stream(device=device) if swap else None
        # An attention workgroup holds a whole CU and a swap-in workgroup (one per request)
        # needs one too: an attention that runs beside the next wave's swap-in is sized for
        # the CUs that swap leaves free, so the swap never waits for the attention to drain.
        cus = torch.cuda.get_device_properties(device).multi_processor_count if swap else 0
        self.cus_beside_swap = max(64, cus - num_reqs)
        self.e_resolve = torch.cuda.Event()
        self.e_swap = [torch.cuda.Event() for _ in range(rows_per_req)]
        self.e_attn = [torch.cuda.Event() for _ in range(rows_per_req)]

    # -- resident batch ---------------------------------------------------------------
    def run_resident(self, topk_pos, req_id, causal_limit, block_table, block_size, q, kv_pool,
                     scale):
        b = self.buf
        hs_resolve_topk(topk_pos, req_id, causal_limit, block_table, block_size, block_size,
                        b.slots, b.valid)
        hs_sparse_decode_attn(q, kv_pool, b.slots, scale, self.d_v, b.out, b.lse, b.workspace)

    def run_resident_fused(self, topk_pos, req_id, causal_limit, block_table, block_size, q,
                           kv_pool, scale):
        """Same result as run_resident in one call: positions are resolved inside the
        attention kernel (the rows are not written out)."""
        b = self.buf
        hs_sparse_decode_attn_paged(q, kv_pool, topk_pos, req_id, causal_limit, block_table,
                                    block_size, block_size, scale, self.d_v, b.out, b.lse,
                                    b.workspace)

    # -- swap batch (waves) -------------------------------------------------------------
    def overlaps(self, state: HotState, tick0: int) -> bool:
        """Whether wave r+1's swap may run during wave r's attention (see the module doc)."""
        return (self.capacity >= 2 * self.K and state.max_stamp is not None
                and tick0 > state.max_stamp)

    def run_swap(self, state: HotState, topk_pos, req_id, causal_limit, block_table, block_size,
                 q, scale, tick0: int, finalize: Optional[dict] = None,
                 timing: Optional[dict] = None):
        """One swap-path step.  ``timing`` (optional): lists "swap" and "attn" of R
        (start, end) timing events each and a "finalize" pair, recorded around each call on
        the stream it runs on (so their elapsed times are those calls' device durations);
        a kind left out is not recorded (each record is a packet on its stream)."""
        b, B, R = self.buf, self.B, self.R

        def mark(kind, r, i, stream):
            if timing is not None and kind in timing:
                ev = timing[kind][r] if r is not None else timing[kind]
                ev[i].record(stream)
        main = torch.cuda.current_stream()
        copy = self.copy_stream
        serialize = not self.overlaps(state, tick0)
        hs_resolve_topk(topk_pos, req_id, causal_limit, block_table, block_size, block_size,
                        b.slots, b.valid)
        self.e_resolve.record(main)
        copy.wait_event(self.e_resolve)
        # The greedy choice needs only the logits; finalize reads its result at the end.  It
        # runs beside a swap-in: after wave 0's attention when another wave follows (then
        # wave 0's swap-in does not start behind its 384 workgroups), else after resolve.
        argmax_after = 0 if R > 1 else -1
        if finalize is not None and argmax_after < 0:
            hs_greedy_argmax(finalize["logits"], b.argmax, stream=main)
        for r in range(R):
            lo, hi = r * B, (r + 1) * B
            if r >= 1 and serialize:
                copy.wait_event(self.e_attn[r - 1])
            elif r >= 2:
                copy.wait_event(self.e_attn[r - 2])
            mark("swap", r, 0, copy)
            hs_swap_in(state, b.slots[lo:hi], tick0 + r, b.hot_idx[lo:hi], b.miss_count[r],
                       None if b.miss_pos is None else b.miss_pos[lo:hi], stream=copy)
            mark("swap", r, 1, copy)
            self.e_swap[r].record(copy)
            main.wait_event(self.e_swap[r])
            mark("attn", r, 0, main)
            if r + 1 < R and not serialize:  # the next wave's swap-in runs beside it
                hs_sparse_decode_attn_cus(q[lo:hi], state.hot_kv, b.hot_idx[lo:hi], scale,
                                          self.d_v, b.out[lo:hi], b.lse[lo:hi], b.workspace,
                                          self.cus_beside_swap, stream=main)
            else:
                hs_sparse_decode_attn(q[lo:hi], state.hot_kv, b.hot_idx[lo:hi], scale, self.d_v,
                                      b.out[lo:hi], b.lse[lo:hi], b.workspace, stream=main)
            mark("attn", r, 1, main)
            if r + (1 if serialize else 2) < R:  # a later swap-in waits for this attention
                self.e_attn[r].record(main)
            if finalize is not None and r == argmax_after:
                hs_greedy_argmax(finalize["logits"], b.argmax, stream=main)
        if finalize is not None:
            mark("finalize", None, 0, main)
            hs_finalize_accepted(state, None, finalize["draft_ids"], finalize["new_kv"], R,
                                 finalize["seq_len"], block_table, block_size, tick0 + R,
                                 b.argmax, b.accept_len, b.next_token, stream=main)
            mark("finalize", None, 1, main)
            d = finalize.get("dflash")
            if d is not None:  # P2 ⑤: the draft model's context KV takes the accepted prefix
                hs_append_accepted(d["ctx_cache"], d["ctx_block_table"], d["ctx_len"],
                                   d["ctx_rows"], b.accept_len, d["block_size"], d["block_size"],
                                   R, stream=main)

    # -- mixed batch: per-request residency ---------------------------------------------
    def run_mixed(self, state: HotState, topk_pos, req_id_resident, req_id_swap, row_sel,
                  causal_limit, resident_block_table, host_block_table, block_size, q, kv_pool,
                  scale, tick0: int):
        """A batch in which fully resident requests read the resident pool and the others
        swap into the hot buffer (the per-batch switch of P3's build_offload_command made
        per request).  ``req_id_resident`` / ``req_id_swap`` are the rows' request ids with
        the other kind's rows set to -1, ``row_sel`` is 1 on rows that read the hot buffer
        (see ResidencyTracker.row_inputs)."""
        b, B, R = self.buf, self.B, self.R
        if b.slots_res is None:
            raise ValueError("run_mixed needs a DecodeStep built with capacity > 0 and mixed=True")
        main = torch.cuda.current_stream()
        copy = self.copy_stream
        serialize = not self.overlaps(state, tick0)
        hs_resolve_topk(topk_pos, req_id_swap, causal_limit, host_block_table, block_size,
                        block_size, b.slots, b.valid)
        self.e_resolve.record(main)
        copy.wait_event(self.e_resolve)
        hs_resolve_topk(topk_pos, req_id_resident, causal_limit, resident_block_table,
                        block_size, block_size, b.slots_res, None)
        for r in range(R):
            lo, hi = r * B, (r + 1) * B
            if r >= 1 and serialize:
                copy.wait_event(self.e_attn[r - 1])
            elif r >= 2:
                copy.wait_event(self.e_attn[r - 2])
            hs_swap_in(state, b.slots[lo:hi], tick0 + r, b.hot_idx[lo:hi], b.miss_count[r],
                       None if b.miss_pos is None else b.miss_pos[lo:hi], stream=copy)
            self.e_swap[r].record(copy)
            main.wait_event(self.e_swap[r])
            beside = r + 1 < R and not serialize  # the next wave's swap-in runs beside it
            hs_sparse_decode_attn_mixed(q[lo:hi], kv_pool, b.slots_res[lo:hi], state.hot_kv,
                                        b.hot_idx[lo:hi], row_sel[lo:hi], scale, self.d_v,
                                        b.out[lo:hi], b.lse[lo:hi], b.workspace, stream=main,
                                        max_cus=self.cus_beside_swap if beside else None)
            if r + (1 if serialize else 2) < R:  # a later swap-in waits for this attention
                self.e_attn[r].record(main)


class ResidencyTracker:
    """Host bookkeeping of which requests still have all their KV in the resident pool.

    P3 reclaim_resident_blocks: when the cache manager runs short, the coordinator asks the
    resident manager for reclaimable pages (every request's older pages, never its last
    two), picks victims, and releases them: the table entry becomes null and the block
    returns to the pool.  A request with a released page is no longer fully resident.
    This tracker keeps the resident block table on the host, answers those questions and
    builds the per-row inputs of DecodeStep.run_mixed.
    """

    def __init__(self, block_table: np.ndarray, seq_len: np.ndarray, block_size: int):
        self.block_table = np.array(block_table, dtype=np.int32, copy=True)
        self.seq_len = np.asarray(seq_len, dtype=np.int64)
        self.block_size = block_size
        self.free_blocks: list[int] = []

    def _used_pages(self) -> np.ndarray:
        return (self.seq_len + self.block_size - 1) // self.block_size

    def reclaimable_pages(self) -> list[tuple[int, int]]:
        used = self._used_pages()
        out = []
        for b in range(self.block_table.shape[0]):
            pages = np.flatnonzero(self.block_table[b, :max(0, int(used[b]) - 2)] >= 0)
            out.extend((b, int(p)) for p in pages)
        return out

    def release_resident_page(self, b: int, page: int) -> None:
        blk = int(self.block_table[b, page])
        if blk >= 0:
            self.block_table[b, page] = -1
            self.free_blocks.append(blk)

    def reclaim(self, deficit: int, priority=None, hot_pages=None) -> list[tuple[int, int]]:
        """Give back up to ``deficit`` resident pages and return them as (request, page).

        P3 reclaim_resident_blocks: the cache manager is ``deficit`` blocks short; of the
        reclaimable pages (older pages, never a request's last two) the hot ones are
        screened out (``hot_pages`` [num_reqs, bt_stride] bool, e.g. pages the latest
        selections touched), the rest go in the order request priority ascending
        (``priority[b]``, default 0; a larger value keeps its pages longer), then oldest
        page first, then request id, up to the deficit.  Each chosen page is released (its
        table entry becomes -1, the block goes to the free list), so its request is no
        longer fully resident.  Fewer than ``deficit`` pages means the caller's allocation
        still falls short."""
        prio = np.zeros(self.block_table.shape[0], np.int64) if priority is None \
            else np.asarray(priority, np.int64)
        if prio.shape != (self.block_table.shape[0],):
            raise ValueError("priority must have one entry per request")
        if hot_pages is not None and np.shape(hot_pages) != self.block_table.shape:
            raise ValueError("hot_pages must be [num_reqs, bt_stride]")
        cands = [(int(prio[b]), p, b) for (b, p) in self.reclaimable_pages()
                 if hot_pages is None or not hot_pages[b][p]]
        cands.sort()
        chosen = [(b, p) for (_, p, b) in cands[:max(0, int(deficit))]]
        for b, p in chosen:
            self.release_resident_page(b, p)
        return chosen

    def fully_resident(self) -> np.ndarray:
        used = self._used_pages()
        width = self.block_table.shape[1]
        cols = np.arange(width)[None, :]
        need = cols < used[:, None]
        mapped = (self.block_table >= 0) | ~need
        return (used <= width) & mapped.all(axis=1)

    def row_inputs(self, req_id_rows: np.ndarray, device) -> tuple:
        """(req_id_resident, req_id_swap, row_sel) device int32 arrays for run_mixed."""
        res = self.fully_resident()
        req = np.asarray(req_id_rows, dtype=np.int64)
        ok = (req >= 0) & (req < len(res))
        row_res = np.zeros(len(req), dtype=bool)
        row_res[ok] = res[req[ok]]
        to = lambda a: torch.as_tensor(a.astype(np.int32)).to(device)  # noqa: E731
        return (to(np.where(row_res, req, -1)), to(np.where(row_res, -1, req)),
                to((~row_res).astype(np.int32)))

    def table(self, device) -> torch.Tensor:
        return torch.as_tensor(self.block_table).to(device)



@dataclass
class PageTransfer:
    """One page to back up: the source block of every cache (layer), the destination host
    block and the page inside it (P3's SparseKVPageTransfer fields)."""
    source_block_ids: Sequence[int]
    destination_block_id: int
    destination_page_offset: int


class BackupStager:
    """Device -> host backup of whole pages, as P3's HiSparseWorker._enqueue_transfers.

    The control plane stays on the host, as on the pages.  Row lists are written into one
    of two pinned staging buffers: a buffer is reused only after the event recorded after
    its device copy has fired.  The lists are copied to the device with non-blocking
    copies, hs_backup_rows copies the rows of every layer on the same stream, and an
    event is recorded after it.  ``ready(ticket)`` polls that event
    (P1 "3. HiSparse staging": collect_ready_reqs waits on the backup event).
    """

    def __init__(self, dev_cache: torch.Tensor, host_cache: torch.Tensor, kernel_block_size: int,
                 blocks_per_kv_block: int, max_pages: int, src_block_size: int = 1,
                 src_block_stride: int = 1):
        self.dev_cache, self.host_cache = dev_cache, host_cache
        self.layers = dev_cache.shape[0] if dev_cache.dim() == 3 else 1
        self.kbs, self.per = kernel_block_size, blocks_per_kv_block
        self.src_bs, self.src_stride = src_block_size, src_block_stride
        n = max_pages * kernel_block_size
        dev = dev_cache.device
        # flat buffers: the first layers * n entries are viewed as [layers, n] per call
        self._src_cpu = [torch.empty((self.layers * n,), dtype=torch.int32, pin_memory=True)
                         for _ in range(2)]
        self._dst_cpu = [torch.empty((n,), dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self._staging_done = [None, None]
        self._src_dev = torch.empty((self.layers * n,), dtype=torch.int32, device=dev)
        self._dst_dev = torch.empty((n,), dtype=torch.int32, device=dev)
        self._next = 0
        self.max_pages = max_pages

    def enqueue(self, transfers: Sequence[PageTransfer], stream=None) -> torch.cuda.Event:
        """Queue the backup of `transfers`; returns the event that marks the host rows
        written."""
        if not transfers:
            ev = torch.cuda.Event()
            ev.record(stream)
            return ev
        if len(transfers) > self.max_pages:
            raise ValueError(f"{len(transfers)} pages exceed the stager's {self.max_pages}")
        i = self._next
        self._next ^= 1
        if self._staging_done[i] is not None:
            self._staging_done[i].synchronize()  # the copy that last read this buffer is done
        kbs, n = self.kbs, len(transfers) * self.kbs
        off = np.arange(kbs, dtype=np.int64)
        src_blocks = np.array([t.source_block_ids for t in transfers], dtype=np.int64)  # [P, L]
        if src_blocks.shape[1] != self.layers:
            raise ValueError("each transfer needs one source block per layer")
        host_pages = np.array([t.destination_block_id * self.per + t.destination_page_offset
                               for t in transfers], dtype=np.int64)
        m = self.layers * n
        src = self._src_cpu[i].numpy()
        dst = self._dst_cpu[i].numpy()
        src[:m] = (src_blocks.T[:, :, None] * kbs + off).reshape(m)  # layer-major
        dst[:n] = (host_pages[:, None] * kbs + off).reshape(n)
        s = torch.cuda.current_stream() if stream is None else stream
        with torch.cuda.stream(s):
            self._src_dev[:m].copy_(self._src_cpu[i][:m], non_blocking=True)
            self._dst_dev[:n].copy_(self._dst_cpu[i][:n], non_blocking=True)
            staged = torch.cuda.Event()
            staged.record(s)
            self._staging_done[i] = staged
            src_dev = self._src_dev[:m].view(self.layers, n) if self.layers > 1 else self._src_dev[:n]
            hs_backup_rows(self.dev_cache, self.host_cache, src_dev, self._dst_dev[:n], self.src_bs,
                           self.src_stride, stream=s)
            written = torch.cuda.Event()
            written.record(s)
        return written

    @staticmethod
    def ready(written: torch.cuda.Event) -> bool:
        """True once the host rows of that enqueue hold the copies (non-blocking poll)."""
        return written.query()
