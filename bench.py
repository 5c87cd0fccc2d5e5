#!/usr/bin/env python3
"""Benchmark of the HiSparse sparse-decode hot path on one MI355X.

Headline workload: the mixed batch with verification and finalize, the largest one-GPU
workload.  128 requests, seq_len log-uniform in [1024, 131072], 3 query rows per request
(anchor + 2 draft rows), top-k 2048 (rows whose causal limit is below 2048 padded with -1),
block size 64, 4096 hot slots per request, top-k reuse 0.6 from the previous step's set,
a pinned host pool of 576-wide bf16 latent rows for every token (4.1 GB), 128 query heads
sharing the latent row (value = first 512 dims, scale 1/sqrt(576)), then greedy acceptance
over bf16 logits [384, 129280] and finalize of the accepted prefix.

One step = hs_resolve_topk over the 384 rows, then per wave r (row r of every request)
hs_swap_in on a copy stream overlapped with hs_sparse_decode_attn of the previous wave on
the main stream, then hs_finalize_accepted.  Before every step (untimed) the hot state,
hot buffer and the host rows finalize writes are restored from snapshots, so every step
does the same work; each step is timed as device time between HIP events (a short spin
kernel ahead of it covers the host-side marshalling of its first call).  Inputs are
synthetic (seeded) and resident before the timed region: device tensors in HBM, the host
pool in pinned host memory (the path reads it over the host link by design).

Prints ONE JSON line.  `value` = query rows/s of the step.  `roofline` = the dominant
kernel, the swap-in (its copy is bound by the host link), with the miss bytes per launch
over its live-measured launch duration against the link's published rate.  Secondary
objects: `hbm_roofline` (the step's attention dispatches against the 8 TB/s HBM peak),
`host_link` (B_host: a 1 GiB pinned -> device copy and a streaming zero-copy read kernel),
`long_context_step` (64 requests x 4 rows at seq_len 131072, 9.66 GB pinned pool),
`resident_decode` (8 fully resident rows, warm and cold caches), `attn_sweep`, `swap_in`
(the 32-request MTP workload), `finalize`, `backup`, `resolve`, and `cpu_baseline` (the CPU
oracle on a sample of the headline step).  `--part power` (not in the default run) adds
`attn_power`: socket power and gfx clock (amd-smi) while the attention op runs back to back.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--part NAME]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# MI355X host interface: PCIe 5.0 x16, 64 GB/s per direction (published).
HOST_LINK_PEAK_GBS = 64.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
SETTLE_MS = 50.0  # untimed back-to-back work before a timed attention region (clock settling)
METRIC = "sparse-decode query rows/s at topk=2048; achieved HBM GB/s (% of peak)"
HEADLINE = "mixed_finalize"


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def attn_alg_bytes(valid_per_row, heads, d_qk, d_v, topk, elem=2):
    """Algorithmic bytes of one attention launch: each valid selected KV row once, the
    query and output rows once, the index row once."""
    rows = len(valid_per_row)
    kv = int(sum(valid_per_row)) * d_qk * elem
    return kv + rows * (heads * d_qk * elem + heads * d_v * elem + topk * 4)


SOURCES = {
    "attn": ("attn.hip", "attn64.hip", "attn128.hip", "attn_tile.h", "common.h"),
    "swap": ("swap.hip", "ops.h", "common.h"),
}


def source_hash(kind):
    """Hash of a kernel family's sources (ties stored counter figures to them)."""
    h = hashlib.sha256()
    for f in SOURCES[kind]:
        with open(os.path.join(ROOT, "sparse_attention_kv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_counters(profile, kind):
    """`key: value` lines of a committed rocprofv3 counter summary, if it was taken on the
    current sources of that kernel family; else None."""
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "|")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash(kind):
        return None
    return kv


def stored_int(profile, kind, key):
    kv = stored_counters(profile, kind)
    try:
        return int(kv[key]) if kv else None
    except (KeyError, ValueError):
        return None


STEP_SPIN_US = 1000.0


def gpu_busy(us=100.0):
    """Keep the GPU busy for about ``us`` microseconds, so that an event recorded after it
    times the device work of the calls enqueued meanwhile, not their host-side marshalling."""
    import torch
    torch.cuda._sleep(int(us * 2000))  # spin kernel counting shader clocks (~2 GHz)


def ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


def raw_np(t):
    """Raw numpy view of a CPU tensor (uint16 bit patterns for bf16); no copy."""
    import numpy as np
    import torch
    t = t.detach()
    if t.is_cuda:
        t = t.cpu()
    t = t.contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


# ----------------------------------------------------------------------------------------
# host link
# ----------------------------------------------------------------------------------------
def measure_host_link(dev, nbytes=1 << 30, reps=3):
    """B_host, the better of a 1 GiB pinned -> device copy (DMA) and a streaming zero-copy
    read kernel over the same 1 GiB (hs_host_read: 16-byte loads through the pinned
    buffer's device mapping, the kind of access the swap-in copy makes)."""
    import torch

    import sparse_attention_kv_amd as hs
    main = torch.cuda.current_stream()
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    src.fill_(3)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    hs.hs_host_read(src, dst)
    torch.cuda.synchronize()
    a, z = ev(), ev()
    a.record(main)
    for _ in range(reps):
        dst.copy_(src, non_blocking=True)
    z.record(main)
    torch.cuda.synchronize()
    memcpy = reps * nbytes / (a.elapsed_time(z) / 1e3) / 1e9
    a.record(main)
    for _ in range(reps):
        hs.hs_host_read(src, dst)
    z.record(main)
    torch.cuda.synchronize()
    zero_copy = reps * nbytes / (a.elapsed_time(z) / 1e3) / 1e9
    ok = bool(torch.equal(dst[:4096].cpu(), src[:4096]))
    del src, dst
    return {"B_host_GBps": max(memcpy, zero_copy), "memcpy_pinned_to_device_GBps": memcpy,
            "zero_copy_read_kernel_GBps": zero_copy, "bytes": nbytes, "zero_copy_read_checked": ok,
            "published_peak_GBps": HOST_LINK_PEAK_GBS}


# ----------------------------------------------------------------------------------------
# whole swap-path steps (headline, long context)
# ----------------------------------------------------------------------------------------
class StepRig:
    """One swap-path workload set up for repeated steps: device inputs, hot state, snapshots
    of everything a step changes (restored before each step, untimed) and the step driver."""

    def __init__(self, dev, name):
        import numpy as np
        import torch

        import sparse_attention_kv_amd as hs
        from sparse_attention_kv_amd.pipeline import DecodeStep, build_hot_state
        from workloads import generate, spec

        self.s = s = spec(name)
        log(f"generate {s.name} (pinned host pool)")
        self.w = w = generate(s, big_device="cuda", pin_host_pool=True)

        def d(a):
            return torch.as_tensor(np.ascontiguousarray(a)).to(device=dev, dtype=torch.int32)

        self.topk_pos, self.req_id, self.lim = d(w.topk_pos), d(w.req_id), d(w.causal_limit)
        self.bt, self.seq = d(w.block_table), d(w.seq_len)
        self.st = build_hot_state(torch.from_numpy(w.init_pos), torch.from_numpy(w.init_stamp),
                                  self.seq, self.bt, s.block_size, w.kv_pool, dev)
        st = self.st
        self.snap = [t.clone() for t in (st.slot_loc, st.slot_stamp, st.loc_to_hot, st.hot_kv)]
        self.snap_max = st.max_stamp
        self.step = DecodeStep(num_reqs=s.num_reqs, rows_per_req=s.rows_per_req, topk=s.topk,
                               num_heads=s.num_heads, d_qk=s.d_qk, d_v=s.d_v,
                               dtype=torch.bfloat16, capacity=s.capacity, finalize=s.finalize,
                               device=dev)
        self.q = w.q.to(dev)
        self.fin = None
        self.host_rows = None
        if s.finalize:
            self.fin = dict(logits=w.logits.to(dev), draft_ids=d(w.draft_ids),
                            new_kv=w.new_kv.to(dev), seq_len=self.seq)
            # host rows finalize may write: the verify rows' positions, resolved by the
            # library (setup only)
            B, R = s.num_reqs, s.rows_per_req
            pos = (torch.as_tensor(w.seq_len, dtype=torch.int64)[:, None] - R +
                   torch.arange(R)[None, :]).to(torch.int32).contiguous().to(dev)
            rows = torch.empty_like(pos)
            hs.hs_resolve_topk(pos, torch.arange(B, dtype=torch.int32, device=dev), self.seq,
                               self.bt, s.block_size, s.block_size, rows)
            r = rows.view(-1).cpu().long()
            self.host_rows = r[r >= 0]
            self.host_snap = w.kv_pool[self.host_rows].clone()
        torch.cuda.synchronize()

    def restore(self):
        st = self.st
        for t, c in zip((st.slot_loc, st.slot_stamp, st.loc_to_hot, st.hot_kv), self.snap):
            t.copy_(c)
        st.max_stamp = self.snap_max
        if self.host_rows is not None:
            self.w.kv_pool[self.host_rows] = self.host_snap

    def run(self, timing=None):
        s = self.s
        self.step.run_swap(self.st, self.topk_pos, self.req_id, self.lim, self.bt, s.block_size,
                           self.q, s.scale, s.tick0, finalize=self.fin, timing=timing)

    def outputs(self):
        """Everything a step produces, cloned (for the replay check)."""
        b, st = self.step.buf, self.st
        ts = [b.slots, b.valid, b.hot_idx, b.miss_count, b.out, b.lse, st.slot_loc, st.slot_stamp,
              st.loc_to_hot, st.hot_kv]
        if self.fin is not None:
            ts += [b.argmax, b.accept_len, b.next_token]
        return [t.clone() for t in ts]

    def release(self):
        import torch
        del self.w, self.st, self.snap, self.step, self.q, self.fin
        torch.cuda.empty_cache()


def measure_step(rig, steps, warmup, b_host):
    """W untimed steps, then K timed steps (each restored first, untimed): device time
    between events on the main stream, the second after it has waited for the copy stream.
    The timed steps run the step exactly as a caller does, with no event inside it (an
    event recorded between two launches on a stream is a packet of its own, and the
    per-call events cost the step ≈50 µs).  Then K more steps record an event pair around
    every swap-in, attention and finalize launch on the stream it runs on: those give each
    launch's device time (the per-wave figures and the swap-in launch time of the
    roofline), not the step time."""
    import numpy as np
    import torch

    s, step = rig.s, rig.step
    R = s.rows_per_req
    main = torch.cuda.current_stream()
    first = None
    for i in range(warmup):
        rig.restore()
        torch.cuda.synchronize()
        rig.run()
        main.wait_stream(step.copy_stream)
        torch.cuda.synchronize()
        if first is None:
            first = rig.outputs()
    step_ms, marked_ms, swap_us, attn_us, fin_us = [], [], [], [], []
    for marked in (False, True):
        for i in range(steps):
            rig.restore()
            torch.cuda.synchronize()
            timing = {"swap": [(ev(), ev()) for _ in range(R)],
                      "attn": [(ev(), ev()) for _ in range(R)],
                      "finalize": (ev(), ev())} if marked else None
            e0, e1 = ev(), ev()
            # a spin long enough that the host has enqueued the whole step (≈15 calls)
            # before the first event: a host-side pause while enqueueing cannot then show
            # up as device idle time inside the step
            gpu_busy(STEP_SPIN_US)
            e0.record(main)
            rig.run(timing)
            main.wait_stream(step.copy_stream)
            e1.record(main)
            torch.cuda.synchronize()
            (marked_ms if marked else step_ms).append(e0.elapsed_time(e1))
            if not marked:
                continue
            swap_us.append([a.elapsed_time(z) * 1e3 for a, z in timing["swap"]])
            attn_us.append([a.elapsed_time(z) * 1e3 for a, z in timing["attn"]])
            if rig.fin is not None:
                fin_us.append(timing["finalize"][0].elapsed_time(timing["finalize"][1]) * 1e3)
    last = rig.outputs()
    if first is None:
        first = last
    replay_identical = all(torch.equal(a, b) for a, b in zip(first, last))
    b = step.buf
    miss = b.miss_count.cpu().numpy().astype(np.int64)            # [R, B]
    row_bytes = s.d_qk * 2
    wave_miss_bytes = [int(miss[r].sum()) * row_bytes for r in range(R)]
    valid = b.valid.cpu().numpy()
    wave_alg = [attn_alg_bytes(valid[r * s.num_reqs:(r + 1) * s.num_reqs], s.num_heads, s.d_qk,
                               s.d_v, s.topk) for r in range(R)]
    ms = float(np.mean(step_ms))
    swap_mean = float(np.mean(swap_us))
    attn_mean = float(np.mean(attn_us))
    swap_gbs = sum(wave_miss_bytes) / (np.mean(np.sum(swap_us, axis=1)) / 1e6) / 1e9
    attn_gbs = sum(wave_alg) / (np.mean(np.sum(attn_us, axis=1)) / 1e6) / 1e9
    # the last wave's attention runs alone (no swap-in after it); the earlier ones run
    # beside the next wave's swap-in, whose host reads slow their HBM gathers
    last_us = float(np.mean(np.asarray(attn_us)[:, R - 1]))
    last_gbs = wave_alg[R - 1] / (last_us / 1e6) / 1e9
    total_miss = sum(wave_miss_bytes)
    out = {
        "workload": s.name, "rows_per_step": s.rows, "waves": R, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "step_ms_median": float(np.median(step_ms)),
        "step_ms_min": float(np.min(step_ms)), "step_ms_max": float(np.max(step_ms)),
        "marked_steps_ms_mean": float(np.mean(marked_ms)),
        "per_launch_timing": "per-launch figures (swap_*, attn_*, finalize_us_mean) come from "
                             f"{steps} further steps with an event pair around each launch",
        "rows_per_s": s.rows / (ms / 1e3),
        "miss_bytes_per_step": total_miss, "wave_miss_bytes": wave_miss_bytes,
        "misses_per_row": float(miss.sum() / max(1, (valid > 0).sum())),
        "hit_rate": float(1 - miss.sum() / max(1, valid.sum())),
        "step_miss_GBps": total_miss / (ms / 1e3) / 1e9,
        "step_frac_of_B_host": total_miss / (ms / 1e3) / 1e9 / b_host,
        "host_link_floor_ms": total_miss / (b_host * 1e9) * 1e3,
        "swap_launch_us_mean": swap_mean, "swap_wave_us_mean": np.mean(swap_us, axis=0).tolist(),
        "swap_GBps": swap_gbs, "swap_frac_of_B_host": swap_gbs / b_host,
        "attn_launch_us_mean": attn_mean, "attn_wave_us_mean": np.mean(attn_us, axis=0).tolist(),
        "attn_alg_bytes_per_wave": wave_alg, "attn_GBps": attn_gbs,
        "attn_hbm_frac": attn_gbs / HBM_PEAK_GBS,
        "attn_last_wave_us": last_us, "attn_last_wave_GBps": last_gbs,
        "attn_last_wave_hbm_frac": last_gbs / HBM_PEAK_GBS,
        "replay_bit_identical": bool(replay_identical),
    }
    if fin_us:
        out["finalize_us_mean"] = float(np.mean(fin_us))
        out["accept_length_histogram"] = np.bincount(b.accept_len.cpu().numpy(),
                                                     minlength=R).tolist()
    return out


# ----------------------------------------------------------------------------------------
# CPU baseline: the oracle on a sample of the headline step
# ----------------------------------------------------------------------------------------
def cpu_baseline(s, w, sample_reqs=64, reps=3):
    """The oracle (numpy, float64 attention, loop-level swap/LRU) runs the headline step for
    the first `sample_reqs` requests (all their rows and waves): resolve, the waves' swap-ins,
    attention over every sampled row, greedy acceptance and finalize.  Each stage is timed
    separately, median of `reps` runs from the same starting state; rows/s = sampled rows /
    sum of the stage medians.  Once with numpy's own thread pool (all host cores), once
    limited to one thread."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    B, R, Bs = s.num_reqs, s.rows_per_req, min(sample_reqs, s.num_reqs)
    rows = np.array([r * B + b for r in range(R) for b in range(Bs)])
    pool = raw_np(w.kv_pool)
    q = raw_np(w.q)[rows]
    logits = raw_np(w.logits)[rows]
    new_kv = raw_np(w.new_kv)[rows]
    topk, lim, draft = w.topk_pos[rows], w.causal_limit[rows], w.draft_ids[rows]
    req = w.req_id[rows]
    bt, seq = w.block_table[:Bs], w.seq_len[:Bs]
    st0 = oracle.build_hot_state(w.init_pos[:Bs], w.init_stamp[:Bs], seq, bt, s.block_size, pool)
    # host rows finalize writes, saved and put back after every run (the pool is shared)
    vpos = (seq.astype(np.int64)[:, None] - R + np.arange(R)[None]).astype(np.int32)
    vrows, _ = oracle.resolve_topk(vpos, np.arange(Bs, dtype=np.int32), seq, bt, s.block_size,
                                   s.block_size, Bs)
    vrows = vrows[vrows >= 0]
    saved = pool[vrows].copy()

    def one():
        st = st0.copy()
        t = {}
        a = time.perf_counter()
        slots, _ = oracle.resolve_topk(topk, req, lim, bt, s.block_size, s.block_size, Bs)
        t["resolve"] = time.perf_counter() - a
        a = time.perf_counter()
        hot = np.empty_like(slots)
        for r in range(R):
            hot[r * Bs:(r + 1) * Bs], _, _ = oracle.swap_in(st, slots[r * Bs:(r + 1) * Bs],
                                                           s.tick0 + r, pool)
        t["swap_in"] = time.perf_counter() - a
        a = time.perf_counter()
        oracle.sparse_decode_attn(q, st.hot_kv, hot, s.scale, s.d_v)
        t["attention"] = time.perf_counter() - a
        a = time.perf_counter()
        acc, _, _ = oracle.greedy_accept(logits, draft, Bs, R)
        t["accept"] = time.perf_counter() - a
        a = time.perf_counter()
        oracle.finalize_accepted(st, pool, new_kv, acc, seq, bt, s.block_size, R, s.tick0 + R)
        t["finalize"] = time.perf_counter() - a
        pool[vrows] = saved
        return t

    def run():
        runs = [one() for _ in range(reps)]
        med = {k: statistics.median(r[k] for r in runs) for k in runs[0]}
        return med, sum(med.values())

    t0 = time.perf_counter()
    med, tot = run()
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    with threadpool_limits(limits=1):
        med1, tot1 = run()
    wall = time.perf_counter() - t0
    n = len(rows)
    return {"value": n / tot, "unit": "rows/s", "cores": int(threads), "kind": "oracle",
            "sample": f"headline step restricted to its first {Bs} of {B} requests ({n} rows, "
                      f"{R} waves: resolve, swap-in, float64 attention, greedy accept, finalize), "
                      f"median of {reps} runs per stage, {os.cpu_count()} visible host CPUs; "
                      f"{wall:.1f} s in all",
            "stage_ms": {k: v * 1e3 for k, v in med.items()},
            "one_thread": {"value": n / tot1, "unit": "rows/s", "cores": 1,
                           "stage_ms": {k: v * 1e3 for k, v in med1.items()}}}


# ----------------------------------------------------------------------------------------
# resident decode (8 rows, warm and cold caches)
# ----------------------------------------------------------------------------------------
def measure_resident(dev, steps, warmup, cold_sets=24):
    """Fully resident decode: 8 requests, seq_len U[6144, 8192], one row each, top-k 2048,
    one hs_sparse_decode_attn_paged call (positions resolved in the attention prologue).
    Warm: K back-to-back calls on one input set (its 21 MB stay in the 256 MB Infinity Cache).
    Cold: the calls rotate over `cold_sets` input sets with their own paged pools and queries
    (the same index structure; 24 x 21 MB of distinct rows read between two uses of a set,
    so every call reads HBM).  Also the two-call form and a captured HIP graph (warm)."""
    import numpy as np
    import torch

    import sparse_attention_kv_amd as hs
    from sparse_attention_kv_amd.pipeline import DecodeStep
    from workloads import generate, spec

    s = spec("resident")
    w = generate(s, big_device="cuda")

    def d(a):
        return torch.as_tensor(np.ascontiguousarray(a)).to(device=dev, dtype=torch.int32)

    topk_pos, req_id, lim, bt = d(w.topk_pos), d(w.req_id), d(w.causal_limit), d(w.block_table)
    step = DecodeStep(num_reqs=s.num_reqs, rows_per_req=1, topk=s.topk, num_heads=s.num_heads,
                      d_qk=s.d_qk, d_v=s.d_v, dtype=torch.bfloat16, device=dev)
    b = step.buf
    step.run_resident(topk_pos, req_id, lim, bt, s.block_size, w.q.to(dev), w.kv_pool, s.scale)
    torch.cuda.synchronize()
    alg = attn_alg_bytes(b.valid.cpu().numpy(), s.num_heads, s.d_qk, s.d_v, s.topk)
    g = torch.Generator(device=dev).manual_seed(77)
    sets = [(w.q.to(dev), w.kv_pool)]
    for _ in range(cold_sets - 1):
        sets.append((torch.randn(w.q.shape, generator=g, device=dev).to(torch.bfloat16),
                     torch.randn(w.kv_pool.shape, generator=g, device=dev).to(torch.bfloat16)))
    calls = [hs.PagedAttnCall(q, kv, topk_pos, req_id, lim, bt, s.block_size, s.block_size,
                              s.scale, s.d_v, b.out, b.lse, b.workspace) for q, kv in sets]
    main = torch.cuda.current_stream()
    a, z = ev(), ev()

    def timed(fn, n):
        a.record(main)
        for i in range(n):
            fn(i)
        z.record(main)
        torch.cuda.synchronize()
        return a.elapsed_time(z) / n

    n = max(steps, 100)
    for i in range(max(warmup, 3000)):  # settles the shader clock (~50 ms of calls)
        calls[0]()
    torch.cuda.synchronize()
    warm_ms = timed(lambda i: calls[0](), n)
    for i in range(2 * cold_sets):
        calls[i % cold_sets]()
    cold_ms = timed(lambda i: calls[i % cold_sets](), n)
    two_call_ms = timed(lambda i: step.run_resident(topk_pos, req_id, lim, bt, s.block_size,
                                                    sets[0][0], sets[0][1], s.scale), n)
    graph_ms = None
    gr = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(main)
    with torch.cuda.stream(cap):
        calls[0]()
        torch.cuda.synchronize()
        with torch.cuda.graph(gr, stream=cap):
            calls[0]()
    torch.cuda.synchronize()
    ref = b.out.clone()
    for _ in range(200):
        gr.replay()
    torch.cuda.synchronize()
    graph_ms = timed(lambda i: gr.replay(), n)
    graph_ok = bool(torch.equal(b.out, ref))
    traffic = stored_int("attn_resident_counters.txt", "attn", "traffic_bytes_per_launch")
    ws = hs.hs_attn_workspace_bytes(s.rows, s.num_heads, s.d_qk, s.d_v, s.topk, torch.bfloat16)
    del sets, calls
    torch.cuda.empty_cache()

    def frac(ms):
        return alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBS
    return {
        "workload": "resident decode: 8 requests, seq_len U[6144,8192], 1 row each, top-k 2048, "
                    "block 64, 128 heads x 576/512 bf16 latent KV, one paged-attention call",
        "rows_per_step": s.rows, "alg_bytes_per_launch": alg,
        "cold": {"us": cold_ms * 1e3, "rows_per_s": s.rows / (cold_ms / 1e3),
                 "GBps": alg / (cold_ms / 1e3) / 1e9, "hbm_frac": frac(cold_ms),
                 "input_sets": cold_sets, "distinct_bytes_between_uses": alg * (cold_sets - 1)},
        "warm": {"us": warm_ms * 1e3, "rows_per_s": s.rows / (warm_ms / 1e3),
                 "GBps": alg / (warm_ms / 1e3) / 1e9, "hbm_frac": frac(warm_ms)},
        "two_call_us": two_call_ms * 1e3, "graph_us": graph_ms * 1e3, "graph_replay_matches": graph_ok,
        "split_workspace_bytes": ws, "traffic_bytes_per_launch": traffic,
    }


# ----------------------------------------------------------------------------------------
# attention alone at the swap workloads' batch sizes (cold caches)
# ----------------------------------------------------------------------------------------
def measure_attn_sweep(dev, sizes=(32, 64, 128, 256), reps=40):
    """The attention op alone at the batch sizes of the other workloads: one swap wave of
    the MTP workload (32 rows), of the long-context workload (64), of the mixed workload
    (128), and the long-context workload's 256 rows at once.  Top-k 2048 distinct rows per
    query row, drawn uniformly from a resident pool of 1M bf16 576-wide latent rows
    (1.15 GB, N(0,1)); 128 heads, value = first 512 dims, scale 1/sqrt(576).  Each size
    rotates over enough index sets (and queries) that ~600 MB of other rows are read
    between two uses of a set, so every call reads HBM; the kernel (32-, 64- or 128-head
    workgroups) is the library planner's choice."""
    import torch

    import sparse_attention_kv_amd as hs
    H, D, DV, K, N = 128, 576, 512, 2048, 1 << 20
    g = torch.Generator(device=dev).manual_seed(20261202)
    kv = torch.randn((N, D), generator=g, device=dev).to(torch.bfloat16)
    main = torch.cuda.current_stream()
    out_rows = []
    for rows in sizes:
        alg = attn_alg_bytes([K] * rows, H, D, DV, K)
        nsets = max(2, min(16, math.ceil(600e6 / alg)))
        qs = [torch.randn((rows, H, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(nsets)]
        idx = [torch.stack([torch.randperm(N, generator=g, device=dev)[:K] for _ in range(rows)])
               .to(torch.int32).contiguous() for _ in range(nsets)]
        out = torch.empty((rows, H, DV), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((rows, H), dtype=torch.float32, device=dev)
        wsb = hs.hs_attn_workspace_bytes(rows, H, D, DV, K, torch.bfloat16)
        ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device=dev) if wsb else None

        def call(i):
            hs.hs_sparse_decode_attn(qs[i % nsets], kv, idx[i % nsets], D ** -0.5, DV, out, lse, ws)
        a, z = ev(), ev()
        a.record(main)
        for i in range(5):
            call(i)
        z.record(main)
        torch.cuda.synchronize()
        est_us = a.elapsed_time(z) * 1e3 / 5
        for i in range(int(SETTLE_MS * 1e3 / max(est_us, 1.0)) + nsets):
            call(i)
        torch.cuda.synchronize()
        a.record(main)
        for i in range(reps):
            call(i)
        z.record(main)
        torch.cuda.synchronize()
        us = a.elapsed_time(z) * 1e3 / reps
        flops = rows * K * 2 * H * (D + DV)
        hpw, spl = hs.hs_attn_plan_info(rows, H, D, DV, K, torch.bfloat16)
        out_rows.append({"rows": rows, "kernel_heads_per_wg": hpw, "splits": spl, "us": us,
                         "rows_per_s": rows / (us / 1e6), "GBps": alg / (us / 1e6) / 1e9,
                         "hbm_frac": alg / (us / 1e6) / 1e9 / HBM_PEAK_GBS,
                         "TFLOPs": flops / (us / 1e6) / 1e12,
                         "mfma_frac": flops / (us / 1e6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                         "index_sets": nsets, "split_workspace_bytes": wsb})
        del qs, idx, out, lse, ws
    del kv
    torch.cuda.empty_cache()
    return {"workload": "attention op alone, top-k 2048 distinct rows of a 1M-row resident pool, "
                        "128 heads x 576/512 bf16, cold caches", "sizes": out_rows}


def smi_power_clock():
    """(socket W, gfx MHz) from one `amd-smi metric -p -c --json` reading, or None."""
    import subprocess
    try:
        p = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True,
                           text=True, timeout=20)
        d = json.loads(p.stdout)
    except (OSError, ValueError, subprocess.SubprocessError):
        return None
    g = d[0] if isinstance(d, list) else d
    if isinstance(g, dict) and "gpu_data" in g:
        g = g["gpu_data"][0]

    def val(x):
        return x.get("value") if isinstance(x, dict) else x
    try:
        return float(val(g["power"]["socket_power"])), float(val(g["clock"]["gfx_0"]["clk"]))
    except (KeyError, TypeError, ValueError):
        return None


def measure_power(dev, sizes=(8, 32, 64, 128, 256), secs=6.0):
    """Socket power and gfx clock while the attention op runs back to back for `secs` at
    each size (the sweep's inputs: top-k 2048 distinct rows of a 1M-row pool, 128 heads,
    cold index sets), read with amd-smi from a second thread 2, 3 and 4 s into the run.
    Shows which sizes run at the board's power limit, where time per call follows energy
    per call rather than cycles."""
    import threading

    import torch

    import sparse_attention_kv_amd as hs
    H, D, DV, K, N = 128, 576, 512, 2048, 1 << 20
    g = torch.Generator(device=dev).manual_seed(20261202)
    kv = torch.randn((N, D), generator=g, device=dev).to(torch.bfloat16)
    main = torch.cuda.current_stream()
    idle = smi_power_clock()
    out_rows = []
    for rows in sizes:
        alg = attn_alg_bytes([K] * rows, H, D, DV, K)
        nsets = max(2, min(16, math.ceil(600e6 / alg)))
        qs = [torch.randn((rows, H, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(nsets)]
        idx = [torch.stack([torch.randperm(N, generator=g, device=dev)[:K] for _ in range(rows)])
               .to(torch.int32).contiguous() for _ in range(nsets)]
        out = torch.empty((rows, H, DV), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((rows, H), dtype=torch.float32, device=dev)
        wsb = hs.hs_attn_workspace_bytes(rows, H, D, DV, K, torch.bfloat16)
        ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device=dev) if wsb else None

        def call(i):
            hs.hs_sparse_decode_attn(qs[i % nsets], kv, idx[i % nsets], D ** -0.5, DV, out, lse, ws)
        for i in range(2 * nsets):
            call(i)
        torch.cuda.synchronize()
        readings = []

        def sample():
            time.sleep(2.0)
            for _ in range(3):
                r = smi_power_clock()
                if r is not None:
                    readings.append(r)
                time.sleep(0.5)
        th = threading.Thread(target=sample)
        a, z = ev(), ev()
        t0 = time.time()
        th.start()
        a.record(main)
        n = 0
        while time.time() - t0 < secs:
            for i in range(100):
                call(n + i)
            n += 100
            torch.cuda.synchronize()
        z.record(main)
        torch.cuda.synchronize()
        th.join()
        us = a.elapsed_time(z) * 1e3 / n
        hpw, spl = hs.hs_attn_plan_info(rows, H, D, DV, K, torch.bfloat16)
        out_rows.append({
            "rows": rows, "kernel_heads_per_wg": hpw, "splits": spl, "us": us, "calls": n,
            "hbm_frac": alg / (us / 1e6) / 1e9 / HBM_PEAK_GBS,
            "socket_W": statistics.median(w for w, _ in readings) if readings else None,
            "gfx_MHz": statistics.median(c for _, c in readings) if readings else None,
            "energy_per_row_mJ": (statistics.median(w for w, _ in readings) * us / 1e6 / rows * 1e3
                                  if readings else None)})
        del qs, idx, out, lse, ws
    del kv
    torch.cuda.empty_cache()
    return {"workload": "attention op back to back, top-k 2048 distinct rows of a 1M-row pool, "
                        "128 heads x 576/512 bf16, cold index sets; amd-smi socket power and gfx clock",
            "idle_W_MHz": idle, "board_power_limit_W": 1400, "sizes": out_rows}


# ----------------------------------------------------------------------------------------
# MTP swap workload: waves, plan reuse, mixed batch, cold wave
# ----------------------------------------------------------------------------------------
def measure_swap(dev, b_host, reps=5):
    """Swap path on the 32-request MTP workload (4 rows per request, top-k 2048, 4096 hot
    slots per request, reuse 0.7, 1.21 GB pinned host pool): the whole step, the swap-in
    kernel wave by wave, plan reuse on two follower layers, a mixed batch (half of the
    requests resident) and a cold all-miss wave.  State restored before every repetition
    (not timed); each timed region starts behind a short spin kernel (device time)."""
    import numpy as np
    import torch

    import sparse_attention_kv_amd as hs
    from sparse_attention_kv_amd.pipeline import DecodeStep, ResidencyTracker

    rig = StepRig(dev, "mtp_swap")
    s, w, st, b = rig.s, rig.w, rig.st, rig.step.buf
    main = torch.cuda.current_stream()
    whole = measure_step(rig, reps, 2, b_host)
    row_bytes = s.d_qk * 2

    # mixed batch (per-request residency): 16 of the 32 requests lost one resident page and
    # swap in; the other 16 read a resident pool (a device copy of the host pool, same rows)
    tracker = ResidencyTracker(w.block_table, w.seq_len, s.block_size)
    for bq in range(0, s.num_reqs, 2):
        page = next(p for (bb, p) in tracker.reclaimable_pages() if bb == bq)
        tracker.release_resident_page(bq, page)
    n_resident = int(tracker.fully_resident().sum())
    req_res, req_swap, sel = tracker.row_inputs(w.req_id, dev)
    res_bt = tracker.table(dev)
    dev_pool = w.kv_pool.to(dev)
    mstep = DecodeStep(num_reqs=s.num_reqs, rows_per_req=s.rows_per_req, topk=s.topk,
                       num_heads=s.num_heads, d_qk=s.d_qk, d_v=s.d_v, dtype=torch.bfloat16,
                       capacity=s.capacity, mixed=True, device=dev)
    mtimes = []
    for rep in range(reps + 2):
        rig.restore()
        torch.cuda.synchronize()
        a, z = ev(), ev()
        gpu_busy()
        a.record(main)
        mstep.run_mixed(st, rig.topk_pos, req_res, req_swap, sel, rig.lim, res_bt, rig.bt,
                        s.block_size, rig.q, dev_pool, s.scale, s.tick0)
        main.wait_stream(mstep.copy_stream)
        z.record(main)
        torch.cuda.synchronize()
        if rep >= 2:
            mtimes.append(a.elapsed_time(z))
    mixed_ms = float(np.median(mtimes))
    del dev_pool, mstep

    # swap-in alone, wave by wave, from the same starting state: one untimed pass (the
    # GPU's first touch of host-pool pages that no earlier call read), then the median of
    # three timed passes per wave
    rig.restore()
    hs.hs_resolve_topk(rig.topk_pos, rig.req_id, rig.lim, rig.bt, s.block_size, s.block_size,
                       b.slots, b.valid)
    passes = []
    for rep in range(4):
        rig.restore()
        torch.cuda.synchronize()
        us = []
        for r in range(s.rows_per_req):
            lo, hi = r * s.num_reqs, (r + 1) * s.num_reqs
            a, z = ev(), ev()
            gpu_busy()
            a.record(main)
            hs.hs_swap_in(st, b.slots[lo:hi], s.tick0 + r, b.hot_idx[lo:hi], b.miss_count[r])
            z.record(main)
            torch.cuda.synchronize()
            us.append(a.elapsed_time(z) * 1e3)
        if rep >= 1:
            passes.append(us)
    wave_us = [float(np.median([p_[r] for p_ in passes])) for r in range(s.rows_per_req)]
    wave_bytes = [int(b.miss_count[r].sum().item()) * row_bytes for r in range(s.rows_per_req)]
    warm_gbs = sum(wave_bytes) / (sum(wave_us) / 1e6) / 1e9

    # plan reuse: the leader's swap plan applied to 2 follower layers (own hot buffers and
    # pinned host pools, same slot assignment), wave by wave from the same starting state
    C = 2
    host_rows = w.kv_pool.shape[0]
    f_hot = torch.empty((C, s.num_reqs * s.capacity, s.d_qk), dtype=torch.bfloat16, device=dev)
    f_pool = torch.empty((C, host_rows, s.d_qk), dtype=torch.bfloat16, pin_memory=True)
    mpos = torch.empty((s.num_reqs, s.topk), dtype=torch.int32, device=dev)
    rig.restore()
    for r in range(s.rows_per_req):  # untimed pass: the GPU's first touch of the new pools
        lo, hi = r * s.num_reqs, (r + 1) * s.num_reqs
        hs.hs_swap_in(st, b.slots[lo:hi], s.tick0 + r, b.hot_idx[lo:hi], b.miss_count[r], mpos)
        hs.hs_apply_plan(f_hot, f_pool, b.slots[lo:hi], b.hot_idx[lo:hi], b.miss_count[r], mpos,
                         s.capacity)
    rig.restore()
    torch.cuda.synchronize()
    lead_us, apply_us = [], []
    for r in range(s.rows_per_req):
        lo, hi = r * s.num_reqs, (r + 1) * s.num_reqs
        a, m, z = ev(), ev(), ev()
        gpu_busy()
        a.record(main)
        hs.hs_swap_in(st, b.slots[lo:hi], s.tick0 + r, b.hot_idx[lo:hi], b.miss_count[r], mpos)
        m.record(main)
        hs.hs_apply_plan(f_hot, f_pool, b.slots[lo:hi], b.hot_idx[lo:hi], b.miss_count[r], mpos,
                         s.capacity)
        z.record(main)
        torch.cuda.synchronize()
        lead_us.append(a.elapsed_time(m) * 1e3)
        apply_us.append(m.elapsed_time(z) * 1e3)
    apply_gbs = C * sum(wave_bytes) / (sum(apply_us) / 1e6) / 1e9
    del f_hot, f_pool

    # cold wave: empty hot buffer, every selected row is a miss (a gather over the link)
    st.slot_loc.fill_(-1)
    st.slot_stamp.fill_(-1)
    st.loc_to_hot.fill_(-1)
    a, z = ev(), ev()
    gpu_busy()
    a.record(main)
    hs.hs_swap_in(st, b.slots[0:s.num_reqs], s.tick0, b.hot_idx[0:s.num_reqs], b.miss_count[0])
    z.record(main)
    torch.cuda.synchronize()
    cold_us = a.elapsed_time(z) * 1e3
    cold_bytes = int(b.miss_count[0].sum().item()) * row_bytes
    cold_gbs = cold_bytes / (cold_us / 1e6) / 1e9
    rig.release()
    return {
        "workload": "MTP swap decode: 32 requests x 4 rows, seq_len 32768, top-k 2048, 4096 hot "
                    "slots per request, reuse 0.7, 1.21 GB pinned host pool",
        "step": whole, "rows_per_s": whole["rows_per_s"],
        "swap_waves_us": wave_us, "swap_miss_bytes": wave_bytes,
        "swap_GBps": warm_gbs, "swap_frac_of_B_host": warm_gbs / b_host,
        "cold_wave_us": cold_us, "cold_wave_bytes": cold_bytes, "cold_wave_GBps": cold_gbs,
        "mixed_batch": {"resident_requests": n_resident, "step_ms": mixed_ms,
                        "rows_per_s": s.rows / (mixed_ms / 1e3),
                        "all_swap_step_ms": whole["ms_per_step"]},
        "plan_reuse": {"followers": C, "leader_swap_us": lead_us, "apply_plan_us": apply_us,
                       "apply_GBps": apply_gbs, "apply_frac_of_B_host": apply_gbs / b_host},
    }


def measure_finalize(dev, reps=10):
    """Greedy accept + accepted-prefix finalize on the mixed workload's verify shape: 128
    requests x 3 rows, logits [384, 129280] bf16 (99.3 MB), 4096 hot slots per request.
    The sequence lengths are drawn from [2048, 4096] instead of up to 128 K to keep the
    pinned host pool small; the logits, rows and hot buffer are the workload's.  Hot state
    is restored from a device snapshot before every repetition (not timed).  Each call is
    timed as device time: a spin kernel ahead of it covers the host-side marshalling."""
    import numpy as np
    import torch

    import sparse_attention_kv_amd as hs
    from sparse_attention_kv_amd.pipeline import build_hot_state
    from workloads import generate, spec

    s = spec("mixed_finalize", seq_rule=("uniform", 2048, 4096))
    log(f"generate {s.name} (finalize shape)")
    w = generate(s, pin_host_pool=True)

    def d(a):
        return torch.as_tensor(np.ascontiguousarray(a)).to(device=dev, dtype=torch.int32)

    seq, bt = d(w.seq_len), d(w.block_table)
    st = build_hot_state(torch.from_numpy(w.init_pos), torch.from_numpy(w.init_stamp), seq, bt,
                         s.block_size, w.kv_pool, dev)
    snap = [t.clone() for t in (st.slot_loc, st.slot_stamp, st.loc_to_hot)]
    logits, draft, new_kv = w.logits.to(dev), d(w.draft_ids), w.new_kv.to(dev)
    rows = s.rows
    am = torch.empty(rows, dtype=torch.int32, device=dev)
    acc = torch.empty(s.num_reqs, dtype=torch.int32, device=dev)
    nxt = torch.empty(s.num_reqs, dtype=torch.int32, device=dev)
    main = torch.cuda.current_stream()
    times = []
    for rep in range(reps + 2):
        for t, c in zip((st.slot_loc, st.slot_stamp, st.loc_to_hot), snap):
            t.copy_(c)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        gpu_busy()
        e0.record(main)
        hs.hs_finalize_accepted(st, logits, draft, new_kv, s.rows_per_req, seq, bt, s.block_size,
                                s.tick0 + s.rows_per_req, am, acc, nxt)
        e1.record(main)
        torch.cuda.synchronize()
        if rep >= 2:
            times.append(e0.elapsed_time(e1) * 1e3)
    us = float(np.median(times))
    # draft-model context KV append of the accepted prefix (P2 ⑤): 128 requests, context
    # cache of 8 pages x 64 rows each, the verify rows' context K/V as new rows
    ctx_bs, ctx_pages = 64, 8
    ctx_cache = torch.zeros((s.num_reqs * ctx_pages * ctx_bs, s.d_qk), dtype=torch.bfloat16,
                            device=dev)
    ctx_bt = torch.arange(s.num_reqs * ctx_pages, dtype=torch.int32, device=dev).view(
        s.num_reqs, ctx_pages)
    ctx_len0 = torch.full((s.num_reqs,), 100, dtype=torch.int32, device=dev)
    ctx_len = ctx_len0.clone()
    app_times = []
    for rep in range(reps + 2):
        ctx_len.copy_(ctx_len0)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        gpu_busy()
        e0.record(main)
        hs.hs_append_accepted(ctx_cache, ctx_bt, ctx_len, new_kv, acc, ctx_bs, ctx_bs,
                              s.rows_per_req)
        e1.record(main)
        torch.cuda.synchronize()
        if rep >= 2:
            app_times.append(e0.elapsed_time(e1) * 1e3)
    app_rows = int((acc.clamp(0, s.rows_per_req - 1) + 1).sum().item())
    logit_bytes = rows * s.vocab * 2
    return {
        "workload": "greedy accept + finalize: 128 requests x 3 rows, logits [384, 129280] bf16, "
                    "4096 hot slots per request",
        "call_us": us, "logits_bytes": logit_bytes,
        "logits_GBps": logit_bytes / (us / 1e6) / 1e9,
        "logits_frac_of_hbm_peak": logit_bytes / (us / 1e6) / 1e9 / HBM_PEAK_GBS,
        "accept_length_histogram": np.bincount(acc.cpu().numpy(), minlength=s.rows_per_req).tolist(),
        "dflash_context_append_us": float(np.median(app_times)), "dflash_rows_appended": app_rows,
    }


def measure_resolve(dev, reps=100):
    """hs_resolve_topk alone, back-to-back calls, at the batch shapes of the resident (8
    rows), MTP swap (128 rows) and long-context (256 rows, 2048-page tables) workloads;
    a spin kernel ahead of the timed calls covers their host-side marshalling, so the time
    is the device's.  Algorithmic bytes per call: the positions read and the rows written (4 B each per
    entry), plus request id, causal limit and valid count per row; block-table lines are
    not counted."""
    import numpy as np
    import torch

    import sparse_attention_kv_amd as hs
    from workloads import generate, spec

    main = torch.cuda.current_stream()
    out = []
    for name in ("resident", "mtp_swap", "long"):
        s = spec(name)
        w = generate(s, tensors=False)

        def d(a):
            return torch.as_tensor(np.ascontiguousarray(a)).to(device=dev, dtype=torch.int32)

        topk_pos, req_id, lim, bt = d(w.topk_pos), d(w.req_id), d(w.causal_limit), d(w.block_table)
        rows = topk_pos.shape[0]
        slots = torch.empty_like(topk_pos)
        valid = torch.empty((rows,), dtype=torch.int32, device=dev)
        for _ in range(5):
            hs.hs_resolve_topk(topk_pos, req_id, lim, bt, s.block_size, s.block_size, slots, valid)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        gpu_busy(reps * 25.0)  # covers the marshalling of every call: device time only
        e0.record(main)
        for _ in range(reps):
            hs.hs_resolve_topk(topk_pos, req_id, lim, bt, s.block_size, s.block_size, slots, valid)
        e1.record(main)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        alg = rows * s.topk * 8 + rows * 12
        out.append({"workload": s.name, "rows": rows, "topk": s.topk, "us": us,
                    "GBps": alg / (us / 1e6) / 1e9,
                    "hbm_frac": alg / (us / 1e6) / 1e9 / HBM_PEAK_GBS})
    return out


def measure_backup(dev, reps=5):
    """Device -> host backup of prefill KV (staging): 8 requests x 4096 prompt tokens in
    pages of 64 rows, 4 layers of 576 bf16 latent rows -> 512 page transfers, 131072 rows,
    151 MB over the host link.  Device cache 4 x 65536 rows, pinned host cache 4 x 65536
    rows (302 MB each).  Timed: the backup kernel alone (index lists already on the device)
    and the whole BackupStager enqueue (host planning, index copies, kernel), against a
    device -> pinned copy of the same byte count."""
    import numpy as np
    import torch

    import sparse_attention_kv_amd as hs
    from sparse_attention_kv_amd.pipeline import BackupStager, PageTransfer

    L, kbs, per, dev_blocks, host_blocks, pages = 4, 64, 4, 1024, 256, 512
    rows_per_layer = dev_blocks * kbs
    dev_cache = torch.randn((L, rows_per_layer, 576), device=dev).to(torch.bfloat16)
    host_cache = torch.empty((L, host_blocks * per * kbs, 576), dtype=torch.bfloat16,
                             pin_memory=True)
    rng = np.random.default_rng(0)
    src_blocks = rng.permutation(dev_blocks)[:pages]
    host_pages = rng.permutation(host_blocks * per)[:pages]
    transfers = [PageTransfer((int(src_blocks[i]),) * L, int(host_pages[i]) // per,
                              int(host_pages[i]) % per) for i in range(pages)]
    n = pages * kbs
    off = np.arange(kbs)
    src = torch.as_tensor((src_blocks[:, None] * kbs + off).reshape(n).astype(np.int32), device=dev)
    dst = torch.as_tensor((host_pages[:, None] * kbs + off).reshape(n).astype(np.int32), device=dev)
    nbytes = L * n * 1152
    main_s = torch.cuda.current_stream()

    def timed(fn):
        times = []
        for rep in range(reps + 2):
            torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            e0.record(main_s)
            fn()
            e1.record(main_s)
            torch.cuda.synchronize()
            if rep >= 2:
                times.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(times))

    kern_us = timed(lambda: hs.hs_backup_rows(dev_cache, host_cache, src, dst))
    stager = BackupStager(dev_cache, host_cache, kbs, per, max_pages=pages)
    stage_us = timed(lambda: stager.enqueue(transfers))
    flat_dev = dev_cache.view(-1)[: nbytes // 2]
    flat_host = host_cache.view(-1)[: nbytes // 2]
    copy_us = timed(lambda: flat_host.copy_(flat_dev, non_blocking=True))
    b_d2h = nbytes / (copy_us / 1e6) / 1e9
    gbs = nbytes / (kern_us / 1e6) / 1e9
    return {
        "workload": "prefill staging backup: 8 requests x 4096 tokens, 512 pages of 64 rows, "
                    "4 layers of 1152-B rows, device -> pinned host",
        "rows": L * n, "bytes": nbytes, "kernel_us": kern_us, "kernel_GBps": gbs,
        "stager_us": stage_us, "stager_GBps": nbytes / (stage_us / 1e6) / 1e9,
        "memcpy_device_to_pinned_GBps": b_d2h, "kernel_frac_of_memcpy": gbs / b_d2h,
    }


def calibrate_counters(dev):
    """Plain streaming kernel of known size (counter calibration for rocprofv3 --pmc runs):
    the 64 MiB source is written first, then a 512 MiB buffer evicts it from the L2s, so
    the elementwise bitwise_not reads 64 MiB from HBM and writes 64 MiB."""
    import torch
    n = 64 << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(2)
    dst = torch.empty_like(src)
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del flush, src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--part", default="all",
                    choices=["all", "headline", "long", "resident", "sweep", "swap", "finalize",
                             "backup", "resolve", "power"],
                    help="run one section only (for profiler runs); the JSON line then holds "
                         "that section's object, and the headline fields only with 'headline'")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        raise SystemExit("--steps must be >= 1 and --warmup >= 0")

    import torch

    dev = torch.device("cuda:0")
    torch.zeros(1, device=dev)
    calibrate_counters(dev)
    log("host link")
    link = measure_host_link(dev)
    b_host = link["B_host_GBps"]
    if args.part not in ("all", "headline"):
        res = {"part": args.part, "host_link": link}
        run_sections(dev, args, b_host, res, [args.part])
        print(json.dumps(res))
        return

    log(f"headline: {HEADLINE} step, warmup {args.warmup}, steps {args.steps}")
    rig = StepRig(dev, HEADLINE)
    head = measure_step(rig, args.steps, args.warmup, b_host)
    s = rig.s
    swap_counters = stored_counters("swap_in_mixed_finalize_counters.txt", "swap")
    traffic = None
    if swap_counters:
        try:
            traffic = int(swap_counters["traffic_bytes_per_launch"])
        except (KeyError, ValueError):
            traffic = None
    alg_per_launch = head["miss_bytes_per_step"] / s.rows_per_req
    achieved = head["swap_GBps"]
    ms = head["ms_per_step"]
    res = {
        "metric": METRIC, "value": head["rows_per_s"], "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mixed batch + finalize: 128 requests x 3 rows (anchor + 2 drafts), "
                               "seq_len log-uniform [1024, 131072], top-k 2048 (-1 padded below "
                               "2048), block 64, 4096 hot slots per request, reuse 0.6, pinned "
                               "host pool of bf16 576-wide latent rows (4.1 GB), 128 heads x "
                               "576/512, greedy accept over logits [384, 129280] + finalize",
                   "rows_per_step": s.rows, "topk": s.topk, "heads": s.num_heads,
                   "timing": "per step: state restored (untimed), then device time between "
                             "events around resolve + 3 waves (swap-in on a copy stream under "
                             "the previous wave's attention) + accept/finalize, with no event "
                             "inside the step; ms_per_step = mean over the K timed steps"},
        "roofline": {"bound": "host_link", "achieved": achieved, "peak": HOST_LINK_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HOST_LINK_PEAK_GBS, "traffic": traffic,
                     "kernel": "swap_in_kernel (hs_swap_in): zero-copy gather of the missed "
                               "1152-B rows from the pinned host pool",
                     "alg_bytes_per_launch": alg_per_launch,
                     "alg_bytes_read_and_write_per_launch": 2 * alg_per_launch,
                     "launch_us": head["swap_launch_us_mean"],
                     "launch_us_from": "events around each swap-in launch on the copy stream, "
                                       "in K steps run right after the timed ones",
                     "measured_B_host_GBps": b_host, "frac_of_B_host": achieved / b_host,
                     "peak_source": "PCIe 5.0 x16, 64 GB/s per direction (MI355X host interface)"},
        "hbm_roofline": {"bound": "hbm", "kernel": "attention dispatch of the step's last wave "
                                                   "(128 rows, hot buffer; it runs alone)",
                         "achieved": head["attn_last_wave_GBps"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": head["attn_last_wave_hbm_frac"],
                         "alg_bytes_per_launch": float(head["attn_alg_bytes_per_wave"][-1]),
                         "launch_us": head["attn_last_wave_us"],
                         "beside_swap": {"note": "mean over all waves; the earlier waves' "
                                                 "attention runs beside the next wave's swap-in, "
                                                 "whose host reads slow its gathers",
                                         "achieved": head["attn_GBps"],
                                         "frac": head["attn_hbm_frac"],
                                         "launch_us": head["attn_launch_us_mean"]},
                         "power_bound": "from 64 rows up the attention op runs at the board's "
                                        "1400 W limit (bench.py --part power)"},
        "headline_step": head,
        "host_link": link,
    }
    if not args.no_cpu:
        log("cpu baseline (oracle) on a sample of the headline step")
        res["cpu_baseline"] = cpu_baseline(rig.s, rig.w)
    rig.release()
    del rig
    if args.part == "all":
        run_sections(dev, args, b_host, res,
                     ["long", "resident", "sweep", "swap", "finalize", "backup", "resolve"])
    print(json.dumps(res))


def run_sections(dev, args, b_host, res, parts):
    """The secondary measurements, each an object of the JSON line."""
    for part in parts:
        if part == "long":
            log("long-context step")
            lrig = StepRig(dev, "long")
            res["long_context_step"] = measure_step(lrig, min(args.steps, 10),
                                                    max(1, min(args.warmup, 2)), b_host)
            lrig.release()
            del lrig
        elif part == "resident":
            log("resident decode (warm and cold)")
            res["resident_decode"] = measure_resident(dev, args.steps, args.warmup)
        elif part == "sweep":
            log("attention sweep (cold)")
            res["attn_sweep"] = measure_attn_sweep(dev)
        elif part == "swap":
            log("MTP swap workload")
            res["swap_in"] = measure_swap(dev, b_host)
        elif part == "finalize":
            log("finalize")
            res["finalize"] = measure_finalize(dev)
        elif part == "backup":
            log("backup")
            res["backup"] = measure_backup(dev)
        elif part == "resolve":
            log("resolve")
            res["resolve"] = measure_resolve(dev)
        elif part == "power":
            log("attention power and clock")
            res["attn_power"] = measure_power(dev)


if __name__ == "__main__":
    main()
