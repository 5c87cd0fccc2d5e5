#!/usr/bin/env python3
"""Benchmark of the HiSparse sparse-decode hot path on one MI355X.

Default workload (the one the headline metric is quoted on): fully resident decode,
8 requests with seq_len ~ U[6144, 8192], one query row each, top-k 2048, block size 64,
128 query heads sharing one 576-wide bf16 latent KV row (value = first 512), scale
1/sqrt(576).  One step = hs_resolve_topk over the 8 rows + hs_sparse_decode_attn on
the paged device pool.  Inputs are synthetic (seeded) and resident in HBM before the
timed region.

Prints ONE JSON line.  `value` = query rows/s of the whole step: K steps launched back to
back on one stream, bracketed by device synchronisation (a captured HIP graph of the step
replayed K times is reported alongside).
`roofline` = that attention op (its dispatches) against the 8 TB/s HBM peak, with its
algorithmic bytes per launch; `cpu_baseline` = the CPU oracle
on the host cores over the same workload.

A second object, `swap_in`, measures the swap path on the 32-request MTP workload: the
host-link reference rate (1 GiB pinned->device copy, and a cold swap-in wave that misses
on every row), the swap-in kernel's rate over its miss bytes, and the whole step.  A third,
`finalize`, times greedy accept + accepted-prefix finalize on the mixed workload's verify
shape (the argmax over 99.3 MB of logits is HBM-bound).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-swap]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ROW_BYTES = 576 * 2


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def attn_alg_bytes(valid_per_row, heads, d_qk, d_v, topk, elem=2):
    """Algorithmic bytes of one attention launch: each valid selected KV row once, the
    query and output rows once, the index row once."""
    rows = len(valid_per_row)
    kv = int(sum(valid_per_row)) * d_qk * elem
    return kv + rows * (heads * d_qk * elem + heads * d_v * elem + topk * 4)


ATTN_SOURCES = ("attn.hip", "attn64.hip", "attn128.hip", "attn_tile.h", "common.h")


def kernel_source_hash():
    """Hash of the attention kernels' sources (ties stored counter figures to them)."""
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, "sparse_attention_kv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary
    (lines `key: value`), if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"attn_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "|")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, s, budget_s=12.0, one_thread_s=6.0):
    """The oracle (numpy, float64) over the same rows, repeated for ~budget_s seconds with
    numpy's own thread pool (all host cores), then for ~one_thread_s seconds limited to one
    thread.  The resolve and attention stages are timed separately."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    def raw(t):
        import torch
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    q, kv = raw(w.q), raw(w.kv_pool)

    def run(budget):
        t_res = t_att = 0.0
        reps = 0
        t0 = time.perf_counter()
        while True:
            a = time.perf_counter()
            slots, _ = oracle.resolve_topk(w.topk_pos, w.req_id, w.causal_limit, w.block_table,
                                           s.block_size, s.block_size, s.num_reqs)
            m = time.perf_counter()
            oracle.sparse_decode_attn(q, kv, slots, s.scale, s.d_v)
            z = time.perf_counter()
            t_res += m - a
            t_att += z - m
            reps += 1
            if z - t0 >= budget:
                break
        return reps, time.perf_counter() - t0, t_res / reps, t_att / reps

    reps, dt, res_s, att_s = run(budget_s)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    with threadpool_limits(limits=1):
        reps1, dt1, res1, att1 = run(one_thread_s)
    return {"value": reps * s.rows / dt, "unit": "rows/s", "cores": int(threads), "kind": "oracle",
            "sample": f"full {s.name} step ({s.rows} rows: resolve_topk + float64 attention) "
                      f"x {reps} repetitions, {dt:.1f} s on {os.cpu_count()} visible host CPUs",
            "stage_ms": {"resolve": res_s * 1e3, "attention": att_s * 1e3},
            "one_thread": {"value": reps1 * s.rows / dt1, "unit": "rows/s",
                           "stage_ms": {"resolve": res1 * 1e3, "attention": att1 * 1e3},
                           "sample": f"{reps1} repetitions, {dt1:.1f} s"}}


def measure_swap(dev, reps=5):
    """Swap path on the 32-request MTP workload (4 rows per request, top-k 2048, 4096 hot
    slots per request, 1.21 GB pinned host pool): host-link reference rate, swap-in
    kernel rates and the whole step.  Hot state is restored from a device snapshot before
    every repetition (not timed).  Each timed region starts behind a short spin kernel, so
    it measures device time, not the host-side marshalling of the first call."""
    import numpy as np
    import torch

    import sparse_attention_kv_amd as hs
    from sparse_attention_kv_amd.pipeline import DecodeStep, build_hot_state
    from workloads import generate, spec

    s = spec("mtp_swap")
    log(f"generate {s.name} (pinned host pool)")
    w = generate(s, pin_host_pool=True)

    def d(a):
        return torch.as_tensor(np.ascontiguousarray(a)).to(device=dev, dtype=torch.int32)

    topk_pos, req_id, lim, bt, seq = (d(w.topk_pos), d(w.req_id), d(w.causal_limit),
                                      d(w.block_table), d(w.seq_len))
    st = build_hot_state(torch.from_numpy(w.init_pos), torch.from_numpy(w.init_stamp), seq, bt,
                         s.block_size, w.kv_pool, dev)
    snap = [t.clone() for t in (st.slot_loc, st.slot_stamp, st.loc_to_hot)]

    def restore():
        for t, c in zip((st.slot_loc, st.slot_stamp, st.loc_to_hot), snap):
            t.copy_(c)

    step = DecodeStep(num_reqs=s.num_reqs, rows_per_req=s.rows_per_req, topk=s.topk,
                      num_heads=s.num_heads, d_qk=s.d_qk, d_v=s.d_v, dtype=torch.bfloat16,
                      capacity=s.capacity, device=dev)
    b = step.buf
    q = w.q.to(dev)
    row_bytes = s.d_qk * 2
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    main = torch.cuda.current_stream()
    copy = step.copy_stream

    # host-link reference: 1 GiB pinned -> device copy
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record(main)
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    e1.record(main)
    torch.cuda.synchronize()
    memcpy_gbs = 3 * n / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst

    # whole step: resolve + 4 waves of (swap-in on the copy stream, attention)
    def run():
        step.run_swap(st, topk_pos, req_id, lim, bt, s.block_size, q, s.scale, s.tick0)

    times = []
    for rep in range(reps + 2):
        restore()
        torch.cuda.synchronize()
        gpu_busy()
        e0.record(main)
        run()
        main.wait_stream(copy)
        e1.record(main)
        torch.cuda.synchronize()
        if rep >= 2:
            times.append(e0.elapsed_time(e1))
    step_ms = float(np.median(times))

    # mixed batch (per-request residency): 16 of the 32 requests lost one resident page and
    # swap in; the other 16 read a resident pool (a device copy of the host pool, same rows)
    from sparse_attention_kv_amd.pipeline import ResidencyTracker
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
        restore()
        torch.cuda.synchronize()
        gpu_busy()
        e0.record(main)
        mstep.run_mixed(st, topk_pos, req_res, req_swap, sel, lim, res_bt, bt, s.block_size, q,
                        dev_pool, s.scale, s.tick0)
        main.wait_stream(mstep.copy_stream)
        e1.record(main)
        torch.cuda.synchronize()
        if rep >= 2:
            mtimes.append(e0.elapsed_time(e1))
    mixed_ms = float(np.median(mtimes))
    del dev_pool, mstep

    # swap-in alone, wave by wave, from the same starting state: one untimed pass (the
    # GPU's first touch of host-pool pages that no earlier call read), then the median of
    # three timed passes per wave
    restore()
    hs.hs_resolve_topk(topk_pos, req_id, lim, bt, s.block_size, s.block_size, b.slots, b.valid)
    passes = []
    for rep in range(4):
        restore()
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
    for r in range(s.rows_per_req):  # untimed pass: the GPU's first touch of the new pools
        lo, hi = r * s.num_reqs, (r + 1) * s.num_reqs
        hs.hs_swap_in(st, b.slots[lo:hi], s.tick0 + r, b.hot_idx[lo:hi], b.miss_count[r], mpos)
        hs.hs_apply_plan(f_hot, f_pool, b.slots[lo:hi], b.hot_idx[lo:hi], b.miss_count[r], mpos,
                         s.capacity)
    restore()
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

    # cold wave: empty hot buffer, every selected row is a miss (streaming zero-copy read)
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
    b_host = max(memcpy_gbs, cold_gbs)
    return {
        "workload": "MTP swap decode: 32 requests x 4 rows, seq_len 32768, top-k 2048, 4096 hot "
                    "slots per request, reuse 0.7, 1.21 GB pinned host pool",
        "rows_per_step": s.rows, "step_ms": step_ms, "rows_per_s": s.rows / (step_ms / 1e3),
        "B_host_GBps": b_host, "memcpy_pinned_to_device_GBps": memcpy_gbs,
        "swap_waves_us": wave_us, "swap_miss_bytes": wave_bytes,
        "swap_GBps": warm_gbs, "swap_frac_of_B_host": warm_gbs / b_host,
        "cold_wave_us": cold_us, "cold_wave_bytes": cold_bytes, "cold_wave_GBps": cold_gbs,
        "mixed_batch": {"resident_requests": n_resident, "step_ms": mixed_ms,
                        "rows_per_s": s.rows / (mixed_ms / 1e3), "all_swap_step_ms": step_ms},
        "plan_reuse": {"followers": C, "leader_swap_us": lead_us, "apply_plan_us": apply_us,
                       "apply_GBps": apply_gbs, "apply_frac_of_B_host": apply_gbs / b_host},
    }


def gpu_busy(us=100.0):
    """Keep the GPU busy for about ``us`` microseconds, so that an event recorded after it
    times the device work of the calls enqueued meanwhile, not their host-side marshalling."""
    import torch
    torch.cuda._sleep(int(us * 2000))  # spin kernel counting shader clocks (~2 GHz)


MFMA_BF16_PEAK_TFLOPS = 2500.0
SETTLE_MS = 50.0  # untimed back-to-back work before a timed region (clock settling)


def measure_attn_sweep(dev, sizes=(32, 64, 128, 256), reps=50):
    """The attention op alone at the batch sizes of the other workloads: one swap wave of
    the MTP workload (32 rows), of the long-context workload (64), of the mixed workload
    (128), and the long-context workload's 256 rows at once.  Top-k 2048 distinct rows per
    query row, drawn uniformly from a resident pool of 1M bf16 576-wide latent rows
    (1.15 GB, N(0,1)); 128 heads, value = first 512 dims, scale 1/sqrt(576).  Each size is
    timed over back-to-back calls; the kernel (32-, 64- or 128-head workgroups) is the
    library planner's choice."""
    import torch

    import sparse_attention_kv_amd as hs
    H, D, DV, K, N = 128, 576, 512, 2048, 1 << 20
    g = torch.Generator(device=dev).manual_seed(20261202)
    kv = torch.randn((N, D), generator=g, device=dev).to(torch.bfloat16)
    main = torch.cuda.current_stream()
    out_rows = []
    for rows in sizes:
        q = torch.randn((rows, H, D), generator=g, device=dev).to(torch.bfloat16)
        idx = torch.stack([torch.randperm(N, generator=g, device=dev)[:K] for _ in range(rows)])
        idx = idx.to(torch.int32).contiguous()
        out = torch.empty((rows, H, DV), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((rows, H), dtype=torch.float32, device=dev)
        wsb = hs.hs_attn_workspace_bytes(rows, H, D, DV, K, torch.bfloat16)
        ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device=dev) if wsb else None
        # Untimed warm-up of >= SETTLE_MS of back-to-back calls: the shader clock takes tens
        # of milliseconds of sustained load to settle, and calls timed before that run slow.
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main)
        for _ in range(5):
            hs.hs_sparse_decode_attn(q, kv, idx, D ** -0.5, DV, out, lse, ws)
        e1.record(main)
        torch.cuda.synchronize()
        est_us = e0.elapsed_time(e1) * 1e3 / 5
        for _ in range(int(SETTLE_MS * 1e3 / max(est_us, 1.0)) + 1):
            hs.hs_sparse_decode_attn(q, kv, idx, D ** -0.5, DV, out, lse, ws)
        torch.cuda.synchronize()
        e0.record(main)
        for _ in range(reps):
            hs.hs_sparse_decode_attn(q, kv, idx, D ** -0.5, DV, out, lse, ws)
        e1.record(main)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        alg = attn_alg_bytes([K] * rows, H, D, DV, K)
        flops = rows * K * 2 * H * (D + DV)
        out_rows.append({"rows": rows, "us": us, "rows_per_s": rows / (us / 1e6),
                         "GBps": alg / (us / 1e6) / 1e9,
                         "hbm_frac": alg / (us / 1e6) / 1e9 / HBM_PEAK_GBS,
                         "TFLOPs": flops / (us / 1e6) / 1e12,
                         "mfma_frac": flops / (us / 1e6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                         "split_workspace_bytes": wsb})
        del q, idx, out, lse, ws
    del kv
    return {"workload": "attention op alone, top-k 2048 distinct rows of a 1M-row resident "
                        "pool, 128 heads x 576/512 bf16", "sizes": out_rows}


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
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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


def measure_config_steps(dev, reps=3):
    """Whole steps of the long-context workload (64 requests x 4 rows, seq_len 131072, reuse
    0.5, 9.66 GB pinned host pool) and the mixed + finalize workload (128 requests x 3 rows,
    seq_len log-uniform in [1024, 131072], reuse 0.6, logits [384, 129280]): resolve, then
    per wave swap-in on the copy stream under attention on the main stream, and for the
    mixed workload greedy accept + finalize.  Hot state restored before every repetition;
    each timed region starts behind a spin kernel (device time)."""
    import numpy as np
    import torch

    import sparse_attention_kv_amd as hs
    from sparse_attention_kv_amd.pipeline import DecodeStep, build_hot_state
    from workloads import generate, spec

    main = torch.cuda.current_stream()
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(main)
    for _ in range(4):
        dst.copy_(src, non_blocking=True)
    e1.record(main)
    torch.cuda.synchronize()
    b_host = 4 * n / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    out = {"B_host_GBps": b_host}
    for name in ("long", "mixed_finalize"):
        s = spec(name)
        log(f"generate {s.name} (pinned host pool)")
        w = generate(s, big_device="cuda", pin_host_pool=True)

        def d(a):
            return torch.as_tensor(np.ascontiguousarray(a)).to(device=dev, dtype=torch.int32)

        topk_pos, req_id, lim, bt, seq = (d(w.topk_pos), d(w.req_id), d(w.causal_limit),
                                          d(w.block_table), d(w.seq_len))
        st = build_hot_state(torch.from_numpy(w.init_pos), torch.from_numpy(w.init_stamp), seq,
                             bt, s.block_size, w.kv_pool, dev)
        snap = [t.clone() for t in (st.slot_loc, st.slot_stamp, st.loc_to_hot)]
        step = DecodeStep(num_reqs=s.num_reqs, rows_per_req=s.rows_per_req, topk=s.topk,
                          num_heads=s.num_heads, d_qk=s.d_qk, d_v=s.d_v, dtype=torch.bfloat16,
                          capacity=s.capacity, finalize=s.finalize, device=dev)
        q = w.q.to(dev)
        fin = None
        if s.finalize:
            fin = dict(logits=w.logits.to(dev), draft_ids=d(w.draft_ids), new_kv=w.new_kv.to(dev),
                       seq_len=seq)
        times = []
        for rep in range(reps + 1):
            for t, c in zip((st.slot_loc, st.slot_stamp, st.loc_to_hot), snap):
                t.copy_(c)
            torch.cuda.synchronize()
            gpu_busy()
            e0.record(main)
            step.run_swap(st, topk_pos, req_id, lim, bt, s.block_size, q, s.scale, s.tick0,
                          finalize=fin)
            main.wait_stream(step.copy_stream)
            e1.record(main)
            torch.cuda.synchronize()
            if rep >= 1:
                times.append(e0.elapsed_time(e1))
        ms = float(np.median(times))
        miss_bytes = int(step.buf.miss_count.sum().item()) * s.d_qk * 2
        out[name] = {"workload": s.name, "rows_per_step": s.rows, "waves": s.rows_per_req,
                     "step_ms": ms, "rows_per_s": s.rows / (ms / 1e3), "miss_bytes": miss_bytes,
                     "miss_GBps": miss_bytes / (ms / 1e3) / 1e9,
                     "frac_of_B_host": miss_bytes / (ms / 1e3) / 1e9 / b_host,
                     "finalize": bool(s.finalize)}
        del w, st, step, q, fin, snap
        torch.cuda.empty_cache()
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
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # The default warm-up covers the shader clock's settling time (tens of ms of sustained
    # load; the resident step takes ~17 us, so 3000 steps are ~50 ms): steps timed before
    # that run about 7 % slow.
    ap.add_argument("--warmup", type=int, default=3000)
    ap.add_argument("--workload", default="resident")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-swap", action="store_true", help="skip the swap-path measurement")
    ap.add_argument("--configs", action="store_true",
                    help="also time whole steps of the long-context and mixed workloads "
                         "(9.66 GB pinned host pool; not in the default run)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the attention sweep over larger batches")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_attention_kv_amd as hs
    from sparse_attention_kv_amd.pipeline import DecodeStep
    from workloads import generate, spec

    if args.workload != "resident":
        raise SystemExit("only the resident decode workload is a bench line; the others are "
                         "parity-test cases")
    dev = torch.device("cuda:0")
    s = spec(args.workload)
    log(f"generate {s.name}")
    w = generate(s, big_device="cuda")

    def d(a):
        return torch.as_tensor(np.ascontiguousarray(a)).to(device=dev, dtype=torch.int32)

    topk_pos, req_id, lim, bt = d(w.topk_pos), d(w.req_id), d(w.causal_limit), d(w.block_table)
    q = w.q.to(dev)
    kv = w.kv_pool
    step = DecodeStep(num_reqs=s.num_reqs, rows_per_req=s.rows_per_req, topk=s.topk,
                      num_heads=s.num_heads, d_qk=s.d_qk, d_v=s.d_v, dtype=torch.bfloat16,
                      device=dev)
    b = step.buf

    # resolve + attention in one C-ABI call (positions are resolved in the attention
    # prologue), its arguments marshalled once: the decode buffers stay at fixed addresses.
    fused_call = hs.PagedAttnCall(q, kv, topk_pos, req_id, lim, bt, s.block_size, s.block_size,
                                  s.scale, s.d_v, b.out, b.lse, b.workspace)

    def run_step():
        fused_call()

    def run_step_two_calls():
        step.run_resident(topk_pos, req_id, lim, bt, s.block_size, q, kv, s.scale)

    # plain streaming kernel of known size (counter calibration for rocprofv3 --pmc runs):
    # the 64 MiB source is written first, then a 512 MiB buffer evicts it from the L2s, so
    # the elementwise bitwise_not reads 64 MiB from HBM and writes 64 MiB.
    calib_n = 64 << 20
    src = torch.empty(calib_n, dtype=torch.uint8, device=dev).fill_(1)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(2)
    dst = torch.empty_like(src)
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del flush, src, dst

    log(f"warmup {args.warmup}")
    run_step_two_calls()  # fills b.valid (per-row valid counts) for the algorithmic bytes
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    valid = b.valid.cpu().numpy()
    alg = attn_alg_bytes(valid, s.num_heads, s.d_qk, s.d_v, s.topk)

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # eager launches of the whole step
    e0.record(stream)
    for _ in range(args.steps):
        run_step()
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / args.steps

    # the same step as two calls (hs_resolve_topk, then hs_sparse_decode_attn), for reference
    for _ in range(args.warmup):
        run_step_two_calls()
    e0.record(stream)
    for _ in range(args.steps):
        run_step_two_calls()
    e1.record(stream)
    torch.cuda.synchronize()
    two_call_ms = e0.elapsed_time(e1) / args.steps

    graph_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            run_step()                       # warm on the capture stream
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=cap):
                run_step()
        torch.cuda.synchronize()
        ref_out = b.out.clone()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / args.steps
        assert torch.equal(b.out, ref_out), "graph replay differs from eager result"

    ms = eager_ms
    value = s.rows / (ms / 1e3)
    attn_t = eager_ms  # the step is one attention op (its attention + combine dispatches)
    achieved = alg / (attn_t / 1e3) / 1e9
    traffic = stored_traffic(args.workload)
    plan_ws = hs.hs_attn_workspace_bytes(s.rows, s.num_heads, s.d_qk, s.d_v, s.topk, torch.bfloat16)
    res = {
        "metric": "sparse-decode query rows/s at topk=2048; achieved HBM GB/s (% of peak)",
        "value": value, "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "resident decode: 8 requests, seq_len U[6144,8192], 1 row each, "
                               "top-k 2048, block 64, 128 heads x 576/512 bf16 latent KV",
                   "rows_per_step": s.rows, "topk": s.topk, "heads": s.num_heads,
                   "timing": "K eager steps on one stream between synchronisations (one C-ABI call per step, arguments marshalled once)",
                   "eager_ms_per_step": eager_ms, "graph_ms_per_step": graph_ms,
                   "two_call_ms_per_step": two_call_ms,
                   "attn_split_workspace_bytes": plan_ws},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "kernel": "hs_sparse_decode_attn_paged (attention with position "
                               "resolution + split combine dispatches)",
                     "alg_bytes_per_launch": alg,
                     "launch_us": attn_t * 1e3},
    }
    log("resolve")
    res["resolve"] = measure_resolve(dev)
    if not args.no_sweep:
        log("attention sweep")
        res["attn_sweep"] = measure_attn_sweep(dev)
    if not args.no_swap:
        log("swap path")
        res["swap_in"] = measure_swap(dev)
        log("finalize")
        res["finalize"] = measure_finalize(dev)
        log("backup")
        res["backup"] = measure_backup(dev)
    if args.configs:
        log("whole steps of the long-context and mixed workloads")
        res["config_steps"] = measure_config_steps(dev)
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(w, s)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
