"""CPU oracle for the HiSparse sparse-decode path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct numpy code (float64 for all floating point) that
states what each step of the path computes.  Only the test-suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product path
(the HIP library and its Python binding) never does, and shares no code,
constants or helpers with it.

Sources (the three web pages the method is described on):

* P1 -- Notion page "hiSparse-MTP": the six-stage main line (summary), and the
  core HiSparse state maps listed under "1. 启动阶段" (startup).
* P2 -- blog post "投机解码的 KV 流转：prefill 阶段 DFlash 也要吃下整个 prompt":
  the 5-token-prompt / 3-draft worked example, sections ③-⑥ and the timeline
  table at the end.
* P3 -- CSDN post "vllm 分析（十二）——Hisparse下篇": the
  ``HiSparseCacheHandle.resolve_topk`` listing, the ``HiSparseHotSpec`` /
  ``HiSparseResidentSpec`` classes, the "数据 back up" section
  (``HiSparseWorker._enqueue_transfers`` address arithmetic) and
  ``build_offload_command`` / ``are_requests_fully_resident``.
* P1 "3. HiSparse staging" and P3 "数据 back up" also describe the device -> host
  backup of new KV rows (``plan_backup_rows``, ``backup_rows``).

Every function is pinned by ``tests/test_oracle_*.py`` against things other than
itself (worked example, closed forms, brute force, library routines).
"""

from .hisparse_ref import (  # noqa: F401
    HotState,
    PageTransfer,
    append_accepted,
    apply_plan,
    as_f64,
    backup_rows,
    build_hot_state,
    finalize_accepted,
    greedy_accept,
    is_fully_resident,
    plan_backup_rows,
    reclaimable_pages,
    resolve_topk,
    select_reclaim_pages,
    sparse_decode_attn,
    sparse_decode_attn_mixed,
    swap_in,
)
