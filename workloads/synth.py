"""The five synthetic decode workloads, generated from fixed seeds.

Every shape, size and distribution below follows the workload descriptions the
path is measured on (DeepSeek-style MLA decode: 128 query heads sharing one
576-wide latent KV row whose first 512 entries are the value; top-k 2048 sparse
selection; speculative verify rows).  The pages themselves name no public
dataset; these synthetic inputs stand in for real traffic.

What is drawn here, and nothing more:

* per-request sequence lengths;
* block tables: one random permutation of the physical pages, dealt to the
  requests in order (no page is shared, so host rows belong to one request);
* per query row, a list of top-k token *positions* (distinct, uniform, or
  re-used from the previous step's set with probability ``reuse_p``), padded
  with -1 when the causal limit is shorter than k;
* per request, which token *positions* sit in which hot-buffer slot at the start
  of the step, with their LRU stamps;
* random tensors: the KV pool rows, the queries, and for the finalize workload
  the verify-row KV, draft ids and logits.

Positions are turned into physical rows only by the code under test and by the
oracle, each with its own implementation.  Large tensors can be drawn directly
on a GPU (``big_device="cuda"``) with a seeded generator; the values then differ
from a CPU draw, but every consumer of one ``Workload`` sees the same tensors.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

ROOT_SEED = 20261202


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    index: int                  # seed sub-stream
    num_reqs: int
    rows_per_req: int           # anchor + draft rows verified together
    block_size: int
    bt_stride: int              # block-table row width (pages)
    topk: int
    num_heads: int
    d_qk: int
    d_v: int
    dtype: str                  # "bf16" or "f32"
    resident: bool              # True: all KV in a paged device pool, no swap-in
    capacity: int = 0           # hot slots per request (swap workloads)
    reuse_p: float = 0.0        # probability a top-k entry comes from the previous set
    finalize: bool = False
    vocab: int = 0
    seq_rule: tuple = ()        # ("fixed", [..]) | ("uniform", lo, hi) | ("const", n) | ("loguniform", lo, hi)
    phys_pages: int = 0         # 0: exactly the pages the requests need
    init_resident: str = "prev" # "prev": previous top-k set + older fill; "half": random half (tiny)
    q_acc: float = 0.7          # probability a draft id equals the planted argmax of the row before
    tie_frac: float = 0.1       # fraction of logit rows with a planted tie at the maximum
    tick0: int = 1000

    @property
    def rows(self) -> int:
        return self.num_reqs * self.rows_per_req

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)


CONFIGS = {
    "tiny": WorkloadSpec(
        name="tiny", index=0, num_reqs=2, rows_per_req=3, block_size=16, bt_stride=16,
        topk=16, num_heads=4, d_qk=64, d_v=48, dtype="f32", resident=False, capacity=24,
        reuse_p=0.0, seq_rule=("fixed", [37, 70]), phys_pages=16, init_resident="half"),
    "resident": WorkloadSpec(
        name="resident", index=1, num_reqs=8, rows_per_req=1, block_size=64, bt_stride=128,
        topk=2048, num_heads=128, d_qk=576, d_v=512, dtype="bf16", resident=True,
        seq_rule=("uniform", 6144, 8192)),
    "mtp_swap": WorkloadSpec(
        name="mtp_swap", index=2, num_reqs=32, rows_per_req=4, block_size=64, bt_stride=512,
        topk=2048, num_heads=128, d_qk=576, d_v=512, dtype="bf16", resident=False,
        capacity=4096, reuse_p=0.7, seq_rule=("const", 32768)),
    "long": WorkloadSpec(
        name="long", index=3, num_reqs=64, rows_per_req=4, block_size=64, bt_stride=2048,
        topk=2048, num_heads=128, d_qk=576, d_v=512, dtype="bf16", resident=False,
        capacity=4096, reuse_p=0.5, seq_rule=("const", 131072)),
    "mixed_finalize": WorkloadSpec(
        name="mixed_finalize", index=4, num_reqs=128, rows_per_req=3, block_size=64,
        bt_stride=2048, topk=2048, num_heads=128, d_qk=576, d_v=512, dtype="bf16",
        resident=False, capacity=4096, reuse_p=0.6, finalize=True, vocab=129280,
        seq_rule=("loguniform", 1024, 131072)),
}


def spec(name: str, **overrides) -> WorkloadSpec:
    """A named workload, optionally with fields replaced (smaller test variants)."""
    s = CONFIGS[name]
    return replace(s, **overrides) if overrides else s


@dataclass
class Workload:
    spec: WorkloadSpec
    seq_len: np.ndarray            # int32 [num_reqs]
    block_table: np.ndarray        # int32 [num_reqs, bt_stride], -1 past the request's pages
    num_pages: int
    req_id: np.ndarray             # int32 [rows], row = r * num_reqs + b  ->  b
    causal_limit: np.ndarray       # int32 [rows]
    topk_pos: np.ndarray           # int32 [rows, topk], token positions, -1 padded
    kv_pool: torch.Tensor          # [num_pages * block_size, d_qk]; pinned host or device
    q: torch.Tensor                # [rows, num_heads, d_qk] (CPU)
    init_pos: Optional[np.ndarray] = None    # int32 [num_reqs, capacity]: position held, -1 empty
    init_stamp: Optional[np.ndarray] = None  # int32 [num_reqs, capacity]: LRU stamp, -1 empty
    draft_ids: Optional[np.ndarray] = None   # int32 [rows]
    logits: Optional[torch.Tensor] = None    # bf16 [rows, vocab] (CPU)
    new_kv: Optional[torch.Tensor] = None    # [rows, d_qk] (CPU)
    extra: dict = field(default_factory=dict)

    @property
    def host_rows(self) -> int:
        return self.num_pages * self.spec.block_size


def _torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _randn(shape, dtype: torch.dtype, seed: int, device: str = "cpu", pin: bool = False,
           chunk: int = 1 << 24) -> torch.Tensor:
    """N(0,1) drawn in float32 with a seeded generator on `device`, rounded to `dtype`
    (round-to-nearest-even), delivered on `device` or, with `pin`, in pinned host memory."""
    n = int(np.prod(shape))
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    if pin:
        out = torch.empty(n, dtype=dtype, pin_memory=True)
    else:
        out = torch.empty(n, dtype=dtype, device=device)
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        t = torch.randn(m, generator=gen, device=device, dtype=torch.float32).to(dtype)
        out[i:i + m].copy_(t)
    return out.view(*shape)


def _seq_lens(s: WorkloadSpec, rng: np.random.Generator) -> np.ndarray:
    kind = s.seq_rule[0]
    if kind == "fixed":
        v = np.array(s.seq_rule[1], dtype=np.int64)
    elif kind == "uniform":
        v = rng.integers(s.seq_rule[1], s.seq_rule[2], size=s.num_reqs, endpoint=True)
    elif kind == "const":
        v = np.full(s.num_reqs, s.seq_rule[1], dtype=np.int64)
    elif kind == "loguniform":
        v = np.floor(np.exp(rng.uniform(math.log(s.seq_rule[1]), math.log(s.seq_rule[2]),
                                        size=s.num_reqs))).astype(np.int64)
        v = np.clip(v, s.seq_rule[1], s.seq_rule[2])
    else:
        raise ValueError(kind)
    assert v.shape == (s.num_reqs,)
    return v.astype(np.int32)


def _block_table(s: WorkloadSpec, seq: np.ndarray, rng: np.random.Generator):
    need = [-(-int(n) // s.block_size) for n in seq]
    total = s.phys_pages or sum(need)
    assert total >= sum(need) and max(need) <= s.bt_stride
    perm = rng.permutation(total).astype(np.int32)
    bt = np.full((s.num_reqs, s.bt_stride), -1, dtype=np.int32)
    at = 0
    for b, k in enumerate(need):
        bt[b, :k] = perm[at:at + k]
        at += k
    return bt, total


def _fresh_distinct(rng, c: int, need: int, taken: np.ndarray) -> np.ndarray:
    """`need` distinct positions uniform on [0, c) not marked in `taken` (marks them)."""
    out = []
    while need > 0:
        cand = rng.integers(0, c, size=2 * need + 16)
        _, first = np.unique(cand, return_index=True)
        vals = cand[np.sort(first)]
        vals = vals[~taken[vals]][:need]
        taken[vals] = True
        out.append(vals)
        need -= len(vals)
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def _topk_row(rng, c: int, K: int, prev: Optional[np.ndarray], p: float) -> np.ndarray:
    row = np.full(K, -1, dtype=np.int64)
    if c <= K:
        row[:c] = rng.permutation(c)
        return row
    if prev is None or p <= 0.0 or len(prev) == 0:
        return rng.choice(c, K, replace=False)
    take = rng.random(K) < p
    slots = np.nonzero(take)[0]
    n_reuse = min(len(slots), len(prev))
    reused = rng.permutation(prev)[:n_reuse]
    taken = np.zeros(c, dtype=bool)
    taken[reused] = True
    row[slots[:n_reuse]] = reused
    rest = np.nonzero(row < 0)[0]
    row[rest] = _fresh_distinct(rng, c, len(rest), taken)
    return row


def generate(s: WorkloadSpec, big_device: str = "cpu", pin_host_pool: bool = False,
             tensors: bool = True) -> Workload:
    """Draw one step's inputs for workload `s`.

    `big_device` is where the KV pool is drawn ("cpu" or "cuda"); for swap workloads
    the pool is then delivered in pinned host memory when `pin_host_pool`, and for
    the resident workload it stays on `big_device` (it is the paged device pool).
    With `tensors=False` only the index structure is drawn (kv_pool, q, logits and
    new_kv are None); every index array is the same as with tensors.
    """
    ss = np.random.SeedSequence(ROOT_SEED).spawn(len(CONFIGS) + 8)[s.index]
    r_seq, r_bt, r_topk, r_hot, r_tensor, r_acc = [np.random.default_rng(x) for x in ss.spawn(6)]
    tseeds = [int(x) for x in ss.generate_state(8)]

    R, B, K = s.rows_per_req, s.num_reqs, s.topk
    seq = _seq_lens(s, r_seq)
    bt, num_pages = _block_table(s, seq, r_bt)

    rows = B * R
    req_id = np.tile(np.arange(B, dtype=np.int32), R)                 # wave-major rows
    n = seq.astype(np.int64) - R                                       # committed length
    assert (n >= 0).all()
    causal = np.empty(rows, dtype=np.int32)
    for r in range(R):
        causal[r * B:(r + 1) * B] = n + r + 1

    prev = [None] * B
    if s.reuse_p > 0:
        prev = [r_topk.choice(int(n[b]), min(K, int(n[b])), replace=False) for b in range(B)]
    topk = np.empty((rows, K), dtype=np.int32)
    for r in range(R):
        for b in range(B):
            topk[r * B + b] = _topk_row(r_topk, int(causal[r * B + b]), K, prev[b], s.reuse_p)

    init_pos = init_stamp = None
    if not s.resident:
        cap = s.capacity
        init_pos = np.full((B, cap), -1, dtype=np.int32)
        init_stamp = np.full((B, cap), -1, dtype=np.int32)
        for b in range(B):
            if s.init_resident == "half":
                cnt = min(cap, int(seq[b]) // 2)
                pos = r_hot.choice(int(seq[b]), cnt, replace=False)
                stamp = r_hot.integers(0, 3, size=cnt)
            else:
                pv = prev[b] if prev[b] is not None else np.zeros(0, dtype=np.int64)
                cnt = min(cap, int(n[b]))
                taken = np.zeros(int(n[b]), dtype=bool)
                taken[pv] = True
                others = _fresh_distinct(r_hot, int(n[b]), cnt - len(pv), taken)
                pos = np.concatenate([pv, others])
                stamp = np.concatenate([np.full(len(pv), 999), r_hot.integers(0, 999, size=len(others))])
            slots = r_hot.permutation(cap)[:len(pos)]
            init_pos[b, slots] = pos
            init_stamp[b, slots] = stamp

    dt = _torch_dtype(s.dtype)
    host_rows = num_pages * s.block_size
    if not tensors:
        kv_pool = q = None
    elif s.resident:
        kv_pool = _randn((host_rows, s.d_qk), dt, tseeds[0], device=big_device)
    else:
        kv_pool = _randn((host_rows, s.d_qk), dt, tseeds[0], device=big_device,
                         pin=pin_host_pool and big_device == "cpu")
        if big_device != "cpu":
            host = torch.empty((host_rows, s.d_qk), dtype=dt, pin_memory=pin_host_pool)
            host.copy_(kv_pool)
            kv_pool = host
    if tensors:
        q = _randn((rows, s.num_heads, s.d_qk), dt, tseeds[1])

    w = Workload(spec=s, seq_len=seq, block_table=bt, num_pages=num_pages, req_id=req_id,
                 causal_limit=causal, topk_pos=topk, kv_pool=kv_pool, q=q,
                 init_pos=init_pos, init_stamp=init_stamp)

    if s.finalize:
        V = s.vocab
        logits = _randn((rows, V), torch.bfloat16, tseeds[2]) if tensors else None
        # Plant a maximum per row (a value no N(0,1) bf16 draw reaches), and in a
        # fraction of rows a second, equal maximum: the accept rule then has to break
        # the tie.  Draft ids copy the planted id of the previous row with
        # probability q_acc, so acceptance lengths spread over 0..R-1.
        plant = r_acc.integers(0, V, size=rows)
        if tensors:
            logits[torch.arange(rows), torch.from_numpy(plant)] = 16.0
        tie_rows = np.nonzero(r_acc.random(rows) < s.tie_frac)[0]
        for i in tie_rows:
            other = int(r_acc.integers(0, V - 1))
            other += other >= plant[i]
            if tensors:
                logits[int(i), other] = 16.0
        draft = r_acc.integers(0, V, size=rows).astype(np.int64)
        for r in range(1, R):
            for b in range(B):
                src = plant[(r - 1) * B + b]
                if r_acc.random() < s.q_acc:
                    draft[r * B + b] = src
                else:
                    d = int(r_acc.integers(0, V - 1))
                    draft[r * B + b] = d + (d >= src)
        w.logits = logits
        w.draft_ids = draft.astype(np.int32)
        w.new_kv = _randn((rows, s.d_qk), dt, tseeds[3]) if tensors else None
    return w
