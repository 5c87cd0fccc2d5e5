"""Set up one workload on both sides: the GPU library (through the C ABI) and the oracle.

Both sides read the same generated tensors; each derives its own state (host rows of
the resident positions, reverse map, resident KV) with its own code.
"""

from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
from tests.helpers import raw
from workloads import generate, spec

BF16_TOL = (2e-2, 1e-2)   # (abs, rel) for bf16 attention outputs
F32_TOL = (1e-5, 1e-5)


def log(msg: str):
    print(f"[gpu-test {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(a, dtype=torch.int32):
    return torch.as_tensor(np.ascontiguousarray(a)).to(device=dev(), dtype=dtype)


def make(name: str, tensors: bool = True, **over):
    s = spec(name, **over)
    log(f"generate {name} {over}")
    w = generate(s, big_device="cuda", pin_host_pool=not s.resident, tensors=tensors)
    return s, w


def gpu_inputs(s, w):
    d = dict(topk_pos=to_dev(w.topk_pos), req_id=to_dev(w.req_id),
             causal_limit=to_dev(w.causal_limit), block_table=to_dev(w.block_table),
             seq_len=to_dev(w.seq_len))
    if w.q is not None:
        d["q"] = w.q.to(dev())
    return d


def oracle_resolve(s, w):
    return oracle.resolve_topk(w.topk_pos, w.req_id, w.causal_limit, w.block_table,
                               s.block_size, s.block_size, s.num_reqs)


def assert_close(got: np.ndarray, ref: np.ndarray, tol, what: str):
    atol, rtol = tol
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside |d|<={atol}+{rtol}|ref|; "
                           f"max err {err.max():.3e}, worst at {np.unravel_index(np.argmax(err - bound), err.shape)}")


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()
