"""Determinism of whole steps: each swap workload's full step (resolve, every wave's swap-in
under the previous wave's attention, and accept + finalize on the mixed workload) run twice
from the same restored state gives bit-identical outputs, LSE, indices, miss counts, maps,
stamps, hot buffer and host rows; the resident call likewise."""

import pytest
import torch

from tests.gpu_cases import dev, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["mtp_swap", "long", "mixed_finalize"])
def test_whole_step_replays_bit_identically(name):
    import bench
    rig = bench.StepRig(dev(), name)
    runs = []
    for rep in range(2):
        rig.restore()
        torch.cuda.synchronize()
        log(f"replay {name}: run {rep}")
        rig.run()
        torch.cuda.current_stream().wait_stream(rig.step.copy_stream)
        torch.cuda.synchronize()
        outs = rig.outputs()
        if rig.host_rows is not None:
            outs.append(rig.w.kv_pool[rig.host_rows].clone())
        runs.append(outs)
    for i, (a, b) in enumerate(zip(*runs)):
        assert torch.equal(a, b), f"{name}: output {i} differs between runs"
    rig.release()


def test_resident_call_replays_bit_identically():
    import numpy as np

    import sparse_attention_kv_amd as hs
    from sparse_attention_kv_amd.pipeline import DecodeStep
    from tests.gpu_cases import gpu_inputs, make
    s, w = make("resident")
    g = gpu_inputs(s, w)
    step = DecodeStep(num_reqs=s.num_reqs, rows_per_req=1, topk=s.topk, num_heads=s.num_heads,
                      d_qk=s.d_qk, d_v=s.d_v, dtype=torch.bfloat16, device=dev())
    outs = []
    for rep in range(3):
        step.run_resident_fused(g["topk_pos"], g["req_id"], g["causal_limit"], g["block_table"],
                                s.block_size, g["q"], w.kv_pool, s.scale)
        torch.cuda.synchronize()
        outs.append((step.buf.out.clone(), step.buf.lse.clone()))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    assert np.isfinite(outs[0][1].cpu().numpy()).all()
    assert hs.hs_attn_plan_info(s.rows, s.num_heads, s.d_qk, s.d_v, s.topk, torch.bfloat16)[1] > 1
