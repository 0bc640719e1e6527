"""The SageSLA step captured in a HIP graph (SageSLAPlan.capture / replay):
every replay reproduces the eager step bit for bit, with eager work and
synchronizations between the replays and the outputs cleared before each."""
import pytest
import torch

import bit_sparse_attention_amd as ssa
from bit_sparse_attention_amd.workloads import make_qkv

pytestmark = pytest.mark.gpu


def _plan(B, H, N, topk, seed, linear=True):
    q, k, v = (t.cuda() for t in make_qkv(B, H, N, 128, seed=seed))
    plan = ssa.SageSLAPlan(B, H, N, topk, linear=linear, device="cuda", want_f32=True)
    return plan.bind(q, k, v)


@pytest.mark.parametrize("topk,linear", [(0.25, True), (0.25, False), (None, False)])
def test_plan_graph_replays_match_eager(topk, linear):
    B, H, N = 1, 2, 3000  # 24 query blocks, 47 key blocks (the last ragged)
    plan = _plan(B, H, N, topk, seed=3, linear=linear)
    plan.run()
    torch.cuda.synchronize()
    ref = plan.out.clone()
    ref32 = plan.out32.clone()
    ref_q = plan.q_i8.clone()
    ref_kidx = None if plan.kidx is None else plan.kidx.clone()
    plan.capture()
    other = _plan(B, H, N, topk, seed=4, linear=linear)  # eager work between replays
    for _ in range(3):
        plan.out.zero_()
        plan.out32.zero_()
        plan.q_i8.zero_()
        plan.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.out, ref)
        assert torch.equal(plan.out32, ref32)
        assert torch.equal(plan.q_i8, ref_q)
        if ref_kidx is not None:
            assert torch.equal(plan.kidx, ref_kidx)
        other.run()
        torch.cuda.synchronize()
        assert not torch.equal(other.out, ref)


def test_replay_without_capture_is_refused():
    plan = _plan(1, 1, 256, 0.5, seed=0)
    with pytest.raises(RuntimeError):
        plan.replay()
