"""The chunked forward captured into a HIP graph (through torch's graph
capture of the launch stream) and replayed: every replay, with other eager
work and synchronisations between replays, must reproduce the eager result
bit for bit.  The forward path issues kernel launches only (no memset, no
allocation), so it is capturable."""

import pytest
import torch

from delta_rule_recurrence_amd import falcon as fb
from delta_rule_recurrence_amd import inputs as I

from gpu_utils import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("variant,per_col", [("falcon1", False), ("falcon1a", False), ("falcon2", True)])
def test_chunked_forward_graph_replay(variant, per_col):
    B, H, T = 2, 3, 300
    d = to_dev(I.make_inputs(B, H, T, 64, 64, seed=91, io_dtype="bf16", per_column_beta=per_col))
    other = to_dev(I.make_inputs(B, H, T, 64, 64, seed=92, io_dtype="bf16", per_column_beta=per_col))
    p = fb.make_problem(B, H, T, 64, 64, variant=variant, io_dtype=torch.bfloat16)
    ws = torch.empty(max(fb.falcon_workspace_bytes(p, 64), 16), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, H, T, 64), dtype=torch.bfloat16, device="cuda")
    S_T = torch.empty((B, H, 64, 64), dtype=torch.float32, device="cuda")

    def step(x):
        fb.falcon_fwd_chunked(x["phi_k"], x["phi_q"], x["v"], x["beta"], x["lam"], variant=variant, C=64,
                              o=o, S_T=S_T, workspace=ws)

    step(d)
    torch.cuda.synchronize()
    o_ref, S_ref = o.clone(), S_T.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(d)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(d)

    for rep in range(3):
        # eager work on the same buffers between replays
        step(other)
        torch.cuda.synchronize()
        assert not torch.equal(o, o_ref)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"{variant}: replay {rep} differs from the eager outputs"
        assert torch.equal(S_T, S_ref), f"{variant}: replay {rep} differs from the eager final state"
