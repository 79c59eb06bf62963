"""The allocation-free chunked entry point (falcon_fwd_chunked_noalloc)
against falcon_fwd_chunked on the same inputs: the same kernels run, so the
results must be identical bit for bit.  Two calls in a row, the second with
a smaller problem, so the second reuses the static scratch the first left
behind; the first is large enough to be processed in two sequence groups."""

import pytest
import torch

from delta_rule_recurrence_amd import falcon as fb
from delta_rule_recurrence_amd import inputs as I

from gpu_utils import to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # (variant, B, H, T): first call, then the smaller second call
    ("falcon1", (8, 12, 2048), (2, 3, 500)),      # Falcon-1 bf16: 100.7 MB of scratch -> 2 groups
    ("falcon1a", (2, 12, 16384), (1, 5, 1300)),   # Falcon-1A tiles: aggregates in the scratch
    ("falcon2", (2, 4, 700), (1, 2, 130)),        # per-column kernel: no scratch at all
]


def _pair(variant, shape, seed, with_state):
    B, H, T = shape
    x = to_dev(I.make_inputs(B, H, T, 64, 64, seed=seed, io_dtype="bf16",
                             per_column_beta=variant in ("falcon2", "falcon2a")))
    S0 = I.random_state((B, H, 64, 64), seed=seed + 1).cuda() if with_state else None
    kp = x["phi_k"][:, :, 0].contiguous() if with_state else None
    ref_o, ref_s = fb.falcon_fwd_chunked(x["phi_k"], x["phi_q"], x["v"], x["beta"], x["lam"],
                                         variant=variant, C=64, S0=S0, k_prev=kp)
    o = torch.empty_like(ref_o)
    S_T = torch.empty_like(ref_s)
    got_o, got_s = fb.falcon_fwd_chunked_noalloc(x["phi_k"], x["phi_q"], x["v"], x["beta"], x["lam"],
                                                 o, variant=variant, C=64, S0=S0, k_prev=kp, S_T=S_T)
    torch.cuda.synchronize()
    return ref_o, ref_s, got_o, got_s


@pytest.mark.parametrize("variant,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_entry_point(variant, first, second):
    for i, (shape, with_state) in enumerate(((first, False), (second, True))):
        print(f"noalloc {variant} call {i + 1}: {shape}", flush=True)
        ref_o, ref_s, got_o, got_s = _pair(variant, shape, 40 + i, with_state)
        assert torch.equal(got_o, ref_o), f"{variant} call {i + 1}: outputs differ"
        assert torch.equal(got_s, ref_s), f"{variant} call {i + 1}: final states differ"
