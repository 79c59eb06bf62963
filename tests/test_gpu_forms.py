"""The two forms of the Falcon-1 bf16 chunked fast path -- one launch (chunk
workgroups and per-sequence chains side by side, handing chunk matrices over
through flags) and two launches (all chunk matrices, then the chains) --
compute the same chunk form ("Fast Weight Attention for Continual Learning",
Section 4.2, chunk-parallel implementation; Eq. 3.3 per chunk) with the same
roundings.  Their outputs and final states must agree bit for bit, on shapes
with one chunk, a ragged tail, a carried state and key, a sequence count that
is not a multiple of the eight XCDs, and the full workload shape.  Each form
is checked against the oracle by the parity tests; this pins the hand-over of
the one-launch form against the other, independently scheduled form."""

import numpy as np
import pytest
import torch

from delta_rule_recurrence_amd import falcon as fb
from delta_rule_recurrence_amd import inputs as I

from gpu_utils import to_dev

pytestmark = pytest.mark.gpu

CASES = {
    "one_chunk": (1, 1, 64, False),
    "ragged_carry": (1, 3, 200, True),
    "18_sequences": (2, 9, 1000, False),
    "workload_carry": (8, 12, 2048, True),
}


def inputs(B, H, T, carry, seed):
    x = I.make_inputs(B, H, T, 64, 64, seed=seed, io_dtype="bf16")
    if carry:
        g = np.random.default_rng([seed, 3])
        x["S0"] = torch.from_numpy((0.1 * g.standard_normal((B, H, 64, 64))).astype(np.float32))
        x["k_prev"] = torch.from_numpy(np.abs(g.standard_normal((B, H, 64))).astype(np.float32)).to(torch.bfloat16)
    return to_dev(x)


def run(d, form):
    prev = fb.falcon_set_f1_launch_form(form)
    try:
        o, S_T = fb.falcon_fwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], C=64,
                                       S0=d.get("S0"), k_prev=d.get("k_prev"))
        torch.cuda.synchronize()
    finally:
        fb.falcon_set_f1_launch_form(prev)
    return o.cpu(), S_T.cpu()


@pytest.mark.parametrize("name", sorted(CASES))
def test_launch_forms_bit_identical(name):
    B, H, T, carry = CASES[name]
    print(f"[forms] {name}: B={B} H={H} T={T} carry={carry}", flush=True)
    d = inputs(B, H, T, carry, seed=1200 + len(name))
    o1, s1 = run(d, fb.F1_ONE_LAUNCH)
    o2, s2 = run(d, fb.F1_TWO_LAUNCH)
    assert torch.isfinite(o1.float()).all() and torch.isfinite(s1).all()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "outputs differ between the launch forms"
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32)), "final states differ between the launch forms"


@pytest.mark.parametrize("form", [0, 1], ids=["one_launch", "two_launch"])
def test_wait_that_gives_up_poisons_either_form(form):
    """A wait limit of 0 set from the host makes every bounded wait give up
    at once; in either form every kernel still exits and every output and
    final-state element is NaN."""
    d = inputs(2, 3, 300, False, seed=1300)
    prev = fb.falcon_set_wait_limit(0)
    try:
        o, S_T = run(d, form)
    finally:
        fb.falcon_set_wait_limit(prev)
    assert torch.isnan(o.float()).all() and torch.isnan(S_T).all()
