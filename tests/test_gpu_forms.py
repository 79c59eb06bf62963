"""The two forms of the Falcon-1 bf16 chunked fast path -- one launch (chunk
workgroups and per-sequence chains side by side, handing chunk matrices over
through flags) and two launches (all chunk matrices, then the chains) --
compute the same chunk form ("Fast Weight Attention for Continual Learning",
Section 4.2, chunk-parallel implementation; Eq. 3.3 per chunk) with the same
roundings.  Each form is held to the oracle at the bf16 tolerance (whole
tensors and every sequence), repeats its results bit for bit, and the two
agree bit for bit, on shapes with one chunk, odd and even chunk counts with
ragged tails, a carried state and key, a sequence count that is not a
multiple of the eight XCDs, batches at and past the 256 sequences up to which
the default runs in one launch, long sequences (256 chunks, and a ragged 6001
tokens) and the full workload shape.  The bit
agreement pins the hand-over of the one-launch form against the other,
independently scheduled form."""

import numpy as np
import pytest
import torch

from delta_rule_recurrence_amd import falcon as fb
from delta_rule_recurrence_amd import inputs as I

from gpu_utils import TOL, check, oracle_forward, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    "one_chunk": (1, 1, 64, False),
    "three_chunks_ragged_carry": (1, 3, 150, True),
    "four_chunks_ragged_carry": (1, 3, 200, True),
    "18_sequences": (2, 9, 1000, False),
    "31_chunks_carry": (2, 5, 1950, True),
    "256_sequences": (16, 16, 100, False),
    "264_sequences": (8, 33, 128, True),
    "workload_carry": (8, 12, 2048, True),
    "long_16384_carry": (1, 2, 16384, True),
    "long_ragged": (2, 3, 6001, False),
}
FORMS = {"one_launch": fb.F1_ONE_LAUNCH, "two_launch": fb.F1_TWO_LAUNCH}


def host_inputs(B, H, T, carry, seed):
    x = I.make_inputs(B, H, T, 64, 64, seed=seed, io_dtype="bf16")
    if carry:
        g = np.random.default_rng([seed, 3])
        x["S0"] = torch.from_numpy((0.1 * g.standard_normal((B, H, 64, 64))).astype(np.float32))
        x["k_prev"] = torch.from_numpy(np.abs(g.standard_normal((B, H, 64))).astype(np.float32)).to(torch.bfloat16)
    return x


_ORACLE = {}


def case(name):
    """Host inputs and the oracle's output and final state, once per case."""
    if name not in _ORACLE:
        B, H, T, carry = CASES[name]
        x = host_inputs(B, H, T, carry, seed=1200 + len(name))
        _ORACLE[name] = (x, oracle_forward("falcon1", x, S0=x.get("S0"), k_prev=x.get("k_prev")))
    return _ORACLE[name]


def run(d, form):
    prev = fb.falcon_set_f1_launch_form(form)
    try:
        o, S_T = fb.falcon_fwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], C=64,
                                       S0=d.get("S0"), k_prev=d.get("k_prev"))
        torch.cuda.synchronize()
    finally:
        fb.falcon_set_f1_launch_form(prev)
    return o.cpu(), S_T.cpu()


def same_bits(a, b):
    view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(view), b.view(view))


@pytest.mark.parametrize("name", sorted(CASES))
def test_launch_forms(name):
    B, H, T, carry = CASES[name]
    print(f"[forms] {name}: B={B} H={H} T={T} carry={carry}", flush=True)
    x, (O_ref, S_ref) = case(name)
    d = to_dev(x)
    got = {}
    for form, code in sorted(FORMS.items()):
        o, S_T = run(d, code)
        eo, es = check(o, S_T, O_ref, S_ref, TOL["bf16"], f"{name} {form}")
        print(f"[forms] {name} {form}: rel L2 o={eo:.3e} S_T={es:.3e}", flush=True)
        o2, s2 = run(d, code)
        assert same_bits(o, o2) and same_bits(S_T, s2), f"{form}: two runs differ"
        got[form] = (o, S_T)
    (o1, s1), (o2, s2) = got["one_launch"], got["two_launch"]
    assert same_bits(o1, o2), "outputs differ between the launch forms"
    assert same_bits(s1, s2), "final states differ between the launch forms"


@pytest.mark.parametrize("form", [0, 1], ids=["one_launch", "two_launch"])
def test_wait_that_gives_up_poisons_either_form(form):
    """A wait limit of 0 set from the host makes every bounded wait give up
    at once; in either form every kernel still exits and every output and
    final-state element is NaN."""
    d = to_dev(host_inputs(2, 3, 300, False, seed=1300))
    prev = fb.falcon_set_wait_limit(0)
    try:
        o, S_T = run(d, form)
    finally:
        fb.falcon_set_wait_limit(prev)
    assert torch.isnan(o.float()).all() and torch.isnan(S_T).all()
