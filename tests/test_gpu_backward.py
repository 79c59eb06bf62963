"""GPU parity of the Falcon-1 backward (falcon_bwd_chunked through the C ABI)
against the fp64 adjoint oracle on identical seeded inputs.

Tolerance: relative L2 per gradient tensor <= 1e-5 for both I/O dtypes.  The
backward computes in float32 throughout (bf16 I/O only rounds the inputs,
and the oracle sees the same rounded values), so both dtypes carry the same
float32 rounding error: unit roundoff 6e-8 amplified by the 32-token
triangular solves and the state chain over T (a few times 1e-7 at T = 2048);
1e-5 leaves a factor of 20 above that and is ten times tighter than the
forward's float32 bar."""

import numpy as np
import pytest
import torch

from delta_rule_recurrence_amd import falcon as fb
from delta_rule_recurrence_amd import inputs as I
from oracle import falcon_backward as ob

from gpu_utils import rel_l2, to_dev

pytestmark = pytest.mark.gpu

BWD_TOL = 1e-5
NAMES = ("dphi_k", "dphi_q", "dv", "dbeta", "dlam", "dS0", "dk_prev")


def oracle_grads(d, cot, *, S0=None, k_prev=None, eps=1e-6, eps_gamma=1e-6):
    f = I.as_f64
    return ob.falcon1_backward(f(d["phi_k"]), f(d["phi_q"]), f(d["v"]), f(d["beta"]), f(d["lam"]),
                               f(cot["dO"]), eps=eps, eps_gamma=eps_gamma,
                               S0=None if S0 is None else f(S0),
                               k_prev=None if k_prev is None else f(k_prev),
                               dS_T=None if cot["dS_T"] is None else f(cot["dS_T"]))


def gpu_grads(d, cot, *, S0=None, k_prev=None, eps=1e-6, eps_gamma=1e-6):
    dd, cc = to_dev(d), to_dev(cot)
    g = fb.falcon_bwd_chunked(dd["phi_k"], dd["phi_q"], dd["v"], dd["beta"], dd["lam"], cc["dO"],
                              S0=None if S0 is None else S0.cuda(),
                              k_prev=None if k_prev is None else k_prev.cuda(),
                              dS_T=cc["dS_T"], eps=eps, eps_gamma=eps_gamma)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in g.items()}


def compare(got, ref, what, tol=BWD_TOL, names=NAMES):
    errs = {}
    for n in names:
        if ref[n] is None:
            assert got[n] is None, f"{what}: {n} should be absent"
            continue
        assert np.all(np.isfinite(got[n])), f"{what}: non-finite {n}"
        errs[n] = rel_l2(got[n], ref[n])
    bad = {n: e for n, e in errs.items() if e > tol}
    assert not bad, f"{what}: rel L2 above {tol:.0e}: " + ", ".join(f"{n}={e:.3e}" for n, e in bad.items())
    return errs


# (io, B, H, T): one chunk, a single token, several chunks with a ragged tail
SMALL = [
    ("f32", 1, 1, 32),
    ("f32", 1, 1, 1),
    ("f32", 2, 3, 100),
    ("f32", 1, 2, 64),
    ("bf16", 2, 2, 97),
    ("bf16", 1, 3, 160),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_backward_small(case):
    io, B, H, T = case
    d = I.make_inputs(B, H, T, 64, 64, seed=300 + T, io_dtype=io)
    cot = I.make_cotangents(B, H, T, 64, seed=300 + T, io_dtype=io)
    ref = oracle_grads(d, cot)
    got = gpu_grads(d, cot)
    errs = compare(got, ref, f"backward {case}")
    # the last key is read by no token
    assert np.all(got["dphi_k"][..., T - 1, :] == 0.0)
    print(case, {k: f"{v:.2e}" for k, v in errs.items()})


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_backward_carried_state(io):
    """Carried state S0, previous key and a loss on the final state."""
    B, H, T = 2, 3, 130
    d = I.make_inputs(B, H, T, 64, 64, seed=41, io_dtype=io)
    cot = I.make_cotangents(B, H, T, 64, seed=41, io_dtype=io, with_state=True)
    S0 = I.random_state((B, H, 64, 64), seed=42)
    k_prev = I.make_inputs(B, H, 1, 64, 64, seed=43, io_dtype=io)["phi_k"][:, :, 0].contiguous()
    ref = oracle_grads(d, cot, S0=S0, k_prev=k_prev)
    got = gpu_grads(d, cot, S0=S0, k_prev=k_prev)
    errs = compare(got, ref, f"carried {io}")
    print(io, {k: f"{v:.2e}" for k, v in errs.items()})


def test_backward_clamp_active():
    """Tokens where the decay clamp binds (eta lam > 1 - eps_gamma): gamma is
    constant there and passes no gradient to eta or lam."""
    B, H, T = 1, 2, 96
    d = I.make_inputs(B, H, T, 64, 64, seed=51, io_dtype="f32")
    d["beta"][..., ::3] = 1.9
    d["lam"][..., ::3] = 10.0
    cot = I.make_cotangents(B, H, T, 64, seed=51, io_dtype="f32", with_state=True)
    ref = oracle_grads(d, cot, eps_gamma=1e-3)
    got = gpu_grads(d, cot, eps_gamma=1e-3)
    compare(got, ref, "clamp")


def test_backward_no_tokens():
    """T = 0: dS0 = dS_T and the previous key reaches nothing."""
    B, H = 2, 2
    dS_T = I.random_state((B, H, 64, 64), seed=61).cuda()
    z = torch.zeros((B, H, 0, 64), dtype=torch.float32, device="cuda")
    s = torch.zeros((B, H, 0), dtype=torch.float32, device="cuda")
    kp = torch.ones((B, H, 64), dtype=torch.float32, device="cuda")
    dkp = torch.full((B, H, 64), 7.0, dtype=torch.float32, device="cuda")
    g = fb.falcon_bwd_chunked(z, z, z, s, s, z, k_prev=kp, dS_T=dS_T, grads={"dk_prev": dkp})
    torch.cuda.synchronize()
    assert torch.equal(g["dS0"], dS_T)
    assert torch.count_nonzero(g["dk_prev"]).item() == 0
    g = fb.falcon_bwd_chunked(z, z, z, s, s, z)
    torch.cuda.synchronize()
    assert torch.count_nonzero(g["dS0"]).item() == 0


def test_backward_repeatable():
    """No atomics: two calls give bitwise identical gradients."""
    B, H, T = 2, 2, 200
    d = I.make_inputs(B, H, T, 64, 64, seed=71, io_dtype="bf16")
    cot = I.make_cotangents(B, H, T, 64, seed=71, io_dtype="bf16", with_state=True)
    a = gpu_grads(d, cot)
    b = gpu_grads(d, cot)
    for n in NAMES:
        if a[n] is not None:
            assert np.array_equal(a[n], b[n]), n


def test_backward_full_workload_sampled():
    """The 8 x 12 x 2048, d = 64, bf16 training shape in one call (as the
    benchmark launches it); the oracle checks a seeded sample of (b, h)
    sequences (sequences are independent)."""
    w = I.WORKLOADS["f1_backward_8x12x2048_d64"]
    d = I.workload_inputs(w)
    cot = I.make_cotangents(w.B, w.H, w.T, w.dv, seed=w.seed, io_dtype=w.io_dtype, with_state=True)
    got = gpu_grads(d, cot, eps=w.eps, eps_gamma=w.eps_gamma)
    rng = np.random.default_rng(5)
    pairs = [(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(3)]
    for b, h in pairs:
        sub = {k: v[b:b + 1, h:h + 1] for k, v in d.items()}
        csub = {"dO": cot["dO"][b:b + 1, h:h + 1], "dS_T": cot["dS_T"][b:b + 1, h:h + 1]}
        ref = oracle_grads(sub, csub, eps=w.eps, eps_gamma=w.eps_gamma)
        gsub = {k: (None if v is None else v[b:b + 1, h:h + 1]) for k, v in got.items()}
        errs = compare(gsub, ref, f"full workload (b={b}, h={h})")
        print((b, h), {k: f"{v:.2e}" for k, v in errs.items()})


def test_backward_long_single_sequence():
    """One sequence of 4130 tokens: 130 chunks (the chain ring's last group is
    partial), a single workgroup per chain, the persistent kernels' grids
    larger than the work."""
    B, H, T = 1, 1, 4130
    d = I.make_inputs(B, H, T, 64, 64, seed=81, io_dtype="bf16")
    cot = I.make_cotangents(B, H, T, 64, seed=81, io_dtype="bf16", with_state=True)
    S0 = I.random_state((B, H, 64, 64), seed=82)
    ref = oracle_grads(d, cot, S0=S0)
    got = gpu_grads(d, cot, S0=S0)
    errs = compare(got, ref, "long single sequence")
    print({k: f"{v:.2e}" for k, v in errs.items()})
