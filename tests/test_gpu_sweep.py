"""A seeded random sweep of the forward entry points against the oracle.

Each case draws a variant (Falcon-1, 1A, 2, 2A), an I/O dtype, feature and
value widths and a chunk size (half of the bf16 cases take the MFMA fast
paths' dk = dv = C = 64), a batch, a length of 1..599 tokens (one token,
partial chunks and ragged tails), eps (including 0, so zero-energy rows take
the eta := 0 convention), the clamp epsilon, a feature scale (small features
drive the step size towards beta / lam), beta scaled into (1, 2) or not, lam
scaled up so that the decay clamp binds or not ("Fast Weight Attention for
Continual Learning", Section 3.1 after Eq. 3.4 and Section 4.3, decay
positivity), and a carried state and previous key or a fresh start.  Both
falcon_fwd_chunked and falcon_fwd_recurrent must meet the stated tolerance
(float32 1e-4, bf16 2e-2 relative L2) on the whole output and final state and
on every sequence."""

import numpy as np
import pytest
import torch

from delta_rule_recurrence_amd import falcon as fb
from delta_rule_recurrence_amd import inputs as I

from gpu_utils import TOL, check, oracle_forward, to_dev

pytestmark = pytest.mark.gpu

N_CASES = 120


def draw(rng):
    variant = str(rng.choice(["falcon1", "falcon1a", "falcon2", "falcon2a"]))
    io = str(rng.choice(["bf16", "f32"]))
    fast = io == "bf16" and rng.random() < 0.5
    dk = 64 if fast else int(rng.choice([16, 32, 64]))
    dv = 64 if fast else int(rng.choice([16, 32, 64]))
    C = 64 if fast else int(rng.choice([16, 32, 64]))
    B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    T = int(rng.integers(1, 600))
    eps = float(rng.choice([1e-6, 0.0]))
    eps_gamma = float(rng.choice([1e-6, 1e-3]))
    fs = float(rng.choice([1.0 / np.sqrt(dk), 0.02, 0.5]))
    x = I.make_inputs(B, H, T, dk, dv, seed=int(rng.integers(1 << 30)), io_dtype=io,
                      per_column_beta=variant in ("falcon2", "falcon2a"), feature_scale=fs)
    if rng.random() < 0.4:
        x["beta"] = x["beta"] * 1.95
    if rng.random() < 0.3:
        x["lam"] = x["lam"] * 20.0
    S0 = torch.from_numpy((0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32)) if rng.random() < 0.5 else None
    kp = None
    if rng.random() < 0.5:
        kp = torch.from_numpy((fs * rng.standard_normal((B, H, dk))).astype(np.float32)).to(I.TORCH_DTYPE[io])
    return dict(variant=variant, io=io, C=C, eps=eps, eps_gamma=eps_gamma, x=x, S0=S0, k_prev=kp,
                shape=(B, H, T, dk, dv))


def test_random_sweep_against_oracle():
    rng = np.random.default_rng(20261202)
    for i in range(N_CASES):
        c = draw(rng)
        B, H, T, dk, dv = c["shape"]
        what = (f"case {i}: {c['variant']} {c['io']} B={B} H={H} T={T} dk={dk} dv={dv} C={c['C']} "
                f"eps={c['eps']} eps_gamma={c['eps_gamma']} S0={c['S0'] is not None} k_prev={c['k_prev'] is not None}")
        O_ref, S_ref = oracle_forward(c["variant"], c["x"], eps=c["eps"], eps_gamma=c["eps_gamma"],
                                      S0=c["S0"], k_prev=c["k_prev"])
        d = to_dev(c["x"])
        kw = dict(variant=c["variant"], eps=c["eps"], eps_gamma=c["eps_gamma"],
                  S0=None if c["S0"] is None else c["S0"].cuda(),
                  k_prev=None if c["k_prev"] is None else c["k_prev"].cuda())
        o, S_T = fb.falcon_fwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], C=c["C"], **kw)
        check(o, S_T, O_ref, S_ref, TOL[c["io"]], what + " chunked")
        o, S_T = fb.falcon_fwd_recurrent(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], **kw)
        check(o, S_T, O_ref, S_ref, TOL[c["io"]], what + " recurrent")
