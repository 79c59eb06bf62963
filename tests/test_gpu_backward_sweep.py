"""A seeded random sweep of the Falcon-1 backward (falcon_bwd_chunked through
the C ABI) against the fp64 adjoint oracle.

Each case draws an I/O dtype, a batch, a length of 1..399 tokens (one
token, partial chunks, ragged tails), eps (including 0), the clamp epsilon,
a feature scale, beta scaled into (1, 2) or not and lam scaled up or not, a
carried state and previous key or a fresh start, and a final-state
cotangent or none.  Small features with beta in (1, 2) make the decay clamp
bind on most tokens ("Fast Weight Attention for Continual Learning",
Section 4.3, decay positivity) next to unclamped tokens whose decay sits
just above eps_gamma: the regime where the log-decay gradient of a row,
divided by that row's small decay, and the clamped decay itself must keep
float32 accuracy relative to the decay.  Every gradient tensor must meet
the backward's bar, 1e-5 relative L2."""

import numpy as np
import pytest
import torch

from delta_rule_recurrence_amd import inputs as I

from gpu_utils import rel_l2
from test_gpu_backward import BWD_TOL, NAMES, gpu_grads, oracle_grads

pytestmark = pytest.mark.gpu

N_CASES = 150


def draw(rng):
    io = str(rng.choice(["bf16", "f32"]))
    B, H, T = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 400))
    eps = float(rng.choice([1e-6, 0.0]))
    eps_gamma = float(rng.choice([1e-6, 1e-3]))
    fs = float(rng.choice([1.0 / 8, 0.02, 0.5]))
    seed = int(rng.integers(1 << 30))
    d = I.make_inputs(B, H, T, 64, 64, seed=seed, io_dtype=io, feature_scale=fs)
    if rng.random() < 0.4:
        d["beta"] = d["beta"] * 1.95
    if rng.random() < 0.3:
        d["lam"] = d["lam"] * 20.0
    cot = I.make_cotangents(B, H, T, 64, seed=seed + 1, io_dtype=io, with_state=bool(rng.random() < 0.5))
    S0 = torch.from_numpy((0.1 * rng.standard_normal((B, H, 64, 64))).astype(np.float32)) if rng.random() < 0.5 else None
    kp = None
    if rng.random() < 0.5:
        kp = torch.from_numpy((fs * rng.standard_normal((B, H, 64))).astype(np.float32)).to(I.TORCH_DTYPE[io])
    return dict(io=io, d=d, cot=cot, S0=S0, k_prev=kp, eps=eps, eps_gamma=eps_gamma,
                what=f"{io} B={B} H={H} T={T} eps={eps} eps_gamma={eps_gamma} fs={fs} "
                     f"beta_max={float(d['beta'].max()):.2f} S0={S0 is not None} k_prev={kp is not None} "
                     f"dS_T={cot['dS_T'] is not None}")


def test_backward_random_sweep_against_oracle():
    rng = np.random.default_rng(20261203)
    for i in range(N_CASES):
        c = draw(rng)
        kw = dict(S0=c["S0"], k_prev=c["k_prev"], eps=c["eps"], eps_gamma=c["eps_gamma"])
        ref = oracle_grads(c["d"], c["cot"], **kw)
        got = gpu_grads(c["d"], c["cot"], **kw)
        errs = {}
        for n in NAMES:
            if ref[n] is None:
                assert got[n] is None, f"case {i} ({c['what']}): {n} should be absent"
                continue
            assert np.all(np.isfinite(got[n])), f"case {i} ({c['what']}): non-finite {n}"
            errs[n] = rel_l2(got[n], ref[n])
        bad = {n: e for n, e in errs.items() if e > BWD_TOL}
        assert not bad, f"case {i} ({c['what']}): " + ", ".join(f"{n}={e:.2e}" for n, e in bad.items())




def test_backward_decay_just_above_the_clamp():
    """A row whose decay gamma = 1 - eta lam sits just above eps_gamma (beta in
    (1, 2) with small keys, "Fast Weight Attention for Continual Learning",
    Section 3.1 and Section 4.3): on these seeded inputs (float32 I/O, keys
    scaled to 0.02, beta scaled by 1.95, a carried state and previous key)
    sequence 3 has gamma = 5.8e-6 at token 8, the difference of two nearly
    equal terms.  Formed in float arithmetic, gamma kept about two digits
    there, and the gradient of beta, which takes the log decay's gradient
    divided by gamma, missed the bar (5.1e-5 relative L2)."""
    B, H, T, seed = 2, 2, 208, 935896980
    d = I.make_inputs(B, H, T, 64, 64, seed=seed, io_dtype="f32", feature_scale=0.02)
    d["beta"] = d["beta"] * 1.95
    cot = I.make_cotangents(B, H, T, 64, seed=seed + 1, io_dtype="f32", with_state=False)
    rng = np.random.default_rng(seed + 2)
    S0 = torch.from_numpy((0.1 * rng.standard_normal((B, H, 64, 64))).astype(np.float32))
    kp = torch.from_numpy((0.02 * rng.standard_normal((B, H, 64))).astype(np.float32))
    kw = dict(S0=S0, k_prev=kp, eps=1e-6, eps_gamma=1e-6)
    ref = oracle_grads(d, cot, **kw)
    got = gpu_grads(d, cot, **kw)
    for n in NAMES:
        if ref[n] is None:
            continue
        e = rel_l2(got[n], ref[n])
        assert e <= BWD_TOL, f"{n}: rel L2 {e:.2e}"
