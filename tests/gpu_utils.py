"""Shared helpers of the GPU parity tests: seeded inputs, oracle runs and the
relative-L2 metric.  Expected values always come from the CPU oracle."""

import numpy as np
import torch

from delta_rule_recurrence_amd import inputs as I
from oracle import falcon_oracle as orc

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def to_dev(d):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def oracle_forward(variant, d, *, eps=1e-6, eps_gamma=1e-6, S0=None, k_prev=None):
    f = I.as_f64
    return orc.falcon_forward(variant, f(d["phi_k"]), f(d["phi_q"]), f(d["v"]), f(d["beta"]),
                              f(d["lam"]), eps=eps, eps_gamma=eps_gamma,
                              S0=None if S0 is None else f(S0),
                              k_prev=None if k_prev is None else f(k_prev))


def worst_sequence(got, ref):
    """Largest relative L2 over the (b, h) sequences (leading two axes)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.ndim < 3:
        return rel_l2(got, ref)
    B, H = got.shape[:2]
    return max(rel_l2(got[b, h], ref[b, h]) for b in range(B) for h in range(H))


def check(o, S_T, O_ref, S_ref, tol, what=""):
    """The stated tolerance on the whole output and final state and on every
    sequence's output and final state."""
    got_o = o.float().cpu().numpy()
    got_s = S_T.cpu().numpy()
    assert np.all(np.isfinite(got_o)), f"{what}: non-finite output"
    assert np.all(np.isfinite(got_s)), f"{what}: non-finite final state"
    eo, es = rel_l2(got_o, O_ref), rel_l2(got_s, S_ref)
    wo, ws = worst_sequence(got_o, O_ref), worst_sequence(got_s, S_ref)
    assert max(eo, es, wo, ws) <= tol, (f"{what}: rel L2 o={eo:.3e} S_T={es:.3e}, worst sequence "
                                        f"o={wo:.3e} S_T={ws:.3e}, tol={tol:.0e}")
    return eo, es
