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


def check(o, S_T, O_ref, S_ref, tol, what=""):
    eo = rel_l2(o.float().cpu().numpy(), O_ref)
    es = rel_l2(S_T.cpu().numpy(), S_ref)
    assert np.all(np.isfinite(o.float().cpu().numpy())), f"{what}: non-finite output"
    assert eo <= tol and es <= tol, f"{what}: rel L2 o={eo:.3e} S_T={es:.3e} tol={tol:.0e}"
    return eo, es
