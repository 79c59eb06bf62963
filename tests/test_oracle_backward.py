"""Pins of the Falcon-1 backward oracle.

The adjoint recurrence in oracle/falcon_backward.py is checked against
central finite differences of the forward oracle (the differences use the
forward only, so a wrong sign, a dropped term or a transposed operand in the
adjoint fails here).  Cases: fresh start, a carried state with a previous
key, and the positive-decay clamp active on some tokens.
"""

import numpy as np
import pytest

from oracle import falcon_backward as ob


def _inputs(seed, B=1, H=2, T=7, dk=3, dv=2, clamp_case=False):
    rng = np.random.default_rng(seed)
    d = dict(
        phi_k=rng.standard_normal((B, H, T, dk)) * 0.7,
        phi_q=rng.standard_normal((B, H, T, dk)) * 0.7,
        v=rng.standard_normal((B, H, T, dv)),
        beta=1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T)))),
        lam=np.log1p(np.exp(rng.standard_normal((B, H, T)) - 1.0)),
    )
    if clamp_case:
        # beta near 1.9 and a large ridge drive eta*lam past 1 - eps_gamma on some tokens
        d["beta"] = 1.9 * np.ones((B, H, T))
        d["lam"][..., ::2] = 10.0
    dO = rng.standard_normal((B, H, T, dv))
    return d, dO, rng


def _fd(fun, arr, h=1e-6):
    g = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = arr[i]
        arr[i] = old + h
        fp = fun()
        arr[i] = old - h
        fm = fun()
        arr[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("case", ["fresh", "carried", "clamp"])
def test_backward_matches_finite_differences(case):
    d, dO, rng = _inputs(11 + ["fresh", "carried", "clamp"].index(case), clamp_case=(case == "clamp"))
    B, H, T, dk = d["phi_k"].shape
    dv = d["v"].shape[-1]
    kw = dict(eps=1e-6, eps_gamma=1e-3 if case == "clamp" else 1e-6)
    S0 = k_prev = dS_T = None
    if case != "fresh":
        S0 = rng.standard_normal((B, H, dk, dv)) * 0.3
        dS_T = rng.standard_normal((B, H, dk, dv))
    if case == "carried":
        k_prev = rng.standard_normal((B, H, dk)) * 0.7
    g = ob.falcon1_backward(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], dO, S0=S0, k_prev=k_prev,
                            dS_T=dS_T, **kw)
    if case == "clamp":
        # the clamp must actually bind somewhere in this case
        from oracle.falcon_oracle import step_size
        X = np.concatenate([np.zeros((B, H, 1, dk)), d["phi_k"][..., :-1, :]], axis=-2)
        eta = np.stack([step_size(X[..., t, :], d["beta"][..., t], d["lam"][..., t], 1e-6, sentinel=(t == 0))
                        for t in range(T)], axis=-1)
        assert np.any(eta * d["lam"] > 1 - kw["eps_gamma"])

    def L():
        return ob.loss(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], dO, S0=S0, k_prev=k_prev,
                       dS_T=dS_T, **kw)

    checks = [("dphi_k", d["phi_k"]), ("dphi_q", d["phi_q"]), ("dv", d["v"]), ("dbeta", d["beta"]),
              ("dlam", d["lam"])]
    if S0 is not None:
        checks.append(("dS0", S0))
    if k_prev is not None:
        checks.append(("dk_prev", k_prev))
    for name, arr in checks:
        fd = _fd(L, arr)
        np.testing.assert_allclose(g[name], fd, rtol=1e-6, atol=1e-7, err_msg=name)


def test_last_key_and_first_gates_have_no_gradient_on_a_fresh_start():
    """phi(k_T) is never read, and beta_1, lam_1 are ignored at a fresh start
    (eta_1 := 0, gamma_1 = 1)."""
    d, dO, _ = _inputs(5)
    g = ob.falcon1_backward(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], dO, eps=1e-6)
    assert np.all(g["dphi_k"][..., -1, :] == 0.0)
    assert np.all(g["dbeta"][..., 0] == 0.0) and np.all(g["dlam"][..., 0] == 0.0)
