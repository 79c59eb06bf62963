"""Plain fp64 CPU oracle for the gradients of the Falcon-1 forward.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this module; the
product path never imports, calls or links anything here.

The forward is the sequential read-after-write recurrence of
``falcon_oracle.falcon_forward`` for Falcon-1 (paper §4 naming and formula
summary; Eq. 3.4 step size; §4.3 "Decay positivity" clamp).  The pages give
the forward only; training "differentiates through the update" (§3), so the
backward here is the reverse-mode (adjoint) form of that recurrence, derived
by hand one token at a time:

  forward, token t:   x = phi(k_{t-1}),  E = ||x||^2,  eta = beta / (E + lam + eps),
                      gamma = 1 - min(eta lam, 1 - eps_gamma),
                      r = v - S_{t-1}^T x,  S_t = gamma S_{t-1} + eta x r^T,  o = S_t^T q
  backward, token t (L = dL/dS_t, accumulated from the later tokens and dS_T):
      L += q do^T,                    dq = S_t do
      dgamma = <L, S_{t-1}>,          deta = x^T L r,            dv = eta L^T x
      dx = eta L r - eta S_{t-1} (L^T x)
      dL/dS_{t-1} = gamma L - eta x (x^T L)
      gamma: unless clamped, deta -= lam dgamma, dlam -= eta dgamma
      eta:   unless it is the fresh-start sentinel or 0/0, dbeta = deta / den,
             dlam -= deta eta / den, dx -= 2 (deta eta / den) x
      shift: dphi(k_{t-1}) += dx (dk_prev for t = 1 when a previous key was given)
  dS0 = dL/dS_0.

It is pinned against central finite differences of the forward oracle in
tests/test_oracle_backward.py (an independent check: the differences use the
forward only).
"""

from __future__ import annotations

import numpy as np

from .falcon_oracle import _f64, decay, falcon_forward, step_size


def falcon1_backward(phi_k, phi_q, v, beta, lam, dO, *, eps, eps_gamma=1e-6, S0=None, k_prev=None,
                     dS_T=None, clamp=True):
    """Gradients of L = <dO, O> + <dS_T, S_T> for the Falcon-1 forward.

    Shapes as in ``falcon_forward`` (leading batch axes, then [T, d]).
    Returns a dict with dphi_k, dphi_q, dv, dbeta, dlam, dS0 and dk_prev
    (None when no previous key was given), all float64.
    """
    K, Q, V = _f64(phi_k), _f64(phi_q), _f64(v)
    beta, lam, dO = _f64(beta), _f64(lam), _f64(dO)
    lead = K.shape[:-2]
    T, dk = K.shape[-2:]
    dv_ = V.shape[-1]
    fresh = k_prev is None
    kp = np.zeros(lead + (dk,)) if fresh else _f64(k_prev)
    S = np.zeros(lead + (dk, dv_)) if S0 is None else _f64(S0).copy()

    # forward sweep, keeping what the backward needs
    xs, etas, gammas, clamped, dens, live_eta, rs, S_prev, S_post = [], [], [], [], [], [], [], [], []
    for t in range(T):
        x = kp if t == 0 else K[..., t - 1, :]
        sentinel = (t == 0 and fresh)
        eta = step_size(x, beta[..., t], lam[..., t], eps, sentinel=sentinel)
        alpha = eta * lam[..., t]
        gamma = decay(eta, lam[..., t], eps_gamma, clamp=clamp)
        den = np.sum(x * x, axis=-1) + lam[..., t] + eps
        r = V[..., t, :] - np.einsum("...kv,...k->...v", S, x)
        S_prev.append(S)
        S = gamma[..., None, None] * S + (eta[..., None, None] * x[..., :, None]) * r[..., None, :]
        S_post.append(S)
        xs.append(x)
        etas.append(eta)
        gammas.append(gamma)
        clamped.append((alpha > 1.0 - eps_gamma) if clamp else np.zeros_like(alpha, dtype=bool))
        dens.append(den)
        live_eta.append(np.logical_and(~np.asarray(sentinel), den != 0.0))
        rs.append(r)

    dK = np.zeros_like(K)
    dQ = np.zeros_like(Q)
    dV = np.zeros_like(V)
    dbeta = np.zeros_like(beta)
    dlam = np.zeros_like(lam)
    dkp = np.zeros(lead + (dk,))
    L = np.zeros(lead + (dk, dv_)) if dS_T is None else _f64(dS_T).copy()
    for t in range(T - 1, -1, -1):
        x, eta, gamma, r, Sp = xs[t], etas[t], gammas[t], rs[t], S_prev[t]
        do = dO[..., t, :]
        # read o_t = S_t^T q_t
        dQ[..., t, :] = np.einsum("...kv,...v->...k", S_post[t], do)
        L = L + Q[..., t, :, None] * do[..., None, :]
        # write S_t = gamma S_{t-1} + eta x r^T, r = v - S_{t-1}^T x
        Lx = np.einsum("...kv,...k->...v", L, x)                 # L^T x
        dgamma = np.sum(L * Sp, axis=(-2, -1))
        deta = np.sum(Lx * r, axis=-1)
        dV[..., t, :] = eta[..., None] * Lx
        dx = eta[..., None] * np.einsum("...kv,...v->...k", L, r) \
            - eta[..., None] * np.einsum("...kv,...v->...k", Sp, Lx)
        L = gamma[..., None, None] * L - eta[..., None, None] * x[..., :, None] * Lx[..., None, :]
        # gamma = 1 - min(eta lam, 1 - eps_gamma)
        free = ~clamped[t]
        deta = deta - np.where(free, lam[..., t] * dgamma, 0.0)
        dlam[..., t] -= np.where(free, eta * dgamma, 0.0)
        # eta = beta / (||x||^2 + lam + eps)
        den = np.where(dens[t] == 0.0, 1.0, dens[t])
        on = live_eta[t]
        dbeta[..., t] = np.where(on, deta / den, 0.0)
        dden = np.where(on, -deta * eta / den, 0.0)
        dlam[..., t] += dden
        dx = dx + 2.0 * dden[..., None] * x
        # x_t = phi(k_{t-1})
        if t >= 1:
            dK[..., t - 1, :] += dx
        else:
            dkp = dx
    return {
        "dphi_k": dK, "dphi_q": dQ, "dv": dV, "dbeta": dbeta, "dlam": dlam, "dS0": L,
        "dk_prev": None if fresh else dkp,
    }


def loss(phi_k, phi_q, v, beta, lam, dO, *, eps, eps_gamma=1e-6, S0=None, k_prev=None, dS_T=None,
         clamp=True):
    """L = <dO, O> + <dS_T, S_T> through the forward oracle (for finite differences)."""
    O, S_T = falcon_forward("falcon1", phi_k, phi_q, v, beta, lam, eps=eps, eps_gamma=eps_gamma,
                            S0=S0, k_prev=k_prev, clamp=clamp)
    out = float(np.sum(_f64(dO) * O))
    if dS_T is not None:
        out += float(np.sum(_f64(dS_T) * S_T))
    return out
