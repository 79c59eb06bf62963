"""Plain fp64 CPU oracle for the Falcon fast-weight recurrences.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The
product path (the HIP library and its Python binding) never imports, calls
or links anything here, and this module imports nothing from the product.

What it computes is the sequential recurrence exactly as the paper states it,
one token at a time, in float64, vectorised only over the independent
(batch, head) axes.  Citations refer to *Fast Weight Attention for Continual
Learning* (arXiv 2608.27763) as rendered on the hyper.ai page (English body):
section / equation numbers are the paper's.  "[juho]" is the juhoplayground
post on the same paper (its complexity table), "[rainbus]" the
paper.rainbus.top review.

Readings taken where the pages leave a step open (each also listed in the
design notes):
  * t = 1 sentinel: x_1 := 0 and eta_1 := 0 (alpha_1 = 0, gamma_1 = 1) on a
    fresh start (§3 "Indexing and causality conventions"; §4 naming summary).
    With an explicit previous key ``k_prev`` the first pair is real:
    x_1 = k_prev and eta_1 is computed normally (continuation reading).
  * eta_t := 0 when ||x_t||^2 + lam_t + eps == 0 (§3.1, after Eq. 3.4).
  * The positive-decay clamp alpha <- min(eta*lam, 1 - eps_gamma) (§4.3
    "Decay positivity") is applied in every form unless ``clamp=False``;
    the write gain stays eta (surrogate ridge alpha/eta).
  * beta_t, lam_t belong to step t like v_t; only the key is shifted; the
    read uses the unshifted query phi(q_t) (§4 naming summary).
  * Falcon-2 / 2A: beta is per column, lam is one scalar per token shared by
    the columns, and the clamp acts per column (§4.2 "Per-column NLMS step
    sizes", Eq. 4.7 and the clamp paragraph of §4.3).

Array conventions: leading axes are arbitrary batch axes (typically B, H);
keys/queries ``[..., T, dk]``, values ``[..., T, dv]``, beta ``[..., T]``
(``[..., T, dv]`` for Falcon-2 / 2A), lam ``[..., T]``, states
``[..., dk, dv]``.  All inputs are converted to float64.
"""

from __future__ import annotations

import numpy as np

VARIANTS = ("falcon1", "falcon1a", "falcon2", "falcon2a")
_PER_COLUMN = {"falcon2", "falcon2a"}
_REGRESSION = {"falcon1", "falcon2"}


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def step_size(x, beta, lam, eps, *, sentinel):
    """NLMS step size, Eq. (3.4) (and §4.3 "Falcon-1A/Falcon-2A step sizes"
    for the inner-product variants, which use the same E_t = ||x_t||^2).

    ``x``: [..., dk]; ``beta``: [...] or [..., dv]; ``lam``: [...].
    ``sentinel``: True where the step is the fresh-start boundary t = 1, whose
    eta is forced to 0.  Returns eta with beta's shape.
    """
    energy = np.sum(x * x, axis=-1)                    # ||x_t||^2
    denom = energy + lam + eps                         # [...]
    sentinel = np.broadcast_to(np.asarray(sentinel, dtype=bool), denom.shape)
    if beta.ndim == denom.ndim + 1:                    # per-column gains
        denom = denom[..., None]
        sentinel = sentinel[..., None]
    safe = np.where(denom == 0.0, 1.0, denom)
    eta = np.where(denom == 0.0, 0.0, beta / safe)
    return np.where(sentinel, 0.0, eta)


def decay(eta, lam, eps_gamma, *, clamp=True):
    """alpha = eta*lam, clamped to 1 - eps_gamma, gamma = 1 - alpha
    (§4.3 "Decay positivity"; the same derived variables appear in §4.5)."""
    if eta.ndim == lam.ndim + 1:
        lam = lam[..., None]
    alpha = eta * lam
    if clamp:
        alpha = np.minimum(alpha, 1.0 - eps_gamma)
    return 1.0 - alpha


def falcon_forward(variant, phi_k, phi_q, v, beta, lam, *, eps, eps_gamma=1e-6,
                   S0=None, k_prev=None, clamp=True, return_states=False):
    """Sequential read-after-write recurrence, one token at a time.

    For each (batch, head) and t = 1..T (0-based index t-1 below):
      x_t = phi(k_{t-1})   (x_1 = k_prev, or 0 on a fresh start)
      eta_t from Eq. (3.4); gamma_t = 1 - min(eta_t lam_t, 1 - eps_gamma)
      Falcon-1  (§4 summary; Eq. 3.3):   r = v_t - S^T x;  S = gamma S + eta x r^T
      Falcon-1A (§4 summary; §4.3):     S = gamma S + eta x v_t^T
      Falcon-2  (§4 summary; §4.2):     S = S Diag(gamma) + x (eta ⊙ r)^T
      Falcon-2A (§4 summary; Eq. 4.7):   S = S Diag(gamma) + x (eta ⊙ v_t)^T
      o_t = S_t^T phi(q_t)                (read after write, §4 summary)
    The residual r uses the state before the write (Eq. 3.3), and the first
    step follows the t = 1 sentinel of §3.

    Returns ``(O, S_T)`` (and the list of states S_1..S_T when
    ``return_states``), all float64.
    """
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    K, Q, V = _f64(phi_k), _f64(phi_q), _f64(v)
    beta, lam = _f64(beta), _f64(lam)
    lead = K.shape[:-2]
    T, dk = K.shape[-2:]
    dv = V.shape[-1]
    S = np.zeros(lead + (dk, dv)) if S0 is None else _f64(S0).copy()
    fresh = k_prev is None
    kp = np.zeros(lead + (dk,)) if fresh else _f64(k_prev)
    O = np.zeros(lead + (T, dv))
    states = []
    for t in range(T):
        x = kp if t == 0 else K[..., t - 1, :]
        b = beta[..., t, :] if variant in _PER_COLUMN else beta[..., t]
        lt = lam[..., t]
        eta = step_size(x, b, lt, eps, sentinel=(t == 0 and fresh))
        gamma = decay(eta, lt, eps_gamma, clamp=clamp)
        vt = V[..., t, :]
        if variant in _REGRESSION:
            target = vt - np.einsum("...kv,...k->...v", S, x)   # r_t
        else:
            target = vt                                          # y_t
        if variant in _PER_COLUMN:
            S = S * gamma[..., None, :] + x[..., :, None] * (eta[..., None, :] * target[..., None, :])
        else:
            S = gamma[..., None, None] * S + (eta[..., None, None] * x[..., :, None]) * target[..., None, :]
        O[..., t, :] = np.einsum("...kv,...k->...v", S, Q[..., t, :])
        if return_states:
            states.append(S.copy())
    if return_states:
        return O, S, states
    return O, S


def falcon_decode_step(variant, S, phi_k_prev, phi_q, v, beta, lam, *, eps,
                       eps_gamma=1e-6, is_first=None, clamp=True):
    """One read-after-write step from a carried state (the recurrent form at
    inference, [juho] complexity table "O(1) state").

    ``S``: [..., dk, dv]; ``phi_k_prev``: the previous step's key feature
    [..., dk]; ``phi_q``: [..., dk]; ``v``: [..., dv]; ``beta``: [...] or
    [..., dv]; ``lam``: [...]; ``is_first``: boolean [...] (broadcast) marking
    sequences whose current token is t = 1 (sentinel: eta := 0).
    Returns ``(o, S_new)``.
    """
    S = _f64(S)
    x = _f64(phi_k_prev)
    b, lt = _f64(beta), _f64(lam)
    sentinel = np.zeros(lt.shape, dtype=bool) if is_first is None else np.broadcast_to(
        np.asarray(is_first, dtype=bool), lt.shape)
    eta = step_size(x, b, lt, eps, sentinel=sentinel)
    gamma = decay(eta, lt, eps_gamma, clamp=clamp)
    vt = _f64(v)
    if variant in _REGRESSION:
        target = vt - np.einsum("...kv,...k->...v", S, x)
    else:
        target = vt
    if variant in _PER_COLUMN:
        S_new = S * gamma[..., None, :] + x[..., :, None] * (eta[..., None, :] * target[..., None, :])
    else:
        S_new = gamma[..., None, None] * S + (eta[..., None, None] * x[..., :, None]) * target[..., None, :]
    o = np.einsum("...kv,...k->...v", S_new, _f64(phi_q))
    return o, S_new


# ---------------------------------------------------------------------------
# Masked-parallel (attention) forms, used only to cross-check the recurrence.
# ---------------------------------------------------------------------------

def _shifted_stream(K, k_prev):
    """X with rows x_t = phi(k_{t-1}), x_1 = k_prev or 0 (§2.2 shifted stream)."""
    X = np.zeros_like(K)
    X[..., 1:, :] = K[..., :-1, :]
    if k_prev is not None:
        X[..., 0, :] = _f64(k_prev)
    return X


def _gates(X, beta, lam, eps, eps_gamma, fresh, clamp):
    T = X.shape[-2]
    eta = np.stack([step_size(X[..., t, :], beta[..., t], lam[..., t], eps,
                              sentinel=(t == 0 and fresh)) for t in range(T)], axis=-1)
    gamma = decay(eta, lam, eps_gamma, clamp=clamp)
    return eta, gamma


def _carry_products(gamma):
    """P[t, j] = prod_{r=j+1}^{t} gamma_r for j <= t (1 on the diagonal), 0
    above; and delta_t = prod_{r<=t} gamma_r (§4.6 definitions)."""
    T = gamma.shape[-1]
    P = np.zeros(gamma.shape[:-1] + (T, T))
    for t in range(T):
        acc = np.ones(gamma.shape[:-1])
        for j in range(t, -1, -1):
            P[..., t, j] = acc
            acc = acc * gamma[..., j]
    delta = np.cumprod(gamma, axis=-1)
    return P, delta


def falcon1a_masked(phi_k, phi_q, v, beta, lam, *, eps, eps_gamma=1e-6, S0=None,
                    k_prev=None, clamp=True):
    """Masked-attention form of the scalar inner-product rule.

    §4.6 gives O = Diag(delta) Q S_0 + (Q X^T ⊙ M) V with the structured
    mask M_{t,j} = sum_{s=j}^{min(t, j+B-1)} (eta_s/B_s) prod_{r=s+1}^t gamma_r.  With window B = 1 the rule is Falcon-1A (end of §4.5) and
    the mask collapses to M_{t,j} = eta_j prod_{r=j+1}^t gamma_r.
    Returns ``(O, S_T)``.
    """
    K, Q, V = _f64(phi_k), _f64(phi_q), _f64(v)
    beta, lam = _f64(beta), _f64(lam)
    X = _shifted_stream(K, k_prev)
    eta, gamma = _gates(X, beta, lam, eps, eps_gamma, k_prev is None, clamp)
    P, delta = _carry_products(gamma)
    M = P * eta[..., None, :]
    dk, dv = K.shape[-1], V.shape[-1]
    S0 = np.zeros(K.shape[:-2] + (dk, dv)) if S0 is None else _f64(S0)
    QX = np.einsum("...tk,...jk->...tj", Q, X)
    O = delta[..., :, None] * np.einsum("...tk,...kv->...tv", Q, S0) + np.einsum("...tj,...jv->...tv", QX * M, V)
    S_T = delta[..., -1, None, None] * S0 + np.einsum("...j,...jk,...jv->...kv", M[..., -1, :], X, V)
    return O, S_T


def falcon1_masked(phi_k, phi_q, v, beta, lam, *, eps, eps_gamma=1e-6, S0=None,
                   k_prev=None, clamp=True):
    """Masked-parallel form of Falcon-1 over the whole sequence as one block,
    with a dense linear solve for the residual coupling.

    Derivation (from the Falcon-1 line of the §4 summary): write the scaled
    residual rho_t = eta_t r_t, so S_t = gamma_t S_{t-1} + x_t rho_t^T unrolls to
    S_t = delta_t S_0 + sum_{j<=t} P[t,j] x_j rho_j^T.  Substituting S_{t-1}
    into r_t = v_t - S_{t-1}^T x_t gives, for every t,
        rho_t + sum_{j<t} eta_t P[t-1,j] (x_t . x_j) rho_j
              = eta_t v_t - eta_t delta_{t-1} S_0^T x_t          (delta_0 = 1),
    a unit-lower-triangular system (I + L) R = Diag(eta) V - Diag(eta delta_{-1}) X S_0
    whose operator is the decayed strictly-lower Gram matrix; this is the
    "one multi-RHS TriSolve" the paper and [juho] attribute to Falcon-1's
    WY form.  The read is O = Diag(delta) Q S_0 + (Q X^T ⊙ P) R (read after
    write keeps the diagonal).  ``numpy.linalg.solve`` is used as a library
    primitive on the dense matrix.  Returns ``(O, S_T)``.
    """
    K, Q, V = _f64(phi_k), _f64(phi_q), _f64(v)
    beta, lam = _f64(beta), _f64(lam)
    X = _shifted_stream(K, k_prev)
    eta, gamma = _gates(X, beta, lam, eps, eps_gamma, k_prev is None, clamp)
    P, delta = _carry_products(gamma)
    T = K.shape[-2]
    dk, dv = K.shape[-1], V.shape[-1]
    S0 = np.zeros(K.shape[:-2] + (dk, dv)) if S0 is None else _f64(S0)
    delta_prev = np.concatenate([np.ones(delta.shape[:-1] + (1,)), delta[..., :-1]], axis=-1)
    G = np.einsum("...tk,...jk->...tj", X, X)
    Pprev = np.zeros_like(P)                            # P[t-1, j] for j < t
    Pprev[..., 1:, :] = P[..., :-1, :]
    L = np.tril(eta[..., :, None] * Pprev * G, k=-1)
    rhs = eta[..., :, None] * V - (eta * delta_prev)[..., :, None] * np.einsum("...tk,...kv->...tv", X, S0)
    R = np.linalg.solve(np.eye(T) + L, rhs)
    QX = np.einsum("...tk,...jk->...tj", Q, X)
    O = delta[..., :, None] * np.einsum("...tk,...kv->...tv", Q, S0) + np.einsum("...tj,...jv->...tv", QX * P, R)
    S_T = delta[..., -1, None, None] * S0 + np.einsum("...j,...jk,...jv->...kv", P[..., -1, :], X, R)
    return O, S_T


def ridge_loss(S, x, y, lam):
    """Instantaneous ridge objective l_t(S) = 1/2||S^T x - y||^2 + lam/2 ||S||_F^2
    (Eq. 3.1) and its gradient x (S^T x - y)^T + lam S (§3.1)."""
    S, x, y = _f64(S), _f64(x), _f64(y)
    e = S.T @ x - y
    loss = 0.5 * float(e @ e) + 0.5 * lam * float(np.sum(S * S))
    grad = np.outer(x, e) + lam * S
    return loss, grad
