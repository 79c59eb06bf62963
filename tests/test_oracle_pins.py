"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests compares the oracle with a retyped copy of itself: each
one checks a worked example, a closed form, an invariant, a special case that
reduces to a textbook computation, or an independently derived form.
All run on the CPU in float64.
"""

import json
import os

import numpy as np
import pytest

from oracle import falcon_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "falcon_worked_examples.json")


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


def _gates(rng, lead, T, per_col_dv=None):
    zb = rng.standard_normal(lead + ((T, per_col_dv) if per_col_dv else (T,)))
    beta = 1 / (1 + np.exp(-zb))
    lam = np.log1p(np.exp(rng.standard_normal(lead + (T,)) - 2))
    return beta, lam


def _case(seed=0, lead=(2, 3), T=12, dk=5, dv=4, per_col=False):
    rng = np.random.default_rng(seed)
    K = _rand(lead + (T, dk), rng, 1 / np.sqrt(dk))
    Q = _rand(lead + (T, dk), rng, 1 / np.sqrt(dk))
    V = _rand(lead + (T, dv), rng, 1 / np.sqrt(dk))
    beta, lam = _gates(rng, lead, T, dv if per_col else None)
    return K, Q, V, beta, lam


# ---------------------------------------------------------------------------
# Worked examples (hand-derived; tests/golden/falcon_worked_examples.json)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("idx", [0, 1, 2])
def test_worked_examples(idx):
    case = json.load(open(GOLDEN))["cases"][idx]
    O, S = orc.falcon_forward(case["variant"], np.array(case["phi_k"]), np.array(case["phi_q"]),
                              np.array(case["v"]), np.array(case["beta"]), np.array(case["lam"]),
                              eps=case["eps"])
    np.testing.assert_allclose(O, np.array(case["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, np.array(case["S_T"]), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P1: fresh-start boundary x_1 = 0, eta_1 = 0 (§3 indexing conventions)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("variant", orc.VARIANTS)
def test_boundary_first_step_is_noop(variant):
    per_col = variant in ("falcon2", "falcon2a")
    K, Q, V, beta, lam = _case(1, per_col=per_col)
    rng = np.random.default_rng(7)
    S0 = rng.standard_normal((2, 3, 5, 4))
    O, S_T, states = orc.falcon_forward(variant, K, Q, V, beta, lam, eps=1e-6, S0=S0, return_states=True)
    # S_1 = S_0 and o_1 = S_0^T q_1 even with a carried state and lam_1 > 0.
    np.testing.assert_allclose(states[0], S0, rtol=0, atol=0)
    np.testing.assert_allclose(O[..., 0, :], np.einsum("...kv,...k->...v", S0, Q[..., 0, :]), atol=1e-14)
    # The last key, beta_1, lam_1 and v_1 never influence the outputs.
    K2, V2, beta2, lam2 = K.copy(), V.copy(), beta.copy(), lam.copy()
    K2[..., -1, :] = 100.0
    V2[..., 0, :] = -50.0
    if per_col:
        beta2[..., 0, :] = 1.9
    else:
        beta2[..., 0] = 1.9
    lam2[..., 0] = 30.0
    O2, S2 = orc.falcon_forward(variant, K2, Q, V2, beta2, lam2, eps=1e-6, S0=S0)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(S_T, S2)


# ---------------------------------------------------------------------------
# P2: lam = 0 Falcon-1A is shifted unnormalised linear attention (§2.2 Eq. 2.4
#     with lam = 0; end of §4.5), computed here by brute-force prefix sums.
# ---------------------------------------------------------------------------

def test_falcon1a_lam0_is_shifted_linear_attention():
    K, Q, V, beta, _ = _case(2, lead=(3,), T=10, dk=4, dv=3)
    lam = np.zeros_like(beta)
    eps = 1e-3
    O, _ = orc.falcon_forward("falcon1a", K, Q, V, beta, lam, eps=eps)
    T = K.shape[-2]
    ref = np.zeros_like(O)
    for b in range(K.shape[0]):
        for t in range(T):                  # 0-based t is the paper's t+1
            acc = np.zeros(V.shape[-1])
            for j in range(1, t + 1):       # paper's j = 2..t+1
                x = K[b, j - 1]
                eta = beta[b, j] / (x @ x + eps)
                acc += eta * (Q[b, t] @ x) * V[b, j]
            ref[b, t] = acc
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# P3: beta = 1, lam = 0, eps = 0 makes the write an exact projection
#     (orthogonal projection remark of §2.3; NLMS remark of §3.1); in general
#     x_t^T S_t = (1 - beta_t) x_t^T S_{t-1} + beta_t v_t^T (eigen-structure of
#     the transition, [juho]).
# ---------------------------------------------------------------------------

def test_projection_identity():
    K, Q, V, beta, lam = _case(3, lead=(2,), T=9, dk=6, dv=3)
    beta = np.ones_like(beta)
    lam = np.zeros_like(lam)
    _, _, states = orc.falcon_forward("falcon1", K, Q, V, beta, lam, eps=0.0, return_states=True)
    for t in range(1, K.shape[-2]):
        x = K[:, t - 1]
        np.testing.assert_allclose(np.einsum("bkv,bk->bv", states[t], x), V[:, t], rtol=1e-12, atol=1e-12)


def test_transition_along_key_direction():
    K, Q, V, beta, lam = _case(4, lead=(2,), T=9, dk=6, dv=3)
    beta = beta * 1.8                       # includes the beta > 1 sign-flip regime
    lam = np.zeros_like(lam)
    S0 = np.random.default_rng(5).standard_normal((2, 6, 3))
    _, _, states = orc.falcon_forward("falcon1", K, Q, V, beta, lam, eps=0.0, S0=S0, return_states=True)
    prev = [S0] + states[:-1]
    for t in range(1, K.shape[-2]):
        x = K[:, t - 1]
        lhs = np.einsum("bkv,bk->bv", states[t], x)
        rhs = (1 - beta[:, t])[:, None] * np.einsum("bkv,bk->bv", prev[t], x) + beta[:, t][:, None] * V[:, t]
        np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-12)
        # Directions orthogonal to x are only decayed by gamma = 1 (lam = 0).
        u = np.random.default_rng(t).standard_normal(x.shape)
        u -= (np.sum(u * x, -1) / np.sum(x * x, -1))[:, None] * x
        np.testing.assert_allclose(np.einsum("bkv,bk->bv", states[t], u),
                                   np.einsum("bkv,bk->bv", prev[t], u), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# P4: the masked-parallel forms (§4.6 for the inner-product rule; the dense
#     triangular-solve form for Falcon-1) reproduce the recurrence.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("with_kprev", [False, True])
def test_masked_parallel_equals_recurrence(with_state, with_kprev):
    K, Q, V, beta, lam = _case(5, lead=(2, 2), T=40, dk=8, dv=6)
    rng = np.random.default_rng(9)
    S0 = rng.standard_normal((2, 2, 8, 6)) * 0.3 if with_state else None
    kp = rng.standard_normal((2, 2, 8)) / np.sqrt(8) if with_kprev else None
    lam = lam * 3.0                        # stronger decay
    for variant, masked in (("falcon1", orc.falcon1_masked), ("falcon1a", orc.falcon1a_masked)):
        O_r, S_r = orc.falcon_forward(variant, K, Q, V, beta, lam, eps=1e-6, S0=S0, k_prev=kp)
        O_m, S_m = masked(K, Q, V, beta, lam, eps=1e-6, S0=S0, k_prev=kp)
        np.testing.assert_allclose(O_m, O_r, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(S_m, S_r, rtol=1e-10, atol=1e-12)


def test_masked_parallel_with_active_clamp():
    K, Q, V, beta, lam = _case(6, lead=(2,), T=24, dk=4, dv=4)
    beta = np.full_like(beta, 1.9)
    lam = np.full_like(lam, 10.0)
    K = K * 0.05                            # tiny energy: eta*lam close to beta > 1
    for variant, masked in (("falcon1", orc.falcon1_masked), ("falcon1a", orc.falcon1a_masked)):
        O_r, S_r = orc.falcon_forward(variant, K, Q, V, beta, lam, eps=1e-6, eps_gamma=1e-3)
        O_m, S_m = masked(K, Q, V, beta, lam, eps=1e-6, eps_gamma=1e-3)
        np.testing.assert_allclose(O_m, O_r, rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(S_m, S_r, rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------------------
# Continuation: a split run with (S_T1, phi(k_T1)) handed over equals one run.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("variant", orc.VARIANTS)
def test_continuation(variant):
    per_col = variant in ("falcon2", "falcon2a")
    K, Q, V, beta, lam = _case(7, T=20, per_col=per_col)
    O, S = orc.falcon_forward(variant, K, Q, V, beta, lam, eps=1e-6)
    T1 = 7
    O1, S1 = orc.falcon_forward(variant, K[..., :T1, :], Q[..., :T1, :], V[..., :T1, :],
                                beta[..., :T1, :] if per_col else beta[..., :T1],
                                lam[..., :T1], eps=1e-6)
    b2 = beta[..., T1:, :] if per_col else beta[..., T1:]
    O2, S2 = orc.falcon_forward(variant, K[..., T1:, :], Q[..., T1:, :], V[..., T1:, :], b2,
                                lam[..., T1:], eps=1e-6, S0=S1, k_prev=K[..., T1 - 1, :])
    np.testing.assert_allclose(np.concatenate([O1, O2], axis=-2), O, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# P7: Falcon-2 with tied gains is Falcon-1; each Falcon-2 column is an
#     independent scalar-step rule (§4.2 "Per-column NLMS step sizes").
# ---------------------------------------------------------------------------

def test_falcon2_tied_is_falcon1():
    K, Q, V, beta, lam = _case(8)
    tied = np.repeat(beta[..., None], V.shape[-1], axis=-1)
    for v2, v1 in (("falcon2", "falcon1"), ("falcon2a", "falcon1a")):
        O2, S2 = orc.falcon_forward(v2, K, Q, V, tied, lam, eps=1e-6)
        O1, S1 = orc.falcon_forward(v1, K, Q, V, beta, lam, eps=1e-6)
        np.testing.assert_allclose(O2, O1, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-14)


def test_falcon2_columns_are_independent_scalar_rules():
    K, Q, V, beta, lam = _case(9, per_col=True)
    for v2, v1 in (("falcon2", "falcon1"), ("falcon2a", "falcon1a")):
        O2, S2 = orc.falcon_forward(v2, K, Q, V, beta, lam, eps=1e-6)
        for j in range(V.shape[-1]):
            Oj, Sj = orc.falcon_forward(v1, K, Q, V[..., j:j + 1], beta[..., j], lam, eps=1e-6)
            np.testing.assert_allclose(O2[..., j:j + 1], Oj, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(S2[..., j:j + 1], Sj, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# P9: Lemma 3.1 per-step descent of the unclamped update on the ridge loss.
# ---------------------------------------------------------------------------

def test_lemma_3_1_descent():
    K, Q, V, beta, lam = _case(10, lead=(1,), T=30, dk=6, dv=5)
    beta = beta * 1.9                        # whole admissible range (0, 2)
    eps = 1e-3
    S0 = np.random.default_rng(11).standard_normal((1, 6, 5))
    _, _, states = orc.falcon_forward("falcon1", K, Q, V, beta, lam, eps=eps, S0=S0,
                                      clamp=False, return_states=True)
    prev = [S0] + states[:-1]
    for t in range(1, K.shape[-2]):
        x, y, lt = K[0, t - 1], V[0, t], lam[0, t]
        L = x @ x + lt
        eta = beta[0, t] / (L + eps)
        f0, g0 = orc.ridge_loss(prev[t][0], x, y, lt)
        f1, _ = orc.ridge_loss(states[t][0], x, y, lt)
        bound = f0 - eta * (2 - eta * L) / 2 * np.sum(g0 * g0)
        assert f1 <= bound + 1e-12 * max(1.0, abs(f0))
        # The update is exactly one gradient step of the ridge loss (Eq. 3.3).
        np.testing.assert_allclose(states[t][0], prev[t][0] - eta * g0, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# P10: linearity in (S_0, V) for fixed features and gates; P11: scale law.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("variant", orc.VARIANTS)
def test_linearity_in_state_and_values(variant):
    per_col = variant in ("falcon2", "falcon2a")
    K, Q, V, beta, lam = _case(12, per_col=per_col)
    rng = np.random.default_rng(13)
    V2 = rng.standard_normal(V.shape)
    Sa, Sb = rng.standard_normal((2, 3, 5, 4)), rng.standard_normal((2, 3, 5, 4))
    a, b = 0.7, -1.3
    Oa, STa = orc.falcon_forward(variant, K, Q, V, beta, lam, eps=1e-6, S0=Sa)
    Ob, STb = orc.falcon_forward(variant, K, Q, V2, beta, lam, eps=1e-6, S0=Sb)
    Oc, STc = orc.falcon_forward(variant, K, Q, a * V + b * V2, beta, lam, eps=1e-6, S0=a * Sa + b * Sb)
    np.testing.assert_allclose(Oc, a * Oa + b * Ob, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(STc, a * STa + b * STb, rtol=1e-11, atol=1e-12)


def test_scale_law():
    K, Q, V, beta, lam = _case(14)
    c, eps = 3.0, 1e-2
    O, S = orc.falcon_forward("falcon1", K, Q, V, beta, lam, eps=eps)
    Oc, Sc = orc.falcon_forward("falcon1", c * K, Q, V, beta, c * c * lam, eps=c * c * eps)
    np.testing.assert_allclose(Oc, O / c, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(Sc, S / c, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------------------
# P12: the unshifted delta rule (§2.3) with ridge, fed the shifted stream and
#      eta_1 = 0, is Falcon-1 (§4.2 "standard vs. next-latent").
# ---------------------------------------------------------------------------

def test_unshifted_delta_rule_on_shifted_stream():
    K, Q, V, beta, lam = _case(15, lead=(1,), T=15, dk=4, dv=3)
    eps = 1e-6
    O, S_T = orc.falcon_forward("falcon1", K, Q, V, beta, lam, eps=eps)
    X = np.concatenate([np.zeros((1, 1, 4)), K[:, :-1]], axis=1)
    S = np.zeros((4, 3))
    for t in range(K.shape[1]):
        k = X[0, t]
        eta = 0.0 if t == 0 else beta[0, t] / (k @ k + lam[0, t] + eps)
        # (I - eta k k^T) S + eta k v^T, plus the ridge shrinkage -eta lam S
        S = (np.eye(4) - eta * np.outer(k, k)) @ S + eta * np.outer(k, V[0, t]) - eta * lam[0, t] * S
        np.testing.assert_allclose(S.T @ Q[0, t], O[0, t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, S_T[0], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# P13: single-pass decode algebra; decode steps reproduce the forward pass.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("variant", orc.VARIANTS)
def test_decode_steps_equal_forward(variant):
    per_col = variant in ("falcon2", "falcon2a")
    K, Q, V, beta, lam = _case(16, T=10, per_col=per_col)
    O, S_T = orc.falcon_forward(variant, K, Q, V, beta, lam, eps=1e-6)
    S = np.zeros((2, 3, 5, 4))
    for t in range(K.shape[-2]):
        x = np.zeros((2, 3, 5)) if t == 0 else K[..., t - 1, :]
        b = beta[..., t, :] if per_col else beta[..., t]
        o, S = orc.falcon_decode_step(variant, S, x, Q[..., t, :], V[..., t, :], b, lam[..., t],
                                      eps=1e-6, is_first=np.full((2, 3), t == 0))
        np.testing.assert_allclose(o, O[..., t, :], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, S_T, rtol=1e-12, atol=1e-14)


def test_decode_single_pass_read():
    rng = np.random.default_rng(17)
    S = rng.standard_normal((4, 6, 5))
    x, q, v = rng.standard_normal((4, 6)), rng.standard_normal((4, 6)), rng.standard_normal((4, 5))
    beta, lam = np.full(4, 0.6), np.full(4, 0.3)
    o, _ = orc.falcon_decode_step("falcon1", S, x, q, v, beta, lam, eps=1e-6)
    eta = beta / (np.sum(x * x, -1) + lam + 1e-6)
    gamma = 1 - eta * lam
    r = v - np.einsum("bkv,bk->bv", S, x)
    p = np.einsum("bkv,bk->bv", S, q)
    np.testing.assert_allclose(o, gamma[:, None] * p + (eta * np.sum(x * q, -1))[:, None] * r,
                               rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# P14: clamp semantics (§4.3 "Decay positivity"): gamma = eps_gamma, write
#      gain still eta.
# ---------------------------------------------------------------------------

def test_clamp_semantics():
    rng = np.random.default_rng(18)
    S = rng.standard_normal((1, 3, 2))
    x = rng.standard_normal((1, 3)) * 0.01
    q, v = rng.standard_normal((1, 3)), rng.standard_normal((1, 2))
    beta, lam, eg = np.array([1.9]), np.array([10.0]), 1e-4
    o, S1 = orc.falcon_decode_step("falcon1", S, x, q, v, beta, lam, eps=1e-6, eps_gamma=eg)
    eta = 1.9 / (x[0] @ x[0] + 10.0 + 1e-6)
    assert eta * 10.0 > 1 - eg                      # the clamp is active
    r = v[0] - S[0].T @ x[0]
    np.testing.assert_allclose(S1[0], eg * S[0] + eta * np.outer(x[0], r), rtol=1e-12, atol=1e-14)
    _, S1u = orc.falcon_decode_step("falcon1", S, x, q, v, beta, lam, eps=1e-6, clamp=False)
    np.testing.assert_allclose(S1u[0], (1 - eta * 10.0) * S[0] + eta * np.outer(x[0], r), rtol=1e-12)


def test_zero_denominator_gives_zero_step():
    S = np.ones((1, 2, 2))
    x = np.zeros((1, 2))
    o, S1 = orc.falcon_decode_step("falcon1", S, x, np.ones((1, 2)), np.ones((1, 2)),
                                   np.array([0.5]), np.array([0.0]), eps=0.0)
    np.testing.assert_array_equal(S1, S)
