"""A binding decay clamp yields gamma = eps_gamma itself in every forward
path ("Fast Weight Attention for Continual Learning", Section 4.3, decay
positivity: alpha is capped at 1 - eps_gamma, so gamma is eps_gamma).

With zero keys and a zero previous key every energy is 0, so
eta = beta / (lam + eps) and, with beta = 1.5, alpha = eta lam > 1: every
step clamps and the write x r^T vanishes, leaving S_t = eps_gamma S_{t-1}
exactly.  The final state is then eps_gamma^T S0 and each output
eps_gamma^(t+1) S0^T q_t.  A decay formed as 1 minus the float nearest
1 - eps_gamma is off by up to 5 % at eps_gamma = 1e-6, and by T times that
after T steps; the forward tolerances elsewhere cannot see it because the
clamped term is tiny next to the write.  Here it is the whole result, so the
float32 final states are held element by element, and each output vector in
relative L2, to 1e-5 (a few float32 roundings per step and the exponential
of a log-decay sum near -70), and the bf16-I/O fast path's float32 final
state likewise."""

import numpy as np
import pytest
import torch

from delta_rule_recurrence_amd import falcon as fb
from delta_rule_recurrence_amd import inputs as I

from gpu_utils import oracle_forward, to_dev

pytestmark = pytest.mark.gpu

VARIANTS = ("falcon1", "falcon1a", "falcon2", "falcon2a")
# (eps_gamma, T): eps_gamma^T stays a normal float32
STEPS = ((1e-6, 5), (1e-3, 11))


def clamped_inputs(variant, io, T, dk, dv, seed):
    B, H = 2, 3
    x = I.make_inputs(B, H, T, dk, dv, seed=seed, io_dtype=io,
                      per_column_beta=variant in ("falcon2", "falcon2a"))
    x["phi_k"] = torch.zeros_like(x["phi_k"])
    x["beta"] = torch.full_like(x["beta"], 1.5)
    g = np.random.default_rng([seed, 7])
    S0 = torch.from_numpy(g.standard_normal((B, H, dk, dv)).astype(np.float32))
    k_prev = torch.zeros((B, H, dk), dtype=I.TORCH_DTYPE[io])
    return x, S0, k_prev


def rel_elementwise(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300)))


def rel_rows(got, ref):
    """Largest relative L2 error over the output vectors (last axis): an
    output element is a dot product that may cancel, its vector does not."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)))


def run(entry, variant, x, S0, k_prev, eps_gamma, C):
    d = to_dev(x)
    kw = dict(variant=variant, eps=1e-6, eps_gamma=eps_gamma, S0=S0.cuda(), k_prev=k_prev.cuda())
    if entry == "chunked":
        kw["C"] = C
        o, S_T = fb.falcon_fwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], **kw)
    else:
        o, S_T = fb.falcon_fwd_recurrent(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S_T.cpu().numpy()


@pytest.mark.parametrize("eps_gamma,T", STEPS, ids=["eps_gamma_1e-6", "eps_gamma_1e-3"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_clamped_decay_is_eps_gamma_f32(variant, eps_gamma, T):
    x, S0, k_prev = clamped_inputs(variant, "f32", T, 32, 16, seed=4100 + T)
    O_ref, S_ref = oracle_forward(variant, x, eps=1e-6, eps_gamma=eps_gamma, S0=S0, k_prev=k_prev)
    # the oracle's own 1 - (1 - eps_gamma) in float64 is within 1e-9 of eps_gamma
    assert np.allclose(S_ref, eps_gamma ** T * S0.double().numpy(), rtol=1e-8, atol=0)
    for entry, C in (("chunked", 16), ("chunked", 64), ("recurrent", None)):
        o, S_T = run(entry, variant, x, S0, k_prev, eps_gamma, C)
        what = f"{variant} {entry} C={C} eps_gamma={eps_gamma} T={T}"
        print(f"[clamp] {what}", flush=True)
        es, eo = rel_elementwise(S_T, S_ref), rel_rows(o, O_ref)
        assert es <= 1e-5 and eo <= 1e-5, f"{what}: relative error S_T={es:.2e} (element-wise) o={eo:.2e} (per vector)"


@pytest.mark.parametrize("eps_gamma,T", STEPS, ids=["eps_gamma_1e-6", "eps_gamma_1e-3"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_clamped_decay_is_eps_gamma_bf16_fast_path(variant, eps_gamma, T):
    """dk = dv = C = 64 with bf16 I/O takes the MFMA paths; their final state
    is float32."""
    x, S0, k_prev = clamped_inputs(variant, "bf16", T, 64, 64, seed=4200 + T)
    _, S_ref = oracle_forward(variant, x, eps=1e-6, eps_gamma=eps_gamma, S0=S0, k_prev=k_prev)
    for entry in ("chunked", "recurrent"):
        _, S_T = run(entry, variant, x, S0, k_prev, eps_gamma, 64)
        es = rel_elementwise(S_T, S_ref)
        assert es <= 1e-5, f"{variant} {entry} bf16 eps_gamma={eps_gamma} T={T}: S_T element-wise {es:.2e}"


@pytest.mark.parametrize("eps_gamma", (1e-6, 1e-3))
@pytest.mark.parametrize("variant", VARIANTS)
def test_clamped_decay_is_eps_gamma_decode(variant, eps_gamma):
    """T decode steps with a zero previous key: S is scaled by eps_gamma each
    step, and each output is the scaled state applied to the query."""
    steps = 5 if eps_gamma == 1e-6 else 11
    x, S0, _ = clamped_inputs(variant, "f32", steps, 32, 16, seed=4300)
    d = to_dev(x)
    S = S0.cuda().clone()
    zero = torch.zeros_like(d["phi_k"][:, :, 0])
    for t in range(steps):
        o = fb.falcon_decode_step(zero, d["phi_q"][:, :, t].contiguous(), d["v"][:, :, t].contiguous(),
                                  d["beta"][:, :, t].contiguous(), d["lam"][:, :, t].contiguous(), S,
                                  variant=variant, eps=1e-6, eps_gamma=eps_gamma)
        torch.cuda.synchronize()
        S_ref = eps_gamma ** (t + 1) * S0.double().numpy()
        o_ref = np.einsum("bhkv,bhk->bhv", S_ref, x["phi_q"][:, :, t].double().numpy())
        es, eo = rel_elementwise(S.cpu().numpy(), S_ref), rel_rows(o.cpu().numpy(), o_ref)
        assert es <= 1e-5 and eo <= 1e-5, f"{variant} decode step {t}: S {es:.2e} o {eo:.2e}"
