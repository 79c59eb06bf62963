"""GPU parity at the benchmark workloads' full sizes, launched exactly as
bench.py launches them, against the CPU oracle on identical seeded inputs."""

import numpy as np
import pytest
import torch

from delta_rule_recurrence_amd import falcon as fb
from delta_rule_recurrence_amd import inputs as I
from oracle import falcon_oracle as orc

from gpu_utils import TOL, check, oracle_forward, rel_l2, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["f1_chunked_8x12x2048_d64", "f1a_chunked_2x12x16384_d64",
                                  "f2_chunked_8x12x2048_d64", "f1_chunked_f32_8x12x2048_d64"])
def test_full_workload(name):
    w = I.WORKLOADS[name]
    d = I.workload_inputs(w)
    dev = to_dev(d)
    o, S_T = fb.falcon_fwd_chunked(dev["phi_k"], dev["phi_q"], dev["v"], dev["beta"], dev["lam"],
                                   variant=w.variant, C=w.C, eps=w.eps, eps_gamma=w.eps_gamma)
    torch.cuda.synchronize()
    O_ref, S_ref = oracle_forward(w.variant, d, eps=w.eps, eps_gamma=w.eps_gamma)
    eo, es = check(o, S_T, O_ref, S_ref, TOL[w.io_dtype], name)
    # also per-sequence worst case, reported on failure
    got = o.float().cpu().numpy()
    worst = max(rel_l2(got[b, h], O_ref[b, h]) for b in range(w.B) for h in range(w.H))
    assert worst <= TOL[w.io_dtype], f"{name}: worst per-sequence rel L2 {worst:.3e}"
    print(f"{name}: rel L2 o={eo:.3e} S_T={es:.3e} worst-seq={worst:.3e}")


def test_decode_workload_full_batch():
    """Decode at batch 512 x 12 heads, d = 128: a 128-token prefix builds the
    state (chunked forward on the GPU, the recurrence in the oracle), then
    decode steps run on the full batch; a seeded subset of sequences is
    checked against the oracle step by step."""
    D = I.DECODE
    B, H, dk, dv = D["B"], D["H"], D["dk"], D["dv"]
    steps = 48
    pre = I.make_inputs(B, H, D["prefix"], dk, dv, seed=D["seed"], io_dtype=D["io_dtype"])
    dev = to_dev(pre)
    _, S = fb.falcon_fwd_chunked(dev["phi_k"], dev["phi_q"], dev["v"], dev["beta"], dev["lam"],
                                 C=64, eps=D["eps"], eps_gamma=D["eps_gamma"])
    rows = np.random.default_rng(99).choice(B, size=8, replace=False)
    sub = {k: v[rows] for k, v in pre.items()}
    _, S_ref = oracle_forward("falcon1", sub, eps=D["eps"], eps_gamma=D["eps_gamma"])
    torch.cuda.synchronize()
    assert rel_l2(S[rows].cpu().numpy(), S_ref) <= TOL["bf16"]
    x = dev["phi_k"][:, :, -1].contiguous()
    x_ref = I.as_f64(pre["phi_k"][rows][:, :, -1])
    worst_o = 0.0
    for s in range(1, steps + 1):
        st = I.decode_step_inputs(s, B, H, dk, dv, seed=D["seed"], io_dtype=D["io_dtype"])
        sd = to_dev(st)
        o = fb.falcon_decode_step(x, sd["phi_q"], sd["v"], sd["beta"], sd["lam"], S,
                                  eps=D["eps"], eps_gamma=D["eps_gamma"])
        o_ref, S_ref = orc.falcon_decode_step("falcon1", S_ref, x_ref, I.as_f64(st["phi_q"][rows]),
                                              I.as_f64(st["v"][rows]), I.as_f64(st["beta"][rows]),
                                              I.as_f64(st["lam"][rows]), eps=D["eps"],
                                              eps_gamma=D["eps_gamma"])
        worst_o = max(worst_o, rel_l2(o[rows].float().cpu().numpy(), o_ref))
        x = sd["phi_k"]
        x_ref = I.as_f64(st["phi_k"][rows])
    torch.cuda.synchronize()
    es = rel_l2(S[rows].cpu().numpy(), S_ref)
    assert worst_o <= TOL["bf16"] and es <= TOL["bf16"], f"decode: o {worst_o:.3e} S {es:.3e}"
    print(f"decode: worst per-step rel L2 o={worst_o:.3e}, S={es:.3e}")
