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


def _decode_inputs_batch(steps, D, pool):
    """Inputs of the given decode steps, drawn in parallel (one generator per
    step, so the values do not depend on the thread count)."""
    B, H, dk, dv = D["B"], D["H"], D["dk"], D["dv"]
    return list(pool.map(lambda s: I.decode_step_inputs(s, B, H, dk, dv, seed=D["seed"],
                                                        io_dtype=D["io_dtype"]), steps))


def test_decode_workload_full_batch():
    """The decode workload as stated: batch 512 x 12 heads, d = 128, float32
    state, 1000 sequential decode steps from a state built by a seeded random
    prefix.  The prefix (128 tokens, float32 I/O) runs through the chunked
    forward on the GPU; its final state is checked against the oracle's
    recurrence on a seeded subset of 32 batch rows (1e-4) and then handed,
    identically, to the GPU decode (full batch) and the oracle decode (the
    subset).  Every step's output and the state every 100 steps are checked
    on the subset (2e-2)."""
    from concurrent.futures import ThreadPoolExecutor

    D = I.DECODE
    B, H, dk, dv = D["B"], D["H"], D["dk"], D["dv"]
    steps = D["steps"]
    pre = I.make_inputs(B, H, D["prefix"], dk, dv, seed=D["seed"], io_dtype="f32")
    dev = to_dev(pre)
    _, S = fb.falcon_fwd_chunked(dev["phi_k"], dev["phi_q"], dev["v"], dev["beta"], dev["lam"],
                                 C=64, eps=D["eps"], eps_gamma=D["eps_gamma"])
    rows = np.sort(np.random.default_rng(99).choice(B, size=32, replace=False))
    sub = {k: v[rows] for k, v in pre.items()}
    _, S_pre_ref = oracle_forward("falcon1", sub, eps=D["eps"], eps_gamma=D["eps_gamma"])
    torch.cuda.synchronize()
    S_init = S[rows].cpu()
    e_pre = rel_l2(S_init.numpy(), S_pre_ref)
    print(f"decode prefix: float32 chunked state vs oracle on {len(rows)} rows: rel L2 {e_pre:.2e}")
    assert e_pre <= TOL["f32"]
    S_ref = I.as_f64(S_init)
    rows_dev = torch.from_numpy(rows).cuda()
    # the key read by step 1 is the prefix's last key, in the decode I/O dtype
    x = dev["phi_k"][:, :, -1].to(torch.bfloat16).contiguous()
    x_ref = I.as_f64(x[rows_dev].cpu())
    o = torch.empty((B, H, dv), dtype=torch.bfloat16, device="cuda")
    worst_o, worst_s = 0.0, 0.0
    chunk = 50
    with ThreadPoolExecutor(8) as pool:
        for s0 in range(1, steps + 1, chunk):
            batch = _decode_inputs_batch(range(s0, min(s0 + chunk, steps + 1)), D, pool)
            outs = []
            for st in batch:
                sd = to_dev(st)
                fb.falcon_decode_step(x, sd["phi_q"], sd["v"], sd["beta"], sd["lam"], S, o=o,
                                      eps=D["eps"], eps_gamma=D["eps_gamma"])
                outs.append(o[rows_dev].float().cpu())
                x = sd["phi_k"]
            for j, st in enumerate(batch):
                o_ref, S_ref = orc.falcon_decode_step(
                    "falcon1", S_ref, x_ref, I.as_f64(st["phi_q"][rows]), I.as_f64(st["v"][rows]),
                    I.as_f64(st["beta"][rows]), I.as_f64(st["lam"][rows]), eps=D["eps"],
                    eps_gamma=D["eps_gamma"])
                worst_o = max(worst_o, rel_l2(outs[j].numpy(), o_ref))
                x_ref = I.as_f64(st["phi_k"][rows])
            s_last = s0 + len(batch) - 1
            if s_last % 100 == 0:
                es = rel_l2(S[rows_dev].cpu().numpy(), S_ref)
                worst_s = max(worst_s, es)
                print(f"decode step {s_last}: worst per-step rel L2 o so far {worst_o:.3e}, S {es:.3e}",
                      flush=True)
    torch.cuda.synchronize()
    es = rel_l2(S[rows_dev].cpu().numpy(), S_ref)
    print(f"decode {steps} steps: worst per-step rel L2 o={worst_o:.3e}, final S={es:.3e}, "
          f"worst checkpoint S={worst_s:.3e}")
    assert worst_o <= TOL["bf16"] and es <= TOL["bf16"] and worst_s <= TOL["bf16"]
