"""Benchmark of the Falcon-1 chunked forward on one MI355X.

Workload: Falcon-1 chunk-parallel forward, B=8, H=12, T=2048, dk=dv=64,
C=64, bf16 features/values/outputs, float32 gates and state, S_0 = 0,
synthetic seeded inputs (seed 1).  One step = one falcon_fwd_chunked call
over the whole batch.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/sec + % MFMA peak, Falcon-1 chunked fwd B=8 H=12 T=2048 d=64 bf16"
WORKLOAD = "f1_chunked_8x12x2048_d64"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 MFMA, published
# The headline step runs two launches: a fill of the hand-over flags, then one
# kernel whose chunk workgroups build the chunk matrices while per-sequence
# chain workgroups carry the state and write the outputs.
STEP_KERNELS = ["zero_ints_kernel", "falcon1_fused_kernel"]
# rocprofv3 counter summaries under profiles/ (<name>_counters.md), each valid
# while the sources of its kernels hash to the value recorded in it.
_CSRC = "delta_rule_recurrence_amd/csrc/"
PROFILE_SOURCES = {
    "falcon1_chunked_8x12x2048_d64": [_CSRC + "falcon_chunked_wy.hip", _CSRC + "falcon_mfma_frag.h",
                                      _CSRC + "falcon_chunked.hip", _CSRC + "falcon_device.h"],
    "falcon1a_chunked_2x12x16384_d64": [_CSRC + "falcon_chunked_scan.hip", _CSRC + "falcon_mfma_frag.h",
                                        _CSRC + "falcon_device.h"],
    "falcon2_chunked_8x12x2048_d64": [_CSRC + "falcon_chunked_percol.hip", _CSRC + "falcon_mfma_frag.h",
                                      _CSRC + "falcon_device.h"],
    "falcon1_decode_512x12_d128": [_CSRC + "falcon_recurrent.hip", _CSRC + "falcon_device.h"],
    "falcon1_recurrent_8x12x2048_d64": [_CSRC + "falcon_recurrent.hip", _CSRC + "falcon_device.h"],
    "falcon1_chunked_f32_8x12x2048_d64": [_CSRC + "falcon_generic_kernel.h", _CSRC + "falcon_chunked_generic.hip",
                                          _CSRC + "falcon_chunked_generic_c64.hip", _CSRC + "falcon_device.h"],
    "falcon1_backward_8x12x2048_d64": [_CSRC + "falcon_backward.hip", _CSRC + "falcon_device.h"],
}


def algorithmic_bytes(B, H, T, dk, dv, io_bytes=2, per_column_beta=False):
    """Compulsory HBM bytes of one forward: read phi(k), phi(q), v once, beta
    (one per token, or one per token and value column) and lam once, write o
    once and S_T once (S_0 = 0 is not read)."""
    th = B * H * T
    gates = th * ((dv if per_column_beta else 1) + 1) * 4
    return th * (2 * dk + dv) * io_bytes + gates + th * dv * io_bytes + B * H * dk * dv * 4


def algorithmic_flops(B, H, T, dk, dv, C):
    """Falcon-1 chunked-form flops per token-head, triangles counted once:
    W S, X^T R and Q S (2 dk dv each), the decayed Gram and Q X^T (C dk each),
    the W and U factors (C (dk + dv)), the intra-chunk read (C dv) and the
    triangular inverse (C^2 / 3)."""
    per = 6 * dk * dv + 2 * C * dk + C * (dk + dv) + C * dv + C * C / 3
    return B * H * T * per


# MI355X fp32 vector peak without packed fp32 instructions (the build turns
# them off): 256 CUs x 4 SIMDs x 16 lanes x 2 flops (FMA) x 2.4 GHz.  The
# published 157.3 TFLOP/s figure counts packed (two-wide) fp32 issue.
FP32_VALU_PEAK_TFLOPS = 78.6


def recurrence_flops(B, H, T, dk, dv):
    """Arithmetic the per-column rules (Falcon-2 / 2A) cannot avoid, per
    token-head: the residual read S^T x (2 dk dv), the decayed rank-1 write
    gamma_j S + x (eta_j r_j) (3 dk dv: a multiply and a multiply-add per
    element) and the output read S^T q (2 dk dv)."""
    return 7.0 * B * H * T * dk * dv


def kernel_source_hash(name):
    h = hashlib.sha256()
    for rel in PROFILE_SOURCES[name]:
        p = os.path.join(ROOT, rel)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def profile_counters(name):
    """Per-call totals from the committed rocprofv3 summary
    profiles/<name>_counters.md (HBM traffic from FETCH_SIZE / WRITE_SIZE
    scaled by a plain copy, MFMA flops from SQ_INSTS_VALU_MFMA_MOPS_*, kernel
    time), or None when the kernel sources changed after the counters were
    taken."""
    path = os.path.join(ROOT, "profiles", f"{name}_counters.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"^pmc_json:\s*(\{.*\})\s*$", open(path).read(), flags=re.M)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("kernel_source_sha256_16") != kernel_source_hash(name):
        return None
    return d


def counter_fields(name, ms):
    """Roofline `traffic` and the counter-derived MFMA share of peak for a leg
    whose call takes `ms` milliseconds (None where no valid summary exists)."""
    c = profile_counters(name)
    if c is None:
        return None, None
    t = ms * 1e-3
    mfma = {"bf16_pct_of_peak": 100.0 * c["mfma_bf16_flops"] / t / (BF16_MFMA_PEAK_TFLOPS * 1e12),
            "f32_pct_of_peak": 100.0 * c["mfma_f32_flops"] / t / (FP32_MFMA_PEAK_TFLOPS * 1e12),
            "bf16_flops_per_call": c["mfma_bf16_flops"], "f32_flops_per_call": c["mfma_f32_flops"],
            "source": f"profiles/{name}_counters.md (SQ_INSTS_VALU_MFMA_MOPS_* x 512)"}
    return c["traffic_bytes"], mfma


def attach_counters(out, profile, ms):
    """Fill a leg's roofline `traffic` and its counter-derived MFMA share from
    the committed summary of its kernels (left null when none is valid)."""
    traffic, mfma = counter_fields(profile, ms)
    if "roofline" in out:
        out["roofline"]["traffic"] = traffic
    out["mfma_counters"] = mfma
    out["counters_profile"] = f"profiles/{profile}_counters.md"
    return out


def decode_bytes(B, H, dk, dv, io_bytes=2):
    """Compulsory HBM bytes of one decode step: the float32 state read and
    written once, x, q, v read, beta and lam read, o written."""
    bh = B * H
    return 2 * bh * dk * dv * 4 + bh * (2 * dk + dv) * io_bytes + bh * 2 * 4 + bh * dv * io_bytes


def bench_decode(warmup=5):
    """The decode workload as stated: batch 512 x 12 heads, d = 128, float32
    state (~384 MiB) resident in HBM, built by a seeded 128-token prefix
    (chunked forward, float32 I/O), then the 1000 sequential decode steps
    with their own inputs, all pre-staged in HBM before timing.  The warm-up
    steps run on a copy of the state."""
    from concurrent.futures import ThreadPoolExecutor

    import torch

    from delta_rule_recurrence_amd import falcon as fb
    from delta_rule_recurrence_amd import inputs as I

    D = I.DECODE
    B, H, dk, dv, steps = D["B"], D["H"], D["dk"], D["dv"], D["steps"]
    pre = {k: v.cuda() for k, v in I.make_inputs(B, H, D["prefix"], dk, dv, seed=D["seed"],
                                                 io_dtype="f32").items()}
    _, S_init = fb.falcon_fwd_chunked(pre["phi_k"], pre["phi_q"], pre["v"], pre["beta"], pre["lam"],
                                      C=64, eps=D["eps"], eps_gamma=D["eps_gamma"])
    x0 = pre["phi_k"][:, :, -1].to(torch.bfloat16).contiguous()
    del pre
    with ThreadPoolExecutor(8) as pool:
        host = list(pool.map(lambda s: I.decode_step_inputs(s, B, H, dk, dv, seed=D["seed"],
                                                            io_dtype=D["io_dtype"]), range(1, steps + 1)))
    staged = [{k: v.cuda() for k, v in st.items()} for st in host]
    del host
    xs = [x0] + [st["phi_k"] for st in staged[:-1]]
    o = torch.empty((B, H, dv), dtype=torch.bfloat16, device="cuda")

    def step(S, i):
        st = staged[i]
        fb.falcon_decode_step(xs[i], st["phi_q"], st["v"], st["beta"], st["lam"], S, o=o,
                              eps=D["eps"], eps_gamma=D["eps_gamma"])

    S = S_init.clone()
    for i in range(warmup):
        step(S, i)
    S.copy_(S_init)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(S, i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = decode_bytes(B, H, dk, dv)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"workload": D["name"], "steps": steps, "state": "from a 128-token prefix (chunked, f32 I/O)",
           "us_per_step": ms * 1e3, "tokens_per_s": B / (ms * 1e-3), "algorithmic_bytes": nbytes,
           "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": nbytes,
                        "kernels": ["decode_kernel"]}}
    return attach_counters(out, "falcon1_decode_512x12_d128", ms)


def warm(step, min_calls, seconds=0.3):
    """Untimed warm-up of a leg beside the headline: at least min_calls calls
    and at least `seconds` of wall time, so that the GPU's clocks have ramped
    again after the host-side work between legs.  Returns the calls made."""
    import time

    import torch

    n = 0
    t0 = time.perf_counter()
    while n < min_calls or time.perf_counter() - t0 < seconds:
        step()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def bench_chunked_workload(name, steps=20, warmup=3):
    """Another chunked workload (inputs resident in HBM), timed with HIP events
    on the launch stream; reported beside the headline line."""
    import torch

    from delta_rule_recurrence_amd import falcon as fb
    from delta_rule_recurrence_amd import inputs as I

    w = I.WORKLOADS[name]
    d = {k: v.cuda() for k, v in I.workload_inputs(w).items()}
    io = I.TORCH_DTYPE[w.io_dtype]
    o = torch.empty((w.B, w.H, w.T, w.dv), dtype=io, device="cuda")
    S_T = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    p = fb.make_problem(w.B, w.H, w.T, w.dk, w.dv, variant=w.variant, io_dtype=io,
                        eps=w.eps, eps_gamma=w.eps_gamma)
    ws = torch.empty(max(fb.falcon_workspace_bytes(p, w.C), 16), dtype=torch.uint8, device="cuda")

    def step():
        fb.falcon_fwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], variant=w.variant,
                              C=w.C, o=o, S_T=S_T, workspace=ws)

    calls = warm(step, warmup)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = algorithmic_bytes(w.B, w.H, w.T, w.dk, w.dv, io_bytes=4 if w.io_dtype == "f32" else 2,
                               per_column_beta=w.variant in ("falcon2", "falcon2a"))
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"workload": name, "variant": w.variant, "io": w.io_dtype, "steps": steps, "warmup_calls": calls,
           "us_per_step": ms * 1e3,
           "tokens_per_s": w.B * w.T / (ms * 1e-3), "algorithmic_bytes": nbytes,
           "workspace_bytes": int(ws.numel()), "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
    if w.variant in ("falcon2", "falcon2a"):
        # the roofline of the workload is HBM (its arithmetic intensity is far
        # below the ridge); the kernel is limited by vector-ALU issue of the
        # per-column substitution, reported beside it against the non-packed
        # fp32 VALU peak (packed fp32 is disabled in the build)
        flops = recurrence_flops(w.B, w.H, w.T, w.dk, w.dv)
        tf = flops / (ms * 1e-3) / 1e12
        out["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": gbs / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": nbytes,
                           "kernels": ["falcon2_chunked_kernel"]}
        out["valu"] = {"achieved_tflops": tf, "peak_tflops": FP32_VALU_PEAK_TFLOPS, "frac": tf / FP32_VALU_PEAK_TFLOPS,
                       "algorithmic_flops": flops,
                       "note": "7 dk dv flops per token-head (residual read, decayed rank-1 write, "
                               "output read) against 256 CUs x 64 fp32 FMA lanes x 2 flops x 2.4 GHz"}
    elif w.io_dtype == "f32":
        # the general chunked kernel: chunks of a sequence are dependent and one
        # workgroup fills a CU's LDS
        out["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": gbs / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": nbytes,
                           "kernels": ["chunked_generic_kernel"]}
        out["limited_by"] = "latency (dependent chunks per sequence, one wave per SIMD)"
    elif w.variant == "falcon1a":
        out["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": gbs / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": nbytes,
                           "kernels": ["falcon1a_tile_kernel<false>", "falcon1a_tile_scan_kernel",
                                       "falcon1a_tile_kernel<true>"]}
    profile = {"f1a_chunked_2x12x16384_d64": "falcon1a_chunked_2x12x16384_d64",
               "f2_chunked_8x12x2048_d64": "falcon2_chunked_8x12x2048_d64",
               "f1_chunked_f32_8x12x2048_d64": "falcon1_chunked_f32_8x12x2048_d64"}.get(name)
    return attach_counters(out, profile, ms) if profile else out


def bench_recurrent(name="f1_chunked_8x12x2048_d64", steps=5, warmup=1):
    """The recurrent entry point (falcon_fwd_recurrent: one pass over T per
    sequence with the state on chip) on the headline workload, timed like the
    chunked legs."""
    import torch

    from delta_rule_recurrence_amd import falcon as fb
    from delta_rule_recurrence_amd import inputs as I

    w = I.WORKLOADS[name]
    d = {k: v.cuda() for k, v in I.workload_inputs(w).items()}
    o = torch.empty((w.B, w.H, w.T, w.dv), dtype=torch.bfloat16, device="cuda")
    S_T = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")

    def step():
        fb.falcon_fwd_recurrent(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], variant=w.variant,
                                o=o, S_T=S_T, eps=w.eps, eps_gamma=w.eps_gamma)

    calls = warm(step, warmup)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = algorithmic_bytes(w.B, w.H, w.T, w.dk, w.dv)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"workload": name, "entry": "falcon_fwd_recurrent", "steps": steps, "warmup_calls": calls,
           "us_per_step": ms * 1e3,
           "tokens_per_s": w.B * w.T / (ms * 1e-3), "algorithmic_bytes": nbytes, "hbm_gbs": gbs,
           "hbm_frac": gbs / HBM_PEAK_GBS,
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": nbytes,
                        "kernels": ["recurrent_kernel"]},
           "limited_by": "latency (T dependent steps per sequence)"}
    return attach_counters(out, "falcon1_recurrent_8x12x2048_d64", ms)


def backward_bytes(B, H, T, dk, dv, io_bytes=2):
    """Compulsory HBM bytes of one Falcon-1 backward: read phi(k), phi(q), v and
    dO once (io dtype), beta and lam once, dS_T once; write the float32
    gradients dphi_k, dphi_q, dv, dbeta, dlam once and dS0 once."""
    th = B * H * T
    state = B * H * dk * dv * 4
    return th * ((2 * dk + 2 * dv) * io_bytes + 8) + th * ((2 * dk + dv) * 4 + 8) + 2 * state




def backward_flops(B, H, T, dk=64, dv=64, C=32):
    """Matrix-core flops of the Falcon-1 backward as designed (32-token
    chunks; the products the design forms, counted once whichever matrix
    cores run them: float32, bf16 for products of two bf16 inputs, or bf16
    on a float operand split into three exact parts), per chunk:
      maps:  Gram and M (2 C^2 d), W and U (C^2 (dk + dv)), P, H and G
             (3 C dk dv, dk^2 C for P), Q~ (C^2 dk)
      chains: P S and Lam^T P (2 dk^2 dv)
      chunk: the recomputed Gram and M (W, U and T come from the maps);
             X^ Lam, W S, dO S^T, (X^ Lam) S^T, R Lam^T (5 C dk dv); M^T dO,
             M^T dQ~, dM (2), (dM o D) X and (dM o D)^T Q, T^T dW, T^T dU,
             dA (2), dK X, dK^T X (12 C^2 d).
    Multiply-adds count two flops; VALU work is not counted."""
    nchunks = -(-T // C)
    d = dk
    maps = 2 * C * C * d + C * C * (dk + dv) + dk * dk * C + 2 * C * dk * dv + C * C * dk
    chains = 2 * dk * dk * dv
    chunk = 2 * C * C * d + 5 * C * dk * dv + 12 * C * C * d
    return 2.0 * B * H * nchunks * (maps + chains + chunk)


def bench_backward(name="f1_backward_8x12x2048_d64", steps=10, warmup=2):
    """The Falcon-1 backward (falcon_bwd_chunked) at the training shape, with a
    loss on both the outputs and the final state; inputs, cotangents, gradient
    buffers and workspace resident in HBM, timed with HIP events on the
    launch stream."""
    import torch

    from delta_rule_recurrence_amd import falcon as fb
    from delta_rule_recurrence_amd import inputs as I

    w = I.WORKLOADS[name]
    d = {k: v.cuda() for k, v in I.workload_inputs(w).items()}
    cot = I.make_cotangents(w.B, w.H, w.T, w.dv, seed=w.seed, io_dtype=w.io_dtype, with_state=True)
    cot = {k: v.cuda() for k, v in cot.items()}
    p = fb.make_problem(w.B, w.H, w.T, w.dk, w.dv, variant="falcon1", io_dtype=torch.bfloat16,
                        eps=w.eps, eps_gamma=w.eps_gamma)
    ws = torch.empty(fb.falcon_bwd_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    grads = fb.falcon_bwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], cot["dO"],
                                  dS_T=cot["dS_T"], eps=w.eps, eps_gamma=w.eps_gamma, workspace=ws)

    def step():
        fb.falcon_bwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], cot["dO"],
                              dS_T=cot["dS_T"], eps=w.eps, eps_gamma=w.eps_gamma, grads=grads,
                              workspace=ws)

    calls = warm(step, warmup)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = backward_bytes(w.B, w.H, w.T, w.dk, w.dv)
    gbs = nbytes / (ms * 1e-3) / 1e9
    # the method's work: every product of the forward chunk form yields two
    # products of the same size in reverse mode (one per operand), so twice
    # the forward's algorithmic flops at the backward's chunk size (32)
    flops = 2.0 * algorithmic_flops(w.B, w.H, w.T, w.dk, w.dv, 32)
    design = backward_flops(w.B, w.H, w.T, w.dk, w.dv)
    tflops = flops / (ms * 1e-3) / 1e12
    out = {"workload": name, "steps": steps, "warmup_calls": calls, "us_per_step": ms * 1e3,
            "tokens_per_s": w.B * w.T / (ms * 1e-3), "algorithmic_bytes": nbytes,
            "workspace_bytes": int(ws.numel()), "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": FP32_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tflops / FP32_MFMA_PEAK_TFLOPS,
                         "traffic": None, "algorithmic_flops": flops, "dtype": "f32",
                         "kernels": ["falcon1_bwd_maps_kernel", "falcon1_bwd_chain_kernel",
                                     "falcon1_bwd_chunk_kernel"]},
            "design_flops": design,
            "design_tflops": design / (ms * 1e-3) / 1e12,
            "flops_note": "roofline counts 2x the forward chunk form's algorithmic flops (C = 32); "
                          "design_flops adds the recomputed forward and the chain products the "
                          "implementation runs"}
    return attach_counters(out, "falcon1_backward_8x12x2048_d64", ms)


def oracle_sample(kind, budget_s=3.0):
    """The oracle as it stands, timed on one host core over a bounded sample of
    another workload (a few seconds each), scaled to that workload's unit.
    Returns the bench-line object."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from delta_rule_recurrence_amd import inputs as I
    from oracle import falcon_backward as ob
    from oracle import falcon_oracle as orc

    f = I.as_f64
    with threadpool_limits(limits=1):
        if kind in ("f1a", "f2"):
            name = "f1a_chunked_2x12x16384_d64" if kind == "f1a" else "f2_chunked_8x12x2048_d64"
            w = I.WORKLOADS[name]
            Ts = 2048 if kind == "f1a" else w.T
            d = I.workload_inputs(w)
            t0 = time.perf_counter()
            orc.falcon_forward(w.variant, f(d["phi_k"][:, :, :Ts]), f(d["phi_q"][:, :, :Ts]),
                               f(d["v"][:, :, :Ts]), f(d["beta"][:, :, :Ts]), f(d["lam"][:, :, :Ts]),
                               eps=w.eps, eps_gamma=w.eps_gamma)
            dt = time.perf_counter() - t0
            return {"value": w.B * Ts / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                    "sample": f"all {w.B}x{w.H} sequences, first {Ts} of {w.T} tokens (fp64 numpy)",
                    "seconds": round(dt, 3)}
        if kind == "decode":
            D = I.DECODE
            rows = 64
            S = f(I.random_state((D["B"], D["H"], D["dk"], D["dv"]), seed=D["seed"], scale=0.05)[:rows])
            st = {k: f(v[:rows]) for k, v in I.decode_step_inputs(1, D["B"], D["H"], D["dk"], D["dv"],
                                                                   seed=D["seed"]).items()}
            t0 = time.perf_counter()
            orc.falcon_decode_step("falcon1", S, st["phi_k"], st["phi_q"], st["v"], st["beta"], st["lam"],
                                   eps=D["eps"], eps_gamma=D["eps_gamma"])
            dt = time.perf_counter() - t0
            return {"value": rows / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                    "sample": f"one decode step for {rows} of {D['B']} batch rows x {D['H']} heads (fp64 numpy)",
                    "seconds": round(dt, 4)}
        if kind == "backward":
            w = I.WORKLOADS["f1_backward_8x12x2048_d64"]
            d = I.workload_inputs(w)
            cot = I.make_cotangents(w.B, w.H, w.T, w.dv, seed=w.seed, io_dtype=w.io_dtype, with_state=True)
            hs = 4   # sequences (b = 0, h = 0..3): the oracle keeps every state of the sweep
            sl = (slice(0, 1), slice(0, hs))
            t0 = time.perf_counter()
            ob.falcon1_backward(f(d["phi_k"][sl]), f(d["phi_q"][sl]), f(d["v"][sl]), f(d["beta"][sl]),
                                f(d["lam"][sl]), f(cot["dO"][sl]), eps=w.eps, eps_gamma=w.eps_gamma,
                                dS_T=f(cot["dS_T"][sl]))
            dt = time.perf_counter() - t0
            # tokens/s of the whole batch at this per-sequence rate
            return {"value": hs * w.T / dt / w.H, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                    "sample": f"{hs} of {w.B}x{w.H} sequences x {w.T} tokens (fp64 numpy); value = "
                              f"B*T tokens/s at that per-sequence rate",
                    "seconds": round(dt, 3)}
    raise ValueError(kind)


def measured_peaks():
    """Achievable figures on this machine, next to the published peaks: a plain
    2 GiB device-to-device copy (reads and writes each byte once) and square
    GEMMs through torch (hipBLASLt) in bf16 and fp32."""
    import torch

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    nbytes = 1 << 31
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    t_copy = timed(lambda: b.copy_(a), 10)
    del a, b
    out = {"copy_gbs": 2 * nbytes / t_copy / 1e9}
    for name, dt, n in (("bf16_gemm_tflops", torch.bfloat16, 8192), ("fp32_gemm_tflops", torch.float32, 4096)):
        x = torch.randn(n, n, device="cuda", dtype=dt)
        y = torch.randn(n, n, device="cuda", dtype=dt)
        t = timed(lambda: torch.mm(x, y), 10)
        out[name] = 2 * n ** 3 / t / 1e12
        del x, y
    out["note"] = ("copy = 2 x bytes / time; GEMMs through torch.mm (hipBLASLt), "
                   "bf16 8192^3 and fp32 4096^3")
    return out


def calibrate_copy(nbytes=1 << 28, reps=5):
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE /
    WRITE_SIZE counters (each copy reads and writes nbytes once)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_per_copy": nbytes, "copies": reps}))


def _oracle_slice(args):
    """Pool worker: the oracle on sequences [lo, hi) of a workload (inputs
    regenerated from the seed, not timed), started after a barrier so that
    all workers compute at once.  Returns (start, end) wall-clock times."""
    name, lo, hi, Ts = args
    from threadpoolctl import threadpool_limits

    from delta_rule_recurrence_amd import inputs as I
    from oracle import falcon_oracle as orc

    w = I.WORKLOADS[name]
    d = I.workload_inputs(w)
    f = I.as_f64
    sl = {k: f(v.reshape((w.B * w.H,) + tuple(v.shape[2:]))[lo:hi, :Ts]) for k, v in d.items()}
    _POOL_BARRIER.wait(timeout=300)
    with threadpool_limits(limits=1):
        t0 = time.time()
        orc.falcon_forward(w.variant, sl["phi_k"], sl["phi_q"], sl["v"], sl["beta"], sl["lam"],
                           eps=w.eps, eps_gamma=w.eps_gamma)
        t1 = time.time()
    return t0, t1


_POOL_BARRIER = None


def make_oracle_pool():
    """A process pool for the all-core oracle run, forked before this process
    touches the GPU (the workers only run numpy).  Sized to the host share of
    one GPU (at most 16 workers)."""
    import multiprocessing as mp
    global _POOL_BARRIER
    n = max(1, min(16, os.cpu_count() or 1))
    ctx = mp.get_context("fork")
    _POOL_BARRIER = ctx.Barrier(n)
    return ctx.Pool(n), n


def cpu_baseline(d, w, o_gpu, S_gpu, pool=None, nproc=1):
    """The oracle as it stands, timed on the host over the same workload (all
    sequences, all tokens): once on one thread, and once split over (batch,
    head) across `nproc` worker processes (every core of the host share)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from delta_rule_recurrence_amd import inputs as I
    from oracle import falcon_oracle as orc

    Ts = w.T
    f = I.as_f64
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O, S = orc.falcon_forward(w.variant, f(d["phi_k"][:, :, :Ts]), f(d["phi_q"][:, :, :Ts]),
                                  f(d["v"][:, :, :Ts]), f(d["beta"][:, :, :Ts]),
                                  f(d["lam"][:, :, :Ts]), eps=w.eps, eps_gamma=w.eps_gamma)
        dt = time.perf_counter() - t0
    ref = np.asarray(O)
    got = o_gpu[:, :, :Ts].float().cpu().numpy()
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    one = {"value": w.B * Ts / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
           "sample": f"the whole workload: all {w.B}x{w.H} sequences x {Ts} tokens (fp64 numpy, 1 thread)",
           "seconds": round(dt, 3), "rel_l2_o_vs_gpu": rel}
    if pool is None or nproc <= 1:
        one["os_cpu_count"] = os.cpu_count()
        return one
    n_seq = w.B * w.H
    bounds = [(i * n_seq) // nproc for i in range(nproc + 1)]
    spans = pool.map(_oracle_slice, [(w.name, bounds[i], bounds[i + 1], Ts) for i in range(nproc)])
    wall = max(e for _, e in spans) - min(s for s, _ in spans)
    return {"value": w.B * Ts / wall, "unit": "tokens/s", "cores": nproc, "kind": "oracle",
            "sample": f"the whole workload: all {w.B}x{w.H} sequences x {Ts} tokens (fp64 numpy), "
                      f"sequences split over {nproc} worker processes, one thread each",
            "seconds": round(wall, 3), "os_cpu_count": os.cpu_count(), "single_core": one}


# Other workloads that --leg runs alone (for profiling): name -> fn(steps, warmup)
LEGS = {
    "decode": lambda steps, warmup: bench_decode(warmup=warmup),
    "f1a": lambda steps, warmup: bench_chunked_workload("f1a_chunked_2x12x16384_d64", steps, warmup),
    "f2": lambda steps, warmup: bench_chunked_workload("f2_chunked_8x12x2048_d64", steps, warmup),
    "f32": lambda steps, warmup: bench_chunked_workload("f1_chunked_f32_8x12x2048_d64", steps, warmup),
    "recurrent": lambda steps, warmup: bench_recurrent(steps=steps, warmup=warmup),
    "backward": lambda steps, warmup: bench_backward(steps=steps, warmup=warmup),
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (Falcon-1A 2x12x16384, Falcon-2 8x12x2048, "
                         "the Falcon-1 backward 8x12x2048, the recurrent entry point)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain copy of known size (for PMC counter scaling)")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time the Falcon-1 backward leg (--steps calls), for profiling")
    ap.add_argument("--leg", choices=sorted(LEGS),
                    help="only time this other workload (--steps calls after --warmup), for profiling")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the copy and GEMM reference rates (for profiling the headline step)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the Falcon forward "
              "shards by (batch, head) with no communication, so there is no multi-GPU path here.",
              file=sys.stderr)
        sys.exit(2)

    # the all-core oracle pool is forked before anything touches the GPU
    pool, nproc = (None, 1)
    if not args.no_cpu_baseline and not (args.calibrate_copy or args.backward_only):
        pool, nproc = make_oracle_pool()

    import torch

    from delta_rule_recurrence_amd import falcon as fb
    from delta_rule_recurrence_amd import inputs as I

    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.backward_only:
        print(json.dumps({"f1_backward": bench_backward(steps=args.steps, warmup=1)}))
        return
    if args.leg:
        print(json.dumps({args.leg: LEGS[args.leg](args.steps, args.warmup)}))
        return
    w = I.WORKLOADS[WORKLOAD]
    d = I.workload_inputs(w)
    dev = {k: v.cuda() for k, v in d.items()}
    o = torch.empty((w.B, w.H, w.T, w.dv), dtype=torch.bfloat16, device="cuda")
    S_T = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    p = fb.make_problem(w.B, w.H, w.T, w.dk, w.dv, variant=w.variant, io_dtype=torch.bfloat16,
                        eps=w.eps, eps_gamma=w.eps_gamma)
    ws_bytes = fb.falcon_workspace_bytes(p, w.C)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def step():
        fb.falcon_fwd_chunked(dev["phi_k"], dev["phi_q"], dev["v"], dev["beta"], dev["lam"],
                              variant=w.variant, C=w.C, o=o, S_T=S_T, workspace=ws)

    # the copy and GEMM reference rates are measured first: about a second of
    # GPU work, after which the clocks have ramped up for the timed steps
    peaks = None if args.no_peaks else measured_peaks()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = max(wall * 1e3 / args.steps, ev_ms)

    tokens = w.B * w.T
    bytes_alg = algorithmic_bytes(w.B, w.H, w.T, w.dk, w.dv)
    flops_alg = algorithmic_flops(w.B, w.H, w.T, w.dk, w.dv, w.C)
    # The step is the two launches back to back on one stream; the event time
    # brackets both, and the roofline is taken over the whole step.
    achieved_gbs = bytes_alg / (ev_ms * 1e-3) / 1e9
    traffic, mfma_counters = counter_fields("falcon1_chunked_8x12x2048_d64", ev_ms)
    line = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/8 features and values, sigmoid/softplus gates)",
        "config": {"workload": WORKLOAD, "variant": w.variant, "B": w.B, "H": w.H, "T": w.T,
                   "dk": w.dk, "dv": w.dv, "C": w.C, "io": "bf16", "state": "f32"},
        # algorithmic flops of the chunk form (not a counter) over the step time
        "mfma_pct_of_peak_algorithmic": 100.0 * flops_alg / (ev_ms * 1e-3) / (BF16_MFMA_PEAK_TFLOPS * 1e12),
        # flops the matrix cores executed (rocprofv3 SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, committed
        # summary) over the step time
        "mfma_pct_of_peak_counters": None if mfma_counters is None else mfma_counters["bf16_pct_of_peak"],
        "mfma_counters": mfma_counters,
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": bytes_alg, "kernel_ms": ev_ms, "kernels": STEP_KERNELS},
    }
    if peaks:
        line["measured_peaks"] = peaks
        line["roofline"]["frac_of_measured_copy"] = achieved_gbs / peaks["copy_gbs"]
    if not args.no_decode:
        line["decode"] = bench_decode()
    if not args.no_extra:
        line["f1a_chunked"] = bench_chunked_workload("f1a_chunked_2x12x16384_d64")
        line["f2_chunked"] = bench_chunked_workload("f2_chunked_8x12x2048_d64", steps=100, warmup=1)
        line["f1_backward"] = bench_backward()
        rb = line["f1_backward"]["roofline"]
        if peaks:
            rb["frac_of_measured_fp32_gemm"] = rb["achieved"] / peaks["fp32_gemm_tflops"]
        line["f1_recurrent"] = bench_recurrent(steps=20)
        line["f1_chunked_f32"] = bench_chunked_workload("f1_chunked_f32_8x12x2048_d64", steps=20, warmup=1)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(d, w, o, S_T, pool, nproc)
        pool.close()
        pool.join()
        # the oracle beside every other workload, on a bounded sample each
        if not args.no_decode:
            line["decode"]["cpu_oracle"] = oracle_sample("decode")
        if not args.no_extra:
            line["f1a_chunked"]["cpu_oracle"] = oracle_sample("f1a")
            line["f2_chunked"]["cpu_oracle"] = oracle_sample("f2")
            line["f1_backward"]["cpu_oracle"] = oracle_sample("backward")
            # the recurrent entry point computes the headline workload: same oracle figure
            line["f1_recurrent"]["cpu_oracle"] = dict(line["cpu_baseline"]["single_core"]
                                                      if "single_core" in line["cpu_baseline"]
                                                      else line["cpu_baseline"])
            # the same recurrence in float32 I/O (the oracle computes in fp64 either way)
            line["f1_chunked_f32"]["cpu_oracle"] = dict(line["f1_recurrent"]["cpu_oracle"])
    print(json.dumps(line))


if __name__ == "__main__":
    main()
