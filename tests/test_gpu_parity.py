"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on
identical seeded inputs, element by element (relative L2 over the whole
tensor, per the stated tolerances: 1e-4 for float32 I/O, 2e-2 for bf16 I/O
with the float32 state)."""

import numpy as np
import pytest
import torch

from delta_rule_recurrence_amd import falcon as fb
from delta_rule_recurrence_amd import inputs as I

from gpu_utils import TOL, check, oracle_forward, rel_l2, to_dev

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _run(entry, d, variant, C=64, S0=None, k_prev=None, **kw):
    if entry == "recurrent":
        return fb.falcon_fwd_recurrent(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"],
                                       variant=variant, S0=S0, k_prev=k_prev, **kw)
    return fb.falcon_fwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"],
                                 variant=variant, C=C, S0=S0, k_prev=k_prev, **kw)


# ---- the tiny float32 workload (1 x 1 x 64, d = 16, C = 16, seed 0) ---------

@pytest.mark.parametrize("entry", ["recurrent", "chunked"])
def test_tiny_f32_workload(entry):
    w = I.WORKLOADS["f1_recurrent_tiny"]
    d = I.workload_inputs(w)
    O_ref, S_ref = oracle_forward(w.variant, d)
    o, S_T = _run(entry, to_dev(d), w.variant, C=w.C)
    torch.cuda.synchronize()
    check(o, S_T, O_ref, S_ref, TOL["f32"], f"{entry} tiny")


# ---- small shapes: every variant, dtype, width, chunk, ragged T -------------

SMALL = [
    # (variant, io, B, H, T, dk, dv, C)
    ("falcon1", "f32", 2, 3, 100, 16, 16, 16),
    ("falcon1", "f32", 1, 2, 77, 32, 64, 32),
    ("falcon1", "f32", 2, 2, 130, 64, 64, 64),
    ("falcon1", "bf16", 2, 2, 130, 64, 64, 64),
    ("falcon1", "bf16", 1, 3, 200, 128, 128, 64),
    ("falcon1", "bf16", 1, 2, 67, 128, 32, 16),
    ("falcon1a", "f32", 2, 2, 90, 64, 64, 32),
    ("falcon1a", "bf16", 2, 3, 150, 64, 64, 64),
    ("falcon2", "f32", 2, 2, 90, 32, 32, 16),
    ("falcon2", "bf16", 2, 3, 150, 64, 64, 64),
    ("falcon2a", "f32", 1, 2, 70, 64, 16, 32),
    ("falcon2a", "bf16", 2, 2, 65, 64, 64, 64),
]


@pytest.mark.parametrize("entry", ["recurrent", "chunked"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_small_shapes(entry, case):
    variant, io, B, H, T, dk, dv, C = case
    d = I.make_inputs(B, H, T, dk, dv, seed=100 + T, io_dtype=io,
                      per_column_beta=variant in ("falcon2", "falcon2a"))
    O_ref, S_ref = oracle_forward(variant, d)
    o, S_T = _run(entry, to_dev(d), variant, C=C)
    torch.cuda.synchronize()
    check(o, S_T, O_ref, S_ref, TOL[io], f"{entry} {case}")


@pytest.mark.parametrize("entry", ["recurrent", "chunked"])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_carried_state_and_continuation(entry, io):
    """A run split at T1 with (S_T1, phi(k_T1)) handed over equals one run,
    and a carried state without k_prev uses the fresh-start boundary."""
    B, H, T, dk, dv, T1 = 2, 3, 150, 64, 64, 70
    d = I.make_inputs(B, H, T, dk, dv, seed=7, io_dtype=io)
    S0 = I.random_state((B, H, dk, dv), seed=8)
    O_ref, S_ref = oracle_forward("falcon1", d, S0=S0)
    dd = to_dev(d)
    o, S_T = _run(entry, dd, "falcon1", S0=S0.cuda())
    torch.cuda.synchronize()
    check(o, S_T, O_ref, S_ref, TOL[io], f"{entry} carried S0")
    first = {k: v[:, :, :T1].contiguous() for k, v in dd.items()}
    second = {k: v[:, :, T1:].contiguous() for k, v in dd.items()}
    o1, S1 = _run(entry, first, "falcon1", S0=S0.cuda())
    kp = dd["phi_k"][:, :, T1 - 1].contiguous()
    o2, S2 = _run(entry, second, "falcon1", S0=S1, k_prev=kp)
    torch.cuda.synchronize()
    check(torch.cat([o1, o2], dim=2), S2, O_ref, S_ref, TOL[io], f"{entry} split")


@pytest.mark.parametrize("entry", ["recurrent", "chunked"])
def test_state_in_place_and_optional_outputs(entry):
    B, H, T, dk, dv = 1, 2, 40, 32, 32
    d = to_dev(I.make_inputs(B, H, T, dk, dv, seed=9, io_dtype="f32"))
    S = I.random_state((B, H, dk, dv), seed=10).cuda()
    O_ref, S_ref = oracle_forward("falcon1", {k: v.cpu() for k, v in d.items()}, S0=S.cpu())
    o, S_T = _run(entry, d, "falcon1", C=16, S0=S, S_T=S)   # S_T aliases S0
    torch.cuda.synchronize()
    check(o, S, O_ref, S_ref, TOL["f32"], f"{entry} in place")
    o2, none = _run(entry, d, "falcon1", C=16, S0=None, return_state=False)
    torch.cuda.synchronize()
    assert none is None
    O_ref2, _ = oracle_forward("falcon1", {k: v.cpu() for k, v in d.items()})
    assert rel_l2(o2.cpu().numpy(), O_ref2) <= TOL["f32"]


def test_empty_sequence_copies_state():
    B, H, dk, dv = 2, 2, 16, 16
    d = to_dev(I.make_inputs(B, H, 1, dk, dv, seed=11, io_dtype="f32"))
    d = {k: v[:, :, :0].contiguous() for k, v in d.items()}
    S0 = I.random_state((B, H, dk, dv), seed=12).cuda()
    for entry in ("recurrent", "chunked"):
        o, S_T = _run(entry, d, "falcon1", C=16, S0=S0)
        torch.cuda.synchronize()
        assert o.numel() == 0
        assert torch.equal(S_T, S0)


def test_chunk_size_invariance():
    B, H, T, dk, dv = 2, 3, 256, 64, 64
    d = to_dev(I.make_inputs(B, H, T, dk, dv, seed=13, io_dtype="f32"))
    outs = [fb.falcon_fwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], C=C)
            for C in (16, 32, 64)]
    torch.cuda.synchronize()
    for o, s in outs[1:]:
        assert rel_l2(o.cpu().numpy(), outs[0][0].cpu().numpy()) <= 1e-5
        assert rel_l2(s.cpu().numpy(), outs[0][1].cpu().numpy()) <= 1e-5


def test_clamp_active_stress():
    """beta near 2, large lam and tiny keys: the positive-decay clamp and
    gamma = eps_gamma are exercised on every path."""
    B, H, T, dk, dv = 1, 2, 96, 32, 32
    d = I.make_inputs(B, H, T, dk, dv, seed=14, io_dtype="f32", feature_scale=0.01)
    d["beta"] = torch.full_like(d["beta"], 1.9)
    d["lam"] = torch.full_like(d["lam"], 10.0)
    O_ref, S_ref = oracle_forward("falcon1", d, eps_gamma=1e-3)
    for entry in ("recurrent", "chunked"):
        o, S_T = _run(entry, to_dev(d), "falcon1", C=32, eps_gamma=1e-3)
        torch.cuda.synchronize()
        check(o, S_T, O_ref, S_ref, TOL["f32"], f"{entry} clamp")


def test_nan_propagates_without_hang():
    B, H, T, dk, dv = 1, 1, 64, 16, 16
    d = I.make_inputs(B, H, T, dk, dv, seed=15, io_dtype="f32")
    d["lam"][0, 0, 20] = float("nan")
    for entry in ("recurrent", "chunked"):
        o, S_T = _run(entry, to_dev(d), "falcon1", C=16)
        torch.cuda.synchronize()
        assert torch.isnan(o[0, 0, 20:]).any()
        assert torch.isfinite(o[0, 0, :20]).all()


# ---- Falcon-1A chunk tiles (bf16, d = 64, C = 64): tile aggregates, scan, sweep ---

@pytest.mark.parametrize("B,H,T", [(1, 1, 4096), (2, 3, 805), (3, 2, 1000), (1, 2, 256)])
def test_falcon1a_tiles(B, H, T):
    """Many tiles per sequence (a deep look-back chain), ragged tails and a
    sequence that is exactly one tile."""
    d = I.make_inputs(B, H, T, 64, 64, seed=300 + T, io_dtype="bf16")
    O_ref, S_ref = oracle_forward("falcon1a", d)
    o, S_T = _run("chunked", to_dev(d), "falcon1a")
    torch.cuda.synchronize()
    check(o, S_T, O_ref, S_ref, TOL["bf16"], f"falcon1a tiles {B}x{H}x{T}")


def test_falcon1a_tiles_carried_state_and_continuation():
    B, H, T, T1 = 2, 2, 1300, 517
    d = I.make_inputs(B, H, T, 64, 64, seed=21, io_dtype="bf16")
    S0 = I.random_state((B, H, 64, 64), seed=22)
    O_ref, S_ref = oracle_forward("falcon1a", d, S0=S0)
    dd = to_dev(d)
    o, S_T = _run("chunked", dd, "falcon1a", S0=S0.cuda())
    torch.cuda.synchronize()
    check(o, S_T, O_ref, S_ref, TOL["bf16"], "falcon1a tiles carried S0")
    first = {k: v[:, :, :T1].contiguous() for k, v in dd.items()}
    second = {k: v[:, :, T1:].contiguous() for k, v in dd.items()}
    o1, S1 = _run("chunked", first, "falcon1a", S0=S0.cuda())
    kp = dd["phi_k"][:, :, T1 - 1].contiguous()
    o2, S2 = _run("chunked", second, "falcon1a", S0=S1, k_prev=kp)
    torch.cuda.synchronize()
    check(torch.cat([o1, o2], dim=2), S2, O_ref, S_ref, TOL["bf16"], "falcon1a tiles split")


def test_falcon1a_tiles_repeatable():
    """Two calls on one workspace give the same bits: no state from the
    previous call survives in the workspace, and the tile scan has a fixed
    order."""
    d = to_dev(I.make_inputs(2, 2, 900, 64, 64, seed=23, io_dtype="bf16"))
    p = fb.make_problem(2, 2, 900, 64, 64, variant="falcon1a", io_dtype=torch.bfloat16)
    ws = torch.full((fb.falcon_workspace_bytes(p, 64),), 0x7f, dtype=torch.uint8, device="cuda")
    o1, s1 = _run("chunked", d, "falcon1a", workspace=ws)
    o2, s2 = _run("chunked", d, "falcon1a", workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


# ---- Falcon-1 chunk matrices and chain (bf16, d = 64, C = 64) ------------------

@pytest.mark.parametrize("B,H,T", [(1, 1, 64), (3, 5, 1000), (2, 7, 4100), (1, 9, 129)])
def test_falcon1_chunk_maps(B, H, T):
    """Falcon-1 bf16 d=64: chunk-parallel chunk matrices and the chain.
    Covers a single chunk, ragged tails, many chunks per sequence, and
    batch x head counts that leave part of the last group of eight
    sequences empty."""
    d = I.make_inputs(B, H, T, 64, 64, seed=400 + T, io_dtype="bf16")
    O_ref, S_ref = oracle_forward("falcon1", d)
    o, S_T = _run("chunked", to_dev(d), "falcon1")
    torch.cuda.synchronize()
    check(o, S_T, O_ref, S_ref, TOL["bf16"], f"falcon1 chunk maps {B}x{H}x{T}")


def test_falcon1_chunk_maps_carried_state_and_continuation():
    B, H, T, T1 = 2, 3, 1300, 517
    d = I.make_inputs(B, H, T, 64, 64, seed=31, io_dtype="bf16")
    S0 = I.random_state((B, H, 64, 64), seed=32)
    O_ref, S_ref = oracle_forward("falcon1", d, S0=S0)
    dd = to_dev(d)
    o, S_T = _run("chunked", dd, "falcon1", S0=S0.cuda())
    torch.cuda.synchronize()
    check(o, S_T, O_ref, S_ref, TOL["bf16"], "falcon1 chunk maps carried S0")
    first = {k: v[:, :, :T1].contiguous() for k, v in dd.items()}
    second = {k: v[:, :, T1:].contiguous() for k, v in dd.items()}
    o1, S1 = _run("chunked", first, "falcon1", S0=S0.cuda())
    kp = dd["phi_k"][:, :, T1 - 1].contiguous()
    o2, S2 = _run("chunked", second, "falcon1", S0=S1, k_prev=kp)
    torch.cuda.synchronize()
    check(torch.cat([o1, o2], dim=2), S2, O_ref, S_ref, TOL["bf16"], "falcon1 chunk maps split")


def test_falcon1_chunk_maps_repeatable():
    """Two calls on one workspace prefilled with garbage give the same bits."""
    d = to_dev(I.make_inputs(3, 3, 700, 64, 64, seed=33, io_dtype="bf16"))
    p = fb.make_problem(3, 3, 700, 64, 64, variant="falcon1", io_dtype=torch.bfloat16)
    ws = torch.full((fb.falcon_workspace_bytes(p, 64),), 0x7f, dtype=torch.uint8, device="cuda")
    o1, s1 = _run("chunked", d, "falcon1", workspace=ws)
    o2, s2 = _run("chunked", d, "falcon1", workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


# ---- per-column rules (Falcon-2 / 2A, bf16, d = 64, C = 64) --------------------

@pytest.mark.parametrize("variant", ["falcon2", "falcon2a"])
def test_per_column_carried_state_and_continuation(variant):
    B, H, T, T1 = 2, 2, 300, 130
    d = I.make_inputs(B, H, T, 64, 64, seed=31, io_dtype="bf16", per_column_beta=True)
    S0 = I.random_state((B, H, 64, 64), seed=32)
    O_ref, S_ref = oracle_forward(variant, d, S0=S0)
    dd = to_dev(d)
    o, S_T = _run("chunked", dd, variant, S0=S0.cuda())
    torch.cuda.synchronize()
    check(o, S_T, O_ref, S_ref, TOL["bf16"], f"{variant} carried S0")
    first = {k: v[:, :, :T1].contiguous() for k, v in dd.items()}
    second = {k: v[:, :, T1:].contiguous() for k, v in dd.items()}
    o1, S1 = _run("chunked", first, variant, S0=S0.cuda())
    kp = dd["phi_k"][:, :, T1 - 1].contiguous()
    o2, S2 = _run("chunked", second, variant, S0=S1, k_prev=kp)
    torch.cuda.synchronize()
    check(torch.cat([o1, o2], dim=2), S2, O_ref, S_ref, TOL["bf16"], f"{variant} split")


def test_per_column_clamp_active():
    """Large gains and ridge weights with small keys drive the per-column decay
    onto its positive clamp."""
    B, H, T = 1, 2, 200
    d = I.make_inputs(B, H, T, 64, 64, seed=33, io_dtype="bf16", per_column_beta=True,
                      feature_scale=0.05)
    d["beta"] = 1.0 + 0.9 * torch.rand(d["beta"].shape, generator=torch.Generator().manual_seed(34))
    d["lam"] = torch.full_like(d["lam"], 5.0)
    O_ref, S_ref = oracle_forward("falcon2", d, eps_gamma=1e-3)
    o, S_T = _run("chunked", to_dev(d), "falcon2", eps_gamma=1e-3)
    torch.cuda.synchronize()
    check(o, S_T, O_ref, S_ref, TOL["bf16"], "falcon2 clamp")


# ---- decode ------------------------------------------------------------------

@pytest.mark.parametrize("variant", ["falcon1", "falcon1a", "falcon2", "falcon2a"])
@pytest.mark.parametrize("io,dk,dv", [("f32", 16, 16), ("bf16", 64, 128), ("bf16", 128, 128),
                                      ("f32", 128, 32)])
def test_decode_steps_match_forward(variant, io, dk, dv):
    B, H, T = 3, 2, 12
    per_col = variant in ("falcon2", "falcon2a")
    d = I.make_inputs(B, H, T, dk, dv, seed=16, io_dtype=io, per_column_beta=per_col)
    O_ref, S_ref = oracle_forward(variant, d)
    dd = to_dev(d)
    S = torch.zeros((B, H, dk, dv), dtype=torch.float32, device="cuda")
    first = torch.ones(B, dtype=torch.uint8, device="cuda")
    outs = []
    for t in range(T):
        x = torch.zeros_like(dd["phi_k"][:, :, 0]) if t == 0 else dd["phi_k"][:, :, t - 1].contiguous()
        beta = dd["beta"][:, :, t].contiguous()
        outs.append(fb.falcon_decode_step(x, dd["phi_q"][:, :, t].contiguous(),
                                          dd["v"][:, :, t].contiguous(), beta,
                                          dd["lam"][:, :, t].contiguous(), S, variant=variant,
                                          is_first=first if t == 0 else None))
    torch.cuda.synchronize()
    check(torch.stack(outs, dim=2), S, O_ref, S_ref, TOL[io], f"decode {variant}")


# ---- sequences shorter than a staged block or a chunk -------------------------

@pytest.mark.parametrize("entry", ["recurrent", "chunked"])
@pytest.mark.parametrize("case", [("falcon1", "bf16", 1, 64, 64), ("falcon1", "f32", 5, 16, 16),
                                  ("falcon1a", "bf16", 17, 64, 64), ("falcon2", "f32", 33, 32, 64),
                                  ("falcon2a", "bf16", 5, 128, 32), ("falcon1", "bf16", 17, 128, 128)],
                         ids=lambda c: "-".join(map(str, c)))
def test_short_sequences(entry, case):
    """T below the recurrent form's 16/32-token staging block and the 64-token
    chunk (the first block is also the ragged last one), with a carried state
    and a previous key."""
    variant, io, T, dk, dv = case
    B, H = 2, 3
    per_col = variant in ("falcon2", "falcon2a")
    d = I.make_inputs(B, H, T, dk, dv, seed=200 + T, io_dtype=io, per_column_beta=per_col)
    S0 = I.random_state((B, H, dk, dv), seed=201)
    kp = I.make_inputs(B, H, 1, dk, dv, seed=202, io_dtype=io)["phi_k"][:, :, 0].contiguous()
    O_ref, S_ref = oracle_forward(variant, d, S0=S0, k_prev=kp)
    o, S_T = _run(entry, to_dev(d), variant, C=64 if dk == 64 and dv == 64 else 16, S0=S0.cuda(),
                  k_prev=kp.cuda())
    torch.cuda.synchronize()
    check(o, S_T, O_ref, S_ref, TOL[io], f"{entry} short {case}")


# ---- general chunked kernel: every value-tile width ---------------------------

# The general kernel narrows its value tile (64 -> 32 -> 16 columns) while the
# narrower tiles still give no more workgroups than the 256 CUs, so small
# batches run 16-column tiles; these batches keep 32- and 64-column tiles
# (and the LDS-driven 32-column tile of a per-column rule at dk = dv = 128).
GENERAL_TILES = [
    # (variant, io, B, H, T, dk, dv, C)                    value tile
    ("falcon1", "f32", 8, 12, 130, 64, 64, 64),            # 32: B*H = 96
    ("falcon2", "f32", 8, 12, 100, 64, 64, 32),            # 32
    ("falcon1a", "bf16", 16, 16, 70, 64, 64, 32),          # 64: B*H = 256
    ("falcon2a", "f32", 16, 16, 50, 32, 64, 16),           # 64, dk = 32
    ("falcon1", "bf16", 4, 40, 90, 128, 64, 32),           # 64, dk = 128 (two key-row groups)
    ("falcon2", "bf16", 2, 64, 40, 128, 128, 64),          # 32 (LDS), two tiles per sequence
    ("falcon1", "f32", 4, 40, 70, 128, 64, 64),            # 64: the largest LDS footprint (150 KB)
]


@pytest.mark.parametrize("case", GENERAL_TILES, ids=lambda c: "-".join(map(str, c)))
def test_general_kernel_value_tiles(case):
    variant, io, B, H, T, dk, dv, C = case
    per_col = variant in ("falcon2", "falcon2a")
    d = I.make_inputs(B, H, T, dk, dv, seed=300 + T, io_dtype=io, per_column_beta=per_col)
    S0 = I.random_state((B, H, dk, dv), seed=301)
    kp = I.make_inputs(B, H, 1, dk, dv, seed=302, io_dtype=io)["phi_k"][:, :, 0].contiguous()
    O_ref, S_ref = oracle_forward(variant, d, S0=S0, k_prev=kp)
    o, S_T = _run("chunked", to_dev(d), variant, C=C, S0=S0.cuda(), k_prev=kp.cuda())
    torch.cuda.synchronize()
    check(o, S_T, O_ref, S_ref, TOL[io], f"general tiles {case}")
