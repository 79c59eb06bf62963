"""Long sequences on the fast paths and the recurrent entry point, against
the oracle: Falcon-2 and Falcon-2A chunked (bf16, d = 64, C = 64; 128 chunks
per sequence through the per-column kernel's two row buffers), Falcon-1A
chunked (tiles, scan and output sweep over 64 tiles of one sequence) and the
recurrent form of Falcon-1, each with a carried state and previous key
("Fast Weight Attention for Continual Learning", Section 4 rules; Section
4.2 chunk-parallel form).  Tolerance: the bf16 bar (2e-2 relative L2) on the
whole output and final state and on every sequence."""

import numpy as np
import pytest
import torch

from delta_rule_recurrence_amd import falcon as fb
from delta_rule_recurrence_amd import inputs as I

from gpu_utils import TOL, check, oracle_forward, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    "falcon2_chunked": ("falcon2", "chunked", 1, 2, 8192),
    "falcon2a_chunked": ("falcon2a", "chunked", 2, 1, 8000),
    "falcon1a_chunked": ("falcon1a", "chunked", 1, 1, 32768),
    "falcon1_recurrent": ("falcon1", "recurrent", 1, 2, 16384),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_long_sequence(name):
    variant, entry, B, H, T = CASES[name]
    print(f"[long] {name}: B={B} H={H} T={T}", flush=True)
    x = I.make_inputs(B, H, T, 64, 64, seed=2600 + T, io_dtype="bf16",
                      per_column_beta=variant in ("falcon2", "falcon2a"))
    g = np.random.default_rng([T, 11])
    S0 = torch.from_numpy((0.1 * g.standard_normal((B, H, 64, 64))).astype(np.float32))
    k_prev = torch.from_numpy((g.standard_normal((B, H, 64)) / 8).astype(np.float32)).to(torch.bfloat16)
    O_ref, S_ref = oracle_forward(variant, x, S0=S0, k_prev=k_prev)
    d = to_dev(x)
    kw = dict(variant=variant, S0=S0.cuda(), k_prev=k_prev.cuda())
    if entry == "chunked":
        o, S_T = fb.falcon_fwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], C=64, **kw)
    else:
        o, S_T = fb.falcon_fwd_recurrent(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], **kw)
    torch.cuda.synchronize()
    eo, es = check(o, S_T, O_ref, S_ref, TOL["bf16"], name)
    print(f"[long] {name}: rel L2 o={eo:.3e} S_T={es:.3e}", flush=True)
