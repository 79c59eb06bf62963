"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments with the documented status
before launching anything.  Only argument-validation paths are exercised
here (fake device addresses are never dereferenced)."""

import ctypes
import os
import re
import subprocess

import pytest

from delta_rule_recurrence_amd import falcon as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "falcon.h")

OK, NULL, SHAPE, DTYPE, CHUNK, ALIGN, WORKSPACE, VARIANT, HIP, VALUE, ALIAS = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(falcon_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return fb.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"falcon_fwd_recurrent", "falcon_fwd_chunked", "falcon_decode_step"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", fb.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\w+)$", out, flags=re.M))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_abi_version_and_strings(lib):
    assert fb.falcon_abi_version() == 1
    for s in (OK, NULL, SHAPE, DTYPE, CHUNK, ALIGN, WORKSPACE, VARIANT, HIP, VALUE, ALIAS):
        txt = fb.falcon_status_string(s)
        assert txt and txt != "unknown falcon_status"
    assert fb.falcon_status_string(12345) == "unknown falcon_status"


# Fake, 16-byte aligned, non-overlapping "device" addresses.
BASE = 1 << 40
STRIDE = 1 << 32


def fake(i, misalign=0):
    return ctypes.c_void_p(BASE + i * STRIDE + misalign)


def prob(**kw):
    d = dict(B=2, H=3, T=40, dk=64, dv=64, variant="falcon1", io_dtype=None, eps=1e-6, eps_gamma=1e-6)
    d.update(kw)
    import torch
    p = fb.FalconProblem(d["B"], d["H"], d["T"], d["dk"], d["dv"],
                         fb.VARIANTS[d["variant"]] if isinstance(d["variant"], str) else d["variant"],
                         1 if d["io_dtype"] is None else d["io_dtype"], d["eps"], d["eps_gamma"])
    return p


def fwd_args(**over):
    a = dict(k=fake(0), q=fake(1), v=fake(2), beta=fake(3), lam=fake(4), S0=None, kp=None,
             o=fake(5), ST=fake(6))
    a.update(over)
    return a


def call_chunked(lib, p, C=64, ws=None, wsb=0, **over):
    a = fwd_args(**over)
    return lib.falcon_fwd_chunked(ctypes.byref(p) if p is not None else None, a["k"], a["q"], a["v"],
                                  a["beta"], a["lam"], a["S0"], a["kp"], a["o"], a["ST"], C, ws, wsb,
                                  None)


def call_recurrent(lib, p, **over):
    a = fwd_args(**over)
    return lib.falcon_fwd_recurrent(ctypes.byref(p) if p is not None else None, a["k"], a["q"],
                                    a["v"], a["beta"], a["lam"], a["S0"], a["kp"], a["o"], a["ST"],
                                    None)


@pytest.mark.parametrize("call", ["chunked", "recurrent"])
def test_problem_validation(lib, call):
    f = (lambda p, **kw: call_chunked(lib, p, **kw)) if call == "chunked" else (
        lambda p, **kw: call_recurrent(lib, p, **kw))
    assert f(None) == NULL
    assert f(prob(dk=48)) == SHAPE
    assert f(prob(dv=256)) == SHAPE
    assert f(prob(B=-1)) == SHAPE
    assert f(prob(T=-5)) == SHAPE
    assert f(prob(variant=0)) == VARIANT
    assert f(prob(variant=5)) == VARIANT
    assert f(prob(io_dtype=7)) == DTYPE
    assert f(prob(eps=-1.0)) == VALUE
    assert f(prob(eps=float("nan"))) == VALUE
    assert f(prob(eps_gamma=0.0)) == VALUE
    assert f(prob(eps_gamma=1.0)) == VALUE
    for name in ("k", "q", "v", "beta", "lam", "o"):
        assert f(prob(), **{name: None}) == NULL, name
    for i, name in enumerate(("k", "q", "v", "beta", "lam", "o", "ST")):
        assert f(prob(), **{name: fake(i, misalign=4)}) == ALIGN, name
    assert f(prob(), S0=fake(8, misalign=8)) == ALIGN
    assert f(prob(), kp=fake(9, misalign=2)) == ALIGN


def test_alias_detection(lib):
    p = prob()
    # o overlapping v, or overlapping phi_k by a partial range
    assert call_chunked(lib, p, o=fake(2)) == ALIAS
    assert call_chunked(lib, p, o=ctypes.c_void_p(BASE + 64)) == ALIAS
    # S_T may alias S0 exactly, but not an input
    assert call_chunked(lib, prob(T=0), S0=fake(7), ST=fake(7)) == OK   # empty: no launch
    assert call_chunked(lib, p, ST=fake(3)) == ALIAS


def test_chunk_size_validation(lib):
    for C in (0, 8, 48, 128, -64):
        assert call_chunked(lib, prob(), C=C) == CHUNK
    assert fb.falcon_workspace_bytes(prob(), 8) == ctypes.c_size_t(-1).value
    assert fb.falcon_workspace_bytes(prob(dk=12), 64) == ctypes.c_size_t(-1).value
    for C in (16, 32, 64):
        assert fb.falcon_workspace_bytes(prob(), C) != ctypes.c_size_t(-1).value


def test_empty_problems_do_nothing(lib):
    # No token and no state to write: valid, nothing is launched.
    assert call_chunked(lib, prob(T=0), ST=None) == OK
    assert call_recurrent(lib, prob(B=0), ST=None) == OK
    assert call_chunked(lib, prob(H=0)) == OK
    p = prob(B=0)
    assert lib.falcon_decode_step(ctypes.byref(p), None, None, None, None, None, None, None, None,
                                  None) == OK


def test_decode_validation(lib):
    p = prob(dk=128, dv=128)

    def dec(**over):
        a = dict(x=fake(0), q=fake(1), v=fake(2), beta=fake(3), lam=fake(4), S=fake(5), first=None,
                 o=fake(6))
        a.update(over)
        return lib.falcon_decode_step(ctypes.byref(p), a["x"], a["q"], a["v"], a["beta"], a["lam"],
                                      a["S"], a["first"], a["o"], None)

    for name in ("x", "q", "v", "beta", "lam", "S", "o"):
        assert dec(**{name: None}) == NULL, name
        assert dec(**{name: fake(9, misalign=4)}) == ALIGN, name
    assert dec(o=fake(5)) == ALIAS
    assert dec(S=fake(1)) == ALIAS


def call_bwd(lib, p, ws=None, wsb=0, **over):
    a = dict(k=fake(0), q=fake(1), v=fake(2), beta=fake(3), lam=fake(4), S0=None, kp=None,
             dO=fake(5), dST=None, dk=fake(6), dq=fake(7), dv=fake(8), dbeta=fake(9),
             dlam=fake(10), dS0=fake(11), dkp=None)
    a.update(over)
    return lib.falcon_bwd_chunked(ctypes.byref(p) if p is not None else None, a["k"], a["q"],
                                  a["v"], a["beta"], a["lam"], a["S0"], a["kp"], a["dO"], a["dST"],
                                  a["dk"], a["dq"], a["dv"], a["dbeta"], a["dlam"], a["dS0"],
                                  a["dkp"], ws, wsb, None)


def test_backward_validation(lib):
    need = fb.falcon_bwd_workspace_bytes(prob())
    # per 32-token chunk per (b, h), in floats: the maps (P, H, G: 3 x 64 x 64),
    # the saved state and adjoint (2 x 64 x 64) and the forward factors (W, U:
    # 2 x 32 x 64, T: 32 x 32, eight gate rows and gamma: 9 x 32); T = 40 -> 2
    # chunks, B*H = 6
    per_chunk = 3 * 4096 + 2 * 4096 + (2 * 2048 + 1024 + 9 * 32)
    assert need == 6 * 2 * per_chunk * 4
    ws = fake(20)
    assert call_bwd(lib, None) == NULL
    assert call_bwd(lib, prob(variant="falcon1a"), ws, need) == VARIANT
    assert call_bwd(lib, prob(variant="falcon2"), ws, need) == VARIANT
    assert call_bwd(lib, prob(dk=32, dv=32), ws, need) == SHAPE
    assert call_bwd(lib, prob(dv=128), ws, need) == SHAPE
    assert fb.falcon_bwd_workspace_bytes(prob(dk=32)) == ctypes.c_size_t(-1).value
    assert fb.falcon_bwd_workspace_bytes(prob(variant="falcon2")) == ctypes.c_size_t(-1).value
    assert call_bwd(lib, prob(eps_gamma=2.0), ws, need) == VALUE
    for name in ("k", "q", "v", "beta", "lam", "dO", "dk", "dq", "dv", "dbeta", "dlam"):
        assert call_bwd(lib, prob(), ws, need, **{name: None}) == NULL, name
    for i, name in enumerate(("k", "q", "v", "dO", "dk", "dq", "dS0")):
        assert call_bwd(lib, prob(), ws, need, **{name: fake(30 + i, misalign=4)}) == ALIGN, name
    assert call_bwd(lib, prob(), None, 0) == WORKSPACE
    assert call_bwd(lib, prob(), ws, need - 1) == WORKSPACE
    assert call_bwd(lib, prob(), fake(20, misalign=8), need) == ALIGN
    # outputs may overlap neither an input nor one another
    assert call_bwd(lib, prob(), ws, need, dq=fake(1)) == ALIAS
    assert call_bwd(lib, prob(), ws, need, dv=fake(6)) == ALIAS
    assert call_bwd(lib, prob(), ws, need, dS0=fake(40), dST=fake(40)) == ALIAS
    assert call_bwd(lib, prob(), ws, need, dkp=fake(6), kp=fake(41)) == ALIAS
    # dk_prev is ignored on a fresh start, so it cannot alias then
    assert call_bwd(lib, prob(B=0), dkp=fake(6)) == OK
    # nothing to do
    assert call_bwd(lib, prob(B=0)) == OK
    assert call_bwd(lib, prob(H=0), k=None, dk=None) == OK


def test_workspace_overlap_is_rejected(lib):
    p = prob(T=200)
    need = fb.falcon_workspace_bytes(p, 64)
    assert need > 0
    # the workspace may overlap no input and no output
    for name, i in (("k", 0), ("v", 2), ("beta", 3), ("o", 5), ("ST", 6)):
        assert call_chunked(lib, p, ws=fake(i), wsb=need) == ALIAS, name
    assert call_chunked(lib, p, ws=fake(20), wsb=need, S0=ctypes.c_void_p(BASE + 20 * STRIDE + 4096)) == ALIAS
    # backward: the workspace against an output
    bneed = fb.falcon_bwd_workspace_bytes(prob())
    assert call_bwd(lib, prob(), fake(6), bneed) == ALIAS
    assert call_bwd(lib, prob(), fake(2), bneed) == ALIAS


# ---- the Python binding checks shapes, dtypes and devices before any pointer
# crosses the C ABI (CPU tensors: the checks run before the device check) ----

def _fwd_tensors(B=2, H=3, T=40, dk=64, dv=64, io=None, per_col=False):
    import torch
    io = torch.bfloat16 if io is None else io
    return dict(phi_k=torch.zeros(B, H, T, dk, dtype=io), phi_q=torch.zeros(B, H, T, dk, dtype=io),
                v=torch.zeros(B, H, T, dv, dtype=io),
                beta=torch.zeros((B, H, T, dv) if per_col else (B, H, T)),
                lam=torch.zeros(B, H, T))


@pytest.mark.parametrize("fn", ["chunked", "recurrent"])
def test_binding_rejects_mismatched_forward_arguments(fn):
    import torch
    call = fb.falcon_fwd_chunked if fn == "chunked" else fb.falcon_fwd_recurrent

    def run(variant="falcon1", **over):
        d = _fwd_tensors(per_col=variant in ("falcon2", "falcon2a"))
        extra = {k: over.pop(k) for k in list(over) if k in ("S0", "k_prev", "o", "S_T", "workspace")}
        d.update(over)
        if fn == "recurrent":
            extra.pop("workspace", None)
        return call(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], variant=variant, **extra)

    bad = [
        (dict(phi_q=torch.zeros(2, 3, 41, 64, dtype=torch.bfloat16)), "phi_q"),
        (dict(phi_q=torch.zeros(2, 3, 40, 64)), "phi_q"),                 # f32 query, bf16 values
        (dict(v=torch.zeros(2, 3, 40, 64, dtype=torch.float16)), "io dtype"),
        (dict(beta=torch.zeros(2, 3, 40, dtype=torch.float64)), "beta"),
        (dict(lam=torch.zeros(2, 3)), "lam"),
        (dict(S0=torch.zeros(2, 3, 64, 64, dtype=torch.bfloat16)), "S0"),
        (dict(S0=torch.zeros(2, 3, 64, 32)), "S0"),
        (dict(k_prev=torch.zeros(2, 3, 64)), "k_prev"),
        (dict(o=torch.zeros(2, 3, 39, 64, dtype=torch.bfloat16)), "^o:"),
        (dict(S_T=torch.zeros(2, 3, 64, 64, dtype=torch.float64)), "S_T"),
        (dict(phi_k=torch.zeros(2, 3, 40)), "phi_k"),
    ]
    for over, what in bad:
        with pytest.raises(ValueError, match=what):
            run(**over)
    # a Falcon-2 call needs per-column gains
    with pytest.raises(ValueError, match="beta"):
        d = _fwd_tensors()
        call(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], variant="falcon2")
    with pytest.raises(ValueError, match="variant"):
        run(variant="falcon3")
    if fn == "chunked":
        with pytest.raises(ValueError, match="workspace"):
            run(workspace=torch.zeros(16, dtype=torch.uint8))
    # well-formed CPU tensors get as far as the device check
    with pytest.raises(ValueError, match="device"):
        run()


def test_binding_rejects_mismatched_decode_and_backward_arguments():
    import torch
    B, H, dk, dv = 2, 3, 64, 64
    bf = torch.bfloat16
    x, q, v = torch.zeros(B, H, dk, dtype=bf), torch.zeros(B, H, dk, dtype=bf), torch.zeros(B, H, dv, dtype=bf)
    beta, lam, S = torch.zeros(B, H), torch.zeros(B, H), torch.zeros(B, H, dk, dv)
    with pytest.raises(ValueError, match="lam"):
        fb.falcon_decode_step(x, q, v, beta, torch.zeros(B, H, 1), S)
    with pytest.raises(ValueError, match="beta"):
        fb.falcon_decode_step(x, q, v, beta, lam, S, variant="falcon2")
    with pytest.raises(ValueError, match="^S:"):
        fb.falcon_decode_step(x, q, v, beta, lam, torch.zeros(B, H, dk, dv, dtype=bf))
    with pytest.raises(ValueError, match="is_first"):
        fb.falcon_decode_step(x, q, v, beta, lam, S, is_first=torch.zeros(B, dtype=torch.int32))
    with pytest.raises(ValueError, match="^o:"):
        fb.falcon_decode_step(x, q, v, beta, lam, S, o=torch.zeros(B, H, dv))
    with pytest.raises(ValueError, match="device"):
        fb.falcon_decode_step(x, q, v, beta, lam, S)
    d = _fwd_tensors()
    dO = torch.zeros(2, 3, 40, 64, dtype=bf)
    with pytest.raises(ValueError, match="dO"):
        fb.falcon_bwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], dO.float())
    with pytest.raises(ValueError, match="dS_T"):
        fb.falcon_bwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], dO,
                              dS_T=torch.zeros(2, 3, 64))
    with pytest.raises(ValueError, match="dbeta"):
        fb.falcon_bwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], dO,
                              grads={"dbeta": torch.zeros(2, 3, 41)})
    with pytest.raises(ValueError, match="unknown"):
        fb.falcon_bwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], dO,
                              grads={"dx": torch.zeros(1)})
    with pytest.raises(ValueError, match="workspace"):
        fb.falcon_bwd_chunked(d["phi_k"], d["phi_q"], d["v"], d["beta"], d["lam"], dO,
                              workspace=torch.zeros(8, dtype=torch.uint8))


def test_wait_limit_setting(lib):
    prev = fb.falcon_set_wait_limit(1000)
    try:
        assert prev == 1 << 22
        assert fb.falcon_set_wait_limit(0) == 1000
        assert lib.falcon_set_wait_limit(-5) == -1          # rejected, unchanged
        assert fb.falcon_set_wait_limit(7) == 0
        with pytest.raises(ValueError):
            fb.falcon_set_wait_limit(-1)
    finally:
        fb.falcon_set_wait_limit(prev)
    assert fb.falcon_set_wait_limit(prev) == prev


def test_f1_launch_form_setting(lib):
    prev = fb.falcon_set_f1_launch_form(fb.F1_TWO_LAUNCH)
    try:
        assert prev == fb.F1_ONE_LAUNCH                        # the default
        assert lib.falcon_set_f1_launch_form(2) == -1          # rejected, unchanged
        assert lib.falcon_set_f1_launch_form(-1) == -1
        assert fb.falcon_set_f1_launch_form(fb.F1_ONE_LAUNCH) == fb.F1_TWO_LAUNCH
        with pytest.raises(ValueError):
            fb.falcon_set_f1_launch_form(5)
    finally:
        fb.falcon_set_f1_launch_form(prev)


def test_noalloc_validation(lib):
    def call(p, C=64, **over):
        a = fwd_args(**over)
        return lib.falcon_fwd_chunked_noalloc(ctypes.byref(p) if p is not None else None, a["k"], a["q"],
                                              a["v"], a["beta"], a["lam"], a["S0"], a["kp"], a["o"],
                                              a["ST"], C, None)
    assert call(None) == NULL
    assert call(prob(dk=48)) == SHAPE
    assert call(prob(), C=8) == CHUNK
    assert call(prob(), o=fake(2)) == ALIAS
    assert call(prob(), k=None) == NULL
    # one sequence beyond the 64 MiB static buffer: Falcon-1 with 2048 chunks,
    # Falcon-1A with 2^21 tokens (4096 tiles of aggregates)
    assert call(prob(B=1, H=1, T=2048 * 64)) == -11
    assert call(prob(B=1, H=1, T=1 << 21, variant="falcon1a")) == -11
    assert "scratch" in fb.falcon_status_string(-11)
    assert call(prob(T=0), ST=None) == OK                   # nothing to do, nothing launched
