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
    # 101 KiB per 32-token chunk per (b, h): T = 40 -> 2 chunks, B*H = 6
    assert need == 6 * 2 * 101 * 1024
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
