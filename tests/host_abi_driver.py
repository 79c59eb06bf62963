"""Drives the C ABI of the host-sanitised, bounds-checked build
(libfalcon_san.so) on a machine with no visible GPU.

Run by tests/test_host_sanitizers.py in a child process that preloads the
ASan runtime and hides every device.  Every entry point is called on fake,
never-dereferenced device addresses (256-byte aligned, non-overlapping
unless a case wants an overlap): argument validation, workspace sizing, the
noalloc grouping and the launchers' host-side bounds model run for real, and
the launches themselves fail with FALCON_ERR_HIP because no device exists.
AddressSanitizer, UndefinedBehaviorSanitizer or a bounds assertion aborts
the process on the first error; the parent test then fails with its report.
argv: path of libfalcon_san.so.
"""

import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from delta_rule_recurrence_amd import falcon as fb  # noqa: E402

lib = fb.load_library(sys.argv[1])
OK, NULL, SHAPE, DTYPE, CHUNK, ALIGN, WS, VARIANT, HIP, VALUE, ALIAS, SCRATCH = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11)
LAUNCHED = (OK, HIP)            # valid arguments: the launch itself fails without a device
NONE = ctypes.c_size_t(-1).value


class Fake:
    """Distinct fake device addresses, each range followed by a gap."""

    def __init__(self):
        self.next = 1 << 44

    def __call__(self, nbytes):
        a = self.next
        self.next += (max(int(nbytes), 1) + 4095) // 4096 * 4096 + 1 << 20
        return a


def problem(B, H, T, dk, dv, variant, bf16=True, eps=1e-6, eps_gamma=1e-6):
    return fb.FalconProblem(B, H, T, dk, dv, variant, 1 if bf16 else 0, eps, eps_gamma)


def fwd_buffers(fake, p, per_col, S0=True, kp=True, ST=True):
    io = 2 if p.io_dtype == 1 else 4
    th = p.B * p.H * p.T
    d = dict(phi_k=fake(th * p.dk * io), phi_q=fake(th * p.dk * io), v=fake(th * p.dv * io),
             beta=fake(th * (p.dv if per_col else 1) * 4), lam=fake(th * 4),
             S0=fake(p.B * p.H * p.dk * p.dv * 4) if S0 else None,
             k_prev=fake(p.B * p.H * p.dk * io) if kp else None,
             o=fake(th * p.dv * io), S_T=fake(p.B * p.H * p.dk * p.dv * 4) if ST else None)
    return d


def P(x):
    return ctypes.c_void_p(x) if x else None


calls = 0


def chunked(p, C, d, ws=None, ws_bytes=None):
    global calls
    need = lib.falcon_workspace_bytes(ctypes.byref(p), C)
    if ws_bytes is None:
        ws_bytes = 0 if need == NONE else need
    calls += 1
    return lib.falcon_fwd_chunked(ctypes.byref(p), P(d["phi_k"]), P(d["phi_q"]), P(d["v"]), P(d["beta"]),
                                  P(d["lam"]), P(d["S0"]), P(d["k_prev"]), P(d["o"]), P(d["S_T"]), C,
                                  P(ws), ctypes.c_size_t(ws_bytes), None), need


def main():
    global calls
    fake = Fake()
    variants = {"falcon1": 1, "falcon1a": 2, "falcon2": 3, "falcon2a": 4}
    shapes = [(1, 1, 1), (1, 1, 63), (1, 1, 64), (1, 1, 65), (2, 3, 200), (1, 2, 4096), (3, 5, 2048),
              (8, 12, 2048), (2, 12, 16384), (1, 1, 1 << 20), (600, 1, 64), (1, 9, 0)]
    for vname, var in variants.items():
        per_col = vname in ("falcon2", "falcon2a")
        for (dk, dv) in ((64, 64), (32, 64), (16, 16), (128, 128)):
            for bf16 in (True, False):
                for (B, H, T) in shapes:
                    if B * H * T * max(dk, dv) > (1 << 31):
                        continue
                    p = problem(B, H, T, dk, dv, var, bf16)
                    for C in (16, 32, 64):
                        for opt in ((True, True, True), (False, False, True), (False, False, False)):
                            d = fwd_buffers(fake, p, per_col, *opt)
                            st, need = chunked(p, C, d, ws=fake(1 << 12) if True else None)
                            if need != NONE and need > 0:
                                st, _ = chunked(p, C, d, ws=fake(need), ws_bytes=need)
                                assert st in LAUNCHED, (vname, dk, dv, bf16, B, H, T, C, opt, st)
                                st2, _ = chunked(p, C, d, ws=fake(need), ws_bytes=need - 1)
                                assert st2 == WS, ("short workspace", vname, B, H, T, C, st2)
                            elif need == 0:
                                assert st in LAUNCHED, (vname, dk, dv, bf16, B, H, T, C, opt, st)
                            else:
                                assert st in (SHAPE, CHUNK), (vname, dk, dv, B, H, T, C, st)
                    # recurrent form
                    d = fwd_buffers(fake, p, per_col)
                    calls += 1
                    st = lib.falcon_fwd_recurrent(ctypes.byref(p), P(d["phi_k"]), P(d["phi_q"]), P(d["v"]),
                                                  P(d["beta"]), P(d["lam"]), P(d["S0"]), P(d["k_prev"]),
                                                  P(d["o"]), P(d["S_T"]), None)
                    assert st in LAUNCHED + (SHAPE,), (vname, dk, dv, B, H, T, st)
    # noalloc: groups of sequences that fit the static array, or FALCON_ERR_SCRATCH
    for (B, H, T, var) in ((8, 12, 2048, 1), (1, 1, 2048 * 64, 1), (1, 1, 130880, 1), (2, 12, 16384, 2),
                           (1, 1, 1 << 21, 2), (4, 4, 1000, 3)):
        p = problem(B, H, T, 64, 64, var)
        d = fwd_buffers(fake, p, var >= 3)
        calls += 1
        st = lib.falcon_fwd_chunked_noalloc(ctypes.byref(p), P(d["phi_k"]), P(d["phi_q"]), P(d["v"]),
                                            P(d["beta"]), P(d["lam"]), P(d["S0"]), P(d["k_prev"]), P(d["o"]),
                                            P(d["S_T"]), 64, None)
        assert st in LAUNCHED + (SCRATCH,), (B, H, T, var, st)
    # decode
    for var in (1, 2, 3, 4):
        for (B, H, dk, dv) in ((512, 12, 128, 128), (1, 1, 64, 64), (3, 7, 16, 32)):
            p = problem(B, H, 1, dk, dv, var)
            io = 2
            x, q, v = fake(B * H * dk * io), fake(B * H * dk * io), fake(B * H * dv * io)
            beta, lam = fake(B * H * (dv if var >= 3 else 1) * 4), fake(B * H * 4)
            S, first, o = fake(B * H * dk * dv * 4), fake(B), fake(B * H * dv * io)
            calls += 1
            st = lib.falcon_decode_step(ctypes.byref(p), P(x), P(q), P(v), P(beta), P(lam), P(S), P(first),
                                        P(o), None)
            assert st in LAUNCHED, (var, B, H, dk, dv, st)
            calls += 1
            st = lib.falcon_decode_step(ctypes.byref(p), P(x), P(q), P(v), P(beta), P(lam), P(S), P(first),
                                        P(S + 64), None)
            assert st == ALIAS, ("decode output inside S", st)
    # backward
    for bf16 in (True, False):
        for (B, H, T) in ((1, 1, 1), (2, 3, 200), (8, 12, 2048), (1, 1, 0), (1, 1, 100000)):
            p = problem(B, H, T, 64, 64, 1, bf16)
            need = lib.falcon_bwd_workspace_bytes(ctypes.byref(p))
            assert need != NONE
            d = fwd_buffers(fake, p, False)
            io = 2 if bf16 else 4
            th = B * H * T
            g = [fake(th * 64 * io), fake(B * H * 64 * 64 * 4), fake(th * 64 * 4), fake(th * 64 * 4),
                 fake(th * 64 * 4), fake(th * 4), fake(th * 4), fake(B * H * 64 * 64 * 4), fake(B * H * 64 * 4)]
            for ws_bytes, want in ((need, LAUNCHED), (max(need - 1, 0), (WS,) if need > 0 else LAUNCHED)):
                calls += 1
                st = lib.falcon_bwd_chunked(ctypes.byref(p), P(d["phi_k"]), P(d["phi_q"]), P(d["v"]),
                                            P(d["beta"]), P(d["lam"]), P(d["S0"]), P(d["k_prev"]),
                                            *[P(x) for x in g], P(fake(max(need, 1))), ctypes.c_size_t(ws_bytes),
                                            None)
                assert st in want, (bf16, B, H, T, ws_bytes, need, st)
    # invalid arguments: each rejected before any launch
    p = problem(2, 3, 200, 64, 64, 1)
    d = fwd_buffers(fake, p, False)
    need = lib.falcon_workspace_bytes(ctypes.byref(p), 64)
    ws = fake(need)
    for key, val, want in (("phi_k", 0, NULL), ("o", d["o"] + 8, ALIGN), ("o", d["phi_q"], ALIAS),
                           ("S_T", d["o"] + 64, ALIAS)):
        dd = dict(d)
        dd[key] = val
        st, _ = chunked(p, 64, dd, ws=ws, ws_bytes=need)
        assert st == want, (key, st, want)
    st, _ = chunked(p, 64, d, ws=d["v"], ws_bytes=need)
    assert st == ALIAS, ("workspace over an input", st)
    for bad, want in ((problem(2, 3, 200, 64, 64, 9), VARIANT), (problem(2, 3, 200, 48, 64, 1), SHAPE),
                      (problem(-1, 3, 200, 64, 64, 1), SHAPE), (problem(2, 3, 200, 64, 64, 1, eps=-1.0), VALUE),
                      (problem(2, 3, 200, 64, 64, 1, eps_gamma=1.0), VALUE)):
        st, _ = chunked(bad, 64, d, ws=ws, ws_bytes=need)
        assert st == want, (st, want)
    st, _ = chunked(p, 48, d, ws=ws, ws_bytes=need)
    assert st == CHUNK, st
    for s in range(-12, 1):
        assert lib.falcon_status_string(s)
    print(f"host ABI driver: {calls} calls checked", flush=True)


if __name__ == "__main__":
    main()
