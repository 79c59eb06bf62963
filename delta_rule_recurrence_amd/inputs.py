"""Seeded synthetic inputs for the Falcon recurrences.

This module is shared by the tests, the benchmark and ``smoke()``; it holds
no arithmetic of the recurrence itself, only random draws, the workload
recipe for the gates, and one rounding to the I/O dtype.

Recipe (the paper prints no inputs; its models feed RMS-normalised q/k
projections and learned gates, §4.1 and §3 "Implicit fast-memory objective"):
  * features phi(k), phi(q) and values v: i.i.d. N(0,1) scaled by 1/sqrt(dk),
    so ||x_t||^2 is about 1 (the regime of RMS-normalised features divided by
    sqrt(d));
  * beta = sigmoid(N(0,1)) in (0, 1) (scalar per token, or per value column);
  * lam = softplus(N(-2,1)), a positive ridge;
  * draw order: phi(k), phi(q), v, then the beta logits, then the lam logits,
    from ``numpy.random.default_rng(seed)``;
  * features/values are rounded ONCE to the I/O dtype (round-to-nearest-even
    through torch); beta and lam are float32.  The rounded values, upcast to
    float64, are what both the oracle and the GPU see.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """A named synthetic workload."""
    name: str
    variant: str           # "falcon1" | "falcon1a" | "falcon2" | "falcon2a"
    B: int
    H: int
    T: int
    dk: int
    dv: int
    C: int
    io_dtype: str          # "f32" | "bf16"
    seed: int
    eps: float = 1e-6
    eps_gamma: float = 1e-6


# The workloads the build is measured and checked on.
WORKLOADS = {
    "f1_recurrent_tiny": Workload("f1_recurrent_tiny", "falcon1", 1, 1, 64, 16, 16, 16, "f32", 0),
    "f1_chunked_8x12x2048_d64": Workload("f1_chunked_8x12x2048_d64", "falcon1", 8, 12, 2048, 64, 64, 64, "bf16", 1),
    "f1a_chunked_2x12x16384_d64": Workload("f1a_chunked_2x12x16384_d64", "falcon1a", 2, 12, 16384, 64, 64, 64, "bf16", 2),
    "f2_chunked_8x12x2048_d64": Workload("f2_chunked_8x12x2048_d64", "falcon2", 8, 12, 2048, 64, 64, 64, "bf16", 3),
    # the backward of the Falcon-1 training shape (C names the forward's chunk)
    "f1_backward_8x12x2048_d64": Workload("f1_backward_8x12x2048_d64", "falcon1", 8, 12, 2048, 64, 64, 64, "bf16", 5),
    # the training shape with float32 I/O: served by the general chunked kernel
    "f1_chunked_f32_8x12x2048_d64": Workload("f1_chunked_f32_8x12x2048_d64", "falcon1", 8, 12, 2048, 64, 64, 64, "f32", 6),
}

# Decode workload: batch 512, 12 heads, d = 128, 1000 steps after a prefix.
DECODE = dict(name="f1_decode_512x12_d128", variant="falcon1", B=512, H=12, dk=128, dv=128,
              steps=1000, prefix=128, io_dtype="bf16", seed=4, eps=1e-6, eps_gamma=1e-6)

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _round(a: np.ndarray, io_dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(TORCH_DTYPE[io_dtype]).contiguous()


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _softplus(z):
    return np.log1p(np.exp(z))


def make_inputs(B, H, T, dk, dv, *, seed, io_dtype="bf16", per_column_beta=False,
                feature_scale=None, rng=None):
    """Draw one batch of inputs.

    Returns a dict of CPU torch tensors: ``phi_k``, ``phi_q`` ``[B,H,T,dk]`` and
    ``v`` ``[B,H,T,dv]`` in the I/O dtype, ``beta`` ``[B,H,T]`` (or
    ``[B,H,T,dv]``) and ``lam`` ``[B,H,T]`` in float32.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    scale = (1.0 / np.sqrt(dk)) if feature_scale is None else feature_scale
    k = rng.standard_normal((B, H, T, dk)) * scale
    q = rng.standard_normal((B, H, T, dk)) * scale
    v = rng.standard_normal((B, H, T, dv)) * scale
    zb = rng.standard_normal((B, H, T, dv) if per_column_beta else (B, H, T))
    zl = rng.standard_normal((B, H, T))
    return {
        "phi_k": _round(k, io_dtype),
        "phi_q": _round(q, io_dtype),
        "v": _round(v, io_dtype),
        "beta": torch.from_numpy(_sigmoid(zb).astype(np.float32)),
        "lam": torch.from_numpy(_softplus(zl - 2.0).astype(np.float32)),
    }


def workload_inputs(w: Workload):
    return make_inputs(w.B, w.H, w.T, w.dk, w.dv, seed=w.seed, io_dtype=w.io_dtype,
                       per_column_beta=w.variant in ("falcon2", "falcon2a"))


def make_cotangents(B, H, T, dv, *, seed, io_dtype="bf16", dk=None, with_state=False):
    """Seeded upstream gradients for the backward: ``dO`` ``[B,H,T,dv]`` in
    the I/O dtype (N(0,1) scaled by 1/sqrt(dv), rounded once) and, when
    ``with_state``, ``dS_T`` ``[B,H,dk,dv]`` float32 (N(0,1) * 0.1), drawn in
    that order from ``default_rng([seed, 1])``."""
    rng = np.random.default_rng([seed, 1])
    out = {"dO": _round(rng.standard_normal((B, H, T, dv)) / np.sqrt(dv), io_dtype), "dS_T": None}
    if with_state:
        dk = dv if dk is None else dk
        out["dS_T"] = torch.from_numpy((rng.standard_normal((B, H, dk, dv)) * 0.1).astype(np.float32))
    return out


def random_state(shape, *, seed, scale=0.1):
    """A seeded float32 state tensor (used for carried-state cases)."""
    rng = np.random.default_rng(seed)
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32))


def decode_step_inputs(step: int, B, H, dk, dv, *, seed, io_dtype="bf16"):
    """Inputs of decode step ``step`` (1-based): drawn from
    ``default_rng([seed, step])`` in the order phi(q), v, beta logits, lam
    logits, next phi(k).  The key *read* at step s is the key drawn at step
    s-1 (the prefix's last key for s = 1)."""
    rng = np.random.default_rng([seed, step])
    scale = 1.0 / np.sqrt(dk)
    q = rng.standard_normal((B, H, dk)) * scale
    v = rng.standard_normal((B, H, dv)) * scale
    zb = rng.standard_normal((B, H))
    zl = rng.standard_normal((B, H))
    k = rng.standard_normal((B, H, dk)) * scale
    return {
        "phi_q": _round(q, io_dtype),
        "v": _round(v, io_dtype),
        "beta": torch.from_numpy(_sigmoid(zb).astype(np.float32)),
        "lam": torch.from_numpy(_softplus(zl - 2.0).astype(np.float32)),
        "phi_k": _round(k, io_dtype),
    }


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a (rounded) tensor to a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()
