"""Seeded synthetic Mamba-layer inputs.

Shapes follow the selective scan's functional signature on the Keras/TensorFlow
tutorial page ("Mamba SSM concept and implementation in Keras and TensorFlow",
the ``selective_scan`` and ``MambaBlock.ssm`` code): u, delta and z are
(batch, d_inner, L) here (L contiguous), B and C are (batch, d_state, L) and are
shared by every channel, A is (d_inner, d_state), D and the delta bias are
(d_inner,).

Value distributions follow the initialisations those pages give:
  * A[d, n] = -(n + 1): the tutorial sets A_log = log(1..N) and A = -exp(A_log)
    (S4D-real); ``a_kind="random"`` instead draws an unstructured negative A.
  * D = 1 (the tutorial initialises D to ones).
  * dt ~ exp(U(ln 1e-3, ln 1e-1)) per channel, floored at 1e-4, and the delta
    bias is the inverse softplus of dt, so softplus(bias) = dt (the mamba-jax
    README's dt_min / dt_max / dt_init_floor flags; the upstream README notes
    that the bias of the delta projection is what targets the Delta range).
  * u, raw delta, z, B, C ~ N(0, 1).

Draw order for one scan input set, from numpy ``Generator(PCG64(seed))``:
u, delta_raw, z (skipped when there is no gate), B, C, dt, then A when it is
random.  bf16 tensors are drawn in fp32 and rounded to nearest-even bf16, so
their float32 arrays hold exactly the values a bf16 tensor holds.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

# The five seeded workloads.  Shapes are Mamba layer shapes: d_inner is
# 2 x d_model (expand 2) for the 130M (d_model 768) and 2.8B (d_model 2560)
# models listed in the upstream README's model table; d_state is 16.
CONFIGS = {
    "tiny_fp32": dict(kind="scan", batch=2, d_inner=64, d_state=16, L=256,
                      dtype="f32", with_z=True),
    "mamba130m_fp32": dict(kind="scan", batch=8, d_inner=1536, d_state=16, L=2048,
                           dtype="f32", with_z=True),
    "mamba2p8b_bf16": dict(kind="scan", batch=4, d_inner=5120, d_state=16, L=2048,
                           dtype="bf16", with_z=True),
    "long_fp32": dict(kind="scan", batch=1, d_inner=1536, d_state=16, L=131072,
                      dtype="f32", with_z=False),
    "decode_bf16": dict(kind="decode", batch=64, d_inner=5120, d_state=16, steps=1024,
                        dtype="bf16", with_z=True),
}

DT_MIN, DT_MAX, DT_FLOOR = 1e-3, 1e-1, 1e-4


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.  NaN and
    infinity do not occur in these inputs and are not treated specially.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return bits.astype(np.uint32).view(np.float32)


def _draw_normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        v = round_to_bf16(v)
    return v


def _draw_dt_bias(rng: np.random.Generator, d_inner: int) -> np.ndarray:
    """Per-channel delta bias b with softplus(b) = dt, dt log-uniform in [1e-3, 1e-1]."""
    u01 = rng.random(size=d_inner)  # float64
    dt = np.exp(u01 * (np.log(DT_MAX) - np.log(DT_MIN)) + np.log(DT_MIN))
    dt = np.maximum(dt, DT_FLOOR)
    # inverse softplus, log(expm1(dt)), written in its cancellation-free form
    bias = dt + np.log(-np.expm1(-dt))
    return bias.astype(np.float32)


def _draw_A(rng: Optional[np.random.Generator], d_inner: int, d_state: int,
            a_kind: str) -> np.ndarray:
    if a_kind == "s4d":
        return np.tile(-np.arange(1, d_state + 1, dtype=np.float32), (d_inner, 1))
    if a_kind == "random":
        # unstructured negative real A: -exp(U(ln 0.5, ln 16)) per (d, n)
        mag = np.exp(rng.uniform(np.log(0.5), np.log(16.0), size=(d_inner, d_state)))
        return (-mag).astype(np.float32)
    raise ValueError(f"unknown a_kind {a_kind!r}")


@dataclass
class ScanInputs:
    u: np.ndarray            # (batch, d_inner, L) float32 (bf16-exact when dtype == "bf16")
    delta: np.ndarray        # (batch, d_inner, L) raw delta, before bias and softplus
    z: Optional[np.ndarray]  # (batch, d_inner, L) or None
    A: np.ndarray            # (d_inner, d_state) float32
    B: np.ndarray            # (batch, d_state, L) float32
    C: np.ndarray            # (batch, d_state, L) float32
    D: np.ndarray            # (d_inner,) float32
    delta_bias: np.ndarray   # (d_inner,) float32
    dtype: str               # "f32" or "bf16": the storage type of u, delta, z and out

    @property
    def shape(self):
        b, d, L = self.u.shape
        return b, d, self.A.shape[1], L


def scan_inputs(batch: int, d_inner: int, d_state: int, L: int, dtype: str = "f32",
                with_z: bool = True, seed: int = 0, a_kind: str = "s4d") -> ScanInputs:
    """Draw one seeded input set for the forward scan."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    rng = np.random.Generator(np.random.PCG64(seed))
    u = _draw_normal(rng, (batch, d_inner, L), dtype)
    delta = _draw_normal(rng, (batch, d_inner, L), dtype)
    z = _draw_normal(rng, (batch, d_inner, L), dtype) if with_z else None
    B = rng.standard_normal(size=(batch, d_state, L), dtype=np.float32)
    C = rng.standard_normal(size=(batch, d_state, L), dtype=np.float32)
    bias = _draw_dt_bias(rng, d_inner)
    A = _draw_A(rng, d_inner, d_state, a_kind)
    D = np.ones(d_inner, dtype=np.float32)
    return ScanInputs(u=u, delta=delta, z=z, A=A, B=B, C=C, D=D, delta_bias=bias,
                      dtype=dtype)


@dataclass
class DecodeInputs:
    x: np.ndarray       # (steps, batch, d_inner) float32, bf16-exact when dtype == "bf16"
    dt: np.ndarray      # (steps, batch, d_inner) raw dt, before bias and softplus
    z: Optional[np.ndarray]
    B: np.ndarray       # (steps, batch, d_state) float32
    C: np.ndarray       # (steps, batch, d_state) float32
    A: np.ndarray       # (d_inner, d_state)
    D: np.ndarray       # (d_inner,)
    dt_bias: np.ndarray  # (d_inner,)
    dtype: str


def decode_inputs(batch: int, d_inner: int, d_state: int, steps: int, dtype: str = "bf16",
                  with_z: bool = True, seed: int = 0, a_kind: str = "s4d") -> DecodeInputs:
    """Draw the inputs of `steps` chained one-token decode steps.

    Layer parameters (dt bias, then A when random) come from
    ``Generator(PCG64(SeedSequence(seed, spawn_key=(0,))))``; step s draws x, dt,
    z, B, C in that order from ``SeedSequence(seed, spawn_key=(1, s))``, so any
    step can be regenerated on its own.
    """
    prng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(0,))))
    bias = _draw_dt_bias(prng, d_inner)
    A = _draw_A(prng, d_inner, d_state, a_kind)
    D = np.ones(d_inner, dtype=np.float32)
    xs = np.empty((steps, batch, d_inner), np.float32)
    dts = np.empty_like(xs)
    zs = np.empty_like(xs) if with_z else None
    Bs = np.empty((steps, batch, d_state), np.float32)
    Cs = np.empty_like(Bs)
    for s in range(steps):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(1, s))))
        xs[s] = _draw_normal(rng, (batch, d_inner), dtype)
        dts[s] = _draw_normal(rng, (batch, d_inner), dtype)
        if with_z:
            zs[s] = _draw_normal(rng, (batch, d_inner), dtype)
        Bs[s] = rng.standard_normal(size=(batch, d_state), dtype=np.float32)
        Cs[s] = rng.standard_normal(size=(batch, d_state), dtype=np.float32)
    return DecodeInputs(x=xs, dt=dts, z=zs, B=Bs, C=Cs, A=A, D=D, dt_bias=bias, dtype=dtype)


# Mamba-2 SSD layer workloads (the upstream README's Mamba-2 block: state size 64 by default, 64 or
# 128 in use; d_model 2560 with expand 2 as for the 2.8B / 2.7B models gives d_inner 5120, here as 80 heads
# of 64 channels; one group of B / C).  Layout (batch, L, heads, headdim).
SSD_CONFIGS = {
    "ssd_tiny": dict(batch=2, L=256, heads=4, headdim=64, groups=1, d_state=64, dtype="bf16", with_z=True),
    "ssd_2p7b_n64": dict(batch=4, L=2048, heads=80, headdim=64, groups=1, d_state=64, dtype="bf16",
                         with_z=True),
    "ssd_2p7b_n128": dict(batch=4, L=2048, heads=80, headdim=64, groups=1, d_state=128, dtype="bf16",
                          with_z=True),
}


@dataclass
class SSDInputs:
    x: np.ndarray            # (batch, L, heads, headdim) float32, bf16-exact when dtype == "bf16"
    dt: np.ndarray           # (batch, L, heads) raw dt, before bias and softplus
    z: Optional[np.ndarray]  # (batch, L, heads, headdim) or None
    A: np.ndarray            # (heads,) float32, negative
    B: np.ndarray            # (batch, L, groups, d_state), bf16-exact when dtype == "bf16"
    C: np.ndarray            # (batch, L, groups, d_state)
    D: np.ndarray            # (heads,) float32
    dt_bias: np.ndarray      # (heads,) float32
    dtype: str


def ssd_inputs(batch: int, L: int, heads: int, headdim: int, groups: int, d_state: int,
               dtype: str = "bf16", with_z: bool = True, seed: int = 0) -> SSDInputs:
    """One seeded input set for the SSD layer.  Draw order from Generator(PCG64(seed)): x, dt, z
    (skipped without a gate), B, C, the dt bias (as for the S6 layer, per head), then A: one value
    per head, -U(1, 16) (the span of the tutorial's S4D-real values 1..16, one scalar per head as
    Mamba-2 ties them).  D = 1.  x, dt, z, B, C are drawn in fp32 and rounded to bf16 for bf16."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _draw_normal(rng, (batch, L, heads, headdim), dtype)
    dt = _draw_normal(rng, (batch, L, heads), dtype)
    z = _draw_normal(rng, (batch, L, heads, headdim), dtype) if with_z else None
    B = _draw_normal(rng, (batch, L, groups, d_state), dtype)
    C = _draw_normal(rng, (batch, L, groups, d_state), dtype)
    bias = _draw_dt_bias(rng, heads)
    A = (-rng.uniform(1.0, 16.0, size=heads)).astype(np.float32)
    D = np.ones(heads, dtype=np.float32)
    return SSDInputs(x=x, dt=dt, z=z, A=A, B=B, C=C, D=D, dt_bias=bias, dtype=dtype)


def sample_rows(n_rows: int, k: int, seed: int = 1) -> np.ndarray:
    """k distinct flat row indices in [0, n_rows): the first and last rows plus seeded picks."""
    k = min(k, n_rows)
    rng = np.random.Generator(np.random.PCG64(seed))
    picks = {0, n_rows - 1}
    if k > len(picks):
        extra = rng.choice(n_rows, size=min(n_rows, 4 * k), replace=False)
        for r in extra:
            if len(picks) >= k:
                break
            picks.add(int(r))
    return np.array(sorted(picks)[:k], dtype=np.int64)
