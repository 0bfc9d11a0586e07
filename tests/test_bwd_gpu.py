"""GPU parity of mss_selective_scan_bwd (gradients of the forward scan) against the fp64 oracle,
element by element, on seeded inputs: small, ragged and flag-varied cases, every segment
split, and the Mamba-2.8B layer shape at full size.

Tolerance per element: |gpu - ref| <= rtol_out |ref| + rtol_sum M + atol, where M is the
oracle's sum of |terms| behind that element (its magnitude mode).  Every output is a sum
(over states, time, channels or batch) that the GPU evaluates in fp32 in another order, from
fp32 recurrences; such an evaluation's error is proportional to M, not to the possibly
cancelled |ref|.  rtol_sum = 1e-4 (the forward's fp32 bound) and atol = 1e-6 for all outputs;
rtol_out = 0 for fp32 outputs and 2e-2 for the bf16-rounded du / ddelta / dz.
"""
import numpy as np
import pytest

from synth import CONFIGS, scan_inputs
from tests.gpu_helpers import dev, host64

pytestmark = pytest.mark.gpu

RTOL_SUM = 1e-4
ATOL = 1e-6
ROUNDED = ("du", "ddelta", "dz")


@pytest.fixture(scope="module")
def mss():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_06_amd as m
    m.load_library()
    return m


def _dout(s, seed):
    g = np.random.default_rng(500 + seed).standard_normal(s.u.shape).astype(np.float32)
    if s.dtype == "bf16":
        from synth import round_to_bf16
        g = round_to_bf16(g)
    return g


def _gpu(mss, s, dout, use_z=True, use_D=True, use_bias=True, softplus=True):
    z = dev(s.z, s.dtype) if (use_z and s.z is not None) else None
    return mss.selective_scan_bwd(dev(s.u, s.dtype), dev(s.delta, s.dtype), dev(s.A), dev(s.B),
                                  dev(s.C), dev(dout, s.dtype), D=dev(s.D) if use_D else None, z=z,
                                  delta_bias=dev(s.delta_bias) if use_bias else None,
                                  delta_softplus=softplus)


def _ref(orc, s, dout, magnitude, use_z=True, use_D=True, use_bias=True, softplus=True):
    return orc.selective_scan_bwd(s.u, s.delta, s.A, s.B, s.C,
                                  D=s.D if use_D else None,
                                  z=s.z if (use_z and s.z is not None) else None,
                                  delta_bias=s.delta_bias if use_bias else None,
                                  softplus_flag=softplus, dout=dout, magnitude=magnitude)


def _check(mss, orc, s, seed, what, **flags):
    import torch
    dout = _dout(s, seed)
    g = _gpu(mss, s, dout, **flags)
    torch.cuda.synchronize()
    ref = _ref(orc, s, dout, False, **flags)
    mag = _ref(orc, s, dout, True, **flags)
    worst = {}
    for k, r in ref.items():
        if r is None:
            assert g[k] is None, k
            continue
        got = host64(g[k])
        assert got.shape == r.shape, (what, k, got.shape, r.shape)
        assert np.all(np.isfinite(got)), f"{what} {k}: non-finite"
        rtol_out = 2e-2 if (k in ROUNDED and s.dtype == "bf16") else 0.0
        lim = rtol_out * np.abs(r) + RTOL_SUM * mag[k] + ATOL
        err = np.abs(got - r)
        ratio = err / lim
        i = np.unravel_index(np.argmax(ratio), ratio.shape) if ratio.size else None
        worst[k] = float(ratio.max()) if ratio.size else 0.0
        assert worst[k] <= 1.0, (f"{what} {k}: {int((ratio > 1).sum())} of {ratio.size} out of "
                                 f"tolerance; worst at {i}: gpu={got[i]!r} ref={r[i]!r} "
                                 f"mag={mag[k][i]!r}")
    print(f"[{what}] worst err/limit: " + ", ".join(f"{k} {v:.3f}" for k, v in worst.items()),
          flush=True)
    return g


@pytest.mark.parametrize("Bt,Dn,L,dtype,a_kind", [
    (1, 64, 1, "f32", "s4d"), (2, 64, 64, "f32", "s4d"), (2, 70, 33, "f32", "s4d"),
    (1, 130, 200, "f32", "random"), (2, 128, 256, "bf16", "s4d"), (1, 100, 100, "bf16", "s4d"),
    (2, 192, 520, "bf16", "random"), (1, 1, 9, "f32", "s4d"), (3, 5, 17, "bf16", "s4d")])
def test_bwd_parity_shapes(mss, oracle_mod, Bt, Dn, L, dtype, a_kind):
    s = scan_inputs(Bt, Dn, 16, L, dtype=dtype, seed=70 + L, a_kind=a_kind)
    _check(mss, oracle_mod, s, L, f"bwd {Bt}x{Dn}x{L} {dtype} {a_kind}")


@pytest.mark.parametrize("flags", [
    dict(use_z=False), dict(use_D=False, use_bias=False), dict(softplus=False, use_bias=False),
    dict(use_z=False, use_D=False, use_bias=False)])
def test_bwd_optional_arguments(mss, oracle_mod, flags):
    s = scan_inputs(2, 96, 16, 300, dtype="f32", seed=71)
    if not flags.get("softplus", True):
        s.delta = np.abs(s.delta) * 0.05
    _check(mss, oracle_mod, s, 71, f"bwd flags {flags}", **flags)


@pytest.mark.parametrize("segments", ["1", "2", "7", "40"])
def test_bwd_segment_splits(mss, oracle_mod, segments, monkeypatch):
    monkeypatch.setenv("MSS_BWD_SEGMENTS", segments)
    s = scan_inputs(1, 128, 16, 320, dtype="f32", seed=72)
    _check(mss, oracle_mod, s, 72, f"bwd segments={segments}")


def test_bwd_mamba2p8b_full(mss, oracle_mod):
    c = CONFIGS["mamba2p8b_bf16"]
    s = scan_inputs(c["batch"], c["d_inner"], 16, c["L"], dtype="bf16", seed=73)
    _check(mss, oracle_mod, s, 73, "bwd mamba2p8b")


def test_bwd_deterministic_and_linear(mss):
    import torch
    s = scan_inputs(2, 256, 16, 1024, dtype="f32", seed=74)
    d1, d2 = _dout(s, 1), _dout(s, 2)
    g1 = _gpu(mss, s, d1)
    g1b = _gpu(mss, s, d1)
    g2 = _gpu(mss, s, d2)
    g3 = _gpu(mss, s, (2.0 * d1 - 0.5 * d2).astype(np.float32))
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g1b[k]), k
        a, b, c = host64(g1[k]), host64(g2[k]), host64(g3[k])
        scale = np.abs(2.0 * a).max() + np.abs(0.5 * b).max()
        np.testing.assert_allclose(c, 2.0 * a - 0.5 * b, rtol=0, atol=1e-5 * scale, err_msg=k)


def test_bwd_empty_sequence(mss):
    import torch
    A = dev(-np.tile(np.arange(1, 17, dtype=np.float32), (64, 1)))
    u = torch.empty((2, 64, 0), dtype=torch.float32, device="cuda")
    B = torch.empty((2, 16, 0), dtype=torch.float32, device="cuda")
    g = mss.selective_scan_bwd(u, u.clone(), A, B, B.clone(), u.clone())
    torch.cuda.synchronize()
    assert torch.all(g["dA"] == 0) and torch.all(g["dD"] == 0) and torch.all(g["ddelta_bias"] == 0)
    assert g["du"].shape == (2, 64, 0) and g["dB"].shape == (2, 16, 0)
