"""Shared helpers of the GPU parity tests: upload seeded inputs, run the library through its
C ABI, and compare with the fp64 oracle element by element."""
from __future__ import annotations

import numpy as np

# Tolerances: |gpu - ref| <= atol + rtol * |ref|, elementwise.
TOL_F32 = dict(rtol=1e-4, atol=1e-5)    # fp32 inputs
TOL_BF16 = dict(rtol=2e-2, atol=1e-5)   # bf16 u / delta / z / out, fp32 state


def waves_for(Bt, Dn, pieces):
    """Wavefront count that gives the fast forward `pieces` equal pieces of each 64-channel group
    (the plan spreads the (group, tile) work evenly over the wavefronts)."""
    return int(pieces) * Bt * ((Dn + 63) // 64)


def torch_dev():
    import torch
    return torch.device("cuda:0")


def dev(arr, dtype="f32"):
    """numpy float32 (bf16-exact when dtype == 'bf16') -> device tensor, exactly."""
    import torch
    if arr is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(torch_dev())
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def host64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


# worst |gpu - ref| / (atol + rtol |ref|) of every named comparison in this session (tests that
# record margins add to it; conftest writes it out when MSS_PARITY_MARGINS names a file)
MARGINS = {}


def record_margin(what, ratio):
    MARGINS[what] = max(float(ratio), MARGINS.get(what, 0.0))
    return ratio


def assert_close(gpu, ref, rtol, atol, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    lim = atol + rtol * np.abs(ref)
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance "
            f"(rtol={rtol}, atol={atol}); worst at {i}: gpu={gpu[i]!r} ref={ref[i]!r} "
            f"err={err[i]:.3e} lim={lim[i]:.3e}")
    return float((err / (atol + rtol * np.abs(ref))).max()) if err.size else 0.0


def run_scan(mss, s, use_z=True, use_D=True, use_bias=True, softplus=True):
    """Upload a ScanInputs set and run mss_selective_scan_fwd; returns device (out, last_state)."""
    u = dev(s.u, s.dtype)
    dl = dev(s.delta, s.dtype)
    z = dev(s.z, s.dtype) if (use_z and s.z is not None) else None
    return mss.selective_scan_fwd(u, dl, dev(s.A), dev(s.B), dev(s.C),
                                  D=dev(s.D) if use_D else None, z=z,
                                  delta_bias=dev(s.delta_bias) if use_bias else None,
                                  delta_softplus=softplus, return_last_state=True)


def oracle_scan(oracle, s, rows=None, use_z=True, use_D=True, use_bias=True, softplus=True):
    return oracle.selective_scan(s.u, s.delta, s.A, s.B, s.C,
                                 D=s.D if use_D else None,
                                 z=s.z if (use_z and s.z is not None) else None,
                                 delta_bias=s.delta_bias if use_bias else None,
                                 softplus_flag=softplus, rows=rows)
