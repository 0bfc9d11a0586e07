"""GPU parity of the Mamba-2 SSD chunked scan (mss_ssd_scan_fwd, through the C ABI) against the
fp64 oracle (oracle.ssd_scan: the step-by-step recurrence with tied parameters).

Tolerance (elementwise): |gpu - ref| <= rtol |ref| + eps M + atol, M = the oracle's magnitude mode
(every term in absolute value).  The chunked form reassociates the recurrence into dense products:
fp32 operands enter the bf16 matrix cores as hi + lo pairs (relative error ~2^-17 per product), and
each decay exp(A (cs_t - cs_s)) is taken from differences of fp32 running sums of delta inside a
64-step chunk (error <= |A| 64 2^-24 max cs, about 4e-4 relative for |A| <= 16 and cs <= 6.4), so
errors scale with M, not with a possibly cancelled |ref|: eps = 1e-3.  out is bf16: rtol 2e-2; the
fp32 final state: rtol 0.
"""
import numpy as np
import pytest

from synth import SSD_CONFIGS, round_to_bf16, ssd_inputs
from tests.gpu_helpers import dev, host64, record_margin

pytestmark = pytest.mark.gpu

EPS = 1e-3


@pytest.fixture(scope="module")
def mss():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_06_amd as m
    m.load_library()
    return m


def _close(gpu, ref, mag, rtol, atol, what):
    gpu, ref, mag = np.asarray(gpu, np.float64), np.asarray(ref, np.float64), np.asarray(mag, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    lim = rtol * np.abs(ref) + EPS * mag + atol
    err = np.abs(gpu - ref)
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err / lim), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance; worst at {i}: "
                             f"gpu={gpu[i]!r} ref={ref[i]!r} M={mag[i]!r} err={err[i]:.3e} lim={lim[i]:.3e}")
    return record_margin(what, float((err / lim).max()) if err.size else 0.0)


def _run(mss, s, use_z=True, use_D=True, use_bias=True, softplus=True):
    import torch
    out, last = mss.ssd_scan_fwd(dev(s.x, "bf16"), dev(s.dt, "bf16"), dev(s.A), dev(s.B, "bf16"), dev(s.C, "bf16"),
                                 D=dev(s.D) if use_D else None, z=dev(s.z, "bf16") if (use_z and s.z is not None) else None,
                                 dt_bias=dev(s.dt_bias) if use_bias else None, dt_softplus=softplus)
    torch.cuda.synchronize()
    return host64(out), host64(last)


def _check(mss, orc, s, what, pairs=None, use_z=True, use_D=True, use_bias=True, softplus=True):
    go, gl = _run(mss, s, use_z, use_D, use_bias, softplus)
    kw = dict(D=s.D if use_D else None, z=s.z if use_z else None, dt_bias=s.dt_bias if use_bias else None,
              softplus_flag=softplus, pairs=pairs)
    ro, rl = orc.ssd_scan(s.x, s.dt, s.A, s.B, s.C, **kw)
    mo, ml = orc.ssd_scan(s.x, s.dt, s.A, s.B, s.C, magnitude=True, **kw)
    H = s.x.shape[2]
    if pairs is not None:
        sel = [(p // H, p % H) for p in pairs]
        go = np.stack([go[b, :, h] for b, h in sel]); ro = np.stack([ro[b, :, h] for b, h in sel])
        mo = np.stack([mo[b, :, h] for b, h in sel])
        gl = np.stack([gl[b, h] for b, h in sel]); rl = np.stack([rl[b, h] for b, h in sel])
        ml = np.stack([ml[b, h] for b, h in sel])
    m1 = _close(go, ro, mo, 2e-2, 1e-5, what + " out")
    m2 = _close(gl, rl, ml, 0.0, 1e-6, what + " last_state")
    print(f"[{what}] out worst/limit {m1:.3f}, last_state worst/limit {m2:.3f}", flush=True)


def _cfg(name, **over):
    c = dict(SSD_CONFIGS[name])
    c.update(over)
    return ssd_inputs(c["batch"], c["L"], c["heads"], c["headdim"], c["groups"], c["d_state"], dtype=c["dtype"],
                      with_z=c["with_z"], seed=over.pop("seed", 0) if "seed" in over else 0)


@pytest.mark.parametrize("N", [64, 128])
def test_ssd_tiny(mss, oracle_mod, N):
    _check(mss, oracle_mod, _cfg("ssd_tiny", d_state=N), f"ssd tiny N={N}")


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 200, 333])
def test_ssd_lengths(mss, oracle_mod, L):
    """Sequence lengths that are not whole 64-step chunks, and shorter than one chunk."""
    s = ssd_inputs(2, L, 4, 64, 2, 64, dtype="bf16", with_z=True, seed=10 + L)
    _check(mss, oracle_mod, s, f"ssd L={L}")


@pytest.mark.parametrize("flags", [dict(use_z=False), dict(use_D=False), dict(use_bias=False),
                                   dict(softplus=False, use_bias=False), dict(use_z=False, use_D=False, use_bias=False)])
def test_ssd_optional_arguments(mss, oracle_mod, flags):
    s = ssd_inputs(2, 300, 4, 64, 1, 64, dtype="bf16", with_z=True, seed=30)
    if not flags.get("softplus", True):
        s.dt = round_to_bf16(np.abs(s.dt) * 0.05)  # delta used as given: a valid positive step (bf16-exact)
    _check(mss, oracle_mod, s, f"ssd {flags}", **flags)


@pytest.mark.parametrize("H,G,N", [(6, 3, 64), (8, 2, 128), (4, 4, 128)])
def test_ssd_groups(mss, oracle_mod, H, G, N):
    """Several groups of B / C, heads in contiguous blocks per group."""
    s = ssd_inputs(2, 257, H, 64, G, N, dtype="bf16", with_z=True, seed=40 + H)
    _check(mss, oracle_mod, s, f"ssd H={H} G={G} N={N}")


@pytest.mark.parametrize("name", ["ssd_2p7b_n64", "ssd_2p7b_n128"])
def test_ssd_full_layer_all_heads(mss, oracle_mod, name):
    """The Mamba-2 layer at 2.7B width (4 x 2048 steps, 80 heads of 64, one group): every output
    and final state of all 320 (batch, head) pairs against the oracle."""
    _check(mss, oracle_mod, _cfg(name), name)


@pytest.mark.parametrize("segments", [1, 2, 3, 7, 16])
def test_ssd_segment_splits(mss, oracle_mod, segments, plan):
    """The chunks of each (batch, head) cut into segments (local end states folded into the state
    entering each segment), up to one chunk per segment; a ragged last chunk."""
    plan(ssd_segments=segments)
    s = ssd_inputs(2, 16 * 64 - 20, 4, 64, 2, 128 if segments % 2 else 64, dtype="bf16", with_z=True,
                   seed=60 + segments)
    _check(mss, oracle_mod, s, f"ssd segments={segments}")


def test_ssd_empty_sequence_zeroes_state(mss):
    import torch
    x = torch.empty((2, 0, 4, 64), dtype=torch.bfloat16, device="cuda")
    dt = torch.empty((2, 0, 4), dtype=torch.bfloat16, device="cuda")
    B = torch.empty((2, 0, 1, 64), dtype=torch.bfloat16, device="cuda")
    A = -torch.ones(4, device="cuda")
    out, last = mss.ssd_scan_fwd(x, dt, A, B, B.clone())
    torch.cuda.synchronize()
    assert out.shape == x.shape and torch.count_nonzero(last) == 0


def test_ssd_deterministic(mss):
    s = ssd_inputs(2, 300, 4, 64, 1, 128, dtype="bf16", with_z=True, seed=50)
    a = _run(mss, s)
    b = _run(mss, s)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
