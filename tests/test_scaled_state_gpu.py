"""GPU parity of the forward's scaled state form (the S4D power path of bf16 rows at d_state 16
and of every row at d_state 128) on inputs that stress it: the kernels keep the state divided by
the step scale s_t = delta_t u_t + copysign(2^-40, delta_t u_t), so these cases put exact zeros,
values near the bottom of the bf16 / fp32 range and very large inputs into delta u, mixed within
a row, and compare every output and final state with the fp64 oracle.

Large inputs make large states whose C . h cancels down to ordinary outputs, which no fp32
evaluation resolves to rtol |ref| (a plain fp32 recurrence misses one such output, -0.00188 from
terms summing to 3800 in absolute value, by 2.3e-4).  So the bound here adds the magnitude term
of the backward's and the SSD layer's tolerances: |gpu - ref| <= atol + rtol |ref| + 1e-6 M, with M
the sum of the absolute values of the terms behind the element (computed below in fp64 from the
same recurrence with every term taken in absolute value), rtol / atol as in test_parity_gpu.
"""
import numpy as np
import pytest

from synth import round_to_bf16, scan_inputs
from tests.gpu_helpers import TOL_BF16, TOL_F32, assert_close, host64, oracle_scan, record_margin, run_scan

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mss():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_06_amd as m
    m.load_library()  # raises if the HIP library is not built: no fallback
    return m


def _stressed(Bt, Dn, N, L, dtype, seed):
    """Seeded scan inputs with S4D A whose delta u spans zero, the underflow range and large
    magnitudes: per row a random mix of exact zeros and tiny u, delta_raw far below the bias
    (delta ~ e^-60) or far above it (delta ~ 20), and u up to 64."""
    s = scan_inputs(Bt, Dn, N, L, dtype=dtype, with_z=True, seed=seed, a_kind="s4d")
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    u, d = s.u.copy(), s.delta.copy()
    pick = rng.random(u.shape)
    u[pick < 0.15] = 0.0                                       # delta u = 0 exactly
    tiny = (pick >= 0.15) & (pick < 0.25)
    u[tiny] = 1e-30 * np.sign(u[tiny] + 0.5)                   # delta u underflows in fp32
    big = (pick >= 0.25) & (pick < 0.30)
    u[big] = 64.0 * np.sign(u[big] + 0.5)
    pd = rng.random(d.shape)
    d[pd < 0.1] = -60.0                                        # delta ~ e^-60
    d[(pd >= 0.1) & (pd < 0.15)] = 20.0                        # delta ~ 20: abar ~ e^-20 (n+1)
    if dtype == "bf16":
        u, d = round_to_bf16(u), round_to_bf16(d)
    s.u, s.delta = u.astype(np.float32), d.astype(np.float32)
    return s


def _magnitudes(s):
    """M of every output and final-state element: the recurrence with each term in absolute value
    (|abar| h + |delta u B|, then |C| . h + |D u|, times |silu(z)| for the output)."""
    u, raw = s.u.astype(np.float64), s.delta.astype(np.float64)
    dt = np.logaddexp(0.0, raw + s.delta_bias.astype(np.float64)[None, :, None])
    A = s.A.astype(np.float64)                                        # (Dn, N)
    Bm, Cm = np.abs(s.B.astype(np.float64)), np.abs(s.C.astype(np.float64))   # (Bt, N, L)
    Bt, Dn, L = u.shape
    hm = np.zeros((Bt, Dn, A.shape[1]))
    mo = np.empty((Bt, Dn, L))
    zz = s.z.astype(np.float64)
    sil = np.abs(zz / (1.0 + np.exp(-zz)))
    for t in range(L):
        hm = np.exp(dt[:, :, t, None] * A[None]) * hm + np.abs(dt[:, :, t] * u[:, :, t])[..., None] * Bm[:, None, :, t]
        mo[:, :, t] = (np.einsum("bdn,bn->bd", hm, Cm[:, :, t]) + np.abs(s.D[None, :] * u[:, :, t])) * sil[:, :, t]
    return mo, hm


def _close_mag(gpu, ref, mag, rtol, atol, what):
    err = np.abs(gpu - ref)
    lim = atol + rtol * np.abs(ref) + 1e-6 * mag
    bad = err > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} out of tolerance; worst "
                           f"err {err.flat[np.argmax(err - lim)]:.3e} lim {lim.flat[np.argmax(err - lim)]:.3e}")
    return float((err / lim).max())


@pytest.mark.parametrize("Bt,Dn,N,L,dtype", [
    (2, 128, 16, 520, "bf16"),     # fast path, scaled step; a ragged last tile
    (1, 192, 16, 2048, "bf16"),    # fast path over several pieces per group
    (2, 96, 16, 300, "f32"),       # fast path, plain step (fp32 rows), same inputs
    (2, 64, 128, 333, "bf16"),     # general path at d_state 128, scaled step
    (1, 48, 128, 256, "f32"),      # general path at d_state 128 with fp32 rows
])
def test_scaled_state_stressed_inputs(mss, oracle_mod, Bt, Dn, N, L, dtype):
    import torch
    s = _stressed(Bt, Dn, N, L, dtype, seed=Bt * 1000 + N + L)
    out, last = run_scan(mss, s)
    torch.cuda.synchronize()
    ref_out, ref_last = oracle_scan(oracle_mod, s)
    what = f"scaled stress {Bt}x{Dn}x{N}x{L} {dtype}"
    go, gl = host64(out).reshape(Bt * Dn, L), host64(last).reshape(Bt * Dn, N)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    m_out, m_last = _magnitudes(s)
    mo = record_margin(what + " out", _close_mag(go, ref_out.reshape(Bt * Dn, L), m_out.reshape(Bt * Dn, L),
                                                 what=what + " out", **tol))
    ml = record_margin(what + " last_state", _close_mag(gl, ref_last.reshape(Bt * Dn, N), m_last.reshape(Bt * Dn, N),
                                                        what=what + " last_state", **TOL_F32))
    print(f"[{what}] out worst/limit = {mo:.3f}, last_state worst/limit = {ml:.3f}", flush=True)


def test_scaled_state_zero_input_rows(mss, oracle_mod):
    """Rows whose u is zero at every step: the recurrence adds nothing (h = 0, out = 0); the scaled
    step adds 2^-40 B per step, so the final state stays within 2^-40 sum |B| of zero."""
    import torch
    s = scan_inputs(2, 128, 16, 512, dtype="bf16", with_z=True, seed=77, a_kind="s4d")
    s.u[:, :64, :] = 0.0
    out, last = run_scan(mss, s)
    torch.cuda.synchronize()
    go = host64(out).reshape(2, 128, 512)
    gl = host64(last).reshape(2, 128, 16)
    # |h_t[n]| <= 2^-40 sum_t |B_t[n]| (each step adds at most 2^-40 |B_t[n]|, decays only shrink
    # it), and |out_t| <= |silu(z_t)| sum_n |C_t[n]| that bound, with |silu(z)| <= |z|
    hb = 2.0 ** -40 * np.abs(s.B).sum(axis=2)                                   # (batch, N)
    ob = np.einsum("bnt,bn->bt", np.abs(s.C), hb)[:, None, :] * np.abs(s.z[:, :64, :])
    assert np.all(np.abs(gl[:, :64, :]) <= 1.01 * hb[:, None, :])
    assert np.all(np.abs(go[:, :64, :]) <= 1.01 * ob)
    ref_out, ref_last = oracle_scan(oracle_mod, s)
    assert_close(go.reshape(256, 512), ref_out.reshape(256, 512), what="zero rows out", **TOL_BF16)
    assert_close(gl.reshape(256, 16), ref_last.reshape(256, 16), what="zero rows last_state", **TOL_F32)
