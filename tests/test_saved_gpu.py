"""GPU parity of the forward that saves states (mss_selective_scan_fwd_save) and the backward
that reads them (mss_selective_scan_bwd_saved) against the fp64 oracle.

The saved state at index k is the recurrence's state entering step 8k.  The oracle's definition
of it: the final state of the same scan stopped after min(len_b, 8k) steps (the state is held
past a sequence's end), which is the oracle's varlen scan with those lengths.  Tolerances as
for last_state (fp32 rtol 1e-4 / atol 1e-5); gradients as in test_bwd_gpu.py (rtol 1e-4 of the
sum of |terms| behind each element, atol 1e-6; bf16 du / ddelta / dz also 2e-2 of |ref|).
"""
import numpy as np
import pytest

from synth import CONFIGS, scan_inputs
from tests.gpu_helpers import TOL_F32, assert_close, dev, host64, waves_for

pytestmark = pytest.mark.gpu

RTOL_SUM = 1e-4
ATOL = 1e-6
ROUNDED = ("du", "ddelta", "dz")
GRADS = ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias")


@pytest.fixture(scope="module")
def mss():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_06_amd as m
    m.load_library()
    return m


def _extras(s, seed, with_h0, with_lens):
    Bt, Dn, L = s.u.shape
    rng = np.random.default_rng(900 + seed)
    h0 = (0.5 * rng.standard_normal((Bt, Dn, 16))).astype(np.float32) if with_h0 else None
    lens = None
    if with_lens:
        lens = np.array(([0, 1, 8, L // 2 + 3, L, L - 1, 9] * 4)[:Bt], dtype=np.int32).clip(0, L)
    dout = rng.standard_normal(s.u.shape).astype(np.float32)
    if s.dtype == "bf16":
        from synth import round_to_bf16
        dout = round_to_bf16(dout)
    dlast = rng.standard_normal((Bt, Dn, 16)).astype(np.float32)
    return h0, lens, dout, dlast


def _fwd_save(mss, s, h0, lens):
    import torch
    z = dev(s.z, s.dtype) if s.z is not None else None
    return mss.selective_scan_fwd_save(
        dev(s.u, s.dtype), dev(s.delta, s.dtype), dev(s.A), dev(s.B), dev(s.C), D=dev(s.D), z=z,
        delta_bias=dev(s.delta_bias), initial_state=None if h0 is None else dev(h0),
        seq_lens=None if lens is None else torch.from_numpy(lens).to("cuda"))


@pytest.mark.parametrize("Bt,Dn,L,dtype,with_h0,with_lens", [
    (2, 64, 64, "f32", False, False), (3, 70, 37, "f32", True, True),
    (2, 128, 200, "bf16", False, False), (4, 96, 131, "bf16", True, True),
    (1, 64, 1, "f32", True, False), (1, 5, 17, "bf16", False, False)])
def test_saved_states_match_oracle(mss, oracle_mod, Bt, Dn, L, dtype, with_h0, with_lens):
    import torch
    s = scan_inputs(Bt, Dn, 16, L, dtype=dtype, seed=90 + L)
    h0, lens, _, _ = _extras(s, L, with_h0, with_lens)
    out, last, saved = _fwd_save(mss, s, h0, lens)
    # the forward without saving: out and last_state bit for bit
    args = (dev(s.u, s.dtype), dev(s.delta, s.dtype), dev(s.A), dev(s.B), dev(s.C))
    kw = dict(initial_state=None if h0 is None else dev(h0), D=dev(s.D), z=dev(s.z, s.dtype),
              delta_bias=dev(s.delta_bias))
    if lens is None:
        ref_out, ref_last = mss.selective_scan_fwd_with_state(*args, **kw)
    else:
        ref_out, ref_last = mss.selective_scan_fwd_varlen(*args, torch.from_numpy(lens).to("cuda"), **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(last, ref_last)
    full = lens if lens is not None else np.full(Bt, L, np.int32)
    assert saved.shape == ((L + 7) // 8, 4, Bt * Dn * 4)
    got = host64(mss.saved_state_blocks(saved))
    for k in range(got.shape[0]):
        _, want = oracle_mod.selective_scan(s.u, s.delta, s.A, s.B, s.C, D=s.D, z=s.z,
                                            delta_bias=s.delta_bias, h0=h0,
                                            seq_lens=np.minimum(full, 8 * k))
        assert_close(got[k], want.reshape(Bt * Dn, 16), what=f"saved[{k}]", **TOL_F32)


@pytest.mark.parametrize("segments", ["1", "2", "5", "40"])
def test_saved_states_segment_splits(mss, oracle_mod, segments, plan):
    """The forward split along L into segments (each starts from the carried state)."""
    import torch
    plan(fast_waves=waves_for(2, 64, segments))
    s = scan_inputs(2, 64, 16, 520, dtype="bf16", seed=93)
    h0, lens, _, _ = _extras(s, 93, True, True)
    _, last, saved = _fwd_save(mss, s, h0, lens)
    torch.cuda.synchronize()
    got = host64(mss.saved_state_blocks(saved))
    for k in range(0, got.shape[0], 5):
        _, want = oracle_mod.selective_scan(s.u, s.delta, s.A, s.B, s.C, D=s.D, z=s.z,
                                            delta_bias=s.delta_bias, h0=h0,
                                            seq_lens=np.minimum(lens, 8 * k))
        assert_close(got[k], want.reshape(-1, 16), what=f"saved[{k}]", **TOL_F32)


def _bwd_saved(mss, s, saved, dout, lens, dlast):
    import torch
    z = dev(s.z, s.dtype) if s.z is not None else None
    return mss.selective_scan_bwd(
        dev(s.u, s.dtype), dev(s.delta, s.dtype), dev(s.A), dev(s.B), dev(s.C), dev(dout, s.dtype),
        D=dev(s.D), z=z, delta_bias=dev(s.delta_bias),
        seq_lens=None if lens is None else torch.from_numpy(lens).to("cuda"),
        dlast_state=None if dlast is None else dev(dlast), return_dinitial_state=True,
        saved_states=saved)


def _check_grads(orc, s, g, dout, h0, lens, dlast, what):
    kw = dict(D=s.D, z=s.z, delta_bias=s.delta_bias, dout=dout, h0=h0, seq_lens=lens, dlast=dlast)
    ref = orc.selective_scan_bwd(s.u, s.delta, s.A, s.B, s.C, **kw)
    mag = orc.selective_scan_bwd(s.u, s.delta, s.A, s.B, s.C, magnitude=True, **kw)
    worst = {}
    for k in GRADS:
        got = host64(g[k])
        assert np.all(np.isfinite(got)), (what, k)
        rtol_out = 2e-2 if (k in ROUNDED and s.dtype == "bf16") else 0.0
        lim = rtol_out * np.abs(ref[k]) + RTOL_SUM * mag[k] + ATOL
        ratio = np.abs(got - ref[k]) / lim
        worst[k] = float(ratio.max()) if ratio.size else 0.0
        assert worst[k] <= 1.0, (what, k, int((ratio > 1).sum()), worst[k])
    got, want = host64(g["dinitial_state"]), ref["dh0"]
    np.testing.assert_allclose(got, want, rtol=1e-4, atol=1e-5 * max(np.abs(want).max(), 1e-30),
                               err_msg=what + " dinitial_state")
    print(f"[{what}] worst err/limit: " + ", ".join(f"{k} {v:.3f}" for k, v in worst.items()),
          flush=True)


@pytest.mark.parametrize("Bt,Dn,L,dtype,with_h0,with_lens,nan_pad", [
    (2, 64, 64, "f32", False, False, False), (2, 70, 33, "f32", True, True, False),
    (1, 130, 200, "f32", False, False, False), (2, 128, 256, "bf16", True, False, False),
    (4, 64, 256, "bf16", True, True, False), (4, 64, 256, "bf16", True, True, True),
    (4, 70, 101, "f32", True, True, True), (3, 5, 17, "bf16", False, True, False),
    (1, 64, 1, "f32", True, False, False)])
def test_bwd_saved_parity(mss, oracle_mod, Bt, Dn, L, dtype, with_h0, with_lens, nan_pad):
    """nan_pad: past each sequence's end u, delta, z, B, C and dout hold NaN / inf (the oracle
    never reads them); neither the saved states nor any gradient may pick them up."""
    import torch
    s = scan_inputs(Bt, Dn, 16, L, dtype=dtype, seed=95 + L)
    h0, lens, dout, dlast = _extras(s, L, with_h0, with_lens)
    if nan_pad:
        for b, n in enumerate(lens):
            s.u[b, :, n:] = np.nan
            s.delta[b, :, n:] = np.inf
            s.z[b, :, n:] = np.nan
            s.B[b, :, n:] = np.inf
            s.C[b, :, n:] = np.nan
            dout[b, :, n:] = np.nan
    _, _, saved = _fwd_save(mss, s, h0, lens)
    g = _bwd_saved(mss, s, saved, dout, lens, dlast)
    torch.cuda.synchronize()
    _check_grads(oracle_mod, s, g, dout, h0, lens, dlast, f"bwd_saved {Bt}x{Dn}x{L} {dtype}")
    if lens is not None:
        for k in ("du", "ddelta", "dz"):   # past each sequence's end: exactly zero
            got = host64(g[k])
            for b, lb in enumerate(lens):
                assert not np.any(got[b, :, lb:]), (k, b)


@pytest.mark.parametrize("segments", ["1", "3", "40"])
def test_bwd_saved_segment_splits(mss, oracle_mod, segments, plan):
    import torch
    plan(bwd_segments=int(segments))
    s = scan_inputs(1, 128, 16, 320, dtype="f32", seed=96)
    h0, lens, dout, dlast = _extras(s, 96, True, False)
    _, _, saved = _fwd_save(mss, s, h0, lens)
    g = _bwd_saved(mss, s, saved, dout, lens, dlast)
    torch.cuda.synchronize()
    _check_grads(oracle_mod, s, g, dout, h0, lens, dlast, f"bwd_saved segments={segments}")


@pytest.mark.parametrize("L", [2048, 2047])
def test_bwd_saved_mamba2p8b_full(mss, oracle_mod, L):
    """The 2.8B layer (4 x 5120 x 16, bf16 activations) at full size, every element."""
    import torch
    c = CONFIGS["mamba2p8b_bf16"]
    s = scan_inputs(c["batch"], c["d_inner"], 16, L, dtype="bf16", seed=97)
    _, _, dout, _ = _extras(s, 97, False, False)
    _, _, saved = _fwd_save(mss, s, None, None)
    g = _bwd_saved(mss, s, saved, dout, None, None)
    torch.cuda.synchronize()
    _check_grads(oracle_mod, s, g, dout, None, None, None, f"bwd_saved mamba2p8b L={L}")


def test_bwd_saved_agrees_with_recompute(mss):
    """The two backwards differ only in where the tile-start states come from (saved by the
    forward vs recomputed): gradients agree to fp32 rounding of the states."""
    import torch
    s = scan_inputs(2, 256, 16, 1000, dtype="f32", seed=98)
    h0, lens, dout, dlast = _extras(s, 98, True, True)
    _, _, saved = _fwd_save(mss, s, h0, lens)
    g1 = _bwd_saved(mss, s, saved, dout, lens, dlast)
    g2 = mss.selective_scan_bwd(dev(s.u), dev(s.delta), dev(s.A), dev(s.B), dev(s.C), dev(dout),
                                D=dev(s.D), z=dev(s.z), delta_bias=dev(s.delta_bias),
                                initial_state=dev(h0), seq_lens=torch.from_numpy(lens).to("cuda"),
                                dlast_state=dev(dlast), return_dinitial_state=True)
    g1b = _bwd_saved(mss, s, saved, dout, lens, dlast)
    torch.cuda.synchronize()
    for k in GRADS + ("dinitial_state",):
        assert torch.equal(g1[k], g1b[k]), k          # deterministic
        a, b = host64(g1[k]), host64(g2[k])
        np.testing.assert_allclose(a, b, rtol=1e-4, atol=1e-5 * np.abs(b).max(), err_msg=k)


def test_autograd_saving_states_matches_oracle(mss, oracle_mod):
    import torch
    s = scan_inputs(2, 96, 16, 200, dtype="f32", seed=99)
    _, _, dout, _ = _extras(s, 99, False, False)
    ts = {k: dev(getattr(s, k)).requires_grad_(True)
          for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")}
    out = mss.SelectiveScanFunction.apply(ts["u"], ts["delta"], ts["A"], ts["B"], ts["C"], ts["D"],
                                          ts["z"], ts["delta_bias"], True, True)
    (out * dev(dout)).sum().backward()
    torch.cuda.synchronize()
    kw = dict(D=s.D, z=s.z, delta_bias=s.delta_bias, dout=dout)
    ref = oracle_mod.selective_scan_bwd(s.u, s.delta, s.A, s.B, s.C, **kw)
    mag = oracle_mod.selective_scan_bwd(s.u, s.delta, s.A, s.B, s.C, magnitude=True, **kw)
    names = dict(u="du", delta="ddelta", A="dA", B="dB", C="dC", D="dD", z="dz", delta_bias="ddelta_bias")
    for k, gk in names.items():
        got = host64(ts[k].grad)
        lim = RTOL_SUM * mag[gk] + ATOL
        assert np.all(np.abs(got - ref[gk]) <= lim), (k, float((np.abs(got - ref[gk]) / lim).max()))


def test_save_empty_sequence(mss):
    import torch
    A = dev(-np.tile(np.arange(1, 17, dtype=np.float32), (64, 1)))
    u = torch.zeros((2, 64, 0), dtype=torch.float32, device="cuda")
    B = torch.zeros((2, 16, 0), dtype=torch.float32, device="cuda")
    out, last, saved = mss.selective_scan_fwd_save(u, u.clone(), A, B, B.clone())
    g = mss.selective_scan_bwd(u, u.clone(), A, B, B.clone(), u.clone(), saved_states=saved)
    torch.cuda.synchronize()
    assert saved.shape == (0, 4, 512) and out.shape == (2, 64, 0)
    assert torch.all(g["dA"] == 0) and torch.all(g["dD"] == 0)
