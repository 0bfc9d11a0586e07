"""Seeded random sweep of shapes and options through every GPU entry point, each case against the
fp64 oracle: the hand-picked cases elsewhere cover the structure; this covers combinations of
batch / channels / length / dtype / A kind / optional arguments / lengths / starting states /
misaligned views / segment counts / d_state that nobody picked.

Each case prints its parameters before running, so a failure names the case.  Tolerances as in
test_parity_gpu.py (forward, conv) and test_bwd_gpu.py (backward).
"""
import numpy as np
import pytest

from synth import scan_inputs
from tests.gpu_helpers import TOL_BF16, TOL_F32, assert_close, dev, host64

pytestmark = pytest.mark.gpu

N_CASES = 24


@pytest.fixture(scope="module")
def mss():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_06_amd as m
    m.load_library()
    return m


def _case(i):
    rng = np.random.default_rng(7000 + i)
    return dict(
        Bt=int(rng.integers(1, 5)), Dn=int(rng.choice([1, 7, 64, 65, 130, 200])),
        L=int(rng.choice([1, 2, 5, 16, 31, 64, 100, 257, 600, 1024])),
        dtype=str(rng.choice(["f32", "bf16"])), a_kind=str(rng.choice(["s4d", "random"])),
        use_z=bool(rng.random() < 0.7), use_D=bool(rng.random() < 0.8),
        use_bias=bool(rng.random() < 0.8), with_h0=bool(rng.random() < 0.4),
        with_lens=bool(rng.random() < 0.4), offset=bool(rng.random() < 0.25),
        segments=int(rng.choice([0, 0, 1, 3, 9])), seed=int(rng.integers(0, 1 << 30)))


def _sweep_waves(c):
    """Wavefronts for a forced split: `segments` pieces per 64-channel group plus one, so that
    wavefront ranges start and end inside groups and cross from one group into the next."""
    return c["segments"] * c["Bt"] * ((c["Dn"] + 63) // 64) + 1


def _to_dev(a, dtype, offset):
    """Device copy; with offset, a view one element into a larger buffer (rows lose alignment)."""
    import torch
    t = dev(a, dtype)
    if not offset:
        return t
    flat = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = flat[1:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("i", range(N_CASES))
def test_forward_sweep(mss, oracle_mod, plan, i):
    import torch
    c = _case(i)
    print(f"[sweep fwd {i}] {c}", flush=True)
    if c["segments"]:
        plan(fast_waves=_sweep_waves(c))
    s = scan_inputs(c["Bt"], c["Dn"], 16, c["L"], dtype=c["dtype"], seed=c["seed"] % 100000,
                    a_kind=c["a_kind"], with_z=c["use_z"])
    rng = np.random.default_rng(c["seed"])
    h0 = (0.5 * rng.standard_normal((c["Bt"], c["Dn"], 16))).astype(np.float32) if c["with_h0"] else None
    lens = rng.integers(0, c["L"] + 1, c["Bt"]).astype(np.int32) if c["with_lens"] else None
    dt = c["dtype"]
    args = [_to_dev(s.u, dt, c["offset"]), _to_dev(s.delta, dt, c["offset"]), dev(s.A), dev(s.B), dev(s.C)]
    kw = dict(D=dev(s.D) if c["use_D"] else None,
              z=_to_dev(s.z, dt, c["offset"]) if c["use_z"] else None,
              delta_bias=dev(s.delta_bias) if c["use_bias"] else None)
    if lens is not None:
        out, last = mss.selective_scan_fwd_varlen(*args, torch.from_numpy(lens).to("cuda"),
                                                  initial_state=None if h0 is None else dev(h0), **kw)
    else:
        out, last = mss.selective_scan_fwd_with_state(*args, None if h0 is None else dev(h0), **kw)
    torch.cuda.synchronize()
    ref_out, ref_last = oracle_mod.selective_scan(
        s.u, s.delta, s.A, s.B, s.C, D=s.D if c["use_D"] else None, z=s.z if c["use_z"] else None,
        delta_bias=s.delta_bias if c["use_bias"] else None, h0=h0, seq_lens=lens)
    assert_close(host64(out), ref_out, what=f"sweep fwd {i} out", **(TOL_BF16 if dt == "bf16" else TOL_F32))
    assert_close(host64(last), ref_last, what=f"sweep fwd {i} last_state", **TOL_F32)


@pytest.mark.parametrize("i", range(12))
def test_forward_dstate_sweep(mss, oracle_mod, plan, i):
    """The same sweep at d_state 32, 64 and 128 (the general kernels), with forced segment counts."""
    import torch
    c = _case(100 + i)
    N = int(np.random.default_rng(8000 + i).choice([32, 64, 128]))
    print(f"[sweep fwd d_state {N} {i}] {c}", flush=True)
    if c["segments"]:
        plan(generic_segments=c["segments"])
    s = scan_inputs(c["Bt"], c["Dn"], N, c["L"], dtype=c["dtype"], seed=c["seed"] % 100000,
                    a_kind=c["a_kind"], with_z=c["use_z"])
    rng = np.random.default_rng(c["seed"])
    h0 = (0.5 * rng.standard_normal((c["Bt"], c["Dn"], N))).astype(np.float32) if c["with_h0"] else None
    lens = rng.integers(0, c["L"] + 1, c["Bt"]).astype(np.int32) if c["with_lens"] else None
    dt = c["dtype"]
    args = [_to_dev(s.u, dt, c["offset"]), _to_dev(s.delta, dt, c["offset"]), dev(s.A), dev(s.B), dev(s.C)]
    kw = dict(D=dev(s.D) if c["use_D"] else None,
              z=_to_dev(s.z, dt, c["offset"]) if c["use_z"] else None,
              delta_bias=dev(s.delta_bias) if c["use_bias"] else None)
    if lens is not None:
        out, last = mss.selective_scan_fwd_varlen(*args, torch.from_numpy(lens).to("cuda"),
                                                  initial_state=None if h0 is None else dev(h0), **kw)
    else:
        out, last = mss.selective_scan_fwd_with_state(*args, None if h0 is None else dev(h0), **kw)
    torch.cuda.synchronize()
    ref_out, ref_last = oracle_mod.selective_scan(
        s.u, s.delta, s.A, s.B, s.C, D=s.D if c["use_D"] else None, z=s.z if c["use_z"] else None,
        delta_bias=s.delta_bias if c["use_bias"] else None, h0=h0, seq_lens=lens)
    what = f"sweep fwd d_state {N} {i}"
    assert_close(host64(out), ref_out, what=what + " out", **(TOL_BF16 if dt == "bf16" else TOL_F32))
    assert_close(host64(last), ref_last, what=what + " last_state", **TOL_F32)


@pytest.mark.parametrize("i", range(0, N_CASES, 2))
def test_backward_sweep(mss, oracle_mod, plan, i):
    import torch
    c = _case(i)
    print(f"[sweep bwd {i}] {c}", flush=True)
    if c["segments"]:
        plan(bwd_segments=c["segments"])
    s = scan_inputs(c["Bt"], c["Dn"], 16, c["L"], dtype=c["dtype"], seed=c["seed"] % 100000,
                    a_kind=c["a_kind"], with_z=c["use_z"])
    rng = np.random.default_rng(c["seed"] + 1)
    dout = rng.standard_normal(s.u.shape).astype(np.float32)
    if c["dtype"] == "bf16":
        from synth import round_to_bf16
        dout = round_to_bf16(dout)
    h0 = (0.5 * rng.standard_normal((c["Bt"], c["Dn"], 16))).astype(np.float32) if c["with_h0"] else None
    dlast = rng.standard_normal((c["Bt"], c["Dn"], 16)).astype(np.float32) if c["with_h0"] else None
    lens = rng.integers(0, c["L"] + 1, c["Bt"]).astype(np.int32) if c["with_lens"] else None
    dt = c["dtype"]
    g = mss.selective_scan_bwd(
        _to_dev(s.u, dt, c["offset"]), _to_dev(s.delta, dt, c["offset"]), dev(s.A), dev(s.B),
        dev(s.C), _to_dev(dout, dt, c["offset"]), D=dev(s.D) if c["use_D"] else None,
        z=_to_dev(s.z, dt, c["offset"]) if c["use_z"] else None,
        delta_bias=dev(s.delta_bias) if c["use_bias"] else None,
        initial_state=None if h0 is None else dev(h0),
        seq_lens=None if lens is None else torch.from_numpy(lens).to("cuda"),
        dlast_state=None if dlast is None else dev(dlast))
    torch.cuda.synchronize()
    kw = dict(D=s.D if c["use_D"] else None, z=s.z if c["use_z"] else None,
              delta_bias=s.delta_bias if c["use_bias"] else None, dout=dout, h0=h0,
              seq_lens=lens, dlast=dlast)
    ref = oracle_mod.selective_scan_bwd(s.u, s.delta, s.A, s.B, s.C, **kw)
    mag = oracle_mod.selective_scan_bwd(s.u, s.delta, s.A, s.B, s.C, magnitude=True, **kw)
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias"):
        if ref[k] is None:
            continue
        got = host64(g[k])
        rtol_out = 2e-2 if (k in ("du", "ddelta", "dz") and dt == "bf16") else 0.0
        lim = rtol_out * np.abs(ref[k]) + 1e-4 * mag[k] + 1e-6
        ratio = np.abs(got - ref[k]) / lim
        assert np.all(np.isfinite(got)) and ratio.max() <= 1.0, (i, k, float(ratio.max()))


@pytest.mark.parametrize("i", range(1, N_CASES, 2))
def test_saved_states_sweep(mss, oracle_mod, plan, i):
    """The forward that saves states, then the backward from them (the cases the backward sweep
    above skips): out, last_state, the first and last saved blocks and every gradient."""
    import torch
    c = _case(i)
    print(f"[sweep saved {i}] {c}", flush=True)
    if c["segments"]:
        plan(fast_waves=_sweep_waves(c), bwd_segments=c["segments"])
    s = scan_inputs(c["Bt"], c["Dn"], 16, c["L"], dtype=c["dtype"], seed=c["seed"] % 100000,
                    a_kind=c["a_kind"], with_z=c["use_z"])
    rng = np.random.default_rng(c["seed"] + 2)
    dout = rng.standard_normal(s.u.shape).astype(np.float32)
    if c["dtype"] == "bf16":
        from synth import round_to_bf16
        dout = round_to_bf16(dout)
    h0 = (0.5 * rng.standard_normal((c["Bt"], c["Dn"], 16))).astype(np.float32) if c["with_h0"] else None
    dlast = rng.standard_normal((c["Bt"], c["Dn"], 16)).astype(np.float32) if c["with_h0"] else None
    lens = rng.integers(0, c["L"] + 1, c["Bt"]).astype(np.int32) if c["with_lens"] else None
    dt = c["dtype"]
    u, delta = _to_dev(s.u, dt, c["offset"]), _to_dev(s.delta, dt, c["offset"])
    z = _to_dev(s.z, dt, c["offset"]) if c["use_z"] else None
    D = dev(s.D) if c["use_D"] else None
    bias = dev(s.delta_bias) if c["use_bias"] else None
    lens_d = None if lens is None else torch.from_numpy(lens).to("cuda")
    out, last, saved = mss.selective_scan_fwd_save(u, delta, dev(s.A), dev(s.B), dev(s.C), D=D, z=z,
                                                   delta_bias=bias, initial_state=None if h0 is None else dev(h0),
                                                   seq_lens=lens_d)
    g = mss.selective_scan_bwd(u, delta, dev(s.A), dev(s.B), dev(s.C), _to_dev(dout, dt, c["offset"]), D=D, z=z,
                               delta_bias=bias, seq_lens=lens_d, dlast_state=None if dlast is None else dev(dlast),
                               saved_states=saved)
    torch.cuda.synchronize()
    okw = dict(D=s.D if c["use_D"] else None, z=s.z if c["use_z"] else None,
               delta_bias=s.delta_bias if c["use_bias"] else None, h0=h0)
    ref_out, ref_last = oracle_mod.selective_scan(s.u, s.delta, s.A, s.B, s.C, seq_lens=lens, **okw)
    assert_close(host64(out), ref_out, what=f"sweep saved {i} out", **(TOL_BF16 if dt == "bf16" else TOL_F32))
    assert_close(host64(last), ref_last, what=f"sweep saved {i} last_state", **TOL_F32)
    blocks = host64(mss.saved_state_blocks(saved))
    full = lens if lens is not None else np.full(c["Bt"], c["L"], np.int32)
    for k in sorted({0, blocks.shape[0] - 1}):
        _, want = oracle_mod.selective_scan(s.u, s.delta, s.A, s.B, s.C, seq_lens=np.minimum(full, 8 * k), **okw)
        assert_close(blocks[k], want.reshape(-1, 16), what=f"sweep saved {i} block {k}", **TOL_F32)
    kw = dict(D=okw["D"], z=okw["z"], delta_bias=okw["delta_bias"], dout=dout, h0=h0, seq_lens=lens, dlast=dlast)
    ref = oracle_mod.selective_scan_bwd(s.u, s.delta, s.A, s.B, s.C, **kw)
    mag = oracle_mod.selective_scan_bwd(s.u, s.delta, s.A, s.B, s.C, magnitude=True, **kw)
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias"):
        if ref[k] is None:
            continue
        got = host64(g[k])
        rtol_out = 2e-2 if (k in ("du", "ddelta", "dz") and dt == "bf16") else 0.0
        lim = rtol_out * np.abs(ref[k]) + 1e-4 * mag[k] + 1e-6
        ratio = np.abs(got - ref[k]) / lim
        assert np.all(np.isfinite(got)) and ratio.max() <= 1.0, (i, k, float(ratio.max()))


@pytest.mark.parametrize("i", range(N_CASES))
def test_conv_sweep(mss, oracle_mod, i):
    import torch
    c = _case(i)
    rng = np.random.default_rng(c["seed"] + 2)
    K = int(rng.integers(1, 5))
    print(f"[sweep conv {i}] {c} K={K}", flush=True)
    x = rng.standard_normal((c["Bt"], c["Dn"], c["L"])).astype(np.float32)
    st = rng.standard_normal((c["Bt"], c["Dn"], K - 1)).astype(np.float32)
    if c["dtype"] == "bf16":
        from synth import round_to_bf16
        x, st = round_to_bf16(x), round_to_bf16(st)
    w = (0.5 * rng.standard_normal((c["Dn"], K))).astype(np.float32)
    b = rng.standard_normal(c["Dn"]).astype(np.float32) if c["use_bias"] else None
    dt = c["dtype"]
    out, fin = mss.causal_conv1d_fwd(_to_dev(x, dt, c["offset"]), dev(w), None if b is None else dev(b),
                                     initial_state=dev(st, dt) if c["with_h0"] else None,
                                     silu=c["use_z"], return_final_state=True)
    torch.cuda.synchronize()
    ref, rfin = oracle_mod.causal_conv1d(x, w, b, state=st if c["with_h0"] else None, silu=c["use_z"])
    assert_close(host64(out), ref, what=f"sweep conv {i}", **(TOL_BF16 if dt == "bf16" else TOL_F32))
    np.testing.assert_array_equal(host64(fin), rfin)
