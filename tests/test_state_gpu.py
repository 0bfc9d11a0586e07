"""GPU parity of mss_selective_scan_fwd_with_state (the scan continued from a given state)
against the fp64 oracle, plus the chunked-prefill identity on the GPU: scanning a sequence
in pieces, each from the previous piece's last_state, reproduces one scan of the whole.

Tolerances as in test_parity_gpu.py: fp32 rtol 1e-4 / atol 1e-5; bf16 out rtol 2e-2.
"""
import numpy as np
import pytest

from synth import CONFIGS, scan_inputs
from tests.gpu_helpers import TOL_BF16, TOL_F32, assert_close, dev, host64, run_scan, waves_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mss():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_06_amd as m
    m.load_library()
    return m


def _h0(Bt, Dn, seed, scale=0.5):
    rng = np.random.default_rng(1000 + seed)
    return (scale * rng.standard_normal((Bt, Dn, 16))).astype(np.float32)


def _run(mss, s, h0, **kw):
    u, dl = dev(s.u, s.dtype), dev(s.delta, s.dtype)
    z = dev(s.z, s.dtype) if s.z is not None else None
    return mss.selective_scan_fwd_with_state(u, dl, dev(s.A), dev(s.B), dev(s.C),
                                             None if h0 is None else dev(h0), D=dev(s.D), z=z,
                                             delta_bias=dev(s.delta_bias), **kw)


def _check(mss, orc, s, h0, rows=None, what=""):
    import torch
    out, last = _run(mss, s, h0)
    torch.cuda.synchronize()
    ref_out, ref_last = orc.selective_scan(s.u, s.delta, s.A, s.B, s.C, D=s.D, z=s.z,
                                           delta_bias=s.delta_bias, rows=rows, h0=h0)
    Bt, Dn, L = s.u.shape
    go, gl = host64(out).reshape(Bt * Dn, L), host64(last).reshape(Bt * Dn, 16)
    if rows is None:
        ref_out, ref_last = ref_out.reshape(Bt * Dn, L), ref_last.reshape(Bt * Dn, 16)
    else:
        go, gl = go[rows], gl[rows]
    tol = TOL_BF16 if s.dtype == "bf16" else TOL_F32
    r1 = assert_close(go, ref_out, what=what + " out", **tol)
    r2 = assert_close(gl, ref_last, what=what + " last_state", **TOL_F32)
    print(f"[{what}] out {r1:.3f} last_state {r2:.3f} of the limit", flush=True)


@pytest.mark.parametrize("Bt,Dn,L,dtype,a_kind", [
    (1, 64, 1, "f32", "s4d"), (2, 70, 100, "f32", "s4d"), (2, 128, 700, "f32", "random"),
    (1, 100, 129, "bf16", "s4d"), (2, 192, 520, "bf16", "s4d"), (1, 128, 400, "bf16", "random"),
    (2, 5, 33, "f32", "s4d")])
def test_with_state_parity(mss, oracle_mod, Bt, Dn, L, dtype, a_kind):
    s = scan_inputs(Bt, Dn, 16, L, dtype=dtype, seed=40 + L, a_kind=a_kind)
    _check(mss, oracle_mod, s, _h0(Bt, Dn, L), what=f"h0 {Bt}x{Dn}x{L} {dtype} {a_kind}")


@pytest.mark.parametrize("segments", ["1", "2", "5", "64"])
def test_with_state_segment_splits(mss, oracle_mod, segments, plan):
    plan(fast_waves=waves_for(1, 128, segments))
    s = scan_inputs(1, 128, 16, 1000, dtype="f32", seed=41)
    _check(mss, oracle_mod, s, _h0(1, 128, 41), what=f"h0 segments={segments}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_with_state_generic_path(mss, oracle_mod, dtype, plan):
    plan(force_generic=True)
    s = scan_inputs(2, 96, 16, 300, dtype=dtype, seed=42)
    _check(mss, oracle_mod, s, _h0(2, 96, 42), what=f"h0 generic {dtype}")


def test_with_state_mamba2p8b_all_rows(mss, oracle_mod):
    """The 2.8B layer continued from a given state: all 20480 rows against the oracle."""
    c = CONFIGS["mamba2p8b_bf16"]
    s = scan_inputs(c["batch"], c["d_inner"], 16, c["L"], dtype="bf16", seed=43)
    h0 = _h0(c["batch"], c["d_inner"], 43)
    _check(mss, oracle_mod, s, h0, what="h0 mamba2p8b")


def test_zero_or_absent_state_is_the_plain_scan(mss):
    """initial_state NULL or all zeros gives the plain forward scan bit for bit."""
    import torch
    s = scan_inputs(2, 128, 16, 1500, dtype="bf16", seed=44)
    o0, l0 = run_scan(mss, s)
    o1, l1 = _run(mss, s, None)
    o2, l2 = _run(mss, s, np.zeros((2, 128, 16), np.float32))
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert torch.equal(o0, o2) and torch.equal(l0, l2)


def test_empty_sequence_copies_state(mss):
    import torch
    h0 = dev(_h0(2, 64, 45))
    u = torch.empty((2, 64, 0), dtype=torch.float32, device="cuda")
    A = dev(-np.tile(np.arange(1, 17, dtype=np.float32), (64, 1)))
    B = torch.empty((2, 16, 0), dtype=torch.float32, device="cuda")
    out, last = mss.selective_scan_fwd_with_state(u, u.clone(), A, B, B.clone(), h0)
    torch.cuda.synchronize()
    assert out.shape == (2, 64, 0) and torch.equal(last, h0)


@pytest.mark.parametrize("dtype,cuts", [("f32", [0, 96, 97, 500, 1024]),
                                        ("bf16", [0, 256, 640, 2048]),
                                        ("bf16", [0, 1, 33, 2048])])
def test_chunked_prefill_equals_one_scan(mss, oracle_mod, dtype, cuts):
    """Scan [c_k, c_k+1) from the previous chunk's last_state; compare with the oracle's one scan."""
    import torch
    L = cuts[-1]
    s = scan_inputs(2, 192, 16, L, dtype=dtype, seed=46 + L)
    state = None
    outs = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        piece = scan_inputs(2, 192, 16, L, dtype=dtype, seed=46 + L)
        for name in ("u", "delta", "z", "B", "C"):
            setattr(piece, name, np.ascontiguousarray(getattr(s, name)[..., a:b]))
        o, state_next = _run(mss, piece, None) if state is None else _run_dev_state(mss, piece, state)
        outs.append(o)
        state = state_next
    torch.cuda.synchronize()
    ref_out, ref_last = oracle_mod.selective_scan(s.u, s.delta, s.A, s.B, s.C, D=s.D, z=s.z,
                                                  delta_bias=s.delta_bias)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    assert_close(host64(torch.cat(outs, dim=-1)), ref_out, what="chunked out", **tol)
    assert_close(host64(state), ref_last, what="chunked state", **TOL_F32)


def _run_dev_state(mss, s, state):
    u, dl = dev(s.u, s.dtype), dev(s.delta, s.dtype)
    return mss.selective_scan_fwd_with_state(u, dl, dev(s.A), dev(s.B), dev(s.C), state,
                                             D=dev(s.D), z=dev(s.z, s.dtype),
                                             delta_bias=dev(s.delta_bias))


def test_state_buffer_reuse_is_rejected(mss):
    """last_state may not be initial_state: the call fails before any launch."""
    import torch
    s = scan_inputs(1, 64, 16, 64, dtype="f32", seed=47)
    h = dev(_h0(1, 64, 47))
    keep = h.clone()
    with pytest.raises(mss.MssError) as e:
        mss.selective_scan_fwd_with_state(dev(s.u), dev(s.delta), dev(s.A), dev(s.B), dev(s.C), h,
                                          last_state=h)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert torch.equal(h, keep)
