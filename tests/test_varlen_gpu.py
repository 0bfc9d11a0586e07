"""GPU parity of mss_selective_scan_fwd_varlen (a batch of sequences of different lengths)
against the fp64 oracle: outputs up to each sequence's end, zeros past it, and the state after
each sequence's own last step -- on both paths, every segment split, with and without a
starting state -- plus full lengths giving the plain scan bit for bit and decode continuing from
each sequence's own end.

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


def _lens(Bt, L, seed):
    rng = np.random.default_rng(600 + seed)
    fixed = [0, 1, 3, L, L - 1, max(L // 2 + 1, 0)]
    out = [fixed[i] if i < len(fixed) else int(rng.integers(0, L + 1)) for i in range(Bt)]
    return np.clip(np.array(out, dtype=np.int32), 0, L)


def _run(mss, s, lens, h0=None):
    import torch
    u, dl = dev(s.u, s.dtype), dev(s.delta, s.dtype)
    z = dev(s.z, s.dtype) if s.z is not None else None
    ld = torch.from_numpy(lens).to("cuda")
    return mss.selective_scan_fwd_varlen(u, dl, dev(s.A), dev(s.B), dev(s.C), ld,
                                         initial_state=None if h0 is None else dev(h0), D=dev(s.D),
                                         z=z, delta_bias=dev(s.delta_bias))


def _check(mss, orc, s, lens, h0=None, rows=None, what=""):
    import torch
    out, last = _run(mss, s, lens, h0)
    torch.cuda.synchronize()
    ref_out, ref_last = orc.selective_scan(s.u, s.delta, s.A, s.B, s.C, D=s.D, z=s.z,
                                           delta_bias=s.delta_bias, rows=rows, h0=h0, seq_lens=lens)
    Bt, Dn, L = s.u.shape
    go, gl = host64(out).reshape(Bt * Dn, L), host64(last).reshape(Bt * Dn, 16)
    if rows is None:
        ref_out, ref_last = ref_out.reshape(Bt * Dn, L), ref_last.reshape(Bt * Dn, 16)
    else:
        go, gl = go[rows], gl[rows]
    r1 = assert_close(go, ref_out, what=what + " out", **(TOL_BF16 if s.dtype == "bf16" else TOL_F32))
    r2 = assert_close(gl, ref_last, what=what + " last_state", **TOL_F32)
    # past each sequence's end the outputs are exactly zero
    bidx = (np.arange(Bt * Dn) // Dn) if rows is None else (np.asarray(rows) // Dn)
    t = np.arange(L)[None, :]
    assert not np.any(go[t >= lens[bidx][:, None]]), what + ": nonzero output past a sequence's end"
    print(f"[{what}] out {r1:.3f} last_state {r2:.3f} of the limit", flush=True)


@pytest.mark.parametrize("Bt,Dn,L,dtype,a_kind", [
    (6, 64, 256, "bf16", "s4d"), (6, 70, 128, "f32", "s4d"), (8, 128, 520, "bf16", "random"),
    (6, 100, 96, "f32", "random"), (7, 5, 33, "f32", "s4d"), (6, 64, 1, "f32", "s4d")])
@pytest.mark.parametrize("with_h0", [False, True])
def test_varlen_parity(mss, oracle_mod, Bt, Dn, L, dtype, a_kind, with_h0):
    s = scan_inputs(Bt, Dn, 16, L, dtype=dtype, seed=60 + L, a_kind=a_kind)
    h0 = (0.5 * np.random.default_rng(61).standard_normal((Bt, Dn, 16))).astype(np.float32) if with_h0 else None
    _check(mss, oracle_mod, s, _lens(Bt, L, L), h0, what=f"varlen {Bt}x{Dn}x{L} {dtype} {a_kind} h0={with_h0}")


@pytest.mark.parametrize("segments", ["1", "3", "16"])
def test_varlen_segment_splits(mss, oracle_mod, segments, plan):
    plan(fast_waves=waves_for(6, 128, segments))
    s = scan_inputs(6, 128, 16, 1000, dtype="bf16", seed=62)
    _check(mss, oracle_mod, s, _lens(6, 1000, 62), what=f"varlen segments={segments}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_varlen_generic_path(mss, oracle_mod, dtype, plan):
    plan(force_generic=True)
    s = scan_inputs(6, 96, 16, 300, dtype=dtype, seed=63)
    _check(mss, oracle_mod, s, _lens(6, 300, 63), what=f"varlen generic {dtype}")


@pytest.mark.parametrize("dtype,generic", [("bf16", False), ("f32", False), ("bf16", True), ("f32", True)])
def test_varlen_padding_never_reaches_results(mss, oracle_mod, dtype, generic, plan):
    """Past each sequence's end the tensors hold NaN / inf (u, delta, z and B, C of that batch):
    the oracle never reads there, so outputs and final states must match it exactly as with finite
    padding -- masked steps may not multiply padding by zero."""
    if generic:
        plan(force_generic=True)
    Bt, Dn, L = 6, 96, 300
    s = scan_inputs(Bt, Dn, 16, L, dtype=dtype, seed=66)
    lens = _lens(Bt, L, 66)
    for b, n in enumerate(lens):
        s.u[b, :, n:] = np.nan
        s.delta[b, :, n:] = np.inf
        s.z[b, :, n:] = np.nan
        s.B[b, :, n:] = np.inf
        s.C[b, :, n:] = np.nan
    _check(mss, oracle_mod, s, lens, what=f"varlen nan padding {dtype} generic={generic}")


@pytest.mark.parametrize("L", [2047, 2041, 1001])
def test_varlen_ragged_length_mamba2p8b_all_rows(mss, oracle_mod, L):
    """Lengths and L that are not whole 16-byte vectors (rows start at odd element offsets): all
    20480 rows against the oracle."""
    c = CONFIGS["mamba2p8b_bf16"]
    s = scan_inputs(c["batch"], c["d_inner"], 16, L, dtype="bf16", seed=67)
    lens = np.array([L, 1, L - 8, 1000], dtype=np.int32)
    _check(mss, oracle_mod, s, lens, what=f"varlen mamba2p8b L={L}")


def test_varlen_mamba2p8b_all_rows(mss, oracle_mod):
    c = CONFIGS["mamba2p8b_bf16"]
    s = scan_inputs(c["batch"], c["d_inner"], 16, c["L"], dtype="bf16", seed=64)
    lens = np.array([2048, 1, 1000, 1537], dtype=np.int32)
    _check(mss, oracle_mod, s, lens, what="varlen mamba2p8b")


def test_full_lengths_are_the_plain_scan(mss):
    import torch
    s = scan_inputs(4, 128, 16, 1024, dtype="bf16", seed=65)
    o0, l0 = run_scan(mss, s)
    o1, l1 = _run(mss, s, np.full(4, 1024, dtype=np.int32))
    o2, l2 = _run(mss, s, np.full(4, 5000, dtype=np.int32))   # clamped to L
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert torch.equal(o0, o2) and torch.equal(l0, l2)


def test_decode_continues_each_sequence(mss, oracle_mod):
    """Prefill sequences of lengths l_b, then decode 5 more tokens of each from its own state."""
    import torch
    Bt, Dn, L = 4, 128, 96
    s = scan_inputs(Bt, Dn, 16, L, dtype="f32", seed=66)
    lens = np.array([10, 40, 61, 90], dtype=np.int32)
    _, state = _run(mss, s, lens)
    A, D, bias = dev(s.A), dev(s.D), dev(s.delta_bias)
    steps = 5
    outs = []
    for k in range(steps):
        t = lens + k                                      # next position of each sequence
        x = np.stack([s.u[b, :, t[b]] for b in range(Bt)])
        dt = np.stack([s.delta[b, :, t[b]] for b in range(Bt)])
        zz = np.stack([s.z[b, :, t[b]] for b in range(Bt)])
        Bk = np.stack([s.B[b, :, t[b]] for b in range(Bt)])
        Ck = np.stack([s.C[b, :, t[b]] for b in range(Bt)])
        outs.append(mss.selective_state_update(state, dev(x), dev(dt), A, dev(Bk), dev(Ck), D=D,
                                               z=dev(zz), dt_bias=bias))
    torch.cuda.synchronize()
    ref_out, ref_last = oracle_mod.selective_scan(s.u, s.delta, s.A, s.B, s.C, s.D, s.z,
                                                  s.delta_bias, seq_lens=lens + steps)
    got = host64(torch.stack(outs, -1))                  # (Bt, Dn, steps)
    want = np.stack([ref_out[b][:, lens[b]:lens[b] + steps] for b in range(Bt)])
    assert_close(got, want, what="decode after varlen prefill", **TOL_F32)
    assert_close(host64(state), ref_last, what="state after decode", **TOL_F32)
