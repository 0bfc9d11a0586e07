"""GPU parity of the forward scan at d_state 32, 64 and 128 (mss_selective_scan_fwd and its
starting-state and per-sequence-length forms, through the C ABI) against the fp64 oracle,
element by element.  At these sizes d_state / 16 neighbouring lanes of a wavefront share a
channel and their parts of C.h meet through DPP adds; the cases cover channel counts that leave a
partial wavefront, lengths that leave partial tiles, both storage types with and without
16-byte-aligned rows, the power path (A = -(n+1)) and an unstructured A, every optional argument,
segment splits, starting states, per-sequence lengths, L = 0, and the Mamba-2.8B layer width on
sampled rows.

Tolerances as in test_parity_gpu.py: fp32 rtol 1e-4 / atol 1e-5; bf16 out rtol 2e-2; the fp32
final state keeps the fp32 bound.
"""
import numpy as np
import pytest

from synth import scan_inputs
from tests.gpu_helpers import (TOL_BF16, TOL_F32, assert_close, dev, host64, oracle_scan, record_margin,
                               run_scan)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mss():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_06_amd as m
    m.load_library()  # raises if the HIP library is not built: no fallback
    return m


def _cmp(go, gl, ref_out, ref_last, dtype, what):
    r1 = assert_close(go, ref_out, what=what + " out", **(TOL_BF16 if dtype == "bf16" else TOL_F32))
    r2 = assert_close(gl, ref_last, what=what + " last_state", **TOL_F32)
    record_margin(what + " out", r1)
    record_margin(what + " last_state", r2)
    print(f"[{what}] out {r1:.3f} last_state {r2:.3f} of the limit", flush=True)


def _check(mss, orc, s, what, rows=None, **flags):
    import torch
    out, last = run_scan(mss, s, **flags)
    torch.cuda.synchronize()
    Bt, Dn, L = s.u.shape
    N = s.A.shape[1]
    ref_out, ref_last = oracle_scan(orc, s, rows=rows, **flags)
    go, gl = host64(out).reshape(Bt * Dn, L), host64(last).reshape(Bt * Dn, N)
    if rows is None:
        ref_out, ref_last = ref_out.reshape(Bt * Dn, L), ref_last.reshape(Bt * Dn, N)
    else:
        go, gl = go[rows], gl[rows]
    _cmp(go, gl, ref_out, ref_last, s.dtype, what)


@pytest.mark.parametrize("Bt,Dn,N,L,dtype,a_kind", [
    (2, 64, 32, 300, "f32", "s4d"), (1, 50, 32, 129, "bf16", "random"), (2, 40, 64, 256, "bf16", "s4d"),
    (3, 16, 64, 100, "f32", "random"), (1, 20, 128, 333, "f32", "s4d"), (2, 13, 128, 64, "bf16", "random"),
    (1, 7, 64, 7, "f32", "s4d"), (1, 9, 128, 1, "bf16", "s4d"), (2, 33, 32, 1000, "bf16", "s4d")])
def test_dstate_parity(mss, oracle_mod, Bt, Dn, N, L, dtype, a_kind):
    s = scan_inputs(Bt, Dn, N, L, dtype=dtype, seed=700 + N + L, a_kind=a_kind)
    _check(mss, oracle_mod, s, f"d_state {N}: {Bt}x{Dn}x{L} {dtype} {a_kind}")


@pytest.mark.parametrize("flags", [dict(use_z=False), dict(use_D=False), dict(use_bias=False),
                                   dict(softplus=False, use_bias=False)])
@pytest.mark.parametrize("N", [32, 128])
def test_dstate_optional_arguments(mss, oracle_mod, N, flags):
    s = scan_inputs(2, 24, N, 200, dtype="f32", seed=720 + N)
    if not flags.get("softplus", True):
        s.delta = np.abs(s.delta) * np.float32(0.05)  # delta used as given: a valid positive step
    _check(mss, oracle_mod, s, f"d_state {N} {flags}", **flags)


@pytest.mark.parametrize("segments", [1, 2, 3, 7, 16])
@pytest.mark.parametrize("N", [64, 128])
def test_dstate_segment_splits(mss, oracle_mod, plan, N, segments):
    """The sequence cut into segments: per-segment local end states and sums of delta, folded in
    order by the combine kernel into each segment's starting state."""
    plan(generic_segments=segments)
    s = scan_inputs(2, 20, N, 16 * 32 - 5, dtype="bf16" if segments % 2 else "f32", seed=730 + segments,
                    a_kind="random" if N == 64 else "s4d")
    _check(mss, oracle_mod, s, f"d_state {N} segments={segments}")


@pytest.mark.parametrize("N", [32, 64, 128])
def test_dstate_with_state_and_split(mss, oracle_mod, plan, N):
    """A given starting state, carried through a 3-segment split; then L = 0 copies it."""
    import torch
    plan(generic_segments=3)
    s = scan_inputs(2, 18, N, 250, dtype="f32", seed=740 + N, a_kind="random")
    h0 = (0.5 * np.random.default_rng(N).standard_normal((2, 18, N))).astype(np.float32)
    out, last = mss.selective_scan_fwd_with_state(dev(s.u), dev(s.delta), dev(s.A), dev(s.B), dev(s.C), dev(h0),
                                                  D=dev(s.D), z=dev(s.z), delta_bias=dev(s.delta_bias))
    torch.cuda.synchronize()
    ref_out, ref_last = oracle_mod.selective_scan(s.u, s.delta, s.A, s.B, s.C, D=s.D, z=s.z,
                                                  delta_bias=s.delta_bias, h0=h0)
    _cmp(host64(out).reshape(36, 250), host64(last).reshape(36, N), ref_out.reshape(36, 250),
         ref_last.reshape(36, N), "f32", f"d_state {N} with state")
    e = lambda *shape: torch.empty(shape, dtype=torch.float32, device="cuda")
    out0, last0 = mss.selective_scan_fwd_with_state(e(2, 18, 0), e(2, 18, 0), dev(s.A), e(2, N, 0), e(2, N, 0),
                                                    dev(h0))
    torch.cuda.synchronize()
    assert out0.numel() == 0 and np.array_equal(host64(last0), h0.astype(np.float64))
    out0, last0 = mss.selective_scan_fwd(e(2, 18, 0), e(2, 18, 0), dev(s.A), e(2, N, 0), e(2, N, 0))
    torch.cuda.synchronize()
    assert last0.shape == (2, 18, N) and torch.count_nonzero(last0) == 0


@pytest.mark.parametrize("N", [64, 128])
def test_dstate_varlen(mss, oracle_mod, N):
    """Per-sequence lengths: outputs up to each end, zeros past it, each sequence's own final state."""
    import torch
    Bt, Dn, L = 6, 24, 130
    s = scan_inputs(Bt, Dn, N, L, dtype="bf16", seed=750 + N)
    lens = np.array([0, 1, 3, L, L - 1, 66], np.int32)
    out, last = mss.selective_scan_fwd_varlen(dev(s.u, "bf16"), dev(s.delta, "bf16"), dev(s.A), dev(s.B), dev(s.C),
                                              torch.from_numpy(lens).to("cuda"), D=dev(s.D), z=dev(s.z, "bf16"),
                                              delta_bias=dev(s.delta_bias))
    torch.cuda.synchronize()
    ref_out, ref_last = oracle_mod.selective_scan(s.u, s.delta, s.A, s.B, s.C, D=s.D, z=s.z,
                                                  delta_bias=s.delta_bias, seq_lens=lens)
    go, gl = host64(out).reshape(Bt * Dn, L), host64(last).reshape(Bt * Dn, N)
    _cmp(go, gl, ref_out.reshape(Bt * Dn, L), ref_last.reshape(Bt * Dn, N), "bf16", f"d_state {N} varlen")
    t = np.arange(L)[None, :]
    assert not np.any(go[t >= lens[np.arange(Bt * Dn) // Dn][:, None]])


@pytest.mark.parametrize("N,a_kind", [(64, "s4d"), (128, "s4d"), (128, "random")])
def test_dstate_mamba2p8b_width_all_rows(mss, oracle_mod, N, a_kind):
    """The Mamba-2.8B layer shape (4 x 5120 x 2048, bf16 activations) at d_state 64 and 128: every
    output and final state of all 20480 rows against the oracle (S4D A: at d_state 128 the scaled
    state step; random A: an exponential per update)."""
    s = scan_inputs(4, 5120, N, 2048, dtype="bf16", seed=760 + N, a_kind=a_kind)
    _check(mss, oracle_mod, s, f"d_state {N} mamba2p8b width" + ("" if a_kind == "s4d" else " random A"))


def test_dstate_deterministic(mss):
    import torch
    s = scan_inputs(2, 40, 64, 700, dtype="bf16", seed=770)
    a = run_scan(mss, s)
    b = run_scan(mss, s)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
