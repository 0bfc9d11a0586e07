"""GPU parity: libmamba_scan (through its C ABI) against the fp64 oracle, element by element,
on seeded inputs -- the five workloads at full size plus small, ragged and degenerate cases.

Tolerances (|gpu - ref| <= atol + rtol |ref|): fp32 inputs rtol 1e-4 / atol 1e-5 on out and
on the final state; bf16 u / delta / z rtol 2e-2 / atol 1e-5 on the bf16 out, while the fp32
final state keeps the fp32 bound.
"""
import os

import numpy as np
import pytest

from synth import CONFIGS, decode_inputs, sample_rows, scan_inputs
from tests.gpu_helpers import (TOL_BF16, TOL_F32, assert_close, dev, host64, oracle_scan,
                               record_margin, run_scan, waves_for)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mss():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_06_amd as m
    m.load_library()  # raises if the HIP library is not built: no fallback
    return m


@pytest.fixture(scope="module")
def orc(oracle_mod):
    return oracle_mod


def _tol(dtype):
    return TOL_BF16 if dtype == "bf16" else TOL_F32


def _check_scan(mss, orc, s, rows=None, what="", **flags):
    import torch
    out, last = run_scan(mss, s, **flags)
    torch.cuda.synchronize()
    ref_out, ref_last = oracle_scan(orc, s, rows=rows, **flags)
    Bt, Dn, L = s.u.shape
    go, gl = host64(out).reshape(Bt * Dn, L), host64(last).reshape(Bt * Dn, -1)
    if rows is not None:
        go, gl = go[rows], gl[rows]
    else:
        ref_out, ref_last = ref_out.reshape(Bt * Dn, L), ref_last.reshape(Bt * Dn, -1)
    mo = record_margin(what + " out", assert_close(go, ref_out, what=what + " out", **_tol(s.dtype)))
    ml = record_margin(what + " last_state", assert_close(gl, ref_last, what=what + " last_state", **TOL_F32))
    print(f"[{what}] out worst/limit = {mo:.3f}, last_state worst/limit = {ml:.3f}", flush=True)
    return out, last


# ------------------------------------------------------------------ the five workloads

def _cfg_inputs(name, a_kind="s4d", **over):
    c = dict(CONFIGS[name])
    c.update(over)
    return scan_inputs(c["batch"], c["d_inner"], c["d_state"], c["L"], dtype=c["dtype"],
                       with_z=c["with_z"], seed=0, a_kind=a_kind)


def test_tiny_fp32_full(mss, orc):
    _check_scan(mss, orc, _cfg_inputs("tiny_fp32"), what="tiny_fp32")


def test_mamba130m_fp32_full(mss, orc):
    _check_scan(mss, orc, _cfg_inputs("mamba130m_fp32"), what="mamba130m_fp32")


def test_mamba2p8b_bf16_full(mss, orc):
    _check_scan(mss, orc, _cfg_inputs("mamba2p8b_bf16"), what="mamba2p8b_bf16")


def test_mamba2p8b_bf16_random_A_full(mss, orc):
    """The 2.8B layer with an unstructured negative A (what a trained layer holds): every state
    update takes its own exp (no power chain), every row against the oracle."""
    _check_scan(mss, orc, _cfg_inputs("mamba2p8b_bf16", a_kind="random"), what="mamba2p8b_bf16 random A")


def test_long_fp32_random_A_all_rows(mss, orc):
    """The long-context workload with an unstructured negative A, every row and step against the
    oracle."""
    _check_scan(mss, orc, _cfg_inputs("long_fp32", a_kind="random"), what="long_fp32 random A")


@pytest.mark.parametrize("Bt,Dn", [(4, 640), (1, 5120)])
def test_mamba2p8b_shard_shapes(mss, orc, Bt, Dn):
    """The 2.8B layer as one GPU's share: d_inner split 8 ways or batch split 4 ways (rows are
    independent; fewer of them make the plan cut L into many more segments)."""
    _check_scan(mss, orc, _cfg_inputs("mamba2p8b_bf16", batch=Bt, d_inner=Dn), what=f"mamba2p8b shard {Bt}x{Dn}")


@pytest.mark.parametrize("name,L", [("mamba2p8b_bf16", 2047), ("mamba2p8b_bf16", 2044), ("mamba130m_fp32", 2047),
                                    ("mamba130m_fp32", 2046)])
def test_ragged_length_full_size(mss, orc, name, L):
    """L that is not a whole number of 16-byte vectors: rows start at element offsets that are
    not 16-byte aligned and end in a partial vector (the fast path's element-aligned variant)."""
    _check_scan(mss, orc, _cfg_inputs(name, L=L), what=f"{name} L={L}")


def test_ragged_rows_match_generic_path(mss, plan):
    """The element-aligned fast path and the generic kernels agree to rounding on ragged rows."""
    import torch
    s = scan_inputs(3, 200, 16, 777, dtype="bf16", seed=24)
    out_f, last_f = run_scan(mss, s)
    plan(force_generic=True)
    out_g, last_g = run_scan(mss, s)
    torch.cuda.synchronize()
    assert_close(host64(out_f), host64(out_g), what="fast vs generic out", **TOL_BF16)
    assert_close(host64(last_f), host64(last_g), what="fast vs generic last_state", **TOL_F32)


def test_long_fp32_all_rows(mss, orc):
    """The long-context workload (1 x 1536 x 16 x 131072, fp32, no gate): all 1536 rows, every
    step, against the oracle."""
    _check_scan(mss, orc, _cfg_inputs("long_fp32"), what="long_fp32")


def test_decode_bf16_1024_steps(mss, orc):
    import torch
    c = CONFIGS["decode_bf16"]
    Bt, Dn, N, steps = c["batch"], c["d_inner"], c["d_state"], c["steps"]
    di = decode_inputs(Bt, Dn, N, steps, dtype="bf16", seed=0)
    x, dt, z = dev(di.x, "bf16"), dev(di.dt, "bf16"), dev(di.z, "bf16")
    Bs, Cs = dev(di.B), dev(di.C)
    A, D, bias = dev(di.A), dev(di.D), dev(di.dt_bias)
    state = torch.zeros((Bt, Dn, N), dtype=torch.float32, device="cuda")
    outs = torch.empty((steps, Bt, Dn), dtype=torch.bfloat16, device="cuda")
    for s in range(steps):
        mss.selective_state_update(state, x[s], dt[s], A, Bs[s], Cs[s], D=D, z=z[s], dt_bias=bias,
                                   out=outs[s])
    torch.cuda.synchronize()
    rows = sample_rows(Bt * Dn, 16384, seed=4)  # 5% of the rows, every step
    ref_state = np.zeros((rows.size, N))
    ref_out = np.empty((steps, rows.size))
    for s in range(steps):
        ref_out[s] = orc.selective_state_update(ref_state, di.x[s], di.dt[s], di.A, di.B[s], di.C[s],
                                                D=di.D, z=di.z[s], dt_bias=di.dt_bias, rows=rows)
    go = host64(outs).reshape(steps, Bt * Dn)[:, rows]
    gs = host64(state).reshape(Bt * Dn, N)[rows]
    record_margin("decode_bf16 1024 steps out", assert_close(go, ref_out, what="decode out", **TOL_BF16))
    record_margin("decode_bf16 1024 steps state", assert_close(gs, ref_state, what="decode state", **TOL_F32))


@pytest.mark.parametrize("Bt,Dn,dtype,with_z,a_kind", [
    (1, 1, "f32", True, "s4d"), (1, 3, "bf16", True, "s4d"), (5, 7, "f32", False, "random"),
    (3, 130, "bf16", True, "s4d"), (7, 333, "f32", True, "random"), (2, 5120, "bf16", False, "s4d"),
    (129, 64, "bf16", True, "s4d")])
def test_decode_row_counts(mss, orc, Bt, Dn, dtype, with_z, a_kind):
    """Row counts that leave partial groups of rows and partial wavefronts: every row of three
    chained steps, state and out, against the oracle."""
    import torch
    steps = 3
    di = decode_inputs(Bt, Dn, 16, steps, dtype=dtype, with_z=with_z, seed=Bt * 1000 + Dn, a_kind=a_kind)
    state0 = (0.5 * np.random.default_rng(Bt + Dn).standard_normal((Bt, Dn, 16))).astype(np.float32)
    state = dev(state0)
    A, D, bias = dev(di.A), dev(di.D), dev(di.dt_bias)
    ref_state = state0.astype(np.float64).reshape(Bt * Dn, 16).copy()
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for s in range(steps):
        z = dev(di.z[s], dtype) if with_z else None
        out = mss.selective_state_update(state, dev(di.x[s], dtype), dev(di.dt[s], dtype), A,
                                         dev(di.B[s]), dev(di.C[s]), D=D, z=z, dt_bias=bias)
        torch.cuda.synchronize()
        ref = orc.selective_state_update(ref_state, di.x[s], di.dt[s], di.A, di.B[s], di.C[s], D=di.D,
                                         z=di.z[s] if with_z else None, dt_bias=di.dt_bias,
                                         rows=np.arange(Bt * Dn))
        assert_close(host64(out).reshape(-1), ref.reshape(-1), what=f"decode out step {s}", **tol)
        assert_close(host64(state).reshape(Bt * Dn, 16), ref_state, what=f"decode state step {s}", **TOL_F32)


@pytest.mark.parametrize("Bt,Dn,N,dtype,with_z,a_kind", [
    (1, 1, 32, "f32", True, "s4d"), (3, 130, 32, "bf16", True, "random"), (1, 3, 64, "bf16", True, "s4d"),
    (7, 333, 64, "f32", True, "random"), (5, 7, 128, "f32", False, "random"), (129, 64, 128, "bf16", True, "s4d"),
    (2, 5120, 128, "bf16", False, "s4d")])
def test_decode_state_sizes(mss, orc, Bt, Dn, N, dtype, with_z, a_kind):
    """d_state 32, 64 and 128 (a lane holds N / 4 states of its row): every row of three chained
    steps, state and out, against the oracle, with partial wavefronts and the 2.8B-wide d_inner."""
    import torch
    steps = 3
    di = decode_inputs(Bt, Dn, N, steps, dtype=dtype, with_z=with_z, seed=Bt * 1000 + Dn + N, a_kind=a_kind)
    state0 = (0.5 * np.random.default_rng(Bt + Dn + N).standard_normal((Bt, Dn, N))).astype(np.float32)
    state = dev(state0)
    A, D, bias = dev(di.A), dev(di.D), dev(di.dt_bias)
    ref_state = state0.astype(np.float64).reshape(Bt * Dn, N).copy()
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for s in range(steps):
        z = dev(di.z[s], dtype) if with_z else None
        out = mss.selective_state_update(state, dev(di.x[s], dtype), dev(di.dt[s], dtype), A,
                                         dev(di.B[s]), dev(di.C[s]), D=D, z=z, dt_bias=bias)
        torch.cuda.synchronize()
        ref = orc.selective_state_update(ref_state, di.x[s], di.dt[s], di.A, di.B[s], di.C[s], D=di.D,
                                         z=di.z[s] if with_z else None, dt_bias=di.dt_bias,
                                         rows=np.arange(Bt * Dn))
        record_margin(f"decode N={N} {Bt}x{Dn} out",
                      assert_close(host64(out).reshape(-1), ref.reshape(-1), what=f"decode N={N} out step {s}", **tol))
        record_margin(f"decode N={N} {Bt}x{Dn} state",
                      assert_close(host64(state).reshape(Bt * Dn, N), ref_state, what=f"decode N={N} state step {s}",
                                   **TOL_F32))


# ------------------------------------------------------------------ shapes and flags

@pytest.mark.parametrize("Bt,Dn,L,dtype", [
    (1, 64, 1, "f32"), (1, 64, 3, "f32"), (2, 5, 33, "f32"), (1, 70, 100, "f32"),
    (3, 130, 255, "f32"), (1, 64, 4, "f32"), (2, 64, 7, "bf16"), (1, 100, 129, "bf16"),
    (2, 192, 520, "bf16"), (1, 1, 64, "f32")])
def test_ragged_shapes(mss, orc, Bt, Dn, L, dtype):
    s = scan_inputs(Bt, Dn, 16, L, dtype=dtype, seed=L + Dn)
    _check_scan(mss, orc, s, what=f"ragged {Bt}x{Dn}x{L} {dtype}")


@pytest.mark.parametrize("flags", [
    dict(use_z=False), dict(use_D=False), dict(use_bias=False), dict(softplus=False, use_bias=False),
    dict(use_z=False, use_D=False, use_bias=False)])
def test_optional_arguments(mss, orc, flags):
    s = scan_inputs(2, 96, 16, 300, dtype="f32", seed=21)
    if not flags.get("softplus", True):
        s.delta = np.abs(s.delta) * 0.05  # a valid positive step size without softplus
    _check_scan(mss, orc, s, what=f"flags {flags}", **flags)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_random_A_general_path(mss, orc, dtype):
    s = scan_inputs(2, 128, 16, 700, dtype=dtype, seed=22, a_kind="random")
    _check_scan(mss, orc, s, what=f"random A {dtype}")


@pytest.mark.parametrize("segments", ["1", "2", "5", "64"])
def test_segment_split_counts(mss, orc, segments, plan):
    plan(fast_waves=waves_for(1, 128, segments))
    s = scan_inputs(1, 128, 16, 1000, dtype="f32", seed=23)
    _check_scan(mss, orc, s, what=f"segments={segments}")


@pytest.mark.parametrize("waves,dtype,a_kind", [
    (1, "bf16", "s4d"), (5, "f32", "random"), (7, "bf16", "random"), (13, "f32", "s4d"),
    (50, "bf16", "s4d"), (299, "f32", "s4d"), (1000, "bf16", "random")])
def test_wavefront_ranges_cross_groups(mss, orc, waves, dtype, a_kind, plan):
    """The fast forward's work split at any wavefront count: one wavefront scanning all twelve
    channel groups in turn, ranges that start and end inside groups and run on into the next
    group, and one-tile pieces (the count is capped at the 300 (group, tile) pairs)."""
    plan(fast_waves=waves)
    s = scan_inputs(3, 200, 16, 777 if dtype == "bf16" else 400, dtype=dtype, seed=25, a_kind=a_kind)
    _check_scan(mss, orc, s, what=f"waves={waves} {dtype} {a_kind}")


def test_empty_sequence_zeroes_state(mss):
    import torch
    u = torch.empty((2, 64, 0), dtype=torch.float32, device="cuda")
    A = dev(-np.tile(np.arange(1, 17, dtype=np.float32), (64, 1)))
    B = torch.empty((2, 16, 0), dtype=torch.float32, device="cuda")
    last = torch.full((2, 64, 16), 7.0, device="cuda")
    out, last = mss.selective_scan_fwd(u, u.clone(), A, B, B.clone(), last_state=last)
    torch.cuda.synchronize()
    assert out.shape == (2, 64, 0) and torch.all(last == 0)


def test_memoryless_extreme_decay(mss, orc):
    s = scan_inputs(1, 64, 16, 200, dtype="f32", seed=24)
    s.A = np.full_like(s.A, -1e6)
    _check_scan(mss, orc, s, what="memoryless")


# ------------------------------------------------------------------ invariants on the GPU

def test_causality_exact(mss):
    import torch
    s = scan_inputs(2, 128, 16, 640, dtype="f32", seed=25)
    base, _ = run_scan(mss, s)
    t0 = 333
    rng = np.random.default_rng(5)
    for name in ("u", "delta", "z", "B", "C"):
        a = getattr(s, name).copy()
        a[..., t0:] = rng.standard_normal(a[..., t0:].shape).astype(np.float32)
        setattr(s, name, a)
    pert, _ = run_scan(mss, s)
    torch.cuda.synchronize()
    assert torch.equal(base[..., :t0], pert[..., :t0])
    assert not torch.equal(base[..., t0:], pert[..., t0:])


def test_deterministic(mss):
    import torch
    s = scan_inputs(2, 256, 16, 1024, dtype="bf16", seed=26)
    o1, l1 = run_scan(mss, s)
    o2, l2 = run_scan(mss, s)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_chain_matches_scan(mss):
    """L chained decode steps from h = 0 reproduce the scan's outputs and final state."""
    import torch
    s = scan_inputs(2, 128, 16, 96, dtype="f32", seed=27)
    out, last = run_scan(mss, s)
    state = torch.zeros_like(last)
    A, D, bias = dev(s.A), dev(s.D), dev(s.delta_bias)
    outs = []
    for t in range(s.u.shape[2]):
        outs.append(mss.selective_state_update(
            state, dev(s.u[..., t]), dev(s.delta[..., t]), A, dev(s.B[..., t]), dev(s.C[..., t]),
            D=D, z=dev(s.z[..., t]), dt_bias=bias))
    dec = torch.stack(outs, dim=-1)
    torch.cuda.synchronize()
    assert_close(host64(dec), host64(out), what="chain vs scan out", **TOL_F32)
    assert_close(host64(state), host64(last), what="chain vs scan state", **TOL_F32)


def test_scan_then_decode_continues(mss, orc):
    import torch
    s = scan_inputs(1, 192, 16, 160, dtype="bf16", seed=28)
    L1 = 128
    head = scan_inputs(1, 192, 16, 160, dtype="bf16", seed=28)
    for name in ("u", "delta", "z", "B", "C"):
        setattr(head, name, np.ascontiguousarray(getattr(s, name)[..., :L1]))
    _, state = run_scan(mss, head)
    A, D, bias = dev(s.A), dev(s.D), dev(s.delta_bias)
    outs = []
    for t in range(L1, 160):
        outs.append(mss.selective_state_update(
            state, dev(s.u[..., t], "bf16"), dev(s.delta[..., t], "bf16"), A, dev(s.B[..., t]),
            dev(s.C[..., t]), D=D, z=dev(s.z[..., t], "bf16"), dt_bias=bias))
    torch.cuda.synchronize()
    ref_out, ref_last = oracle_scan(orc, s)
    assert_close(host64(torch.stack(outs, -1)), ref_out[..., L1:], what="continued out", **TOL_BF16)
    assert_close(host64(state), ref_last, what="continued state", **TOL_F32)


def test_linear_in_u_on_gpu(mss):
    import torch
    s = scan_inputs(1, 128, 16, 512, dtype="f32", seed=29)
    o1, _ = run_scan(mss, s, use_z=False)
    u1 = s.u
    rng = np.random.default_rng(6)
    u2 = rng.standard_normal(u1.shape).astype(np.float32)
    s.u = u2
    o2, _ = run_scan(mss, s, use_z=False)
    s.u = (np.float32(0.5) * u1 + np.float32(-1.5) * u2).astype(np.float32)
    o3, _ = run_scan(mss, s, use_z=False)
    torch.cuda.synchronize()
    ref = 0.5 * host64(o1) - 1.5 * host64(o2)
    assert_close(host64(o3), ref, rtol=1e-4, atol=3e-5, what="linearity")


def test_nondefault_stream(mss, orc):
    import torch
    s = scan_inputs(2, 128, 16, 400, dtype="f32", seed=30)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        out, last = run_scan(mss, s)
    st.synchronize()
    ref_out, ref_last = oracle_scan(orc, s)
    assert_close(host64(out), ref_out, what="side stream out", **TOL_F32)


def test_launch_timing_records(mss, orc):
    """The timing hook records each call's kernels without changing its results."""
    import torch
    s = scan_inputs(2, 128, 16, 1024, dtype="f32", seed=31)
    mss.profile_enable(True)
    try:
        out, last = run_scan(mss, s)
        out2, _ = run_scan(mss, s)
    finally:
        mss.profile_enable(False)
    out3, _ = run_scan(mss, s)  # not recorded
    torch.cuda.synchronize()
    calls, carry_ms, main_ms = mss.profile_fwd()  # the records outlive disabling
    assert calls == 2
    assert main_ms > 0.0 and carry_ms >= 0.0
    assert torch.equal(out, out2) and torch.equal(out, out3)
    ref_out, ref_last = oracle_scan(orc, s)
    assert_close(host64(out), ref_out, what="timed out", **TOL_F32)


def test_decode_graph_replays_match_eager(mss):
    """A captured HIP graph of chained decode steps gives the eager results on every replay."""
    import torch
    dev = torch.device("cuda:0")
    d = decode_inputs(4, 256, 16, 8, dtype="bf16", with_z=True, seed=41)
    up = lambda a, bf=False: (torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)
                              if bf else torch.from_numpy(np.ascontiguousarray(a)).to(dev))
    X, DT, Z, Bs, Cs = up(d.x, True), up(d.dt, True), up(d.z, True), up(d.B), up(d.C)
    A, D, bias = up(d.A), up(d.D), up(d.dt_bias)
    state = torch.zeros((4, 256, 16), dtype=torch.float32, device=dev)
    outs = torch.empty((8, 4, 256), dtype=torch.bfloat16, device=dev)

    def chain():
        for k in range(8):
            mss.selective_state_update(state, X[k], DT[k], A, Bs[k], Cs[k], D=D, z=Z[k],
                                       dt_bias=bias, out=outs[k])

    chain()
    torch.cuda.synchronize()
    ref_state, ref_outs = state.clone(), outs.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        state.zero_()
        chain()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    for rep in range(3):
        state.zero_()
        outs.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, ref_state), f"replay {rep}: state"
        assert torch.equal(outs, ref_outs), f"replay {rep}: out"
