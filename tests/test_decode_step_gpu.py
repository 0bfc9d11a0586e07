"""GPU tests of StateUpdateStep and Conv1dUpdateStep: the one-token entry points bound once to
fixed device buffers, then called per token with their input buffers refilled in place (a decode
loop).  Every row of every step against the fp64 oracle (tolerances as in the other decode tests),
and bit for bit against the unbound call on a second state."""
import numpy as np
import pytest

from synth import decode_inputs
from tests.gpu_helpers import TOL_BF16, TOL_F32, assert_close, dev, host64, record_margin

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mss():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_06_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("Bt,Dn,N,dtype,with_z,side_stream", [
    (3, 333, 16, "bf16", True, False), (2, 130, 64, "f32", False, False), (4, 5120, 16, "bf16", True, True),
    (2, 96, 128, "bf16", True, False), (1, 70, 32, "f32", True, True),
])
def test_bound_step_chain(mss, oracle_mod, Bt, Dn, N, dtype, with_z, side_stream):
    import torch
    steps = 5
    di = decode_inputs(Bt, Dn, N, steps, dtype=dtype, with_z=with_z, seed=7 * Bt + Dn + N)
    state0 = (0.5 * np.random.default_rng(Bt * Dn + N).standard_normal((Bt, Dn, N))).astype(np.float32)
    state, state_ref = dev(state0), dev(state0)
    A, D, bias = dev(di.A), dev(di.D), dev(di.dt_bias)
    # the buffers the step is bound to, refilled every token
    x, dt = dev(di.x[0], dtype), dev(di.dt[0], dtype)
    z = dev(di.z[0], dtype) if with_z else None
    Bb, Cb = dev(di.B[0]), dev(di.C[0])
    stream = torch.cuda.Stream() if side_stream else None
    step = mss.StateUpdateStep(state, x, dt, A, Bb, Cb, D=D, z=z, dt_bias=bias, stream=stream)
    ref_state = state0.astype(np.float64).reshape(Bt * Dn, N).copy()
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for s in range(steps):
        x.copy_(dev(di.x[s], dtype)); dt.copy_(dev(di.dt[s], dtype))
        Bb.copy_(dev(di.B[s])); Cb.copy_(dev(di.C[s]))
        if with_z:
            z.copy_(dev(di.z[s], dtype))
        torch.cuda.synchronize()
        out = step()
        torch.cuda.synchronize()
        out_ref = mss.selective_state_update(state_ref, x, dt, A, Bb, Cb, D=D, z=z, dt_bias=bias)
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref) and torch.equal(state, state_ref), f"step {s}: bound != unbound"
        ref = oracle_mod.selective_state_update(ref_state, di.x[s], di.dt[s], di.A, di.B[s], di.C[s], D=di.D,
                                                z=di.z[s] if with_z else None, dt_bias=di.dt_bias,
                                                rows=np.arange(Bt * Dn))
        record_margin(f"bound decode step {Bt}x{Dn}x{N} {dtype} out",
                      assert_close(host64(out).reshape(-1), ref.reshape(-1), what=f"bound step out {s}", **tol))
        record_margin(f"bound decode step {Bt}x{Dn}x{N} {dtype} state",
                      assert_close(host64(state).reshape(Bt * Dn, N), ref_state, what=f"bound step state {s}",
                                   **TOL_F32))


def test_bound_step_rejects_bad_shapes_per_call(mss):
    """Validation runs on every call: a buffer bound with the wrong shape is refused (before any
    GPU work) each time the step is called."""
    import torch
    state = torch.zeros((2, 64, 16), device="cuda")
    x = torch.zeros((2, 65), device="cuda")  # d_inner does not match the state
    dt = torch.zeros((2, 64), device="cuda")
    A, Bv, Cv = -torch.ones((64, 16), device="cuda"), torch.zeros((2, 16), device="cuda"), torch.zeros((2, 16), device="cuda")
    step = mss.StateUpdateStep(state, x, dt, A, Bv, Cv, out=torch.empty((2, 64), device="cuda"))
    for _ in range(2):
        with pytest.raises(mss.MssError):
            step()
    assert torch.count_nonzero(state) == 0


@pytest.mark.parametrize("dtype,K,silu", [("bf16", 4, True), ("f32", 3, False), ("bf16", 2, True)])
def test_bound_conv_update_chain(mss, oracle_mod, dtype, K, silu):
    """Conv1dUpdateStep over a chain of tokens (its x buffer refilled per token): bit for bit the
    unbound call, and the whole chain equal to the oracle's conv over the sequence."""
    import torch
    rng = np.random.default_rng(K)
    Bt, Dn, L = 3, 200, 6
    x = rng.standard_normal((Bt, Dn, L)).astype(np.float32)
    w = (0.5 * rng.standard_normal((Dn, K))).astype(np.float32)
    b = (0.1 * rng.standard_normal(Dn)).astype(np.float32)
    st0 = rng.standard_normal((Bt, Dn, K - 1)).astype(np.float32)
    if dtype == "bf16":
        from synth import round_to_bf16
        x, st0 = round_to_bf16(x), round_to_bf16(st0)
    wd, bd = dev(w), dev(b)
    state, state_ref = dev(st0, dtype), dev(st0, dtype)
    xb = dev(x[..., 0], dtype)
    step = mss.Conv1dUpdateStep(state, xb, wd, bd, silu=silu, stream=torch.cuda.Stream())
    outs = []
    for t in range(L):
        xb.copy_(dev(np.ascontiguousarray(x[..., t]), dtype))
        torch.cuda.synchronize()
        step()  # on its own stream: wait for it before reading out on this one
        torch.cuda.synchronize()
        out = step.out.clone()
        ref_out = mss.causal_conv1d_update(state_ref, xb, wd, bd, silu=silu)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(state, state_ref), f"token {t}: bound != unbound"
        outs.append(host64(out))
    ref, rfin = oracle_mod.causal_conv1d(x, w, b, state=st0, silu=silu)
    record_margin(f"bound conv update K={K} {dtype}",
                  assert_close(np.stack(outs, -1), ref, what="bound conv update chain",
                               **(TOL_BF16 if dtype == "bf16" else TOL_F32)))
    np.testing.assert_array_equal(host64(state), rfin)


def test_bound_steps_replayed_from_a_graph(mss):
    """A chain of bound steps captured in a HIP graph on their own stream: every replay (with eager
    work and synchronisations between them) matches the unbound eager chain from the same state,
    bit for bit."""
    import torch
    Bt, Dn, N, steps = 4, 640, 16, 8
    di = decode_inputs(Bt, Dn, N, steps, dtype="bf16", with_z=True, seed=99)
    A, D, bias = dev(di.A), dev(di.D), dev(di.dt_bias)
    X, DT, Z = dev(di.x, "bf16"), dev(di.dt, "bf16"), dev(di.z, "bf16")
    Bs, Cs = dev(di.B), dev(di.C)
    state_g = dev((0.5 * np.random.default_rng(5).standard_normal((Bt, Dn, N))).astype(np.float32))
    state_e = torch.empty_like(state_g)
    outs_g = torch.zeros((steps, Bt, Dn), dtype=torch.bfloat16, device="cuda")
    outs_e = torch.empty_like(outs_g)
    s = torch.cuda.Stream()
    bound = [mss.StateUpdateStep(state_g, X[j], DT[j], A, Bs[j], Cs[j], D=D, z=Z[j], dt_bias=bias, out=outs_g[j],
                                 stream=s) for j in range(steps)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for step in bound:
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        state_e.copy_(state_g)
        for j in range(steps):
            mss.selective_state_update(state_e, X[j], DT[j], A, Bs[j], Cs[j], D=D, z=Z[j], dt_bias=bias,
                                       out=outs_e[j])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs_g, outs_e), f"replay {rep}: out"
        assert torch.equal(state_g, state_e), f"replay {rep}: state"
