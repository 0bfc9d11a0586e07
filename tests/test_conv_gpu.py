"""GPU parity of mss_causal_conv1d_fwd / mss_causal_conv1d_update against the fp64 oracle,
element by element, plus identities that hold bit for bit on the GPU: chunked prefill equals one
call, and one-token steps from the carried window equal the whole-sequence conv.

Tolerance: |gpu - ref| <= atol + rtol |ref| with fp32 rtol 1e-4 / atol 1e-5 and, for bf16 outputs
(rounded to bf16), rtol 2e-2 / atol 1e-5.  The carried states are copies of inputs: bit-exact.
"""
import numpy as np
import pytest

from synth import CONFIGS, round_to_bf16
from tests.gpu_helpers import TOL_BF16, TOL_F32, assert_close, dev, host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mss():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_06_amd as m
    m.load_library()
    return m


def _inputs(Bt, Dn, L, K, dtype, seed):
    rng = np.random.default_rng(900 + seed)
    x = rng.standard_normal((Bt, Dn, L)).astype(np.float32)
    st = rng.standard_normal((Bt, Dn, K - 1)).astype(np.float32)
    if dtype == "bf16":
        x, st = round_to_bf16(x), round_to_bf16(st)
    w = (0.5 * rng.standard_normal((Dn, K))).astype(np.float32)
    b = rng.standard_normal(Dn).astype(np.float32)
    return x, w, b, st


def _tol(dtype):
    return TOL_BF16 if dtype == "bf16" else TOL_F32


@pytest.mark.parametrize("Bt,Dn,L,K,dtype", [
    (2, 64, 256, 4, "f32"), (2, 64, 256, 4, "bf16"), (1, 70, 33, 4, "f32"), (3, 5, 17, 4, "bf16"),
    (2, 48, 64, 3, "f32"), (2, 48, 64, 2, "bf16"), (1, 32, 40, 1, "f32"), (1, 3, 2, 4, "f32"),
    (4, 100, 1000, 4, "bf16"), (1, 1, 4, 4, "bf16")])
@pytest.mark.parametrize("with_state,silu", [(False, True), (True, True), (True, False)])
def test_conv_parity(mss, oracle_mod, Bt, Dn, L, K, dtype, with_state, silu):
    x, w, b, st = _inputs(Bt, Dn, L, K, dtype, L + K)
    out, fin = mss.causal_conv1d_fwd(dev(x, dtype), dev(w), dev(b),
                                     initial_state=dev(st, dtype) if with_state else None,
                                     silu=silu, return_final_state=True)
    ref, rfin = oracle_mod.causal_conv1d(x, w, b, state=st if with_state else None, silu=silu)
    assert_close(host64(out), ref, what=f"conv {Bt}x{Dn}x{L} K{K} {dtype}", **_tol(dtype))
    np.testing.assert_array_equal(host64(fin), rfin)


def test_conv_no_bias(mss, oracle_mod):
    x, w, _, _ = _inputs(2, 64, 128, 4, "f32", 1)
    out = mss.causal_conv1d_fwd(dev(x), dev(w), None)
    ref, _ = oracle_mod.causal_conv1d(x, w, None)
    assert_close(host64(out), ref, what="conv no bias", **TOL_F32)


@pytest.mark.parametrize("L", [2048, 2047, 2042])
def test_conv_mamba2p8b_full(mss, oracle_mod, L):
    """The 2.8B layer shape; L not a multiple of 8 runs the element-aligned variant."""
    c = CONFIGS["mamba2p8b_bf16"]
    x, w, b, st = _inputs(c["batch"], c["d_inner"], L, 4, "bf16", 2)
    out, fin = mss.causal_conv1d_fwd(dev(x, "bf16"), dev(w), dev(b), initial_state=dev(st, "bf16"),
                                     return_final_state=True)
    ref, rfin = oracle_mod.causal_conv1d(x, w, b, state=st)
    assert_close(host64(out), ref, what=f"conv mamba2p8b L={L}", **TOL_BF16)
    np.testing.assert_array_equal(host64(fin), rfin)


@pytest.mark.parametrize("dtype,cuts", [("bf16", [0, 8, 1000, 2048]), ("f32", [0, 1, 2, 7, 64]),
                                        ("bf16", [0, 3, 256, 259])])
def test_chunked_prefill_is_bit_exact(mss, dtype, cuts):
    import torch
    L = cuts[-1]
    x, w, b, st = _inputs(2, 96, L, 4, dtype, 3)
    xd, wd, bd = dev(x, dtype), dev(w), dev(b)
    whole, wfin = mss.causal_conv1d_fwd(xd, wd, bd, initial_state=dev(st, dtype),
                                        return_final_state=True)
    state = dev(st, dtype)
    pieces = []
    for a_, b_ in zip(cuts[:-1], cuts[1:]):
        o, state = mss.causal_conv1d_fwd(xd[..., a_:b_].contiguous(), wd, bd, initial_state=state,
                                         return_final_state=True)
        pieces.append(o)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(pieces, -1), whole)
    assert torch.equal(state, wfin)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_update_chain_equals_prefill(mss, dtype):
    """Tokens one at a time through the rolling window reproduce the whole-sequence conv."""
    import torch
    L = 40
    x, w, b, st = _inputs(2, 130, L, 4, dtype, 4)
    xd, wd, bd = dev(x, dtype), dev(w), dev(b)
    whole, wfin = mss.causal_conv1d_fwd(xd, wd, bd, initial_state=dev(st, dtype),
                                        return_final_state=True)
    state = dev(st, dtype)
    outs = [mss.causal_conv1d_update(state, xd[..., t].contiguous(), wd, bd) for t in range(L)]
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(outs, -1), whole)
    assert torch.equal(state, wfin)


def test_update_parity(mss, oracle_mod):
    x, w, b, st = _inputs(64, 5120 // 8, 1, 4, "bf16", 5)
    state = dev(st, "bf16")
    out = mss.causal_conv1d_update(state, dev(x[..., 0], "bf16"), dev(w), dev(b))
    ref, rfin = oracle_mod.causal_conv1d(x, w, b, state=st)
    assert_close(host64(out), ref[..., 0], what="conv update", **TOL_BF16)
    np.testing.assert_array_equal(host64(state), rfin)


def test_empty_sequence_passes_state_through(mss):
    import torch
    x, w, b, st = _inputs(2, 64, 0, 4, "bf16", 6)
    sd = dev(st, "bf16")
    out, fin = mss.causal_conv1d_fwd(dev(x, "bf16"), dev(w), dev(b), initial_state=sd,
                                     return_final_state=True)
    torch.cuda.synchronize()
    assert out.shape == (2, 64, 0) and torch.equal(fin, sd)


def test_conv_then_scan_pipeline(mss, oracle_mod):
    """u = silu(conv(x)) from the conv kernel feeds the scan: the chain matches the oracle's chain."""
    from synth import scan_inputs
    s = scan_inputs(2, 128, 16, 512, dtype="f32", seed=7)
    x, w, b, _ = _inputs(2, 128, 512, 4, "f32", 7)
    u = mss.causal_conv1d_fwd(dev(x), dev(w), dev(b))
    out, last = mss.selective_scan_fwd(u, dev(s.delta), dev(s.A), dev(s.B), dev(s.C), D=dev(s.D),
                                       z=dev(s.z), delta_bias=dev(s.delta_bias))
    uref, _ = oracle_mod.causal_conv1d(x, w, b)
    ref, rlast = oracle_mod.selective_scan(uref, s.delta, s.A, s.B, s.C, s.D, s.z, s.delta_bias)
    assert_close(host64(out), ref, what="conv -> scan out", **TOL_F32)
    assert_close(host64(last), rlast, what="conv -> scan state", **TOL_F32)
