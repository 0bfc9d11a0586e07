"""Tensors past 2^31 elements: the forward scan (d_state 16 and 128), its backward and the causal conv1d on a
(1, 65600, 32768) bf16 layer (2.15e9 elements per activation tensor, 4.3 GB), so element
offsets beyond the 32-bit range occur in every kernel.  Rows at the start, middle and end of
the tensors (the last rows lie past element 2^31) are checked against the fp64 oracle.

Inputs at this size are drawn on the device with a seeded torch generator, from the same
distributions as the other workloads (u, delta_raw, z, B, C, dout ~ N(0, 1) rounded to bf16
where bf16; A = -(n + 1), D = 1 and the dt bias from the seeded host generators); only the
sampled rows come back to the host.  Tolerances as elsewhere: out rtol 2e-2 (bf16), last_state
and conv rtol / atol as fp32 / bf16 outputs; du / ddelta / dz as in test_bwd_gpu.py.
"""
import numpy as np
import pytest

from synth import scan_inputs
from tests.gpu_helpers import TOL_BF16, TOL_F32, assert_close, host64

pytestmark = pytest.mark.gpu

BT, DN, N, L = 1, 65600, 16, 32768
ROWS = [0, 1, 31000, 65536, 65598, 65599]   # flat rows b * DN + d; 65536 * L > 2^31


@pytest.fixture(scope="module")
def mss():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    props = torch.cuda.get_device_properties(0)
    if props.total_memory < 80 * 2**30:
        pytest.skip("needs about 60 GB of device memory")
    import selective_state_space_06_amd as m
    m.load_library()
    return m


@pytest.fixture(scope="module")
def layer(mss):
    import torch
    assert BT * DN * L > 2**31
    g = torch.Generator(device="cuda").manual_seed(2024)
    big = lambda: torch.randn((BT, DN, L), generator=g, device="cuda", dtype=torch.bfloat16)
    u, delta, z = big(), big(), big()
    B = torch.randn((BT, N, L), generator=g, device="cuda", dtype=torch.float32)
    C = torch.randn((BT, N, L), generator=g, device="cuda", dtype=torch.float32)
    small = scan_inputs(1, DN, N, 1, dtype="f32", seed=7)   # A, D, dt bias of DN channels
    p = {k: torch.from_numpy(getattr(small, k)).to("cuda") for k in ("A", "D", "delta_bias")}
    yield dict(u=u, delta=delta, z=z, B=B, C=C, **p)
    del u, delta, z, B, C
    torch.cuda.empty_cache()


def _row(t, r):
    """Row r of a (BT, DN, L) device tensor as float64 on the host."""
    return host64(t.reshape(BT * DN, -1)[r])


def _one_row_problem(x, r):
    """The inputs of flat row r as a (1, 1, L) problem (B / C of its batch, A / D / bias of its
    channel) in float64 on the host."""
    b, d = divmod(r, DN)
    return dict(u=_row(x["u"], r)[None, None], delta=_row(x["delta"], r)[None, None],
                z=_row(x["z"], r)[None, None], B=host64(x["B"][b])[None], C=host64(x["C"][b])[None],
                A=host64(x["A"][d])[None], D=host64(x["D"][d : d + 1]),
                delta_bias=host64(x["delta_bias"][d : d + 1]))


def test_forward_past_2_31_elements(mss, oracle_mod, layer):
    import torch
    out, last = mss.selective_scan_fwd(layer["u"], layer["delta"], layer["A"], layer["B"], layer["C"],
                                       D=layer["D"], z=layer["z"], delta_bias=layer["delta_bias"])
    torch.cuda.synchronize()
    for r in ROWS:
        q = _one_row_problem(layer, r)
        ref_out, ref_last = oracle_mod.selective_scan(q["u"], q["delta"], q["A"], q["B"], q["C"], D=q["D"],
                                                      z=q["z"], delta_bias=q["delta_bias"])
        assert_close(_row(out, r), ref_out[0, 0], what=f"out row {r}", **TOL_BF16)
        assert_close(host64(last.reshape(-1, N)[r]), ref_last[0, 0], what=f"last_state row {r}", **TOL_F32)
    del out, last
    torch.cuda.empty_cache()


def test_forward_dstate128_past_2_31_elements(mss, oracle_mod, layer):
    """The general kernels (d_state 128, four-wavefront workgroups) on the same u / delta / z with
    B, C of 128 states: the sampled rows' outputs and final states against the oracle."""
    import torch
    N2 = 128
    g = torch.Generator(device="cuda").manual_seed(2029)
    B = torch.randn((BT, N2, L), generator=g, device="cuda", dtype=torch.float32)
    C = torch.randn((BT, N2, L), generator=g, device="cuda", dtype=torch.float32)
    small = scan_inputs(1, DN, N2, 1, dtype="f32", seed=9)
    A = torch.from_numpy(small.A).to("cuda")
    out, last = mss.selective_scan_fwd(layer["u"], layer["delta"], A, B, C, D=layer["D"], z=layer["z"],
                                       delta_bias=layer["delta_bias"])
    torch.cuda.synchronize()
    for r in ROWS:
        b, d = divmod(r, DN)
        ref_out, ref_last = oracle_mod.selective_scan(
            _row(layer["u"], r)[None, None], _row(layer["delta"], r)[None, None], host64(A[d])[None],
            host64(B[b])[None], host64(C[b])[None], D=host64(layer["D"][d : d + 1]), z=_row(layer["z"], r)[None, None],
            delta_bias=host64(layer["delta_bias"][d : d + 1]))
        assert_close(_row(out, r), ref_out[0, 0], what=f"d_state 128 out row {r}", **TOL_BF16)
        assert_close(host64(last.reshape(-1, N2)[r]), ref_last[0, 0], what=f"d_state 128 last_state row {r}",
                     **TOL_F32)
    del out, last, B, C
    torch.cuda.empty_cache()


def test_backward_past_2_31_elements(mss, oracle_mod, layer):
    """du, ddelta, dz of the sampled rows (each depends only on its own row); the sums over rows
    (dA, dB, dC, dD, dbias) must be finite."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(2025)
    dout = torch.randn((BT, DN, L), generator=g, device="cuda", dtype=torch.bfloat16)
    grads = mss.selective_scan_bwd(layer["u"], layer["delta"], layer["A"], layer["B"], layer["C"], dout,
                                   D=layer["D"], z=layer["z"], delta_bias=layer["delta_bias"])
    torch.cuda.synchronize()
    for k in ("dA", "dB", "dC", "dD", "ddelta_bias"):
        assert bool(torch.isfinite(grads[k]).all()), k
    for r in ROWS:
        q = _one_row_problem(layer, r)
        kw = dict(D=q["D"], z=q["z"], delta_bias=q["delta_bias"], dout=_row(dout, r)[None, None])
        ref = oracle_mod.selective_scan_bwd(q["u"], q["delta"], q["A"], q["B"], q["C"], **kw)
        mag = oracle_mod.selective_scan_bwd(q["u"], q["delta"], q["A"], q["B"], q["C"], magnitude=True, **kw)
        for k in ("du", "ddelta", "dz"):
            got = _row(grads[k], r)
            lim = 2e-2 * np.abs(ref[k][0, 0]) + 1e-4 * mag[k][0, 0] + 1e-6
            ratio = np.abs(got - ref[k][0, 0]) / lim
            assert ratio.max() <= 1.0, (k, r, float(ratio.max()), int((ratio > 1).sum()))
    del grads, dout
    torch.cuda.empty_cache()


def test_conv1d_past_2_31_elements(mss, oracle_mod, layer):
    import torch
    g = torch.Generator(device="cuda").manual_seed(2026)
    w = torch.randn((DN, 4), generator=g, device="cuda") * 0.5
    bias = torch.randn((DN,), generator=g, device="cuda")
    out, fin = mss.causal_conv1d_fwd(layer["u"], w, bias, return_final_state=True)
    torch.cuda.synchronize()
    for r in ROWS:
        d = r % DN
        ref, ref_fin = oracle_mod.causal_conv1d(_row(layer["u"], r)[None, None], host64(w[d])[None],
                                                host64(bias[d : d + 1]))
        assert_close(_row(out, r), ref[0, 0], what=f"conv row {r}", **TOL_BF16)
        assert np.array_equal(_row(fin, r), ref_fin[0, 0]), r   # the last K - 1 inputs, exactly
    del out, fin
    torch.cuda.empty_cache()


def test_saved_states_past_2_31_elements(mss, oracle_mod, layer):
    """The forward that saves states and the backward that reads them (saved states of 4.3 GB,
    offsets past 2^31 floats): sampled saved blocks and du / ddelta / dz rows against the oracle."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(2027)
    dout = torch.randn((BT, DN, L), generator=g, device="cuda", dtype=torch.bfloat16)
    _, _, saved = mss.selective_scan_fwd_save(layer["u"], layer["delta"], layer["A"], layer["B"], layer["C"],
                                              D=layer["D"], z=layer["z"], delta_bias=layer["delta_bias"])
    grads = mss.selective_scan_bwd(layer["u"], layer["delta"], layer["A"], layer["B"], layer["C"], dout,
                                   D=layer["D"], z=layer["z"], delta_bias=layer["delta_bias"],
                                   saved_states=saved)
    torch.cuda.synchronize()
    for r in ROWS[-2:]:
        q = _one_row_problem(layer, r)
        for k8 in (1, L // 8 - 1):   # state entering step 8 k8: the row's scan stopped there
            _, want = oracle_mod.selective_scan(q["u"], q["delta"], q["A"], q["B"], q["C"], D=q["D"], z=q["z"],
                                                delta_bias=q["delta_bias"], seq_lens=np.array([8 * k8]))
            got = host64(saved[k8].reshape(4, BT * DN, 4)[:, r, :].reshape(-1))
            assert_close(got, want[0, 0], what=f"saved[{k8}] row {r}", **TOL_F32)
        kw = dict(D=q["D"], z=q["z"], delta_bias=q["delta_bias"], dout=_row(dout, r)[None, None])
        ref = oracle_mod.selective_scan_bwd(q["u"], q["delta"], q["A"], q["B"], q["C"], **kw)
        mag = oracle_mod.selective_scan_bwd(q["u"], q["delta"], q["A"], q["B"], q["C"], magnitude=True, **kw)
        for k in ("du", "ddelta", "dz"):
            got = _row(grads[k], r)
            lim = 2e-2 * np.abs(ref[k][0, 0]) + 1e-4 * mag[k][0, 0] + 1e-6
            ratio = np.abs(got - ref[k][0, 0]) / lim
            assert ratio.max() <= 1.0, (k, r, float(ratio.max()), int((ratio > 1).sum()))
    del grads, dout, saved
    torch.cuda.empty_cache()


@pytest.mark.parametrize("N,Bt", [(16, 2100), (128, 260)])
def test_decode_past_2_31_state_elements(mss, oracle_mod, N, Bt):
    """One decode step on a (2100, 65600, 16) or (260, 65600, 128) state (2.2e9 floats, 8.8 GB):
    sampled rows past element 2^31 against the oracle."""
    import torch
    rows = [0, 65599, int(0.99 * Bt * DN), Bt * DN - 1]   # the last two past element 2^31
    assert Bt * DN * N > 2**31
    g = torch.Generator(device="cuda").manual_seed(2028)
    state = torch.randn((Bt, DN, N), generator=g, device="cuda") * 0.5
    x, dt, z = (torch.randn((Bt, DN), generator=g, device="cuda", dtype=torch.bfloat16) for _ in range(3))
    B = torch.randn((Bt, N), generator=g, device="cuda")
    C = torch.randn((Bt, N), generator=g, device="cuda")
    small = scan_inputs(1, DN, N, 1, dtype="f32", seed=8)
    A, D, bias = (torch.from_numpy(getattr(small, k)).to("cuda") for k in ("A", "D", "delta_bias"))
    before = [np.ascontiguousarray(host64(state.reshape(-1, N)[r]).reshape(1, 1, N)) for r in rows]
    out = mss.selective_state_update(state, x, dt, A, B, C, D=D, z=z, dt_bias=bias)
    torch.cuda.synchronize()
    for r, ref_state in zip(rows, before):   # each row as a (1, 1, N) problem of its own
        b, d = divmod(r, DN)
        one = lambda t: host64(t[b, d]).reshape(1, 1)
        ref_out = oracle_mod.selective_state_update(ref_state, one(x), one(dt), host64(A[d]).reshape(1, N),
                                                    host64(B[b]).reshape(1, N), host64(C[b]).reshape(1, N),
                                                    D=host64(D[d : d + 1]), z=one(z),
                                                    dt_bias=host64(bias[d : d + 1]))
        assert_close(host64(out[b, d]).reshape(1, 1), ref_out, what=f"decode out row {r}", **TOL_BF16)
        assert_close(host64(state[b, d]).reshape(1, 1, N), ref_state, what=f"decode state row {r}", **TOL_F32)
    del state, x, dt, z, B, C, out
    torch.cuda.empty_cache()
