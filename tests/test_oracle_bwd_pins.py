"""Pins of the fp64 backward oracle (gradients of L = sum(dout * out)).

The pages print no gradient, so every check here is computed by a route independent of the
adjoint loop: central finite differences of the (separately pinned) forward oracle, a
closed form at L = 1 derived by hand from the forward formula, and properties every correct
adjoint has (linearity in dout, zero dout, |grad| <= sum |terms|).
"""
import numpy as np
import pytest
from scipy.special import expit

from synth import scan_inputs

GRAD_OF = {"u": "du", "delta": "ddelta", "z": "dz", "A": "dA", "B": "dB", "C": "dC",
           "D": "dD", "delta_bias": "ddelta_bias"}


def _fields(s, **over):
    a = dict(u=s.u, delta=s.delta, A=s.A, B=s.B, C=s.C, D=s.D, z=s.z, delta_bias=s.delta_bias)
    a.update(over)
    return {k: (None if v is None else np.asarray(v, dtype=np.float64)) for k, v in a.items()}


def _loss(orc, a, dout, softplus):
    out, _ = orc.selective_scan(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                a["delta_bias"], softplus_flag=softplus)
    return float(np.sum(out * dout))


def _bwd(orc, a, dout, softplus, **kw):
    return orc.selective_scan_bwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                  a["delta_bias"], softplus_flag=softplus, dout=dout, **kw)


def _fd_check(orc, a, dout, softplus, names, sample=None, seed=0, h=1e-6):
    g = _bwd(orc, a, dout, softplus)
    rng = np.random.default_rng(seed)
    for name in names:
        base = a[name]
        idx = list(np.ndindex(base.shape))
        if sample is not None and len(idx) > sample:
            idx = [idx[i] for i in rng.choice(len(idx), sample, replace=False)]
        for i in idx:
            p, m = base.copy(), base.copy()
            p[i] += h
            m[i] -= h
            fd = (_loss(orc, {**a, name: p}, dout, softplus) -
                  _loss(orc, {**a, name: m}, dout, softplus)) / (2 * h)
            got = g[GRAD_OF[name]][i]
            assert abs(got - fd) <= 2e-7 + 1e-6 * abs(fd), (name, i, got, fd)


@pytest.mark.parametrize("case", ["full", "bare", "no_softplus", "random_A"])
def test_gradients_match_finite_differences(oracle_mod, case):
    s = scan_inputs(2, 3, 5, 12, dtype="f32", seed=51, a_kind="random" if case == "random_A" else "s4d")
    dout = np.random.default_rng(52).standard_normal(s.u.shape)
    softplus = case != "no_softplus"
    if case == "bare":
        a = _fields(s, D=None, z=None, delta_bias=None)
        names = ["u", "delta", "A", "B", "C"]
    else:
        a = _fields(s)
        names = list(GRAD_OF)
    if case == "no_softplus":  # delta used directly: keep it a valid positive step
        a["delta"] = np.abs(a["delta"]) * 0.05
        a["delta_bias"] = np.full(3, 0.01)
    _fd_check(oracle_mod, a, dout, softplus, names)
    if case == "bare":  # gradients at D = 0 and bias = 0 are still defined
        g = _bwd(oracle_mod, a, dout, softplus)
        a0 = {**a, "D": np.zeros(3), "delta_bias": np.zeros(3)}
        _fd_check(oracle_mod, a0, dout, softplus, ["D", "delta_bias"])
        g0 = _bwd(oracle_mod, a0, dout, softplus)
        np.testing.assert_allclose(g["dD"], g0["dD"], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(g["ddelta_bias"], g0["ddelta_bias"], rtol=1e-14, atol=1e-15)


def test_long_sequence_sampled_finite_differences(oracle_mod):
    """Gradients reaching back across 200 steps (the adjoint's carry through abar)."""
    s = scan_inputs(1, 2, 16, 200, dtype="f32", seed=53)
    s.delta_bias = np.full_like(s.delta_bias, -4.0)  # small steps: long memory
    a = _fields(s)
    dout = np.zeros(s.u.shape)
    dout[..., -1] = 1.0                               # only the last output matters
    _fd_check(oracle_mod, a, dout, True, list(GRAD_OF), sample=12, seed=54)


def test_single_step_closed_form(oracle_mod):
    """L = 1 from h_0 = 0: out = (dt u C.B + D u) silu(z), differentiated by hand."""
    s = scan_inputs(2, 4, 6, 1, dtype="f32", seed=55)
    a = _fields(s)
    dout = np.random.default_rng(56).standard_normal(s.u.shape)
    g = _bwd(oracle_mod, a, dout, True)
    u, z, dl_raw = a["u"][..., 0], a["z"][..., 0], a["delta"][..., 0]      # (Bt, Dn)
    pre = dl_raw + a["delta_bias"][None, :]
    dt = np.logaddexp(0.0, pre)
    CB = np.einsum("bn,bn->b", a["C"][..., 0], a["B"][..., 0])[:, None]    # (Bt, 1)
    sig = expit(z)
    silu = z * sig
    go = dout[..., 0]
    dy = go * silu
    y = dt * u * CB + a["D"][None, :] * u
    np.testing.assert_allclose(g["du"][..., 0], dy * (dt * CB + a["D"][None, :]), rtol=1e-12)
    np.testing.assert_allclose(g["ddelta"][..., 0], dy * u * CB * expit(pre), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(g["dz"][..., 0], go * y * sig * (1 + z * (1 - sig)), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(g["dD"], np.sum(dy * u, axis=0), rtol=1e-12)
    np.testing.assert_allclose(g["ddelta_bias"], np.sum(dy * u * CB * expit(pre), axis=0), rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(g["dA"], 0.0)                              # h_0 = 0
    w = dy * dt * u                                                           # (Bt, Dn)
    np.testing.assert_allclose(g["dB"][..., 0], np.sum(w, 1)[:, None] * a["C"][..., 0], rtol=1e-12)
    np.testing.assert_allclose(g["dC"][..., 0], np.sum(w, 1)[:, None] * a["B"][..., 0], rtol=1e-12)


def test_linear_in_dout_and_zero(oracle_mod):
    s = scan_inputs(2, 3, 5, 20, dtype="f32", seed=57)
    a = _fields(s)
    rng = np.random.default_rng(58)
    d1, d2 = rng.standard_normal(s.u.shape), rng.standard_normal(s.u.shape)
    g1, g2 = _bwd(oracle_mod, a, d1, True), _bwd(oracle_mod, a, d2, True)
    g3 = _bwd(oracle_mod, a, 2.0 * d1 - 0.5 * d2, True)
    g0 = _bwd(oracle_mod, a, np.zeros(s.u.shape), True)
    for k in GRAD_OF.values():
        np.testing.assert_allclose(g3[k], 2.0 * g1[k] - 0.5 * g2[k], rtol=1e-11, atol=1e-13)
        assert not np.any(g0[k])


def test_magnitude_bounds_gradient(oracle_mod):
    s = scan_inputs(2, 3, 5, 30, dtype="f32", seed=59, a_kind="random")
    a = _fields(s)
    dout = np.random.default_rng(60).standard_normal(s.u.shape)
    g = _bwd(oracle_mod, a, dout, True)
    m = _bwd(oracle_mod, a, dout, True, magnitude=True)
    for k in GRAD_OF.values():
        assert np.all(m[k] >= 0)
        assert np.all(np.abs(g[k]) <= m[k] * (1 + 1e-12) + 1e-300), k
    # a one-term sum: dD with one batch and one step is |dy u|
    s1 = scan_inputs(1, 3, 5, 1, dtype="f32", seed=61)
    a1 = _fields(s1)
    d1 = np.random.default_rng(62).standard_normal(s1.u.shape)
    np.testing.assert_allclose(_bwd(oracle_mod, a1, d1, True, magnitude=True)["dD"],
                               np.abs(_bwd(oracle_mod, a1, d1, True)["dD"]), rtol=1e-14)


def test_rows_and_threads_agree(oracle_mod):
    """Row subsets give the same per-row values; dB/dC do not depend on the thread count."""
    s = scan_inputs(2, 8, 16, 40, dtype="f32", seed=63)
    a = _fields(s)
    dout = np.random.default_rng(64).standard_normal(s.u.shape)
    g1 = _bwd(oracle_mod, a, dout, True, nthreads=1)
    g4 = _bwd(oracle_mod, a, dout, True, nthreads=4)
    for k in GRAD_OF.values():
        np.testing.assert_allclose(g4[k], g1[k], rtol=1e-13, atol=1e-15)
    rows = np.array([3, 9, 14])
    gr = _bwd(oracle_mod, a, dout, True, rows=rows)
    flat = lambda x: x.reshape(16, -1)
    np.testing.assert_array_equal(gr["du"], flat(g1["du"])[rows])
    np.testing.assert_array_equal(gr["ddelta"], flat(g1["ddelta"])[rows])
    np.testing.assert_array_equal(gr["dz"], flat(g1["dz"])[rows])

# ---------------------------------------------------------------- starting state, lengths, dL/dh_L

def _loss_ext(orc, a, dout, dlast, h0, lens):
    out, last = orc.selective_scan(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                   a["delta_bias"], h0=h0, seq_lens=lens)
    return float(np.sum(out * dout) + np.sum(last * dlast))


@pytest.mark.parametrize("lens", [None, [7, 12]])
def test_state_and_final_state_gradients_by_finite_differences(oracle_mod, lens):
    """L = sum(dout out) + sum(dlast h_L) from a given h0: every input's gradient and dL/dh0."""
    s = scan_inputs(2, 3, 5, 12, dtype="f32", seed=90)
    a = _fields(s)
    rng = np.random.default_rng(91)
    dout, dlast = rng.standard_normal(s.u.shape), rng.standard_normal((2, 3, 5))
    h0 = rng.standard_normal((2, 3, 5))
    ln = None if lens is None else np.array(lens)
    g = oracle_mod.selective_scan_bwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                      a["delta_bias"], dout=dout, h0=h0, seq_lens=ln, dlast=dlast)
    h = 1e-6
    targets = dict(GRAD_OF, h0="dh0")
    for name, gk in targets.items():
        base = h0 if name == "h0" else a[name]
        for i in np.ndindex(base.shape):
            p, m = base.copy(), base.copy()
            p[i] += h
            m[i] -= h
            if name == "h0":
                fp = _loss_ext(oracle_mod, a, dout, dlast, p, ln)
                fm = _loss_ext(oracle_mod, a, dout, dlast, m, ln)
            else:
                fp = _loss_ext(oracle_mod, {**a, name: p}, dout, dlast, h0, ln)
                fm = _loss_ext(oracle_mod, {**a, name: m}, dout, dlast, h0, ln)
            fd = (fp - fm) / (2 * h)
            assert abs(g[gk][i] - fd) <= 2e-7 + 1e-6 * abs(fd), (name, i, g[gk][i], fd)


def test_lengths_equal_truncated_rows(oracle_mod):
    """With lengths, each batch's gradients are those of its truncated problem; past the end 0."""
    s = scan_inputs(3, 2, 4, 10, dtype="f32", seed=92)
    a = _fields(s)
    rng = np.random.default_rng(93)
    dout, dlast, h0 = rng.standard_normal(s.u.shape), rng.standard_normal((3, 2, 4)), rng.standard_normal((3, 2, 4))
    lens = np.array([0, 4, 10])
    g = oracle_mod.selective_scan_bwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                      a["delta_bias"], dout=dout, h0=h0, seq_lens=lens, dlast=dlast)
    for b, lb in enumerate(lens):
        sl = (slice(b, b + 1), Ellipsis, slice(0, lb))
        gt = oracle_mod.selective_scan_bwd(a["u"][sl], a["delta"][sl], a["A"], a["B"][sl], a["C"][sl],
                                           a["D"], a["z"][sl], a["delta_bias"], dout=dout[sl],
                                           h0=h0[b:b + 1], dlast=dlast[b:b + 1])
        for k in ("du", "ddelta", "dz"):
            np.testing.assert_array_equal(g[k][b, :, :lb], gt[k][0])
            assert not np.any(g[k][b, :, lb:])
        np.testing.assert_array_equal(g["dh0"][b], gt["dh0"][0])
        np.testing.assert_array_equal(g["dB"][b, :, :lb], gt["dB"][0])
        assert not np.any(g["dB"][b, :, lb:]) and not np.any(g["dC"][b, :, lb:])
    np.testing.assert_array_equal(g["dh0"][0], dlast[0])        # empty sequence: dL/dh0 = dL/dh_L
