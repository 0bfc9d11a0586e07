"""Pins of the fp64 causal conv1d oracle (the depthwise, causally padded Conv1D + swish in front
of the scan in the tutorial page's `MambaBlock`).

Independent routes: numpy.convolve and scipy.signal.lfilter (a causal FIR filter is the same
sum with the taps reversed), an impulse response read off by hand, the Keras 'causal' padding
convention at t = 0, and chunking / one-token continuation identities.
"""
import numpy as np
import pytest
from scipy.signal import lfilter
from scipy.special import expit


def _case(seed, Bt=2, Dn=3, L=40, K=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((Bt, Dn, L)), rng.standard_normal((Dn, K)),
            rng.standard_normal(Dn), rng.standard_normal((Bt, Dn, K - 1)))


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_matches_numpy_convolve(oracle_mod, K):
    x, w, b, _ = _case(80 + K, K=K)
    out, _ = oracle_mod.causal_conv1d(x, w, b, silu=False)
    for bi in range(x.shape[0]):
        for d in range(x.shape[1]):
            padded = np.concatenate([np.zeros(K - 1), x[bi, d]])
            ref = np.convolve(padded, w[d][::-1], mode="valid") + b[d]
            np.testing.assert_allclose(out[bi, d], ref, rtol=1e-13, atol=1e-14)


def test_matches_lfilter_with_state_and_silu(oracle_mod):
    x, w, b, st = _case(85)
    out, fin = oracle_mod.causal_conv1d(x, w, b, state=st, silu=True)
    for bi in range(x.shape[0]):
        for d in range(x.shape[1]):
            seq = np.concatenate([st[bi, d], x[bi, d]])
            y = lfilter(w[d][::-1], [1.0], seq)[3:] + b[d]
            np.testing.assert_allclose(out[bi, d], y * expit(y), rtol=1e-12, atol=1e-14)
            np.testing.assert_array_equal(fin[bi, d], x[bi, d, -3:])


def test_impulse_response_and_causal_padding(oracle_mod):
    K, L, t0 = 4, 12, 5
    x = np.zeros((1, 1, L))
    x[0, 0, t0] = 1.0
    w = np.array([[0.1, -0.2, 0.3, 0.7]])
    out, _ = oracle_mod.causal_conv1d(x, w, None, silu=False)
    expect = np.zeros(L)
    expect[t0:t0 + K] = w[0][::-1]            # the newest tap answers first
    np.testing.assert_array_equal(out[0, 0], expect)
    x2 = np.arange(1.0, L + 1.0).reshape(1, 1, L)
    out2, _ = oracle_mod.causal_conv1d(x2, w, np.array([0.5]), silu=False)
    assert out2[0, 0, 0] == 0.5 + 0.7 * 1.0   # zero left padding: only w[K-1] x[0] at t = 0


@pytest.mark.parametrize("cut", [0, 1, 2, 17, 40])
def test_chunked_equals_whole(oracle_mod, cut):
    x, w, b, st = _case(86)
    whole, fin = oracle_mod.causal_conv1d(x, w, b, state=st)
    o1, s1 = oracle_mod.causal_conv1d(x[..., :cut], w, b, state=st)
    o2, s2 = oracle_mod.causal_conv1d(x[..., cut:], w, b, state=s1)
    np.testing.assert_allclose(np.concatenate([o1, o2], -1), whole, rtol=0, atol=0)
    np.testing.assert_array_equal(s2, fin)


def test_short_sequence_keeps_old_state(oracle_mod):
    x, w, b, st = _case(87, L=1)
    _, fin = oracle_mod.causal_conv1d(x, w, b, state=st)
    np.testing.assert_array_equal(fin[..., :2], st[..., 1:])
    np.testing.assert_array_equal(fin[..., 2], x[..., 0])
