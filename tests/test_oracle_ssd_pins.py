"""Pins of the Mamba-2 SSD oracle (oracle_ssd_scan), each independent of its loop:

* the tie to the S6 oracle: SSD is the selective recurrence with A[d, n] = A[h] for every channel
  of head h and every state, delta shared by the head's channels and B / C of the head's group
  (contiguous blocks of H / G heads per group), so every (head, channel) row must equal
  oracle.selective_scan run on that row with those tied parameters (an S6 oracle pinned on its own);
* the quadratic ("masked attention") form, brute force: y_t = sum_{s <= t} (C_t . B_s)
  exp(A sum_{r=s+1}^{t} delta_r) delta_s x_s + D x_t, then the gate -- the unrolled recurrence
  written as a T x T matrix times x, with the exponent summed directly;
* the final state as the same unrolled sum;
* L = 1 closed form; a sequence cut in two and continued from the first part's state;
* magnitude mode: >= |value| everywhere and equal to it for all-positive inputs without a gate.
"""
import numpy as np
import pytest
from scipy.special import expit

from synth import ssd_inputs


def _sp(x):
    return np.logaddexp(0.0, x)


def _small(seed=1, Bt=2, L=20, H=4, P=3, G=2, N=5, with_z=True):
    s = ssd_inputs(Bt, L, H, P, G, N, dtype="f32", with_z=with_z, seed=seed)
    return s


def test_ssd_equals_tied_s6_rows(oracle_mod):
    s = _small()
    Bt, L, H, P = s.x.shape
    G, N = s.B.shape[2], s.B.shape[3]
    out, last = oracle_mod.ssd_scan(s.x, s.dt, s.A, s.B, s.C, D=s.D, z=s.z, dt_bias=s.dt_bias)
    hpg = H // G
    for h in range(H):
        g = h // hpg
        # S6 rows: channel p of head h; u, delta, z as (Bt, P, L); B, C as (Bt, N, L) of group g
        u = np.transpose(s.x[:, :, h, :], (0, 2, 1))
        dl = np.repeat(s.dt[:, None, :, h], P, axis=1)
        z = np.transpose(s.z[:, :, h, :], (0, 2, 1))
        A = np.full((P, N), s.A[h])
        B = np.transpose(s.B[:, :, g, :], (0, 2, 1))
        C = np.transpose(s.C[:, :, g, :], (0, 2, 1))
        o6, l6 = oracle_mod.selective_scan(u, dl, A, B, C, D=np.full(P, s.D[h]), z=z,
                                           delta_bias=np.full(P, s.dt_bias[h]))
        np.testing.assert_allclose(np.transpose(out[:, :, h, :], (0, 2, 1)), o6, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(last[:, h], l6, rtol=1e-13, atol=1e-14)


def test_ssd_quadratic_form(oracle_mod):
    s = _small(seed=2, L=17)
    Bt, L, H, P = s.x.shape
    G = s.B.shape[2]
    out, last = oracle_mod.ssd_scan(s.x, s.dt, s.A, s.B, s.C, D=s.D, z=s.z, dt_bias=s.dt_bias)
    x, B, C = s.x.astype(np.float64), s.B.astype(np.float64), s.C.astype(np.float64)
    delta = _sp(s.dt.astype(np.float64) + s.dt_bias.astype(np.float64))  # (Bt, L, H)
    hpg = H // G
    for b in range(Bt):
        for h in range(H):
            g = h // hpg
            a = float(s.A[h])
            M = np.zeros((L, L))
            for t in range(L):
                for r in range(t + 1):
                    M[t, r] = (C[b, t, g] @ B[b, r, g]) * np.exp(a * delta[b, r + 1:t + 1, h].sum()) * delta[b, r, h]
            y = M @ x[b, :, h, :] + s.D[h] * x[b, :, h, :]
            zz = s.z[b, :, h, :].astype(np.float64)
            y = y * zz * expit(zz)
            np.testing.assert_allclose(out[b, :, h, :], y, rtol=1e-11, atol=1e-12)
            # final state: sum_r exp(a sum_{q=r+1}^{L-1} delta_q) delta_r B_r x_r^T  -> (P, N)
            st = np.zeros((P, B.shape[3]))
            for r in range(L):
                st += np.exp(a * delta[b, r + 1:, h].sum()) * delta[b, r, h] * np.outer(x[b, r, h], B[b, r, g])
            np.testing.assert_allclose(last[b, h], st, rtol=1e-11, atol=1e-12)


def test_ssd_single_step_closed_form(oracle_mod):
    s = _small(seed=3, L=1)
    out, last = oracle_mod.ssd_scan(s.x, s.dt, s.A, s.B, s.C, D=s.D, z=s.z, dt_bias=s.dt_bias)
    Bt, _, H, P = s.x.shape
    G = s.B.shape[2]
    for b in range(Bt):
        for h in range(H):
            g = h // (H // G)
            d = _sp(float(s.dt[b, 0, h]) + float(s.dt_bias[h]))
            xv = s.x[b, 0, h].astype(np.float64)
            st = d * np.outer(xv, s.B[b, 0, g])
            np.testing.assert_allclose(last[b, h], st, rtol=1e-13)
            zz = s.z[b, 0, h].astype(np.float64)
            y = (d * xv * float(s.C[b, 0, g].astype(np.float64) @ s.B[b, 0, g].astype(np.float64)) + s.D[h] * xv)
            np.testing.assert_allclose(out[b, 0, h], y * zz * expit(zz), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("cut", [1, 7, 19])
def test_ssd_continued_from_state(oracle_mod, cut):
    s = _small(seed=4, L=20)
    full_out, full_last = oracle_mod.ssd_scan(s.x, s.dt, s.A, s.B, s.C, D=s.D, z=s.z, dt_bias=s.dt_bias)
    o1, l1 = oracle_mod.ssd_scan(s.x[:, :cut], s.dt[:, :cut], s.A, s.B[:, :cut], s.C[:, :cut], D=s.D,
                                 z=s.z[:, :cut], dt_bias=s.dt_bias)
    o2, l2 = oracle_mod.ssd_scan(s.x[:, cut:], s.dt[:, cut:], s.A, s.B[:, cut:], s.C[:, cut:], D=s.D,
                                 z=s.z[:, cut:], dt_bias=s.dt_bias, h0=l1)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), full_out)
    np.testing.assert_array_equal(l2, full_last)


def test_ssd_magnitude_mode(oracle_mod):
    s = _small(seed=5)
    out, last = oracle_mod.ssd_scan(s.x, s.dt, s.A, s.B, s.C, D=s.D, z=s.z, dt_bias=s.dt_bias)
    mo, ml = oracle_mod.ssd_scan(s.x, s.dt, s.A, s.B, s.C, D=s.D, z=s.z, dt_bias=s.dt_bias, magnitude=True)
    assert np.all(mo >= np.abs(out) * (1 - 1e-12)) and np.all(ml >= np.abs(last) * (1 - 1e-12))
    ax, aB, aC = np.abs(s.x), np.abs(s.B), np.abs(s.C)
    po, pl = oracle_mod.ssd_scan(ax, s.dt, s.A, aB, aC, D=s.D, dt_bias=s.dt_bias)
    mo2, ml2 = oracle_mod.ssd_scan(s.x, s.dt, s.A, s.B, s.C, D=s.D, dt_bias=s.dt_bias, magnitude=True)
    np.testing.assert_array_equal(mo2, po)
    np.testing.assert_array_equal(ml2, pl)


def test_ssd_pairs_subset_matches_full(oracle_mod):
    s = _small(seed=6)
    out, last = oracle_mod.ssd_scan(s.x, s.dt, s.A, s.B, s.C, D=s.D, z=s.z, dt_bias=s.dt_bias)
    H = s.x.shape[2]
    pairs = [1, 2 * H - 1]
    o2, l2 = oracle_mod.ssd_scan(s.x, s.dt, s.A, s.B, s.C, D=s.D, z=s.z, dt_bias=s.dt_bias, pairs=pairs)
    for bh in pairs:
        b, h = divmod(bh, H)
        np.testing.assert_array_equal(o2[b, :, h], out[b, :, h])
        np.testing.assert_array_equal(l2[b, h], last[b, h])
    assert np.isnan(o2[0, :, 0]).all()
