"""The plain-C example (selective_state_space_06_amd/examples/scan_from_c.c, built by the package
build) drives the library without Python or PyTorch: a forward scan over an L that is not a
whole number of 16-byte vectors, then one decode step from its final state.  Its inputs and
results, written to a file, are checked here against the fp64 oracle (fp32 tolerance: rtol
1e-4, atol 1e-5)."""
import os
import subprocess

import numpy as np
import pytest

from tests.gpu_helpers import TOL_F32, assert_close

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "selective_state_space_06_amd", "examples", "scan_from_c")


def _read(path):
    raw = open(path, "rb").read()
    Bt, Dn, N, L = np.frombuffer(raw[:16], dtype=np.int32)
    data = np.frombuffer(raw[16:], dtype=np.float32)
    shapes = [("u", (Bt, Dn, L)), ("delta", (Bt, Dn, L)), ("z", (Bt, Dn, L)), ("A", (Dn, N)),
              ("B", (Bt, N, L)), ("C", (Bt, N, L)), ("D", (Dn,)), ("bias", (Dn,)),
              ("out", (Bt, Dn, L)), ("last", (Bt, Dn, N)), ("x1", (Bt, Dn)), ("dt1", (Bt, Dn)),
              ("z1", (Bt, Dn)), ("B1", (Bt, N)), ("C1", (Bt, N)), ("state", (Bt, Dn, N)),
              ("out1", (Bt, Dn))]
    out, k = {}, 0
    for name, shp in shapes:
        n = int(np.prod(shp))
        out[name] = data[k:k + n].reshape(shp)
        k += n
    assert k == data.size
    return out


def test_c_program_matches_oracle(tmp_path, oracle_mod):
    assert os.path.exists(EXE), "build the package first (python -m selective_state_space_06_amd.build)"
    path = str(tmp_path / "scan_from_c.bin")
    r = subprocess.run([EXE, path], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    d = _read(path)
    assert d["u"].shape[2] % 4 != 0  # rows that are not whole 16-byte vectors
    ref_out, ref_last = oracle_mod.selective_scan(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                                                  z=d["z"], delta_bias=d["bias"])
    assert_close(d["out"].astype(np.float64), ref_out, what="C example out", **TOL_F32)
    assert_close(d["last"].astype(np.float64), ref_last, what="C example last_state", **TOL_F32)
    # the decode step continued from the GPU's own final state
    state = d["last"].astype(np.float64).copy()
    ref_out1 = oracle_mod.selective_state_update(state, d["x1"], d["dt1"], d["A"], d["B1"], d["C1"], D=d["D"],
                                                 z=d["z1"], dt_bias=d["bias"])
    assert_close(d["out1"].astype(np.float64), ref_out1, what="C example decode out", **TOL_F32)
    assert_close(d["state"].astype(np.float64), state, what="C example decode state", **TOL_F32)
