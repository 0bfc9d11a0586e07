"""The scan forward (d_state 16, 64 and 128), the forward that saves states, both backwards and the
decode step captured in a HIP graph
(torch.cuda.graph) and replayed: every replay, with new inputs copied in between and eager
library calls interleaved, must give exactly the eager results for those inputs.  The library's
workspace belongs to a (device, stream) pair, so one warm-up call on the capture stream comes
first (it allocates the workspace outside the capture); the kernels clear their scratch with
kernels, not memset nodes.
"""
import numpy as np
import pytest

from synth import scan_inputs
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mss():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_06_amd as m
    m.load_library()
    return m


def _inputs(dtype, seed, Bt=2, Dn=192, L=520):
    s = scan_inputs(Bt, Dn, 16, L, dtype=dtype, seed=seed)
    g = np.random.default_rng(700 + seed).standard_normal(s.u.shape).astype(np.float32)
    return dict(u=dev(s.u, dtype), delta=dev(s.delta, dtype), z=dev(s.z, dtype), B=dev(s.B), C=dev(s.C),
                dout=dev(g, dtype)), dict(A=dev(s.A), D=dev(s.D), bias=dev(s.delta_bias))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_graph_replays_match_eager(mss, dtype):
    import torch
    x, p = _inputs(dtype, 1)
    Bt, Dn, L = x["u"].shape
    out = torch.empty_like(x["u"])
    last = torch.empty((Bt, Dn, 16), dtype=torch.float32, device="cuda")
    out_s = torch.empty_like(x["u"])
    last_s = torch.empty_like(last)
    saved = torch.empty(((L + 7) // 8, 4, Bt * Dn * 4), dtype=torch.float32, device="cuda")

    def body():
        mss.selective_scan_fwd(x["u"], x["delta"], p["A"], x["B"], x["C"], D=p["D"], z=x["z"],
                               delta_bias=p["bias"], out=out, last_state=last)
        mss.selective_scan_fwd_save(x["u"], x["delta"], p["A"], x["B"], x["C"], D=p["D"], z=x["z"],
                                    delta_bias=p["bias"], out=out_s, last_state=last_s, saved_states=saved)
        g1 = mss.selective_scan_bwd(x["u"], x["delta"], p["A"], x["B"], x["C"], x["dout"], D=p["D"],
                                    z=x["z"], delta_bias=p["bias"])
        g2 = mss.selective_scan_bwd(x["u"], x["delta"], p["A"], x["B"], x["C"], x["dout"], D=p["D"],
                                    z=x["z"], delta_bias=p["bias"], saved_states=saved)
        return g1, g2

    def snapshot(g1, g2):
        r = {"out": out.clone(), "last": last.clone(), "out_s": out_s.clone(), "last_s": last_s.clone(),
             "saved": saved.clone()}
        for k, v in g1.items():
            if v is not None:
                r["g1_" + k] = v.clone()
        for k, v in g2.items():
            if v is not None:
                r["g2_" + k] = v.clone()
        return r

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        body()  # warm-up on the capture stream: the workspace is allocated here
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        gg1, gg2 = body()
    torch.cuda.synchronize()

    for rep in range(3):
        nx, _ = _inputs(dtype, 10 + rep)
        for k in x:
            x[k].copy_(nx[k])
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):  # eager on the same inputs (and the same workspace)
            e1, e2 = body()
        torch.cuda.synchronize()
        eager = snapshot(e1, e2)
        graph.replay()
        torch.cuda.synchronize()
        replayed = snapshot(gg1, gg2)
        assert set(eager) == set(replayed)
        for k in eager:
            assert torch.equal(eager[k], replayed[k]), (dtype, rep, k)
        # the results changed with the inputs (the replay did run)
        if rep > 0:
            assert not torch.equal(replayed["out"], prev_out)
        prev_out = replayed["out"].clone()


def test_graph_replays_after_the_workspace_grew(mss):
    """A graph captured while its stream's workspace was small keeps replaying correctly after a
    larger call on the same stream replaced that workspace (the library keeps the old buffer)."""
    import torch
    x, p = _inputs("bf16", 2, Bt=1, Dn=64, L=256)
    out = torch.empty_like(x["u"])
    last = torch.empty((1, 64, 16), dtype=torch.float32, device="cuda")

    def small():
        mss.selective_scan_fwd(x["u"], x["delta"], p["A"], x["B"], x["C"], D=p["D"], z=x["z"],
                               delta_bias=p["bias"], out=out, last_state=last)
        return mss.selective_scan_bwd(x["u"], x["delta"], p["A"], x["B"], x["C"], x["dout"], D=p["D"],
                                      z=x["z"], delta_bias=p["bias"])

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        small()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        gg = small()
    torch.cuda.synchronize()
    big_x, big_p = _inputs("bf16", 3, Bt=2, Dn=1024, L=2048)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):  # needs far more workspace: the stream's buffer is replaced
        mss.selective_scan_fwd(big_x["u"], big_x["delta"], big_p["A"], big_x["B"], big_x["C"], D=big_p["D"],
                               z=big_x["z"], delta_bias=big_p["bias"])
        mss.selective_scan_bwd(big_x["u"], big_x["delta"], big_p["A"], big_x["B"], big_x["C"], big_x["dout"],
                               D=big_p["D"], z=big_x["z"], delta_bias=big_p["bias"])
    torch.cuda.synchronize()
    for rep in range(2):
        nx, _ = _inputs("bf16", 20 + rep, Bt=1, Dn=64, L=256)
        for k in x:
            x[k].copy_(nx[k])
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e = small()
            eager = {"out": out.clone(), "last": last.clone(), **{k: v.clone() for k, v in e.items() if v is not None}}
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replayed = {"out": out, "last": last, **{k: v for k, v in gg.items() if v is not None}}
        for k in eager:
            assert torch.equal(eager[k], replayed[k]), (rep, k)


def test_capture_that_needs_a_larger_workspace_is_refused(mss):
    """Under stream capture nothing can be allocated: a call whose stream has no workspace yet is
    refused with MSS_ERR_UNSUPPORTED (before any HIP call), and the capture can still end."""
    import torch
    x, p = _inputs("bf16", 4, Bt=1, Dn=64, L=256)
    stream = torch.cuda.Stream()  # never used by the library: no workspace
    stream.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(mss.MssError) as ei:
        with torch.cuda.graph(graph, stream=stream):
            x["u"].mul_(1.0)  # the graph is not empty
            mss.selective_scan_fwd(x["u"], x["delta"], p["A"], x["B"], x["C"], D=p["D"], z=x["z"],
                                   delta_bias=p["bias"])
    assert ei.value.status == -6  # MSS_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):  # outside the capture the same call runs
        out, _ = mss.selective_scan_fwd(x["u"], x["delta"], p["A"], x["B"], x["C"], D=p["D"], z=x["z"],
                                        delta_bias=p["bias"])
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()


def test_concurrent_streams_have_separate_workspaces(mss):
    """Forward + backward (and the saved-state pair) on two streams at once, each on its own inputs:
    the workspace belongs to the (device, stream) pair, so the overlapping calls must give
    exactly what each gives alone."""
    import torch
    xs, ps = zip(*[_inputs("bf16", 40 + k, Bt=2, Dn=320, L=1536) for k in range(2)])
    torch.cuda.synchronize()  # the inputs were made on the default stream

    def work(x, p):
        out, last = mss.selective_scan_fwd(x["u"], x["delta"], p["A"], x["B"], x["C"], D=p["D"], z=x["z"],
                                           delta_bias=p["bias"])
        _, _, saved = mss.selective_scan_fwd_save(x["u"], x["delta"], p["A"], x["B"], x["C"], D=p["D"],
                                                  z=x["z"], delta_bias=p["bias"])
        g = mss.selective_scan_bwd(x["u"], x["delta"], p["A"], x["B"], x["C"], x["dout"], D=p["D"], z=x["z"],
                                   delta_bias=p["bias"])
        gs = mss.selective_scan_bwd(x["u"], x["delta"], p["A"], x["B"], x["C"], x["dout"], D=p["D"],
                                    z=x["z"], delta_bias=p["bias"], saved_states=saved)
        r = {"out": out, "last": last, "saved": saved}
        r.update({"g_" + k: v for k, v in g.items() if v is not None})
        r.update({"gs_" + k: v for k, v in gs.items() if v is not None})
        return r

    streams = [torch.cuda.Stream() for _ in range(2)]
    alone = []
    for k in range(2):  # one at a time (also allocates each stream's workspace)
        with torch.cuda.stream(streams[k]):
            alone.append({n: v.clone() for n, v in work(xs[k], ps[k]).items()})
        torch.cuda.synchronize()
    for rep in range(3):  # both queued before either is waited for
        res = []
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                res.append(work(xs[k], ps[k]))
        torch.cuda.synchronize()
        for k in range(2):
            for n, v in alone[k].items():
                assert torch.equal(res[k][n], v), (rep, k, n)


def test_ssd_graph_replays_match_eager(mss):
    """Mamba-2's SSD layer (segment split: its segment states pass through the workspace) captured
    after a warm-up on the capture stream: every replay, with new inputs copied in, equals the eager
    call on those inputs bit for bit."""
    import torch
    from synth import ssd_inputs

    def inputs(seed):
        s = ssd_inputs(2, 700, 4, 64, 2, 64, dtype="bf16", with_z=True, seed=seed)
        return dict(x=dev(s.x, "bf16"), dt=dev(s.dt, "bf16"), z=dev(s.z, "bf16"), B=dev(s.B, "bf16"),
                    C=dev(s.C, "bf16")), dict(A=dev(s.A), D=dev(s.D), bias=dev(s.dt_bias))

    x, p = inputs(80)
    out = torch.empty_like(x["x"])
    last = torch.empty((2, 4, 64, 64), dtype=torch.float32, device="cuda")

    def body():
        mss.ssd_scan_fwd(x["x"], x["dt"], p["A"], x["B"], x["C"], D=p["D"], z=x["z"], dt_bias=p["bias"],
                         out=out, last_state=last)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        body()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        body()
    torch.cuda.synchronize()
    prev = None
    for rep in range(3):
        nx, _ = inputs(81 + rep)
        for k in x:
            x[k].copy_(nx[k])
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            body()
        torch.cuda.synchronize()
        eager = (out.clone(), last.clone())
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(eager[0], out) and torch.equal(eager[1], last), rep
        if prev is not None:
            assert not torch.equal(prev, out)
        prev = out.clone()


@pytest.mark.parametrize("N", [64, 128])
def test_dstate_graph_replays_match_eager(mss, N):
    """The general forward at d_state 64 / 128 with a segment split (its aggregates and the
    combine kernel go through the workspace) and a decode step at the same d_state, captured after
    a warm-up on the capture stream: every replay, with new inputs copied in and the decode state
    reset, equals the eager calls on those inputs bit for bit."""
    import torch
    from synth import decode_inputs

    Bt, Dn, L = 1, 96, 600

    def inputs(seed):
        s = scan_inputs(Bt, Dn, N, L, dtype="bf16", seed=seed, a_kind="random" if N == 64 else "s4d")
        d = decode_inputs(Bt, Dn, N, 1, dtype="bf16", seed=seed)
        return dict(u=dev(s.u, "bf16"), delta=dev(s.delta, "bf16"), z=dev(s.z, "bf16"), B=dev(s.B), C=dev(s.C),
                    x1=dev(d.x[0], "bf16"), dt1=dev(d.dt[0], "bf16"), B1=dev(d.B[0]), C1=dev(d.C[0])), \
            dict(A=dev(s.A), D=dev(s.D), bias=dev(s.delta_bias))

    x, p = inputs(90)
    out = torch.empty_like(x["u"])
    last = torch.empty((Bt, Dn, N), dtype=torch.float32, device="cuda")
    state0 = torch.randn((Bt, Dn, N), device="cuda") * 0.5
    state = state0.clone()
    out1 = torch.empty((Bt, Dn), dtype=torch.bfloat16, device="cuda")

    def body():
        mss.selective_scan_fwd(x["u"], x["delta"], p["A"], x["B"], x["C"], D=p["D"], z=x["z"],
                               delta_bias=p["bias"], out=out, last_state=last)
        mss.selective_state_update(state, x["x1"], x["dt1"], p["A"], x["B1"], x["C1"], D=p["D"],
                                   dt_bias=p["bias"], out=out1)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        body()  # allocates the workspace outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        body()
    torch.cuda.synchronize()
    prev = None
    for rep in range(3):
        nx, _ = inputs(91 + rep)
        for k in x:
            x[k].copy_(nx[k])
        state.copy_(state0)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            body()
        torch.cuda.synchronize()
        eager = (out.clone(), last.clone(), state.clone(), out1.clone())
        state.copy_(state0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (out, last, state, out1)
        for k in range(4):
            assert torch.equal(eager[k], got[k]), (N, rep, k)
        if prev is not None:
            assert not torch.equal(prev, out)
        prev = out.clone()
