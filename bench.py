#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

One step = the whole hot path over one batch of the Mamba-2.8B-shaped layer
(batch 4, d_inner 5120, d_state 16, L 2048; bf16 u / delta / z / out, fp32 A / B / C / D /
state; softplus, delta bias, D skip and silu(z) gate on):
  1. mss_selective_scan_fwd over the 2048-token sequence (prefill), writing out and h_L;
  2. one mss_selective_state_update token continuing from h_L (decode).
Inputs are seeded synthetic data (synth.scan_inputs, seed 0) resident in HBM before timing.
Three copies of the inputs are rotated so that a step never finds its inputs in the 256 MB
Infinity Cache from the previous step.

Before its W warm-up steps every timed section runs its own call, untimed, for 0.25 s of wall
time (`clock_ramp` in the line): the GPU's clocks ramp up over the first few hundred
milliseconds of work after the host-side input generation, and the K timed steps should see
the steady clocks a serving process runs at (with 5 warm-up steps alone, 20 timed steps of the
forward average 0.27 ms per call against 0.235 ms at steady clocks).

Prints ONE JSON line.  `value` is algorithmic GB/s of the whole step (every input read once,
every output written once) over the K timed steps; the scan alone is also timed with HIP
events on the stream it runs on, and the library's launch-timing hook (mss_profile_enable /
mss_profile_fwd) times its two kernels separately over a second pass of the same steps (the
hook's events between the kernels cost ~11 us per call, so the timed steps run without it).

`roofline` prices the scan's dominant kernel, the main scan kernel, against HBM: achieved =
the call's algorithmic bytes (every input read once, every output written once: 338,272,256
bytes on this layer) / the main kernel's average duration (HIP events the library records on
the stream it launches on), against the 8 TB/s MI355X peak; `call_frac` is the same bytes over
the whole call (aggregate kernel + main kernel).  `traffic` is the main kernel's HBM bytes per
launch from rocprofv3 counters taken on this exact kernel source (null otherwise).  The scan is
in fact limited by VALU issue: `valu` gives the main kernel's counted instructions per
(b, d, t) and the issue rate they imply, against the one-instruction-per-4-cycles rate of a
wave64 fp32 VALU instruction on a 16-lane SIMD (1024 SIMDs at 2.4 GHz).

Beside the headline the line carries legs for the rest of the path: the backward, the causal
conv, the forward at shard shapes and with an unstructured A, the decode chain (cache- and
HBM-resident states; launches through the per-call wrapper, through bound steps and from a HIP
graph; beside the HBM-resident chains, torch's own in-place elementwise kernel over the same
states as a reference for what one launch over those bytes reaches), the fp32 workloads, and Mamba-2's SSD layer at d_state 64 and 128
(`ssd_scan`: call time, algorithmic GB/s and HBM fraction, MFMA TFLOP/s of the chunked form).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, AMD published peak
WORKLOAD = "mamba2p8b_bf16"
# VALU issue ceiling: 256 CUs x 4 SIMDs, one wave64 fp32 instruction per 4 cycles each (16 lanes),
# 2.4 GHz: 614.4e9 wave-instructions per second.  (Transcendentals take longer than one such slot;
# timing probes that are not shipped put v_exp_f32 near 8 and v_log_f32 / v_rcp_f32 near 12 cycles
# per wave instruction -- unverified here, and nothing below depends on it.)
VALU_WAVE_INSTR_PER_S = 256 * 4 * 2.4e9 / 4

# The GPU's clocks ramp up over the first few hundred milliseconds of work after an idle spell
# (generating inputs on the host leaves it idle): the 2.8B-layer forward takes 0.27 ms per call
# over its first ~30 calls, 0.235 ms once the clocks are up.  So each timed section first runs
# its own call for RAMP_S of wall time (untimed, on top of its warm-up calls) and times the
# steady state that a serving process runs at.
RAMP_S = 0.25


def ramp_clocks(torch, fn, seconds=RAMP_S, batch=8):
    """Runs fn(k) for k = 0, 1, ... in batches until `seconds` of wall time have passed; returns
    the number of calls."""
    t_end = time.perf_counter() + seconds
    n = 0
    while True:
        for _ in range(batch):
            fn(n)
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            return n

# Memory-side bytes per launch of the main scan kernel on this workload, from rocprofv3 --pmc
# runs of the headline alone (`python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-bwd
# --no-conv --no-shard --no-general-a --no-decode-chain --no-configs --no-ssd --no-dstate`): FETCH_SIZE, then
# WRITE_SIZE, each scaled by what the counter reads for a plain 1 GiB device copy (FETCH_SIZE x2:
# the L2 fills whole 128-byte lines, one TCC_EA0_RDREQ each, and the counter prices a request at 64
# bytes; WRITE_SIZE x1), and the VALU instructions per (b, d, t) (SQ_INSTS_VALU x 64 / B D L).
# Valid only for the kernel source with this SHA-256 prefix; otherwise reported as null.  (Taken
# on an earlier revision of this source that differs in comments and in where the step scale's
# helper is defined; every kernel compiles to the same machine code from both.)
MAIN_COUNTERS = {"src_sha256": "2339725ab3a89351", "fetch_bytes": 507106918, "write_bytes": 91376230,
                 "valu_per_bdt": 84.73}


def progress(what):
    """One line per finished leg on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {what} done", file=sys.stderr, flush=True)


def kernel_source_digest():
    import hashlib
    path = os.path.join(ROOT, "selective_state_space_06_amd", "csrc", "scan_fast.hip")
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def scan_bytes(Bt, Dn, N, L, es_io=2, with_z=True, last_state=True):
    """Algorithmic bytes of one forward scan: each input read once, each output written once."""
    io = Bt * Dn * L * es_io
    n = io * (3 if with_z else 2)          # u, delta (, z)
    n += 2 * Bt * N * L * 4                # B, C
    n += Dn * N * 4 + 2 * Dn * 4           # A, D, delta_bias
    n += io                                # out
    n += Bt * Dn * N * 4 if last_state else 0
    return n


def decode_bytes(Bt, Dn, N, es_io=2):
    rows = Bt * Dn
    return (2 * rows * N * 4                # state read + write
            + 3 * rows * es_io + rows * es_io  # x, dt, z in; out
            + 2 * Bt * N * 4 + Dn * N * 4 + 2 * Dn * 4)


def cpu_baseline(s, Bt, Dn, N, L, min_cpu_s=12.0, max_reps=8):
    """The fp64 oracle (as it stands) on the host cores, over the same step, repeated until about
    min_cpu_s seconds of CPU time (wall x threads) have been spent; the rate is over all reps."""
    import numpy as np
    import oracle
    threads = oracle.max_threads()
    reps, total = 0, 0.0
    while reps < max_reps and (reps == 0 or total * threads < min_cpu_s):
        t = time.perf_counter()
        _, last = oracle.selective_scan(s.u, s.delta, s.A, s.B, s.C, s.D, s.z, s.delta_bias)
        state = np.ascontiguousarray(last)
        oracle.selective_state_update(state, s.u[..., -1], s.delta[..., -1], s.A, s.B[..., -1],
                                      s.C[..., -1], D=s.D, z=s.z[..., -1], dt_bias=s.delta_bias)
        total += time.perf_counter() - t
        reps += 1
    nbytes = scan_bytes(Bt, Dn, N, L) + decode_bytes(Bt, Dn, N)
    return {"value": nbytes * reps / total / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{reps} full steps (all {Bt * Dn} rows x {L} steps of the scan + 1 decode token "
                      f"each), fp64, {total:.2f} s wall on {threads} threads",
            "cpu_model": cpu_model(), "single_thread_130m": single_thread_130m()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def single_thread_130m(rows=1536):
    """The oracle on one host thread over one batch row block (1536 of the 12288 rows) of the
    Mamba-130M fp32 workload (8 x 1536 x 16 x 2048): state updates per second."""
    import oracle
    from synth import CONFIGS, scan_inputs
    c = CONFIGS["mamba130m_fp32"]
    s = scan_inputs(1, c["d_inner"], c["d_state"], c["L"], dtype="f32", with_z=True, seed=0)
    t = time.perf_counter()
    oracle.selective_scan(s.u, s.delta, s.A, s.B, s.C, s.D, s.z, s.delta_bias, nthreads=1)
    wall = time.perf_counter() - t
    n = rows * c["L"] * c["d_state"]
    return {"state_updates_per_s": n / wall, "rows": rows, "L": c["L"], "wall_s": round(wall, 3)}


def decode_hbm_chain(mss, torch, devc, steps=1024, states=16, pool=64, N=None):
    """Chained one-token updates of `states` distinct (64, 5120, N) fp32 states in turn (one per
    layer of a model, as generation steps a whole stack); at N = 16, 16 x 21 MB = 336 MB, at
    N = 128, 4 x 168 MB: more than the 256 MB Infinity Cache, so every step reads and writes its
    state in HBM.  Timed as replays of a captured HIP graph of `pool` steps (inputs cycle through
    `pool` resident sets)."""
    import numpy as np
    from synth import CONFIGS, decode_inputs
    c = CONFIGS["decode_bf16"]
    Bt, Dn = c["batch"], c["d_inner"]
    N = N or c["d_state"]
    d = decode_inputs(Bt, Dn, N, pool, dtype="bf16", with_z=True, seed=0)
    up = lambda a, bf=False: (torch.from_numpy(np.ascontiguousarray(a)).to(devc).to(torch.bfloat16)
                              if bf else torch.from_numpy(np.ascontiguousarray(a)).to(devc))
    X, DT, Z = up(d.x, True), up(d.dt, True), up(d.z, True)
    Bs, Cs = up(d.B), up(d.C)
    A, D, bias = up(d.A), up(d.D), up(d.dt_bias)
    st = [torch.zeros((Bt, Dn, N), dtype=torch.float32, device=devc) for _ in range(states)]
    outs = torch.empty((pool, Bt, Dn), dtype=torch.bfloat16, device=devc)

    def run(k):
        j = k % pool
        mss.selective_state_update(st[k % states], X[j], DT[j], A, Bs[j], Cs[j], D=D, z=Z[j], dt_bias=bias,
                                   out=outs[j])

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for k in range(pool):
            run(k)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for k in range(pool):
            run(k)
    g.replay()
    torch.cuda.synchronize()
    ramp_clocks(torch, lambda k: g.replay(), batch=1)
    reps = max(1, steps // pool)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * pool)
    nbytes = decode_bytes(Bt, Dn, N)
    gbps = nbytes / (us * 1e-6) / 1e9
    # for comparison: torch's own in-place elementwise kernel (state *= 0.5) over the same states in
    # the same graph-chain shape, which reads and writes each step's state once and nothing else
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        for k in range(pool):
            st[k % states].mul_(0.5)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(gr):
        for k in range(pool):
            st[k % states].mul_(0.5)
    gr.replay()
    torch.cuda.synchronize()
    ramp_clocks(torch, lambda k: gr.replay(), batch=1)
    e0.record()
    for _ in range(reps):
        gr.replay()
    e1.record()
    torch.cuda.synchronize()
    rmw_us = e0.elapsed_time(e1) * 1e3 / (reps * pool)
    rmw_bytes = 2 * Bt * Dn * N * 4
    return {"shape": [Bt, Dn, N], "distinct_states": states, "state_bytes_total": states * Bt * Dn * N * 4,
            "steps": reps * pool, "graph_us_per_step": round(us, 3), "graph_gbps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "torch_inplace_scale_same_states": {"us_per_step": round(rmw_us, 3),
                                                "gbps": round(rmw_bytes / (rmw_us * 1e-6) / 1e9, 1)},
            "note": f"each step's state is one of {states} ({states * Bt * Dn * N * 4 / 1e6:.0f} MB in all, above "
                    "the 256 MB Infinity Cache): HBM-resident"}


def fwd_leg(mss, torch, devc, Bt, Dn, N, L, a_kind, calls=20, warmup=3, copies=2):
    """The forward on a layer shape with A of `a_kind` (synth: "s4d" is A = -(n+1), "random" an
    unstructured negative A, what a trained layer holds, so every state update takes its own
    exp).  Rotated input copies, events on the stream, and the library's kernel split."""
    import numpy as np
    from synth import scan_inputs
    s = scan_inputs(Bt, Dn, N, L, dtype="bf16", with_z=True, seed=0, a_kind=a_kind)
    up = lambda a, bf=False: (torch.from_numpy(np.ascontiguousarray(a)).to(devc).to(torch.bfloat16)
                              if bf else torch.from_numpy(np.ascontiguousarray(a)).to(devc))
    A, D, bias = up(s.A), up(s.D), up(s.delta_bias)
    sets = [dict(u=up(s.u, True), d=up(s.delta, True), z=up(s.z, True), B=up(s.B), C=up(s.C)) for _ in range(copies)]
    del s
    out = torch.empty_like(sets[0]["u"])
    last = torch.empty((Bt, Dn, N), dtype=torch.float32, device=devc)

    def call(k):
        p = sets[k % copies]
        mss.selective_scan_fwd(p["u"], p["d"], A, p["B"], p["C"], D=D, z=p["z"], delta_bias=bias, out=out,
                               last_state=last)

    ramp_clocks(torch, call)
    for k in range(warmup):
        call(k)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for k in range(calls):
        ev[k][0].record(stream)
        call(k)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    mss.profile_enable(True)  # the kernel split: a second pass with the timing hook on
    for k in range(calls):
        call(k)
    torch.cuda.synchronize()
    mss.profile_enable(False)
    n, carry, main = mss.profile_fwd()
    ms = [a.elapsed_time(b) for a, b in ev]
    avg = sum(ms) / len(ms)
    nb = scan_bytes(Bt, Dn, N, L)
    main_ms = main / max(n, 1)
    return {"shape": [Bt, Dn, N, L],
            "a": "A = -(n+1) (synth a_kind=s4d)" if a_kind == "s4d" else "random negative (synth a_kind=random)",
            "avg_ms": round(avg, 4), "min_ms": round(min(ms), 4),
            "state_updates_per_s": round(Bt * Dn * L * N / (avg * 1e-3), 1),
            "gbps": round(nb / (avg * 1e-3) / 1e9, 2),
            "frac_hbm_peak": round(nb / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "carry_stage_avg_ms": round(carry / max(n, 1), 4), "main_avg_ms": round(main_ms, 4),
            "main_frac_hbm_peak": round(nb / (main_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


def general_a_leg(mss, torch, devc, Bt, Dn, N, L):
    return fwd_leg(mss, torch, devc, Bt, Dn, N, L, "random")


def ssd_bytes(Bt, L, H, P, G, N):
    """Algorithmic bytes of one SSD layer call: x, z, out (bf16), dt (bf16), B, C (bf16), A, D,
    dt_bias (fp32) and the final state (fp32), each once."""
    return 3 * Bt * L * H * P * 2 + Bt * L * H * 2 + 2 * Bt * L * G * N * 2 + 3 * H * 4 + Bt * H * P * N * 4


def ssd_flops(Bt, L, H, P, N, Q=64):
    """Multiply-adds x 2 of the chunked form per (b, h, chunk of Q): C B^T and M X over the causal
    triangle (Q (Q + 1) / 2 pairs), C H^T and the state update X^T (w B) in full."""
    chunks = Bt * H * ((L + Q - 1) // Q)
    tri = Q * (Q + 1) // 2
    return chunks * 2 * (tri * N + tri * P + 2 * Q * N * P)


def ssd_leg(mss, torch, devc, calls=20, warmup=3, copies=2):
    """Mamba-2's SSD layer (mss_ssd_scan_fwd) at the 2.7B width (batch 4, L 2048, 80 heads of 64
    channels, one group) for d_state 64 and 128: rotated input copies, HIP events on the stream.
    The layer is HBM-bound in principle (about 60 flops per algorithmic byte against a bf16 ridge
    of 2.5 PFLOP/s / 8 TB/s = 312); the MFMA rate is reported beside the HBM fraction."""
    import numpy as np
    from synth import SSD_CONFIGS, ssd_inputs
    out_res = {}
    for name in ("ssd_2p7b_n64", "ssd_2p7b_n128"):
        c = SSD_CONFIGS[name]
        Bt, L, H, P, G, N = c["batch"], c["L"], c["heads"], c["headdim"], c["groups"], c["d_state"]
        s = ssd_inputs(Bt, L, H, P, G, N, seed=0)
        up = lambda a, bf=False: (torch.from_numpy(np.ascontiguousarray(a)).to(devc).to(torch.bfloat16)
                                  if bf else torch.from_numpy(np.ascontiguousarray(a)).to(devc))
        A, D, bias = up(s.A), up(s.D), up(s.dt_bias)
        sets = [dict(x=up(s.x, True), dt=up(s.dt, True), z=up(s.z, True), B=up(s.B, True), C=up(s.C, True))
                for _ in range(copies)]
        del s
        out = torch.empty_like(sets[0]["x"])
        last = torch.empty((Bt, H, P, N), dtype=torch.float32, device=devc)

        def call(k):
            p = sets[k % copies]
            mss.ssd_scan_fwd(p["x"], p["dt"], A, p["B"], p["C"], D=D, z=p["z"], dt_bias=bias, out=out,
                             last_state=last)

        ramp_clocks(torch, call)
        for k in range(warmup):
            call(k)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for k in range(calls):
            ev[k][0].record(stream)
            call(k)
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ev]
        avg = sum(ms) / len(ms)
        nb, fl = ssd_bytes(Bt, L, H, P, G, N), ssd_flops(Bt, L, H, P, N)
        gbps = nb / (avg * 1e-3) / 1e9
        out_res[name] = {"shape": {"batch": Bt, "seq_len": L, "heads": H, "headdim": P, "groups": G, "d_state": N},
                         "avg_ms": round(avg, 4), "min_ms": round(min(ms), 4), "algorithmic_bytes": nb,
                         "gbps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                         "algorithmic_flops": fl, "tflops": round(fl / (avg * 1e-3) / 1e12, 2),
                         "frac_bf16_mfma_peak": round(fl / (avg * 1e-3) / 2.5e15, 4)}
        del sets, out, last
        torch.cuda.empty_cache()
    return out_res


def decode_chain(mss, torch, devc, steps=1024, pool=64):
    """Chained one-token state updates at the decode workload's shape (64 x 5120 x 16, bf16
    x / dt / z / out, fp32 state): `steps` launches cycling through `pool` resident input sets,
    timed as plain stream launches (through the per-call wrapper, then through steps bound once
    to their buffers) and as replays of a captured HIP graph of `pool` steps."""
    import numpy as np
    from synth import CONFIGS, decode_inputs
    c = CONFIGS["decode_bf16"]
    Bt, Dn, N = c["batch"], c["d_inner"], c["d_state"]
    d = decode_inputs(Bt, Dn, N, pool, dtype="bf16", with_z=True, seed=0)
    up = lambda a, bf=False: (torch.from_numpy(np.ascontiguousarray(a)).to(devc).to(torch.bfloat16)
                              if bf else torch.from_numpy(np.ascontiguousarray(a)).to(devc))
    X, DT, Z = up(d.x, True), up(d.dt, True), up(d.z, True)
    Bs, Cs = up(d.B), up(d.C)
    A, D, bias = up(d.A), up(d.D), up(d.dt_bias)
    state = torch.zeros((Bt, Dn, N), dtype=torch.float32, device=devc)
    outs = torch.empty((pool, Bt, Dn), dtype=torch.bfloat16, device=devc)

    def run(k):
        j = k % pool
        mss.selective_state_update(state, X[j], DT[j], A, Bs[j], Cs[j], D=D, z=Z[j], dt_bias=bias,
                                   out=outs[j])

    for k in range(pool):
        run(k)
    torch.cuda.synchronize()
    ramp_clocks(torch, run, batch=64)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(steps):
        run(k)
    e1.record()
    torch.cuda.synchronize()
    stream_us = e0.elapsed_time(e1) * 1e3 / steps
    # the same chain through steps bound once to their buffers (no per-call descriptor packing)
    bound = [mss.StateUpdateStep(state, X[j], DT[j], A, Bs[j], Cs[j], D=D, z=Z[j], dt_bias=bias,
                                 out=outs[j]) for j in range(pool)]
    run_bound = lambda k: bound[k % pool]()
    ramp_clocks(torch, run_bound, batch=64)
    e0.record()
    for k in range(steps):
        run_bound(k)
    e1.record()
    torch.cuda.synchronize()
    bound_us = e0.elapsed_time(e1) * 1e3 / steps
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for k in range(pool):  # warm the side stream once outside the capture
            run(k)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for k in range(pool):
            run(k)
    g.replay()
    torch.cuda.synchronize()
    ramp_clocks(torch, lambda k: g.replay(), batch=1)
    reps = max(1, steps // pool)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / (reps * pool)
    nbytes = decode_bytes(Bt, Dn, N)
    return {"shape": [Bt, Dn, N], "steps": steps, "input_sets": pool,
            "stream_us_per_step": round(stream_us, 3), "bound_step_us_per_step": round(bound_us, 3),
            "graph_us_per_step": round(graph_us, 3),
            "graph_gbps": round(nbytes / (graph_us * 1e-6) / 1e9, 1),
            "note": "state (21 MB) stays resident in the 256 MB Infinity Cache across steps"}


def bwd_bytes(Bt, Dn, N, L, es_io=2):
    """Algorithmic bytes of one backward call: u, delta, z, dout read and du, ddelta, dz
    written once (dtype of u); B, C read and dB, dC written (fp32); A, D, bias read and dA, dD,
    dbias written."""
    io = Bt * Dn * L * es_io
    return 7 * io + 4 * Bt * N * L * 4 + 2 * (Dn * N * 4 + 2 * Dn * 4)


def backward_leg(mss, torch, sets, A, D, bias, Bt, Dn, N, L, fwd_ms, calls=10, warmup=2):
    """mss_selective_scan_bwd on the same workload (gradients of the forward for a random dout),
    timed with events on the stream it runs on; input sets rotated as in the forward steps."""
    gen = torch.Generator(device="cuda:0").manual_seed(1)
    douts = [torch.randn(p["u"].shape, generator=gen, device="cuda:0").to(torch.bfloat16) for p in sets]

    def call(k):
        p = sets[k % len(sets)]
        return mss.selective_scan_bwd(p["u"], p["delta"], A, p["B"], p["C"], douts[k % len(sets)],
                                      D=D, z=p["z"], delta_bias=bias)

    ramp_clocks(torch, call, batch=2)
    for k in range(warmup):
        call(k)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for k in range(calls):
        ev[k][0].record(stream)
        call(k)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    avg = sum(ms) / len(ms)
    nb = bwd_bytes(Bt, Dn, N, L)

    # forward + backward per training step: recomputing the states vs keeping them
    saved = torch.empty(((L + 7) // 8, N // 4, Bt * Dn * 4), dtype=torch.float32, device="cuda:0")
    out = torch.empty_like(sets[0]["u"])
    last = torch.empty((Bt, Dn, N), dtype=torch.float32, device="cuda:0")

    def pair(k, keep):
        p = sets[k % len(sets)]
        if keep:
            mss.selective_scan_fwd_save(p["u"], p["delta"], A, p["B"], p["C"], D=D, z=p["z"],
                                        delta_bias=bias, out=out, last_state=last, saved_states=saved)
        else:
            mss.selective_scan_fwd(p["u"], p["delta"], A, p["B"], p["C"], D=D, z=p["z"],
                                   delta_bias=bias, out=out, last_state=last)
        return mss.selective_scan_bwd(p["u"], p["delta"], A, p["B"], p["C"], douts[k % len(sets)], D=D,
                                      z=p["z"], delta_bias=bias, saved_states=saved if keep else None)

    pairs = {}
    for keep in (False, True):
        ramp_clocks(torch, lambda k: pair(k, keep), batch=2)
        for k in range(warmup):
            pair(k, keep)
        torch.cuda.synchronize()
        evp = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for k in range(calls):
            evp[k][0].record(stream)
            pair(k, keep)
            evp[k][1].record(stream)
        torch.cuda.synchronize()
        pairs[keep] = sum(a.elapsed_time(b) for a, b in evp) / calls
    return {"avg_ms": round(avg, 4), "min_ms": round(min(ms), 4), "calls": calls,
            "gbps": round(nb / (avg * 1e-3) / 1e9, 2), "algorithmic_bytes": nb,
            "ratio_to_fwd": round(avg / fwd_ms, 2),
            "outputs": "du, ddelta, dz (bf16); dA, dB, dC, dD, ddelta_bias (fp32)",
            "fwd_bwd_recompute_ms": round(pairs[False], 4), "fwd_bwd_saved_states_ms": round(pairs[True], 4),
            "saved_state_bytes": saved.numel() * 4}


def conv_leg(mss, torch, devc, Bt, Dn, L, K=4, calls=20, warmup=3, copies=3):
    """mss_causal_conv1d_fwd (K = 4, bias, silu, final state) on the same layer shape with bf16
    x / out: a streaming kernel, priced against HBM (x read once, out written once)."""
    gen = torch.Generator(device=devc).manual_seed(2)
    xs = [torch.randn((Bt, Dn, L), generator=gen, device=devc).to(torch.bfloat16) for _ in range(copies)]
    w = torch.randn((Dn, K), generator=gen, device=devc) * 0.5
    b = torch.randn((Dn,), generator=gen, device=devc)
    outs = [torch.empty_like(x) for x in xs]
    fin = torch.empty((Bt, Dn, K - 1), dtype=torch.bfloat16, device=devc)

    def call(k):
        mss.causal_conv1d_fwd(xs[k % copies], w, b, out=outs[k % copies], return_final_state=True,
                              final_state=fin)

    ramp_clocks(torch, call)
    for k in range(warmup):
        call(k)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for k in range(calls):
        ev[k][0].record(stream)
        call(k)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(c) for a, c in ev]
    avg = sum(ms) / len(ms)
    nb = 2 * Bt * Dn * L * 2 + Dn * K * 4 + Dn * 4 + Bt * Dn * (K - 1) * 2
    gbps = nb / (avg * 1e-3) / 1e9
    return {"avg_us": round(avg * 1e3, 2), "min_us": round(min(ms) * 1e3, 2), "calls": calls,
            "algorithmic_bytes": nb,
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4)}}


def configs_leg(mss, torch, devc, warmup=3):
    """The forward on the other scan workloads (fp32 u / delta / z / out): tiny (2 x 64 x 16 x 256),
    Mamba-130M (8 x 1536 x 16 x 2048) and long context (1 x 1536 x 16 x 131072, no gate), each
    from the seeded generators, with last_state, timed with events on the stream it runs on."""
    import numpy as np
    from synth import CONFIGS, scan_inputs
    out = {}
    for name, calls in (("tiny_fp32", 50), ("mamba130m_fp32", 20), ("long_fp32", 10)):
        c = CONFIGS[name]
        Bt, Dn, N, L = c["batch"], c["d_inner"], c["d_state"], c["L"]
        s = scan_inputs(Bt, Dn, N, L, dtype="f32", with_z=c["with_z"], seed=0)
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(devc)
        u, dl, z, B, C = t(s.u), t(s.delta), t(s.z), t(s.B), t(s.C)
        A, D, bias = t(s.A), t(s.D), t(s.delta_bias)
        del s
        o = torch.empty_like(u)
        last = torch.empty((Bt, Dn, N), dtype=torch.float32, device=devc)

        def call():
            mss.selective_scan_fwd(u, dl, A, B, C, D=D, z=z, delta_bias=bias, out=o, last_state=last)

        ramp_clocks(torch, lambda k: call())
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for k in range(calls):
            ev[k][0].record(stream)
            call()
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ev]
        avg = sum(ms) / len(ms)
        nb = scan_bytes(Bt, Dn, N, L, es_io=4, with_z=c["with_z"])
        out[name] = {"shape": [Bt, Dn, N, L], "gate": bool(c["with_z"]), "avg_ms": round(avg, 4),
                     "min_ms": round(min(ms), 4), "calls": calls, "gbps": round(nb / (avg * 1e-3) / 1e9, 2),
                     "frac_hbm_peak": round(nb / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "state_updates_per_s": Bt * Dn * L * N / (avg * 1e-3)}
        del u, dl, z, B, C, A, D, bias, o, last
        torch.cuda.empty_cache()
    return out


def shard_leg(mss, torch, devc, s, Bt, Dn, N, L, calls=20, warmup=3):
    """The forward at the per-GPU shapes of two ways to spread the layer over GPUs without any
    exchange (rows are independent; B / C are replicated): channel split over 8 GPUs
    (d_inner / 8 rows each) and batch split over 4 (one sequence each).  One GPU runs one
    shard; the shapes have 8x / 4x fewer rows, so the segment plan has to fill the chip with
    longer splits of L."""
    import numpy as np
    out = {}
    for name, (b0, b1, d0, d1) in {"channel_split_8": (0, Bt, 0, Dn // 8),
                                   "batch_split_4": (0, Bt // 4, 0, Dn)}.items():
        sb, sd = slice(b0, b1), slice(d0, d1)

        def t(a, bf16=False):
            x = torch.from_numpy(np.ascontiguousarray(a)).to(devc)
            return x.to(torch.bfloat16) if bf16 else x
        u, dl, z = t(s.u[sb, sd], True), t(s.delta[sb, sd], True), t(s.z[sb, sd], True)
        B, C = t(s.B[sb]), t(s.C[sb])
        A, D, bias = t(s.A[sd]), t(s.D[sd]), t(s.delta_bias[sd])
        o = torch.empty_like(u)
        last = torch.empty((b1 - b0, d1 - d0, N), dtype=torch.float32, device=devc)
        ramp_clocks(torch, lambda k: mss.selective_scan_fwd(u, dl, A, B, C, D=D, z=z, delta_bias=bias, out=o,
                                                              last_state=last))
        for _ in range(warmup):
            mss.selective_scan_fwd(u, dl, A, B, C, D=D, z=z, delta_bias=bias, out=o, last_state=last)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        for k in range(calls):
            ev[k][0].record(stream)
            mss.selective_scan_fwd(u, dl, A, B, C, D=D, z=z, delta_bias=bias, out=o, last_state=last)
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(c) for a, c in ev]
        avg = sum(ms) / len(ms)
        nb = scan_bytes(b1 - b0, d1 - d0, N, L)
        out[name] = {"shape": [b1 - b0, d1 - d0, N, L], "avg_ms": round(avg, 4),
                     "min_ms": round(min(ms), 4), "gbps": round(nb / (avg * 1e-3) / 1e9, 2)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=3, help="input sets rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-chain", action="store_true")
    ap.add_argument("--no-dstate", action="store_true", help="skip the d_state 64 / 128 forward legs")
    ap.add_argument("--no-general-a", action="store_true", help="skip the random-A forward leg")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--no-shard", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the tiny / 130M / long-context fp32 forward")
    ap.add_argument("--no-ssd", action="store_true", help="skip the Mamba-2 SSD layer leg")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library runs the scan on a single MI355X "
              "(no multi-GPU path); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import selective_state_space_06_amd as mss
    from synth import CONFIGS, scan_inputs

    c = CONFIGS[WORKLOAD]
    Bt, Dn, N, L = c["batch"], c["d_inner"], c["d_state"], c["L"]
    mss.load_library()
    s = scan_inputs(Bt, Dn, N, L, dtype="bf16", with_z=True, seed=0)
    devc = torch.device("cuda:0")
    torch.cuda.set_device(devc)

    def up(a, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(a)).to(devc)
        return t.to(torch.bfloat16) if bf16 else t

    A, D, bias = up(s.A), up(s.D), up(s.delta_bias)
    sets = []
    for _ in range(max(1, args.copies)):
        sets.append(dict(u=up(s.u, True), delta=up(s.delta, True), z=up(s.z, True),
                         B=up(s.B), C=up(s.C),
                         out=torch.empty((Bt, Dn, L), dtype=torch.bfloat16, device=devc),
                         last=torch.empty((Bt, Dn, N), dtype=torch.float32, device=devc),
                         x1=up(s.u[..., -1], True), dt1=up(s.delta[..., -1], True),
                         z1=up(s.z[..., -1], True), B1=up(np.ascontiguousarray(s.B[..., -1])),
                         C1=up(np.ascontiguousarray(s.C[..., -1])),
                         out1=torch.empty((Bt, Dn), dtype=torch.bfloat16, device=devc)))
    stream = torch.cuda.current_stream(devc)

    def step(k, ev=None):
        p = sets[k % len(sets)]
        if ev is not None:
            ev[0].record(stream)
        mss.selective_scan_fwd(p["u"], p["delta"], A, p["B"], p["C"], D=D, z=p["z"],
                               delta_bias=bias, out=p["out"], last_state=p["last"])
        if ev is not None:
            ev[1].record(stream)
        mss.selective_state_update(p["last"], p["x1"], p["dt1"], A, p["B1"], p["C1"], D=D,
                                   z=p["z1"], dt_bias=bias, out=p["out1"])
        if ev is not None:
            ev[2].record(stream)

    ramp_calls = ramp_clocks(torch, step)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k, evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # The kernel split comes from a second pass of the same steps with the library's timing hook
    # on: its events between the two kernels cost ~11 us per call (239 against 227 us for the
    # forward on this layer), so the timed steps above run without it.
    mss.profile_enable(True)
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    mss.profile_enable(False)
    n_calls, carry_ms_tot, main_ms_tot = mss.profile_fwd()

    scan_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_per_step = wall * 1e3 / args.steps
    sb, db = scan_bytes(Bt, Dn, N, L), decode_bytes(Bt, Dn, N)
    value = (sb + db) * args.steps / wall / 1e9
    scan_avg_ms = float(np.mean(scan_ms))
    scan_gbps = sb / (scan_avg_ms * 1e-3) / 1e9
    updates = Bt * Dn * L * N + Bt * Dn * N
    main_ms = main_ms_tot / max(n_calls, 1)
    carry_ms = carry_ms_tot / max(n_calls, 1)
    achieved = sb / (main_ms * 1e-3) / 1e9
    counted = MAIN_COUNTERS["src_sha256"] == kernel_source_digest()
    traffic = (MAIN_COUNTERS["fetch_bytes"] + MAIN_COUNTERS["write_bytes"]) if counted else None
    valu = None
    if counted:
        per = MAIN_COUNTERS["valu_per_bdt"]
        need_s = per * Bt * Dn * L / 64 / VALU_WAVE_INSTR_PER_S
        valu = {"instr_per_bdt": per, "issue_time_ms_at_peak": round(need_s * 1e3, 4),
                "issue_frac": round(need_s / (main_ms * 1e-3), 4),
                "peak": "1 wave64 fp32 VALU instruction per 4 cycles per SIMD, 1024 SIMDs, 2.4 GHz"}

    res = {
        "metric": "selective-scan fwd GB/s + state-updates/s (B*D*L*N/s), % of MI355X HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp": {"seconds": RAMP_S, "steps": ramp_calls,
                       "note": "untimed steps before the warm-up steps, until the GPU's clocks are up"},
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage": "bf16 u/delta/z/out; f32 A/B/C/D/delta_bias/state",
        "data": "synthetic (seeded: N(0,1) u/delta/z/B/C, S4D-real A=-(n+1), D=1, "
                "dt bias = inv_softplus(logU[1e-3,1e-1]))",
        "config": {"workload": f"{WORKLOAD}: selective scan fwd (prefill) + 1 decode token",
                   "batch": Bt, "d_inner": Dn, "d_state": N, "seq_len": L,
                   "input_copies_rotated": len(sets)},
        "state_updates_per_s": round(updates * args.steps / wall, 1),
        "scan_fwd": {"avg_ms": round(scan_avg_ms, 4), "min_ms": round(float(np.min(scan_ms)), 4),
                     "gbps": round(scan_gbps, 2), "frac_hbm_peak": round(scan_gbps / HBM_PEAK_GBPS, 4),
                     "state_updates_per_s": round(Bt * Dn * L * N / (scan_avg_ms * 1e-3), 1)},
        "decode_token": {"avg_us": round(float(np.mean(dec_ms)) * 1e3, 2)},
        "kernels": {"calls_timed": n_calls, "carry_stage_avg_ms": round(carry_ms, 4),
                    "main_avg_ms": round(main_ms, 4),
                    "carry_share_of_call": round(carry_ms / scan_avg_ms, 4),
                    "note": "a separate pass of the same steps with the library's timing hook on "
                            "(its events between the kernels are left out of the timed steps)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "scan_main_kernel (the main kernel of mss_selective_scan_fwd), "
                               "timed by the library's HIP events on its stream",
                     "algorithmic_bytes": sb,
                     "call_achieved": round(scan_gbps, 1), "call_frac": round(scan_gbps / HBM_PEAK_GBPS, 4)},
        "valu": valu,
    }
    progress("headline steps")
    if not args.no_bwd:
        res["scan_bwd"] = backward_leg(mss, torch, sets, A, D, bias, Bt, Dn, N, L, scan_avg_ms)
        progress("backward")
    if not args.no_conv:
        res["conv1d"] = conv_leg(mss, torch, devc, Bt, Dn, L)
        progress("conv1d")
    if not args.no_shard:
        res["shard_fwd"] = shard_leg(mss, torch, devc, s, Bt, Dn, N, L)
        progress("shard shapes")
    if not args.no_general_a:
        res["scan_fwd_general_A"] = general_a_leg(mss, torch, devc, Bt, Dn, N, L)
        progress("general A")
    if not args.no_dstate:
        # the same layer at d_state 64 and 128 (the general kernels: d_state / 16 lanes per channel)
        res["scan_fwd_dstate"] = {f"{n}_{k}": fwd_leg(mss, torch, devc, Bt, Dn, n, L, k, calls=10, copies=2)
                                  for n in (64, 128) for k in ("s4d", "random")}
        progress("d_state 64 / 128 forward")
    if not args.no_decode_chain:
        res["decode_chain"] = decode_chain(mss, torch, devc)
        res["decode_chain_hbm"] = decode_hbm_chain(mss, torch, devc)
        res["decode_chain_hbm_n128"] = decode_hbm_chain(mss, torch, devc, states=4, N=128)
        progress("decode chains")
    if not args.no_configs:
        res["other_configs"] = configs_leg(mss, torch, devc)
        progress("fp32 workloads")
    if not args.no_ssd:
        res["ssd_scan"] = ssd_leg(mss, torch, devc)
        progress("ssd")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(s, Bt, Dn, N, L)
        progress("cpu baseline")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
