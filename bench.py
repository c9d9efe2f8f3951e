#!/usr/bin/env python3
"""Benchmark of the causal chunkwise linear attention (Lightning Attention) hot path.

Forward pass (the headline): one step = la_forward_states + la_forward_outputs
(exactly la_forward_ex) over the 1,048,576-token grouped-query workload
(B=1, 128 query heads over 32 KV heads, d = dv = 128, bf16 inputs and output,
float32 state, 64-token blocks), seeded synthetic inputs resident in HBM.
Reported: tokens/s, TFLOP/s against the bf16 dense matrix-core peak, and the
HBM roofline of the dominant kernel (the output kernel), timed with HIP
events on the stream it runs on.

Backward (secondary): la_backward (dQ, dK, dV and the initial-state gradient)
on the same workload with a seeded N(0,1) upstream gradient, timed with HIP
events per call; reported as tokens/s and algorithmic HBM GB/s.

Forward variants (secondary): la_forward_variant with the ReLU feature map,
causal normalised and non-causal, on the same workload.

Decode (secondary): 256 sequences x 32 KV heads of float32 128x128 state
(512 MiB) initialised by the forward kernel over a seeded 8192-token prefix,
then single-token steps; reported as HBM GB/s.

CPU baseline: the fp64 oracle (test infrastructure) timed on a bounded sample
of the same forward workload on this host.

Prints ONE JSON line.  Single GPU only.
"""
import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Lightning-attn fwd tokens/s + % bf16 MFMA peak at N=1M; decode HBM GB/s"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak, TFLOP/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_gqa_1m_decode_256.md")


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel's source has changed since the counters were taken."""
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    for m in re.finditer(r"traffic (\S+) (\S+) bytes=(\d+) source=(\S+) sha256=([0-9a-f]+)", text):
        if (m.group(1), m.group(2)) != (kernel, workload):
            continue
        # source: the kernel's file and the headers it includes, joined by '+'.
        try:
            texts = [open(os.path.join(ROOT, "long_context_attention_chunkwise_amd", "csrc", name)).read()
                     for name in m.group(4).split("+")]
        except OSError:
            return None
        return int(m.group(3)) if code_digest(texts) == m.group(5) else None
    return None


def code_digest(texts):
    """SHA-256 of C++/HIP sources with comments removed, whitespace runs
    inside a line collapsed to one space and blank lines dropped (string and
    character literals kept as written), so that an edit to comments,
    indentation or blank lines leaves it unchanged and any edit to the code
    changes it.  The texts are taken in order."""
    import hashlib
    import re
    token = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)
    lines = []
    for text in texts:
        code = token.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), text)
        lines.extend(" ".join(line.split()) for line in code.splitlines())
    return hashlib.sha256("\n".join(line for line in lines if line).encode()).hexdigest()


def forward_flops(w, N):
    """Algorithmic flops of the causal forward (per the block recurrence).

    Per token and query head: in-block scores d(C+1) and their product with V
    dv(C+1) (lower triangle incl. diagonal, 2 flops per multiply-add), the
    inter-block product 2 d dv, and the state update 2 d dv shared by the
    Hq/Hkv query heads of a KV head.  The dense-tile count (what the matrix
    cores execute) replaces C+1 by 2C.
    """
    C, d, dv, G = w.block, w.d, w.dv, w.Hq // w.Hkv
    per_alg = (d + dv) * (C + 1) + 2 * d * dv + 2 * d * dv / G
    per_tile = (d + dv) * 2 * C + 2 * d * dv + 2 * d * dv / G
    n = w.B * w.Hq * N
    return per_alg * n, per_tile * n


def forward_bytes(w, N, out_bytes=2):
    """Algorithmic HBM bytes of one forward pass: read q, k, v once, write o once."""
    e = 2  # bf16
    return w.B * N * (w.Hq * w.d * e + w.Hkv * (w.d + w.dv) * e + w.Hq * w.dv * out_bytes)


def host_cores():
    """Cores this process may run on (its affinity mask)."""
    return len(os.sched_getaffinity(0))


def blas_limit(threads):
    """Context pinning the BLAS thread pools to `threads` (threadpoolctl), and
    a function returning the thread count the pools report inside it."""
    from threadpoolctl import threadpool_info, threadpool_limits
    lim = threadpool_limits(limits=threads)

    def used():
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return lim, used


def cpu_baseline(q, k, v, w, groups=1):
    """Time the fp64 oracle on the first `groups` KV groups (each with its G
    query heads, all tokens), one group at a time, with the BLAS pools pinned
    to this process's affinity mask: about 13 s per group at 1M tokens."""
    import numpy as np
    import oracle
    cores = host_cores()
    lim, used = blas_limit(cores)
    G = w.Hq // w.Hkv
    N = q.shape[2]
    groups = min(groups, w.Hkv)
    dt = 0.0
    with lim:
        threads = used()
        for g in range(groups):
            qs = q[:, g * G:(g + 1) * G].float().cpu().numpy().astype(np.float64)
            ks = k[:, g:g + 1].float().cpu().numpy().astype(np.float64)
            vs = v[:, g:g + 1].float().cpu().numpy().astype(np.float64)
            t0 = time.perf_counter()
            oracle.chunkwise(qs, ks, vs, w.block)
            dt += time.perf_counter() - t0
            del qs, ks, vs
    # The sample is groups/Hkv of the work per token of the full workload.
    return {"value": N * groups / dt / w.Hkv, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "affinity_cores": cores,
            "sample": f"fp64 chunkwise oracle on KV heads 0-{groups - 1} (query heads 0-{groups * G - 1}), "
                      f"all {N} tokens, {dt:.2f} s; value scaled to the full {w.Hkv}-KV-head workload "
                      f"(x{groups}/{w.Hkv})"}


def cpu_small_baselines(synth, torch):
    """The fp64 oracle over the two small workloads in full (the 256-token
    float32 one and the 4096-token 8/8-head one), on all cores of the affinity
    mask and on one thread: tokens/s (B * N / time), best of three runs."""
    import numpy as np
    import oracle
    out = {}
    cores = host_cores()
    for name in ("tiny_f32", "mha_4k"):
        w = synth.WORKLOADS[name]
        q, k, v = (x.double().numpy() for x in synth.make_qkv(w, "cpu", seed=0))
        rec = {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d}
        for label, threads in (("all_cores", cores), ("one_thread", 1)):
            lim, used = blas_limit(threads)
            with lim:
                n_used = used()
                best = float("inf")
                for _ in range(3):
                    t0 = time.perf_counter()
                    oracle.chunkwise(q, k, v, w.block)
                    best = min(best, time.perf_counter() - t0)
            rec[label] = {"tokens_per_s": round(w.B * w.N / best, 1), "seconds": round(best, 5), "threads": n_used}
        out[name] = rec
        del q, k, v
    return out


def bench_forward(la, synth, torch, w, steps, warmup, scrub_bytes=0):
    import ctypes
    lib = la.load_library()
    dev = torch.device("cuda:0")
    log(f"[bench] generating {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} dv={w.dv}")
    q, k, v = synth.make_qkv(w, dev, seed=0)
    o = torch.empty((w.B, w.Hq, w.N, w.dv), dtype=torch.bfloat16, device=dev)
    ws_bytes = la.workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d, w.dv, w.block, torch.bfloat16)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p
    args_states = (P(k.data_ptr()), P(v.data_ptr()), w.B, w.Hq, w.Hkv, w.N, w.d, w.dv, w.block, la.LA_BF16,
                   None, P(ws.data_ptr()), ws_bytes, sp)
    args_out = (P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()), w.B, w.Hq, w.Hkv, w.N, w.d,
                w.dv, w.block, la.LA_BF16, la.LA_BF16, None, None, P(ws.data_ptr()), ws_bytes, sp)

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        st = lib.la_forward_states(*args_states)
        if evs:
            evs[1].record(stream)
        st2 = lib.la_forward_outputs(*args_out)
        if evs:
            evs[2].record(stream)
        if st or st2:
            raise RuntimeError(f"forward failed: {la.status_str(st or st2)}")

    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / steps
    t_states = [e[0].elapsed_time(e[1]) for e in evs]
    t_main = [e[1].elapsed_time(e[2]) for e in evs]
    t_step = [e[0].elapsed_time(e[2]) for e in evs]
    finite = bool(torch.isfinite(o).all().item())
    if not finite:
        raise RuntimeError("non-finite forward output")
    events = {"median": round(statistics.median(t_step), 4), "min": round(min(t_step), 4),
              "mean": round(statistics.mean(t_step), 4),
              "cache": "warm: steps back to back, inputs may stay in the L2 / Infinity Cache if they fit"}
    if scrub_bytes > 0:
        # the same steps with scrub_bytes of device memory written between
        # them (evicting the inputs from the 4 MB L2s and the 256 MB
        # Infinity Cache), each step timed alone with events
        scrub = torch.empty(scrub_bytes // 4, dtype=torch.int32, device=dev)
        sevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(steps):
            scrub.fill_(i)
            step(sevs[i])
        torch.cuda.synchronize()
        t_scr = [e[0].elapsed_time(e[2]) for e in sevs]
        t_scr_main = [e[1].elapsed_time(e[2]) for e in sevs]
        events["scrubbed"] = {"scrub_bytes": scrub_bytes, "median": round(statistics.median(t_scr), 4),
                              "min": round(min(t_scr), 4), "mean": round(statistics.mean(t_scr), 4),
                              "outputs_mean": round(statistics.mean(t_scr_main), 4)}
        del scrub
        events["graph"] = graph_steps(lib, torch, stream, args_states, args_out, steps)
    return q, k, v, ms_step, statistics.mean(t_states), statistics.mean(t_main), ws_bytes, events


def graph_steps(lib, torch, stream, args_states, args_out, reps, per_graph=10):
    """Steps of a small workload as a caller that captures them in a HIP graph
    runs them: `per_graph` steps (both calls each) captured once, the graph
    replayed `reps` times back to back (cache-warm), per-step time from
    events around each replay.  Without the per-launch gaps this is what the
    kernels themselves take."""
    import ctypes

    def launch(sp):
        for _ in range(per_graph):
            st = lib.la_forward_states(*args_states[:-1], sp)
            st2 = lib.la_forward_outputs(*args_out[:-1], sp)
            if st or st2:
                raise RuntimeError("forward failed under graph capture")
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        launch(ctypes.c_void_p(side.cuda_stream))  # warm-up on the capture stream
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    g.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) / per_graph for a, b in evs]
    del g
    return {"steps_per_graph": per_graph, "replays": reps, "median": round(statistics.median(per), 4),
            "min": round(min(per), 4), "cache": "warm"}


def backward_flops(w, N):
    """Algorithmic flops of the backward pass (per the block recurrences).

    Per token and query head: dQ is a forward pass over (dO, V, K); dK and dV
    take two masked score products (Q K^T, dO V^T) and their two products
    with dO and Q, (d + dv)(C + 1) each pair, the reverse-state update 2 d dv,
    and the two inter products 4 d dv shared by the Hq/Hkv query heads.
    """
    C, d, dv, G = w.block, w.d, w.dv, w.Hq // w.Hkv
    per = 3 * (d + dv) * (C + 1) + 4 * d * dv + 6 * d * dv / G
    return per * w.B * w.Hq * N


def backward_bytes(w, N, grad_bytes=2):
    """Algorithmic HBM bytes of one backward pass: read q, k, v, dO once,
    write dq, dk, dv once."""
    e = 2
    reads = w.B * N * (w.Hq * w.d + w.Hkv * (w.d + w.dv) + w.Hq * w.dv) * e
    writes = w.B * N * (w.Hq * w.d + w.Hkv * (w.d + w.dv)) * grad_bytes
    return reads + writes


def bench_backward(la, synth, torch, w, q, k, v, steps, warmup):
    import ctypes
    lib = la.load_library()
    dev = torch.device("cuda:0")
    log(f"[bench] backward: upstream gradient for {w.name}")
    do = synth.make_grad((w.B, w.Hq, w.N, w.dv), dev, seed=1)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ds = torch.empty((w.B, w.Hkv, w.d, w.dv), dtype=torch.float32, device=dev)
    ws_bytes = la.backward_workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d, w.dv, w.block, torch.bfloat16)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    P = ctypes.c_void_p
    args = (P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(do.data_ptr()), P(dq.data_ptr()),
            P(dk.data_ptr()), P(dv.data_ptr()), w.B, w.Hq, w.Hkv, w.N, w.d, w.dv, w.block, la.LA_BF16, la.LA_BF16,
            None, None, P(ds.data_ptr()), P(ws.data_ptr()), ws_bytes, P(stream.cuda_stream))
    for _ in range(warmup):
        st = lib.la_backward(*args)
        if st:
            raise RuntimeError(f"backward failed: {la.status_str(st)}")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record(stream)
        st = lib.la_backward(*args)
        evs[i][1].record(stream)
        if st:
            raise RuntimeError(f"backward failed: {la.status_str(st)}")
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    if not all(bool(torch.isfinite(x).all().item()) for x in (dq, dk, dv, ds)):
        raise RuntimeError("non-finite gradient")
    per = [a.elapsed_time(b) for a, b in evs]
    ms = statistics.mean(per)
    nbytes = backward_bytes(w, w.N)
    flops = backward_flops(w, w.N)
    del dq, dk, dv, ws
    # the initial-state gradient alone (la_backward_state): q and dO read once
    sws_bytes = int(lib.la_backward_state_workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d, w.dv, la.LA_BF16))
    sws = torch.empty(max(sws_bytes, 16), dtype=torch.uint8, device=dev)
    sargs = (P(q.data_ptr()), P(do.data_ptr()), w.B, w.Hq, w.Hkv, w.N, w.d, w.dv, la.LA_BF16, None,
             P(ds.data_ptr()), P(sws.data_ptr()), sws_bytes, P(stream.cuda_stream))
    sev = []
    for i in range(1 + steps):
        e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        e[0].record(stream)
        st = lib.la_backward_state(*sargs)
        e[1].record(stream)
        if st:
            raise RuntimeError(f"backward state failed: {la.status_str(st)}")
        if i:
            sev.append(e)
    torch.cuda.synchronize()
    sms = statistics.mean(a.elapsed_time(b) for a, b in sev)
    sbytes = w.B * w.Hq * w.N * (w.d + w.dv) * 2
    state_only = {"ms_per_call": round(sms, 4), "bytes_alg": sbytes,
                  "hbm_gb_per_s": round(sbytes / (sms * 1e-3) / 1e9, 1),
                  "hbm_frac": round(sbytes / (sms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                  "what": "la_backward_state: grad_s_in alone (q and dO read once)"}
    del do, ds, sws
    return {"steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4), "ms_per_step_wall": round(wall, 4),
            "state_only": state_only,
            "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1),
            "config": {"workload": w.name, "grad_dtype": "bf16", "s_in": False, "grad_s_out": False},
            "hbm": {"bytes_alg": nbytes, "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "mfma": {"flops_alg": flops, "tflops_alg": round(flops / (ms * 1e-3) / 1e12, 2),
                     "frac_alg": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "workspace_bytes": ws_bytes}


def bench_state(la, torch, w, k, v, steps, warmup):
    """la_forward_state (the final state without outputs) on the workload's
    k, v: per-call events; algorithmic bytes = k and v read once (the state
    written is negligible)."""
    import ctypes
    lib = la.load_library()
    dev = torch.device("cuda:0")
    ws_bytes = int(lib.la_forward_state_workspace_bytes(w.B, w.Hkv, w.N, w.d, w.dv, la.LA_BF16))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    S = torch.empty((w.B, w.Hkv, w.d, w.dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    P = ctypes.c_void_p
    args = (P(k.data_ptr()), P(v.data_ptr()), w.B, w.Hkv, w.N, w.d, w.dv, la.LA_BF16, None, P(S.data_ptr()),
            P(ws.data_ptr()), ws_bytes, P(stream.cuda_stream))
    evs = []
    for i in range(warmup + steps):
        e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        e[0].record(stream)
        st = lib.la_forward_state(*args)
        e[1].record(stream)
        if st:
            raise RuntimeError(f"state-only pass failed: {la.status_str(st)}")
        if i >= warmup:
            evs.append(e)
    torch.cuda.synchronize()
    ms = statistics.mean(a.elapsed_time(b) for a, b in evs)
    nbytes = w.B * w.Hkv * w.N * (w.d + w.dv) * 2
    del ws, S
    return {"steps": steps, "warmup": warmup, "ms_per_call": round(ms, 4),
            "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1), "bytes_alg": nbytes,
            "hbm_gb_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "workspace_bytes": ws_bytes}


def bench_in_place(la, torch, w, q, k, v, steps, warmup):
    """The forward step with the output written over q (o = q, allowed when
    each query row is read before the same output row is written: groups of
    four query heads on the matrix cores).  Overwrites q, so it runs after
    everything that reads q; the timing does not depend on the values."""
    import ctypes
    lib = la.load_library()
    dev = torch.device("cuda:0")
    ws_bytes = la.workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d, w.dv, w.block, torch.bfloat16)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p
    args_states = (P(k.data_ptr()), P(v.data_ptr()), w.B, w.Hq, w.Hkv, w.N, w.d, w.dv, w.block, la.LA_BF16,
                   None, P(ws.data_ptr()), ws_bytes, sp)
    args_out = (P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(q.data_ptr()), w.B, w.Hq, w.Hkv, w.N, w.d,
                w.dv, w.block, la.LA_BF16, la.LA_BF16, None, None, P(ws.data_ptr()), ws_bytes, sp)
    evs = []
    for i in range(warmup + steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        st = lib.la_forward_states(*args_states)
        e[1].record(stream)
        st2 = lib.la_forward_outputs(*args_out)
        e[2].record(stream)
        if st or st2:
            raise RuntimeError(f"in-place forward failed: {la.status_str(st or st2)}")
        if i >= warmup:
            evs.append(e)
    torch.cuda.synchronize()
    t_step = [e[0].elapsed_time(e[2]) for e in evs]
    t_out = [e[1].elapsed_time(e[2]) for e in evs]
    nbytes = forward_bytes(w, w.N)
    ms_out = statistics.mean(t_out)
    del ws
    return {"steps": steps, "warmup": warmup, "ms_per_step": round(statistics.mean(t_step), 4),
            "outputs_ms": round(ms_out, 4), "tokens_per_s": round(w.B * w.N / (statistics.mean(t_step) * 1e-3), 1),
            "outputs_hbm_frac": round(nbytes / (ms_out * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "note": "o written over q (separate timing; the headline uses a separate o buffer)"}


VARIANTS = (
    # name, causal, feature map, normalize, eps
    ("relu_normalised_causal", True, "relu", True, 1e-6),
    ("relu_noncausal", False, "relu", False, 0.0),
)


def bench_variants(la, torch, w, q, k, v, steps, warmup):
    """la_forward_variant on the forward workload: per-call HIP-event time and
    the algorithmic HBM rate (q, k, v read once, o written once)."""
    import ctypes
    lib = la.load_library()
    dev = torch.device("cuda:0")
    o = torch.empty((w.B, w.Hq, w.N, w.dv), dtype=torch.bfloat16, device=dev)
    S = torch.empty((w.B, w.Hkv, w.d, w.dv), dtype=torch.float32, device=dev)
    Z = torch.empty((w.B, w.Hkv, w.d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    P = ctypes.c_void_p
    nbytes = forward_bytes(w, w.N)
    out = {}
    for name, causal, fmap, norm, eps in VARIANTS:
        ws_bytes = lib.la_forward_variant_workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d, w.dv, w.block, la.LA_BF16,
                                                          int(causal), int(norm))
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        args = (P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(o.data_ptr()), w.B, w.Hq, w.Hkv, w.N, w.d,
                w.dv, w.block, la.LA_BF16, la.LA_BF16, int(causal), 1 if fmap == "relu" else 0, int(norm),
                float(eps), None, P(S.data_ptr()), None, P(Z.data_ptr()) if norm else None, P(ws.data_ptr()),
                ws_bytes, P(stream.cuda_stream))
        for _ in range(warmup):
            st = lib.la_forward_variant(*args)
            if st:
                raise RuntimeError(f"variant {name} failed: {la.status_str(st)}")
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for a, b in evs:
            a.record(stream)
            lib.la_forward_variant(*args)
            b.record(stream)
        torch.cuda.synchronize()
        if not bool(torch.isfinite(o).all().item()):
            raise RuntimeError(f"non-finite output in variant {name}")
        ms = statistics.mean(a.elapsed_time(b) for a, b in evs)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"causal": causal, "feature_map": fmap, "normalize": norm, "eps": eps,
                     "ms_per_call": round(ms, 4), "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1),
                     "hbm_gb_per_s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                     "bytes_alg": nbytes}
        del ws
    del o, S, Z
    return {"steps": steps, "warmup": warmup, "workload": w.name, "variants": out}


STREAM_MODES = {0: "read", 1: "copy", 2: "read_write_3_2", 3: "in_place_update"}


def stream_ceilings(torch, gib=4, reps=5):
    """Practical HBM ceilings on this GPU: the best rate of the library's
    streaming kernels (libla_stream.so) over a few launch shapes, per access
    mix: read only, copy (read + write 1:1) and read + write 3:2 (the byte mix
    of the forward output kernel) and an in-place update (the decode step's
    pattern).  Each launch moves whole 64 KiB (60 KiB) steps of `gib` GiB
    buffers; best event time of `reps` launches."""
    import ctypes
    from long_context_attention_chunkwise_amd import build as _build
    lib = ctypes.CDLL(_build.STREAM_LIB_PATH)
    lib.la_stream_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.la_stream_bytes_moved.argtypes = [ctypes.c_int, ctypes.c_size_t]
    lib.la_stream_bytes_moved.restype = ctypes.c_size_t
    n = gib << 30
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty(n // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.empty(8192 * 256, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    out = {}
    for mode, name in STREAM_MODES.items():
        best = None
        for nt in (0, 1):
            for grid in (256, 1024, 8192):
                args = (mode, nt, ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n,
                        ctypes.c_void_p(sink.data_ptr()), grid, sp)
                if lib.la_stream_run(*args) != 0:
                    raise RuntimeError("stream kernel launch failed")
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(reps)]
                for e0, e1 in evs:
                    e0.record(stream)
                    lib.la_stream_run(*args)
                    e1.record(stream)
                torch.cuda.synchronize()
                ms = min(e0.elapsed_time(e1) for e0, e1 in evs)
                gbs = lib.la_stream_bytes_moved(mode, n) / (ms * 1e-3) / 1e9
                if best is None or gbs > best["gb_per_s"]:
                    best = {"gb_per_s": round(gbs, 1), "nontemporal": bool(nt), "workgroups": grid}
        out[name] = best
    del src, dst, sink
    torch.cuda.empty_cache()
    return out


def cpu_decode_baseline(S, qs, ks, vs, nseq=4, nsteps=10):
    """Time the fp64 oracle's decode step on `nseq` of the sequences (all their
    heads) for `nsteps` steps; sequence-steps per second."""
    import numpy as np
    import oracle
    f64 = lambda t: t[:nseq].float().cpu().numpy().astype(np.float64)
    St = f64(S)
    steps = [(f64(qs[t]), f64(ks[t]), f64(vs[t])) for t in range(nsteps)]
    lim, used = blas_limit(host_cores())
    with lim:
        threads = used()
        t0 = time.perf_counter()
        for q, k, v in steps:
            St, _ = oracle.decode_step(St, q, k, v)
        dt = time.perf_counter() - t0
    return {"value": nseq * nsteps / dt, "unit": "sequence-steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle decode_step on {nseq} sequences (all heads) x {nsteps} steps, {dt:.2f} s"}


def bench_decode(la, synth, torch, w, steps, warmup, cpu=False):
    dev = torch.device("cuda:0")
    S = torch.empty((w.B, w.Hkv, w.d, w.dv), dtype=torch.float32, device=dev)
    batch = 32
    log(f"[bench] decode prefix: {w.B} sequences x {w.N} tokens through the forward kernel, {batch} at a time")
    for i in range(0, w.B, batch):
        q, k, v = synth.make_qkv(w, dev, seed=1000 + i // batch, B=batch)
        la.forward(q, k, v, s_out=S[i:i + batch])
        del q, k, v
    torch.cuda.synchronize()
    T = steps + warmup
    qs, ks, vs = synth.make_decode_steps(w, dev, seed=1, steps=T)
    o = torch.empty((w.B, w.Hq, w.dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for t in range(warmup):
        la.decode_step(S, qs[t], ks[t], vs[t], out=o)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        t = warmup + i
        evs[i][0].record(stream)
        la.decode_step(S, qs[t], ks[t], vs[t], out=o)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = [a.elapsed_time(b) for a, b in evs]
    step_bytes = (2 * S.numel() * 4 + qs[0].numel() * 2 + ks[0].numel() * 2 + vs[0].numel() * 2 + o.numel() * 4)
    mean_ms = statistics.mean(per)
    gbs = step_bytes / (mean_ms * 1e-3) / 1e9
    cpu_rec = cpu_decode_baseline(S, qs, ks, vs) if cpu else None
    return {"steps": steps, "warmup": warmup, "ms_per_step": round(mean_ms, 5),
            "sequence_steps_per_s": round(w.B / (mean_ms * 1e-3), 1), "cpu_baseline": cpu_rec,
            "ms_per_step_median": round(statistics.median(per), 5), "ms_per_step_wall": round(wall, 5),
            "gb_per_s": round(gbs, 1), "unit": "GB/s",
            "config": {"workload": w.name, "sequences": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "dv": w.dv,
                       "prefix_tokens": w.N, "state_dtype": "f32", "io_dtype": "bf16 in, f32 out"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("decode_kernel", w.name),
                         "bytes_per_launch": step_bytes}}


# ---------------------------------------------------------------------------
# Hardware counters of this run: bench.py starts itself as the program of
# rocprofv3 --pmc (one pass per counter set, before this process touches the
# GPU), the child runs two forward steps and a 4 GiB calibration copy, and the
# parent reads the child's counter database.
# ---------------------------------------------------------------------------
COUNTER_PASSES = (("FETCH_SIZE",), ("WRITE_SIZE",), ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"))
COUNTER_KERNELS = "fwd_bf16_g4|fwd_bf16_main|fwd_bf16_solo|state_parts|decode_kernel|stream_kernel"
CALIBRATION_GIB = 4


def counter_child(workload):
    """The program rocprofv3 runs: two forward steps of `workload`, three
    decode steps of the 256-sequence decode workload (states drawn at random:
    the traffic does not depend on their values), then a copy of
    CALIBRATION_GIB GiB by the streaming library (known bytes)."""
    import ctypes
    import torch
    import long_context_attention_chunkwise_amd as la
    from long_context_attention_chunkwise_amd import synth
    from long_context_attention_chunkwise_amd import build as _build
    w = synth.WORKLOADS[workload]
    q, k, v = synth.make_qkv(w, "cuda:0", seed=0)
    o = torch.empty((w.B, w.Hq, w.N, w.dv), dtype=torch.bfloat16, device="cuda:0")
    for _ in range(2):
        la.forward(q, k, v, out=o)
    torch.cuda.synchronize()
    del q, k, v, o
    wd = synth.WORKLOADS["decode_256"]
    S = synth.random_state((wd.B, wd.Hkv, wd.d, wd.dv), "cuda:0", seed=3)
    qs, ks, vs = synth.make_decode_steps(wd, "cuda:0", seed=1, steps=3)
    od = torch.empty((wd.B, wd.Hq, wd.dv), dtype=torch.float32, device="cuda:0")
    for t in range(3):
        la.decode_step(S, qs[t], ks[t], vs[t], out=od)
    torch.cuda.synchronize()
    del S, qs, ks, vs, od
    torch.cuda.empty_cache()
    lib = ctypes.CDLL(_build.STREAM_LIB_PATH)
    lib.la_stream_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    n = CALIBRATION_GIB << 30
    a = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
    b = torch.empty_like(a)
    if lib.la_stream_run(1, 0, ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), n, None, 1024,
                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) != 0:
        raise RuntimeError("calibration copy failed")
    torch.cuda.synchronize()


def read_counter_db(path):
    """{kernel: {counter: mean over dispatches}} from a rocprofv3 database:
    per dispatch, counters summed over their hardware instances, except
    GRBM_* (one per XCD, equal): the largest instance, i.e. the cycles one XCD
    was busy."""
    import collections
    import glob
    import re
    import sqlite3
    files = glob.glob(os.path.join(path, "**", "*.db"), recursive=True)
    if not files:
        raise RuntimeError(f"no counter database under {path}")
    per = collections.defaultdict(lambda: collections.defaultdict(dict))
    for f in files:
        db = sqlite3.connect(f)
        for name, disp, dur, cname, val in db.execute(
                "select name, dispatch_id, duration, counter_name, counter_value from pmc_events"):
            m = re.search(r"(fwd_bf16_g4|fwd_bf16_main|fwd_bf16_solo|state_parts|decode_kernel|stream_kernel<1)", name)
            if not m:
                continue
            d = per[m.group(1)][disp]
            d["duration_ns"] = float(dur)
            if cname.startswith("GRBM_"):
                d[cname] = max(d.get(cname, 0.0), val)
            else:
                d[cname] = d.get(cname, 0.0) + val
        db.close()
    out = {}
    for kern, disps in per.items():
        names = {c for d in disps.values() for c in d}
        out[kern] = {c: sum(d[c] for d in disps.values() if c in d) / sum(1 for d in disps.values() if c in d)
                     for c in names}
        out[kern]["dispatches"] = len(disps)
    return out


def collect_counters(workload, timeout_s=240):
    """Run the counter passes on `workload`; returns per-kernel figures or a
    reason why none were taken.  Must run before this process uses the GPU."""
    import shutil
    import signal
    import subprocess
    import tempfile
    prof = shutil.which("rocprofv3") or ("/opt/rocm/bin/rocprofv3" if os.path.exists("/opt/rocm/bin/rocprofv3")
                                         else None)
    if prof is None:
        return {"error": "rocprofv3 not found"}
    tmp = tempfile.mkdtemp(prefix="la_counters_")
    merged = {}
    try:
        for i, counters in enumerate(COUNTER_PASSES):
            out_dir = os.path.join(tmp, f"pass{i}")
            cmd = [prof, "--pmc", *counters, "--kernel-include-regex", COUNTER_KERNELS, "-d", out_dir, "-o", "run",
                   "--", sys.executable, os.path.abspath(__file__), "--counter-child", "--workload", workload]
            log(f"[bench] counters pass {i + 1}/{len(COUNTER_PASSES)}: {' '.join(counters)}")
            env = dict(os.environ, TMPDIR=os.environ.get("TMPDIR", "/tmp"))
            p = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, start_new_session=True,
                                 env=env, cwd=tmp)
            try:
                text, _ = p.communicate(timeout=timeout_s)
            except subprocess.TimeoutExpired:
                os.killpg(p.pid, signal.SIGKILL)
                p.communicate()
                return {"error": f"counter pass {i + 1} timed out"}
            try:
                vals = read_counter_db(out_dir)
            except Exception as e:  # the profiler may exit non-zero after writing its results
                tail = text.decode(errors="replace").strip().splitlines()[-3:]
                return {"error": f"counter pass {i + 1}: {e}; rc {p.returncode}; " + " | ".join(tail)}
            for kern, d in vals.items():
                merged.setdefault(kern, {}).update(d)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return merged


def counter_figures(raw, cus, kernel, bytes_alg):
    """Traffic (FETCH_SIZE and WRITE_SIZE scaled by the calibration copy), the
    matrix-core busy fraction and the clock of `kernel` from collect_counters."""
    if "error" in raw:
        return {"error": raw["error"]}
    cal = raw.get("stream_kernel<1")
    kr = raw.get(kernel)
    if not cal or not kr or "FETCH_SIZE" not in cal or "WRITE_SIZE" not in cal:
        return {"error": "calibration or kernel counters missing"}
    known = float(CALIBRATION_GIB << 30)
    rscale = known / (cal["FETCH_SIZE"] * 1024.0)
    wscale = known / (cal["WRITE_SIZE"] * 1024.0)
    fetch = kr["FETCH_SIZE"] * 1024.0 * rscale
    write = kr["WRITE_SIZE"] * 1024.0 * wscale
    rec = {"source": "rocprofv3 --pmc child runs of this bench (2 forward steps + 4 GiB calibration copy)",
           "fetch_bytes": round(fetch), "write_bytes": round(write), "traffic": round(fetch + write),
           "fetch_scale": round(rscale, 4), "write_scale": round(wscale, 4)}
    if bytes_alg:
        rec["traffic_over_algorithmic"] = round((fetch + write) / bytes_alg, 4)
    if cus and "SQ_VALU_MFMA_BUSY_CYCLES" in kr and kr.get("GRBM_GUI_ACTIVE"):
        cycles = kr["GRBM_GUI_ACTIVE"]
        rec["mfma_busy"] = round(kr["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * cus * cycles), 4)
        rec["mfma_instructions"] = kr.get("SQ_INSTS_MFMA")
        rec["active_cycles_per_xcd"] = cycles
        dur_ns = kr.get("duration_ns")
        if dur_ns:
            rec["counter_run_kernel_ms"] = round(dur_ns * 1e-6, 4)
            rec["clock_ghz_during_kernel"] = round(cycles / (dur_ns * 1e-9) / 1e9, 3)
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gqa_1m", choices=["mha_4k", "gqa_64k", "gqa_1m", "gqa_1m_d64", "mha_1m_d64"],
                    help="bf16 forward workload (synth.WORKLOADS); the default is the 1M-token one")
    ap.add_argument("--decode-steps", type=int, default=1000, help="0 skips the decode measurement")
    ap.add_argument("--decode-warmup", type=int, default=10)
    ap.add_argument("--variant-steps", type=int, default=5, help="0 skips the forward-variant measurement")
    ap.add_argument("--backward-steps", type=int, default=5, help="0 skips the backward measurement")
    ap.add_argument("--backward-warmup", type=int, default=1)
    ap.add_argument("--state-steps", type=int, default=10,
                    help="calls of la_forward_state (final state only) on the same k, v (0 skips)")
    ap.add_argument("--in-place-steps", type=int, default=5,
                    help="steps of the forward with o written over q, timed last (0 skips)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-counters", action="store_true",
                    help="skip the rocprofv3 counter passes (traffic then comes from the committed profile)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the streaming-kernel HBM ceilings")
    ap.add_argument("--counter-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (hardware-counter calibration)")
    args = ap.parse_args()

    if args.counter_child:
        counter_child(args.workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    # Counter passes first: they run bench.py itself under rocprofv3 in child
    # processes, before this process initialises the GPU.
    counters_raw = None if args.no_counters else collect_counters(args.workload)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import long_context_attention_chunkwise_amd as la
    from long_context_attention_chunkwise_amd import synth
    la.load_library()  # fails loudly when the HIP library is missing

    w = synth.WORKLOADS[args.workload]
    # the output kernel that serves this workload's query-head group size
    G = w.Hq // w.Hkv
    if w.d == 64 and G == 1:
        main_kernel = "fwd_bf16_solo"
    elif G % 4 == 0 or w.d == 64:
        main_kernel = "fwd_bf16_g4"
    else:
        main_kernel = "fwd_bf16_main"
    props = torch.cuda.get_device_properties(0)
    bytes_main = forward_bytes(w, w.N)
    # workloads small enough to stay in the caches are also timed behind a 1 GiB scrub
    scrub = (1 << 30) if bytes_main < (4 << 30) else 0
    q, k, v, ms_step, ms_states, ms_main, ws_bytes, step_events = bench_forward(la, synth, torch, w, args.steps,
                                                                                args.warmup, scrub)
    tokens = w.B * w.N
    value = tokens / (ms_step * 1e-3)
    f_alg, f_tile = forward_flops(w, w.N)
    achieved = bytes_main / (ms_main * 1e-3) / 1e9
    log(f"[bench] forward: {ms_step:.3f} ms/step (states {ms_states:.3f} ms, outputs {ms_main:.3f} ms)")

    cpu = cpu_small = None
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (fp64 oracle) ...")
        cpu = cpu_baseline(q, k, v, w)
        cpu_small = cpu_small_baselines(synth, torch)
    variants = None
    if args.variant_steps > 0:
        variants = bench_variants(la, torch, w, q, k, v, args.variant_steps, 1)
        log("[bench] variants: " + ", ".join(f"{n} {r['ms_per_call']:.3f} ms" for n, r in variants["variants"].items()))
    backward = None
    if args.backward_steps > 0:
        backward = bench_backward(la, synth, torch, w, q, k, v, args.backward_steps, args.backward_warmup)
        log(f"[bench] backward: {backward['ms_per_step']:.3f} ms/step")
    state_only = None
    if args.state_steps > 0:
        state_only = bench_state(la, torch, w, k, v, args.state_steps, 1)
        log(f"[bench] state only: {state_only['ms_per_call']:.3f} ms, {state_only['hbm_gb_per_s']:.0f} GB/s")
    in_place = None
    if args.in_place_steps > 0 and (w.Hq // w.Hkv) % 4 == 0:
        in_place = bench_in_place(la, torch, w, q, k, v, args.in_place_steps, 1)
        log(f"[bench] forward in place: {in_place['ms_per_step']:.3f} ms/step (outputs {in_place['outputs_ms']:.3f} ms)")
    del q, k, v
    torch.cuda.empty_cache()

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    ceilings = None
    if not args.no_ceilings:
        ceilings = stream_ceilings(torch)
        log("[bench] streaming ceilings: " + ", ".join(f"{n} {r['gb_per_s']:.0f} GB/s" for n, r in ceilings.items()))

    decode = None
    if args.decode_steps > 0:
        decode = bench_decode(la, synth, torch, synth.WORKLOADS["decode_256"], args.decode_steps,
                              args.decode_warmup, cpu=not args.no_cpu_baseline)
        if ceilings:
            # decode reads every state and writes it back in place
            decode["roofline"]["frac_of_practical"] = round(
                decode["gb_per_s"] / ceilings["in_place_update"]["gb_per_s"], 4)
            decode["roofline"]["practical"] = "in-place update streaming kernel"
        if counters_raw is not None and "decode_kernel" in counters_raw:
            dc = counter_figures(counters_raw, 0, "decode_kernel", decode["roofline"]["bytes_per_launch"])
            if "traffic" in dc:
                decode["roofline"]["traffic"] = dc["traffic"]
                decode["roofline"]["traffic_source"] = "counters of this run"
                decode["roofline"]["traffic_over_algorithmic"] = dc.get("traffic_over_algorithmic")
        log(f"[bench] decode: {decode['ms_per_step']:.4f} ms/step, {decode['gb_per_s']:.0f} GB/s")

    counters = None
    traffic = measured_traffic(main_kernel, w.name)
    traffic_source = "committed profile (profiles/hbm_traffic_gqa_1m_decode_256.md)" if traffic else None
    if counters_raw is not None:
        counters = {main_kernel: counter_figures(counters_raw, props.multi_processor_count, main_kernel, bytes_main)}
        if "traffic" in counters[main_kernel]:
            traffic = counters[main_kernel]["traffic"]
            traffic_source = "counters of this run"
        if "state_parts" in counters_raw:
            counters["state_parts"] = counter_figures(counters_raw, props.multi_processor_count, "state_parts",
                                                      None)

    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic, "traffic_source": traffic_source,
                "kernel": main_kernel, "kernel_ms": round(ms_main, 4), "bytes_per_launch": bytes_main}
    if ceilings:
        # q, k, v read once and o written once: 3:2 when o is bf16
        roofline["practical"] = "read + write 3:2 streaming kernel"
        roofline["frac_of_practical"] = round(achieved / ceilings["read_write_3_2"]["gb_per_s"], 4)
    mfma = {"tflops_alg": round(f_alg / (ms_step * 1e-3) / 1e12, 2),
            "frac_alg": round(f_alg / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "tflops_tile": round(f_tile / (ms_step * 1e-3) / 1e12, 2),
            "frac_tile": round(f_tile / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "peak_tflops": PEAK_BF16_TFLOPS, "flops_alg": f_alg, "flops_tile": f_tile}
    if counters and "mfma_busy" in counters.get(main_kernel, {}):
        mfma["busy_counter"] = counters[main_kernel]["mfma_busy"]
        mfma["busy_counter_kernel"] = main_kernel

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "seq_len": w.N, "d": w.d,
                   "dv": w.dv, "block": w.block, "io_dtype": "bf16", "state_dtype": "f32"},
        "roofline": roofline,
        "mfma": mfma,
        "counters": counters,
        "phases_ms": {"segment_states": round(ms_states, 4), "outputs": round(ms_main, 4)},
        "ms_per_step_events": step_events,
        "workspace_bytes": ws_bytes,
        "variants": variants,
        "backward": backward,
        "forward_in_place": in_place,
        "state_only": state_only,
        "decode": decode,
        "cpu_baseline": cpu,
        "cpu_baseline_small_workloads": cpu_small,
        "device": {"name": props.name, "gcnArchName": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count, "stream_ceilings": ceilings},
        "inputs": {"generator": "synth.make_qkv (seeded torch draws)", "seed": 0,
                   "outputs_checked_finite": True},
        "software": {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None)},
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
