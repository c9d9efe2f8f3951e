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


def cpu_baseline(q, k, v, w, groups=3):
    """Time the fp64 oracle on the first `groups` KV groups (each with its G
    query heads, all tokens), one group at a time: about 12 s at 1M tokens."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the affinity mask
        threads = len(os.sched_getaffinity(0))
    G = w.Hq // w.Hkv
    N = q.shape[2]
    groups = min(groups, w.Hkv)
    dt = 0.0
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
            "sample": f"fp64 chunkwise oracle on KV heads 0-{groups - 1} (query heads 0-{groups * G - 1}), "
                      f"all {N} tokens, {dt:.2f} s; value scaled to the full {w.Hkv}-KV-head workload "
                      f"(x{groups}/{w.Hkv})"}


def bench_forward(la, synth, torch, w, steps, warmup):
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
              "mean": round(statistics.mean(t_step), 4)}
    return q, k, v, ms_step, statistics.mean(t_states), statistics.mean(t_main), ws_bytes, events


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
    del do, dq, dk, dv, ds, ws
    return {"steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4), "ms_per_step_wall": round(wall, 4),
            "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1),
            "config": {"workload": w.name, "grad_dtype": "bf16", "s_in": False, "grad_s_out": False},
            "hbm": {"bytes_alg": nbytes, "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "mfma": {"flops_alg": flops, "tflops_alg": round(flops / (ms * 1e-3) / 1e12, 2),
                     "frac_alg": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "workspace_bytes": ws_bytes}


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


def copy_bandwidth(torch, mib=1024, reps=7):
    """Read + write GB/s of a plain device-to-device copy of `mib` MiB (the
    runtime's copy kernel), median of `reps` event-timed copies: the practical
    streaming ceiling the HBM-bound kernels are also compared with."""
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        b.copy_(a)
        e1.record()
    torch.cuda.synchronize()
    ms = statistics.median(e0.elapsed_time(e1) for e0, e1 in evs)
    del a, b
    torch.cuda.empty_cache()
    return 2 * n / (ms * 1e-3) / 1e9


def cpu_decode_baseline(S, qs, ks, vs, nseq=4, nsteps=10):
    """Time the fp64 oracle's decode step on `nseq` of the sequences (all their
    heads) for `nsteps` steps; sequence-steps per second."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    f64 = lambda t: t[:nseq].float().cpu().numpy().astype(np.float64)
    St = f64(S)
    steps = [(f64(qs[t]), f64(ks[t]), f64(vs[t])) for t in range(nsteps)]
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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (hardware-counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import long_context_attention_chunkwise_amd as la
    from long_context_attention_chunkwise_amd import synth
    la.load_library()  # fails loudly when the HIP library is missing

    w = synth.WORKLOADS[args.workload]
    # the output kernel that serves this workload's query-head group size
    main_kernel = "fwd_bf16_g4" if (w.Hq // w.Hkv) % 4 == 0 else "fwd_bf16_main"
    props = torch.cuda.get_device_properties(0)
    q, k, v, ms_step, ms_states, ms_main, ws_bytes, step_events = bench_forward(la, synth, torch, w, args.steps,
                                                                                args.warmup)
    tokens = w.B * w.N
    value = tokens / (ms_step * 1e-3)
    f_alg, f_tile = forward_flops(w, w.N)
    bytes_main = forward_bytes(w, w.N)
    achieved = bytes_main / (ms_main * 1e-3) / 1e9
    log(f"[bench] forward: {ms_step:.3f} ms/step (states {ms_states:.3f} ms, outputs {ms_main:.3f} ms)")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (fp64 oracle) ...")
        cpu = cpu_baseline(q, k, v, w)
    variants = None
    if args.variant_steps > 0:
        variants = bench_variants(la, torch, w, q, k, v, args.variant_steps, 1)
        log("[bench] variants: " + ", ".join(f"{n} {r['ms_per_call']:.3f} ms" for n, r in variants["variants"].items()))
    backward = None
    if args.backward_steps > 0:
        backward = bench_backward(la, synth, torch, w, q, k, v, args.backward_steps, args.backward_warmup)
        log(f"[bench] backward: {backward['ms_per_step']:.3f} ms/step")
    del q, k, v
    torch.cuda.empty_cache()

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    copy_gbs = copy_bandwidth(torch)
    log(f"[bench] device copy: {copy_gbs:.0f} GB/s (read + write)")

    decode = None
    if args.decode_steps > 0:
        decode = bench_decode(la, synth, torch, synth.WORKLOADS["decode_256"], args.decode_steps,
                              args.decode_warmup, cpu=not args.no_cpu_baseline)
        decode["roofline"]["frac_of_copy"] = round(decode["gb_per_s"] / copy_gbs, 4)
        log(f"[bench] decode: {decode['ms_per_step']:.4f} ms/step, {decode['gb_per_s']:.0f} GB/s")

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
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(main_kernel, w.name),
                     "kernel": main_kernel, "kernel_ms": round(ms_main, 4), "bytes_per_launch": bytes_main,
                     "frac_of_copy": round(achieved / copy_gbs, 4)},
        "mfma": {"tflops_alg": round(f_alg / (ms_step * 1e-3) / 1e12, 2),
                 "frac_alg": round(f_alg / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                 "tflops_tile": round(f_tile / (ms_step * 1e-3) / 1e12, 2),
                 "frac_tile": round(f_tile / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                 "peak_tflops": PEAK_BF16_TFLOPS, "flops_alg": f_alg, "flops_tile": f_tile},
        "phases_ms": {"segment_states": round(ms_states, 4), "outputs": round(ms_main, 4)},
        "ms_per_step_events": step_events,
        "workspace_bytes": ws_bytes,
        "variants": variants,
        "backward": backward,
        "decode": decode,
        "cpu_baseline": cpu,
        "device": {"name": props.name, "gcnArchName": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count, "copy_gb_per_s": round(copy_gbs, 1)},
        "inputs": {"generator": "synth.make_qkv (seeded torch draws)", "seed": 0,
                   "outputs_checked_finite": True},
        "software": {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None)},
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
