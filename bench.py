#!/usr/bin/env python3
"""Throughput of SnapKV prefill compression on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

A step is one pass of the whole path (obs_score -> vote_pool -> topk_select ->
kv_gather, i.e. one snapkv_compress per layer) over one batch of synthetic
input that already sits in HBM.  The default workload is the Llama-2-7B-shaped
layer: 32 heads MHA, d=128, bf16, L_prompt=16384, L_obs=32, K_pool=7, p=0.05.
Steps rotate over several distinct seeded inputs (more bytes than the 256 MB
Infinity Cache) so every step reads its keys from HBM, as a fresh prefill would.

Prints one JSON line: throughput (prompt tokens compressed per second per layer),
the roofline of the dominant kernel (obs_score) timed with HIP events on the
launch stream over the timed region, and the fp64 CPU oracle timed on the host
cores as a baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prompt tokens compressed/s per layer + % peak HBM GB/s (Llama-7B shape)"
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, AMD public specification
CACHE_BYTES = 256 << 20          # MI355X Infinity Cache
KERNEL_SOURCES = ("kv_cache_compression_amd/csrc/obs_score.hip",)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, help="standard workload 1..5 (2 is the headline)")
    ap.add_argument("--launch", choices=("graph", "eager"), default="graph",
                    help="replay each step as a captured HIP graph (default) or launch eagerly")
    ap.add_argument("--two-pass", action="store_true", help="force the two-pass scoring path")
    ap.add_argument("--lse", action="store_true",
                    help="time snapkv_compress_lse: each window row's log-sum-exp given (as prefill attention "
                         "would provide it), one read of K")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--decode", action="store_true",
                    help="also time snapkv_decode: one query row per head over the last step's compressed cache")
    ap.add_argument("--hit-rate", action="store_true",
                    help="also time snapkv_hit_rate on the last step's selection (random attention, theta 0.05)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 launches) and exit: the known-size "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes")
    return ap.parse_args()


def copy_calibration(mib):
    """dst = src * 1 on float32 buffers of `mib` MiB: reads and writes exactly mib MiB per launch."""
    import torch
    dev = torch.device("cuda:0")
    n = mib * (1 << 20) // 4
    src = torch.rand(n, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    if not torch.equal(src, dst):
        raise RuntimeError("copy calibration produced a wrong copy")
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "launches": 5}), flush=True)


class Hip:
    """The few HIP runtime calls the timing needs (same runtime instance as torch)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = h
        return arr

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profiled_traffic(workload_name):
    """HBM bytes per obs_score launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "obs_score_fused_%s_pmc.md" % workload_name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)\s*\(kernel source ([0-9a-f]+)\)", text)
    if not m or m.group(2) != kernel_source_hash():
        return None
    return float(m.group(1))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d (WORLD_SIZE %d) is not supported. "
              "A multi-GPU split would shard KV heads with no exchange; it is not built here." % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import numpy as np
    import torch
    from kv_cache_compression_amd import _lib, synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    lib = _lib.load()
    hip = Hip()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.workload(args.workload)
    esz = 2 if wl.dtype == "bf16" else 4

    # ---- inputs: distinct seeded layers, resident in HBM --------------------------------
    layer_bytes = 2 * wl.num_kv_heads * wl.total_tokens * wl.head_dim * esz
    layers_per_step = wl.n_layers
    n_sets = 1
    while n_sets * layers_per_step * layer_bytes < 4 * CACHE_BYTES and n_sets < 8:
        n_sets += 1
    gen_threads = min(16, os.cpu_count() or 1)

    def row_lse(q, K, cu):
        """Each window row's log-sum-exp over the keys it sees, in fp32 with plain torch ops
        (input preparation outside the timed region, standing in for prefill attention)."""
        B, Hq, w, d = q.shape
        G = Hq // K.shape[0]
        out = torch.empty((B, Hq, w), dtype=torch.float32, device=q.device)
        for r in range(B):
            t0, t1 = int(cu[r]), int(cu[r + 1])
            P = t1 - t0 - w
            for h0 in range(0, Hq, G):
                kf = K[h0 // G, t0:t1].float().contiguous()                       # [L, d]
                qf = q[r, h0:h0 + G].float().reshape(G * w, d).contiguous()        # [G*w, d]
                s = torch.matmul(qf, kf.t().contiguous()) / math.sqrt(d)          # [G*w, L]
                i = torch.arange(G * w, device=q.device) % w
                j = torch.arange(t1 - t0, device=q.device)
                s = s.masked_fill(j[None, :] > (P + i)[:, None], float("-inf"))
                out[r, h0:h0 + G] = torch.logsumexp(s, dim=1).reshape(G, w)
        return out

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    sets = []
    for s in range(n_sets):
        layers = []
        for l in range(layers_per_step):
            x = synth.make_inputs(wl, layer=s * layers_per_step + l, threads=gen_threads)
            q, K, V = to_dev(x["q_obs"]), to_dev(x["K"]), to_dev(x["V"])
            spec = _lib.make_spec(q, K, x["cu_seqlens"], wl.obs_window, wl.pool_kernel, wl.ratio, wl.budget,
                                  two_pass=args.two_pass)
            lse = row_lse(q, K, x["cu_seqlens"]) if args.lse else None
            layers.append(dict(q=q, K=K, V=V, spec=spec, cu=x["cu_seqlens"], lse=lse,
                               host=x if (s == 0 and l == 0) else None))
        sets.append(layers)
    spec0 = sets[0][0]["spec"]
    K_out = torch.empty((spec0.Hkv, spec0.sum_out, wl.head_dim), dtype=sets[0][0]["K"].dtype, device=dev)
    V_out = torch.empty_like(K_out)
    idx = torch.empty((spec0.Hkv, max(spec0.sum_k, 1)), dtype=torch.int32, device=dev)
    ws = torch.zeros(spec0.ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream(device=dev)  # default priority
    n_launch_max = 16 * layers_per_step

    def enqueue(layers):
        for ly in layers:
            if ly["lse"] is None:
                st = lib.snapkv_compress(ctypes.byref(ly["spec"].pb), ctypes.c_void_p(ly["q"].data_ptr()),
                                         ctypes.c_void_p(ly["K"].data_ptr()), ctypes.c_void_p(ly["V"].data_ptr()),
                                         ctypes.c_void_p(K_out.data_ptr()), ctypes.c_void_p(V_out.data_ptr()),
                                         ctypes.c_void_p(idx.data_ptr()), None, ctypes.c_void_p(ws.data_ptr()),
                                         ctypes.c_size_t(ws.numel()), ctypes.c_void_p(stream.cuda_stream))
            else:
                st = lib.snapkv_compress_lse(ctypes.byref(ly["spec"].pb), ctypes.c_void_p(ly["q"].data_ptr()),
                                             ctypes.c_void_p(ly["K"].data_ptr()), ctypes.c_void_p(ly["V"].data_ptr()),
                                             ctypes.c_void_p(ly["lse"].data_ptr()),
                                             ctypes.c_void_p(K_out.data_ptr()), ctypes.c_void_p(V_out.data_ptr()),
                                             ctypes.c_void_p(idx.data_ptr()), None, ctypes.c_void_p(ws.data_ptr()),
                                             ctypes.c_size_t(ws.numel()), ctypes.c_void_p(stream.cuda_stream))
            if st != 0:
                raise RuntimeError("snapkv_compress: %s" % lib.snapkv_last_error().decode())

    def traced(layers, events):
        lib.snapkv_trace_begin(ctypes.cast(events, ctypes.POINTER(ctypes.c_void_p)), n_launch_max)
        try:
            enqueue(layers)
        finally:
            ids = (ctypes.c_int32 * n_launch_max)()
            n = lib.snapkv_trace_end(ids, n_launch_max)
        return [int(ids[i]) for i in range(min(n, n_launch_max))]

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            enqueue(sets[i % n_sets])
    torch.cuda.synchronize()

    # ---- launch mode: one captured graph per input set ---------------------------------
    launch = args.launch
    graphs = []
    if launch == "graph":
        try:
            for s in range(n_sets):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    enqueue(sets[s])
                graphs.append(g)
            for g in graphs:
                g.replay()
            torch.cuda.synchronize()
            # a replay gives the same bits as an eager run of the same input
            graphs[0].replay()
            torch.cuda.synchronize()
            g_idx, g_k = idx.clone(), K_out.clone()
            with torch.cuda.stream(stream):
                enqueue(sets[0])
            torch.cuda.synchronize()
            if not (torch.equal(g_idx, idx) and torch.equal(g_k, K_out)):
                raise RuntimeError("graph replay differs from an eager run of the same input")
        except Exception as e:  # capture not supported for some launch: measure eagerly
            print("bench.py: graph capture failed (%s); timing eager launches" % e, file=sys.stderr)
            launch, graphs = "eager", []
            torch.cuda.synchronize()

    # The timed graph holds all K steps back to back (step i on input set i mod n_sets), so
    # the timed region is one graph launch; replaying one single-step graph per step adds the
    # host's graph-launch gap to every step, reported beside it.
    single_ms_per_step = None
    if launch == "graph":
        with torch.cuda.stream(stream):
            for i in range(args.steps):
                graphs[i % n_sets].replay()
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for i in range(args.steps):
                graphs[i % n_sets].replay()
        torch.cuda.synchronize()
        single_ms_per_step = (time.perf_counter() - s0) * 1e3 / args.steps
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all, stream=stream):
            for i in range(args.steps):
                enqueue(sets[i % n_sets])
        for _ in range(max(1, -(-args.warmup // args.steps))):
            g_all.replay()
        torch.cuda.synchronize()

    # ---- timed region ---------------------------------------------------------------
    # Eager steps carry the kernel trace (events on the launch stream around every kernel).
    # Graph replays carry none (events inside a captured graph cannot be read back), so in
    # graph mode the same steps then run eagerly with the trace, right after, for the
    # per-kernel durations.
    step_events = [hip.events(2 * n_launch_max) for _ in range(args.steps)]
    step_ids = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        if launch == "graph":
            g_all.replay()
        else:
            for i in range(args.steps):
                step_ids.append(traced(sets[i % n_sets], step_events[i]))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    eager_ms_per_step = None
    if launch == "graph":
        torch.cuda.synchronize()
        e0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for i in range(args.steps):
                step_ids.append(traced(sets[i % n_sets], step_events[i]))
        torch.cuda.synchronize()
        eager_ms_per_step = (time.perf_counter() - e0) * 1e3 / args.steps

    per_kernel = {}
    for st_i in range(args.steps):
        for i, kid in enumerate(step_ids[st_i]):
            name = lib.snapkv_kernel_name(kid).decode()
            per_kernel.setdefault(name, []).append(hip.elapsed_ms(step_events[st_i][2 * i], step_events[st_i][2 * i + 1]))
    kernels_us = {k: round(1e3 * sum(v) / len(v), 3) for k, v in per_kernel.items()}
    launches_per_step = {k: len(v) / args.steps for k, v in per_kernel.items()}

    # ---- algorithmic bytes ----------------------------------------------------------
    # obs_score (per layer): every key row once, the window queries once, the votes written once.
    # kv_gather (per layer): chosen and window rows of K and V, read once and written once, plus idx.
    Hkv, d, T = wl.num_kv_heads, wl.head_dim, wl.total_tokens
    q_bytes = wl.batch * wl.num_q_heads * wl.obs_window * d * esz
    obs_bytes = Hkv * T * d * esz + q_bytes + Hkv * spec0.sum_P * 4
    gather_bytes = 4 * Hkv * spec0.sum_out * d * esz + Hkv * spec0.sum_k * 4
    path_bytes = Hkv * T * d * esz + q_bytes + 4 * Hkv * spec0.sum_out * d * esz  # K once, q once, rows r+w

    # the scoring kernel that ran: fused, the LSE-fed votes pass, or (two-pass) the three launches
    if args.lse:
        obs_name = "obs_score_votes"
    elif "obs_score_fused" in kernels_us:
        obs_name = "obs_score_fused"
    else:
        obs_name = "obs_score_votes"
    obs_us = kernels_us.get(obs_name)
    roof_name = obs_name
    if obs_name == "obs_score_votes" and not args.lse and obs_us is not None:
        obs_us = sum(kernels_us.get(k, 0.0) for k in ("obs_score_stats", "obs_stats_merge", "obs_score_votes"))
        roof_name = "obs_score_stats+obs_stats_merge+obs_score_votes"
    obs_launches = launches_per_step.get(obs_name, 1.0) or 1.0
    obs_bytes_launch = obs_bytes * layers_per_step / obs_launches
    achieved = obs_bytes_launch / (obs_us * 1e-6) / 1e9 if obs_us else None
    traffic = profiled_traffic(wl.name)
    gather_us = kernels_us.get("kv_gather")
    frac_obs_gather = None
    if obs_us and gather_us:
        frac_obs_gather = (obs_bytes + gather_bytes) / ((obs_us + gather_us) * 1e-6) / 1e9 / PEAK_HBM_GBS

    # prompt tokens compressed per second per layer: a step compresses T tokens in each of its layers
    value = T * layers_per_step / (ms_per_step * 1e-3)

    # the outputs of the last timed step equal a fresh eager run of the same input
    last = sets[(args.steps - 1) % n_sets]
    ref_idx, ref_k = idx.clone(), K_out.clone()
    with torch.cuda.stream(stream):
        enqueue(last)
    torch.cuda.synchronize()
    if not (torch.equal(ref_idx, idx) and torch.equal(ref_k, K_out)):
        raise RuntimeError("timed outputs differ from an eager run of the same input")

    # ---- Hit Rate kernel (optional): reads the attention and the selection once -----------
    hit = None
    if args.hit_rate:
        a_cur = torch.rand((Hkv, spec0.sum_P), device=dev) * 0.1
        counts = torch.empty((wl.batch, Hkv, 2), dtype=torch.int32, device=dev)
        n_hit = 20
        # one launch per call, or two (the counts' clearing kernel, then the tiles) when a
        # segment spans several tiles
        ev_h = [hip.events(4) for _ in range(n_hit)]
        n_launch = []
        with torch.cuda.stream(stream):
            for i in range(n_hit + 3):
                if i >= 3:
                    lib.snapkv_trace_begin(ctypes.cast(ev_h[i - 3], ctypes.POINTER(ctypes.c_void_p)), 2)
                st = lib.snapkv_hit_rate(ctypes.byref(spec0.pb), ctypes.c_void_p(a_cur.data_ptr()),
                                         ctypes.c_void_p(idx.data_ptr()), ctypes.c_double(0.05),
                                         ctypes.c_void_p(counts.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
                if i >= 3:
                    ids2 = (ctypes.c_int32 * 2)()
                    n_launch.append(lib.snapkv_trace_end(ids2, 2))
                    if n_launch[-1] not in (1, 2):
                        raise RuntimeError("snapkv_hit_rate: expected one or two launches")
                if st != 0:
                    raise RuntimeError("snapkv_hit_rate: %s" % lib.snapkv_last_error().decode())
        torch.cuda.synchronize()
        two = n_launch[0] == 2
        clear_us = 1e3 * sum(hip.elapsed_ms(ev_h[i][0], ev_h[i][1]) for i in range(n_hit)) / n_hit if two else 0.0
        j = 2 if two else 0
        tiles_us = 1e3 * sum(hip.elapsed_ms(ev_h[i][j], ev_h[i][j + 1]) for i in range(n_hit)) / n_hit
        us = clear_us + tiles_us
        hb = 4 * Hkv * spec0.sum_P + 4 * Hkv * spec0.sum_k + 8 * wl.batch * Hkv
        hit = {"avg_launch_us": round(us, 3), "clear_us": round(clear_us, 3), "tiles_us": round(tiles_us, 3),
               "alg_bytes": hb, "GB/s": round(hb / (us * 1e-6) / 1e9, 1)}

    # ---- decode attention over the compressed cache (optional) ------------------------------
    dec = None
    if args.decode:
        qd = torch.randn((wl.batch, wl.num_q_heads, d), device=dev).to(K_out.dtype)
        cu_rows = np.ascontiguousarray(spec0.cu_out.astype(np.int64))
        dprob = _lib.DecodeProblem()
        dprob.batch, dprob.num_q_heads, dprob.num_kv_heads, dprob.head_dim = wl.batch, wl.num_q_heads, Hkv, d
        dprob.dtype = 1 if wl.dtype == "bf16" else 0
        dprob.kv_head_stride, dprob.kv_token_stride = K_out.stride(0), K_out.stride(1)
        dprob.cu_rows_host = cu_rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        need = ctypes.c_size_t()
        if lib.snapkv_decode_plan(ctypes.byref(dprob), ctypes.byref(need)) != 0:
            raise RuntimeError("snapkv_decode_plan: %s" % lib.snapkv_last_error().decode())
        dws = torch.empty(max(need.value, 256), dtype=torch.uint8, device=dev)
        dout = torch.empty((wl.batch, wl.num_q_heads, d), dtype=torch.float32, device=dev)
        n_dec = 20
        ev_d = [hip.events(4) for _ in range(n_dec)]
        with torch.cuda.stream(stream):
            for i in range(n_dec + 3):
                if i >= 3:
                    lib.snapkv_trace_begin(ctypes.cast(ev_d[i - 3], ctypes.POINTER(ctypes.c_void_p)), 2)
                st = lib.snapkv_decode(ctypes.byref(dprob), ctypes.c_void_p(qd.data_ptr()),
                                       ctypes.c_void_p(K_out.data_ptr()), ctypes.c_void_p(V_out.data_ptr()),
                                       ctypes.c_void_p(dout.data_ptr()), ctypes.c_void_p(dws.data_ptr()),
                                       ctypes.c_size_t(dws.numel()), ctypes.c_void_p(stream.cuda_stream))
                if i >= 3:
                    ids2 = (ctypes.c_int32 * 2)()
                    lib.snapkv_trace_end(ids2, 2)
                if st != 0:
                    raise RuntimeError("snapkv_decode: %s" % lib.snapkv_last_error().decode())
        torch.cuda.synchronize()
        part_us = 1e3 * sum(hip.elapsed_ms(ev_d[i][0], ev_d[i][1]) for i in range(n_dec)) / n_dec
        comb_us = 1e3 * sum(hip.elapsed_ms(ev_d[i][2], ev_d[i][3]) for i in range(n_dec)) / n_dec
        db = 2 * Hkv * spec0.sum_out * d * esz + 2 * wl.batch * wl.num_q_heads * d * (esz + 4)
        dec = {"decode_attention_us": round(part_us, 3), "decode_combine_us": round(comb_us, 3),
               "cache_rows_per_head": int(spec0.sum_out), "alg_bytes": db,
               "GB/s": round(db / ((part_us + comb_us) * 1e-6) / 1e9, 1)}

    # ---- CPU baseline: the oracle on the host cores --------------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        x = sets[0][0]["host"]
        pairs_cpu = [(r, g) for r in range(wl.batch) for g in range(Hkv)]
        if wl.total_tokens * Hkv > 2_000_000:  # bounded sample for the long workloads
            pairs_cpu = pairs_cpu[: max(1, len(pairs_cpu) // 8)]
        times = []
        used = 0
        for _ in range(max(1, args.cpu_reps)):
            dt, used = oracle.run_jobs_timed(x["q_obs"], x["K"], x["cu_seqlens"], wl.obs_window, wl.pool_kernel,
                                             ratio=wl.ratio, budget=wl.budget, pairs=pairs_cpu)
            times.append(dt)
        dt = sorted(times)[len(times) // 2]
        frac = len(pairs_cpu) / (wl.batch * Hkv)
        cpu = {"value": round(T * frac / dt, 1), "unit": "tokens/s", "cores": used, "kind": "oracle",
               "sample": "%d of %d (request, KV head) pairs of one layer, votes+pool+select in fp64, median of %d "
                         "runs, scaled to the layer" % (len(pairs_cpu), wl.batch * Hkv, len(times))}

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "eager_traced_ms_per_step": round(eager_ms_per_step, 5) if eager_ms_per_step else None,
        "single_step_graphs_ms_per_step": round(single_ms_per_step, 5) if single_ms_per_step else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "num_q_heads": wl.num_q_heads, "num_kv_heads": Hkv, "head_dim": d,
                   "batch": wl.batch, "L_prompt": list(wl.lengths) if wl.batch > 1 else wl.lengths[0],
                   "L_obs": wl.obs_window, "K_pool": wl.pool_kernel, "p": wl.ratio, "budget": wl.budget,
                   "layers_per_step": layers_per_step, "input_sets": n_sets,
                   "launch": "one graph of all timed steps" if launch == "graph" else launch,
                   "kernel_timing": "traced eager steps" + (" after the graph replays" if launch == "graph" else ""),
                   "scoring": "lse_fed" if args.lse else ("two_pass" if obs_name != "obs_score_fused" else "fused")},
        "roofline": {"kernel": roof_name, "bound": "hbm",
                     "achieved": round(achieved, 1) if achieved else None, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4) if achieved else None,
                     "traffic": traffic, "alg_bytes_per_launch": int(obs_bytes_launch),
                     "avg_launch_us": obs_us},
        "obs_score_plus_kv_gather_frac": round(frac_obs_gather, 4) if frac_obs_gather else None,
        "end_to_end_frac": round(path_bytes * layers_per_step / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "kernels_us": kernels_us,
        "cpu_baseline": cpu,
    }
    if hit is not None:
        out["hit_rate_kernel"] = hit
    if dec is not None:
        out["decode_over_compressed_cache"] = dec
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
