#!/usr/bin/env python3
"""Throughput of SnapKV prefill compression on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--also 3,4,5]

A step is one pass of the whole path (obs_score -> vote_pool -> topk_select ->
kv_gather, i.e. one snapkv_compress per layer) over one batch of synthetic
input that already sits in HBM.  The headline workload is the Llama-2-7B-shaped
layer: 32 heads MHA, d=128, bf16, L_prompt=16384, L_obs=32, K_pool=7, p=0.05.
Steps rotate over several distinct seeded inputs (more bytes than the 256 MB
Infinity Cache) so every step reads its keys from HBM, as a fresh prefill would.

Prints one JSON line: throughput of the headline workload (prompt tokens
compressed per second per layer), the roofline of its dominant kernel (obs_score)
timed with HIP events on the launch stream, the fp64 CPU oracle timed on the host
cores as a baseline, and a "workloads" block with the same measurements for the
other standard workloads (GQA 32 layers, the 380K-token layer, the ragged batch),
taken in the same run.

Algorithmic bytes (per layer): obs_score reads every key row once and the window
queries once; kv_gather reads and writes every kept and window row of K and V once.
Intermediates (votes, pooled votes, indices) are not counted.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prompt tokens compressed/s per layer + % peak HBM GB/s (Llama-7B shape)"
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, AMD public specification
CACHE_BYTES = 256 << 20          # MI355X Infinity Cache
KERNEL_SOURCES = ("kv_cache_compression_amd/csrc/obs_score.hip", "kv_cache_compression_amd/csrc/obs_score_kernel.h",
                  "kv_cache_compression_amd/csrc/obs_stream.hip", "kv_cache_compression_amd/csrc/obs_onepass.hip",
                  "kv_cache_compression_amd/csrc/obs_onepass2.hip")
SCORING_KERNELS = ("obs_score_onepass", "obs_score_onepass2", "obs_score_fused", "obs_score_stream", "obs_score_stats",
                   "obs_stats_merge", "obs_score_votes", "sum_chunks")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, help="headline workload 1..5 (2 is the Llama-2-7B layer)")
    ap.add_argument("--also", default="3,4,5",
                    help="comma-separated workloads measured after the headline, in the same run ('' for none)")
    ap.add_argument("--launch", choices=("graph", "eager"), default="graph",
                    help="replay the timed steps as one captured HIP graph (default) or launch eagerly")
    ap.add_argument("--two-pass", action="store_true", help="force the two-pass scoring path")
    ap.add_argument("--scoring", choices=("auto", "fused", "stream", "two-pass"), default="auto",
                    help="scoring kernel: the library's choice (default), or force the fused, the streaming "
                         "two-phase or the two-pass one")
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


def say(msg):
    print("bench.py: " + msg, file=sys.stderr, flush=True)


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

    def destroy(self, arr):
        for i in range(len(arr)):
            self.lib.hipEventDestroy(arr[i])

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
    path = os.path.join(ROOT, "profiles", "obs_score_%s_pmc.md" % workload_name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)\s*\(kernel source ([0-9a-f]+)\)", text)
    if not m or m.group(2) != kernel_source_hash():
        return None
    return float(m.group(1))


def scoring_name(kernels_us):
    """Which scoring path a run took, from the kernels it launched."""
    for name, tag in (("obs_score_onepass", "one_read_stream"), ("obs_score_onepass2", "one_read_two_slots"),
                      ("obs_score_fused", "fused"),
                      ("obs_score_stream", "two_phase_stream"), ("obs_score_stats", "two_pass")):
        if name in kernels_us:
            return tag
    return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def row_lse(q, K, cu):
    """Each window row's log-sum-exp over the keys it sees, in fp32 with plain torch ops
    (input preparation outside the timed region, standing in for prefill attention)."""
    import math
    import torch
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


class Run:
    """One workload's inputs on the device, its launches, and their measurement."""

    def __init__(self, lib, hip, dev, n, args, gen_threads):
        import numpy as np
        import torch
        from kv_cache_compression_amd import _lib, synth
        self.lib, self.hip, self.dev, self.args = lib, hip, dev, args
        wl = self.wl = synth.workload(n)
        self.esz = 2 if wl.dtype == "bf16" else 4
        layer_bytes = 2 * wl.num_kv_heads * wl.total_tokens * wl.head_dim * self.esz
        self.layers_per_step = wl.n_layers
        n_sets = 1
        while n_sets * self.layers_per_step * layer_bytes < 4 * CACHE_BYTES and n_sets < 8:
            n_sets += 1
        self.n_sets = n_sets

        def to_dev(a):
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)

        say("workload %d (%s): drawing %d input set(s) of %d layer(s)" % (n, wl.name, n_sets, self.layers_per_step))
        self.sets = []
        for s in range(n_sets):
            layers = []
            for l in range(self.layers_per_step):
                x = synth.make_inputs(wl, layer=s * self.layers_per_step + l, threads=gen_threads)
                q, K, V = to_dev(x["q_obs"]), to_dev(x["K"]), to_dev(x["V"])
                spec = _lib.make_spec(q, K, x["cu_seqlens"], wl.obs_window, wl.pool_kernel, wl.ratio, wl.budget,
                                      two_pass=args.two_pass or args.scoring == "two-pass",
                                      stream=args.scoring == "stream", fused=args.scoring == "fused")
                lse = row_lse(q, K, x["cu_seqlens"]) if args.lse else None
                layers.append(dict(q=q, K=K, V=V, spec=spec, cu=x["cu_seqlens"], lse=lse,
                                   host=x if (s == 0 and l == 0) else None))
                del x
            self.sets.append(layers)
        spec0 = self.spec0 = self.sets[0][0]["spec"]
        self.K_out = torch.empty((spec0.Hkv, spec0.sum_out, wl.head_dim), dtype=self.sets[0][0]["K"].dtype,
                                 device=dev)
        self.V_out = torch.empty_like(self.K_out)
        self.idx = torch.empty((spec0.Hkv, max(spec0.sum_k, 1)), dtype=torch.int32, device=dev)
        self.ws = torch.zeros(spec0.ws_bytes, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        self.stream = torch.cuda.Stream(device=dev)  # default priority
        self.n_launch_max = 16 * self.layers_per_step

    def enqueue(self, layers):
        lib, c = self.lib, ctypes.c_void_p
        for ly in layers:
            common = (c(self.K_out.data_ptr()), c(self.V_out.data_ptr()), c(self.idx.data_ptr()), None,
                      c(self.ws.data_ptr()), ctypes.c_size_t(self.ws.numel()), c(self.stream.cuda_stream))
            if ly["lse"] is None:
                st = lib.snapkv_compress(ctypes.byref(ly["spec"].pb), c(ly["q"].data_ptr()), c(ly["K"].data_ptr()),
                                         c(ly["V"].data_ptr()), *common)
            else:
                st = lib.snapkv_compress_lse(ctypes.byref(ly["spec"].pb), c(ly["q"].data_ptr()),
                                             c(ly["K"].data_ptr()), c(ly["V"].data_ptr()), c(ly["lse"].data_ptr()),
                                             *common)
            if st != 0:
                raise RuntimeError("snapkv_compress: %s" % lib.snapkv_last_error().decode())

    def traced(self, layers, events):
        lib = self.lib
        lib.snapkv_trace_begin(ctypes.cast(events, ctypes.POINTER(ctypes.c_void_p)), self.n_launch_max)
        try:
            self.enqueue(layers)
        finally:
            ids = (ctypes.c_int32 * self.n_launch_max)()
            n = lib.snapkv_trace_end(ids, self.n_launch_max)
        return [int(ids[i]) for i in range(min(n, self.n_launch_max))]

    def error_word(self):
        import torch
        torch.cuda.synchronize()
        return int(self.ws[:4].view(torch.int32).item())

    def measure(self, steps, warmup):
        import torch
        args, hip, lib, stream, n_sets, sets = self.args, self.hip, self.lib, self.stream, self.n_sets, self.sets
        with torch.cuda.stream(stream):
            for i in range(warmup):
                self.enqueue(sets[i % n_sets])
        torch.cuda.synchronize()

        # launch mode: one captured graph per input set, checked against an eager run
        launch = args.launch
        graphs = []
        if launch == "graph":
            try:
                for s in range(n_sets):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=stream):
                        self.enqueue(sets[s])
                    graphs.append(g)
                for g in graphs:
                    g.replay()
                torch.cuda.synchronize()
                graphs[0].replay()
                torch.cuda.synchronize()
                g_idx, g_k = self.idx.clone(), self.K_out.clone()
                with torch.cuda.stream(stream):
                    self.enqueue(sets[0])
                torch.cuda.synchronize()
                if not (torch.equal(g_idx, self.idx) and torch.equal(g_k, self.K_out)):
                    raise RuntimeError("graph replay differs from an eager run of the same input")
            except Exception as e:  # capture not supported for some launch: measure eagerly
                say("graph capture failed (%s); timing eager launches" % e)
                launch, graphs = "eager", []
                torch.cuda.synchronize()

        # The timed graph holds all K steps back to back (step i on input set i mod n_sets), so
        # the timed region is one graph launch; one single-step graph per step adds the host's
        # graph-launch gap to every step, reported beside it.
        single_ms = None
        if launch == "graph":
            with torch.cuda.stream(stream):
                for i in range(steps):
                    graphs[i % n_sets].replay()
            torch.cuda.synchronize()
            s0 = time.perf_counter()
            with torch.cuda.stream(stream):
                for i in range(steps):
                    graphs[i % n_sets].replay()
            torch.cuda.synchronize()
            single_ms = (time.perf_counter() - s0) * 1e3 / steps
            g_all = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_all, stream=stream):
                for i in range(steps):
                    self.enqueue(sets[i % n_sets])
            for _ in range(max(1, -(-warmup // steps))):
                g_all.replay()
            torch.cuda.synchronize()

        # timed region; eager steps carry the kernel trace (HIP events on the launch stream
        # around every dispatch).  Graph replays carry none, so in graph mode the same steps
        # then run eagerly with the trace for the per-kernel durations.
        step_events = [hip.events(2 * self.n_launch_max) for _ in range(steps)]
        step_ids = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            if launch == "graph":
                g_all.replay()
            else:
                for i in range(steps):
                    step_ids.append(self.traced(sets[i % n_sets], step_events[i]))
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_per_step = (t1 - t0) * 1e3 / steps
        word = self.error_word()
        if word:
            raise RuntimeError("%s: the workspace error word is 0x%x after the timed steps" % (self.wl.name, word))
        eager_ms = None
        if launch == "graph":
            e0 = time.perf_counter()
            with torch.cuda.stream(stream):
                for i in range(steps):
                    step_ids.append(self.traced(sets[i % n_sets], step_events[i]))
            torch.cuda.synchronize()
            eager_ms = (time.perf_counter() - e0) * 1e3 / steps

        per_kernel = {}
        for st_i in range(steps):
            for i, kid in enumerate(step_ids[st_i]):
                name = lib.snapkv_kernel_name(kid).decode()
                per_kernel.setdefault(name, []).append(
                    hip.elapsed_ms(step_events[st_i][2 * i], step_events[st_i][2 * i + 1]))
        for ev in step_events:
            hip.destroy(ev)
        # microseconds per layer (a kernel launched n times per layer counts n times)
        kernels_us = {k: round(1e3 * sum(v) / (steps * self.layers_per_step), 3) for k, v in per_kernel.items()}
        launch_us = {k: round(1e3 * sum(v) / len(v), 3) for k, v in per_kernel.items()}
        launches = {k: len(v) / (steps * self.layers_per_step) for k, v in per_kernel.items()}

        # the last timed step's outputs equal a fresh eager run of the same input
        last = sets[(steps - 1) % n_sets]
        ref_idx, ref_k = self.idx.clone(), self.K_out.clone()
        with torch.cuda.stream(stream):
            self.enqueue(last)
        torch.cuda.synchronize()
        if not (torch.equal(ref_idx, self.idx) and torch.equal(ref_k, self.K_out)):
            raise RuntimeError("timed outputs differ from an eager run of the same input")
        if self.error_word():
            raise RuntimeError("%s: the workspace error word is set after the check step" % self.wl.name)

        # algorithmic bytes per layer
        wl, spec0, esz = self.wl, self.spec0, self.esz
        Hkv, d, T = wl.num_kv_heads, wl.head_dim, wl.total_tokens
        q_bytes = wl.batch * wl.num_q_heads * wl.obs_window * d * esz
        obs_bytes = Hkv * T * d * esz + q_bytes
        gather_bytes = 4 * Hkv * spec0.sum_out * d * esz
        scoring = {k: v for k, v in kernels_us.items() if k in SCORING_KERNELS}
        obs_us = sum(scoring.values())
        gather_us = kernels_us.get("kv_gather")
        step_us = ms_per_step * 1e3 / self.layers_per_step
        res = dict(
            workload=wl.name, launch=launch, n_sets=n_sets,
            ms_per_step=ms_per_step, eager_ms=eager_ms, single_ms=single_ms,
            value=T * self.layers_per_step / (ms_per_step * 1e-3),
            kernels_us=kernels_us, launch_us=launch_us, launches_per_layer=launches,
            obs_bytes=obs_bytes, gather_bytes=gather_bytes, obs_us=obs_us, gather_us=gather_us,
            obs_frac=obs_bytes / (obs_us * 1e-6) / 1e9 / PEAK_HBM_GBS if obs_us else None,
            obs_gather_frac=(obs_bytes + gather_bytes) / ((obs_us + gather_us) * 1e-6) / 1e9 / PEAK_HBM_GBS
            if obs_us and gather_us else None,
            end_to_end_frac=(obs_bytes + gather_bytes) / (step_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
        )
        # dominant kernel: the scoring launch with the most time per layer
        if scoring:
            dom = max(scoring, key=scoring.get)
            n_l = launches.get(dom, 1.0) or 1.0
            res["dominant"] = dom
            res["dominant_alg_bytes_per_launch"] = obs_bytes / n_l if dom in ("obs_score_onepass", "obs_score_onepass2",
                                                                            "obs_score_fused",
                                                                            "obs_score_stream",
                                                                            "obs_score_votes") else None
            res["dominant_launch_us"] = launch_us[dom]
        return res

    def summary(self, r):
        """Compact per-workload record for the workloads block."""
        wl = self.wl
        return {"ms_per_step": round(r["ms_per_step"], 5), "layers_per_step": self.layers_per_step,
                "value": round(r["value"], 1), "unit": "tokens/s per layer",
                "obs_score_us": round(r["obs_us"], 3), "obs_score_frac": round(r["obs_frac"], 4) if r["obs_frac"] else None,
                "obs_score_plus_kv_gather_frac": round(r["obs_gather_frac"], 4) if r["obs_gather_frac"] else None,
                "end_to_end_frac": round(r["end_to_end_frac"], 4), "kernels_us_per_layer": r["kernels_us"],
                "launches_per_layer": r["launches_per_layer"], "traffic": profiled_traffic(wl.name),
                "config": {"num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                           "batch": wl.batch, "L_prompt": list(wl.lengths) if wl.batch > 1 else wl.lengths[0],
                           "L_obs": wl.obs_window, "K_pool": wl.pool_kernel, "p": wl.ratio, "budget": wl.budget,
                           "input_sets": self.n_sets}}


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
    from kv_cache_compression_amd import _lib

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    lib = _lib.load()
    hip = Hip()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen_threads = min(16, os.cpu_count() or 1)

    head = Run(lib, hip, dev, args.workload, args, gen_threads)
    r = head.measure(args.steps, args.warmup)
    wl, spec0, esz = head.wl, head.spec0, head.esz
    Hkv, d, T = wl.num_kv_heads, wl.head_dim, wl.total_tokens
    say("workload %d: %.4f ms per step" % (args.workload, r["ms_per_step"]))

    # ---- Hit Rate kernel (optional): reads the attention and the selection once -----------
    hit = None
    stream = head.stream
    if args.hit_rate:
        a_cur = torch.rand((Hkv, spec0.sum_P), device=dev) * 0.1
        counts = torch.empty((wl.batch, Hkv, 2), dtype=torch.int32, device=dev)
        n_hit = 20
        ev_h = [hip.events(4) for _ in range(n_hit)]
        n_launch = []
        with torch.cuda.stream(stream):
            for i in range(n_hit + 3):
                if i >= 3:
                    lib.snapkv_trace_begin(ctypes.cast(ev_h[i - 3], ctypes.POINTER(ctypes.c_void_p)), 2)
                st = lib.snapkv_hit_rate(ctypes.byref(spec0.pb), ctypes.c_void_p(a_cur.data_ptr()),
                                         ctypes.c_void_p(head.idx.data_ptr()), ctypes.c_double(0.05),
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
        K_out, V_out = head.K_out, head.V_out
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
        x = head.sets[0][0]["host"]
        pairs_cpu = [(rq, g) for rq in range(wl.batch) for g in range(Hkv)]
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
        cpu = {"value": round(T * frac / dt, 1), "unit": "tokens/s", "cores": used, "cpu_model": cpu_model(),
               "kind": "oracle",
               "sample": "%d of %d (request, KV head) pairs of one layer, votes+pool+select in fp64, median of %d "
                         "runs, scaled to the layer" % (len(pairs_cpu), wl.batch * Hkv, len(times))}

    headline_layers = head.layers_per_step
    headline_sets = head.n_sets
    del head
    torch.cuda.empty_cache()

    # ---- the other workloads, same measurements, same run ------------------------------------
    others = {}
    for tok in [t for t in args.also.split(",") if t.strip()]:
        n = int(tok)
        if n == args.workload:
            continue
        run = Run(lib, hip, dev, n, args, gen_threads)
        rr = run.measure(args.steps, args.warmup)
        say("workload %d: %.4f ms per step" % (n, rr["ms_per_step"]))
        others[run.wl.name] = run.summary(rr)
        del run
        torch.cuda.empty_cache()

    dom = r.get("dominant")
    dom_bytes = r.get("dominant_alg_bytes_per_launch")
    dom_us = r.get("dominant_launch_us")
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9 if dom_bytes and dom_us else None
    out = {
        "metric": METRIC,
        "value": round(r["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "eager_traced_ms_per_step": round(r["eager_ms"], 5) if r["eager_ms"] else None,
        "single_step_graphs_ms_per_step": round(r["single_ms"], 5) if r["single_ms"] else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "num_q_heads": wl.num_q_heads, "num_kv_heads": Hkv, "head_dim": d,
                   "batch": wl.batch, "L_prompt": list(wl.lengths) if wl.batch > 1 else wl.lengths[0],
                   "L_obs": wl.obs_window, "K_pool": wl.pool_kernel, "p": wl.ratio, "budget": wl.budget,
                   "layers_per_step": headline_layers, "input_sets": headline_sets,
                   "launch": "one graph of all timed steps" if r["launch"] == "graph" else r["launch"],
                   "kernel_timing": "traced eager steps" + (" after the graph replays" if r["launch"] == "graph"
                                                             else ""),
                   "scoring": "lse_fed" if args.lse else scoring_name(r["kernels_us"])},
        "roofline": {"kernel": dom, "bound": "hbm",
                     "achieved": round(achieved, 1) if achieved else None, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4) if achieved else None,
                     "traffic": profiled_traffic(wl.name), "alg_bytes_per_launch": int(dom_bytes) if dom_bytes else None,
                     "avg_launch_us": dom_us},
        "obs_score_plus_kv_gather_frac": round(r["obs_gather_frac"], 4) if r["obs_gather_frac"] else None,
        "end_to_end_frac": round(r["end_to_end_frac"], 4),
        "kernels_us": r["kernels_us"],
        "cpu_baseline": cpu,
        "workloads": others,
    }
    if hit is not None:
        out["hit_rate_kernel"] = hit
    if dec is not None:
        out["decode_over_compressed_cache"] = dec
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
