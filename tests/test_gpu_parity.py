"""GPU parity: libsnapkv (through the C ABI) against the fp64 CPU oracle.

Small shapes cover every kernel instantiation, ragged slab tails, GQA groups whose
row count is not a multiple of 16, both softmax variants, both scoring paths,
ratio and budget modes, ragged batches and the degenerate cases.  The five
standard workloads run at full size in the launch configuration the benchmark
times, checked on sampled (request, KV head) pairs the oracle computes one by one.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_amd import synth
from parity_utils import (check_gather, check_scores, check_select_exact, check_selection, to_numpy_bits,
                          to_torch)

pytestmark = pytest.mark.gpu


def _snap():
    from kv_cache_compression_amd import _lib
    return _lib


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def stream_supported(wl):
    """The streaming scoring kernel takes rows of 256 bytes and up to 256 query rows per KV head."""
    row_bytes = wl.head_dim * (2 if wl.dtype == "bf16" else 4)
    return row_bytes == 256 and wl.group * wl.obs_window <= 256


def run_and_check(wl, *, layer=0, variant=0, two_pass=False, stream=False, fused=False, pairs=None,
                  token_major=False, threads=16, inputs=None):
    snap = _snap()
    _say("case %s layer=%d variant=%d two_pass=%s stream=%s fused=%s token_major=%s" % (
        wl.name, layer, variant, two_pass, stream, fused, token_major))
    x = inputs if inputs is not None else synth.make_inputs(wl, layer, threads=threads)
    w, cu = wl.obs_window, x["cu_seqlens"]
    q = to_torch(x["q_obs"])
    K = to_torch(x["K"])
    V = to_torch(x["V"])
    if token_major:  # storage [T, H_kv, d], viewed as [H_kv, T, d]
        K = K.transpose(0, 1).contiguous().transpose(0, 1)
        V = V.transpose(0, 1).contiguous().transpose(0, 1)
    kw = dict(obs_window=w, pool_kernel=wl.pool_kernel, ratio=wl.ratio, budget=wl.budget)
    spec = snap.make_spec(q, K, cu, w, wl.pool_kernel, wl.ratio, wl.budget, variant, two_pass, stream, fused)
    ws = snap.workspace(spec, K.device)
    votes, pooled = snap.scores(q, K, cu, variant=variant, two_pass=two_pass, stream=stream, fused=fused, ws=ws,
                                **kw)
    torch.cuda.synchronize()
    err_word = int(ws[:4].view(torch.int32).item())
    assert err_word == 0, "scoring reported error word %d" % err_word
    res = snap.compress(q, K, V, cu, variant=variant, two_pass=two_pass, stream=stream, fused=fused,
                        want_pooled=True, ws=ws, **kw)
    torch.cuda.synchronize()
    votes = votes.cpu().numpy()
    pooled_s = pooled.cpu().numpy()
    pooled_c = res["pooled"].cpu().numpy()
    np.testing.assert_array_equal(pooled_s, pooled_c)  # same work, same bits
    idx = res["idx"].cpu().numpy()
    K_out = to_numpy_bits(res["K_out"])
    V_out = to_numpy_bits(res["V_out"])
    ref = oracle.compress(x["q_obs"], x["K"], x["V"], cu, w, wl.pool_kernel, ratio=wl.ratio, budget=wl.budget,
                          variant=variant, pairs=pairs, with_gather=False)
    cu_pfx, cu_k, cu_out = spec.cu_pfx, spec.cu_k, spec.cu_out
    for (r, g), rr in sorted(ref.items()):
        t0, t1 = int(cu[r]), int(cu[r + 1])
        P = t1 - t0 - w
        k = rr["k"]
        assert k == int(spec.k[r])
        tag = "%s r=%d g=%d" % (wl.name, r, g)
        cols = slice(int(cu_pfx[r]), int(cu_pfx[r + 1]))
        check_scores(votes[g, cols], rr["votes"], tag + " votes")
        check_scores(pooled_s[g, cols], rr["pooled"], tag + " pooled")
        ig = idx[g, int(cu_k[r]):int(cu_k[r + 1])]
        check_selection(ig, rr["pooled"], rr["idx"], k, tag + " select")
        check_select_exact(ig, pooled_c[g, cols], k, tag + " select-exact")
        rows = slice(int(cu_out[r]), int(cu_out[r + 1]))
        check_gather(x["K"][g, t0:t1], K_out[g, rows], ig, P, w, tag + " K gather")
        check_gather(x["V"][g, t0:t1], V_out[g, rows], ig, P, w, tag + " V gather")
    return x, res


SMALL = [
    # name, lengths, Hq, Hkv, d, dtype, w, K_pool, ratio, budget, n_plant
    ("mha_bf16_d128_tail", [1000], 4, 4, 128, "bf16", 32, 7, 0.05, None, 8),
    ("mha_bf16_d128_2slabs", [4133], 2, 2, 128, "bf16", 32, 7, 0.05, None, 16),
    ("mha_bf16_d64", [2500], 4, 4, 64, "bf16", 32, 5, 0.05, None, 8),
    ("mha_f32_d64", [1024], 8, 8, 64, "f32", 32, 7, 0.05, None, 0),
    ("f32_d128_M32", [3000], 2, 1, 128, "f32", 16, 7, 0.1, None, 4),
    ("f32_d128_M64", [2100], 4, 2, 128, "f32", 32, 3, 0.05, None, 4),
    ("f32_d128_M256", [900], 8, 1, 128, "f32", 32, 7, None, 100, 4),
    ("gqa_M15_d64", [700], 3, 1, 64, "bf16", 5, 3, 0.1, None, 4),
    ("gqa_M48_d64", [2500], 6, 2, 64, "bf16", 16, 7, 0.05, None, 8),
    ("gqa_M128_d128", [4100], 8, 2, 128, "bf16", 32, 7, 0.05, None, 16),
    ("gqa_M256_d128", [5000], 8, 2, 128, "bf16", 64, 7, None, 300, 16),
    ("gqa_M256_d64", [1500], 16, 4, 64, "bf16", 64, 13, 0.05, None, 8),
    ("w1_d64", [300], 2, 2, 64, "bf16", 1, 7, 0.05, None, 0),
    ("pool1_topk_exact", [2000], 2, 2, 128, "bf16", 32, 1, 0.05, None, 8),
    ("varlen_gqa", [33, 2049, 700, 64, 4500], 8, 2, 128, "bf16", 32, 7, 0.05, None, 8),
    ("pool31_half15", [3000], 4, 2, 64, "bf16", 16, 31, 0.05, None, 8),
    ("gqa_M512_chunks16", [2600], 16, 1, 64, "bf16", 32, 7, 0.05, None, 8),
    ("gqa_M200_ragged_chunk", [3100, 700], 8, 1, 128, "bf16", 25, 7, 0.05, None, 8),
    ("f32_d64_M96", [1500], 6, 2, 64, "f32", 32, 5, 0.1, None, 4),
    ("pool17_run32", [20000], 2, 1, 64, "bf16", 16, 17, 0.05, None, 8),
    ("pool33_run32", [20000], 2, 1, 64, "bf16", 16, 33, 0.05, None, 8),
    ("pool41_pool_kernel", [2600, 900], 4, 2, 64, "bf16", 16, 41, 0.05, None, 8),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes(case):
    name, lengths, Hq, Hkv, d, dt, w, kp, ratio, budget, n_plant = case
    wl = synth.custom(lengths, Hq, Hkv, d, dtype=dt, obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget,
                      n_plant=n_plant, name=name)
    x, _ = run_and_check(wl)
    run_and_check(wl, two_pass=True, inputs=x)
    if stream_supported(wl):
        run_and_check(wl, stream=True, inputs=x)
        if wl.group * wl.obs_window <= 32:  # the default there is the one-read kernel
            run_and_check(wl, fused=True, inputs=x)


# Fused scoring over several grid iterations of 256 workgroups (rows the streaming kernel does
# not take: 128-byte rows, or more than 256 query rows per KV head): segments of 32, 64 and 16
# items (3 requests, 8 row chunks of 32 rows), and of 243 items (one per iteration), are laid
# out so that none crosses an iteration boundary.
PACKED = [
    # name, lengths, Hq, Hkv, d, dtype, w, K_pool, ratio, budget, n_plant
    ("packed_varlen_chunks8_d64", [8000, 16000, 4000], 32, 4, 64, "bf16", 32, 7, 0.05, None, 8),
    ("packed_one_segment_per_iteration", [40000], 64, 2, 128, "bf16", 9, 7, 0.05, None, 8),
]


def _launched_kernels(fn):
    """Kernel ids that fn's library calls launched (through the library's kernel trace)."""
    lib = _snap().load()
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    n = 64
    ev = (ctypes.c_void_p * (2 * n))()
    for i in range(2 * n):
        h = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(h)) == 0
        ev[i] = h
    try:
        assert lib.snapkv_trace_begin(ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)), n) == 0
        fn()
        ids = (ctypes.c_int32 * n)()
        count = lib.snapkv_trace_end(ids, n)
        torch.cuda.synchronize()
    finally:
        for i in range(2 * n):
            hip.hipEventDestroy(ev[i])
    return [int(ids[i]) for i in range(min(count, n))]


@pytest.mark.parametrize("case", PACKED, ids=[c[0] for c in PACKED])
def test_fused_packed_iterations(case):
    name, lengths, Hq, Hkv, d, dt, w, kp, ratio, budget, n_plant = case
    wl = synth.custom(lengths, Hq, Hkv, d, dtype=dt, obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget,
                      n_plant=n_plant, name=name)
    x = synth.make_inputs(wl, 0, threads=16)
    snap = _snap()
    q, K = to_torch(x["q_obs"]), to_torch(x["K"])
    kw = dict(obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget)
    ids = _launched_kernels(lambda: snap.scores(q, K, x["cu_seqlens"], **kw))
    assert 1 in ids and 2 not in ids and 15 not in ids, "expected the fused scoring kernel, launched %s" % ids
    run_and_check(wl, inputs=x)


# The streaming two-phase kernel: grouped-query heads of 64 to 256 rows, several requests,
# slabs of 256 to 1024 keys, more items than one pass of the grid, the prefix-only variant, a
# request shorter than a step, and MHA forced onto it.
STREAM = [
    # name, lengths, Hq, Hkv, d, dtype, w, K_pool, ratio, budget, n_plant, variant
    ("stream_gqa_M256_many_items", [40000, 7000, 129], 32, 8, 128, "bf16", 64, 7, None, 2048, 16, 0),
    ("stream_gqa_M128_varlen", [3000, 33, 16000, 9000, 700], 32, 8, 128, "bf16", 32, 7, 0.05, None, 16, 0),
    ("stream_mha_long", [120000], 8, 8, 128, "bf16", 32, 13, 0.05, None, 64, 0),
    ("stream_gqa_M64_f32", [5000, 12000], 4, 2, 64, "f32", 32, 7, 0.05, None, 8, 0),
    ("stream_prefix_only_M96", [7000, 1000], 6, 2, 128, "bf16", 16, 5, 0.1, None, 8, 1),
    ("stream_many_requests", [40 + 97 * i for i in range(40)], 8, 2, 128, "bf16", 16, 3, 0.2, None, 2, 0),
]


@pytest.mark.parametrize("case", STREAM, ids=[c[0] for c in STREAM])
def test_stream_kernel(case):
    name, lengths, Hq, Hkv, d, dt, w, kp, ratio, budget, n_plant, variant = case
    wl = synth.custom(lengths, Hq, Hkv, d, dtype=dt, obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget,
                      n_plant=n_plant, name=name)
    x = synth.make_inputs(wl, 0, threads=16)
    snap = _snap()
    q, K = to_torch(x["q_obs"]), to_torch(x["K"])
    kw = dict(obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget, variant=variant)
    mha = Hq == Hkv  # MHA takes the one-read kernel unless the two-phase one is asked for
    ids = _launched_kernels(lambda: snap.scores(q, K, x["cu_seqlens"], stream=mha, **kw))
    assert 15 in ids and 1 not in ids, "expected the streaming scoring kernel, launched %s" % ids
    run_and_check(wl, variant=variant, inputs=x)
    run_and_check(wl, variant=variant, stream=True, inputs=x)


# The one-read streaming kernel (the default for up to 32 rows of 256 bytes per KV head when a
# layer's 2048-key items fit one pass of the 256 resident workgroups):
# segments that merge per item (at most 32 items) and through the published shifts (more:
# 40000 tokens are 20 items, 70000 are 35),
# ragged slab tails, a request shorter than one step, a request with an empty prefix, grouped
# heads of 15 and 32 rows, fp32, the prefix-only variant, and a segment of 245 items (near the
# 256 workgroups the MI355X keeps resident).
ONEPASS = [
    # name, lengths, Hq, Hkv, d, dtype, w, K_pool, ratio, budget, n_plant, variant
    ("onepass_mha_ragged", [5000, 1024, 2100, 40], 8, 8, 128, "bf16", 32, 7, 0.05, None, 16, 0),
    ("onepass_central_merge", [70000, 66000, 900], 2, 2, 128, "bf16", 32, 13, 0.05, None, 32, 0),
    ("onepass_empty_prefix", [32, 3000, 64], 4, 4, 128, "bf16", 32, 7, 0.1, None, 4, 0),
    ("onepass_gqa_M15", [4000, 900], 6, 2, 128, "bf16", 5, 3, 0.1, None, 8, 0),
    ("onepass_gqa_M32_f32_d64", [6000], 4, 2, 64, "f32", 16, 7, None, 200, 8, 0),
    ("onepass_prefix_only", [9000, 1500], 4, 4, 128, "bf16", 32, 7, 0.05, None, 8, 1),
    ("onepass_245_items", [500000], 1, 1, 128, "bf16", 32, 7, 0.05, None, 64, 0),
    ("onepass_32_items_self_merge", [65536, 65537], 2, 2, 128, "bf16", 32, 7, 0.05, None, 16, 0),
]


@pytest.mark.parametrize("case", ONEPASS, ids=[c[0] for c in ONEPASS])
def test_onepass_kernel(case):
    name, lengths, Hq, Hkv, d, dt, w, kp, ratio, budget, n_plant, variant = case
    wl = synth.custom(lengths, Hq, Hkv, d, dtype=dt, obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget,
                      n_plant=n_plant, name=name)
    x = synth.make_inputs(wl, 0, threads=16)
    snap = _snap()
    q, K = to_torch(x["q_obs"]), to_torch(x["K"])
    kw = dict(obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget, variant=variant)
    ids = _launched_kernels(lambda: snap.scores(q, K, x["cu_seqlens"], **kw))
    assert 16 in ids and 1 not in ids and 15 not in ids, "expected the one-read scoring kernel, launched %s" % ids
    run_and_check(wl, variant=variant, inputs=x)
    run_and_check(wl, variant=variant, token_major=True, inputs=x)


# The one-read kernel with two items in flight per workgroup (the default for up to 32 rows of
# 256 bytes per KV head when a layer's 2048-key items exceed one pass of the resident grid and
# no segment has more than twice the grid's 1024-key items): segments merged per item (at most
# 32 items) and through the published shifts, mixed in one launch, grouped heads of 32 rows,
# fp32, the prefix-only variant, a request with an empty prefix, and a segment of exactly twice
# the grid's items (the longest it takes; one token more goes to the two-phase kernel).
ONEPASS2 = [
    # name, lengths, Hq, Hkv, d, dtype, w, K_pool, ratio, budget, n_plant, variant
    ("onepass2_central_merge", [300000], 2, 2, 128, "bf16", 32, 13, 0.05, None, 64, 0),
    ("onepass2_self_merge", [30000, 20000, 25000, 9000, 33, 1500], 8, 8, 128, "bf16", 32, 7, 0.05, None, 16, 0),
    ("onepass2_mixed", [45000, 3000, 20000, 700], 8, 8, 128, "bf16", 32, 7, 0.05, None, 16, 0),
    ("onepass2_gqa_M32", [70000, 3000], 16, 8, 128, "bf16", 16, 7, 0.05, None, 16, 0),
    ("onepass2_f32_d64", [40000, 30000], 8, 8, 64, "f32", 32, 5, None, 1000, 16, 0),
    ("onepass2_prefix_only", [70000, 1500, 32], 8, 8, 128, "bf16", 32, 7, 0.05, None, 16, 1),
    # 64 requests in two groups of 32: ~12 items per workgroup from segments of 1 to 39 items,
    # per-item and central merging interleaved in every workgroup
    ("onepass2_many_segments", [700 + (i * 7919) % 39000 for i in range(64)], 8, 8, 128, "bf16", 32, 7, 0.05, None,
     4, 0),
]


def _device_cus():
    return int(torch.cuda.get_device_properties(0).multi_processor_count)


def _check_onepass2(name, lengths, Hq, Hkv, d, dt, w, kp, ratio, budget, n_plant, variant, expect=17):
    wl = synth.custom(lengths, Hq, Hkv, d, dtype=dt, obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget,
                      n_plant=n_plant, name=name)
    x = synth.make_inputs(wl, 0, threads=16)
    snap = _snap()
    q, K = to_torch(x["q_obs"]), to_torch(x["K"])
    kw = dict(obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget, variant=variant)
    ids = _launched_kernels(lambda: snap.scores(q, K, x["cu_seqlens"], **kw))
    assert expect in ids and 16 not in ids and 1 not in ids, "expected scoring kernel %d, launched %s" % (expect, ids)
    run_and_check(wl, variant=variant, inputs=x)
    if expect == 17:
        run_and_check(wl, variant=variant, token_major=True, inputs=x)


@pytest.mark.parametrize("case", ONEPASS2, ids=[c[0] for c in ONEPASS2])
def test_onepass2_kernel(case):
    _check_onepass2(*case)


@pytest.mark.parametrize("extra", [0, 1], ids=["twice_the_grid", "one_token_more"])
def test_onepass2_segment_limit(extra):
    """A segment of 2 * grid 1024-key items takes the two-slot kernel; one token more, the
    two-phase streaming kernel (a segment must fit in both slots of the resident grid)."""
    L = 2 * _device_cus() * 1024 + extra
    _check_onepass2("onepass2_limit_%d" % extra, [L], 2, 2, 128, "bf16", 32, 7, 0.05, None, 64, 0,
                    expect=17 if extra == 0 else 15)


# Segment lengths around every register-run size of the select kernel (4, 8, 16, 32
# positions per thread of 1024), past the 32768 positions it holds on chip, and around the
# tile kernel's 8192-position tiles (an exact multiple, a last tile of one position, one
# position short of a tile boundary).
SELECT_P = [1, 2, 3, 4096, 4097, 8192, 8193, 16384, 16385, 32768, 32769, 49152, 57345, 65535, 70001]


@pytest.mark.parametrize("one_wg", [False, True], ids=["split", "one_wg"])
@pytest.mark.parametrize("levels", [0, 3, 50])
def test_select_exact_on_crafted_votes(levels, one_wg):
    """snapkv_select on given non-negative values equals the oracle's select exactly: heavy
    ties (few distinct levels), exact zeros and negative zeros (which order as +0).  Both
    kernels for segments of up to 32768 positions: split over 8192-position workgroups (with
    three levels a 32768-position segment has about 11000 candidates in the pivot bin, more than
    the 8192 a workgroup holds in LDS) and one workgroup per segment."""
    snap = _snap()
    w = 4
    lengths = [p + w for p in SELECT_P]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, Hkv, d = int(cu[-1]), 2, 64
    q = torch.zeros((len(lengths), 2, w, d), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((Hkv, T, d), dtype=torch.bfloat16, device="cuda")
    rng = np.random.default_rng(1234 + levels)
    sum_P = sum(SELECT_P)
    if levels == 0:
        vals = rng.random((Hkv, sum_P)).astype(np.float32) * np.float32(1e-3)
    else:
        vals = (rng.integers(0, levels, (Hkv, sum_P)) / levels).astype(np.float32)
    vals[:, rng.integers(0, sum_P, 100)] = np.float32(-0.0)
    vals[:, rng.integers(0, sum_P, 100)] = np.float32(0.0)
    pooled = torch.from_numpy(vals).cuda()
    for kw in (dict(ratio=0.37), dict(budget=1), dict(budget=4097), dict(ratio=1.0)):
        _say("select levels=%d one_wg=%s %s" % (levels, one_wg, kw))
        spec = snap.make_spec(q, K, cu, w, 7, kw.get("ratio"), kw.get("budget"))
        ids = _launched_kernels(lambda: snap.select(pooled, q, K, cu, obs_window=w, pool_kernel=7,
                                                    select_one_wg=one_wg, **kw))
        assert (6 if one_wg else 19) in ids and (19 if one_wg else 6) not in ids, "launched %s" % ids
        idx = snap.select(pooled, q, K, cu, obs_window=w, pool_kernel=7, select_one_wg=one_wg, **kw)
        torch.cuda.synchronize()
        idx = idx.cpu().numpy()
        pfx = np.concatenate([[0], np.cumsum(SELECT_P)])
        for r, P in enumerate(SELECT_P):
            k = int(spec.k[r])
            for g in range(Hkv):
                seg = vals[g, pfx[r]:pfx[r + 1]].astype(np.float64) + 0.0  # -0 -> +0
                got = idx[g, int(spec.cu_k[r]):int(spec.cu_k[r + 1])]
                np.testing.assert_array_equal(got.astype(np.int64), oracle.select(seg, k).astype(np.int64),
                                              err_msg="P=%d k=%d g=%d %s" % (P, k, g, kw))


# The split select (taken when a launch group has a segment of more than 16384 positions)
# against one workgroup per segment through the whole call (pooling fused into the select):
# bit-identical pooled votes and indices.  Segments of one chunk beside a longer one, a ragged
# last chunk, exactly 4 chunks, a batch mixing them with a segment for the tile kernel, grouped
# heads, a wide pool window (half-width 16, the widest either kernel pools), budget mode, and
# requests with an empty prefix, with k = 0 (8 positions) and with k = P (1 position), and a
# grid large enough for the 512-thread workgroups.
SPLIT_CASES = [
    # name, lengths, Hq, Hkv, d, w, K_pool, ratio, budget
    ("split_one_chunk", [20000, 2000, 600, 32], 4, 4, 64, 32, 7, 0.05, None),
    ("split_ragged", [9000, 20001], 4, 2, 64, 16, 7, 0.05, None),
    ("split_4_chunks", [32768 + 32], 2, 2, 64, 32, 7, 0.1, None),
    ("split_with_tiles", [40000, 5000, 32768 + 32, 40], 4, 2, 64, 32, 13, 0.05, None),
    ("split_pool33", [20000, 3000], 4, 4, 64, 16, 33, 0.05, None),
    ("split_budget", [7000, 25000, 33], 8, 2, 64, 32, 7, None, 1000),
    # 320 workgroups: past one 1024-thread workgroup per CU, so the 512-thread kernel runs
    ("split_512_threads", [20000] * 12 + [3000] * 4, 8, 8, 64, 32, 7, 0.05, None),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_select_matches_one_workgroup(case):
    name, lengths, Hq, Hkv, d, w, kp, ratio, budget = case
    wl = synth.custom(lengths, Hq, Hkv, d, obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget, n_plant=8,
                      name=name)
    x = synth.make_inputs(wl, 0, threads=16)
    snap = _snap()
    q, K, V = to_torch(x["q_obs"]), to_torch(x["K"]), to_torch(x["V"])
    kw = dict(obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget, want_pooled=True)
    _say("split select %s" % name)
    ids = _launched_kernels(lambda: snap.compress(q, K, V, x["cu_seqlens"], **kw))
    assert 19 in ids and 6 not in ids, "expected the split select, launched %s" % ids
    a = snap.compress(q, K, V, x["cu_seqlens"], **kw)
    b = snap.compress(q, K, V, x["cu_seqlens"], select_one_wg=True, **kw)
    torch.cuda.synchronize()
    for key in ("pooled", "idx", "K_out", "V_out"):
        assert torch.equal(a[key], b[key]), "%s: %s differs between the two select kernels" % (name, key)
    run_and_check(wl, inputs=x)


LSE_CASES = [
    # name, lengths, Hq, Hkv, d, dtype, w, K_pool, ratio, budget, variant
    ("lse_mha_bf16_d128", [3000, 1200], 4, 4, 128, "bf16", 32, 7, 0.05, None, 0),
    ("lse_gqa_chunks", [2600], 16, 2, 64, "bf16", 16, 5, 0.05, None, 0),
    ("lse_prefix_only", [2100, 64], 8, 2, 128, "bf16", 32, 7, 0.1, None, 1),
    ("lse_f32_d64", [1500], 4, 2, 64, "f32", 32, 7, None, 90, 0),
]


@pytest.mark.parametrize("case", LSE_CASES, ids=[c[0] for c in LSE_CASES])
def test_lse_fed_single_pass(case):
    """snapkv_scores_lse / snapkv_compress_lse with each row's log-sum-exp from the oracle
    (rounded to float32) give the oracle's votes, pooled votes, selection and gather."""
    name, lengths, Hq, Hkv, d, dt, w, kp, ratio, budget, variant = case
    snap = _snap()
    wl = synth.custom(lengths, Hq, Hkv, d, dtype=dt, obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget,
                      n_plant=8, name=name)
    _say("case %s" % name)
    x = synth.make_inputs(wl)
    cu = x["cu_seqlens"]
    lse_ref = oracle.lse_all(x["q_obs"], x["K"], cu, w, variant)
    lse = torch.from_numpy(lse_ref.astype(np.float32)).cuda()
    q, K, V = to_torch(x["q_obs"]), to_torch(x["K"]), to_torch(x["V"])
    kw = dict(obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget, variant=variant)
    votes, pooled = snap.scores(q, K, cu, lse=lse, **kw)
    res = snap.compress(q, K, V, cu, lse=lse, want_pooled=True, **kw)
    torch.cuda.synchronize()
    spec = snap.make_spec(q, K, cu, w, kp, ratio, budget, variant)
    ref = oracle.compress(x["q_obs"], x["K"], x["V"], cu, w, kp, ratio=ratio, budget=budget, variant=variant,
                          with_gather=False)
    votes, pooled_c = votes.cpu().numpy(), res["pooled"].cpu().numpy()
    idx = res["idx"].cpu().numpy()
    K_out = to_numpy_bits(res["K_out"])
    for (r, g), rr in sorted(ref.items()):
        t0, t1 = int(cu[r]), int(cu[r + 1])
        P, k = t1 - t0 - w, rr["k"]
        tag = "%s r=%d g=%d" % (name, r, g)
        cols = slice(int(spec.cu_pfx[r]), int(spec.cu_pfx[r + 1]))
        check_scores(votes[g, cols], rr["votes"], tag + " votes")
        check_scores(pooled_c[g, cols], rr["pooled"], tag + " pooled")
        ig = idx[g, int(spec.cu_k[r]):int(spec.cu_k[r + 1])]
        check_selection(ig, rr["pooled"], rr["idx"], k, tag + " select")
        check_select_exact(ig, pooled_c[g, cols], k, tag + " select-exact")
        check_gather(x["K"][g, t0:t1], K_out[g, int(spec.cu_out[r]):int(spec.cu_out[r + 1])], ig, P, w, tag + " gather")


@pytest.mark.parametrize("lengths", [[3000, 40, 1200], [70000], [3000, 32, 70000]],
                         ids=["short", "long", "mixed_with_empty_prefix"])
def test_hit_rate_matches_oracle(lengths):
    """snapkv_hit_rate counts per (request, KV head) give the oracle's Hit Rate exactly: random
    attention with values exactly at theta (as float32) and next to it, and a selection from
    the compression path itself."""
    snap = _snap()
    w, Hkv = 32, 2
    wl = synth.custom(lengths, 4, Hkv, 64, obs_window=w, pool_kernel=7, ratio=0.05, n_plant=4, name="hit")
    x = synth.make_inputs(wl)
    cu = x["cu_seqlens"]
    q, K, V = to_torch(x["q_obs"]), to_torch(x["K"]), to_torch(x["V"])
    res = snap.compress(q, K, V, cu, obs_window=w, pool_kernel=7, ratio=0.05)
    spec = snap.make_spec(q, K, cu, w, 7, 0.05, None)
    rng = np.random.default_rng(11)
    a = (rng.random((Hkv, spec.sum_P)) * 0.1).astype(np.float32)
    theta = 0.05
    t32 = np.float32(theta)
    a.ravel()[rng.integers(0, a.size, 500)] = t32                       # exactly theta in float32
    a.ravel()[rng.integers(0, a.size, 500)] = np.nextafter(t32, np.float32(1))
    a.ravel()[rng.integers(0, a.size, 500)] = np.nextafter(t32, np.float32(0))
    counts = snap.hit_rate_counts(torch.from_numpy(a).cuda(), res["idx"], q, K, cu, obs_window=w, pool_kernel=7,
                                  ratio=0.05, theta=theta)
    torch.cuda.synchronize()
    counts = counts.cpu().numpy().view(np.uint32)
    idx = res["idx"].cpu().numpy()
    for r in range(len(lengths)):
        P = lengths[r] - w
        for g in range(Hkv):
            seg = a[g, int(spec.cu_pfx[r]):int(spec.cu_pfx[r + 1])]
            mask = np.zeros(P, np.uint8)
            mask[idx[g, int(spec.cu_k[r]):int(spec.cu_k[r + 1])]] = 1
            ref = oracle.hit_rate(seg, mask, theta)
            hits, above = int(counts[r, g, 0]), int(counts[r, g, 1])
            assert above == int(np.sum(seg.astype(np.float64) > theta)), (r, g)
            if above == 0:
                assert np.isnan(ref)
            else:
                assert hits / above == ref, (r, g, hits, above, ref)


def test_hit_rate_beyond_one_bitmap_span():
    """A segment of more than 2^20 positions (33 tiles; kept positions near 2^20)."""
    snap = _snap()
    w, Hkv, P = 8, 1, (1 << 20) + 5000
    cu = np.array([0, P + w], np.int32)
    q = torch.zeros((1, 1, w, 64), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((Hkv, P + w, 64), dtype=torch.bfloat16, device="cuda")
    spec = snap.make_spec(q, K, cu, w, 7, None, 4000)
    rng = np.random.default_rng(12)
    keep = np.sort(np.concatenate([rng.choice(P, 3990, replace=False),
                                   [(1 << 20) - 2, (1 << 20) - 1, 1 << 20, (1 << 20) + 1, 0, P - 1]]))
    keep = np.unique(keep)[:4000]
    keep = np.sort(np.concatenate([keep, np.setdiff1d(np.arange(P), keep)[:4000 - keep.size]]))
    idx = torch.from_numpy(keep.astype(np.int32)[None, :]).cuda()
    a = (rng.random((Hkv, P)) * 0.1).astype(np.float32)
    counts = snap.hit_rate_counts(torch.from_numpy(a).cuda(), idx, q, K, cu, obs_window=w, pool_kernel=7,
                                  budget=4000, theta=0.05)
    torch.cuda.synchronize()
    hits, above = (int(v) for v in counts.cpu().numpy().view(np.uint32)[0, 0])
    mask = np.zeros(P, np.uint8)
    mask[keep] = 1
    assert above == int(np.sum(a[0].astype(np.float64) > 0.05))
    assert hits / above == oracle.hit_rate(a[0], mask, 0.05)


def test_hit_rate_large_selection():
    """k above four tiles of positions: each tile finds its run of the ascending idx by
    binary search (kept positions on both sides of every tile edge)."""
    snap = _snap()
    w, Hkv, P, k, tile = 8, 1, 300000, 200000, 32768
    cu = np.array([0, P + w], np.int32)
    q = torch.zeros((1, 1, w, 64), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((Hkv, P + w, 64), dtype=torch.bfloat16, device="cuda")
    rng = np.random.default_rng(13)
    edges = np.array([e + o for e in range(tile, P, tile) for o in (-1, 0)] + [0, P - 1])
    rest = np.setdiff1d(np.arange(P), edges)
    keep = np.sort(np.concatenate([edges, rng.choice(rest, k - edges.size, replace=False)]))
    idx = torch.from_numpy(keep.astype(np.int32)[None, :]).cuda()
    a = (rng.random((Hkv, P)) * 0.1).astype(np.float32)
    counts = snap.hit_rate_counts(torch.from_numpy(a).cuda(), idx, q, K, cu, obs_window=w, pool_kernel=7,
                                  budget=k, theta=0.05)
    torch.cuda.synchronize()
    hits, above = (int(v) for v in counts.cpu().numpy().view(np.uint32)[0, 0])
    mask = np.zeros(P, np.uint8)
    mask[keep] = 1
    assert above == int(np.sum(a[0].astype(np.float64) > 0.05))
    assert hits / above == oracle.hit_rate(a[0], mask, 0.05)


# ---- decode attention over the compressed cache ------------------------------------------------

DECODE_CASES = [
    # name, lengths, Hq, Hkv, d, dtype, w, ratio
    ("dec_mha_bf16", [3000, 1400], 4, 4, 128, "bf16", 32, 0.2),
    ("dec_gqa4_bf16", [9000], 8, 2, 128, "bf16", 32, 0.3),     # several splits per head
    ("dec_gqa3_bf16", [2000, 700], 6, 2, 128, "bf16", 16, 0.5),  # 3 heads per KV head (tile of 4)
    ("dec_gqa16_bf16", [1500], 16, 1, 128, "bf16", 8, 0.5),    # two head tiles of 8
    ("dec_f32_d64", [1800, 64], 4, 2, 64, "f32", 32, 0.4),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_over_compressed_cache(case):
    """snapkv_decode over snapkv_compress's K_out/V_out equals the oracle's decode attention
    over the same rows (fp32 accumulation: |gpu - ref| <= 1e-4 |ref| + 1e-5)."""
    name, lengths, Hq, Hkv, d, dt, w, ratio = case
    snap = _snap()
    wl = synth.custom(lengths, Hq, Hkv, d, dtype=dt, obs_window=w, pool_kernel=7, ratio=ratio, n_plant=4, name=name)
    _say("case %s" % name)
    x = synth.make_inputs(wl)
    q, K, V = to_torch(x["q_obs"]), to_torch(x["K"]), to_torch(x["V"])
    res = snap.compress(q, K, V, x["cu_seqlens"], obs_window=w, pool_kernel=7, ratio=ratio)
    rng = np.random.default_rng(30)
    qd = rng.standard_normal((len(lengths), Hq, d)).astype(np.float32) * 2
    qd = synth.round_bf16(qd) if dt == "bf16" else qd
    out = snap.decode(to_torch(qd), res["K_out"], res["V_out"], res["cu_out"])
    torch.cuda.synchronize()
    ref = oracle.decode_all(qd, to_numpy_bits(res["K_out"]), to_numpy_bits(res["V_out"]), res["cu_out"])
    np.testing.assert_allclose(out.cpu().numpy(), ref, rtol=1e-4, atol=1e-5)


def test_decode_empty_request_and_token_major_cache():
    """A request with no cached rows gets zeros; a token-major cache view gives the same result."""
    snap = _snap()
    rng = np.random.default_rng(31)
    Hq, Hkv, d, T = 4, 2, 128, 700
    cu = np.array([0, 300, 300, 700], np.int64)
    Kn = synth.round_bf16(rng.standard_normal((Hkv, T, d)).astype(np.float32))
    Vn = synth.round_bf16(rng.standard_normal((Hkv, T, d)).astype(np.float32))
    qn = synth.round_bf16(rng.standard_normal((3, Hq, d)).astype(np.float32))
    K, V, q = to_torch(Kn), to_torch(Vn), to_torch(qn)
    out = snap.decode(q, K, V, cu).cpu().numpy()
    Kt = K.transpose(0, 1).contiguous().transpose(0, 1)
    Vt = V.transpose(0, 1).contiguous().transpose(0, 1)
    out_t = snap.decode(q, Kt, Vt, cu).cpu().numpy()
    torch.cuda.synchronize()
    ref = oracle.decode_all(qn, Kn, Vn, cu)
    assert not out[1].any()
    np.testing.assert_allclose(out, ref, rtol=1e-4, atol=1e-5)
    np.testing.assert_array_equal(out, out_t)


def test_prefix_only_variant():
    wl = synth.custom([3000, 1500], 8, 2, 128, obs_window=32, pool_kernel=7, ratio=0.05, n_plant=8,
                      name="prefix_only")
    x, _ = run_and_check(wl, variant=1)
    run_and_check(wl, variant=1, two_pass=True, inputs=x)
    run_and_check(wl, variant=1, stream=True, inputs=x)


def test_token_major_layout():
    wl = synth.custom([2100, 900], 8, 4, 128, obs_window=16, pool_kernel=7, ratio=0.05, n_plant=4,
                      name="token_major")
    run_and_check(wl, token_major=True)


def test_keep_everything_is_bit_exact_copy():
    """ratio = 1 (and budget >= P): the output is the input, bit for bit."""
    snap = _snap()
    wl = synth.custom([700, 1300], 4, 2, 128, obs_window=32, pool_kernel=7, ratio=1.0, name="keep_all")
    x = synth.make_inputs(wl)
    q, K, V = to_torch(x["q_obs"]), to_torch(x["K"]), to_torch(x["V"])
    for kw in (dict(ratio=1.0), dict(budget=10 ** 6)):
        res = snap.compress(q, K, V, x["cu_seqlens"], obs_window=32, pool_kernel=7, **kw)
        torch.cuda.synchronize()
        assert to_numpy_bits(res["K_out"]).tobytes() == x["K"].tobytes()
        assert to_numpy_bits(res["V_out"]).tobytes() == x["V"].tobytes()


def test_window_only_and_zero_k():
    """L_r = L_obs (P = 0) and P > 0 with k = 0: only the window is kept."""
    snap = _snap()
    wl = synth.custom([32, 50, 32], 4, 4, 64, obs_window=32, pool_kernel=7, ratio=0.05, name="window_only")
    x = synth.make_inputs(wl)
    q, K, V = to_torch(x["q_obs"]), to_torch(x["K"]), to_torch(x["V"])
    res = snap.compress(q, K, V, x["cu_seqlens"], obs_window=32, pool_kernel=7, ratio=0.05)
    torch.cuda.synchronize()
    assert list(res["k"]) == [0, 0, 0]
    ko = to_numpy_bits(res["K_out"])
    cu = x["cu_seqlens"]
    for r in range(3):
        exp = x["K"][:, cu[r + 1] - 32:cu[r + 1]]
        assert ko[:, 32 * r:32 * (r + 1)].tobytes() == np.ascontiguousarray(exp).tobytes()


def test_batch_larger_than_one_launch_group():
    lengths = [40 + 37 * i for i in range(40)]
    wl = synth.custom(lengths, 4, 2, 64, obs_window=8, pool_kernel=3, ratio=0.2, n_plant=2, name="batch40")
    run_and_check(wl)


def test_deterministic():
    snap = _snap()
    wl = synth.custom([6000, 3000], 8, 2, 128, obs_window=32, pool_kernel=7, ratio=0.05, n_plant=16, name="det")
    x = synth.make_inputs(wl)
    q, K, V = to_torch(x["q_obs"]), to_torch(x["K"]), to_torch(x["V"])
    a = snap.compress(q, K, V, x["cu_seqlens"], obs_window=32, pool_kernel=7, ratio=0.05, want_pooled=True)
    b = snap.compress(q, K, V, x["cu_seqlens"], obs_window=32, pool_kernel=7, ratio=0.05, want_pooled=True)
    torch.cuda.synchronize()
    assert torch.equal(a["idx"], b["idx"]) and torch.equal(a["pooled"], b["pooled"])
    assert torch.equal(a["K_out"], b["K_out"]) and torch.equal(a["V_out"], b["V_out"])


# One workspace across calls on different inputs of one shape: every counter, flag and tagged
# slot a call uses must be back at zero for the next call, or the next call's votes come out
# wrong (stale row stats would be taken as this call's).
WS_REUSE = [
    # name, lengths, Hq, Hkv, flags
    ("onepass_short_segments", [20000, 7000], 4, 4, {}),
    ("onepass_long_segment", [80000], 2, 2, {}),
    ("onepass2_two_slots", [300000, 40000, 5000], 2, 2, {}),
    ("stream_gqa", [20000, 7000], 16, 4, {}),
    ("stream_mha_forced", [30000], 4, 4, {"stream": True}),
    ("fused_forced", [20000, 3000], 4, 4, {"fused": True}),
]


@pytest.mark.parametrize("case", WS_REUSE, ids=[c[0] for c in WS_REUSE])
def test_workspace_reuse_across_inputs(case):
    name, lengths, Hq, Hkv, flags = case
    snap = _snap()
    wl = synth.custom(lengths, Hq, Hkv, 128, obs_window=32, pool_kernel=7, ratio=0.05, n_plant=8, name=name)
    ws = None
    for layer in (0, 1, 0):
        _say("case %s layer %d" % (name, layer))
        x = synth.make_inputs(wl, layer, threads=16)
        q, K, V = to_torch(x["q_obs"]), to_torch(x["K"]), to_torch(x["V"])
        cu = x["cu_seqlens"]
        spec = snap.make_spec(q, K, cu, 32, 7, 0.05, None, **flags)
        if ws is None:
            ws = snap.workspace(spec, K.device)
        res = snap.compress(q, K, V, cu, obs_window=32, pool_kernel=7, ratio=0.05, want_pooled=True, ws=ws, **flags)
        torch.cuda.synchronize()
        ref = oracle.compress(x["q_obs"], x["K"], x["V"], cu, 32, 7, ratio=0.05, with_gather=False)
        pooled, idx = res["pooled"].cpu().numpy(), res["idx"].cpu().numpy()
        for (r, g), rr in sorted(ref.items()):
            tag = "%s layer %d r=%d g=%d" % (name, layer, r, g)
            cols = slice(int(spec.cu_pfx[r]), int(spec.cu_pfx[r + 1]))
            check_scores(pooled[g, cols], rr["pooled"], tag + " pooled")
            check_selection(idx[g, int(spec.cu_k[r]):int(spec.cu_k[r + 1])], rr["pooled"], rr["idx"], rr["k"],
                            tag + " select")


# One workspace across problems of different shapes: each call's counters and tagged slots
# lie where the previous call may have written votes or indices, so a call on a workspace last
# used with another layout clears its own control regions first.  Every call must give the
# same bits as the same call on a fresh zero-filled workspace.
RESHAPE = [
    # lengths, Hq, Hkv, flags: two-slot one-read (tile select past 32768 positions), two-phase
    # stream (GQA), one-read, fused (forced), then the first again
    ([300000, 40000], 2, 2, {}),
    ([20000, 7000], 16, 4, {}),
    ([9000, 3000], 4, 4, {}),
    ([3000, 1800], 8, 2, {"fused": True}),
    ([300000, 40000], 2, 2, {}),
]


def test_workspace_reuse_across_shapes():
    snap = _snap()
    cases = []
    for n, (lengths, Hq, Hkv, flags) in enumerate(RESHAPE):
        wl = synth.custom(lengths, Hq, Hkv, 128, obs_window=32, pool_kernel=7, ratio=0.05, n_plant=8,
                          name="reshape%d" % n)
        x = synth.make_inputs(wl, n % 2, threads=16)
        q, K, V = to_torch(x["q_obs"]), to_torch(x["K"]), to_torch(x["V"])
        spec = snap.make_spec(q, K, x["cu_seqlens"], 32, 7, 0.05, None, **flags)
        cases.append((q, K, V, x["cu_seqlens"], flags, spec.ws_bytes))
    shared = torch.zeros(max(c[5] for c in cases), dtype=torch.uint8, device="cuda")
    kw = dict(obs_window=32, pool_kernel=7, ratio=0.05, want_pooled=True)
    for n, (q, K, V, cu, flags, nbytes) in enumerate(cases):
        _say("reshape call %d %s" % (n, RESHAPE[n][:3]))
        fresh = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        ref = snap.compress(q, K, V, cu, ws=fresh, **kw, **flags)
        got = snap.compress(q, K, V, cu, ws=shared[:nbytes], **kw, **flags)
        torch.cuda.synchronize()
        for key in ("pooled", "idx", "K_out", "V_out"):
            assert torch.equal(got[key], ref[key]), "call %d: %s differs from a fresh workspace's" % (n, key)
        assert int(shared[:4].view(torch.int32).item()) == 0


def test_workspace_counters_left_zero():
    """The fused path's barrier counters return to zero after every call, so one
    zero-filled workspace serves any number of calls; the error word stays clear."""
    snap = _snap()
    wl = synth.custom([3000, 1800], 8, 2, 128, obs_window=32, pool_kernel=7, ratio=0.05, n_plant=8, name="ws_reuse")
    x = synth.make_inputs(wl)
    q, K, V = to_torch(x["q_obs"]), to_torch(x["K"]), to_torch(x["V"])
    spec = snap.make_spec(q, K, x["cu_seqlens"], 32, 7, 0.05, None)
    ws = snap.workspace(spec, K.device)
    first = None
    for it in range(3):
        res = snap.compress(q, K, V, x["cu_seqlens"], obs_window=32, pool_kernel=7, ratio=0.05, ws=ws)
        torch.cuda.synchronize()
        # error line (256 B) and one 256-B counter line per (request, KV head) segment
        head = ws[:256 * (1 + len(wl.lengths) * wl.num_kv_heads)].cpu().numpy()
        assert not head.any(), "call %d left a nonzero error word or barrier counter" % it
        if first is None:
            first = res["idx"].clone()
        assert torch.equal(first, res["idx"])


def test_unsupported_rows_raise():
    snap = _snap()
    wl = synth.custom([600], 64, 1, 64, obs_window=17, pool_kernel=7, ratio=0.05, name="too_many_rows")
    x = synth.make_inputs(wl)
    q, K, V = to_torch(x["q_obs"]), to_torch(x["K"]), to_torch(x["V"])
    # G * L_obs = 64 * 17 = 1088 rows per KV head: past the 1024 the scoring kernels take
    with pytest.raises(ValueError, match="1024"):
        snap.compress(q, K, V, x["cu_seqlens"], obs_window=17, pool_kernel=7, ratio=0.05)


# ---- the five standard workloads at full size ------------------------------------------------
# Every (request, KV head) pair of a layer is compared with the oracle, entry by entry, in the
# launch configuration the benchmark times.


def test_workload1_full():
    run_and_check(synth.workload(1))


def test_workload2_full():
    run_and_check(synth.workload(2))


def test_workload3_layers_all_heads():
    """All 8 KV heads (each scoring 4 query heads x 64 window rows) of four of the 32 layers."""
    wl = synth.workload(3)
    for layer in (0, 9, 20, wl.n_layers - 1):
        run_and_check(wl, layer=layer)


def test_workload4_all_heads():
    run_and_check(synth.workload(4))


def test_workload5_all_pairs():
    run_and_check(synth.workload(5))


@pytest.mark.parametrize("n", [2, 4, 5])
def test_lse_fed_full_size(n):
    """snapkv_compress_lse at full size with every window row's log-sum-exp from the oracle
    (rounded to float32): votes, pooled votes, selection and gather of every pair."""
    snap = _snap()
    wl = synth.workload(n)
    _say("case lse-fed %s" % wl.name)
    x = synth.make_inputs(wl, 0, threads=16)
    cu, w = x["cu_seqlens"], wl.obs_window
    lse = torch.from_numpy(oracle.lse_all(x["q_obs"], x["K"], cu, w).astype(np.float32)).cuda()
    q, K, V = to_torch(x["q_obs"]), to_torch(x["K"]), to_torch(x["V"])
    kw = dict(obs_window=w, pool_kernel=wl.pool_kernel, ratio=wl.ratio, budget=wl.budget)
    votes, pooled = snap.scores(q, K, cu, lse=lse, **kw)
    res = snap.compress(q, K, V, cu, lse=lse, want_pooled=True, **kw)
    torch.cuda.synchronize()
    spec = snap.make_spec(q, K, cu, w, wl.pool_kernel, wl.ratio, wl.budget)
    ref = oracle.compress(x["q_obs"], x["K"], x["V"], cu, w, wl.pool_kernel, ratio=wl.ratio, budget=wl.budget,
                          with_gather=False)
    votes, pooled_c = votes.cpu().numpy(), res["pooled"].cpu().numpy()
    np.testing.assert_array_equal(pooled.cpu().numpy(), pooled_c)
    idx = res["idx"].cpu().numpy()
    K_out = to_numpy_bits(res["K_out"])
    for (r, g), rr in sorted(ref.items()):
        t0, t1 = int(cu[r]), int(cu[r + 1])
        P, k = t1 - t0 - w, rr["k"]
        tag = "%s lse r=%d g=%d" % (wl.name, r, g)
        cols = slice(int(spec.cu_pfx[r]), int(spec.cu_pfx[r + 1]))
        check_scores(votes[g, cols], rr["votes"], tag + " votes")
        check_scores(pooled_c[g, cols], rr["pooled"], tag + " pooled")
        ig = idx[g, int(spec.cu_k[r]):int(spec.cu_k[r + 1])]
        check_selection(ig, rr["pooled"], rr["idx"], k, tag + " select")
        check_select_exact(ig, pooled_c[g, cols], k, tag + " select-exact")
        check_gather(x["K"][g, t0:t1], K_out[g, int(spec.cu_out[r]):int(spec.cu_out[r + 1])], ig, P, w,
                     tag + " gather")
