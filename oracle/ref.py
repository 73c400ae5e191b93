"""NumPy wrapper over the fp64 C oracle (``snapkv_oracle.c``) -- TEST INFRASTRUCTURE.

Every function here marshals arrays and calls the C oracle; none of the
method's arithmetic is done in Python.  Citations are to the page
"論文解説: SnapKV — アテンションパターン観測によるKVキャッシュ圧縮"
(0h-n0.github.io/posts/paper-2404-14469/).

Inputs are raw element arrays: float32, or bfloat16 bit patterns held in
uint16 arrays.  The C code widens both to double exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "snapkv_oracle.c")
_LIB = os.path.join(_HERE, "libsnapkv_oracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16 = 0, 1


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (plain -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Job(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("keys", ctypes.c_void_p),
        ("key_stride", ctypes.c_int64),
        ("L", ctypes.c_int64),
        ("n_rows", ctypes.c_int32),
        ("w", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("K_pool", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("variant", ctypes.c_int32),
        ("_pad", ctypes.c_int32),
        ("ratio", ctypes.c_double),
        ("budget", ctypes.c_int64),
        ("votes", ctypes.c_void_p),
        ("pooled", ctypes.c_void_p),
        ("idx", ctypes.c_void_p),
        ("k", ctypes.c_int64),
    ]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # SNAPKV_ORACLE_LIB: a separately built copy of the same source (the sanitizer test
            # builds one with AddressSanitizer and UndefinedBehaviorSanitizer)
            lib = ctypes.CDLL(os.environ.get("SNAPKV_ORACLE_LIB") or build())
            vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
            lib.snapkv_oracle_votes.argtypes = [vp, ctypes.c_int, i64, i32, i32, vp, i64, i64, i32, vp, vp]
            lib.snapkv_oracle_votes.restype = None
            lib.snapkv_oracle_row_lse.argtypes = [vp, ctypes.c_int, i64, i32, i32, vp, i64, i64, i32, vp, vp]
            lib.snapkv_oracle_row_lse.restype = None
            lib.snapkv_oracle_decode.argtypes = [vp, ctypes.c_int, i32, i32, vp, vp, i64, i64, vp, vp]
            lib.snapkv_oracle_decode.restype = None
            lib.snapkv_oracle_pool.argtypes = [vp, i64, i32, vp]
            lib.snapkv_oracle_pool.restype = None
            lib.snapkv_oracle_k.argtypes = [i64, i32, dbl, i64]
            lib.snapkv_oracle_k.restype = i64
            lib.snapkv_oracle_select.argtypes = [vp, i64, i64, vp, vp]
            lib.snapkv_oracle_select.restype = None
            lib.snapkv_oracle_gather.argtypes = [vp, i64, i64, i64, i32, vp, i64, vp]
            lib.snapkv_oracle_gather.restype = None
            lib.snapkv_oracle_hit_rate.argtypes = [vp, vp, i64, dbl]
            lib.snapkv_oracle_hit_rate.restype = dbl
            lib.snapkv_oracle_run_jobs.argtypes = [vp, i64, ctypes.c_int]
            lib.snapkv_oracle_run_jobs.restype = ctypes.c_int
            lib.snapkv_oracle_job_size.restype = ctypes.c_int
            if lib.snapkv_oracle_job_size() != ctypes.sizeof(_Job):
                raise RuntimeError("oracle job struct layout mismatch")
            _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 or bfloat16 bits in uint16, got %s" % a.dtype)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def votes(q: np.ndarray, keys: np.ndarray, w: int, variant: int = 0) -> np.ndarray:
    """Vote of one (request, KV head) over all L positions (section 投票メカニズム).

    q: [G*w, d] window queries of the group, row r = (head r // w, window row r % w).
    keys: [L, d] (row stride may exceed d).  Returns float64 [L]; entries < P are C.
    """
    q = np.ascontiguousarray(q)
    if keys.strides[1] != keys.itemsize:
        keys = np.ascontiguousarray(keys)
    dt = _dtype_code(q)
    assert _dtype_code(keys) == dt and q.shape[1] == keys.shape[1] and q.shape[0] % w == 0
    L = keys.shape[0]
    out = np.empty(L, np.float64)
    row_buf = np.empty(max(L, 1), np.float64)
    _load().snapkv_oracle_votes(_ptr(q), dt, q.shape[0], w, q.shape[1], _ptr(keys),
                                keys.strides[0] // keys.itemsize, L, variant, _ptr(out), _ptr(row_buf))
    return out


def row_lse(q: np.ndarray, keys: np.ndarray, w: int, variant: int = 0) -> np.ndarray:
    """Log-sum-exp of each window row's logits over the keys it sees (the softmax
    denominator of section 投票メカニズム in log form); rows as in votes().  float64 [G*w]."""
    q = np.ascontiguousarray(q)
    if keys.strides[1] != keys.itemsize:
        keys = np.ascontiguousarray(keys)
    dt = _dtype_code(q)
    assert _dtype_code(keys) == dt and q.shape[1] == keys.shape[1] and q.shape[0] % w == 0
    L = keys.shape[0]
    out = np.empty(q.shape[0], np.float64)
    row_buf = np.empty(max(L, 1), np.float64)
    _load().snapkv_oracle_row_lse(_ptr(q), dt, q.shape[0], w, q.shape[1], _ptr(keys),
                                  keys.strides[0] // keys.itemsize, L, variant, _ptr(out), _ptr(row_buf))
    return out


def lse_all(q_obs: np.ndarray, K: np.ndarray, cu_seqlens, w: int, variant: int = 0, n_threads: int = 16) -> np.ndarray:
    """row_lse for every request and query head: float64 [B, H_q, w] (q_obs [B, H_q, w, d],
    K [H_kv, T, d]; query head h reads KV head h // G).  The (request, head) calls run on a
    thread pool (each call is independent)."""
    from concurrent.futures import ThreadPoolExecutor
    B, Hq = q_obs.shape[0], q_obs.shape[1]
    G = Hq // K.shape[0]
    out = np.empty((B, Hq, w), np.float64)

    def one(job):
        r, h = job
        t0, t1 = int(cu_seqlens[r]), int(cu_seqlens[r + 1])
        out[r, h] = row_lse(q_obs[r, h], K[h // G, t0:t1], w, variant)

    jobs = [(r, h) for r in range(B) for h in range(Hq)]
    with ThreadPoolExecutor(max_workers=max(1, n_threads)) as ex:
        list(ex.map(one, jobs))
    return out


def decode(q: np.ndarray, keys: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Decode attention of G query rows q [G, d] over cached rows keys/values [n, d]
    (same dtype): softmax(q k^T / sqrt(d)) v in fp64, [G, d]; zeros when n = 0."""
    q = np.ascontiguousarray(q)
    keys = np.ascontiguousarray(keys)
    values = np.ascontiguousarray(values)
    dt = _dtype_code(q)
    assert _dtype_code(keys) == dt == _dtype_code(values) and keys.shape == values.shape
    G, d = q.shape
    n = keys.shape[0]
    out = np.empty((G, d), np.float64)
    row_buf = np.empty(max(n, 1), np.float64)
    _load().snapkv_oracle_decode(_ptr(q), dt, G, d, _ptr(keys), _ptr(values), d, n, _ptr(out), _ptr(row_buf))
    return out


def decode_all(q: np.ndarray, K: np.ndarray, V: np.ndarray, cu_rows) -> np.ndarray:
    """decode() for every request and KV head: q [B, H_q, d], K/V [H_kv, T, d] with request r
    owning rows cu_rows[r] .. cu_rows[r+1]-1; returns fp64 [B, H_q, d]."""
    B, Hq, d = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    out = np.empty((B, Hq, d), np.float64)
    for r in range(B):
        a, b = int(cu_rows[r]), int(cu_rows[r + 1])
        for g in range(Hkv):
            out[r, g * G:(g + 1) * G] = decode(q[r, g * G:(g + 1) * G], K[g, a:b], V[g, a:b])
    return out


def pool(c: np.ndarray, K_pool: int) -> np.ndarray:
    """Max pooling of width K_pool, stride 1, -inf padding (section クラスタリングによる文脈保持)."""
    c = np.ascontiguousarray(c, dtype=np.float64)
    out = np.empty_like(c)
    if c.size:
        _load().snapkv_oracle_pool(_ptr(c), c.size, K_pool, _ptr(out))
    return out


def k_of(P: int, ratio: float | None = None, budget: int | None = None) -> int:
    """k = floor(ratio * P), or min(budget, P) (section 投票メカニズム; アルゴリズム listing)."""
    if (ratio is None) == (budget is None):
        raise ValueError("exactly one of ratio and budget")
    if ratio is not None:
        return int(_load().snapkv_oracle_k(P, 0, float(ratio), 0))
    return int(_load().snapkv_oracle_k(P, 1, 0.0, int(budget)))


def select(pooled: np.ndarray, k: int) -> np.ndarray:
    """Top-k by (value desc, position asc), returned ascending, int32."""
    pooled = np.ascontiguousarray(pooled, dtype=np.float64)
    P = pooled.size
    idx = np.empty(max(P, 1), np.int32)
    scratch = np.empty(max(P, 1) * 2, np.float64)
    if P:
        _load().snapkv_oracle_select(_ptr(pooled), P, k, _ptr(idx), _ptr(scratch))
    return idx[:k].copy()


def gather(rows: np.ndarray, P: int, w: int, idx: np.ndarray) -> np.ndarray:
    """Rows idx then the w window rows P..P+w-1, bit-exact (アルゴリズム listing)."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    k = idx.size
    out = np.empty((k + w, rows.shape[1]), rows.dtype)
    row_bytes = rows.shape[1] * rows.itemsize
    if rows.strides[1] != rows.itemsize:
        rows = np.ascontiguousarray(rows)
    _load().snapkv_oracle_gather(_ptr(rows), row_bytes, rows.strides[0], P, w, _ptr(idx), k, _ptr(out))
    return out


def hit_rate(a_cur: np.ndarray, vote_mask: np.ndarray, theta: float = 0.05) -> float:
    """H = sum(M_thr AND M_vote) / sum(M_thr), M_thr = 1(a_cur > theta) (section Hit Rate)."""
    a = np.ascontiguousarray(a_cur, dtype=np.float64).ravel()
    m = np.ascontiguousarray(vote_mask, dtype=np.uint8).ravel()
    assert a.size == m.size
    return float(_load().snapkv_oracle_hit_rate(_ptr(a), _ptr(m), a.size, float(theta)))


def compress_head(q: np.ndarray, keys: np.ndarray, values: np.ndarray, w: int, K_pool: int,
                  ratio: float | None = None, budget: int | None = None, variant: int = 0) -> dict:
    """Whole path for one (request, KV head): votes, pool, k, select, gather."""
    L = keys.shape[0]
    P = L - w
    v = votes(q, keys, w, variant)
    c = v[:P]
    pl = pool(c, K_pool)
    k = k_of(P, ratio, budget)
    idx = select(pl, k)
    return dict(votes_full=v, votes=c, pooled=pl, k=k, idx=idx,
                K_out=gather(keys, P, w, idx), V_out=gather(values, P, w, idx))


def _jobs_for(q_obs, K, cu_seqlens, w, K_pool, ratio, budget, variant, pairs):
    """Build C job structs for (request, KV head) pairs over packed [H_kv, T, d] inputs."""
    B, Hq, w_, d = q_obs.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    dt = _dtype_code(K)
    mode = 0 if ratio is not None else 1
    jobs = (_Job * len(pairs))()
    keep = []
    outs = []
    for n, (r, g) in enumerate(pairs):
        t0, t1 = int(cu_seqlens[r]), int(cu_seqlens[r + 1])
        L = t1 - t0
        P = L - w
        qg = np.ascontiguousarray(q_obs[r, g * G:(g + 1) * G].reshape(G * w, d))
        kv = K[g, t0:t1]
        vo = np.empty(L, np.float64)
        po = np.empty(max(P, 1), np.float64)
        io = np.empty(max(P, 1), np.int32)
        keep += [qg, kv]
        outs.append((vo, po, io, P))
        jb = jobs[n]
        jb.q, jb.keys = _ptr(qg), _ptr(kv)
        jb.key_stride = kv.strides[0] // kv.itemsize
        jb.L, jb.n_rows, jb.w, jb.d, jb.dtype = L, G * w, w, d, dt
        jb.K_pool, jb.mode, jb.variant = K_pool, mode, variant
        jb.ratio = float(ratio) if ratio is not None else 0.0
        jb.budget = int(budget) if budget is not None else 0
        jb.votes, jb.pooled, jb.idx = _ptr(vo), _ptr(po), _ptr(io)
    return jobs, keep, outs


def compress(q_obs: np.ndarray, K: np.ndarray, V: np.ndarray, cu_seqlens, w: int, K_pool: int,
             ratio: float | None = None, budget: int | None = None, variant: int = 0,
             pairs=None, n_threads: int = 0, with_gather: bool = True) -> dict:
    """Oracle over packed inputs: q_obs [B, H_q, w, d]; K, V [H_kv, T, d]; cu_seqlens [B+1].

    ``pairs`` restricts the work to a sample of (request, KV head) pairs.  Returns
    {(r, g): dict(votes, pooled, k, idx, K_out, V_out)}.
    """
    if (ratio is None) == (budget is None):
        raise ValueError("exactly one of ratio and budget")
    B = q_obs.shape[0]
    Hkv = K.shape[0]
    if pairs is None:
        pairs = [(r, g) for r in range(B) for g in range(Hkv)]
    jobs, keep, outs = _jobs_for(q_obs, K, cu_seqlens, w, K_pool, ratio, budget, variant, pairs)
    _load().snapkv_oracle_run_jobs(ctypes.cast(jobs, ctypes.c_void_p), len(pairs), n_threads)
    res = {}
    for n, (r, g) in enumerate(pairs):
        vo, po, io, P = outs[n]
        k = int(jobs[n].k)
        item = dict(votes_full=vo, votes=vo[:P], pooled=po[:P], k=k, idx=io[:k].copy())
        if with_gather:
            t0, t1 = int(cu_seqlens[r]), int(cu_seqlens[r + 1])
            item["K_out"] = gather(K[g, t0:t1], P, w, item["idx"])
            item["V_out"] = gather(V[g, t0:t1], P, w, item["idx"])
        res[(r, g)] = item
    del keep
    return res


def run_jobs_timed(q_obs, K, cu_seqlens, w, K_pool, ratio=None, budget=None, pairs=None, n_threads=0):
    """Time the oracle's votes+pool+select over ``pairs``; returns (seconds, threads used)."""
    import time
    B = q_obs.shape[0]
    Hkv = K.shape[0]
    if pairs is None:
        pairs = [(r, g) for r in range(B) for g in range(Hkv)]
    jobs, keep, outs = _jobs_for(q_obs, K, cu_seqlens, w, K_pool, ratio, budget, 0, pairs)
    lib = _load()
    t0 = time.perf_counter()
    used = lib.snapkv_oracle_run_jobs(ctypes.cast(jobs, ctypes.c_void_p), len(pairs), n_threads)
    dt = time.perf_counter() - t0
    del keep, outs
    return dt, int(used)
