"""The C-ABI boundary on the CPU: the library loads, exports every declared symbol,
plans problems as the method fixes k and the offsets, and rejects every invalid
argument before any launch (no GPU work happens in these tests)."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

from kv_cache_compression_amd import _lib, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(snapkv_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _declared_symbols()
    assert set(_lib.SYMBOLS) == set(declared)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.snapkv_version() == 100
    assert lib.snapkv_strerror(-1) == b"invalid argument"


def _spec(wl, **over):
    kw = dict(batch=wl.batch, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim,
              obs_window=wl.obs_window, pool_kernel=wl.pool_kernel, ratio=wl.ratio, budget=wl.budget,
              dtype=_lib.BF16 if wl.dtype == "bf16" else _lib.F32, cu_seqlens=wl.cu_seqlens(),
              kv_head_stride=wl.total_tokens * wl.head_dim, kv_token_stride=wl.head_dim)
    kw.update(over)
    return _lib.Spec(**kw)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_plan_of_standard_workloads(n):
    """k = floor(0.05 * P) = P // 20 in ratio mode, min(budget, P) in budget mode
    (section 投票メカニズム; the アルゴリズム listing's min(max_cap, pfx)); offsets are prefix sums."""
    wl = synth.workload(n)
    sp = _spec(wl)
    P = np.array(wl.lengths) - wl.obs_window
    k = P // 20 if wl.ratio is not None else np.minimum(wl.budget, P)
    np.testing.assert_array_equal(sp.k, k)
    np.testing.assert_array_equal(sp.cu_pfx, np.concatenate([[0], np.cumsum(P)]))
    np.testing.assert_array_equal(sp.cu_k, np.concatenate([[0], np.cumsum(k)]))
    np.testing.assert_array_equal(sp.cu_out, np.concatenate([[0], np.cumsum(k + wl.obs_window)]))
    # workspace holds at least the votes and pooled votes
    assert sp.ws_bytes >= 2 * 4 * wl.num_kv_heads * int(P.sum())


BAD = [
    (dict(batch=0), "batch"),
    (dict(num_kv_heads=3), "multiple"),
    (dict(obs_window=0), "obs_window"),
    (dict(pool_kernel=4), "odd"),
    (dict(pool_kernel=0), "odd"),
    (dict(ratio=0.0), "ratio"),
    (dict(ratio=1.5), "ratio"),
    (dict(ratio=None, budget=-1), "budget"),
    (dict(head_dim=96), "head_dim"),
    (dict(kv_token_stride=66), "aligned"),
    (dict(kv_token_stride=32), "kv_token_stride"),
    (dict(cu_seqlens=np.array([0, 20], np.int32)), "shorter"),
    (dict(cu_seqlens=np.array([5, 1029], np.int32)), "cu_seqlens"),
    (dict(num_q_heads=64, num_kv_heads=1, obs_window=17), "1024"),
]


@pytest.mark.parametrize("over,msg", BAD, ids=[m for _, m in BAD])
def test_plan_rejects_invalid_problems(over, msg):
    wl = synth.workload(1)
    with pytest.raises(ValueError, match=msg):
        _spec(wl, **over)


def test_calls_reject_bad_pointers_before_any_launch():
    lib = _lib.load()
    sp = _spec(synth.workload(2))
    pb = ctypes.byref(sp.pb)
    good, odd = ctypes.c_void_p(1 << 20), ctypes.c_void_p((1 << 20) + 4)
    ws, n = ctypes.c_void_p(1 << 24), ctypes.c_size_t(sp.ws_bytes)
    st = lib.snapkv_scores(pb, None, good, None, good, ws, n, None)
    assert st == _lib.EINVAL and b"q_obs" in lib.snapkv_last_error()
    assert lib.snapkv_scores(pb, good, odd, None, good, ws, n, None) == _lib.EINVAL
    assert lib.snapkv_scores(pb, good, good, None, good, None, n, None) == _lib.EWORKSPACE
    assert lib.snapkv_scores(pb, good, good, None, good, ctypes.c_void_p((1 << 24) + 16), n, None) == _lib.EWORKSPACE
    assert lib.snapkv_scores(pb, good, good, None, good, ws, ctypes.c_size_t(sp.ws_bytes - 1), None) == _lib.EWORKSPACE
    assert lib.snapkv_select(pb, None, good, ws, n, None) == _lib.EINVAL
    assert lib.snapkv_gather(pb, good, good, good, good, odd, None) == _lib.EINVAL
    assert lib.snapkv_compress(pb, good, good, good, good, good, odd, None, ws, n, None) == _lib.EINVAL
    assert lib.snapkv_compress(None, good, good, good, good, good, None, None, ws, n, None) == _lib.EINVAL


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", os.path.join(ROOT, "does_not_exist", "libsnapkv.so"))
    with pytest.raises(ImportError):
        _lib.load()
