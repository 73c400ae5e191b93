"""snapkv_compress_noalloc (the call that allocates nothing, for callers under graph capture
or in loops that cannot allocate) against snapkv_compress with a caller workspace: the same
bits on two calls in a row, the second with a smaller input, and oversize problems refused."""
import numpy as np
import pytest
import torch

from kv_cache_compression_amd import synth
from parity_utils import to_torch

pytestmark = pytest.mark.gpu


def _snap():
    from kv_cache_compression_amd import _lib
    return _lib


CASES = [
    # lengths, Hq, Hkv, d, dtype, w, K_pool, ratio, budget, n_plant  (each call smaller than the last)
    ([70000, 1500], 8, 8, 128, "bf16", 32, 7, 0.05, None, 8),    # two-slot one-read scoring
    ([5000, 9000, 3000], 16, 4, 128, "bf16", 32, 7, 0.05, None, 16),  # two-phase streaming scoring
    ([9000, 3000], 4, 4, 128, "bf16", 32, 7, 0.05, None, 8),     # one-read scoring
    ([1500], 8, 2, 128, "bf16", 32, 7, None, 100, 8),
]


def test_noalloc_matches_workspace_call():
    snap = _snap()
    for n, (lengths, Hq, Hkv, d, dt, w, kp, ratio, budget, n_plant) in enumerate(CASES):
        print("noalloc call %d lengths=%s" % (n, lengths), flush=True)
        wl = synth.custom(lengths, Hq, Hkv, d, dtype=dt, obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget,
                          n_plant=n_plant, name="noalloc%d" % n)
        x = synth.make_inputs(wl)
        q, K, V = to_torch(x["q_obs"]), to_torch(x["K"]), to_torch(x["V"])
        kw = dict(obs_window=w, pool_kernel=kp, ratio=ratio, budget=budget)
        ref = snap.compress(q, K, V, x["cu_seqlens"], want_pooled=True, **kw)
        spec = snap.make_spec(q, K, x["cu_seqlens"], w, kp, ratio, budget)
        out = dict(K_out=torch.full_like(ref["K_out"], 7), V_out=torch.full_like(ref["V_out"], 7),
                   idx=torch.full_like(ref["idx"], -1), pooled=torch.full_like(ref["pooled"], -1.0))
        err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        got = snap.compress_noalloc(q, K, V, x["cu_seqlens"], out=out, error_word=err, **kw)
        torch.cuda.synchronize()
        assert int(err.item()) == 0, "error word %d" % int(err.item())
        assert spec.ws_bytes <= snap.NOALLOC_SCRATCH_BYTES
        for key in ("K_out", "V_out", "idx", "pooled"):
            assert torch.equal(got[key], ref[key]), "call %d: %s differs" % (n, key)
        np.testing.assert_array_equal(got["cu_out"], ref["cu_out"])


def test_noalloc_refuses_problems_beyond_its_scratch():
    snap = _snap()
    # 8 KV heads of 4 M positions: the votes alone need 128 MiB of workspace
    L = 4 << 20
    q = torch.zeros((1, 8, 32, 64), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((1, L, 64), dtype=torch.bfloat16, device="cuda").expand(8, L, 64)  # KV head stride 0
    with pytest.raises(ValueError, match="scratch"):
        snap.compress_noalloc(q, K, K, [0, L], obs_window=32, pool_kernel=7, ratio=0.05)
