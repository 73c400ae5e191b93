"""Pins of the fp64 CPU oracle to facts fixed by the pages and by mathematics.

Every test here runs on the CPU.  None of them compares the oracle with a copy of
itself: each checks a closed form, an invariant, a textbook/library routine a
special case reduces to, a hand-worked value (tests/golden/), or brute force over
all candidates on tiny inputs.  Citations are to the page
"論文解説: SnapKV — アテンションパターン観測によるKVキャッシュ圧縮".
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.ndimage
import scipy.special

import oracle
from kv_cache_compression_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _rand(shape, seed, scale=1.0):
    return _f32(np.random.default_rng(seed).standard_normal(shape) * scale)


# ---------------------------------------------------------------- votes (section 投票メカニズム)

@pytest.mark.parametrize("G,w,P,d", [(1, 1, 5, 4), (1, 3, 7, 8), (2, 4, 9, 4), (4, 2, 1, 16), (1, 5, 0, 4)])
def test_uniform_keys_closed_form_causal(G, w, P, d):
    """All keys equal: row i spreads 1/(P+i+1) over its P+i+1 visible keys.

    Prefix position j gets sum_{i<w} 1/(P+i+1) per query head; window position
    P+t gets sum_{i>=t} 1/(P+i+1).  This fixes the causal window reading, the
    window-row bounds of the sum (i = 0..L_obs-1) and the GQA group sum.
    """
    L = P + w
    q = _rand((G * w, d), 1)
    row = _rand((1, d), 2)
    keys = _f32(np.repeat(row, L, axis=0))
    v = oracle.votes(q, keys, w)
    expect = np.empty(L)
    for j in range(L):
        t = max(0, j - P)
        expect[j] = G * sum(1.0 / (P + i + 1) for i in range(t, w))
    np.testing.assert_allclose(v, expect, rtol=1e-13, atol=0)


def test_uniform_keys_prefix_only_variant():
    """Prefix-only denominator (the listing's softmax over k_pfx): every prefix key gets w/P per head."""
    G, w, P, d = 2, 3, 10, 8
    q = _rand((G * w, d), 3)
    keys = _f32(np.repeat(_rand((1, d), 4), P + w, axis=0))
    v = oracle.votes(q, keys, w, variant=1)
    np.testing.assert_allclose(v[:P], np.full(P, G * w / P), rtol=1e-13)
    assert np.all(v[P:] == 0.0)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_single_window_row_is_library_softmax(dt):
    """L_obs = 1: the vote is one softmax row over all L keys of q k^T / sqrt(d)."""
    L, d = 300, 64
    q = _rand((1, d), 5)
    keys = _rand((L, d), 6, scale=1.5)
    if dt == "bf16":
        q, keys = synth.round_bf16(q), synth.round_bf16(keys)
        qv, kv = synth.bf16_to_f32(q).astype(np.float64), synth.bf16_to_f32(keys).astype(np.float64)
    else:
        qv, kv = q.astype(np.float64), keys.astype(np.float64)
    v = oracle.votes(q, keys, 1)
    ref = scipy.special.softmax(kv @ qv[0] / math.sqrt(d))
    np.testing.assert_allclose(v, ref, rtol=1e-12, atol=1e-300)


def test_large_logits_do_not_overflow():
    """Logits near 1e3 (exp would overflow without the max shift): still the library softmax."""
    L, d = 64, 16
    q = _rand((1, d), 7, scale=20.0)
    keys = _rand((L, d), 8, scale=20.0)
    v = oracle.votes(q, keys, 1)
    ref = scipy.special.softmax(keys.astype(np.float64) @ q[0].astype(np.float64) / 4.0)
    assert np.all(np.isfinite(v))
    np.testing.assert_allclose(v, ref, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("G,w,L,d", [(1, 32, 200, 64), (4, 8, 77, 32), (2, 5, 5, 8)])
def test_rows_sum_to_one(G, w, L, d):
    """Each softmax row sums to 1, so prefix plus window votes total L_obs per query head."""
    q = _rand((G * w, d), 9)
    keys = _rand((L, d), 10, scale=2.0)
    v = oracle.votes(q, keys, w)
    assert v.sum() == pytest.approx(G * w, rel=1e-12)
    assert np.all(v >= 0)


def test_golden_hand_worked_three_keys():
    """Hand-worked: q=[1], keys=[0, ln2, ln3], d=1, L_obs=1 -> weights 1/6, 2/6, 3/6."""
    path = os.path.join(GOLDEN, "votes_three_keys.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    keys = _f32([[float(r[0])] for r in rows])
    expect = np.array([float(r[1]) for r in rows])
    v = oracle.votes(_f32([[1.0]]), keys, 1)
    # inputs were rounded to float32, which moves the weights by < 1e-7 relative
    np.testing.assert_allclose(v, expect, rtol=2e-7)


def test_key_equal_to_window_query_wins():
    """One key equals the query and the rest lie on the sphere of radius |q|: by Cauchy-Schwarz
    it has the strictly largest logit, so it has the largest vote and top-1 picks it."""
    rng = np.random.default_rng(11)
    d, P, j_star = 8, 40, 17
    q = rng.standard_normal(d)
    dirs = rng.standard_normal((P + 1, d))
    keys = dirs / np.linalg.norm(dirs, axis=1, keepdims=True) * np.linalg.norm(q)
    keys[j_star] = q
    q32, k32 = _f32(q[None, :]), _f32(keys)
    v = oracle.votes(q32, k32, 1)
    c = v[:P]
    assert int(np.argmax(c)) == j_star and np.sum(c == c.max()) == 1
    assert list(oracle.select(oracle.pool(c, 1), 1)) == [j_star]
    pl = oracle.pool(c, 7)
    assert list(oracle.select(pl, 7)) == list(range(j_star - 3, j_star + 4))
    # plateau of 7 equal maxima: the lower position wins the tie
    assert list(oracle.select(pl, 1)) == [j_star - 3]


def test_shift_invariance():
    """Adding one vector to every key adds a per-row constant to the logits: votes unchanged.
    Entries are multiples of 1/8 so the shifted keys are exact in float32."""
    rng = np.random.default_rng(12)
    G, w, L, d = 2, 4, 50, 8
    q = _f32(rng.integers(-16, 17, (G * w, d)) / 8.0)
    keys = _f32(rng.integers(-16, 17, (L, d)) / 8.0)
    c = _f32(rng.integers(-16, 17, (1, d)) / 8.0)
    v0 = oracle.votes(q, keys, w)
    v1 = oracle.votes(q, _f32(keys + c), w)
    np.testing.assert_allclose(v1, v0, rtol=1e-12, atol=1e-15)


def test_prefix_permutation_equivariance():
    """Permuting prefix keys permutes their votes; the window is untouched."""
    G, w, P, d = 2, 3, 40, 16
    q = _rand((G * w, d), 13)
    keys = _rand((P + w, d), 14)
    perm = np.random.default_rng(15).permutation(P)
    keys_p = keys.copy()
    keys_p[:P] = keys[perm]
    v0 = oracle.votes(q, keys, w)
    v1 = oracle.votes(q, keys_p, w)
    np.testing.assert_allclose(v1[:P], v0[perm], rtol=1e-12)
    np.testing.assert_allclose(v1[P:], v0[P:], rtol=1e-12)


def test_gqa_group_sum_equals_repeated_kv_heads():
    """GQA: query head h reads KV head h // G.  The group vote equals the sum of per-head
    MHA votes against the repeated KV head (the usual repeat-kv formulation), and G identical
    query heads give exactly G times the single-head vote."""
    B, Hq, Hkv, w, d = 1, 6, 2, 4, 16
    G = Hq // Hkv
    L = 37
    rng = np.random.default_rng(16)
    q_obs = _f32(rng.standard_normal((B, Hq, w, d)))
    K = _f32(rng.standard_normal((Hkv, L, d)))
    V = _f32(rng.standard_normal((Hkv, L, d)))
    cu = np.array([0, L], np.int32)
    res = oracle.compress(q_obs, K, V, cu, w, 3, ratio=0.25)
    for g in range(Hkv):
        per_head = sum(oracle.votes(q_obs[0, h], K[g], w) for h in range(g * G, (g + 1) * G))
        np.testing.assert_allclose(res[(0, g)]["votes_full"], per_head, rtol=1e-12)
    same = _f32(np.repeat(q_obs[0, :1], G, axis=0).reshape(G * w, d))
    np.testing.assert_allclose(oracle.votes(same, K[0], w), G * oracle.votes(q_obs[0, 0], K[0], w), rtol=1e-12)


def test_brute_force_double_loop_tiny():
    """Tiny inputs against an independent pure-Python double loop in fp64 (math.exp)."""
    rng = np.random.default_rng(17)
    for G, w, L, d in [(1, 1, 3, 2), (2, 3, 7, 4), (1, 3, 3, 3), (3, 2, 12, 4)]:
        q = _f32(rng.standard_normal((G * w, d)))
        keys = _f32(rng.standard_normal((L, d)))
        P = L - w
        expect = [0.0] * L
        for r in range(G * w):
            i = r % w
            s = [sum(float(q[r, c]) * float(keys[j, c]) for c in range(d)) / math.sqrt(d) for j in range(P + i + 1)]
            m = max(s)
            z = sum(math.exp(x - m) for x in s)
            for j, x in enumerate(s):
                expect[j] += math.exp(x - m) / z
        np.testing.assert_allclose(oracle.votes(q, keys, w), expect, rtol=1e-12)


# ---------------------------------------------------------------- pool (section クラスタリングによる文脈保持)

@pytest.mark.parametrize("K_pool", [1, 3, 5, 7, 13])
def test_pool_matches_library_max_filter(K_pool):
    c = np.random.default_rng(18).random(101)
    ref = scipy.ndimage.maximum_filter1d(c, size=K_pool, mode="constant", cval=-np.inf)
    pl = oracle.pool(c, K_pool)
    np.testing.assert_array_equal(pl, ref)
    assert np.all(pl >= c)


def test_pool_identity_and_plateau():
    c = np.random.default_rng(19).random(50) * 0.1
    np.testing.assert_array_equal(oracle.pool(c, 1), c)
    for K_pool in (5, 7, 13):
        h = K_pool // 2
        for peak in (0, 2, 25, 49):
            x = np.zeros(50)
            x[peak] = 1.0
            pl = oracle.pool(x, K_pool)
            expect = np.zeros(50)
            expect[max(0, peak - h):min(50, peak + h + 1)] = 1.0
            np.testing.assert_array_equal(pl, expect)


# ---------------------------------------------------------------- k and top-k (section 投票メカニズム; アルゴリズム listing)

def test_k_ratio_closed_form():
    """k = floor(0.05 * P) equals P // 20 exactly over the whole range used here."""
    for P in list(range(0, 5000)) + [16352, 32704, 379968, 2_000_000]:
        assert oracle.k_of(P, ratio=0.05) == P // 20
    for P in (0, 1, 7, 1000):
        assert oracle.k_of(P, ratio=1.0) == P
        assert oracle.k_of(P, budget=P) == P
        assert oracle.k_of(P, budget=P + 5) == P
    assert oracle.k_of(32704, budget=2048) == 2048


def test_select_matches_library_lexsort():
    rng = np.random.default_rng(20)
    for P in (1, 10, 257, 4000):
        vals = np.round(rng.random(P) * 50) / 50.0  # many exact ties
        for k in {0, 1, P // 3, P}:
            ref = np.sort(np.lexsort((np.arange(P), -vals))[:k])
            np.testing.assert_array_equal(oracle.select(vals, k), ref)


def test_select_brute_force_over_all_subsets():
    """For tiny P the chosen set is the unique k-subset S such that every member beats every
    non-member: larger value, or equal value at a lower position."""
    rng = np.random.default_rng(21)
    for _ in range(40):
        P = int(rng.integers(1, 9))
        vals = rng.integers(0, 3, P).astype(np.float64)
        k = int(rng.integers(0, P + 1))
        valid = []
        for S in itertools.combinations(range(P), k):
            rest = [j for j in range(P) if j not in S]
            if all(vals[i] > vals[j] or (vals[i] == vals[j] and i < j) for i in S for j in rest):
                valid.append(list(S))
        assert len(valid) == 1
        assert list(oracle.select(vals, k)) == valid[0]


def test_select_uniform_values_takes_lowest_positions():
    assert list(oracle.select(np.full(30, 0.25), 7)) == list(range(7))


# ---------------------------------------------------------------- gather (アルゴリズム listing: gather + concat)

def test_keep_everything_returns_input_bit_for_bit():
    """p = 1 (or a budget >= P) keeps every prefix position: K', V' are the inputs, bit for bit."""
    wl = synth.custom([90], 4, 2, 32, dtype="bf16", obs_window=8, pool_kernel=5, ratio=1.0)
    x = synth.make_inputs(wl)
    for kw in (dict(ratio=1.0), dict(budget=500)):
        res = oracle.compress(x["q_obs"], x["K"], x["V"], x["cu_seqlens"], 8, 5, **kw)
        for g in range(2):
            np.testing.assert_array_equal(res[(0, g)]["idx"], np.arange(82))
            assert res[(0, g)]["K_out"].tobytes() == x["K"][g].tobytes()
            assert res[(0, g)]["V_out"].tobytes() == x["V"][g].tobytes()


def test_gather_rows_and_window():
    rows = np.arange(20 * 4, dtype=np.float32).reshape(20, 4)
    out = oracle.gather(rows, 16, 4, np.array([1, 5, 9], np.int32))
    np.testing.assert_array_equal(out, rows[[1, 5, 9, 16, 17, 18, 19]])


# ---------------------------------------------------------------- Hit Rate (section Hit Rate（適中率）の定式化)

def test_hit_rate_cases():
    a = np.array([0.2, 0.01, 0.07, 0.05, 0.3, 0.0])
    thr = a > 0.05
    assert oracle.hit_rate(a, thr) == 1.0                      # masks coincide
    assert oracle.hit_rate(a, ~thr) == 0.0                     # disjoint
    vote = np.array([1, 1, 1, 1, 0, 0], bool)                  # hits 0.2 and 0.07, misses 0.3
    assert oracle.hit_rate(a, vote) == pytest.approx(2.0 / 3.0)
    assert oracle.hit_rate(np.full(4, 0.05), np.ones(4, bool)) != oracle.hit_rate(np.full(4, 0.05), np.ones(4, bool))  # NaN: strict >


# ---------------------------------------------------------------- batches

def test_varlen_batch_equals_per_request_runs():
    wl = synth.custom([40, 73, 33, 120], 4, 2, 16, dtype="bf16", obs_window=8, pool_kernel=3, ratio=0.2, n_plant=3)
    x = synth.make_inputs(wl)
    res = oracle.compress(x["q_obs"], x["K"], x["V"], x["cu_seqlens"], 8, 3, ratio=0.2)
    cu = x["cu_seqlens"]
    for r in range(4):
        sub = oracle.compress(x["q_obs"][r:r + 1], np.ascontiguousarray(x["K"][:, cu[r]:cu[r + 1]]),
                              np.ascontiguousarray(x["V"][:, cu[r]:cu[r + 1]]), np.array([0, cu[r + 1] - cu[r]]),
                              8, 3, ratio=0.2)
        for g in range(2):
            a, b = res[(r, g)], sub[(0, g)]
            np.testing.assert_array_equal(a["votes"], b["votes"])
            np.testing.assert_array_equal(a["idx"], b["idx"])
            assert a["K_out"].tobytes() == b["K_out"].tobytes()


def test_window_only_request():
    """L_r = L_obs: P = 0, k = 0, the output is the window."""
    wl = synth.custom([8], 2, 2, 16, dtype="f32", obs_window=8, pool_kernel=3, ratio=0.5)
    x = synth.make_inputs(wl)
    res = oracle.compress(x["q_obs"], x["K"], x["V"], x["cu_seqlens"], 8, 3, ratio=0.5)
    assert res[(0, 0)]["k"] == 0 and res[(0, 0)]["K_out"].tobytes() == x["K"][0].tobytes()


# ---- row log-sum-exp (input of the LSE-fed path) ----------------------------------------------

def test_row_lse_uniform_logits_closed_form():
    """q = 0: every visible logit is 0, so lse_i = ln(#visible keys): ln(P + i + 1) with the
    causal window, ln(P) for the prefix-only variant."""
    rng = np.random.default_rng(7)
    w, d, L = 4, 8, 23
    q = np.zeros((2 * w, d), np.float32)
    keys = rng.standard_normal((L, d)).astype(np.float32)
    P = L - w
    lse = oracle.row_lse(q, keys, w, variant=0)
    np.testing.assert_allclose(lse, [np.log(P + (r % w) + 1) for r in range(2 * w)], rtol=0, atol=1e-12)
    lse1 = oracle.row_lse(q, keys, w, variant=1)
    np.testing.assert_allclose(lse1, np.full(2 * w, np.log(P)), rtol=0, atol=1e-12)


def test_row_lse_one_row_matches_scipy_logsumexp():
    from scipy.special import logsumexp
    rng = np.random.default_rng(8)
    d, L = 16, 40
    q = rng.standard_normal((1, d)).astype(np.float32)
    keys = (3 * rng.standard_normal((L, d))).astype(np.float32)
    s = keys.astype(np.float64) @ q[0].astype(np.float64) / np.sqrt(d)
    np.testing.assert_allclose(oracle.row_lse(q, keys, 1), [logsumexp(s)], rtol=1e-13)


def test_row_lse_normalises_the_votes():
    """exp(s_ij - lse_i) summed over rows i equals the vote of every key (votes() computes its
    normaliser separately, from the row max and sum)."""
    rng = np.random.default_rng(9)
    w, d, L = 3, 8, 17
    q = rng.standard_normal((2 * w, d)).astype(np.float32)
    keys = rng.standard_normal((L, d)).astype(np.float32)
    lse = oracle.row_lse(q, keys, w)
    P = L - w
    s = (q.astype(np.float64) @ keys.astype(np.float64).T) / np.sqrt(d)
    v = np.zeros(L)
    for r in range(2 * w):
        n = P + (r % w) + 1
        v[:n] += np.exp(s[r, :n] - lse[r])
    np.testing.assert_allclose(v, oracle.votes(q, keys, w), rtol=1e-12)


# ---- decode attention over the compressed cache -----------------------------------------------

def test_decode_uniform_scores_give_the_mean_value():
    """q = 0: every score is 0, so the output is the mean of the cached value rows."""
    rng = np.random.default_rng(20)
    n, d = 37, 16
    q = np.zeros((3, d), np.float32)
    k = rng.standard_normal((n, d)).astype(np.float32)
    v = rng.standard_normal((n, d)).astype(np.float32)
    np.testing.assert_allclose(oracle.decode(q, k, v), np.tile(v.astype(np.float64).mean(0), (3, 1)), rtol=1e-13)


def test_decode_single_row_and_empty_cache():
    rng = np.random.default_rng(21)
    q = rng.standard_normal((2, 8)).astype(np.float32)
    k = rng.standard_normal((1, 8)).astype(np.float32)
    v = rng.standard_normal((1, 8)).astype(np.float32)
    np.testing.assert_array_equal(oracle.decode(q, k, v), np.tile(v.astype(np.float64), (2, 1)))
    assert not oracle.decode(q, k[:0], v[:0]).any()


def test_decode_matches_torch_sdpa_float64():
    """Against torch's scaled_dot_product_attention on the CPU in float64 (bf16 inputs)."""
    import torch
    from kv_cache_compression_amd import synth
    rng = np.random.default_rng(22)
    G, n, d = 4, 300, 64
    q = synth.round_bf16((2 * rng.standard_normal((G, d))).astype(np.float32))
    k = synth.round_bf16(rng.standard_normal((n, d)).astype(np.float32))
    v = synth.round_bf16(rng.standard_normal((n, d)).astype(np.float32))
    f64 = lambda a: torch.from_numpy(synth.bf16_to_f32(a).astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(f64(q)[None, None], f64(k)[None, None], f64(v)[None, None])
    np.testing.assert_allclose(oracle.decode(q, k, v), ref[0, 0].numpy(), rtol=1e-12, atol=1e-14)
