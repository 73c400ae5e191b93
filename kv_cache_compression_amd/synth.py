"""Seeded synthetic inputs for SnapKV compression workloads.

This module only draws numbers; it holds none of the compression method's
arithmetic.  Both the HIP path and the CPU oracle consume exactly the arrays it
returns (bfloat16 tensors as uint16 bit patterns, fp32 as float32).

Workloads (names follow the pages' notation: L_prompt, L_obs, K_pool, p):
  1  8 heads MHA, d=64, fp32, L=1024, L_obs=32, K_pool=7, p=0.05, iid N(0,1).
  2  Llama-2-7B-shaped layer: 32 heads MHA, d=128, bf16, L=16384, L_obs=32,
     K_pool=7, p=0.05, N(0,1) plus 64 planted heavy-hitter keys per head.
  3  GQA 32/8, d=128, bf16, 32 layers, L=32768, L_obs=64, K_pool=7, budget
     2048 per KV head, 64 planted keys per KV head per layer.
  4  32 heads MHA, d=128, bf16, L=380000, L_obs=32, K_pool=13, p=0.05, keys
     scaled per channel by a fixed log-normal (sigma=1) outlier profile, 512
     planted keys per head.
  5  16 ragged requests, GQA 32/8, d=128, bf16, L_r ~ U{2048..32768}, L_obs=32,
     K_pool=7, p=0.05, packed [H_kv, sum L_r, d] with cu_seqlens, 64 planted
     keys per KV head per request.

Planted heavy hitter: the key row at a uniformly drawn prefix position becomes
2 * (mean of the group's window query rows) + N(0, I).  Every stream comes from
numpy's Philox generator keyed by (workload, layer, request, head, tensor tag),
so any (request, head) block can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TAG_Q, TAG_K, TAG_V, TAG_PLANT_POS, TAG_PLANT_NOISE, TAG_PROFILE, TAG_LENGTHS = range(7)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    workload_id: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                 # "bf16" or "f32"
    lengths: tuple             # L_r per request
    obs_window: int            # L_obs
    pool_kernel: int           # K_pool
    ratio: float | None        # p, or None in budget mode
    budget: int | None         # prefix slots per KV head, or None in ratio mode
    n_layers: int = 1
    n_plant: int = 0           # planted heavy hitters per (request, KV head)
    outlier_profile: bool = False

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([int(k) for k in key])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


def workload(n: int) -> Workload:
    """The five standard workloads, numbered as in the module docstring."""
    if n == 1:
        return Workload("mha8_d64_f32_L1024", 1, 1, 8, 8, 64, "f32", (1024,), 32, 7, 0.05, None)
    if n == 2:
        return Workload("llama2_7b_layer_L16384", 2, 1, 32, 32, 128, "bf16", (16384,), 32, 7, 0.05, None,
                        n_plant=64)
    if n == 3:
        return Workload("gqa32x8_32layers_L32768_budget2048", 3, 1, 32, 8, 128, "bf16", (32768,), 64, 7,
                        None, 2048, n_layers=32, n_plant=64)
    if n == 4:
        return Workload("mha32_L380000_pool13_outliers", 4, 1, 32, 32, 128, "bf16", (380000,), 32, 13, 0.05,
                        None, n_plant=512, outlier_profile=True)
    if n == 5:
        lengths = tuple(int(x) for x in _rng(5, 0, 0, 0, TAG_LENGTHS).integers(2048, 32768, size=16, endpoint=True))
        return Workload("varlen16_gqa32x8_L2048to32768", 5, 16, 32, 8, 128, "bf16", lengths, 32, 7, 0.05, None,
                        n_plant=64)
    raise ValueError("workloads are numbered 1..5")


def custom(lengths, num_q_heads, num_kv_heads, head_dim, dtype="bf16", obs_window=32, pool_kernel=7,
           ratio=0.05, budget=None, n_plant=0, outlier_profile=False, workload_id=100, name="custom") -> Workload:
    lengths = tuple(int(x) for x in lengths)
    return Workload(name, workload_id, len(lengths), num_q_heads, num_kv_heads, head_dim, dtype, lengths,
                    obs_window, pool_kernel, ratio, budget, 1, n_plant, outlier_profile)


def _normal(shape, *key) -> np.ndarray:
    return _rng(*key).standard_normal(size=shape, dtype=np.float32)


def make_inputs(wl: Workload, layer: int = 0, threads: int = 8) -> dict:
    """Draw one layer of ``wl``.

    Returns dict(q_obs [B, H_q, L_obs, d], K [H_kv, T, d], V [H_kv, T, d],
    cu_seqlens int32 [B+1], planted {(r, g): sorted positions}).  bf16 tensors
    are uint16 bit patterns; fp32 tensors are float32.
    """
    B, Hq, Hkv, d, w, G = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.obs_window, wl.group
    cu = wl.cu_seqlens()
    T = int(cu[-1])
    bf = wl.dtype == "bf16"
    edt = np.uint16 if bf else np.float32
    wid = wl.workload_id

    def canon(x):
        return round_bf16(x) if bf else x.astype(np.float32)

    def value_of(x):
        return bf16_to_f32(x) if bf else x

    q_obs = np.empty((B, Hq, w, d), edt)
    for r in range(B):
        for h in range(Hq):
            q_obs[r, h] = canon(_normal((w, d), wid, layer, r, h, TAG_Q))

    profile = None
    if wl.outlier_profile:
        profile = np.exp(_normal((d,), wid, 0, 0, 0, TAG_PROFILE)).astype(np.float32)

    K = np.empty((Hkv, T, d), edt)
    V = np.empty((Hkv, T, d), edt)
    planted = {}

    def fill(job):
        r, g = job
        t0, t1 = int(cu[r]), int(cu[r + 1])
        L = t1 - t0
        P = L - w
        k = _normal((L, d), wid, layer, r, g, TAG_K)
        pos = np.zeros(0, np.int64)
        n = min(wl.n_plant, max(P, 0))
        if n > 0:
            pos = np.sort(_rng(wid, layer, r, g, TAG_PLANT_POS).choice(P, size=n, replace=False))
            qbar = value_of(q_obs[r, g * G:(g + 1) * G]).reshape(G * w, d).astype(np.float32).mean(axis=0)
            k[pos] = 2.0 * qbar[None, :] + _normal((n, d), wid, layer, r, g, TAG_PLANT_NOISE)
        if profile is not None:
            k *= profile[None, :]
        K[g, t0:t1] = canon(k)
        V[g, t0:t1] = canon(_normal((L, d), wid, layer, r, g, TAG_V))
        return (r, g), pos

    jobs = [(r, g) for r in range(B) for g in range(Hkv)]
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        for key, pos in ex.map(fill, jobs):
            planted[key] = pos
    return dict(q_obs=q_obs, K=K, V=V, cu_seqlens=cu, planted=planted)
