"""Helpers shared by the GPU parity tests: inputs to torch, and the parity criteria.

Criteria (GPU vs the fp64 oracle):
  * votes and pooled votes: |gpu - ref| <= 1e-3 * |ref| for every entry.  This is
    the relative bound fixed for this path, with no absolute term.  The only
    exception is a genuine fp32 underflow guard: an entry whose oracle value is
    below UNDERFLOW (1e-30, some 2^100 below any vote these inputs produce) may
    be anything in [0, 2 * UNDERFLOW].  check_scores returns how many entries
    passed only by that guard and, unless told otherwise, asserts there are none.
  * selection: exactly k ascending positions in [0, P); the symmetric difference
    with the oracle's set lies inside the tie band {j : |ref_j - v*| <= 1e-3 * v*},
    v* = the oracle's k-th largest pooled vote.
  * select on the GPU's own pooled votes equals the oracle's select on those same
    fp32 values, exactly (no band).
  * gather: every output row equals the input row the GPU's own index names, bit
    for bit, and the last L_obs rows equal the window.
"""
import numpy as np
import torch

import oracle

RTOL = 1e-3
UNDERFLOW = 1e-30


def to_torch(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def check_scores(gpu: np.ndarray, ref: np.ndarray, what: str, allow_underflow: bool = False) -> int:
    """Asserts the relative bound entry by entry; returns the number of entries that
    passed only by the underflow guard (asserted zero unless allow_underflow)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if ref.size == 0:
        return 0
    err = np.abs(gpu - ref)
    rel_ok = err <= RTOL * np.abs(ref)
    guard_ok = (np.abs(ref) < UNDERFLOW) & (gpu >= 0.0) & (gpu <= 2 * UNDERFLOW)
    bad = np.nonzero(~(rel_ok | guard_ok))[0]
    if bad.size:
        rel = err[bad] / np.maximum(np.abs(ref[bad]), 1e-300)
        worst = bad[np.argmax(rel)]
        raise AssertionError("%s: %d of %d outside 1e-3 relative; worst j=%d gpu=%r ref=%r rel=%.3g" % (
            what, bad.size, ref.size, worst, gpu[worst], ref[worst], float(np.max(rel))))
    n_guard = int(np.sum(guard_ok & ~rel_ok))
    assert allow_underflow or n_guard == 0, "%s: %d entries pass only by the underflow guard" % (what, n_guard)
    return n_guard


def max_rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """Largest |gpu - ref| / |ref| over entries with ref != 0 (diagnostic)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    nz = ref != 0
    if not np.any(nz):
        return 0.0
    return float(np.max(np.abs(gpu[nz] - ref[nz]) / np.abs(ref[nz])))


def check_selection(idx_gpu: np.ndarray, ref_pooled: np.ndarray, ref_idx: np.ndarray, k: int, what: str):
    idx_gpu = np.asarray(idx_gpu, np.int64)
    P = ref_pooled.size
    assert idx_gpu.size == k, (what, idx_gpu.size, k)
    if k == 0:
        return
    assert np.all(np.diff(idx_gpu) > 0), what + ": not strictly ascending"
    assert idx_gpu[0] >= 0 and idx_gpu[-1] < P, what + ": out of range"
    vstar = np.sort(ref_pooled)[::-1][k - 1]
    band = np.abs(ref_pooled - vstar) <= RTOL * vstar
    diff = np.setxor1d(idx_gpu, np.asarray(ref_idx, np.int64))
    assert np.all(band[diff]), "%s: %d positions differ outside the tie band" % (what, int(np.sum(~band[diff])))


def check_select_exact(idx_gpu: np.ndarray, pooled_gpu_f32: np.ndarray, k: int, what: str):
    ref = oracle.select(pooled_gpu_f32.astype(np.float64), k)
    np.testing.assert_array_equal(np.asarray(idx_gpu, np.int64), ref.astype(np.int64), err_msg=what)


def check_gather(rows_in: np.ndarray, out: np.ndarray, idx: np.ndarray, P: int, w: int, what: str):
    """rows_in: [L, d] of one (request, KV head); out: [k + w, d]."""
    k = idx.size
    assert out.shape[0] == k + w, what
    expect = rows_in[np.concatenate([np.asarray(idx, np.int64), np.arange(P, P + w)])]
    assert out.tobytes() == expect.tobytes(), what + ": gathered rows differ"
