"""Helpers shared by the GPU parity tests: inputs to torch, and the parity criteria.

Criteria (GPU vs the fp64 oracle):
  * votes and pooled votes: |gpu - ref| <= 1e-3 * |ref| + 1e-6 * max(ref) per
    (request, KV head).  The relative bound is the one fixed for this path; the
    absolute floor only admits fp32 underflow of weights a million times below the
    segment's largest vote, far below anything top-k can pick.
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
ABS_FLOOR = 1e-6


def to_torch(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def check_scores(gpu: np.ndarray, ref: np.ndarray, what: str):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if ref.size == 0:
        return
    tol = RTOL * np.abs(ref) + ABS_FLOOR * np.max(np.abs(ref))
    err = np.abs(gpu - ref)
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, "%s: %d of %d outside tolerance; worst j=%d gpu=%r ref=%r" % (
        what, bad.size, ref.size, bad[np.argmax(err[bad] / tol[bad])], gpu[bad[0]], ref[bad[0]])


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
