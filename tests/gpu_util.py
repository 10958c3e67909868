"""Helpers shared by the GPU tests: device upload and the parity verdicts.

Parity rules (the pages state none; these readings are in force for every test):
  * scores: |gpu - oracle| <= 1e-3 * |oracle| + 1e-30 elementwise (bf16 inputs,
    fp32 accumulation on the GPU, fp64 in the oracle);
  * kept sets: (a) the GPU's indices equal the oracle's selection applied to the
    GPU's own scores, bit for bit; (b) they equal the oracle's selection on its
    own scores at every position whose oracle score is not within a relative
    1e-5 of the row's selection threshold;
  * gathers: bit-exact against the oracle's gather of the GPU's indices.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import kvc_oracle as O

RTOL = 1e-3
ATOL = 1e-30
GAP = 1e-5


def dev(a: np.ndarray, dtype: str = "f32") -> torch.Tensor:
    """Upload a stored array (float32, bf16 bits as uint16, or integers)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw stored bits of a device tensor (uint16 for bf16, float32 otherwise)."""
    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def check_scores(gpu: np.ndarray, ref: np.ndarray, what: str = "scores"):
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref)
    bad = err > RTOL * np.abs(ref) + ATOL
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(np.abs(ref), 1e-300), 0)), ref.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu {gpu[i]!r} oracle {ref[i]!r}")


def check_kept(idx_gpu: np.ndarray, scores_gpu: np.ndarray, scores_ref: np.ndarray, k: int, n_tail: int):
    N = scores_ref.shape[-1]
    ig = np.asarray(idx_gpu).reshape(-1, k).astype(np.int64)
    sg = np.asarray(scores_gpu, dtype=np.float32).reshape(-1, N).astype(np.float64)
    sr = np.asarray(scores_ref).reshape(-1, N)
    # (a) self-consistency, bit-exact
    self_ref = O.topk_select(sg, k, n_tail)
    if not np.array_equal(ig, self_ref):
        r = int(np.argmax((ig != self_ref).any(axis=1)))
        raise AssertionError(f"kept set differs from the oracle selection on the GPU scores (row {r})")
    # (b) agreement with the oracle outside ambiguous positions
    ref_idx = O.topk_select(sr, k, n_tail)
    E, kp = N - n_tail, k - n_tail
    for r in range(sr.shape[0]):
        if kp <= 0 or kp >= E:
            assert np.array_equal(ig[r], ref_idx[r])
            continue
        elig = sr[r, :E]
        t = np.sort(elig)[::-1][kp - 1]
        amb = np.zeros(N, dtype=bool)
        amb[:E] = np.abs(elig - t) <= GAP * abs(t)
        a = set(ig[r][~amb[ig[r]]].tolist())
        b = set(ref_idx[r][~amb[ref_idx[r]]].tolist())
        if a != b:
            raise AssertionError(f"row {r}: kept sets differ outside ambiguous positions: "
                                 f"gpu-only {sorted(a - b)[:8]} oracle-only {sorted(b - a)[:8]}")
        assert set(range(E, N)) <= set(ig[r].tolist())


def check_gather(k_out, v_out, k_host, v_host, idx_gpu, chan_host=None):
    ko, vo = O.gather_compact(k_host, v_host, np.asarray(idx_gpu), chan_keep=chan_host)
    assert np.array_equal(host_bits(k_out).view(np.uint8), np.ascontiguousarray(ko).view(np.uint8)), "K gather"
    if v_out is not None:
        assert np.array_equal(host_bits(v_out).view(np.uint8), np.ascontiguousarray(vo).view(np.uint8)), "V gather"
