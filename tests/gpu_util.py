"""Helpers shared by the GPU tests: device upload and the parity checks.

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


def unpack_planes(hist: np.ndarray, bg: int, C: int) -> np.ndarray:
    """[C, hist_len] 0/1 matrix of the bit-planes of row bg of a
    [hist_len, rows, ceil(C/32)] int32 history."""
    words = np.ascontiguousarray(hist[:, bg, :]).astype(np.uint32)  # [hist_len, W]
    bits = np.unpackbits(words.view(np.uint8).reshape(words.shape[0], -1), bitorder="little", axis=1)
    return bits[:, :C].T.astype(np.int8)


def unpack_all_planes(hist: np.ndarray, C: int) -> np.ndarray:
    """[rows, C, hist_len] 0/1 matrix of every row's bit-planes."""
    words = np.ascontiguousarray(hist).astype(np.uint32)  # [hist_len, rows, W]
    hl, rows, W = words.shape
    bits = np.unpackbits(words.view(np.uint8).reshape(hl, rows, W * 4), bitorder="little", axis=2)
    return np.ascontiguousarray(bits[:, :, :C].transpose(1, 2, 0))


def oracle_state(valid, planes: np.ndarray, n_rec: int, hist_len: int, since=None) -> "O.LowAttentionState":
    """The oracle's Scissorhands state taken from the GPU's: validity [..., C],
    planes [..., C, hist_len] (recording r lives in plane r % hist_len), the
    recordings made so far and the per-slot observation start (None: 0)."""
    valid = np.asarray(valid, dtype=bool)
    shape = valid.shape
    valid3 = valid.reshape((-1,) + shape[-1:])[None] if valid.ndim != 3 else valid
    planes = np.asarray(planes).reshape(valid3.shape + (hist_len,))
    recs = {r: planes[..., r % hist_len] for r in range(max(0, n_rec - hist_len), n_rec)}
    since = np.zeros(valid3.shape, dtype=np.int64) if since is None else np.asarray(since).reshape(valid3.shape)
    return O.LowAttentionState.from_recordings(valid3, since, recs, n_rec, hist_len)


def low_bits_agree(got: np.ndarray, low: np.ndarray, probs: np.ndarray, valid: np.ndarray) -> bool:
    """The GPU's low bits equal the oracle's except where the probability lies
    within a relative 1e-5 of 1/S_t (both sides decide from fp32 vs fp64 sums)."""
    n_valid = np.asarray(valid).sum(axis=-1, keepdims=True)
    near = np.abs(probs * n_valid - 1.0) <= GAP
    return bool(np.array_equal(np.asarray(got, dtype=bool)[~near], np.asarray(low, dtype=bool)[~near]))
