"""Seeded synthetic inputs for KV-cache scoring and pruning.

This module only draws random numbers, rounds them to the stored precision and
lays them out.  It holds none of the scoring, selection or compaction
arithmetic, so the HIP path and the fp64 oracle both take their inputs from it
without sharing any of the method.

Recipe (every tensor):
  * normal draws come from ``numpy.random.Generator(PCG64)`` seeded with
    ``SeedSequence([SEED_ROOT, workload_id, layer, tensor_id, chunk])``; each
    tensor is filled in chunks of ``CHUNK`` elements so that the draws can run
    on several threads and still give the same values on every machine;
  * structure (heavy-hitter positions, per-channel scales) is drawn from
    ``SeedSequence([SEED_ROOT, workload_id, layer, STRUCT_ID])``;
  * bf16 tensors are rounded from the fp32 draws by round-to-nearest-even and
    kept as raw ``uint16`` bit patterns; fp32 tensors are kept as ``float32``.

The shapes follow the attention layers the pages discuss (grouped-query
attention with 32 query heads and 8 KV heads, head_dim 128, a 64-query
observation window).  Real activations of a trained model are not available;
these draws stand in for them.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED_ROOT = 20261202
CHUNK = 1 << 22
T_Q, T_K, T_V = 1, 2, 3
STRUCT_ID = 99

# workload ids used in seeds
W_TOVA_TINY, W_SNAPKV_32K, W_TOVA_BATCHED, W_SCISSOR, W_THINK_128K, W_RANDOM = 1, 2, 3, 4, 5, 6


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(shape, seed_prefix) -> np.ndarray:
    """Standard normal float32 array; chunk c uses SeedSequence(seed_prefix + [c])."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    chunks = [(c, c * CHUNK, min(n, (c + 1) * CHUNK)) for c in range((n + CHUNK - 1) // CHUNK)]

    def fill(arg):
        c, lo, hi = arg
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_prefix) + [c])))
        out[lo:hi] = g.standard_normal(hi - lo, dtype=np.float32)

    if len(chunks) > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, chunks))
    else:
        for a in chunks:
            fill(a)
    return out.reshape(shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs here are finite draws, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a stored tensor (float32 array or bf16 bits)."""
    if dtype == "bf16":
        return bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


@dataclass
class Problem:
    """One layer's inputs.  q/k/v hold the stored representation."""

    B: int
    H: int
    Hkv: int
    S: int
    D: int
    w: int
    dtype: str  # "f32" or "bf16"
    q: np.ndarray  # [B,H,w,D]
    k: np.ndarray  # [B,Hkv,S,D]
    v: np.ndarray | None  # [B,Hkv,S,D]
    heavy: list = field(default_factory=list)  # per batch: heavy-hitter positions

    @property
    def G(self) -> int:
        return self.H // self.Hkv

    def q64(self):
        return stored_to_f64(self.q, self.dtype)

    def k64(self):
        return stored_to_f64(self.k, self.dtype)

    def v64(self):
        return stored_to_f64(self.v, self.dtype)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(x32) if dtype == "bf16" else x32


def _struct_rng(wid: int, layer: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, wid, layer, STRUCT_ID])))


def tova_tiny(layer: int = 0, S: int = 512) -> Problem:
    """TOVA tiny: B=1, 4 query / 2 KV heads, D=64, w=1, fp32.

    2% of key positions (shared by both KV heads) are replaced by 4x the mean
    query direction of the KV head's group, scaled to sqrt(D) (the expected
    norm of an N(0,1) key), i.e. K = 4*sqrt(D)*u_g with u_g the unit mean of
    the group's window queries.
    """
    B, H, Hkv, D, w = 1, 4, 2, 64, 1
    base = [SEED_ROOT, W_TOVA_TINY, layer]
    q = normal_f32((B, H, w, D), base + [T_Q])
    k = normal_f32((B, Hkv, S, D), base + [T_K])
    v = normal_f32((B, Hkv, S, D), base + [T_V])
    rs = _struct_rng(W_TOVA_TINY, layer)
    n_heavy = int(round(0.02 * S))
    pos = np.sort(rs.choice(S, size=n_heavy, replace=False))
    G = H // Hkv
    for g in range(Hkv):
        m = q[0, g * G:(g + 1) * G].astype(np.float64).reshape(-1, D).mean(axis=0)
        u = m / np.linalg.norm(m)
        k[0, g, pos, :] = (4.0 * np.sqrt(D) * u).astype(np.float32)
    return Problem(B, H, Hkv, S, D, w, "f32", q, k, v, [pos])


def snapkv(layer: int = 0, B: int = 1, H: int = 32, Hkv: int = 8, S: int = 32768, D: int = 128,
           w: int = 64, heavy_frac: float = 0.01, wid: int = W_SNAPKV_32K, with_v: bool = True) -> Problem:
    """SnapKV prefill layer: bf16 N(0,1) Q/K/V; 1% of the prefix positions
    (shared by all KV heads) have K scaled by 4."""
    base = [SEED_ROOT, wid, layer]
    q = normal_f32((B, H, w, D), base + [T_Q])
    k = normal_f32((B, Hkv, S, D), base + [T_K])
    v = normal_f32((B, Hkv, S, D), base + [T_V]) if with_v else None
    rs = _struct_rng(wid, layer)
    heavy = []
    for b in range(B):
        n_heavy = int(round(heavy_frac * (S - w)))
        pos = np.sort(rs.choice(S - w, size=n_heavy, replace=False)) if n_heavy else np.zeros(0, np.int64)
        k[b, :, pos, :] *= 4.0
        heavy.append(pos)
    return Problem(B, H, Hkv, S, D, w, "bf16", _store(q, "bf16"), _store(k, "bf16"),
                   _store(v, "bf16") if with_v else None, heavy)


def tova_batched(layer: int = 0, B: int = 16, H: int = 32, Hkv: int = 8, S: int = 8192, D: int = 128) -> Problem:
    """TOVA batched: bf16 N(0,1); per sequence a fraction f_b ~ U[1%,3%] of the
    positions (shared by the KV heads of that sequence) have K scaled by 4."""
    base = [SEED_ROOT, W_TOVA_BATCHED, layer]
    w = 1
    q = normal_f32((B, H, w, D), base + [T_Q])
    k = normal_f32((B, Hkv, S, D), base + [T_K])
    v = normal_f32((B, Hkv, S, D), base + [T_V])
    rs = _struct_rng(W_TOVA_BATCHED, layer)
    heavy = []
    for b in range(B):
        f = rs.uniform(0.01, 0.03)
        pos = np.sort(rs.choice(S, size=int(round(f * S)), replace=False))
        k[b, :, pos, :] *= 4.0
        heavy.append(pos)
    return Problem(B, H, Hkv, S, D, w, "bf16", _store(q, "bf16"), _store(k, "bf16"), _store(v, "bf16"), heavy)


def scissor_cache(layer: int = 0, B: int = 8, Hkv: int = 8, C: int = 4096, D: int = 128) -> np.ndarray:
    """Scissorhands decode cache keys: bf16 bits [B,Hkv,C,D] ~ N(0,1)."""
    return bf16_bits(normal_f32((B, Hkv, C, D), [SEED_ROOT, W_SCISSOR, layer, T_K]))


def scissor_query(layer: int, t: int, B: int = 8, H: int = 32, D: int = 128) -> np.ndarray:
    """Decode query of step t: bf16 bits [B,H,1,D] ~ N(0,1)."""
    return bf16_bits(normal_f32((B, H, 1, D), [SEED_ROOT, W_SCISSOR, layer, T_Q, 1_000_000 + t]))


def scissor_new_tokens(layer: int, steps: int, B: int = 8, Hkv: int = 8, D: int = 128):
    """K and V of the token each decode step inserts: bf16 bits [steps,B,Hkv,D] ~ N(0,1)."""
    k = bf16_bits(normal_f32((steps, B, Hkv, D), [SEED_ROOT, W_SCISSOR, layer, T_K, 2_000_000]))
    v = bf16_bits(normal_f32((steps, B, Hkv, D), [SEED_ROOT, W_SCISSOR, layer, T_V, 2_000_000]))
    return k, v


def think_snapkv(layer: int = 0, B: int = 1, H: int = 32, Hkv: int = 8, S: int = 131072, D: int = 128,
                 w: int = 64, with_v: bool = True) -> Problem:
    """ThinK + SnapKV long-context layer: bf16 N(0,1) with per-channel scales
    s = exp(U[ln 1/4, ln 4]) drawn independently per (KV head, channel) for K
    and per (query head, channel) for Q; V is not scaled."""
    base = [SEED_ROOT, W_THINK_128K, layer]
    q = normal_f32((B, H, w, D), base + [T_Q])
    k = normal_f32((B, Hkv, S, D), base + [T_K])
    v = normal_f32((B, Hkv, S, D), base + [T_V]) if with_v else None
    rs = _struct_rng(W_THINK_128K, layer)
    s_k = np.exp(rs.uniform(np.log(0.25), np.log(4.0), size=(Hkv, D))).astype(np.float32)
    s_q = np.exp(rs.uniform(np.log(0.25), np.log(4.0), size=(H, D))).astype(np.float32)
    k *= s_k[None, :, None, :]
    q *= s_q[None, :, None, :]
    return Problem(B, H, Hkv, S, D, w, "bf16", _store(q, "bf16"), _store(k, "bf16"),
                   _store(v, "bf16") if with_v else None, [])


def random_problem(seed: int, B: int, H: int, Hkv: int, S: int, D: int, w: int, dtype: str = "bf16",
                   heavy_frac: float = 0.0, heavy_scale: float = 4.0, q_scale: float = 1.0,
                   with_v: bool = True) -> Problem:
    """General seeded problem for parity and property tests."""
    base = [SEED_ROOT, W_RANDOM, seed]
    q = normal_f32((B, H, w, D), base + [T_Q]) * np.float32(q_scale)
    k = normal_f32((B, Hkv, S, D), base + [T_K])
    v = normal_f32((B, Hkv, S, D), base + [T_V]) if with_v else None
    rs = _struct_rng(W_RANDOM, seed)
    heavy = []
    for b in range(B):
        n = int(round(heavy_frac * S))
        pos = np.sort(rs.choice(S, size=n, replace=False)) if n else np.zeros(0, np.int64)
        k[b, :, pos, :] *= np.float32(heavy_scale)
        heavy.append(pos)
    return Problem(B, H, Hkv, S, D, w, dtype, _store(q, dtype), _store(k, dtype),
                   _store(v, dtype) if with_v else None, heavy)


def random_valid(seed: int, B: int, Hkv: int, S: int, p_hole: float) -> np.ndarray:
    """uint8 [B,Hkv,S] validity mask with holes at rate p_hole."""
    rs = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, W_RANDOM, seed, 7])))
    return (rs.random((B, Hkv, S)) >= p_hole).astype(np.uint8)


def random_scores(seed: int, rows: int, n: int, n_levels: int = 0) -> np.ndarray:
    """float32 [rows,n] scores; with n_levels > 0 values come from a small set
    so that exact ties are common."""
    rs = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, W_RANDOM, seed, 8])))
    if n_levels:
        return (rs.integers(0, n_levels, size=(rows, n)).astype(np.float32) / np.float32(n_levels))
    return rs.random((rows, n), dtype=np.float32)
