"""The five workloads of the scoring-and-pruning path and the readings they use.

Each entry names the method, its sizes and its knobs.  The knobs not fixed by
the pages are readings:
  * logit scale 1/sqrt(D) (the SDPA default for attention "after sdpa");
  * window rows are causal (row i of the window is query position S-w+i);
  * TOVA averages over all query heads and repeats the row per KV head; SnapKV
    and Scissorhands average over the query heads of each GQA group;
  * the window mean is a mean (rows of the score sum to 1);
  * the SnapKV budget includes the window; kept indices are ascending and
    ties keep the lowest index.
"""
from __future__ import annotations

from dataclasses import dataclass

REDUCE_GROUP = 0
REDUCE_ALL_HEADS = 1


@dataclass(frozen=True)
class Workload:
    name: str
    method: str  # "tova", "snapkv", "scissorhands", "think_snapkv"
    B: int
    H: int
    Hkv: int
    S: int
    D: int
    w: int
    keep: int  # tokens kept per KV head (including the forced window)
    dtype: str
    reduce: int
    causal: int
    n_tail: int  # forced-keep tail (the observation window for SnapKV)
    d_keep: int = 0  # ThinK: key channels kept per KV head
    steps: int = 0  # Scissorhands decode steps
    hist_len: int = 0  # Scissorhands circular history length
    evict_every: int = 0
    n_evict: int = 0
    layers: int = 1  # distinct layers rotated when timing (defeats the 256 MB Infinity Cache)


TOVA_TINY = Workload("tova_tiny_s512", "tova", 1, 4, 2, 512, 64, 1, 128, "f32", REDUCE_ALL_HEADS, 0, 0)
# 32 distinct layers per timed step: the depth of the Llama-3-8B-shaped model the
# layer shape comes from (a step compresses every layer of one prefill once)
SNAPKV_32K = Workload("snapkv_32k_gqa32x8_w64", "snapkv", 1, 32, 8, 32768, 128, 64, 4096, "bf16",
                      REDUCE_GROUP, 1, 64, layers=32)
TOVA_BATCHED = Workload("tova_batched_b16_s8192", "tova", 16, 32, 8, 8192, 128, 1, 4096, "bf16",
                        REDUCE_ALL_HEADS, 0, 0, layers=2)
SCISSOR_DECODE = Workload("scissorhands_decode_b8_c4096", "scissorhands", 8, 32, 8, 4096, 128, 1, 0,
                          "bf16", REDUCE_GROUP, 0, 0, steps=800, hist_len=400, evict_every=64,
                          n_evict=64, layers=8)
SCISSOR_QUEUE = Workload("scissorhands_queue_decode_b8_c4096", "scissorhands_queue", 8, 32, 8, 4096, 128, 1, 3840,
                         "bf16", REDUCE_GROUP, 0, 0, steps=800, hist_len=400, evict_every=64, n_evict=64, layers=8)
THINK_128K = Workload("think_snapkv_128k_gqa32x8_w64", "think_snapkv", 1, 32, 8, 131072, 128, 64, 8192,
                      "bf16", REDUCE_GROUP, 1, 64, d_keep=64, layers=2)

ALL = [TOVA_TINY, SNAPKV_32K, TOVA_BATCHED, SCISSOR_DECODE, THINK_128K]
# Scissorhands with insertion and an eviction queue: keep = the protected prompt
# length P (global_tokens = -1), n_evict = drop_amount (queue length)
NEXT = [SCISSOR_QUEUE]
