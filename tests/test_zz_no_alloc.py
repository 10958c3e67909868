"""kvc_window_scores_noalloc: the allocation-free entry point (GPU).

It runs the kvc_window_scores kernels on the library's fixed per-GPU scratch,
so its scores must equal kvc_window_scores' bit for bit (both reduce in a
fixed order).  Two calls in a row, the second on a smaller input, on both
kernel paths (two-pass and stored logits); the scratch keeps the first call's
contents, which the second must not depend on.
"""
from __future__ import annotations

import sys

import pytest
import torch

from kv_cache_compression_window_amd import synth
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


def lib():
    from kv_cache_compression_window_amd import binding
    return binding


def say(msg):
    print(f"[no-alloc] {msg}", file=sys.stderr, flush=True)


def both(L, q, k, valid=None, reduce=0, causal=True):
    ref = L.kvc_window_scores(q, k, valid=valid, reduce=reduce, causal=causal)
    got = torch.full_like(ref, float("nan"))
    L.kvc_window_scores_noalloc(q, k, got, valid=valid, reduce=reduce, causal=causal)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("shapes,w,reduce", [
    (((1, 32, 8, 5000), (1, 16, 4, 1500)), 64, 0),   # two-pass path (G*w > 16), causal window
    (((8, 32, 8, 4096), (2, 8, 2, 700)), 1, 0),      # stored-logits path (decode-shaped, w = 1)
    (((4, 32, 8, 2048), (1, 4, 2, 512)), 1, 1),      # stored logits, mean over all heads
])
def test_noalloc_equals_workspace_call(shapes, w, reduce):
    L = lib()
    for i, (B, H, Hkv, S) in enumerate(shapes):
        say(f"call {i}: B={B} H={H} Hkv={Hkv} S={S} w={w} reduce={reduce}")
        p = synth.random_problem(70 + i, B, H, Hkv, S, 128, w, dtype="bf16", heavy_frac=0.02)
        q, k = dev(p.q, "bf16"), dev(p.k, "bf16")
        valid = None
        if w == 1:
            vm = torch.ones((B, Hkv, S), dtype=torch.uint8)
            vm[..., 3::7] = 0  # holes, as a Scissorhands cache has after evictions
            valid = vm.cuda()
        ref, got = both(L, q, k, valid=valid, reduce=reduce, causal=w > 1)
        assert torch.equal(got, ref), f"call {i}: scores differ from kvc_window_scores"

