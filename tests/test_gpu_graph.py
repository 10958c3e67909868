"""A SnapKV layer path (window scores -> top-k with the window forced -> gather)
captured into a HIP graph and replayed (GPU).

The calls take no allocation and enqueue no memset, so the captured graph must
reproduce the eager results bit for bit on every replay.  Three replays, each
after eager work of the program's own and a synchronisation.
"""
from __future__ import annotations

import sys

import pytest
import torch

from kv_cache_compression_window_amd import synth
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


def test_snapkv_path_graph_replays_match_eager():
    from kv_cache_compression_window_amd import binding as L
    print("[gpu-graph] snapkv S=5000 captured path", file=sys.stderr, flush=True)
    p = synth.snapkv(1, S=5000, w=64, H=32, Hkv=8, D=128)
    keep = 1024
    q, k, v = dev(p.q, "bf16"), dev(p.k, "bf16"), dev(p.v, "bf16")
    st = torch.cuda.Stream()
    scores = torch.empty((p.B, p.Hkv, p.S), dtype=torch.float32, device="cuda")
    idx = torch.empty((p.B, p.Hkv, keep), dtype=torch.int32, device="cuda")
    ko = torch.empty((p.B, p.Hkv, keep, p.D), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    ws = torch.empty(L.window_scores_ws_bytes(p.B, p.H, p.Hkv, p.S, p.D, p.w), dtype=torch.uint8, device="cuda")
    tk_ws = torch.empty(L.topk_ws_bytes(p.B * p.Hkv, p.S), dtype=torch.uint8, device="cuda")
    calls = [L.bind_window_scores(q, k, scores, ws, st, reduce=L.KVC_REDUCE_GROUP, causal=True),
             L.bind_topk_select(scores, keep, p.w, idx, tk_ws, st),
             L.bind_gather_compact(k, v, idx, ko, vo, st)]
    st.wait_stream(torch.cuda.current_stream())
    for f in calls:
        f()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (scores, idx, ko, vo)]
    for t in (scores, idx, ko, vo):
        t.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for f in calls:
            f()
    torch.cuda.synchronize()
    for r in range(3):
        x = torch.randn(1 << 20, device="cuda")
        x.mul_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b, name in zip(eager, (scores, idx, ko, vo), ("scores", "idx", "k_out", "v_out")):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager call"
