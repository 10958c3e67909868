"""Throughput of the KV-cache scoring-and-pruning path on one MI355X.

Default workload (the one the metric is quoted on): SnapKV prefill on a
Llama-3-8B-shaped layer (batch 1, 32 query heads, 8 KV heads, head_dim 128,
S = 32768 cached positions, a 64-query observation window that is always kept,
4096 positions kept per KV head), bf16 N(0,1) Q/K/V with 1% of the prefix keys
scaled by 4.  One step runs the whole path on each of 32 distinct layers (the
model's depth): window scores -> top-k with the window forced -> gather of the
kept K/V.  The layers together (4.3 GB of K/V) exceed the 256 MB Infinity Cache
many times over, so every layer's keys come from HBM.

--workload selects one of the other four workloads instead (TOVA tiny, TOVA
batched, Scissorhands decode, ThinK + SnapKV at 128k); each prints the same kind
of line with its own metric.

Prints one JSON line.  value = KV tokens scored and pruned per second per layer
(B * S * layers * steps / elapsed; token-steps for the decode workload).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV tokens scored+pruned/s per layer (32k ctx, GQA 32/8) + % of HBM roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK = 2.5e15  # dense bf16 MFMA, FLOP/s
# sources whose code the recorded HBM counters of a kernel belong to
SCORE_SOURCES = ["window_scores.hip", "kvc_device.h", "kvc_plan.h"]
GATHER_SOURCES = ["gather.hip", "kvc_device.h", "kvc_launch.h"]
WORKLOADS = ["snapkv_32k", "tova_tiny", "tova_batched", "scissor_decode", "think_128k", "think_128k_kc",
             "snapkv_think_32k", "scissor_queue_decode"]
# (timed steps, warm-up steps).  The timed regions last 0.1-0.5 s: measured on
# MI355X, SnapKV 32k (then 8 layers per step) read 6.07e8 tokens/s after 10
# warm-up steps and 6.22e8 after 300 (the clocks settle), and ThinK 128k 5.09e8
# over 10 steps but 5.84e8 over 100 (with two layers per step the streams' start
# and drain weigh on a short run).  The decode workloads time one whole 800-step
# run.
DEFAULT_STEPS = {"snapkv_32k": (250, 50), "tova_tiny": (2000, 200), "tova_batched": (100, 10),
                 "scissor_decode": (800, 0), "think_128k": (200, 20), "think_128k_kc": (200, 20),
                 "snapkv_think_32k": (250, 50), "scissor_queue_decode": (800, 0)}


# kvc_window_scores_ex's compute-unit budget for the workloads whose score calls
# overlap on several streams (0: each call planned to fill the GPU's 256 CUs).
# Measured on MI355X with 3 streams, in interleaved runs: half the GPU per call
# (128) gives the two-pass workloads 5-10% more tokens/s than the whole GPU;
# below that, the budget that leaves the other streams' top-k, gathers and
# channel kernels free CUs without idling the chip depends on how much of that
# work a layer has: SnapKV 32k peaks at 96 (+2% over 128), SnapKV then ThinK at
# 112 (+11%), ThinK 128k at 128 (96: -13%).  The stored-logits workloads gain
# nothing.
DEFAULT_CU_BUDGET = {"snapkv_32k": 96, "snapkv_think_32k": 112, "think_128k": 128, "think_128k_kc": 128}


def kernel_hash(sources=SCORE_SOURCES) -> str:
    """Hash of a kernel's code: its sources without their // comments and blank
    lines, so that a comment edit does not void the recorded counters."""
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "kv_cache_compression_window_amd", "csrc", f), encoding="utf-8") as fh:
            lines = (line.split("//", 1)[0].rstrip() for line in fh.read().splitlines())
            h.update("\n".join(line for line in lines if line).encode())
    return h.hexdigest()[:16]


def score_kernel_hash() -> str:
    return kernel_hash(SCORE_SOURCES)


def recorded_traffic(name: str, sources, cu_budget: int = 0):
    """HBM bytes per launch of the dominant kernel from profiles/traffic_<name>.json
    (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated), or None when there is no such
    record or it was taken on other kernel code or another compute-unit budget."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    if tr.get("kernel_hash") != kernel_hash(sources) or tr.get("cu_budget", 0) != cu_budget:
        return None
    return tr.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default="snapkv_32k", choices=WORKLOADS)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None, help="distinct layers rotated per step")
    ap.add_argument("--streams", type=int, default=3,
                    help="layers are spread round-robin over this many streams in the timed region")
    ap.add_argument("--kernel-reps", type=int, default=20,
                    help="passes over the layers, each timed as one run of back-to-back calls of the dominant kernel")
    ap.add_argument("--cu-budget", type=int, default=None,
                    help="kvc_window_scores_ex's compute-unit budget per score call (0: the whole GPU; "
                         "default per workload)")
    ap.add_argument("--no-alone", action="store_true",
                    help="with a compute-unit budget, skip timing the calls planned to fill the GPU alone")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU work budget of the oracle baseline")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the read-ceiling and exp-rate measurements")
    ap.add_argument("--no-graph", action="store_true", help="skip the hipGraph-captured variant")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM counters)")
    a = ap.parse_args()
    st, wu = DEFAULT_STEPS[a.workload]
    a.steps = st if a.steps is None else a.steps
    a.warmup = wu if a.warmup is None else a.warmup
    if a.cu_budget is None:
        a.cu_budget = DEFAULT_CU_BUDGET.get(a.workload, 0)
    return a


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1]))
    except Exception:  # pragma: no cover
        return 1


def cpu_model() -> str:
    """The host CPU's model name, as /proc/cpuinfo gives it."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def timed_oracle(fn, budget_s):
    """Run fn(n) for n = 0, 1, ... for about budget_s seconds; (calls, seconds)."""
    n = 0
    t0 = time.perf_counter()
    while True:
        fn(n)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return n, el


def measure_ceilings(c, reps: int = 5) -> dict:
    """The box's own ceilings, measured in this run with libkvc_bench.so: a plain
    streaming read of 2 GiB from HBM (the best of `reps` runs) and the v_exp_f32
    rate (256 x 512 threads, eight independent exp2 chains each)."""
    import ctypes
    torch = c.torch
    lib = ctypes.CDLL(os.path.join(ROOT, "kv_cache_compression_window_amd", "libkvc_bench.so"))
    lib.kvc_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.kvc_bench_exp_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    st = torch.cuda.current_stream(c.dev)
    sh = ctypes.c_void_p(st.cuda_stream)
    nbytes, blocks = 2 << 30, 4096
    buf = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=c.dev)
    out = torch.empty(blocks * 512, dtype=torch.int32, device=c.dev)
    best = float("inf")
    for r in range(reps + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        assert lib.kvc_bench_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()),
                                         blocks, sh) == 0
        b.record(st)
        torch.cuda.synchronize()
        if r:  # the first run warms up
            best = min(best, a.elapsed_time(b))
    del buf
    iters, eblocks = 20000, 256
    fout = torch.empty(eblocks * 512, dtype=torch.float32, device=c.dev)
    times = []
    for r in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        assert lib.kvc_bench_exp_rate(ctypes.c_void_p(fout.data_ptr()), eblocks, iters, sh) == 0
        b.record(st)
        torch.cuda.synchronize()
        if r:
            times.append(a.elapsed_time(b))
    exps = eblocks * 512 * 8 * iters
    return {"stream_read_gbs": round(nbytes / (best * 1e-3) / 1e9, 1),
            "exp_per_s": float(f"{exps / (min(times) * 1e-3):.4g}")}


class Ctx:
    def __init__(self, args):
        import torch

        from kv_cache_compression_window_amd import binding, configs, synth
        self.args, self.torch, self.L, self.configs, self.synth = args, torch, binding, configs, synth
        self.dev = torch.device("cuda:0")
        self.streams = [torch.cuda.Stream(device=self.dev) for _ in range(args.streams)]

    def up(self, a, dtype="bf16"):
        t = self.torch
        if dtype == "bf16":
            return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(t.bfloat16).to(self.dev)
        return t.from_numpy(np.ascontiguousarray(a)).to(self.dev)

    def empty(self, shape, dtype):
        return self.torch.empty(shape, dtype=dtype, device=self.dev)


# ---------------------------------------------------------------------------
# Workloads.  Each returns a dict:
#   step()            one step of the timed region (all layers)
#   reset()           optional: restore the initial state before a timed run
#   units_per_step    tokens (or token-steps) per step, summed over the layers
#   layers            distinct layers per step
#   layer_bytes       algorithmic HBM bytes per layer and step
#   kernel            (label, [calls on stream 0], algorithmic bytes per call, traffic)
#   cpu(budget)       oracle baseline dict
#   config            extra config keys
# ---------------------------------------------------------------------------

def wl_snapkv_32k(c: Ctx, then_think: bool = False) -> dict:
    """SnapKV at 32k.  then_think: ThinK after it, on the kept keys only (channel
    scores of the kept keys, channel top-k, kept keys stored with their 64 best
    channels)."""
    L, torch, cfg = c.L, c.torch, c.configs.SNAPKV_32K
    B, H, Hkv, S, D, w, keep = cfg.B, cfg.H, cfg.Hkv, cfg.S, cfg.D, cfg.w, cfg.keep
    dk = 64
    nl = c.args.layers or cfg.layers
    layers, host0 = [], None
    for layer in range(nl):
        p = c.synth.snapkv(layer)
        layers.append(dict(q=c.up(p.q), k=c.up(p.k), v=c.up(p.v)))
        host0 = host0 or p
    cub = c.args.cu_budget
    ws_bytes = L.window_scores_ws_bytes(B, H, Hkv, S, D, w, cu_budget=cub)
    s0 = c.streams[0]
    for i, ly in enumerate(layers):
        st = c.streams[i % len(c.streams)]
        ly["scores"] = c.empty((B, Hkv, S), torch.float32)
        ly["idx"] = c.empty((B, Hkv, keep), torch.int32)
        ly["k_out"] = c.empty((B, Hkv, keep, D), torch.bfloat16)
        ly["v_out"] = c.empty((B, Hkv, keep, D), torch.bfloat16)
        ly["ws"] = c.empty(ws_bytes, torch.uint8)
        ly["tk_ws"] = c.empty(L.topk_ws_bytes(B * Hkv, S), torch.uint8)
        ly["calls"] = [L.bind_window_scores(ly["q"], ly["k"], ly["scores"], ly["ws"], st, reduce=L.KVC_REDUCE_GROUP,
                                            causal=True, cu_budget=cub),
                       L.bind_topk_select(ly["scores"], keep, w, ly["idx"], ly["tk_ws"], st),
                       L.bind_gather_compact(ly["k"], ly["v"], ly["idx"], ly["k_out"], ly["v_out"], st)]
        if then_think:
            ly["cs"] = c.empty((B, Hkv, D), torch.float32)
            ly["ch"] = c.empty((B, Hkv, dk), torch.int32)
            ly["rows"] = torch.arange(keep, dtype=torch.int32, device="cuda").expand(B, Hkv, keep).contiguous()
            ly["kc"] = c.empty((B, Hkv, keep, dk), torch.bfloat16)
            ly["cs_ws"] = c.empty(L.channel_scores_ws_bytes(B, H, Hkv, keep, D, w), torch.uint8)
            ly["calls"] += [L.bind_channel_scores(ly["q"], ly["k_out"], ly["cs"], ly["cs_ws"], st),
                            L.bind_topk_select(ly["cs"], dk, 0, ly["ch"], ly["tk_ws"], st),
                            L.bind_gather_compress(ly["k_out"], None, ly["rows"], ly["ch"], ly["kc"], None, st)]
        ly["kcall"] = L.bind_window_scores(ly["q"], ly["k"], ly["scores"], ly["ws"], s0, reduce=L.KVC_REDUCE_GROUP,
                                           causal=True, cu_budget=cub)
        if cub != 0:  # own workspace and scores: the step's outputs stay those of the budgeted calls
            ly["ws1"] = c.empty(L.window_scores_ws_bytes(B, H, Hkv, S, D, w), torch.uint8)
            ly["scores1"] = c.empty((B, Hkv, S), torch.float32)
            ly["kcall1"] = L.bind_window_scores(ly["q"], ly["k"], ly["scores1"], ly["ws1"], s0,
                                                reduce=L.KVC_REDUCE_GROUP, causal=True)

    def step():
        for ly in layers:
            for f in ly["calls"]:
                f()

    # algorithmic bytes per layer: K read once, Q read, scores written and read
    # by the top-k, indices written and read, kept K and V read and written
    k_bytes, q_bytes, s_bytes = B * Hkv * S * D * 2, B * H * w * D * 2, B * Hkv * S * 4
    i_bytes, g_bytes = B * Hkv * keep * 4, 2 * 2 * B * Hkv * keep * D * 2
    if then_think:
        # kept K read by the channel scores, kept channels read and written
        g_bytes += B * Hkv * keep * D * 2 + 2 * B * Hkv * keep * dk * 2
    layer_bytes = k_bytes + q_bytes + 2 * s_bytes + 2 * i_bytes + g_bytes

    def cpu(budget):
        from oracle import kvc_oracle as O
        q64, k64 = host0.q64(), host0.k64()
        G = H // Hkv

        def one(n):
            g = n % Hkv
            qg, kg = q64[:, g * G:(g + 1) * G], k64[:, g:g + 1]
            if then_think:
                s, idx, cs, ch = O.snapkv_then_think(qg, kg, keep, dk)
                ko, _ = O.gather_compact(host0.k[:, g:g + 1], host0.v[:, g:g + 1], idx)
                O.gather_compress(ko, None, np.broadcast_to(np.arange(keep), idx.shape), ch)
            else:
                s, idx = O.snapkv(qg, kg, keep)
                O.gather_compact(host0.k[:, g:g + 1], host0.v[:, g:g + 1], idx)
        n, el = timed_oracle(one, budget)
        # one KV head is 1/Hkv of a layer's work on all S positions
        return {"value": round(B * S * n / Hkv / el, 1), "unit": "tokens/s", "cores": blas_threads(),
                "kind": "oracle", "sample": f"{n} KV heads (of {Hkv} per layer) of layer 0, S={S}, fp64 numpy "
                                            f"oracle (scores, top-k, gather), {el:.1f} s"}

    traffic = recorded_traffic("window_scores_snapkv_32k" + ("_then_think" if then_think else ""), SCORE_SOURCES, cub)
    # the score call's contraction and exps: one contraction is 2*R*S*D flops per
    # (b, g), R = G*w rows; the two passes compute it twice, with one exp2 per
    # logit in each
    one_contraction = 2.0 * B * H * w * S * D
    compute = {"mfma_flops": 2 * one_contraction, "one_contraction_flops": one_contraction,
               "exps": 2 * B * H * w * S}

    def check_outputs():
        return [t.clone() for t in (layers[0]["scores"], layers[0]["idx"], layers[0]["k_out"], layers[-1]["idx"])]
    return dict(step=step, units_per_step=B * S * nl, layers=nl, layer_bytes=layer_bytes, compute=compute,
                check_outputs=check_outputs,
                kernel=("kvc_window_scores (pass 1 + pass 2)", [ly["kcall"] for ly in layers],
                        k_bytes + q_bytes + s_bytes, traffic),
                kernel_alone=[ly["kcall1"] for ly in layers] if cub != 0 else None,
                cpu=cpu, metric=(f"KV tokens scored+pruned/s per layer ({cfg.name}, then ThinK on the kept keys)"
                                 if then_think else METRIC), unit="tokens/s", dtype="bf16",
                workload=cfg.name + ("_then_think" if then_think else ""),
                config={"B": B, "H": H, "Hkv": Hkv, "S": S, "D": D, "w": w, "keep": keep,
                        **({"d_keep": dk} if then_think else {})})


def wl_tova(c: Ctx, cfg, gen, dtype, tdtype) -> dict:
    L, torch = c.L, c.torch
    B, H, Hkv, S, D, w, keep = cfg.B, cfg.H, cfg.Hkv, cfg.S, cfg.D, cfg.w, cfg.keep
    esz = 2 if dtype == "bf16" else 4
    nl = c.args.layers or cfg.layers
    layers, host0 = [], None
    for layer in range(nl):
        p = gen(layer)
        layers.append(dict(q=c.up(p.q, dtype), k=c.up(p.k, dtype), v=c.up(p.v, dtype)))
        host0 = host0 or p
    cub = c.args.cu_budget
    ws_bytes = L.window_scores_ws_bytes(B, H, Hkv, S, D, w, L.KVC_BF16 if dtype == "bf16" else L.KVC_F32,
                                        cu_budget=cub)
    s0 = c.streams[0]
    for i, ly in enumerate(layers):
        st = c.streams[i % len(c.streams)]
        ly["scores"] = c.empty((B, Hkv, S), torch.float32)
        ly["idx"] = c.empty((B, Hkv, keep), torch.int32)
        ly["k_out"] = c.empty((B, Hkv, keep, D), tdtype)
        ly["v_out"] = c.empty((B, Hkv, keep, D), tdtype)
        ly["ws"] = c.empty(ws_bytes, torch.uint8)
        ly["tk_ws"] = c.empty(L.topk_ws_bytes(B * Hkv, S), torch.uint8)
        ly["calls"] = [L.bind_window_scores(ly["q"], ly["k"], ly["scores"], ly["ws"], st,
                                            reduce=L.KVC_REDUCE_ALL_HEADS, causal=False, cu_budget=cub),
                       L.bind_topk_select(ly["scores"], keep, 0, ly["idx"], ly["tk_ws"], st),
                       L.bind_gather_compact(ly["k"], ly["v"], ly["idx"], ly["k_out"], ly["v_out"], st)]
        ly["kscore"] = L.bind_window_scores(ly["q"], ly["k"], ly["scores"], ly["ws"], s0,
                                            reduce=L.KVC_REDUCE_ALL_HEADS, causal=False, cu_budget=cub)
        ly["kgather"] = L.bind_gather_compact(ly["k"], ly["v"], ly["idx"], ly["k_out"], ly["v_out"], s0)

    def step():
        for ly in layers:
            for f in ly["calls"]:
                f()

    k_bytes, q_bytes, s_bytes = B * Hkv * S * D * esz, B * H * w * D * esz, B * Hkv * S * 4
    i_bytes, g_bytes = B * Hkv * keep * 4, 2 * 2 * B * Hkv * keep * D * esz
    layer_bytes = k_bytes + q_bytes + 2 * s_bytes + 2 * i_bytes + g_bytes
    # the dominant kernel: the gather when it moves more bytes than the scoring reads
    if g_bytes > k_bytes:
        kernel = ("kvc_gather_compact", [ly["kgather"] for ly in layers], g_bytes + i_bytes,
                  recorded_traffic("gather_compact_" + cfg.name, GATHER_SOURCES))
    else:
        kernel = ("kvc_window_scores", [ly["kscore"] for ly in layers], k_bytes + q_bytes + s_bytes,
                  recorded_traffic("window_scores_" + cfg.name, SCORE_SOURCES, cub))

    def cpu(budget):
        from oracle import kvc_oracle as O
        q64, k64 = host0.q64(), host0.k64()

        def one(n):
            b = n % B
            s, idx = O.tova(q64[b:b + 1], k64[b:b + 1], None, keep)
            O.gather_compact(host0.k[b:b + 1], host0.v[b:b + 1], idx)
        n, el = timed_oracle(one, budget)
        return {"value": round(S * n / el, 1), "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
                "sample": f"{n} sequences (of {B} per layer) of layer 0, S={S}, fp64 numpy oracle (scores, top-k, "
                          f"gather), {el:.1f} s"}
    def check_outputs():
        return [t.clone() for t in (layers[0]["scores"], layers[0]["idx"], layers[0]["k_out"], layers[-1]["idx"])]
    return dict(step=step, units_per_step=B * S * nl, layers=nl, layer_bytes=layer_bytes,
                check_outputs=check_outputs,
                kernel=kernel, cpu=cpu, metric=f"KV tokens scored+pruned/s per layer ({cfg.name})",
                unit="tokens/s", dtype=dtype, workload=cfg.name,
                config={"B": B, "H": H, "Hkv": Hkv, "S": S, "D": D, "w": w, "keep": keep})


def wl_think_128k(c: Ctx, compress: bool = False) -> dict:
    """ThinK + SnapKV at 128k.  compress: the kept keys are stored with their
    64 kept channels only and the window queries are cut to the same channels
    (the page's options 3b/3c) instead of zero-filled 128-channel keys (3a)."""
    L, torch, cfg = c.L, c.torch, c.configs.THINK_128K
    B, H, Hkv, S, D, w, keep, dk = cfg.B, cfg.H, cfg.Hkv, cfg.S, cfg.D, cfg.w, cfg.keep, cfg.d_keep
    nl = c.args.layers or cfg.layers
    layers, host0 = [], None
    for layer in range(nl):
        p = c.synth.think_snapkv(layer)
        layers.append(dict(q=c.up(p.q), k=c.up(p.k), v=c.up(p.v)))
        host0 = host0 or p
    cub = c.args.cu_budget
    ws_bytes = L.window_scores_ws_bytes(B, H, Hkv, S, D, w, cu_budget=cub)
    cs_bytes = L.channel_scores_ws_bytes(B, H, Hkv, S, D, w)
    s0 = c.streams[0]
    for i, ly in enumerate(layers):
        st = c.streams[i % len(c.streams)]
        ly["cs"] = c.empty((B, Hkv, D), torch.float32)
        ly["ch"] = c.empty((B, Hkv, dk), torch.int32)
        ly["scores"] = c.empty((B, Hkv, S), torch.float32)
        ly["idx"] = c.empty((B, Hkv, keep), torch.int32)
        ly["k_out"] = c.empty((B, Hkv, keep, dk if compress else D), torch.bfloat16)
        ly["v_out"] = c.empty((B, Hkv, keep, D), torch.bfloat16)
        ly["ws"] = c.empty(max(ws_bytes, cs_bytes), torch.uint8)
        ly["tk_ws"] = c.empty(max(L.topk_ws_bytes(B * Hkv, D), L.topk_ws_bytes(B * Hkv, S)), torch.uint8)
        ly["calls"] = [L.bind_channel_scores(ly["q"], ly["k"], ly["cs"], ly["ws"], st),
                       L.bind_topk_select(ly["cs"], dk, 0, ly["ch"], ly["tk_ws"], st),
                       L.bind_window_scores(ly["q"], ly["k"], ly["scores"], ly["ws"], st, chan_idx=ly["ch"],
                                            reduce=L.KVC_REDUCE_GROUP, causal=True, cu_budget=cub),
                       L.bind_topk_select(ly["scores"], keep, w, ly["idx"], ly["tk_ws"], st)]
        if compress:
            ly["q_c"] = c.empty((B, H, w, dk), torch.bfloat16)
            ly["calls"] += [L.bind_gather_compress(ly["k"], ly["v"], ly["idx"], ly["ch"], ly["k_out"], ly["v_out"], st),
                            L.bind_query_channels(ly["q"], ly["ch"], ly["q_c"], st)]
        else:
            ly["calls"].append(L.bind_gather_compact(ly["k"], ly["v"], ly["idx"], ly["k_out"], ly["v_out"], st,
                                                     chan_idx=ly["ch"]))
        ly["kcall"] = L.bind_window_scores(ly["q"], ly["k"], ly["scores"], ly["ws"], s0, chan_idx=ly["ch"],
                                           reduce=L.KVC_REDUCE_GROUP, causal=True, cu_budget=cub)
        if cub != 0:  # own workspace and scores: the step's outputs stay those of the budgeted calls
            ly["ws1"] = c.empty(L.window_scores_ws_bytes(B, H, Hkv, S, D, w), torch.uint8)
            ly["scores1"] = c.empty((B, Hkv, S), torch.float32)
            ly["kcall1"] = L.bind_window_scores(ly["q"], ly["k"], ly["scores1"], ly["ws1"], s0, chan_idx=ly["ch"],
                                                reduce=L.KVC_REDUCE_GROUP, causal=True)

    def step():
        for ly in layers:
            for f in ly["calls"]:
                f()

    # K once (channel pass and score passes), Q, scores written and read, indices
    # written and read, kept K and V read and written
    k_bytes, q_bytes, s_bytes = B * Hkv * S * D * 2, B * H * w * D * 2, B * Hkv * S * 4
    i_bytes, g_bytes = B * Hkv * keep * 4, 2 * 2 * B * Hkv * keep * D * 2
    if compress:
        # kept K channels read and written, V rows read and written, the window
        # queries' kept channels read and written
        g_bytes = 2 * B * Hkv * keep * dk * 2 + 2 * B * Hkv * keep * D * 2 + 2 * B * H * w * dk * 2
    layer_bytes = k_bytes + q_bytes + 2 * s_bytes + 2 * i_bytes + g_bytes

    def cpu(budget):
        from oracle import kvc_oracle as O
        q64, k64 = host0.q64(), host0.k64()
        G = H // Hkv

        def one(n):
            g = n % Hkv
            _, ch, s, idx = O.think_snapkv(q64[:, g * G:(g + 1) * G], k64[:, g:g + 1], dk, keep)
            if compress:
                O.gather_compress(host0.k[:, g:g + 1], host0.v[:, g:g + 1], idx, ch)
                O.query_channels(host0.q[:, g * G:(g + 1) * G], ch)
            else:
                O.gather_compact(host0.k[:, g:g + 1], host0.v[:, g:g + 1], idx, chan_keep=ch)
        n, el = timed_oracle(one, budget)
        return {"value": round(B * S * n / Hkv / el, 1), "unit": "tokens/s", "cores": blas_threads(),
                "kind": "oracle", "sample": f"{n} KV heads (of {Hkv} per layer) of layer 0, S={S}, fp64 numpy "
                                            f"oracle (channels, scores, top-k, gather), {el:.1f} s"}
    def check_outputs():
        return [t.clone() for t in (layers[0]["ch"], layers[0]["scores"], layers[0]["idx"], layers[0]["k_out"],
                                    layers[-1]["idx"])]
    return dict(step=step, units_per_step=B * S * nl, layers=nl, layer_bytes=layer_bytes,
                check_outputs=check_outputs,
                kernel=("kvc_window_scores with 64 of 128 key channels (pass 1 + pass 2)",
                        [ly["kcall"] for ly in layers], k_bytes + q_bytes + s_bytes,
                        recorded_traffic("window_scores_think_128k", SCORE_SOURCES, cub)),
                kernel_alone=[ly["kcall1"] for ly in layers] if cub != 0 else None,
                cpu=cpu, metric=f"KV tokens scored+pruned/s per layer ({cfg.name}{'_kc' if compress else ''})",
                unit="tokens/s", dtype="bf16", workload=cfg.name + ("_kc" if compress else ""),
                config={"B": B, "H": H, "Hkv": Hkv, "S": S, "D": D, "w": w, "keep": keep, "d_keep": dk,
                        "stored_key_channels": dk if compress else D})


def wl_scissor_decode(c: Ctx) -> dict:
    L, torch, cfg = c.L, c.torch, c.configs.SCISSOR_DECODE
    B, H, Hkv, C, D = cfg.B, cfg.H, cfg.Hkv, cfg.S, cfg.D
    nl = c.args.layers or cfg.layers
    nsteps = c.args.steps
    cub = c.args.cu_budget
    W = (C + 31) // 32
    layers = []
    for layer in range(nl):
        qs = np.stack([c.synth.scissor_query(layer, t) for t in range(nsteps)])  # [T, B, H, 1, D]
        ly = dict(k=c.up(c.synth.scissor_cache(layer)), q=c.up(qs))
        ly["valid"] = c.empty((B, Hkv, C), torch.uint8)
        ly["hist"] = c.empty((cfg.hist_len, B * Hkv, W), torch.int32)
        ly["counts"] = c.empty((B, Hkv, C), torch.int16)
        ly["probs"] = c.empty((B, Hkv, C), torch.float32)
        ly["frac"] = c.empty((B, Hkv, C), torch.float32)
        ly["ev"] = c.empty((B, Hkv, cfg.n_evict), torch.int32)
        ly["ws"] = c.empty(L.window_scores_ws_bytes(B, H, Hkv, C, D, 1, cu_budget=cub),
                           torch.uint8)
        ly["tk_ws"] = c.empty(L.topk_ws_bytes(B * Hkv, C), torch.uint8)
        layers.append(ly)
    s0 = c.streams[0]
    for i, ly in enumerate(layers):
        st = c.streams[i % len(c.streams)]
        ly["st"] = st
        ly["score"] = [L.bind_window_scores(ly["q"][t], ly["k"], ly["probs"], ly["ws"], st, valid=ly["valid"],
                                            reduce=L.KVC_REDUCE_GROUP, causal=False, cu_budget=cub)
                       for t in range(nsteps)]
        ly["kcall"] = L.bind_window_scores(ly["q"][0], ly["k"], ly["probs"], ly["ws"], s0, valid=ly["valid"],
                                           reduce=L.KVC_REDUCE_GROUP, causal=False, cu_budget=cub)
        ly["topk"] = L.bind_topk_select(ly["frac"], cfg.n_evict, 0, ly["ev"], ly["tk_ws"], st)
        ly["record"], ly["record_step"] = L.bind_scissor_update(ly["valid"], ly["hist"], ly["counts"], st,
                                                                probs=ly["probs"])
        ly["record_frac"], ly["record_frac_step"] = L.bind_scissor_update(ly["valid"], ly["hist"], ly["counts"], st,
                                                                          probs=ly["probs"], frac_out=ly["frac"])
        ly["evict"], ly["evict_step"] = L.bind_scissor_update(ly["valid"], ly["hist"], ly["counts"], st,
                                                              evict_idx=ly["ev"])

    state = {"t": 0}

    def reset():
        for ly in layers:
            ly["valid"].fill_(1)
            ly["hist"].zero_()
            ly["counts"].zero_()
        torch.cuda.synchronize()
        state["t"] = 0

    def step():
        t = state["t"]
        evict = (t + 1) % cfg.evict_every == 0
        for ly in layers:
            ly["score"][t]()
            if evict:
                ly["record_frac_step"].value = t
                ly["record_frac"]()
                ly["topk"]()
                ly["evict_step"].value = t
                ly["evict"]()
            else:
                ly["record_step"].value = t
                ly["record"]()
        state["t"] = t + 1

    # token-steps: valid slots per (b, g) at step t, times the batch
    units = sum(B * (C - (t // cfg.evict_every) * cfg.n_evict) for t in range(nsteps))
    k_bytes = B * Hkv * C * D * 2
    # per step: K, Q, probabilities written and read, counts read and written,
    # one bit-plane, validity
    step_bytes = k_bytes + B * H * D * 2 + 2 * B * Hkv * C * 4 + 2 * B * Hkv * C * 2 + B * Hkv * W * 4 + B * Hkv * C

    def cpu(budget):
        from oracle import kvc_oracle as O
        k64 = c.synth.stored_to_f64(c.synth.scissor_cache(0), "bf16")[0:1, 0:1]
        G = H // Hkv
        done = {"units": 0}

        def one(n):
            # the workload's steps again and again, each pass from a full cache
            t = n % nsteps
            if t == 0:
                done["cache"] = O.LowAttentionState(1, 1, C, cfg.hist_len)
            cache = done["cache"]
            q = c.synth.stored_to_f64(c.synth.scissor_query(0, t), "bf16")[0:1, 0:G]
            done["units"] += int(cache.valid.sum())
            O.scissorhands_step(cache, q, k64, t, cfg.evict_every, cfg.n_evict)
        n, el = timed_oracle(one, budget)
        # one (b, g) row is 1/Hkv of a sequence's work in a layer
        return {"value": round(done["units"] / Hkv / el, 1), "unit": "token-steps/s", "cores": blas_threads(),
                "kind": "oracle", "sample": f"{n} decode steps of one (batch, KV head) row of layer 0, C={C}, fp64 "
                                            f"numpy oracle (probabilities, record, eviction), {el:.1f} s"}
    def final_state():
        return [x for ly in layers for x in (ly["valid"], ly["hist"], ly["counts"], ly["frac"], ly["ev"])]

    return dict(step=step, reset=reset, units_per_step=units * nl / nsteps, layers=nl, layer_bytes=step_bytes,
                kernel=("kvc_window_scores (w=1, stored logits)", [ly["kcall"] for ly in layers],
                        k_bytes + B * H * D * 2 + B * Hkv * C * 4,
                        recorded_traffic("window_scores_scissorhands_decode", SCORE_SOURCES, cub)),
                final_state=final_state, graph_block=cfg.evict_every,
                cpu=cpu, metric=f"KV token-steps scored+recorded/s per layer ({cfg.name})", unit="token-steps/s",
                dtype="bf16", workload=cfg.name,
                config={"B": B, "H": H, "Hkv": Hkv, "C": C, "D": D, "decode_steps": nsteps,
                        "hist_len": cfg.hist_len, "evict_every": cfg.evict_every, "n_evict": cfg.n_evict})


def wl_scissor_queue_decode(c: Ctx) -> dict:
    """Scissorhands with insertion: the prompt (the first P = 3840 slots,
    protected) and the generated tokens share C = 4096 slots; each decode step
    inserts its token (into the next free slot, then into the head of the
    eviction queue, refilled with 64 slots whenever it runs out), attends with
    the step's query and records."""
    L, torch, cfg = c.L, c.torch, c.configs.SCISSOR_QUEUE
    B, H, Hkv, C, D, P, m = cfg.B, cfg.H, cfg.Hkv, cfg.S, cfg.D, cfg.keep, cfg.n_evict
    nl = c.args.layers or cfg.layers
    nsteps = c.args.steps
    cub = c.args.cu_budget
    W = (C + 31) // 32
    layers = []
    for layer in range(nl):
        qs = np.stack([c.synth.scissor_query(layer, t) for t in range(nsteps)])  # [T, B, H, 1, D]
        kn, vn = c.synth.scissor_new_tokens(layer, nsteps)
        cache = c.synth.scissor_cache(layer)
        ly = dict(k0=c.up(cache), v0=c.up(cache[:, ::-1].copy()), q=c.up(qs), kn=c.up(kn), vn=c.up(vn))
        ly["k"], ly["v"] = torch.empty_like(ly["k0"]), torch.empty_like(ly["v0"])
        ly["valid"] = c.empty((B, Hkv, C), torch.uint8)
        ly["hist"] = c.empty((cfg.hist_len, B * Hkv, W), torch.int32)
        ly["counts"] = c.empty((B, Hkv, C), torch.int16)
        ly["since"] = c.empty((B, Hkv, C), torch.int64)
        ly["probs"] = c.empty((B, Hkv, C), torch.float32)
        ly["queue"] = c.empty((B, Hkv, m), torch.int32)
        ly["ws"] = c.empty(L.window_scores_ws_bytes(B, H, Hkv, C, D, 1, cu_budget=cub),
                           torch.uint8)
        ly["rf_ws"] = c.empty(L.scissor_refill_ws_bytes(B, Hkv, C), torch.uint8)
        layers.append(ly)
    s0 = c.streams[0]
    for i, ly in enumerate(layers):
        st = c.streams[i % len(c.streams)]
        ly["score"] = [L.bind_window_scores(ly["q"][t], ly["k"], ly["probs"], ly["ws"], st, valid=ly["valid"],
                                            reduce=L.KVC_REDUCE_GROUP, causal=False, cu_budget=cub)
                       for t in range(nsteps)]
        ly["kcall"] = L.bind_window_scores(ly["q"][0], ly["k"], ly["probs"], ly["ws"], s0, valid=ly["valid"],
                                           reduce=L.KVC_REDUCE_GROUP, causal=False, cu_budget=cub)
        ly["record"], ly["record_step"] = L.bind_scissor_update(ly["valid"], ly["hist"], ly["counts"], st,
                                                                probs=ly["probs"])
        ly["refill"], ly["refill_step"] = L.bind_scissor_refill(ly["valid"], ly["counts"], ly["since"], cfg.hist_len,
                                                                P, ly["queue"], ly["rf_ws"], st)
        ly["fill"] = [L.bind_scissor_insert(ly["kn"][t], ly["vn"][t], ly["k"], ly["v"], ly["valid"], ly["hist"],
                                            ly["counts"], ly["since"], st) for t in range(nsteps)]
        ly["pop"] = [L.bind_scissor_insert(ly["kn"][t], ly["vn"][t], ly["k"], ly["v"], ly["valid"], ly["hist"],
                                           ly["counts"], ly["since"], st, queue=ly["queue"]) for t in range(nsteps)]

    state = {"t": 0, "ins": P, "qpos": m}

    def reset():
        for ly in layers:
            ly["k"].copy_(ly["k0"])
            ly["v"].copy_(ly["v0"])
            ly["valid"].zero_()
            ly["valid"][:, :, :P] = 1
            ly["hist"].zero_()
            ly["counts"].zero_()
            ly["since"].zero_()
        torch.cuda.synchronize()
        state.update(t=0, ins=P, qpos=m)

    def step():
        t, ins, qpos = state["t"], state["ins"], state["qpos"]
        refill = ins >= C and qpos == m
        for ly in layers:
            if ins < C:
                call, _, fill_pos, rec = ly["fill"][t]
                fill_pos.value = ins
                rec.value = t
                call()
            else:
                if refill:
                    ly["refill_step"].value = t - 1
                    ly["refill"]()
                call, j, _, rec = ly["pop"][t]
                j.value = 0 if refill else qpos
                rec.value = t
                call()
            ly["score"][t]()
            ly["record_step"].value = t
            ly["record"]()
        if ins >= C:
            state["qpos"] = 1 if refill else qpos + 1
        state.update(t=t + 1, ins=ins + 1)

    # token-steps: valid slots per (b, g) at each step, times the batch
    units = sum(B * min(P + t + 1, C) for t in range(nsteps))
    k_bytes = B * Hkv * C * D * 2
    # per step: the insertion (K and V rows written, one bit in every plane),
    # K, Q, probabilities written and read, counts read and written, one
    # bit-plane, validity
    step_bytes = (2 * B * Hkv * D * 2 + B * Hkv * cfg.hist_len * 4 + k_bytes + B * H * D * 2 + 2 * B * Hkv * C * 4
                  + 2 * B * Hkv * C * 2 + B * Hkv * W * 4 + B * Hkv * C)

    def cpu(budget):
        from oracle import kvc_oracle as O
        G = H // Hkv
        k64 = c.synth.stored_to_f64(c.synth.scissor_cache(0), "bf16")[0:1, 0:1]
        kn, vn = c.synth.scissor_new_tokens(0, nsteps)
        cache = O.ScissorhandsQueue(1, 1, C, D, cfg.hist_len, m, -1)
        cache.prefill(k64[:, :, :P], k64[:, :, :P])
        done = {"units": 0}

        def one(n):
            t = n % nsteps
            q = c.synth.stored_to_f64(c.synth.scissor_query(0, t), "bf16")[0:1, 0:G]
            kt = c.synth.stored_to_f64(kn[t], "bf16")[0:1, 0:1]
            vt = c.synth.stored_to_f64(vn[t], "bf16")[0:1, 0:1]
            O.scissorhands_queue_step(cache, q, kt, vt)
            done["units"] += int(cache.valid.sum())
        n, el = timed_oracle(one, budget)
        return {"value": round(done["units"] / Hkv / el, 1), "unit": "token-steps/s", "cores": blas_threads(),
                "kind": "oracle", "sample": f"{n} decode steps of one (batch, KV head) row of layer 0, C={C}, fp64 "
                                            f"numpy oracle (insertion, probabilities, record, queue), {el:.1f} s"}
    def final_state():
        return [x for ly in layers for x in (ly["k"], ly["v"], ly["valid"], ly["hist"], ly["counts"], ly["since"],
                                              ly["queue"])]

    return dict(step=step, reset=reset, units_per_step=units * nl / nsteps, layers=nl, layer_bytes=step_bytes,
                kernel=("kvc_window_scores (w=1, stored logits)", [ly["kcall"] for ly in layers],
                        k_bytes + B * H * D * 2 + B * Hkv * C * 4,
                        recorded_traffic("window_scores_scissorhands_decode", SCORE_SOURCES, cub)),
                final_state=final_state, graph_block=m,
                cpu=cpu, metric=f"KV token-steps scored+recorded/s per layer ({cfg.name})", unit="token-steps/s",
                dtype="bf16", workload=cfg.name,
                config={"B": B, "H": H, "Hkv": Hkv, "C": C, "D": D, "decode_steps": nsteps, "prompt": P,
                        "hist_len": cfg.hist_len, "queue": m})


def build_workload(c: Ctx) -> dict:
    wl = c.args.workload
    if wl == "snapkv_32k":
        return wl_snapkv_32k(c)
    if wl == "snapkv_think_32k":
        return wl_snapkv_32k(c, then_think=True)
    if wl == "scissor_queue_decode":
        return wl_scissor_queue_decode(c)
    if wl == "tova_tiny":
        return wl_tova(c, c.configs.TOVA_TINY, c.synth.tova_tiny, "f32", c.torch.float32)
    if wl == "tova_batched":
        return wl_tova(c, c.configs.TOVA_BATCHED, c.synth.tova_batched, "bf16", c.torch.bfloat16)
    if wl == "think_128k":
        return wl_think_128k(c)
    if wl == "think_128k_kc":
        return wl_think_128k(c, compress=True)
    return wl_scissor_decode(c)


def time_graph(c, wl, args) -> dict:
    """The same step captured once into a HIP graph (the streams forked from and
    joined to the capture stream) and replayed.  Two checked replays first, each
    after eager work and a synchronisation, must reproduce the eager outputs bit
    for bit; then `steps` replays are timed between two events."""
    torch = c.torch
    cur = torch.cuda.current_stream(c.dev)
    eager = wl["check_outputs"]()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream(device=c.dev)
    cs.wait_stream(cur)
    with torch.cuda.graph(g, stream=cs):
        for st in c.streams:
            st.wait_stream(cs)
        wl["step"]()
        for st in c.streams:
            cs.wait_stream(st)
    torch.cuda.synchronize()
    match = True
    for _ in range(2):
        scratch = torch.randn(1 << 20, device=c.dev)  # eager work between the replays
        scratch.mul_(2.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = wl["check_outputs"]()
        match = match and all(torch.equal(a, b) for a, b in zip(eager, got))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(cur)
    for _ in range(args.steps):
        g.replay()
    b.record(cur)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    del g
    us_layer = ms * 1e3 / (wl["layers"] * args.steps)
    return {"us_per_layer": round(us_layer, 3), "value": round(wl["units_per_step"] * args.steps / (ms * 1e-3), 1),
            "replays_match_eager": bool(match)}


def time_graph_blocks(c, wl, args) -> dict:
    """A decode run captured as one HIP graph per block of `graph_block` steps
    (one eviction or refill period; each block's step numbers, queries and
    insert positions are its own) and replayed block after block from a fresh
    state.  Two checked runs of replays first, each after eager work and a
    synchronisation, must end in the eager run's final state bit for bit; then
    one whole run of replays is timed between two events."""
    torch = c.torch
    cur = torch.cuda.current_stream(c.dev)
    eager = [x.clone() for x in wl["final_state"]()]
    blk = wl["graph_block"]
    wl["reset"]()
    graphs = []
    cs = torch.cuda.Stream(device=c.dev)
    t = 0
    while t < args.steps:
        n = min(blk, args.steps - t)
        g = torch.cuda.CUDAGraph()
        cs.wait_stream(cur)
        with torch.cuda.graph(g, stream=cs):
            for st in c.streams:
                st.wait_stream(cs)
            for _ in range(n):
                wl["step"]()
            for st in c.streams:
                cs.wait_stream(st)
        graphs.append(g)
        t += n
    torch.cuda.synchronize()
    match = True
    for _ in range(2):
        wl["reset"]()
        scratch = torch.randn(1 << 20, device=c.dev)  # eager work between the runs
        scratch.mul_(2.0)
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        got = wl["final_state"]()
        match = match and all(torch.equal(a, b) for a, b in zip(eager, got))
    wl["reset"]()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(cur)
    for g in graphs:
        g.replay()
    b.record(cur)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    del graphs
    return {"us_per_layer": round(ms * 1e3 / (wl["layers"] * args.steps), 3),
            "value": round(wl["units_per_step"] * args.steps / (ms * 1e-3), 1),
            "steps_per_graph": blk, "graphs": (args.steps + blk - 1) // blk, "replays_match_eager": bool(match)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is data-parallel per "
              f"(batch, KV head) and is not sharded here.", file=sys.stderr)
        sys.exit(2)
    if args.workload in ("scissor_decode", "scissor_queue_decode") and not 1 <= args.steps <= 800:
        print("the decode workload runs between 1 and 800 steps", file=sys.stderr)
        sys.exit(2)
    c = Ctx(args)
    torch = c.torch
    t0 = time.time()
    wl = build_workload(c)
    print(f"[bench] {wl['workload']}: set up in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    cur = torch.cuda.current_stream(c.dev)

    def run_steps(n):
        # the streams start after everything queued on the default stream
        for st in c.streams:
            st.wait_stream(cur)
        for _ in range(n):
            wl["step"]()
        for st in c.streams:
            cur.wait_stream(st)

    reset = wl.get("reset")
    if reset is None:
        run_steps(args.warmup)
    else:  # a decode run: the warm-up is one whole run from a fresh state
        reset()
        run_steps(args.steps)
        reset()
    torch.cuda.synchronize()

    # timed region: K steps between a synchronisation on each side
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    run_steps(args.steps)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    elapsed_ms = start.elapsed_time(end)

    # the dominant kernel timed alone: kernel-reps passes over the layers, each
    # pass one run of back-to-back calls on one stream between two HIP events
    # recorded on it, so that the average is the calls' own duration and not the
    # latency of an event and a dispatch per call
    config = {"workload": wl["workload"], **wl["config"], "layers_per_step": wl["layers"], "streams": args.streams,
              "cu_budget": args.cu_budget}
    label, kcalls, kbytes, traffic = wl["kernel"]
    st0 = c.streams[0]
    st0.wait_stream(cur)

    def time_calls(calls):
        kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.kernel_reps)]
        for a, b in kev:
            a.record(st0)
            for f in calls:
                f()
            b.record(st0)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for (a, b) in kev])) / len(calls) * 1e3
    k_us = time_calls(kcalls)
    # the same calls planned to fill the GPU alone (kvc_window_scores without a budget)
    k1_us = time_calls(wl["kernel_alone"]) if wl.get("kernel_alone") and not args.no_alone else None

    units = wl["units_per_step"] * args.steps
    value = units / (elapsed_ms * 1e-3)
    t_layer_us = elapsed_ms * 1e3 / (wl["layers"] * args.steps)
    hbm_frac = wl["layer_bytes"] / (HBM_PEAK_GBS * 1e9) / (t_layer_us * 1e-6)
    achieved = kbytes / (k_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": label,
                "avg_us": round(k_us, 2), "algorithmic_bytes": kbytes,
                "cu_budget": args.cu_budget}
    if k1_us is not None:
        a1 = kbytes / (k1_us * 1e-6) / 1e9
        roofline["planned_alone"] = {"cu_budget": 256, "avg_us": round(k1_us, 2), "achieved": round(a1, 1),
                                     "frac": round(a1 / HBM_PEAK_GBS, 4)}

    graph = None
    if not args.no_graph and wl.get("check_outputs") is not None:
        graph = time_graph(c, wl, args)
    elif not args.no_graph and wl.get("final_state") is not None:
        graph = time_graph_blocks(c, wl, args)

    ceilings = None if args.no_ceilings else measure_ceilings(c)
    if ceilings:
        roofline["frac_of_read_ceiling"] = round(achieved / ceilings["stream_read_gbs"], 4)
    comp = wl.get("compute")
    if comp:
        k_s = k_us * 1e-6
        roofline["compute"] = {
            "mfma_tflops": round(comp["mfma_flops"] / k_s / 1e12, 1),
            "mfma_frac": round(comp["mfma_flops"] / k_s / MFMA_BF16_PEAK, 4),
            "one_contraction_frac": round(comp["one_contraction_flops"] / k_s / MFMA_BF16_PEAK, 4),
            "mfma_peak_tflops": MFMA_BF16_PEAK / 1e12,
            "exps": comp["exps"],
            "exp_frac": round(comp["exps"] / k_s / ceilings["exp_per_s"], 4) if ceilings else None,
        }

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=c.dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None if args.no_cpu_baseline else wl["cpu"](args.cpu_seconds)
    if cpu:
        cpu["cpu_model"] = cpu_model()
    config.update({"us_per_layer": round(t_layer_us, 3), "algorithmic_bytes_per_layer": wl["layer_bytes"],
                   "hbm_roofline_frac": round(hbm_frac, 4), "wall_s": round(wall, 4)})
    if ceilings:
        config["ceilings"] = ceilings
        config["read_ceiling_frac_per_layer"] = round(
            wl["layer_bytes"] / (ceilings["stream_read_gbs"] * 1e9) / (t_layer_us * 1e-6), 4)
    if graph:
        config["graph"] = graph
    out = {
        "metric": wl["metric"],
        "value": round(value, 1),
        "unit": wl["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl["dtype"],
        "data": "synthetic",
        "config": config,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
