"""Parity at the five workloads' full sizes (GPU).

Each test runs the workload's whole path through the C-ABI at its real shape.
The launch configuration is the one bench.py times (the kernels and tilings
depend only on the shape and the compute-unit budget).  Results are compared with the fp64
oracle on the same seeded inputs:
  * scores elementwise (1e-3 relative);
  * kept sets bit-exact against the oracle's selection on the GPU's own scores,
    and equal to the oracle's selection outside positions within a relative
    1e-5 of the row threshold;
  * gathers bit-exact.
The oracle computes a full layer of TOVA tiny, SnapKV 32k, TOVA batched and
ThinK + SnapKV 128k in seconds.  For the 800-step Scissorhands decode it follows
three sampled (batch, KV head) rows in teacher-forced lockstep, while the GPU
runs all 64.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from kv_cache_compression_window_amd import configs, synth
from oracle import kvc_oracle as O
from tests.gpu_util import (check_gather, check_kept, check_scores, dev, host_bits, low_bits_agree,
                             oracle_state, unpack_all_planes, unpack_planes)

pytestmark = pytest.mark.gpu

# The compute-unit budgets the timed loop gives the score calls of the 32K and
# 128K prefill layers (they run side by side on several streams there); the
# tests use the same grid splits.
CUS_SNAPKV_32K, CUS_SNAPKV_THEN_THINK, CUS_THINK_128K = 96, 112, 128


def lib():
    from kv_cache_compression_window_amd import binding
    return binding


def say(msg):
    print(f"[gpu-full] {msg}", file=sys.stderr, flush=True)


def test_tova_tiny_full():
    cfg = configs.TOVA_TINY
    say(cfg.name)
    p = synth.tova_tiny(0)
    L = lib()
    q, k, v = dev(p.q), dev(p.k), dev(p.v)
    s = L.kvc_window_scores(q, k, reduce=L.KVC_REDUCE_ALL_HEADS, causal=False)
    idx = L.kvc_topk_select(s.view(-1, p.S), cfg.keep).view(p.B, p.Hkv, cfg.keep)
    ko, vo = L.kvc_gather_compact(k, v, idx)
    torch.cuda.synchronize()
    ref_s, _ = O.tova(p.q64(), p.k64(), p.v64(), cfg.keep)
    check_scores(s.cpu().numpy(), ref_s, "TOVA tiny scores")
    check_kept(idx.cpu().numpy(), s.cpu().numpy(), ref_s, cfg.keep, 0)
    check_gather(ko, vo, p.k, p.v, idx.cpu().numpy())


def test_snapkv_32k_full():
    cfg = configs.SNAPKV_32K
    say(cfg.name)
    p = synth.snapkv(0)
    L = lib()
    st = torch.cuda.current_stream()
    q, k, v = dev(p.q, "bf16"), dev(p.k, "bf16"), dev(p.v, "bf16")
    scores = torch.empty((p.B, p.Hkv, p.S), dtype=torch.float32, device="cuda")
    idx = torch.empty((p.B, p.Hkv, cfg.keep), dtype=torch.int32, device="cuda")
    ko = torch.empty((p.B, p.Hkv, cfg.keep, p.D), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    ws = torch.empty(L.window_scores_ws_bytes(p.B, p.H, p.Hkv, p.S, p.D, p.w, cu_budget=CUS_SNAPKV_32K),
                     dtype=torch.uint8, device="cuda")
    tk_ws = torch.empty(L.topk_ws_bytes(p.B * p.Hkv, p.S), dtype=torch.uint8, device="cuda")
    # the same pre-bound calls as the timed loop
    L.bind_window_scores(q, k, scores, ws, st, reduce=L.KVC_REDUCE_GROUP, causal=True,
                         cu_budget=CUS_SNAPKV_32K)()
    L.bind_topk_select(scores, cfg.keep, cfg.n_tail, idx, tk_ws, st)()
    L.bind_gather_compact(k, v, idx, ko, vo, st)()
    torch.cuda.synchronize()
    ref_s, _ = O.snapkv(p.q64(), p.k64(), cfg.keep)
    sg = scores.cpu().numpy()
    check_scores(sg, ref_s, "SnapKV 32k scores")
    # every row of scores sums to 1 (the window mean of softmax rows)
    assert np.allclose(sg.sum(axis=-1, dtype=np.float64), 1.0, rtol=0, atol=1e-4)
    check_kept(idx.cpu().numpy(), sg, ref_s, cfg.keep, cfg.n_tail)
    check_gather(ko, vo, p.k, p.v, idx.cpu().numpy())


def test_tova_batched_full():
    cfg = configs.TOVA_BATCHED
    say(cfg.name)
    p = synth.tova_batched(0)
    L = lib()
    q, k, v = dev(p.q, "bf16"), dev(p.k, "bf16"), dev(p.v, "bf16")
    s = L.kvc_window_scores(q, k, reduce=L.KVC_REDUCE_ALL_HEADS, causal=False)
    idx = L.kvc_topk_select(s.view(-1, p.S), cfg.keep).view(p.B, p.Hkv, cfg.keep)
    ko, vo = L.kvc_gather_compact(k, v, idx)
    torch.cuda.synchronize()
    ref_s, _ = O.tova(p.q64(), p.k64(), None, cfg.keep)
    sg = s.cpu().numpy()
    check_scores(sg, ref_s, "TOVA batched scores")
    # TOVA repeats one row per KV head, so the kept sets of a sequence agree
    ig = idx.cpu().numpy()
    assert (ig == ig[:, :1]).all()
    check_kept(ig, sg, ref_s, cfg.keep, 0)
    check_gather(ko, vo, p.k, p.v, ig)


def test_scissorhands_decode_full_sampled():
    """Scissorhands decode at full size: all 800 steps on all 64 (b, g) rows.  Three rows are
    followed in teacher-forced lockstep at every step (probabilities, low bits,
    counts); at each of the 12 eviction steps every row is checked:
    probabilities, low bits, counts, fractions, the eviction set and the
    validity after it."""
    cfg = configs.SCISSOR_DECODE
    say(cfg.name)
    B, H, Hkv, C, D, hl = cfg.B, cfg.H, cfg.Hkv, cfg.S, cfg.D, cfg.hist_len
    G = H // Hkv
    L = lib()
    kb = synth.scissor_cache(0)
    kd = dev(kb, "bf16")
    k64 = synth.stored_to_f64(kb, "bf16")
    sample = [(0, 0), (3, 5), (7, 7)]
    W = (C + 31) // 32
    valid = torch.ones((B, Hkv, C), dtype=torch.uint8, device="cuda")
    hist = torch.zeros((hl, B * Hkv, W), dtype=torch.int32, device="cuda")
    counts = torch.zeros((B, Hkv, C), dtype=torch.int16, device="cuda")
    frac = torch.empty((B, Hkv, C), dtype=torch.float32, device="cuda")
    bgs = [b * Hkv + g for b, g in sample]
    for t in range(cfg.steps):
        qb = synth.scissor_query(0, t)
        v_before = valid.cpu().numpy()
        probs = L.kvc_window_scores(dev(qb, "bf16"), kd, valid=valid, reduce=L.KVC_REDUCE_GROUP, causal=False)
        evict = (t + 1) % cfg.evict_every == 0
        L.kvc_scissor_update(t, valid, hist, counts, probs=probs, frac_out=frac if evict else None)
        idx = None
        if evict:
            idx = L.kvc_topk_select(frac, cfg.n_evict)
            L.kvc_scissor_update(t, valid, hist, counts, evict_idx=idx)
        torch.cuda.synchronize()
        pg = probs.cpu().numpy()
        h_now = hist[:, bgs, :].cpu().numpy()
        cnt = counts.cpu().numpy().view(np.uint16).astype(np.int64)
        q64 = synth.stored_to_f64(qb, "bf16")
        for si, (b, g) in enumerate(sample):
            ref_p = O.window_scores(q64[b:b + 1, g * G:(g + 1) * G], k64[b:b + 1, g:g + 1],
                                    valid=v_before[b:b + 1, g:g + 1], reduce=O.REDUCE_GROUP, causal=False)[0, 0]
            check_scores(pg[b, g], ref_p, f"decode step {t} ({b},{g}) probs")
            planes = unpack_planes(h_now, si, C)
            # the oracle takes the step on the GPU's state: the low test needs only validity and probabilities
            low = oracle_state(v_before[b, g], planes, t, hl).record(ref_p[None, None])[0, 0]
            assert low_bits_agree(planes[:, t % hl], low, ref_p, v_before[b, g]), f"step {t} ({b},{g}) low bits"
            assert np.array_equal(cnt[b, g], planes.sum(axis=1)), f"step {t} ({b},{g}) counts"
            assert cnt[b, g].max() <= min(t + 1, hl)
        if evict:
            # every row at the eviction steps
            ref_all = O.window_scores(q64, k64, valid=v_before, reduce=O.REDUCE_GROUP, causal=False)
            check_scores(pg, ref_all, f"decode step {t} probs (all rows)")
            planes_all = unpack_all_planes(hist.cpu().numpy(), C).reshape(B, Hkv, C, hl)
            low_all = O.LowAttentionState.from_recordings(v_before, np.zeros((B, Hkv, C), np.int64), {}, t,
                                                          hl).record(ref_all)
            assert low_bits_agree(planes_all[..., t % hl], low_all, ref_all, v_before), f"step {t} low bits"
            assert np.array_equal(cnt, planes_all.sum(axis=-1, dtype=np.int64)), f"step {t} counts"
            fr = oracle_state(v_before, planes_all, t + 1, hl).fraction()
            assert np.array_equal(frac.cpu().numpy(), fr.astype(np.float32)), f"step {t} fractions"
            want = O.topk_select(fr.reshape(B * Hkv, C), cfg.n_evict).reshape(B, Hkv, cfg.n_evict)
            assert np.array_equal(idx.cpu().numpy(), want), f"step {t} evictions"
            v_exp = v_before.copy()
            np.put_along_axis(v_exp, want, 0, axis=2)
            assert np.array_equal(valid.cpu().numpy(), v_exp), f"step {t} validity after eviction"
            say(f"  eviction at step {t}: all 64 rows ok")
    # 12 evictions of 64 slots per row
    assert int(valid.sum().item()) == B * Hkv * (C - (cfg.steps // cfg.evict_every) * cfg.n_evict)


def test_scissorhands_decode_resume():
    """Checkpoint and resume of the decode state: 400 steps, a copy of the state
    buffers (validity, bit-planes, counts) through host memory into fresh
    buffers, 400 more steps; the result is bit-identical to 800 uninterrupted
    steps."""
    cfg = configs.SCISSOR_DECODE
    say("Scissorhands decode resume")
    B, Hkv, C, hl = cfg.B, cfg.Hkv, cfg.S, cfg.hist_len
    L = lib()
    kd = dev(synth.scissor_cache(0), "bf16")
    qs = [dev(synth.scissor_query(0, t), "bf16") for t in range(cfg.steps)]
    W = (C + 31) // 32

    def fresh():
        return (torch.ones((B, Hkv, C), dtype=torch.uint8, device="cuda"),
                torch.zeros((hl, B * Hkv, W), dtype=torch.int32, device="cuda"),
                torch.zeros((B, Hkv, C), dtype=torch.int16, device="cuda"))

    def run(state, t0, t1):
        valid, hist, counts = state
        frac = torch.empty((B, Hkv, C), dtype=torch.float32, device="cuda")
        for t in range(t0, t1):
            probs = L.kvc_window_scores(qs[t], kd, valid=valid, reduce=L.KVC_REDUCE_GROUP, causal=False)
            evict = (t + 1) % cfg.evict_every == 0
            L.kvc_scissor_update(t, valid, hist, counts, probs=probs, frac_out=frac if evict else None)
            if evict:
                L.kvc_scissor_update(t, valid, hist, counts, evict_idx=L.kvc_topk_select(frac, cfg.n_evict))
        torch.cuda.synchronize()

    full = fresh()
    run(full, 0, cfg.steps)
    first = fresh()
    half = cfg.steps // 2
    run(first, 0, half)
    snap = [x.cpu().clone() for x in first]
    del first
    resumed = tuple(x.cuda() for x in snap)
    run(resumed, half, cfg.steps)
    for a, b, name in zip(full, resumed, ("valid", "hist", "counts")):
        assert torch.equal(a.cpu(), b.cpu()), name


def test_think_snapkv_128k_full():
    cfg = configs.THINK_128K
    say(cfg.name)
    p = synth.think_snapkv(0)
    L = lib()
    q, k, v = dev(p.q, "bf16"), dev(p.k, "bf16"), dev(p.v, "bf16")
    cs = L.kvc_channel_scores(q, k)
    ch = L.kvc_topk_select(cs.view(-1, p.D), cfg.d_keep).view(p.B, p.Hkv, cfg.d_keep)
    torch.cuda.synchronize()
    q64, k64 = p.q64(), p.k64()
    ref_cs = O.channel_scores(q64, k64)
    csg = cs.cpu().numpy()
    check_scores(csg, ref_cs, "ThinK 128k channel scores")
    chg = ch.cpu().numpy()
    check_kept(chg, csg, ref_cs, cfg.d_keep, 0)
    # the oracle continues with the GPU's channel set
    s = L.kvc_window_scores(q, k, chan_idx=ch, reduce=L.KVC_REDUCE_GROUP, causal=True, cu_budget=CUS_THINK_128K)
    idx = L.kvc_topk_select(s.view(-1, p.S), cfg.keep, cfg.n_tail).view(p.B, p.Hkv, cfg.keep)
    ko, vo = L.kvc_gather_compact(k, v, idx, chan_idx=ch)
    torch.cuda.synchronize()
    ref_s, _ = O.snapkv(q64, k64, cfg.keep, chan_keep=chg)
    sg = s.cpu().numpy()
    check_scores(sg, ref_s, "ThinK 128k scores")
    check_kept(idx.cpu().numpy(), sg, ref_s, cfg.keep, cfg.n_tail)
    check_gather(ko, vo, p.k, p.v, idx.cpu().numpy(), chg)


def test_think_128k_kept_keys_compressed_full():
    """The ThinK + SnapKV 128k layer with the kept keys stored with their 64 channels (bench
    workload think_128k_kc): compressed K, V rows and pruned window queries,
    bit-exact against the oracle on the GPU's kept positions and channels."""
    cfg = configs.THINK_128K
    say(cfg.name + " compressed keys")
    p = synth.think_snapkv(0)
    L = lib()
    q, k, v = dev(p.q, "bf16"), dev(p.k, "bf16"), dev(p.v, "bf16")
    cs = L.kvc_channel_scores(q, k)
    ch = L.kvc_topk_select(cs.view(-1, p.D), cfg.d_keep).view(p.B, p.Hkv, cfg.d_keep)
    s = L.kvc_window_scores(q, k, chan_idx=ch, reduce=L.KVC_REDUCE_GROUP, causal=True, cu_budget=CUS_THINK_128K)
    idx = L.kvc_topk_select(s.view(-1, p.S), cfg.keep, cfg.n_tail).view(p.B, p.Hkv, cfg.keep)
    kc, vc = L.kvc_gather_compress(k, v, idx, ch)
    qc = L.kvc_query_channels(q, ch)
    torch.cuda.synchronize()
    ig, chg = idx.cpu().numpy(), ch.cpu().numpy()
    ref_kc, ref_vc = O.gather_compress(p.k, p.v, ig, chg)
    assert np.array_equal(host_bits(kc), ref_kc) and np.array_equal(host_bits(vc), ref_vc)
    assert np.array_equal(host_bits(qc), O.query_channels(p.q, chg))
    # the zeros added back give the zero-filled cache of the think_128k workload
    full = L.kvc_channel_expand(kc, ch, p.D)
    k0, _ = L.kvc_gather_compact(k, None, idx, chan_idx=ch)
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), k0.view(torch.int16))


def test_snapkv_32k_then_think_full():
    """The SnapKV 32k layer followed by ThinK on its 4096 kept keys (bench workload
    snapkv_think_32k); the oracle follows the GPU's kept positions."""
    cfg = configs.SNAPKV_32K
    say(cfg.name + " then think")
    p = synth.snapkv(0)
    L = lib()
    dk = 64
    q, k, v = dev(p.q, "bf16"), dev(p.k, "bf16"), dev(p.v, "bf16")
    s = L.kvc_window_scores(q, k, reduce=L.KVC_REDUCE_GROUP, causal=True, cu_budget=CUS_SNAPKV_THEN_THINK)
    idx = L.kvc_topk_select(s.view(-1, p.S), cfg.keep, cfg.n_tail).view(p.B, p.Hkv, cfg.keep)
    ko, vo = L.kvc_gather_compact(k, v, idx)
    cs = L.kvc_channel_scores(q, ko)
    ch = L.kvc_topk_select(cs.view(-1, p.D), dk).view(p.B, p.Hkv, dk)
    rows = torch.arange(cfg.keep, dtype=torch.int32, device="cuda").expand(p.B, p.Hkv, cfg.keep).contiguous()
    kc, _ = L.kvc_gather_compress(ko, None, rows, ch)
    torch.cuda.synchronize()
    q64, k64 = p.q64(), p.k64()
    ref_s, _ = O.snapkv(q64, k64, cfg.keep)
    sg, ig = s.cpu().numpy(), idx.cpu().numpy()
    check_scores(sg, ref_s, "SnapKV 32k scores")
    check_kept(ig, sg, ref_s, cfg.keep, cfg.n_tail)
    ref_cs = O.channel_scores(q64, np.take_along_axis(k64, ig.astype(np.int64)[..., None], axis=2))
    csg, chg = cs.cpu().numpy(), ch.cpu().numpy()
    check_scores(csg, ref_cs, "channel scores of the kept keys")
    check_kept(chg, csg, ref_cs, dk, 0)
    k_kept, _ = O.gather_compact(p.k, None, ig)
    ref_kc, _ = O.gather_compress(k_kept, None, np.broadcast_to(np.arange(cfg.keep), ig.shape), chg)
    assert np.array_equal(host_bits(kc), ref_kc)


def test_scissorhands_queue_decode_full_sampled():
    """The Scissorhands decode with insertion at its bench size (B 8, C 4096, a
    protected prompt of 3840, queue 64, 800 steps) on all 64 rows: every refill's
    queue on every row equals the oracle's top-k of the fractions of the GPU's
    state, each slot over its own observations (R14); three sampled rows
    followed in teacher-forced lockstep at every step: every insertion, the
    step's probabilities and low bits."""
    cfg = configs.SCISSOR_QUEUE
    say(cfg.name)
    B, H, Hkv, C, D, P, m, hist_len = cfg.B, cfg.H, cfg.Hkv, cfg.S, cfg.D, cfg.keep, cfg.n_evict, cfg.hist_len
    G = H // Hkv
    W = (C + 31) // 32
    L = lib()
    cache = synth.scissor_cache(0)
    kn, vn = synth.scissor_new_tokens(0, cfg.steps)
    k_cache, v_cache = dev(cache, "bf16"), dev(cache[:, ::-1].copy(), "bf16")
    valid = torch.zeros((B, Hkv, C), dtype=torch.uint8, device="cuda")
    valid[:, :, :P] = 1
    hist = torch.zeros((hist_len, B * Hkv, W), dtype=torch.int32, device="cuda")
    counts = torch.zeros((B, Hkv, C), dtype=torch.int16, device="cuda")
    since = torch.zeros((B, Hkv, C), dtype=torch.int64, device="cuda")
    queue = torch.zeros((B, Hkv, m), dtype=torch.int32, device="cuda")
    sample = [(0, 0), (3, 5), (7, 7)]
    bgs = [b * Hkv + g for b, g in sample]
    ins, qpos, refills = P, m, 0
    for t in range(cfg.steps):
        k_new, v_new = dev(kn[t], "bf16"), dev(vn[t], "bf16")
        if ins < C:
            L.kvc_scissor_insert(k_new, v_new, k_cache, v_cache, valid, hist, counts, since, t, fill_pos=ins)
            slots = np.full((B, Hkv), ins)
        else:
            if qpos == m:
                v_st, since_st = valid.cpu().numpy(), since.cpu().numpy()
                planes_st = unpack_all_planes(hist.cpu().numpy(), C).reshape(B, Hkv, C, hist_len)
                L.kvc_scissor_refill(t - 1, valid, counts, hist_len, P, m, queue=queue, since=since)
                torch.cuda.synchronize()
                fr = oracle_state(v_st, planes_st, t, hist_len, since_st).fraction()
                fr[..., :P] = -np.inf
                want = O.topk_select(fr.reshape(B * Hkv, C), m).reshape(B, Hkv, m)
                assert np.array_equal(queue.cpu().numpy(), want), f"step {t} queue"
                qpos, refills = 0, refills + 1
            slots = queue.cpu().numpy()[:, :, qpos]
            L.kvc_scissor_insert(k_new, v_new, k_cache, v_cache, valid, hist, counts, since, t, queue=queue, j=qpos)
            qpos += 1
        ins += 1
        torch.cuda.synchronize()
        v_ins = valid.cpu().numpy()
        h_ins = hist[:, bgs, :].cpu().numpy()
        cnt_ins = counts.cpu().numpy().view(np.uint16)
        since_ins = since.cpu().numpy()
        q_t = synth.scissor_query(0, t)
        probs = L.kvc_window_scores(dev(q_t, "bf16"), k_cache, valid=valid, reduce=L.KVC_REDUCE_GROUP, causal=False)
        L.kvc_scissor_update(t, valid, hist, counts, probs=probs)
        torch.cuda.synchronize()
        pg = probs.cpu().numpy()
        h_now = hist[:, bgs, :].cpu().numpy()
        q64 = synth.stored_to_f64(q_t, "bf16")
        for si, (b, g) in enumerate(sample):
            e = int(slots[b, g])
            assert e >= P
            row_k = host_bits(k_cache[b, g, e])
            assert np.array_equal(row_k, kn[t][b, g]), f"step {t} inserted K ({b},{g})"
            assert v_ins[b, g, e] == 1 and cnt_ins[b, g, e] == 0 and since_ins[b, g, e] == t
            assert not unpack_planes(h_ins, si, C)[e].any()
            k64 = synth.stored_to_f64(host_bits(k_cache[b:b + 1, g:g + 1]), "bf16")
            ref_p = O.window_scores(q64[b:b + 1, g * G:(g + 1) * G], k64, valid=v_ins[b:b + 1, g:g + 1],
                                    reduce=O.REDUCE_GROUP, causal=False)[0, 0]
            check_scores(pg[b, g], ref_p, f"step {t} ({b},{g}) probs")
            st = oracle_state(v_ins[b, g], unpack_planes(h_ins, si, C), t, hist_len, since_ins[b, g])
            low = st.record(ref_p[None, None])[0, 0]
            got = unpack_planes(h_now, si, C)[:, t % hist_len]
            assert low_bits_agree(got, low, ref_p, v_ins[b, g]), f"step {t} ({b},{g}) low bits"
        if t % 100 == 0:
            say(f"  step {t} ok")
    assert refills > 0
    # the prompt is never replaced
    assert np.array_equal(host_bits(k_cache[:, :, :P].contiguous()), cache[:, :, :P])


def test_window_scores_key_rows_past_4gib():
    """Key rows longer than 2^32 bytes (17 M keys of one KV head, 4.35 GB): the
    K tiles are loaded through buffer descriptors whose 32-bit size saturates
    there.  Every key is the same vector, so each window row's probabilities are
    uniform over the keys its causal mask allows (the closed form of the
    all-keys-equal case, pinned in the oracle tests): score_j = (1/w) * sum over
    the window positions i that allow key j of 1 / (S - w + i + 1).  A key read
    wrongly (as zero, or from another row) changes its logit and the sums."""
    L = lib()
    B, H, Hkv, S, D, w = 1, 32, 1, 17_000_000, 128, 8
    g = torch.Generator(device="cpu").manual_seed(20261202)
    q = torch.randn(B, H, w, D, generator=g).to(torch.bfloat16).cuda()
    krow = torch.randn(D, generator=g).to(torch.bfloat16).cuda()
    k = krow.view(1, 1, 1, D).expand(B, Hkv, S, D).contiguous()
    assert k.numel() * k.element_size() > 2 ** 32
    say(f"window scores, S={S} keys of one KV head, {k.numel() * 2 / 2**30:.2f} GiB of K")
    s = L.kvc_window_scores(q, k, reduce=L.KVC_REDUCE_GROUP, causal=True)
    torch.cuda.synchronize()
    got = s[0, 0].cpu().numpy()
    del k
    exp = np.zeros(S)
    for i in range(w):
        n_i = S - w + i + 1
        exp[:n_i] += 1.0 / n_i
    exp /= w
    check_scores(got, exp, "key rows past 4 GiB")
