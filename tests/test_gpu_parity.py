"""GPU parity of every C-ABI call against the fp64 oracle (small shapes).

The shapes span every kernel variant: the stored-logits path (G*w <= 16), the
two-pass path with 1, 2, 4 and 8 waves of 32 rows and row chunks, several
key tiles and chunks with ragged ends, D = 64 and 128, fp32 and bf16, holes,
channel masks, causal windows and both reductions.
"""
import sys

import numpy as np
import pytest
import torch

from kv_cache_compression_window_amd import synth
from oracle import kvc_oracle as O
from tests.gpu_util import low_bits_agree, oracle_state, unpack_planes, check_gather, check_kept, check_scores, dev, host_bits

pytestmark = pytest.mark.gpu


def lib():
    from kv_cache_compression_window_amd import binding
    return binding


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# (name, B, H, Hkv, S, D, w, dtype, reduce, causal, holes, d_keep, q_scale)
CASES = [
    ("tova_tiny_f32", 1, 4, 2, 512, 64, 1, "f32", 1, 0, 0.0, 0, 1.0),
    ("store_group_holes", 2, 32, 8, 2049, 128, 1, "bf16", 0, 0, 0.2, 0, 1.0),
    ("store_allheads_b3", 3, 32, 8, 1111, 128, 1, "bf16", 1, 0, 0.0, 0, 1.0),
    ("store_w4_causal", 1, 8, 2, 100, 128, 4, "bf16", 0, 1, 0.0, 0, 2.0),
    ("store_s1", 1, 4, 2, 1, 64, 1, "bf16", 0, 1, 0.0, 0, 1.0),
    ("store_f32_d128_chan", 2, 4, 1, 333, 128, 2, "f32", 0, 1, 0.1, 40, 1.0),
    ("two_pass_r32_d64", 1, 4, 1, 300, 64, 8, "bf16", 0, 1, 0.0, 0, 1.0),
    ("two_pass_r64", 1, 8, 2, 777, 128, 16, "bf16", 0, 1, 0.0, 0, 1.0),
    ("two_pass_r96_f32", 1, 4, 2, 500, 128, 48, "f32", 0, 1, 0.0, 0, 1.0),
    # fp32 rows of 128 channels: two waves (R 64), and four-wave row chunks where
    # bf16 would take eight waves (R 256)
    ("f32_d128_r64_nw2_holes", 1, 8, 2, 600, 128, 16, "f32", 0, 1, 0.1, 0, 1.0),
    ("f32_d128_r256_row_chunks", 1, 16, 4, 700, 128, 64, "f32", 0, 1, 0.0, 0, 1.0),
    ("two_pass_r256_snapkv", 1, 32, 8, 1000, 128, 64, "bf16", 0, 1, 0.0, 0, 1.0),
    ("two_pass_r256_allheads", 2, 32, 8, 700, 128, 64, "bf16", 1, 1, 0.0, 0, 1.0),
    ("two_pass_r256_chan", 1, 32, 8, 700, 128, 64, "bf16", 0, 1, 0.0, 64, 1.0),
    ("two_pass_r256_holes", 1, 32, 8, 650, 128, 64, "bf16", 0, 0, 0.3, 0, 3.0),
    ("two_pass_r512", 1, 64, 8, 513, 128, 64, "bf16", 0, 1, 0.0, 0, 1.0),
    ("two_pass_s_eq_w", 1, 8, 2, 40, 64, 40, "bf16", 0, 1, 0.0, 0, 1.0),
    ("two_pass_g1", 1, 4, 4, 260, 128, 32, "bf16", 0, 1, 0.0, 0, 1.0),
    ("stream_r128", 1, 16, 4, 1200, 128, 32, "bf16", 0, 1, 0.0, 0, 1.0),
    # eight-wave kernels: partial row blocks, row chunks, D = 64 with holes and
    # channels, fewer tiles than staging sets, many tiles per chunk
    ("w8_r200_causal", 1, 16, 4, 3000, 128, 50, "bf16", 0, 1, 0.0, 0, 1.0),
    ("w8_r400_chunks", 1, 16, 4, 1500, 128, 100, "bf16", 0, 1, 0.0, 0, 1.0),
    ("w8_d64_holes_chan", 2, 32, 8, 900, 64, 64, "bf16", 0, 1, 0.2, 32, 1.0),
    ("w8_short_s70", 1, 32, 8, 70, 128, 64, "bf16", 0, 1, 0.0, 0, 1.0),
    ("w8_long_s9000_allheads", 1, 8, 2, 9000, 128, 64, "bf16", 1, 1, 0.0, 0, 2.0),
    # kept key channels on 2, 4 and 8 waves, down to a single kept channel
    ("chan_nw2_holes", 2, 8, 2, 900, 128, 16, "bf16", 0, 1, 0.25, 40, 1.0),
    ("chan_nw4_allheads", 1, 16, 4, 1300, 128, 32, "bf16", 1, 1, 0.0, 64, 2.0),
    ("chan_d1", 1, 32, 8, 500, 128, 64, "bf16", 0, 1, 0.0, 1, 1.0),
    ("chan_d65", 1, 32, 8, 400, 128, 64, "bf16", 0, 1, 0.0, 65, 1.0),
    ("chan_r320_chunks_holes", 1, 40, 8, 700, 128, 64, "bf16", 0, 1, 0.1, 48, 1.0),
    # the row limit: 1024 window rows per KV head (four 256-row chunks accumulating)
    ("rows_1024_max", 1, 16, 1, 1500, 128, 64, "bf16", 0, 1, 0.0, 0, 1.0),
    ("rows_1024_allheads_holes", 2, 32, 2, 900, 64, 64, "bf16", 1, 1, 0.15, 0, 1.0),
    # logits spanning hundreds of base-2 units (queries scaled by 20 and 30): the
    # statistics pass moves its reference many times and most probabilities
    # underflow (the score tolerance's absolute floor covers those)
    ("fold_extreme_q30", 1, 32, 8, 3000, 128, 64, "bf16", 0, 1, 0.0, 0, 30.0),
    ("fold_extreme_r128_holes_allheads", 1, 16, 4, 2000, 128, 32, "bf16", 1, 1, 0.1, 0, 20.0),
    # eight waves with 18 tiles per workgroup (the three-staging-set kernels; the
    # cases above stream at most 16)
    ("w8_long_chunks_s36000", 1, 32, 8, 36000, 128, 64, "bf16", 0, 1, 0.0, 0, 1.0),
]


def _make(case, seed):
    name, B, H, Hkv, S, D, w, dt, reduce, causal, holes, d_keep, qs = case
    p = synth.random_problem(seed, B, H, Hkv, S, D, w, dtype=dt, heavy_frac=0.02, q_scale=qs)
    valid = synth.random_valid(seed, B, Hkv, S, holes) if holes > 0 else None
    if valid is not None and B * Hkv > 1:
        valid[0, 0, :] = 0  # one (b, g) with no valid key at all
    chan = None
    if d_keep:
        rs = np.random.default_rng(seed)
        chan = np.stack([np.stack([np.sort(rs.choice(D, d_keep, replace=False)) for _ in range(Hkv)])
                         for _ in range(B)]).astype(np.int32)
    return p, valid, chan


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_window_scores(case):
    name, B, H, Hkv, S, D, w, dt, reduce, causal, holes, d_keep, qs = case
    say(f"window_scores {name}")
    p, valid, chan = _make(case, 100 + CASES.index(case))
    ref = O.window_scores(p.q64(), p.k64(), valid=valid, chan_keep=chan, reduce=reduce, causal=causal)
    L = lib()
    s = L.kvc_window_scores(dev(p.q, dt), dev(p.k, dt), valid=None if valid is None else dev(valid),
                            chan_idx=None if chan is None else dev(chan), reduce=reduce, causal=bool(causal))
    torch.cuda.synchronize()
    check_scores(s.cpu().numpy(), ref, name)
    # determinism: a second call gives the same bits
    s2 = L.kvc_window_scores(dev(p.q, dt), dev(p.k, dt), valid=None if valid is None else dev(valid),
                             chan_idx=None if chan is None else dev(chan), reduce=reduce, causal=bool(causal))
    assert torch.equal(s, s2)


# The compute-unit budget of kvc_window_scores_ex: fewer, longer key chunks
# per call; each budget's scores are within the tolerance of the oracle and
# bit-reproducible.
BUDGET_CASES = [c for n in ("two_pass_r256_snapkv", "two_pass_r256_holes", "store_group_holes",
                            "w8_long_s9000_allheads", "w8_long_chunks_s36000", "f32_d128_r256_row_chunks")
                for c in CASES if c[0] == n]


@pytest.mark.parametrize("cus", [256, 128, 112, 96, 85, 36, 4, 1])
@pytest.mark.parametrize("case", BUDGET_CASES, ids=[c[0] for c in BUDGET_CASES])
def test_window_scores_cu_budget(case, cus):
    name, B, H, Hkv, S, D, w, dt, reduce, causal, holes, d_keep, qs = case
    say(f"window_scores_ex {name} cu_budget={cus}")
    p, valid, chan = _make(case, 100 + CASES.index(case))
    ref = O.window_scores(p.q64(), p.k64(), valid=valid, chan_keep=chan, reduce=reduce, causal=causal)
    L = lib()
    args = dict(valid=None if valid is None else dev(valid), chan_idx=None if chan is None else dev(chan),
                reduce=reduce, causal=bool(causal), cu_budget=cus)
    s1 = L.kvc_window_scores(dev(p.q, dt), dev(p.k, dt), **args)
    s2 = L.kvc_window_scores(dev(p.q, dt), dev(p.k, dt), **args)
    torch.cuda.synchronize()
    check_scores(s1.cpu().numpy(), ref, f"{name} cu_budget {cus}")
    assert torch.equal(s1, s2)
    if cus == 256:  # the whole GPU: the plan of kvc_window_scores, bit for bit
        args.pop("cu_budget")
        s0 = L.kvc_window_scores(dev(p.q, dt), dev(p.k, dt), **args)
        torch.cuda.synchronize()
        assert torch.equal(s0, s1)


# The same (b, g) rows under two grid splits: batch 0 alone, and batch 0 next to
# other sequences, which gives each KV head fewer, longer key chunks (the plan
# aims at a fixed number of workgroups per call).  Two-pass: 8 KV heads take 32
# chunks of 256 keys, 32 take 8 chunks of 1024.  Stored logits: 8 KV heads take
# 16 chunks of 1024 keys, 64 take 8 of 2048.  Each split is bit-reproducible and
# within the score tolerance of the oracle.
@pytest.mark.parametrize("B2,S,w", [(4, 8192, 64), (8, 16384, 1)], ids=["two_pass", "stored_logits"])
def test_window_scores_two_grid_splits(B2, S, w):
    say(f"window_scores grid splits B=1 vs B={B2}, S={S}, w={w}")
    p = synth.random_problem(77, B2, 32, 8, S, 128, w, dtype="bf16", heavy_frac=0.02)
    ref = O.window_scores(p.q64()[:1], p.k64()[:1], causal=w > 1)
    L = lib()
    q, k = dev(p.q, "bf16"), dev(p.k, "bf16")
    one = [L.kvc_window_scores(q[:1].contiguous(), k[:1].contiguous(), causal=w > 1) for _ in range(2)]
    many = [L.kvc_window_scores(q, k, causal=w > 1) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(one[0], one[1]) and torch.equal(many[0], many[1])
    check_scores(one[0].cpu().numpy(), ref, "batch alone")
    check_scores(many[0][:1].cpu().numpy(), ref, f"batch 0 of {B2}")


@pytest.mark.parametrize("rows,n,k,n_tail,levels", [
    (8, 32768, 4096, 64, 0), (3, 1000, 10, 0, 0), (5, 777, 300, 20, 4), (2, 200000, 5000, 64, 0),
    (64, 4096, 64, 0, 401), (7, 129, 64, 0, 3), (1, 50, 50, 5, 0), (4, 60, 5, 5, 0), (3, 64, 1, 0, 2),
    (2, 40000, 39000, 0, 0), (1, 1, 1, 0, 0), (6, 5000, 0, 0, 0),
    # register-resident limit, one past it, and ties that straddle tiles
    (2, 32768, 1000, 0, 1), (3, 32769, 2000, 0, 3), (2, 70000, 30000, 7, 2), (1, 98304, 40000, 0, 0),
    # 16 keys per thread, rows not 16-byte aligned, threshold at the smallest value with pad slots
    (3, 12000, 3000, 0, 5), (3, 30001, 5000, 1, 0), (2, 20000, 15000, 0, 2), (4, 8191, 4000, 3, 2),
    # rows cut into 4096-position slices: one kept, all but one, nothing left to
    # select (k == n_tail), all kept, one value everywhere, -inf holes, odd length
    (3, 50000, 1, 0, 0), (2, 45000, 44999, 0, 0), (2, 40000, 100, 100, 0), (1, 40064, 40064, 64, 0),
    (2, 50000, 7000, 5, 1), (3, 80000, 5000, 0, 401), (2, 65537, 8000, 3, 0),
    # every eligible position kept on a sliced row, and a tail as long as the budget
    (2, 50000, 49999, 1, 0), (2, 50000, 64, 64, 0)])
def test_topk(rows, n, k, n_tail, levels):
    say(f"topk rows={rows} n={n} k={k} tail={n_tail} levels={levels}")
    s = synth.random_scores(rows * 7 + n, rows, n, levels)
    if levels == 401:  # Scissorhands fractions: count / 400 with holes at -inf
        s = np.floor(s * 400).astype(np.float32) / np.float32(400)
        s[:, ::7] = -np.inf
    idx = lib().kvc_topk_select(dev(s), k, n_tail)
    torch.cuda.synchronize()
    ig = idx.cpu().numpy().astype(np.int64)
    if k == 0:
        return
    assert np.array_equal(ig, O.topk_select(s.astype(np.float64), k, n_tail))


def test_topk_two_values():
    """Two distinct values, m of the larger per row: k = m takes the top value's
    bin whole (the radix passes stop at the first digit); k = m - 5 and m + 5
    leave ties at the threshold on either side of it."""
    say("topk two values")
    rng = np.random.default_rng(4242)
    for n, m in ((3000, 700), (30001, 4000), (70000, 9000)):
        rows = 3
        s = np.full((rows, n), 0.25, np.float32)
        for r in range(rows):
            s[r, rng.choice(n, size=m, replace=False)] = np.float32(0.75)
        for k, tail in ((m, 0), (m - 5, 0), (m + 5, 0), (m, 3)):
            idx = lib().kvc_topk_select(dev(s), k, tail)
            torch.cuda.synchronize()
            assert np.array_equal(idx.cpu().numpy().astype(np.int64), O.topk_select(s.astype(np.float64), k, tail))


def test_topk_signed_zeros():
    """Mixed-sign scores with exact +0 and -0 (equal, so the lower index wins)."""
    say("topk signed zeros")
    for n, cases in ((3000, ((1, 0), (700, 3), (2990, 3))), (70000, ((1, 0), (30000, 3), (69990, 3)))):
        s = synth.random_scores(77, 4, n, 0) - np.float32(0.5)
        s[:, 5::9] = np.float32(0.0)
        s[:, 9::9] = np.float32(-0.0)
        for k, tail in cases:
            idx = lib().kvc_topk_select(dev(s), k, tail)
            torch.cuda.synchronize()
            assert np.array_equal(idx.cpu().numpy().astype(np.int64), O.topk_select(s.astype(np.float64), k, tail))


def _bits_equal(t, ref, what):
    got = host_bits(t)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.array_equal(np.ascontiguousarray(got).view(np.uint8), np.ascontiguousarray(ref).view(np.uint8)), what


@pytest.mark.parametrize("dt,D,d_keep,order", [
    ("bf16", 128, 64, "sorted"), ("bf16", 128, 1, "sorted"), ("bf16", 128, 128, "perm"), ("bf16", 64, 37, "perm"),
    ("f32", 128, 64, "perm"), ("f32", 64, 64, "sorted"), ("f32", 128, 3, "perm")])
def test_compressed_key_cache(dt, D, d_keep, order):
    """ThinK options 3b/3c: kept-channel keys, the zeros added back, and the
    pruned queries, bit-exact against the oracle (odd d_keep: rows of the
    compressed keys are not 16-byte multiples)."""
    say(f"compressed key cache {dt} D={D} d_keep={d_keep} {order}")
    B, H, Hkv, S, n_keep, w = 2, 12, 3, 517, 129, 5
    p = synth.random_problem(17, B, H, Hkv, S, D, w, dtype=dt)
    rs = np.random.default_rng(D * 1000 + d_keep)
    idx = np.stack([np.stack([np.sort(rs.choice(S, n_keep, replace=False)) for _ in range(Hkv)])
                    for _ in range(B)]).astype(np.int32)
    ch = np.stack([np.stack([rs.permutation(D)[:d_keep] for _ in range(Hkv)]) for _ in range(B)]).astype(np.int32)
    if order == "sorted":
        ch = np.sort(ch, axis=-1)
    L = lib()
    kd, vd, idd, chd = dev(p.k, dt), dev(p.v, dt), dev(idx), dev(ch)
    kc, vc = L.kvc_gather_compress(kd, vd, idd, chd)
    full = L.kvc_channel_expand(kc, chd, D)
    qc = L.kvc_query_channels(dev(p.q, dt), chd)
    k0, v0 = L.kvc_gather_compact(kd, vd, idd, chan_idx=chd)
    kc_only, none_v = L.kvc_gather_compress(kd, None, idd, chd)
    torch.cuda.synchronize()
    ref_kc, ref_vc = O.gather_compress(p.k, p.v, idx, ch)
    _bits_equal(kc, ref_kc, "compressed K")
    _bits_equal(vc, ref_vc, "V rows")
    _bits_equal(full, O.channel_expand(ref_kc, ch, D), "zeros added back")
    _bits_equal(qc, O.query_channels(p.q, ch), "pruned queries")
    _bits_equal(kc_only, ref_kc, "compressed K without V")
    assert none_v is None
    # option 3b's expansion is option 3a's zero-filled cache
    assert torch.equal(full.view(torch.int16) if dt == "bf16" else full.view(torch.int32),
                       k0.view(torch.int16) if dt == "bf16" else k0.view(torch.int32))


def test_snapkv_then_think_composition():
    """R27 on the GPU: window scores, top-k with the window forced, gather; then
    the channel scores of the kept keys, the channel top-k and the compressed
    gather of the kept keys.  The oracle follows the GPU's kept positions."""
    say("snapkv then think")
    B, H, Hkv, S, D, w, keep, dk = 1, 16, 4, 3000, 128, 16, 512, 64
    p = synth.random_problem(51, B, H, Hkv, S, D, w, dtype="bf16", heavy_frac=0.02)
    L = lib()
    q, k, v = dev(p.q, "bf16"), dev(p.k, "bf16"), dev(p.v, "bf16")
    s = L.kvc_window_scores(q, k, reduce=L.KVC_REDUCE_GROUP, causal=True)
    idx = L.kvc_topk_select(s.view(-1, S), keep, w).view(B, Hkv, keep)
    ko, vo = L.kvc_gather_compact(k, v, idx)
    cs = L.kvc_channel_scores(q, ko)
    ch = L.kvc_topk_select(cs.view(-1, D), dk).view(B, Hkv, dk)
    rows = torch.arange(keep, dtype=torch.int32, device="cuda").expand(B, Hkv, keep).contiguous()
    kc, _ = L.kvc_gather_compress(ko, None, rows, ch)
    torch.cuda.synchronize()
    q64, k64 = p.q64(), p.k64()
    ref_s, _ = O.snapkv(q64, k64, keep)
    sg = s.cpu().numpy()
    check_scores(sg, ref_s, "token scores")
    ig = idx.cpu().numpy()
    check_kept(ig, sg, ref_s, keep, w)
    check_gather(ko, vo, p.k, p.v, ig)
    k_kept = np.take_along_axis(k64, ig.astype(np.int64)[..., None], axis=2)
    ref_cs = O.channel_scores(q64, k_kept)
    csg = cs.cpu().numpy()
    check_scores(csg, ref_cs, "channel scores of the kept keys")
    chg = ch.cpu().numpy()
    check_kept(chg, csg, ref_cs, dk, 0)
    ref_kc, _ = O.gather_compress(p.k, None, ig, chg)
    _bits_equal(kc, ref_kc, "compressed kept keys")


def test_channel_expand_repeated_entry():
    """A repeated channel takes the last of its positions (R25), as the oracle."""
    say("channel expand repeated entry")
    rs = np.random.default_rng(3)
    k_c = rs.standard_normal((1, 2, 70, 4)).astype(np.float32)
    ch = np.array([[[5, 9, 5, 60], [1, 1, 1, 2]]], dtype=np.int32)
    full = lib().kvc_channel_expand(dev(k_c), dev(ch), 64)
    torch.cuda.synchronize()
    _bits_equal(full, O.channel_expand(k_c, ch, 64), "repeated entry")


@pytest.mark.parametrize("dt,D,chan", [("bf16", 128, True), ("bf16", 64, False), ("f32", 128, True),
                                       ("f32", 64, False)])
def test_gather(dt, D, chan):
    say(f"gather {dt} D={D} chan={chan}")
    B, Hkv, S, n_keep = 2, 3, 517, 129
    p = synth.random_problem(7, B, Hkv, Hkv, S, D, 1, dtype=dt)
    rs = np.random.default_rng(1)
    idx = np.stack([np.stack([np.sort(rs.choice(S, n_keep, replace=False)) for _ in range(Hkv)])
                    for _ in range(B)]).astype(np.int32)
    ch = None
    if chan:
        ch = np.stack([np.stack([np.sort(rs.choice(D, D // 2, replace=False)) for _ in range(Hkv)])
                       for _ in range(B)]).astype(np.int32)
    ko, vo = lib().kvc_gather_compact(dev(p.k, dt), dev(p.v, dt), dev(idx), chan_idx=None if ch is None else dev(ch))
    torch.cuda.synchronize()
    check_gather(ko, vo, p.k, p.v, idx, ch)
    # K only
    ko2, vo2 = lib().kvc_gather_compact(dev(p.k, dt), None, dev(idx), chan_idx=None if ch is None else dev(ch))
    assert vo2 is None and torch.equal(ko.view(torch.uint8), ko2.view(torch.uint8))


def test_gather_every_position_kept():
    """n_keep = S with idx = 0..S-1: the compacted cache is the cache, bit for bit;
    with every channel in chan_idx nothing is zeroed."""
    say("gather every position kept")
    B, Hkv, S, D = 2, 4, 1031, 128
    p = synth.random_problem(11, B, Hkv, Hkv, S, D, 1, dtype="bf16")
    idx = np.broadcast_to(np.arange(S, dtype=np.int32), (B, Hkv, S)).copy()
    ch = np.broadcast_to(np.arange(D, dtype=np.int32), (B, Hkv, D)).copy()
    L = lib()
    ko, vo = L.kvc_gather_compact(dev(p.k, "bf16"), dev(p.v, "bf16"), dev(idx), chan_idx=dev(ch))
    kc, _ = L.kvc_gather_compress(dev(p.k, "bf16"), None, dev(idx), dev(ch))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(ko), p.k) and np.array_equal(host_bits(vo), p.v)
    assert np.array_equal(host_bits(kc), p.k)


@pytest.mark.parametrize("dt,D,S,w,G", [("bf16", 128, 3001, 64, 4), ("f32", 64, 130, 3, 2), ("bf16", 64, 1, 1, 1)])
def test_channel_scores(dt, D, S, w, G):
    say(f"channel_scores {dt} D={D} S={S}")
    B, Hkv = 2, 2
    p = synth.random_problem(9, B, G * Hkv, Hkv, S, D, w, dtype=dt)
    ref = O.channel_scores(p.q64(), p.k64())
    cs = lib().kvc_channel_scores(dev(p.q, dt), dev(p.k, dt))
    torch.cuda.synchronize()
    check_scores(cs.cpu().numpy(), ref, "channel scores")
    cs2 = lib().kvc_channel_scores(dev(p.q, dt), dev(p.k, dt))
    assert torch.equal(cs, cs2)


def test_scissorhands_lockstep_small():
    """Teacher-forced lockstep: after every step the oracle adopts the GPU's state
    and checks the step's low bits (except within 1e-5 of the threshold), counts,
    fractions and evictions."""
    say("scissorhands lockstep small")
    B, H, Hkv, C, D, hist_len, every, n_ev, steps = 2, 8, 2, 300, 128, 7, 5, 9, 23
    L = lib()
    k = synth.random_problem(3, B, Hkv, Hkv, C, D, 1, dtype="bf16", heavy_frac=0.05)
    kd = dev(k.k, "bf16")
    k64 = k.k64()
    valid = torch.ones((B, Hkv, C), dtype=torch.uint8, device="cuda")
    W = (C + 31) // 32
    hist = torch.zeros((hist_len, B * Hkv, W), dtype=torch.int32, device="cuda")
    counts = torch.zeros((B, Hkv, C), dtype=torch.int16, device="cuda")
    frac = torch.empty((B, Hkv, C), dtype=torch.float32, device="cuda")
    for t in range(steps):
        q = synth.random_problem(1000 + t, B, H, Hkv, 1, D, 1, dtype="bf16", with_v=False).q
        v_before = valid.cpu().numpy().copy()
        probs = L.kvc_window_scores(dev(q, "bf16"), kd, valid=valid, reduce=0, causal=False)
        evict = (t + 1) % every == 0
        L.kvc_scissor_update(t, valid, hist, counts, probs=probs, frac_out=frac if evict else None)
        idx = None
        if evict:
            idx = L.kvc_topk_select(frac, n_ev)
            L.kvc_scissor_update(t, valid, hist, counts, evict_idx=idx)
        torch.cuda.synchronize()
        pg = probs.cpu().numpy()
        hist_now = hist.cpu().numpy()
        cnt = counts.cpu().numpy().view(np.uint16).astype(np.int64)
        ref_p = O.window_scores(O_bf16(q), k64, valid=v_before, reduce=0, causal=False)
        check_scores(pg, ref_p, f"step {t} probs")
        for b in range(B):
            for g in range(Hkv):
                bg = b * Hkv + g
                planes = unpack_planes(hist_now, bg, C)
                low = oracle_state(v_before[b, g], planes, t, hist_len).record(ref_p[b, g][None, None])[0, 0]
                got = planes[:, t % hist_len]
                assert low_bits_agree(got, low, ref_p[b, g], v_before[b, g]), f"step {t} bg {bg} low bits"
                # the GPU's counts are the popcount of its own planes
                assert np.array_equal(cnt[b, g], planes.sum(axis=1))
                if evict:
                    fr = oracle_state(v_before[b, g], planes, t + 1, hist_len).fraction()[0, 0]
                    fg = frac.cpu().numpy()[b, g]
                    assert np.array_equal(fg, fr.astype(np.float32)), f"step {t} bg {bg} fractions"
                    want = O.topk_select(fr[None], n_ev)[0]
                    assert np.array_equal(idx.cpu().numpy()[b, g], want), f"step {t} evictions"
                    v_exp = v_before[b, g].copy()
                    v_exp[want] = 0
                    assert np.array_equal(valid.cpu().numpy()[b, g], v_exp)


def test_scissorhands_sampled_lockstep_small():
    """Recording every M = 3 steps (R26): the step index passed to the record is
    the number of recordings so far; an eviction step that records nothing asks
    for the fraction alone.  Teacher-forced against the oracle as above."""
    say("scissorhands sampled lockstep small")
    B, H, Hkv, C, D, hist_len, every, n_ev, steps, M = 2, 8, 2, 300, 128, 4, 5, 7, 26, 3
    L = lib()
    k = synth.random_problem(4, B, Hkv, Hkv, C, D, 1, dtype="bf16", heavy_frac=0.05)
    kd = dev(k.k, "bf16")
    k64 = k.k64()
    valid = torch.ones((B, Hkv, C), dtype=torch.uint8, device="cuda")
    W = (C + 31) // 32
    hist = torch.zeros((hist_len, B * Hkv, W), dtype=torch.int32, device="cuda")
    counts = torch.zeros((B, Hkv, C), dtype=torch.int16, device="cuda")
    frac = torch.empty((B, Hkv, C), dtype=torch.float32, device="cuda")
    n_rec = 0
    for t in range(steps):
        record = t % M == 0
        evict = (t + 1) % every == 0
        v_before = valid.cpu().numpy().copy()
        hist_before = hist.cpu().numpy().copy()
        probs = None
        if record:
            q = synth.random_problem(2000 + t, B, H, Hkv, 1, D, 1, dtype="bf16", with_v=False).q
            probs = L.kvc_window_scores(dev(q, "bf16"), kd, valid=valid, reduce=0, causal=False)
            L.kvc_scissor_update(n_rec, valid, hist, counts, probs=probs, frac_out=frac if evict else None)
            n_rec += 1
        elif evict:
            L.kvc_scissor_update(n_rec - 1, valid, hist, counts, frac_out=frac)
        idx = None
        if evict:
            idx = L.kvc_topk_select(frac, n_ev)
            L.kvc_scissor_update(n_rec - 1, valid, hist, counts, evict_idx=idx)
        torch.cuda.synchronize()
        hist_now = hist.cpu().numpy()
        cnt = counts.cpu().numpy().view(np.uint16).astype(np.int64)
        ref_p = None
        if record:
            ref_p = O.window_scores(O_bf16(q), k64, valid=v_before, reduce=0, causal=False)
            check_scores(probs.cpu().numpy(), ref_p, f"step {t} probs")
        for b in range(B):
            for g in range(Hkv):
                bg = b * Hkv + g
                planes_now = unpack_planes(hist_now, bg, C)
                assert np.array_equal(cnt[b, g], planes_now.sum(axis=1))
                if record:
                    st = oracle_state(v_before[b, g], unpack_planes(hist_before, bg, C), n_rec - 1, hist_len)
                    low = st.record(ref_p[b, g][None, None])[0, 0]
                    got = planes_now[:, (n_rec - 1) % hist_len]
                    assert low_bits_agree(got, low, ref_p[b, g], v_before[b, g]), f"step {t} bg {bg} low bits"
                else:
                    # nothing recorded: the history is unchanged
                    assert np.array_equal(hist_now[:, bg], hist_before[:, bg])
                if evict:
                    fr = oracle_state(v_before[b, g], planes_now, n_rec, hist_len).fraction()[0, 0]
                    fg = frac.cpu().numpy()[b, g]
                    assert np.array_equal(fg, fr.astype(np.float32)), f"step {t} bg {bg} fractions"
                    want = O.topk_select(fr[None], n_ev)[0]
                    assert np.array_equal(idx.cpu().numpy()[b, g], want), f"step {t} evictions"
                    v_exp = v_before[b, g].copy()
                    v_exp[want] = 0
                    assert np.array_equal(valid.cpu().numpy()[b, g], v_exp)


def test_scissorhands_queue_lockstep_small():
    """R28-R30 on the GPU: the prompt fills the first P slots, the next C - P
    steps fill the rest, then every step takes its slot from the eviction queue,
    refilled every m steps.  Teacher-forced: every refill's queue equals the
    oracle's top-k of the fractions of the GPU's state, each slot over its own
    observations (R14); every insertion leaves the slot with the new K/V rows,
    valid, a zero count, no history bit and its observation start; every step's
    low bits match the oracle's on the GPU's state."""
    say("scissorhands queue lockstep small")
    B, H, Hkv, C, D, P, hist_len, m, steps = 2, 8, 2, 256, 128, 160, 6, 8, 140
    L = lib()
    prob = synth.random_problem(5, B, Hkv, Hkv, C, D, 1, dtype="bf16", heavy_frac=0.05)
    k_cache, v_cache = dev(prob.k, "bf16").clone(), dev(prob.v, "bf16").clone()
    valid = torch.zeros((B, Hkv, C), dtype=torch.uint8, device="cuda")
    valid[:, :, :P] = 1
    W = (C + 31) // 32
    hist = torch.zeros((hist_len, B * Hkv, W), dtype=torch.int32, device="cuda")
    counts = torch.zeros((B, Hkv, C), dtype=torch.int16, device="cuda")
    since = torch.zeros((B, Hkv, C), dtype=torch.int64, device="cuda")
    queue = torch.zeros((B, Hkv, m), dtype=torch.int32, device="cuda")
    insertions, qpos, n_differ = P, m, 0
    for t in range(steps):
        new = synth.random_problem(3000 + t, B, Hkv, Hkv, 1, D, 1, dtype="bf16")
        q = synth.random_problem(4000 + t, B, H, Hkv, 1, D, 1, dtype="bf16", with_v=False).q
        k_new, v_new = dev(new.k[:, :, 0], "bf16"), dev(new.v[:, :, 0], "bf16")
        if insertions < C:
            L.kvc_scissor_insert(k_new, v_new, k_cache, v_cache, valid, hist, counts, since, t, fill_pos=insertions)
            slots = np.full((B, Hkv), insertions)
        else:
            if qpos == m:
                v_st, since_st, hist_st = valid.cpu().numpy(), since.cpu().numpy(), hist.cpu().numpy()
                cnt_st = counts.cpu().numpy().view(np.uint16).astype(np.int64)
                L.kvc_scissor_refill(t - 1, valid, counts, hist_len, P, m, queue=queue, since=since)
                torch.cuda.synchronize()
                qg = queue.cpu().numpy()
                for b in range(B):
                    for g in range(Hkv):
                        bg = b * Hkv + g
                        st = oracle_state(v_st[b, g], unpack_planes(hist_st, bg, C), t, hist_len, since_st[b, g])
                        fr = st.fraction()[0, 0]
                        fr[:P] = -np.inf
                        want = O.topk_select(fr[None], m)[0]
                        assert np.array_equal(qg[b, g], want), f"step {t} queue ({b},{g})"
                        # the per-slot denominator changes the choice somewhere in this run
                        glob = np.where(v_st[b, g].astype(bool), cnt_st[b, g] / min(t, hist_len), -np.inf)
                        glob[:P] = -np.inf
                        n_differ += int(not np.array_equal(O.topk_select(glob[None], m)[0], want))
                qpos = 0
            slots = queue.cpu().numpy()[:, :, qpos]
            L.kvc_scissor_insert(k_new, v_new, k_cache, v_cache, valid, hist, counts, since, t, queue=queue, j=qpos)
            qpos += 1
        insertions += 1
        torch.cuda.synchronize()
        # the insertion
        hist_ins = hist.cpu().numpy()
        cnt_ins = counts.cpu().numpy().view(np.uint16)
        v_ins = valid.cpu().numpy()
        since_ins = since.cpu().numpy()
        kc_bits = host_bits(k_cache)
        vc_bits = host_bits(v_cache)
        for b in range(B):
            for g in range(Hkv):
                e = int(slots[b, g])
                assert e >= P
                assert np.array_equal(kc_bits[b, g, e], new.k[b, g, 0]) and np.array_equal(vc_bits[b, g, e], new.v[b, g, 0])
                assert v_ins[b, g, e] == 1 and cnt_ins[b, g, e] == 0 and since_ins[b, g, e] == t
                assert not unpack_planes(hist_ins, b * Hkv + g, C)[e].any()
        assert np.array_equal(kc_bits[:, :, :P], prob.k[:, :, :P])  # the prompt is never replaced
        # the step's attention with the new token in the cache, and its record
        probs = L.kvc_window_scores(dev(q, "bf16"), k_cache, valid=valid, reduce=0, causal=False)
        L.kvc_scissor_update(t, valid, hist, counts, probs=probs)
        torch.cuda.synchronize()
        k64 = synth.stored_to_f64(kc_bits, "bf16")
        ref_p = O.window_scores(O_bf16(q), k64, valid=v_ins, reduce=0, causal=False)
        check_scores(probs.cpu().numpy(), ref_p, f"step {t} probs")
        hist_now = hist.cpu().numpy()
        for b in range(B):
            for g in range(Hkv):
                bg = b * Hkv + g
                st = oracle_state(v_ins[b, g], unpack_planes(hist_ins, bg, C), t, hist_len, since_ins[b, g])
                low = st.record(ref_p[b, g][None, None])[0, 0]
                got = unpack_planes(hist_now, bg, C)[:, t % hist_len]
                assert low_bits_agree(got, low, ref_p[b, g], v_ins[b, g]), f"step {t} bg {bg} low bits"
    assert insertions - P == steps and qpos > 0
    assert n_differ > 0, "no refill where the per-slot and the global denominators disagree"


def O_bf16(bits):
    return synth.stored_to_f64(bits, "bf16")


def test_snapkv_path_small_end_to_end():
    """window scores -> top-k with the window forced -> gather, one small layer."""
    say("snapkv end-to-end small")
    p = synth.snapkv(0, S=1500, w=64, H=32, Hkv=8, D=128)
    L = lib()
    q, k, v = dev(p.q, "bf16"), dev(p.k, "bf16"), dev(p.v, "bf16")
    s = L.kvc_window_scores(q, k, reduce=0, causal=True)
    idx = L.kvc_topk_select(s, 256, n_tail=64)
    ko, vo = L.kvc_gather_compact(k, v, idx)
    torch.cuda.synchronize()
    ref_s, _ = O.snapkv(p.q64(), p.k64(), 256)
    check_scores(s.cpu().numpy(), ref_s)
    check_kept(idx.cpu().numpy(), s.cpu().numpy(), ref_s, 256, 64)
    check_gather(ko, vo, p.k, p.v, idx.cpu().numpy())
