"""Property tests of the fp64 oracle over random small shapes (CPU only).

Each property follows from the definitions the oracle restates, not from its
code: probability mass per row, equivariance under permutations of keys and of
the query heads of a group, the selection order of the top-k, ThinK's channel
score under key permutation and query scaling, and the Scissorhands counts and
eviction order.  Hypothesis draws the shapes and a seed; inputs are seeded
normal arrays.
"""
from __future__ import annotations

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import kvc_oracle as O

SETTINGS = settings(max_examples=30, deadline=None, derandomize=True)


@st.composite
def shapes(draw, causal_ok=True):
    B = draw(st.integers(1, 2))
    Hkv = draw(st.sampled_from([1, 2]))
    G = draw(st.sampled_from([1, 2, 4]))
    S = draw(st.integers(1, 48))
    w = draw(st.integers(1, min(S, 6)))
    D = draw(st.sampled_from([8, 16]))
    seed = draw(st.integers(0, 2**31 - 1))
    return B, Hkv * G, Hkv, S, D, w, seed


def problem(B, H, Hkv, S, D, w, seed, scale=1.0):
    rs = np.random.default_rng(seed)
    q = rs.standard_normal((B, H, w, D)) * scale
    k = rs.standard_normal((B, Hkv, S, D))
    return q, k


@SETTINGS
@given(shapes(), st.booleans(), st.floats(0.0, 0.5))
def test_group_scores_carry_the_mass_of_rows_with_an_allowed_key(sh, causal, hole_rate):
    """Each window row's probabilities sum to 1 when the row has an allowed key
    and 0 otherwise, so a KV head's GROUP scores sum to the share of its G*w rows
    that have one."""
    B, H, Hkv, S, D, w, seed = sh
    q, k = problem(*sh)
    rs = np.random.default_rng(seed + 1)
    valid = rs.random((B, Hkv, S)) >= hole_rate
    s = O.window_scores(q, k, valid=valid, reduce=O.REDUCE_GROUP, causal=causal)
    G = H // Hkv
    for b in range(B):
        for g in range(Hkv):
            rows_ok = 0
            for i in range(w):
                lim = S - w + i if causal else S - 1
                rows_ok += bool(valid[b, g, : lim + 1].any())
            assert s[b, g].sum() == pytest.approx(rows_ok / w, abs=1e-12)  # G heads share the rows' key sets
            assert np.all(s[b, g][~valid[b, g]] == 0.0)
            assert np.all(s[b, g] >= 0.0)
    del G


@SETTINGS
@given(shapes(), st.booleans())
def test_all_heads_scores_are_the_mean_of_group_scores(sh, holes):
    """ALL_HEADS averages over all H heads, i.e. over the KV heads' GROUP scores,
    and repeats that row for every KV head."""
    B, H, Hkv, S, D, w, seed = sh
    q, k = problem(*sh)
    valid = (np.random.default_rng(seed + 2).random((B, Hkv, S)) >= 0.3) if holes else None
    grp = O.window_scores(q, k, valid=valid, reduce=O.REDUCE_GROUP, causal=True)
    allh = O.window_scores(q, k, valid=valid, reduce=O.REDUCE_ALL_HEADS, causal=True)
    np.testing.assert_allclose(allh, np.broadcast_to(grp.mean(axis=1, keepdims=True), allh.shape), rtol=1e-12,
                               atol=1e-15)


@SETTINGS
@given(shapes(), st.booleans())
def test_scores_follow_a_permutation_of_the_keys(sh, holes):
    """Without the causal limit the keys form a set: permuting them (and their
    validity) permutes the scores the same way."""
    B, H, Hkv, S, D, w, seed = sh
    q, k = problem(*sh)
    rs = np.random.default_rng(seed + 3)
    valid = (rs.random((B, Hkv, S)) >= 0.25) if holes else np.ones((B, Hkv, S), dtype=bool)
    perm = rs.permutation(S)
    s = O.window_scores(q, k, valid=valid, causal=False)
    sp = O.window_scores(q, k[:, :, perm], valid=valid[:, :, perm], causal=False)
    np.testing.assert_allclose(sp, s[:, :, perm], rtol=1e-12, atol=1e-15)


@SETTINGS
@given(shapes(), st.booleans())
def test_group_scores_ignore_the_order_of_the_group_heads(sh, causal):
    """The GROUP mean runs over the query heads of a group: permuting the heads
    within each group leaves the scores unchanged."""
    B, H, Hkv, S, D, w, seed = sh
    q, k = problem(*sh)
    G = H // Hkv
    rs = np.random.default_rng(seed + 4)
    order = np.concatenate([g * G + rs.permutation(G) for g in range(Hkv)])
    s = O.window_scores(q, k, causal=causal)
    sp = O.window_scores(q[:, order], k, causal=causal)
    np.testing.assert_allclose(sp, s, rtol=1e-12, atol=1e-15)


@SETTINGS
@given(st.integers(1, 40), st.data())
def test_topk_keeps_a_prefix_of_the_score_order(n, data):
    """Every kept eligible position beats every dropped one: a larger score, or
    an equal score at a lower index.  The tail is kept, the output ascending."""
    n_tail = data.draw(st.integers(0, n))
    k = data.draw(st.integers(n_tail, n))
    levels = data.draw(st.sampled_from([0, 3, 7]))
    rs = np.random.default_rng(data.draw(st.integers(0, 2**31 - 1)))
    s = rs.integers(0, levels, n).astype(np.float64) if levels else rs.standard_normal(n)
    idx = O.topk_select(s[None, :], k, n_tail)[0]
    assert len(idx) == k and np.all(np.diff(idx) > 0)
    E = n - n_tail
    assert set(range(E, n)) <= set(idx.tolist())
    kept = [i for i in idx if i < E]
    dropped = sorted(set(range(E)) - set(kept))
    assert len(kept) == k - n_tail
    for i in kept:
        for j in dropped:
            assert s[i] > s[j] or (s[i] == s[j] and i < j)


@SETTINGS
@given(shapes(), st.floats(0.1, 4.0))
def test_channel_scores_ignore_key_order_and_scale_with_the_query(sh, a):
    """ThinK's channel score sums over positions: a key permutation leaves it
    unchanged, and scaling the queries by a scales it by a^2."""
    B, H, Hkv, S, D, w, seed = sh
    q, k = problem(*sh)
    perm = np.random.default_rng(seed + 5).permutation(S)
    cs = O.channel_scores(q, k)
    np.testing.assert_allclose(O.channel_scores(q, k[:, :, perm]), cs, rtol=1e-12)
    np.testing.assert_allclose(O.channel_scores(q * a, k), cs * a * a, rtol=1e-12)


@SETTINGS
@given(st.integers(1, 12), st.integers(1, 6), st.integers(1, 20), st.integers(0, 2**31 - 1))
def test_scissorhands_counts_and_eviction_order(C, hist, steps, seed):
    """Counts never exceed a slot's observations; the fraction is their ratio
    (0 before any observation); eviction takes the valid slots of the largest
    fraction, the lower index first among equals, and leaves the rest."""
    rs = np.random.default_rng(seed)
    stt = O.LowAttentionState(1, 1, C, hist)
    for _ in range(steps):
        p = rs.random((1, 1, C))
        stt.record(p / p.sum())
        if rs.random() < 0.3 and stt.valid.sum() > 1:  # refill one hole now and then
            holes = np.flatnonzero(~stt.valid[0, 0])
            if holes.size:
                stt.occupy(np.array([[int(holes[0])]]))
    cnt, obs = stt.counts(), stt.observations()
    assert np.all(cnt >= 0) and np.all(cnt <= obs) and np.all(obs <= hist)
    fr = stt.fraction()
    v = stt.valid
    np.testing.assert_array_equal(fr[v], np.where(obs[v] > 0, cnt[v] / np.maximum(obs[v], 1), 0.0))
    n_ev = int(rs.integers(1, max(2, int(v.sum()))))
    n_ev = min(n_ev, int(v.sum()))
    before = v.copy()
    ev = stt.evict(n_ev)[0, 0]
    assert np.all(before[0, 0, ev]) and not np.any(stt.valid[0, 0, ev])
    left = np.flatnonzero(stt.valid[0, 0])
    for i in ev:
        for j in left:
            assert fr[0, 0, i] > fr[0, 0, j] or (fr[0, 0, i] == fr[0, 0, j] and i < j)
