"""fp64 CPU oracle for KV-cache scoring and pruning — TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never calls it and it
shares no code with the HIP library; inputs come from the seeded generators
in ``kv_cache_compression_window_amd.synth`` as exact float64 values of the
stored bf16/fp32 data.

Everything is the plain definition, written with numpy in float64, in the
order the pages give the steps.  The sources are the three web pages on the
subject:

  [TOVA]    "Add TOVA press" (NVIDIA kvpress pull request 12), review thread.
  [COLD]    "Implement Scissorhands KV-cache compression & SnapKV prompt
            compression" (AnswerDotAI cold-compress pull request 11): the
            cache.py review hunks and the PR description.
  [THINK]   "Add ThinK_Press" (NVIDIA kvpress pull request 18), review thread.

Readings where the pages are silent or garbled (each is used below):
  R1  logit scale 1/sqrt(D) (the SDPA default; the pages use attention as
      it comes out of sdpa).
  R2  window rows are causal: window row i is query position S-w+i and may
      attend keys j <= S-w+i (only matters for w > 1).
  R3  TOVA averages over ALL query heads and repeats the row per KV head;
      SnapKV and Scissorhands average over the query heads of a GQA group.
  R4  the observation window is averaged (each score row sums to 1).
  R5  the SnapKV budget k includes the w window positions.
  R7  kept indices are returned in ascending position order.
  R8  exact score ties keep the lowest index (also for channels and for
      eviction: the lowest index is evicted first among equals).
  R11 Scissorhands' "keys" is the number of valid cache slots S_t.
  R12 the low test compares the group-mean probability with 1/S_t, strictly.
  R13 Scissorhands records every step.
  R14 the low-attention fraction is count / min(steps recorded, history).
  R15 evicted slots become holes (no insertion), excluded from later softmaxes.
  R16 ThinK's norms sum over positions (window rows for q, all S keys for
      k); only that reading agrees with the materialised channel_attn form.
  R17 ThinK squares the per-channel products (as the code does).
  R18 ThinK's per-query-head scores are summed over the GQA group.
  R21 pruned key channels are written as +0.0.
  R26 sampled recording every M steps records at the steps t with t % M == 0;
      evictions keep their own cadence and use the fraction over the
      recordings so far.
  R27 SnapKV then ThinK: the channel scores use the kept keys only and the
      same window queries.
  R28 Scissorhands with insertion: a decode step puts its token into the next
      free slot while there is one, else into the head of the eviction queue;
      the slot's history and count start empty; the step then attends with the
      new token in the cache and records.
  R29 the eviction queue is refilled when it is empty on a full cache, with
      the top-k (O4) of the low-attention fraction, k = drop_amount,
      ascending positions, popped front to back.
  R30 the first global_tokens slots are never queued (-1: the prompt).
  R25 a compressed key cache keeps the kept channels in chan_idx order; the
      zero-back writes them in increasing j, so a repeated entry keeps the
      last j.
  Rows with no allowed key (every slot a hole) have P = 0.

Parity pins for every function live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np

REDUCE_GROUP = 0
REDUCE_ALL_HEADS = 1


# ----------------------------------------------------------------------------
# O1-O3: window attention and its reductions
# ----------------------------------------------------------------------------

def window_logits(q: np.ndarray, k: np.ndarray, b: int, g: int, chan_keep=None) -> np.ndarray:
    """Logits of the query heads of KV head g against all S keys: [G, w, S].

    [TOVA] SimJeg's reply: only the last window_size rows of the attention
    matrix are computed, shape [batch, heads, window_size, seq_len].
    [COLD] the K/V repeat_interleave hunk fixes the GQA map: query head h
    reads KV head h // (n_head // n_local_heads).
    With a channel list (ThinK, zeroed channels) only kept channels enter the
    dot product, which equals the dot product with the pruned key channels
    set to zero.
    """
    H, D = q.shape[1], q.shape[3]
    G = H // k.shape[1]
    qg = q[b, g * G:(g + 1) * G]  # [G, w, D]
    kg = k[b, g]  # [S, D]
    if chan_keep is not None:
        keep = np.asarray(chan_keep[b, g])
        qg = qg[..., keep]
        kg = kg[:, keep]
    return (qg @ kg.T) / np.sqrt(D)  # R1


def window_allowed(S: int, w: int, valid_bg, causal: bool) -> np.ndarray:
    """[w, S] mask of the keys each window row may attend (R2, R15)."""
    allowed = np.ones((w, S), dtype=bool)
    if valid_bg is not None:
        allowed &= np.asarray(valid_bg, dtype=bool)[None, :]
    if causal and w > 1:
        i = np.arange(w)[:, None]
        j = np.arange(S)[None, :]
        allowed &= j <= (S - w + i)
    return allowed


def softmax_rows(logits: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """O2: P = exp(l - lse) over allowed entries of each row, 0 elsewhere."""
    lm = np.where(allowed, logits, -np.inf)
    m = lm.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(allowed, np.exp(lm - m), 0.0)
    z = e.sum(axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(z > 0, e / np.where(z > 0, z, 1.0), 0.0)


def window_probs(q, k, valid=None, chan_keep=None, causal=True) -> np.ndarray:
    """Window attention probabilities [B, H, w, S] (for small problems)."""
    B, H, w, _ = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    G = H // Hkv
    out = np.zeros((B, H, w, S))
    for b in range(B):
        for g in range(Hkv):
            vbg = None if valid is None else valid[b, g]
            allowed = window_allowed(S, w, vbg, causal)
            out[b, g * G:(g + 1) * G] = softmax_rows(window_logits(q, k, b, g, chan_keep), allowed[None])
    return out


def window_scores(q, k, valid=None, chan_keep=None, reduce=REDUCE_GROUP, causal=True) -> np.ndarray:
    """Per-KV-head token scores [B, Hkv, S].

    GROUP ([COLD] attention-callback hunk: the attention is averaged over the
    query heads that share a KV head; SnapKV scores the
    prefix with the observation window): s[b,g,j] is the mean of P over the
    G query heads of group g and the w window rows (R4).
    ALL_HEADS ([TOVA] hassidm and SimJeg: attn_weights.mean(1) over all
    heads, then repeated once per KV head): s[b,:,j] is the mean of P over
    all H heads and the w rows, the same row for every KV head (R3).
    """
    B, H, w, _ = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    G = H // Hkv
    per_group = np.zeros((B, Hkv, S))
    for b in range(B):
        for g in range(Hkv):
            vbg = None if valid is None else valid[b, g]
            allowed = window_allowed(S, w, vbg, causal)
            P = softmax_rows(window_logits(q, k, b, g, chan_keep), allowed[None])  # [G, w, S]
            per_group[b, g] = P.sum(axis=(0, 1))
    if reduce == REDUCE_GROUP:
        return per_group / (G * w)
    s = per_group.sum(axis=1) / (H * w)  # [B, S]
    return np.repeat(s[:, None, :], Hkv, axis=1)


# ----------------------------------------------------------------------------
# O4: per-row top-k with forced tail
# ----------------------------------------------------------------------------

def topk_select(scores: np.ndarray, k: int, n_tail: int = 0) -> np.ndarray:
    """Indices [R, k] (int64, ascending) of the kept positions of each row.

    The last n_tail positions are always kept ([COLD] PR description: SnapKV
    keeps every observation-window token and compresses only the prefix).
    The first N - n_tail positions compete for k - n_tail slots: larger score
    first, equal scores by lower index (R8).  Output ascending (R7).
    """
    scores = np.asarray(scores)
    R, N = scores.shape
    if not (0 <= n_tail <= k <= N):
        raise ValueError("need 0 <= n_tail <= k <= N")
    E = N - n_tail
    kp = k - n_tail
    out = np.empty((R, k), dtype=np.int64)
    tail = np.arange(E, N)
    for r in range(R):
        s = scores[r, :E].astype(np.float64)
        order = np.lexsort((np.arange(E), -s))  # by score descending, then index ascending
        out[r] = np.concatenate([np.sort(order[:kp]), tail])
    return out


# ----------------------------------------------------------------------------
# O6: ThinK key-channel scores
# ----------------------------------------------------------------------------

def channel_scores(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """ThinK channel scores [B, Hkv, D].

    [THINK] yuhuixu1993's factorised form: query_norm = q.pow(2) summed over
    positions, key_norm = k.pow(2) summed over positions, score = product,
    shape (bsz, heads, head_dim) (R16, R17).  Keys are repeated per the GQA
    map and the per-query-head scores summed over each group (R18).
    """
    B, H, w, D = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    query_norm = (q ** 2).sum(axis=2)  # [B, H, D]
    key_norm = (k ** 2).sum(axis=2)  # [B, Hkv, D]
    per_head = query_norm * np.repeat(key_norm, G, axis=1)  # [B, H, D]
    return per_head.reshape(B, Hkv, G, D).sum(axis=2)


def select_channels(cs: np.ndarray, d_keep: int) -> np.ndarray:
    """Kept key channels [B, Hkv, d_keep] (ascending): the largest scores,
    lowest channel first among equals ([THINK]: zero the least important)."""
    B, Hkv, D = cs.shape
    return topk_select(cs.reshape(B * Hkv, D), d_keep).reshape(B, Hkv, d_keep)


# ----------------------------------------------------------------------------
# O8: gather-compact
# ----------------------------------------------------------------------------

def gather_compact(k: np.ndarray, v: np.ndarray, idx: np.ndarray, chan_keep=None):
    """Compacted cache: K'[b,g,r] = K[b,g,idx[b,g,r]] with the pruned key
    channels set to +0 ([THINK] option 3a, zero in the key cache, R21);
    V'[b,g,r] = V[b,g,idx[b,g,r]].  Copies stored values bit for bit."""
    idx = np.asarray(idx, dtype=np.int64)
    k_out = np.take_along_axis(k, idx[..., None], axis=2)
    if chan_keep is not None:
        B, Hkv, D = k.shape[0], k.shape[1], k.shape[3]
        keep = np.zeros((B, Hkv, D), dtype=bool)
        for b in range(B):
            for g in range(Hkv):
                keep[b, g, np.asarray(chan_keep[b, g])] = True
        k_out = np.where(keep[:, :, None, :], k_out, np.zeros((), dtype=k.dtype))
    v_out = None if v is None else np.take_along_axis(v, idx[..., None], axis=2)
    return k_out, v_out


# ----------------------------------------------------------------------------
# O9: ThinK's compressed key cache (options 3b and 3c)
# ----------------------------------------------------------------------------

def gather_compress(k: np.ndarray, v, idx: np.ndarray, chan_idx: np.ndarray):
    """Kept rows with only the kept key channels, in chan_idx order ([THINK]
    review thread, options 3b/3c: the pruned key cache is stored apart):
    K'[b,g,r,j] = K[b,g,idx[b,g,r],chan_idx[b,g,j]];  V'[b,g,r] = V[b,g,idx[b,g,r]].
    Copies stored values bit for bit."""
    B, Hkv = k.shape[0], k.shape[1]
    n_keep, d_keep = idx.shape[2], chan_idx.shape[2]
    k_out = np.empty((B, Hkv, n_keep, d_keep), dtype=k.dtype)
    for b in range(B):
        for g in range(Hkv):
            rows = k[b, g][np.asarray(idx[b, g], dtype=np.int64)]
            k_out[b, g] = rows[:, np.asarray(chan_idx[b, g], dtype=np.int64)]
    v_out = None if v is None else np.take_along_axis(v, np.asarray(idx, dtype=np.int64)[..., None], axis=2)
    return k_out, v_out


def channel_expand(k_c: np.ndarray, chan_idx: np.ndarray, D: int) -> np.ndarray:
    """The zeros added back ([THINK] option 3b): K[b,g,:,chan_idx[b,g,j]] =
    K_c[b,g,:,j] for each j in increasing order (a repeated entry keeps the
    last j), every other channel +0."""
    B, Hkv, n, d_keep = k_c.shape
    out = np.zeros((B, Hkv, n, D), dtype=k_c.dtype)
    for b in range(B):
        for g in range(Hkv):
            for j in range(d_keep):
                out[b, g, :, int(chan_idx[b, g, j])] = k_c[b, g, :, j]
    return out


def query_channels(q: np.ndarray, chan_idx: np.ndarray) -> np.ndarray:
    """Queries cut to their KV head's kept key channels ([THINK] option 3c:
    prune the query as well): q_c[b,h,i,j] = q[b,h,i,chan_idx[b,h//G,j]]."""
    B, H = q.shape[0], q.shape[1]
    G = H // chan_idx.shape[1]
    out = np.empty(q.shape[:3] + (chan_idx.shape[2],), dtype=q.dtype)
    for b in range(B):
        for h in range(H):
            out[b, h] = q[b, h][:, np.asarray(chan_idx[b, h // G], dtype=np.int64)]
    return out


# ----------------------------------------------------------------------------
# O5: Scissorhands low-attention history and bulk eviction
# ----------------------------------------------------------------------------

class ScissorhandsCache:
    """One layer's Scissorhands state in the page's own layout ([COLD]
    cache.py hunks): attn_history[b, g, slot, step % history] holds the
    low-attention indicator, attn_counter counts recorded steps.
    """

    def __init__(self, B: int, Hkv: int, C: int, history_window_size: int = 400):
        self.valid = np.ones((B, Hkv, C), dtype=bool)
        self.attn_history = np.zeros((B, Hkv, C, history_window_size), dtype=np.int8)
        self.attn_counter = 0
        self.history_window_size = history_window_size

    def update_attn_history(self, attn: np.ndarray) -> np.ndarray:
        """[COLD] update_attn_history: a slot is low when its group-mean
        probability is below uniform attention 1/keys (R11, R12); the
        indicator goes into the circular slot attn_counter % history."""
        keys = self.valid.sum(axis=-1, keepdims=True)
        with np.errstate(divide="ignore"):
            uniform = np.where(keys > 0, 1.0 / np.maximum(keys, 1), 0.0)
        attn_is_low = self.valid & (attn < uniform)
        self.attn_history[..., self.attn_counter % self.history_window_size] = attn_is_low
        self.attn_counter += 1
        return attn_is_low

    def low_counts(self) -> np.ndarray:
        return self.attn_history.sum(axis=-1, dtype=np.int64)

    def low_fraction(self) -> np.ndarray:
        """Fraction of recorded steps with low attention (R14); -inf at holes."""
        n_obs = min(self.attn_counter, self.history_window_size)
        frac = self.low_counts() / float(max(n_obs, 1))
        return np.where(self.valid, frac, -np.inf)

    def evict(self, n_evict: int) -> np.ndarray:
        """[COLD] PR description: evict, per head, the tokens with the highest
        fraction of unimportant attentions; bulk eviction leaves empty slots
        (R15).  Returns the evicted indices [B, Hkv, n_evict] (ascending)."""
        B, Hkv, C = self.valid.shape
        idx = topk_select(self.low_fraction().reshape(B * Hkv, C), n_evict).reshape(B, Hkv, n_evict)
        for b in range(B):
            for g in range(Hkv):
                self.valid[b, g, idx[b, g]] = False
        return idx


def scissorhands_step(cache: ScissorhandsCache, q_t: np.ndarray, k: np.ndarray, t: int,
                      evict_every: int, n_evict: int, record_every: int = 1):
    """One decode step: group-mean attention of the step's query over the
    valid slots, record it, and every evict_every steps evict n_evict slots
    per (batch, KV head).  With record_every = M > 1 the attention is checked
    and recorded only at the steps t with t % M == 0 ([COLD] review thread:
    Scissorhands records every M steps), so the history and the fraction's
    denominator count recorded steps (R26).  Returns (probs, low bits,
    evicted indices or None); probs and low are None at a step that records
    nothing."""
    probs = low = None
    if t % record_every == 0:
        probs = window_scores(q_t, k, valid=cache.valid, reduce=REDUCE_GROUP, causal=False)
        low = cache.update_attn_history(probs)
    evicted = cache.evict(n_evict) if (t + 1) % evict_every == 0 else None
    return probs, low, evicted


class ScissorhandsQueueCache(ScissorhandsCache):
    """Scissorhands with insertion and an eviction queue ([COLD] PR
    description: instead of bulk evictions, an eviction queue is refilled
    periodically and one token is evicted per step; cache.py hunk:
    global_tokens = -1 keeps the prompt).  The cache has C slots and holds K
    and V.  Readings R28-R30:
      * a decode step inserts its token into the next free slot while there is
        one, else into the slot at the head of the eviction queue; the slot's
        history and count start empty;
      * when the queue is empty on a full cache it is refilled with the
        drop_amount slots of the highest low-attention fraction (the top-k of
        O4, ascending positions, popped front to back);
      * the first global_tokens slots are never queued (-1: the prompt).
    """

    def __init__(self, B: int, Hkv: int, C: int, D: int, history_window_size: int, drop_amount: int,
                 global_tokens: int):
        super().__init__(B, Hkv, C, history_window_size)
        self.valid[:] = False
        self.k = np.zeros((B, Hkv, C, D))
        self.v = np.zeros((B, Hkv, C, D))
        self.drop_amount = drop_amount
        self.global_tokens = global_tokens
        self.insertions = 0
        self.queue = np.zeros((B, Hkv, 0), dtype=np.int64)
        self.queue_pos = 0

    def prefill(self, k_prompt: np.ndarray, v_prompt: np.ndarray):
        """The prompt fills the first P slots; global_tokens = -1 becomes P."""
        P = k_prompt.shape[2]
        self.k[:, :, :P] = k_prompt
        self.v[:, :, :P] = v_prompt
        self.valid[:, :, :P] = True
        if self.insertions == 0 and self.global_tokens == -1:
            self.global_tokens = P
        self.insertions += P

    def refill(self):
        """The drop_amount evictable slots of the highest low-attention fraction."""
        B, Hkv, C = self.valid.shape
        frac = self.low_fraction()
        frac[..., :self.global_tokens] = -np.inf
        self.queue = topk_select(frac.reshape(B * Hkv, C), self.drop_amount).reshape(B, Hkv, self.drop_amount)
        self.queue_pos = 0

    def next_slots(self) -> np.ndarray:
        """Slot of the next token per (b, g): the next free slot, else the head of the queue."""
        B, Hkv, C = self.valid.shape
        if self.insertions < C:
            return np.full((B, Hkv), self.insertions, dtype=np.int64)
        if self.queue_pos >= self.queue.shape[2]:
            self.refill()
        slots = self.queue[:, :, self.queue_pos].copy()
        self.queue_pos += 1
        return slots

    def insert(self, slots: np.ndarray, k_new: np.ndarray, v_new: np.ndarray):
        """Write the new token into its slots with an empty history."""
        B, Hkv = slots.shape
        for b in range(B):
            for g in range(Hkv):
                e = int(slots[b, g])
                self.k[b, g, e] = k_new[b, g]
                self.v[b, g, e] = v_new[b, g]
                self.valid[b, g, e] = True
                self.attn_history[b, g, e, :] = 0
        self.insertions += 1


def scissorhands_queue_step(cache: ScissorhandsQueueCache, q_t: np.ndarray, k_new: np.ndarray,
                            v_new: np.ndarray):
    """One decode step with insertion: place the new token (R28), attend with
    the step's query over the valid slots (the new token included) and record
    the low bits.  Returns (slots, probs, low bits)."""
    slots = cache.next_slots()
    cache.insert(slots, k_new, v_new)
    probs = window_scores(q_t, cache.k, valid=cache.valid, reduce=REDUCE_GROUP, causal=False)
    low = cache.update_attn_history(probs)
    return slots, probs, low


# ----------------------------------------------------------------------------
# Compositions of the hot path
# ----------------------------------------------------------------------------

def tova(q, k, v, keep: int):
    """TOVA: head-mean window scores, per-KV-head top-k, compaction."""
    B, Hkv, S = k.shape[0], k.shape[1], k.shape[2]
    s = window_scores(q, k, reduce=REDUCE_ALL_HEADS, causal=False)
    idx = topk_select(s.reshape(B * Hkv, S), keep).reshape(B, Hkv, keep)
    return s, idx


def snapkv(q, k, keep: int, chan_keep=None):
    """SnapKV: the prefix is scored by the window (group mean) and competes for
    keep - w slots; the w window positions are always kept (R5)."""
    B, Hkv, S = k.shape[0], k.shape[1], k.shape[2]
    w = q.shape[2]
    s = window_scores(q, k, chan_keep=chan_keep, reduce=REDUCE_GROUP, causal=True)
    idx = topk_select(s.reshape(B * Hkv, S), keep, n_tail=w).reshape(B, Hkv, keep)
    return s, idx


def snapkv_then_think(q, k, keep: int, d_keep: int):
    """The other order ([THINK] review thread: ThinK combined with a press on
    the sequence dimension, applied after it): SnapKV keeps `keep` positions
    with every channel, then the channel scores are taken over the kept keys
    only, with the same window queries, and d_keep key channels are kept (R27).
    Returns (token scores, kept positions, channel scores, kept channels)."""
    s, idx = snapkv(q, k, keep)
    k_kept = np.take_along_axis(k, np.asarray(idx, dtype=np.int64)[..., None], axis=2)
    cs = channel_scores(q, k_kept)
    ch = select_channels(cs, d_keep)
    return s, idx, cs, ch


def think_snapkv(q, k, d_keep: int, keep: int):
    """ThinK then SnapKV: channel scores from the unpruned window queries and
    keys, keep d_keep channels, score tokens with the channel-pruned keys,
    keep tokens as SnapKV."""
    cs = channel_scores(q, k)
    ch = select_channels(cs, d_keep)
    s, idx = snapkv(q, k, keep, chan_keep=ch)
    return cs, ch, s, idx
