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
  R14 the low-attention fraction of a slot is its low count over its own
      observations: the recordings since its token arrived, at most the last
      `history` of them.  Without insertion that is min(recordings, history)
      for every slot.
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
      never-used slot while there is one, else into the head of the eviction
      queue; the token starts with no observation; the step then attends with
      the new token in the cache and records.
  R29 the eviction queue is rebuilt when it is empty on a full cache, with
      the top-k (O4) of the low-attention fraction, k = drop_amount,
      ascending positions, popped front to back.
  R30 the first n_protect slots are never queued; a negative setting protects
      the prompt, whatever its length.
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
# O5: Scissorhands low-attention counting, bulk eviction and the eviction queue
# ----------------------------------------------------------------------------

class LowAttentionState:
    """One layer's Scissorhands bookkeeping, kept as its plain definition.

    Source: "Implement Scissorhands KV-cache compression & SnapKV prompt
    compression" (cold-compress PR 11).  The cache.py review hunks call a slot
    unimportant at a step when its attention falls below that of uniform
    attention over the cache, and keep those indicators for a bounded number
    of recent steps.  The PR description ranks the tokens of each head by the
    share of their observed steps on which they were unimportant, and the
    review thread counts per token both the unimportant steps (the numerator)
    and the observed steps (the denominator).

    State per (batch, KV head, slot):
      valid  the slot holds a token (bulk eviction leaves holes, R15);
      since  index of the first recording that saw the slot's current token:
             0 for tokens present before the first recording, the number of
             recordings made before its insertion otherwise (R28).
    and every recorded indicator array by recording index; only the last
    `history` recordings can ever count, so older ones are dropped.

    For one slot, with n recordings made so far, the recordings that count are
    those with index r in [max(since, n - history), n) (R14):
      count        how many of them found the slot low;
      observations how many there are;
      fraction     count / observations (0 without an observation), -inf at holes.
    """

    def __init__(self, B: int, Hkv: int, C: int, history: int = 400):
        self.history = history
        self.valid = np.ones((B, Hkv, C), dtype=bool)
        self.since = np.zeros((B, Hkv, C), dtype=np.int64)
        self.recordings: dict[int, np.ndarray] = {}
        self.n = 0

    @classmethod
    def from_recordings(cls, valid, since, recordings: dict, n: int, history: int) -> "LowAttentionState":
        """A state given explicitly: `recordings` maps recording index -> low
        indicators [B, Hkv, C] (indices below n - history are ignored)."""
        valid = np.asarray(valid, dtype=bool)
        st = cls(*valid.shape, history)
        st.valid = valid.copy()
        st.since = np.asarray(since, dtype=np.int64).copy()
        st.n = int(n)
        st.recordings = {int(r): np.asarray(v, dtype=bool).copy() for r, v in recordings.items()
                         if n - history <= r < n}
        return st

    def record(self, probs: np.ndarray) -> np.ndarray:
        """Record one step's group-mean probabilities [B, Hkv, C]: a valid slot
        is low when its probability is below 1/S_t, S_t the number of valid
        slots of its (batch, KV head) (R11, R12; strictly below)."""
        n_valid = self.valid.sum(axis=-1, keepdims=True)
        uniform = np.where(n_valid > 0, 1.0 / np.maximum(n_valid, 1), 0.0)
        low = self.valid & (np.asarray(probs) < uniform)
        self.recordings[self.n] = low.copy()
        self.n += 1
        self.recordings.pop(self.n - 1 - self.history, None)
        return low

    def _first_counted(self) -> np.ndarray:
        return np.maximum(self.since, self.n - self.history)

    def counts(self) -> np.ndarray:
        lo = self._first_counted()
        c = np.zeros(self.valid.shape, dtype=np.int64)
        for r, low in self.recordings.items():
            c += low & (r >= lo)
        return c

    def observations(self) -> np.ndarray:
        return np.maximum(self.n - self._first_counted(), 0)

    def fraction(self) -> np.ndarray:
        obs = self.observations()
        frac = np.where(obs > 0, self.counts() / np.maximum(obs, 1), 0.0)
        return np.where(self.valid, frac, -np.inf)

    def evict(self, n_evict: int) -> np.ndarray:
        """Bulk eviction ([COLD] PR description): per (batch, KV head), the
        n_evict valid slots of the largest fraction (O4: the lowest index first
        among equals) become holes.  Returns them [B, Hkv, n_evict] ascending."""
        B, Hkv, C = self.valid.shape
        idx = topk_select(self.fraction().reshape(B * Hkv, C), n_evict).reshape(B, Hkv, n_evict)
        for b in range(B):
            for g in range(Hkv):
                self.valid[b, g, idx[b, g]] = False
        return idx

    def occupy(self, slots: np.ndarray):
        """A new token in slot slots[b, g] of each row: valid, observed from the
        next recording on."""
        B, Hkv = slots.shape
        for b in range(B):
            for g in range(Hkv):
                e = int(slots[b, g])
                self.valid[b, g, e] = True
                self.since[b, g, e] = self.n


def scissorhands_step(state: LowAttentionState, q_t: np.ndarray, k: np.ndarray, t: int,
                      evict_every: int, n_evict: int, record_every: int = 1):
    """One decode step: the step's group-mean attention over the valid slots is
    recorded, and every evict_every steps n_evict slots per (batch, KV head)
    are evicted.  With record_every = M > 1 the attention is checked and
    recorded only at the steps t with t % M == 0 ([COLD] review thread: the
    paper checks the attention every M steps only), so the window and the
    observations count recordings (R26).  Returns (probs, low bits, evicted
    indices or None); probs and low are None at a step that records nothing."""
    probs = low = None
    if t % record_every == 0:
        probs = window_scores(q_t, k, valid=state.valid, reduce=REDUCE_GROUP, causal=False)
        low = state.record(probs)
    evicted = state.evict(n_evict) if (t + 1) % evict_every == 0 else None
    return probs, low, evicted


class ScissorhandsQueue(LowAttentionState):
    """Scissorhands with insertion and an eviction queue ([COLD] PR description:
    the queue is rebuilt periodically and supplies one slot per step, so no
    hole is left; cache.py hunk: a setting keeps the prompt tokens for good).
    The cache has C slots holding K and V.  Readings R28-R30:
      * a step's token goes to the next never-used slot while there is one,
        else to the slot at the head of the queue; it starts unobserved;
      * an empty queue on a full cache is rebuilt from the drop_amount slots of
        the largest fraction (O4: ascending positions, popped front to back);
      * the first n_protect slots are never queued; a negative setting
        protects the prompt, whatever its length.
    """

    def __init__(self, B: int, Hkv: int, C: int, D: int, history: int, drop_amount: int, protect: int):
        super().__init__(B, Hkv, C, history)
        self.valid[:] = False
        self.k = np.zeros((B, Hkv, C, D))
        self.v = np.zeros((B, Hkv, C, D))
        self.drop_amount = drop_amount
        self.protect = protect
        self.n_protect = max(protect, 0)
        self.filled = 0
        self.queue = np.zeros((B, Hkv, 0), dtype=np.int64)
        self.queue_pos = 0

    def prefill(self, k_prompt: np.ndarray, v_prompt: np.ndarray):
        """The prompt takes the first P slots (observed from the first recording)."""
        P = k_prompt.shape[2]
        self.k[:, :, :P] = k_prompt
        self.v[:, :, :P] = v_prompt
        self.valid[:, :, :P] = True
        self.filled = P
        if self.protect < 0:
            self.n_protect = P

    def refill(self):
        B, Hkv, C = self.valid.shape
        frac = self.fraction()
        frac[..., :self.n_protect] = -np.inf
        self.queue = topk_select(frac.reshape(B * Hkv, C), self.drop_amount).reshape(B, Hkv, self.drop_amount)
        self.queue_pos = 0

    def next_slots(self) -> np.ndarray:
        B, Hkv, C = self.valid.shape
        if self.filled < C:
            return np.full((B, Hkv), self.filled, dtype=np.int64)
        if self.queue_pos >= self.queue.shape[2]:
            self.refill()
        slots = self.queue[:, :, self.queue_pos].copy()
        self.queue_pos += 1
        return slots

    def insert(self, slots: np.ndarray, k_new: np.ndarray, v_new: np.ndarray):
        B, Hkv = slots.shape
        for b in range(B):
            for g in range(Hkv):
                e = int(slots[b, g])
                self.k[b, g, e] = k_new[b, g]
                self.v[b, g, e] = v_new[b, g]
        self.occupy(slots)
        self.filled += 1


def scissorhands_queue_step(cache: ScissorhandsQueue, q_t: np.ndarray, k_new: np.ndarray, v_new: np.ndarray):
    """One decode step with insertion: place the new token (R28), attend with
    the step's query over the valid slots, the new token included, and record.
    Returns (slots, probs, low bits)."""
    slots = cache.next_slots()
    cache.insert(slots, k_new, v_new)
    probs = window_scores(q_t, cache.k, valid=cache.valid, reduce=REDUCE_GROUP, causal=False)
    low = cache.record(probs)
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
