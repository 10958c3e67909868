/*
 * kvc.h — KV-cache scoring and pruning for one transformer layer on MI355X (gfx950).
 *
 * The library scores a layer's KV cache from attention statistics of an
 * observation window of queries and prunes it.  It covers TOVA, SnapKV,
 * Scissorhands and ThinK.  Each of them feeds a per-KV-head top-k and the
 * compaction of K/V into the smaller cache.  Sources (web pages):
 *   [TOVA]  "Add TOVA press", NVIDIA kvpress pull request 12 (review thread).
 *   [COLD]  "Implement Scissorhands KV-cache compression & SnapKV prompt
 *           compression", AnswerDotAI cold-compress pull request 11
 *           (cache.py review hunks and the PR description).
 *   [THINK] "Add ThinK_Press", NVIDIA kvpress pull request 18 (review thread).
 *
 * Conventions for every call:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or keeps a pointer after the call returns.
 *   - Work is enqueued asynchronously on `stream` (NULL = the default stream).
 *     There is no host synchronisation inside the library.  A fault on the device
 *     surfaces at the caller's next synchronisation.
 *   - Arguments are validated before anything is enqueued.  On any error nothing
 *     is enqueued and an error status is returned.  KVC_ERR_HIP reports a
 *     failed launch (hipGetLastError after the launch).
 *   - Tensors are dense, row-major and contiguous in the listed shape.  q, k, v
 *     and the compacted outputs must be 16-byte aligned.
 *   - dtype KVC_BF16 means bfloat16 storage and KVC_F32 float32 storage.
 *     Arithmetic is float32: bf16 x bf16 products are exact in fp32 and are
 *     accumulated in fp32.  Scores are float32; indices are int32.
 *   - head_dim D must be 64 or 128 (KVC_ERR_UNSUPPORTED otherwise).
 *   - Positions along one row (the S keys of a KV head, the C cache slots, the n
 *     entries of a top-k row, the n rows of the channel calls) number at most
 *     2^30 (KVC_ERR_UNSUPPORTED otherwise).
 *   - Query head h reads KV head h / (H / Hkv) (the repeat_interleave order of
 *     [COLD]'s GQA hunk).  Window row i (0 <= i < w) is query position S-w+i.
 *   - Calls that take a workspace `ws` use it like this.  With ws == NULL,
 *     the call writes the required byte count to *ws_bytes, returns KVC_OK and
 *     enqueues nothing.  Otherwise *ws_bytes is the size of ws, and
 *     KVC_ERR_WORKSPACE is returned if it is too small.  Workspace contents
 *     need no initialisation and are scratch after the call.
 *   - Calls are reentrant and the library has no global mutable state.  Two
 *     calls that share a workspace or an output must be ordered by the caller,
 *     for example by using one stream.
 *   - NaN inputs give unspecified (but in-bounds) results.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 5

typedef enum {
  KVC_OK = 0,
  KVC_ERR_NULL = 1,        /* a required pointer is NULL                      */
  KVC_ERR_SHAPE = 2,       /* sizes out of range or inconsistent              */
  KVC_ERR_DTYPE = 3,       /* unknown dtype / reduce mode                      */
  KVC_ERR_ALIGN = 4,       /* q, k, v or a compacted output not 16-B aligned  */
  KVC_ERR_WORKSPACE = 5,   /* *ws_bytes smaller than the required workspace   */
  KVC_ERR_UNSUPPORTED = 6, /* a valid but unsupported size (e.g. D not 64/128) */
  KVC_ERR_HIP = 7          /* a kernel launch failed                           */
} kvc_status;

typedef enum { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype;

typedef enum {
  /* Mean over the G query heads of each GQA group and the w window rows:
   * SnapKV's window scoring and Scissorhands' attention callback ([COLD],
   * attention-callback hunk: the callback receives the attention averaged over
   * the query heads that share a KV head). */
  KVC_REDUCE_GROUP = 0,
  /* Mean over all H query heads and the w window rows, the same row written
   * for every KV head ([TOVA]: attn_weights.mean(1) followed by a repeat
   * over num_key_value_heads). */
  KVC_REDUCE_ALL_HEADS = 1
} kvc_reduce;

typedef struct {
  int32_t B;   /* batch                                    */
  int32_t H;   /* query heads (multiple of Hkv)            */
  int32_t Hkv; /* KV heads                                 */
  int32_t S;   /* cache positions (keys)                   */
  int32_t D;   /* head_dim: 64 or 128                      */
  int32_t w;   /* observation-window rows, 1 <= w <= S     */
} kvc_shape;

/*
 * kvc_window_scores — observation-window attention scores per KV head.
 *
 * Defines ([TOVA] SimJeg's reply: only the last window_size rows of the
 * attention, shape [batch, heads, window_size, seq_len], are computed):
 *   l[b,h,i,j] = sum_{d in keep(b,g)} q[b,h,i,d] * k[b,g,j,d] / sqrt(D),   g = h / (H/Hkv)
 *   allowed(b,g,i,j) = valid[b,g,j] != 0  and  (!causal or j <= S-w+i)
 *   P[b,h,i,j] = exp(l - logsumexp over allowed j of l) on allowed entries, else 0
 *   GROUP:     scores[b,g,j] = 1/(G*w) * sum_{h in group g} sum_i P[b,h,i,j]
 *   ALL_HEADS: scores[b,g,j] = 1/(H*w) * sum_h sum_i P[b,h,i,j]   (same for every g)
 * A row with no allowed key contributes P = 0.
 *
 * Arguments:
 *   sh        shape (B, H, Hkv, S, D, w).  Needs H % Hkv == 0 and G*w <= 1024.
 *   dt        storage type of q_win and k.
 *   q_win     [B, H, w, D] window queries (already position-encoded by the caller).
 *   k         [B, Hkv, S, D] cache keys.
 *   valid     [B, Hkv, S] uint8 (0 = hole, excluded) or NULL (all valid).
 *   chan_idx  [B, Hkv, d_keep] int32 kept key channels, or NULL (all D channels).
 *             Entries must be distinct and in [0, D).  Pruned channels count as zero
 *             keys ([THINK] option 3a: zeros in the key cache).
 *   d_keep    number of kept channels (ignored when chan_idx is NULL), 1..D.
 *   reduce    KVC_REDUCE_GROUP or KVC_REDUCE_ALL_HEADS.
 *   causal    nonzero: window row i attends keys j <= S-w+i (no effect when w == 1).
 *   scores    out [B, Hkv, S] float32.
 *   ws, ws_bytes  workspace (see the conventions above).
 */
kvc_status kvc_window_scores(const kvc_shape* sh, kvc_dtype dt, const void* q_win, const void* k,
                             const uint8_t* valid, const int32_t* chan_idx, int32_t d_keep,
                             kvc_reduce reduce, int32_t causal, float* scores, void* ws,
                             size_t* ws_bytes, hipStream_t stream);

/*
 * kvc_window_scores_ex — kvc_window_scores planned for part of the GPU, for
 * callers that score several layers (or sequences) at the same time on
 * different streams.
 *
 * Same definition, arguments and errors as kvc_window_scores, plus:
 *   cu_budget  the number of the GPU's 256 compute units the call is planned
 *             for.  0 or 256: one call fills the GPU (what kvc_window_scores
 *             does).  Less: the call uses about that many compute units, with
 *             correspondingly longer key chunks per workgroup, so that several
 *             calls (128 each for two) and the other streams' kernels run side
 *             by side instead of each call waiting for the whole chip; a call
 *             running alone then takes longer.  0..256, else KVC_ERR_SHAPE.
 * The budget changes the key chunking and with it the order in which the float
 * sums are added: scores may differ from those of another budget by float
 * rounding (within the same tolerance of the definition); for a given budget
 * they are deterministic.  The workspace size depends on the budget: query it
 * with the same value.
 */
kvc_status kvc_window_scores_ex(const kvc_shape* sh, kvc_dtype dt, const void* q_win, const void* k,
                                const uint8_t* valid, const int32_t* chan_idx, int32_t d_keep,
                                kvc_reduce reduce, int32_t causal, int32_t cu_budget, float* scores,
                                void* ws, size_t* ws_bytes, hipStream_t stream);

/*
 * kvc_window_scores_noalloc — kvc_window_scores without a workspace argument
 * and without any device allocation.
 *
 * For callers that cannot allocate device memory: code under HIP stream
 * capture, serving loops that forbid allocation, harnesses that disallow it.
 * Same arguments, definition, results and errors as kvc_window_scores, minus
 * ws/ws_bytes.  Its scratch (the per-chunk row statistics, the log-normalisers
 * and, for G*w <= 16, the stored logits) lives in one fixed device array of
 * KVC_NOALLOC_SCRATCH_BYTES per GPU, which the library holds from the first
 * call on that GPU until the process ends.  A shape whose kvc_window_scores
 * workspace exceeds that size returns KVC_ERR_WORKSPACE and enqueues nothing.
 * The scratch needs no initialisation.  Every call on one GPU shares that GPU's
 * array: two calls that may overlap on the same GPU (different streams without
 * ordering between them, or different host threads) race and give undefined
 * scores.  Calls on one stream are ordered and safe.
 */
#define KVC_NOALLOC_SCRATCH_BYTES (32u << 20)
kvc_status kvc_window_scores_noalloc(const kvc_shape* sh, kvc_dtype dt, const void* q_win, const void* k,
                                     const uint8_t* valid, const int32_t* chan_idx, int32_t d_keep,
                                     kvc_reduce reduce, int32_t causal, float* scores, hipStream_t stream);

/*
 * kvc_scissor_update — Scissorhands low-attention history (record and evict).
 *
 * [COLD] cache.py hunks: a slot counts as unimportant at a step when its
 * probability is below that of uniform attention over the cache (1/keys), and
 * the newest indicator overwrites the oldest of a circular window of steps.
 * [COLD] PR description: every m steps each head evicts the tokens that were
 * unimportant on the largest share of their observed steps; bulk eviction
 * leaves empty slots.  [COLD] review thread: a token's share counts only the
 * steps on which it was observed (both the numerator and the denominator).
 *
 * State (caller-owned device buffers, which persist across steps):
 *   valid  [B, Hkv, C] uint8, 1 = occupied slot, 0 = hole.
 *   hist   [hist_len][B*Hkv][ceil(C/32)] uint32 bit-planes.  Bit (c % 32) of word
 *          c/32 in plane p holds the indicator recorded at the last recording r
 *          with r % hist_len == p.  Zero it before the first recording.
 *   counts [B, Hkv, C] uint16, the number of set bits of slot c over the planes.
 *          Zero it before the first recording.
 *   since  [B, Hkv, C] int64 or NULL: the number of recordings made before the
 *          slot's current token arrived (kvc_scissor_insert writes it; 0 for
 *          tokens present from the start).  NULL means 0 for every slot.
 *
 * When probs != NULL (recording number `step`, counted from 0):
 *   S_t = number of valid slots of (b, g);
 *   low = valid[c] and probs[c] < 1/S_t (compared exactly: probs is widened to double);
 *   plane = step % hist_len: counts += low - old bit;  bit <- low.
 * If frac_out != NULL, it is written after the record (or from the current
 * counts when probs == NULL, `step` then being the last recording's number):
 *   n_obs = min(step + 1 - since[c], hist_len)  (the slot's own observations)
 *   frac_out[b,g,c] = counts / n_obs (correctly rounded; 0 when n_obs <= 0) at
 *   valid slots and -inf at holes.
 * Sampled recording ([COLD] review thread: the paper checks the attention every
 * M steps only): record with step = the number of recordings so far, and ask
 * for the fraction alone at an eviction step that records nothing.
 * When evict_idx != NULL (after the record, if both are given):
 *   valid[b, g, evict_idx[b,g,e]] = 0 for e < n_evict.  The indices must be in
 *   [0, C) (e.g. kvc_topk_select over frac_out with k = n_evict).
 *
 *   probs     [B, Hkv, C] float32 group-mean probabilities of this step (the
 *             kvc_window_scores output with w = 1, KVC_REDUCE_GROUP and valid), or NULL.
 *   hist_len  1..65535 (400 in [COLD]).  step >= 0.  since 8-byte aligned.
 */
kvc_status kvc_scissor_update(int32_t B, int32_t Hkv, int32_t C, int32_t hist_len, int64_t step,
                              const float* probs, uint8_t* valid, uint32_t* hist, uint16_t* counts,
                              const int64_t* since, float* frac_out, const int32_t* evict_idx, int32_t n_evict,
                              hipStream_t stream);

/*
 * kvc_scissor_refill — refill of the Scissorhands eviction queue.
 *
 * [COLD] PR description: instead of evicting in bulk, an eviction queue is
 * rebuilt periodically and supplies one slot per step; cache.py hunk: a
 * setting keeps the prompt tokens for good.  The queue takes the m slots of
 * the largest low-attention fraction, each over its own observations:
 *   frac[b,g,c] = counts / min(step + 1 - since[c], hist_len) (0 with no
 *                 observation) at valid slots with c >= n_protect, -inf
 *                 elsewhere (holes and the protected prefix);
 *   queue[b,g,:] = kvc_topk_select(frac[b,g,:], m)  (ascending positions, lowest
 *                 index first among equal fractions).
 * `step` is the last recording's number.  At least m slots of every row must be
 * valid and unprotected (else -inf entries, that is holes or protected slots,
 * fill the rest of the queue).
 *   valid [B, Hkv, C] uint8;  counts [B, Hkv, C] uint16;  since [B, Hkv, C] int64
 *         or NULL (kvc_scissor_update's state).
 *   0 <= n_protect < C;  1 <= m <= C - n_protect;  queue out [B, Hkv, m] int32.
 *   ws, ws_bytes  workspace (the fraction and the top-k's; see the conventions above).
 */
kvc_status kvc_scissor_refill(int32_t B, int32_t Hkv, int32_t C, int32_t hist_len, int64_t step,
                              const uint8_t* valid, const uint16_t* counts, const int64_t* since, int32_t n_protect,
                              int32_t m, int32_t* queue, void* ws, size_t* ws_bytes, hipStream_t stream);

/*
 * kvc_scissor_insert — a decode step's new token into the Scissorhands cache.
 *
 * [COLD] PR description: the eviction queue supplies one slot per step, so the
 * new token replaces the evicted one and no hole is left.  The slot of row
 * (b, g) is queue[b,g,j], or fill_pos for every row when queue is NULL (the
 * cache is not full yet).  Then:
 *   k_cache[b,g,slot,:] = k_new[b,g,:];  v_cache likewise (when v_new != NULL);
 *   valid[b,g,slot] = 1;  counts[b,g,slot] = 0;  since[b,g,slot] = rec;  the
 *   slot's bit is cleared in every history plane (the new token starts with no
 *   observation).
 * A slot outside [0, C) leaves its row unchanged.
 *   rec       the number of recordings made before this token (>= 0); the next
 *             kvc_scissor_update record is the first to observe it.
 *   k_new, v_new [B, Hkv, D];  k_cache, v_cache [B, Hkv, C, D] (16-byte aligned).
 *   hist, counts, valid, since: kvc_scissor_update's state (since required,
 *   8-byte aligned).  0 <= j < m; 0 <= fill_pos < C.
 */
kvc_status kvc_scissor_insert(int32_t B, int32_t Hkv, int32_t C, int32_t D, int32_t hist_len, kvc_dtype dt,
                              const int32_t* queue, int32_t m, int32_t j, int32_t fill_pos, int64_t rec,
                              const void* k_new, const void* v_new, void* k_cache, void* v_cache, uint8_t* valid,
                              uint32_t* hist, uint16_t* counts, int64_t* since, hipStream_t stream);

/*
 * kvc_channel_scores — ThinK per-channel key importance.
 *
 * [THINK] yuhuixu1993's factorised score (equal to the squared, summed
 * channel_attn of shape (bsz, num_heads, head_dim, window_size, seq_len)):
 *   chan_scores[b,g,d] = ( sum_{h in group g} sum_{i<w} q[b,h,i,d]^2 ) * ( sum_{j<S} k[b,g,j,d]^2 )
 * Sums run over positions: window rows for q and all S keys for k.  Pruning zeroes
 * the channels with the smallest scores (kvc_topk_select over rows (b,g) with
 * n = D, then chan_idx for kvc_window_scores / kvc_gather_compact).
 *   chan_scores  out [B, Hkv, D] float32.  Sums are deterministic (fixed order).
 */
kvc_status kvc_channel_scores(const kvc_shape* sh, kvc_dtype dt, const void* q_win, const void* k,
                              float* chan_scores, void* ws, size_t* ws_bytes, hipStream_t stream);

/*
 * kvc_topk_select — per-row top-k with a forced tail, in ascending index order.
 *
 * Row r of `scores` has n entries.  Its last n_tail positions are always kept
 * ([COLD] PR description: SnapKV keeps every observation-window token and
 * compresses the prefix).  The first n - n_tail positions compete for
 * k - n_tail slots.  A larger score wins; among equal scores the lower index
 * wins (-0.0 counts as +0.0).  idx[r, :] lists the kept positions in
 * ascending order, so the tail comes last.  The kept set is unique.  The same
 * call picks Scissorhands evictions (largest low-attention fraction) and
 * ThinK channels.
 *   scores [rows, n] float32;  idx out [rows, k] int32;  0 <= n_tail <= k <= n.
 */
kvc_status kvc_topk_select(const float* scores, int32_t rows, int32_t n, int32_t k, int32_t n_tail,
                           int32_t* idx, void* ws, size_t* ws_bytes, hipStream_t stream);

/*
 * kvc_gather_compact — compacted cache from the kept positions.
 *
 *   k_out[b,g,r,:] = k[b,g,idx[b,g,r],:], with the channels not listed in
 *                    chan_idx[b,g,:] written as +0.0 ([THINK] option 3a: zeros
 *                    in the key cache);
 *   v_out[b,g,r,:] = v[b,g,idx[b,g,r],:].
 * This is a bit copy (kept channels are bit-identical).
 *   k, v        [B, Hkv, S, D] (sh->w is ignored); v may be NULL (then v_out is unused).
 *   idx         [B, Hkv, n_keep] int32 in [0, S).
 *   chan_idx    [B, Hkv, d_keep] int32 or NULL (keep every channel).
 *   k_out, v_out  [B, Hkv, n_keep, D] (must not overlap k or v).
 */
kvc_status kvc_gather_compact(const kvc_shape* sh, kvc_dtype dt, const void* k, const void* v,
                              const int32_t* idx, int32_t n_keep, const int32_t* chan_idx,
                              int32_t d_keep, void* k_out, void* v_out, hipStream_t stream);

/*
 * kvc_gather_compress — compacted cache that stores only the kept key channels
 * ([THINK] review thread, options 3b and 3c: keep the pruned key cache apart
 * so that pruning channels also saves their memory).
 *   k_out[b,g,r,j] = k[b,g,idx[b,g,r],chan_idx[b,g,j]]   for j < d_keep
 *   v_out[b,g,r,:] = v[b,g,idx[b,g,r],:]                 (V keeps every channel)
 * A bit copy.  The order of chan_idx is the stored channel order
 * (kvc_topk_select gives ascending); entries must be in [0, D) (an entry
 * outside writes 0).
 *   k, v        [B, Hkv, S, D] (sh->w is ignored); v may be NULL (then v_out is unused).
 *   idx         [B, Hkv, n_keep] int32 in [0, S) (clamped into range).
 *   chan_idx    [B, Hkv, d_keep] int32, required, 1 <= d_keep <= D.
 *   k_out       [B, Hkv, n_keep, d_keep]; k and k_out need element alignment only.
 *   v_out       [B, Hkv, n_keep, D]; v and v_out 16-byte aligned.
 * Outputs must not overlap the inputs.
 */
kvc_status kvc_gather_compress(const kvc_shape* sh, kvc_dtype dt, const void* k, const void* v,
                               const int32_t* idx, int32_t n_keep, const int32_t* chan_idx,
                               int32_t d_keep, void* k_out, void* v_out, hipStream_t stream);

/*
 * kvc_channel_expand — the zeros added back to a compressed key cache
 * ([THINK] option 3b: a cache class that restores the pruned channels as zeros
 * when the keys are used).
 *   k_full[b,g,r,c] = k_c[b,g,r,j] where chan_idx[b,g,j] == c (the largest such
 *                     j if an entry repeats), +0.0 for every other channel.
 *   k_c [B, Hkv, n, d_keep];  chan_idx [B, Hkv, d_keep];  k_full out [B, Hkv, n, D].
 *   1 <= d_keep <= D, D in {64, 128}; n == 0 is a no-op.  Element alignment.
 * Expanding kvc_gather_compress's keys gives kvc_gather_compact's, bit for bit.
 */
kvc_status kvc_channel_expand(int32_t B, int32_t Hkv, int32_t n, int32_t D, kvc_dtype dt, const void* k_c,
                              const int32_t* chan_idx, int32_t d_keep, void* k_full, hipStream_t stream);

/*
 * kvc_query_channels — queries cut to their KV head's kept key channels
 * ([THINK] option 3c: prune the query the same way, so that attention runs on
 * the compressed keys; q_c . k_c equals q . k with the pruned key channels
 * zeroed, up to the order of the sum).
 *   q_c[b,h,i,j] = q[b,h,i,chan_idx[b, h/G, j]],  G = H / Hkv.
 *   q [B, H, n, D];  chan_idx [B, Hkv, d_keep];  q_c out [B, H, n, d_keep].
 *   1 <= d_keep <= D, D in {64, 128}; n == 0 is a no-op.  Element alignment.
 */
kvc_status kvc_query_channels(int32_t B, int32_t H, int32_t Hkv, int32_t n, int32_t D, kvc_dtype dt,
                              const void* q, const int32_t* chan_idx, int32_t d_keep, void* q_c,
                              hipStream_t stream);

/* Text for a status code (static storage). */
const char* kvc_status_string(kvc_status s);

/* KVC_ABI_VERSION of the built library. */
int32_t kvc_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H */
