// C-ABI entry points of libkvc: argument validation, workspace sizing and dispatch.
// Validation runs before any HIP call, so every error path can be exercised on a
// machine without a GPU.
#include "../../include/kvc.h"

#include "kvc_launch.h"
#include "kvc_plan.h"

namespace {

// Most positions per row (keys of a (b, g), cache slots, entries of a top-k row,
// rows of the channel calls): the kernels keep key and slot indices, chunk ends
// and strided loop counters in 32-bit integers, which stay below 2^31 with this
// margin.
constexpr int kMaxPositions = 1 << 30;

inline bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
inline bool misaligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) != 0; }

inline kvc_status hip_status(hipError_t e) { return e == hipSuccess ? KVC_OK : KVC_ERR_HIP; }

// Shape checks shared by the calls that take a kvc_shape.
kvc_status check_shape(const kvc_shape* sh, bool need_window) {
  if (sh->B < 1 || sh->H < 1 || sh->Hkv < 1 || sh->S < 1) return KVC_ERR_SHAPE;
  if (sh->H % sh->Hkv != 0) return KVC_ERR_SHAPE;
  if (sh->B > 65535 || sh->Hkv > 65535) return KVC_ERR_SHAPE;  // grid y/z limits
  if (need_window && (sh->w < 1 || sh->w > sh->S)) return KVC_ERR_SHAPE;
  if (sh->D != 64 && sh->D != 128) return KVC_ERR_UNSUPPORTED;
  if (sh->S > kMaxPositions) return KVC_ERR_UNSUPPORTED;
  return KVC_OK;
}

}  // namespace

extern "C" {

const char* kvc_status_string(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_ERR_NULL: return "a required pointer is NULL";
    case KVC_ERR_SHAPE: return "sizes out of range or inconsistent";
    case KVC_ERR_DTYPE: return "unknown dtype or reduce mode";
    case KVC_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case KVC_ERR_WORKSPACE: return "workspace too small";
    case KVC_ERR_UNSUPPORTED: return "unsupported size";
    case KVC_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

int32_t kvc_abi_version(void) { return KVC_ABI_VERSION; }

}  // extern "C"

static_assert(kvc::kNoAllocScratchBytes == (size_t)KVC_NOALLOC_SCRATCH_BYTES, "scratch size of the header");

namespace {

// Validation and plan of kvc_window_scores (everything but the workspace).
kvc_status window_scores_check(const kvc_shape* sh, kvc_dtype dt, kvc_reduce reduce, const int32_t* chan_idx,
                               int32_t d_keep, int32_t cu_budget, kvc::WsPlan* plan) {
  if (cu_budget < 0 || cu_budget > kvc::kNumCUs) return KVC_ERR_SHAPE;
  if (dt != KVC_F32 && dt != KVC_BF16) return KVC_ERR_DTYPE;
  if (reduce != KVC_REDUCE_GROUP && reduce != KVC_REDUCE_ALL_HEADS) return KVC_ERR_DTYPE;
  kvc_status st = check_shape(sh, true);
  if (st != KVC_OK) return st;
  if (chan_idx && (d_keep < 1 || d_keep > sh->D)) return KVC_ERR_SHAPE;
  if (!kvc::ws_make_plan(sh->B, sh->H, sh->Hkv, sh->S, sh->w, cu_budget == 0 ? kvc::kNumCUs : cu_budget,
                         kvc::ws_max_waves(dt == KVC_F32, sh->D), plan))
    return KVC_ERR_UNSUPPORTED;
  return KVC_OK;
}

kvc_status window_scores_run(const kvc_shape* sh, kvc_dtype dt, const void* q_win, const void* k,
                             const uint8_t* valid, const int32_t* chan_idx, int32_t d_keep, kvc_reduce reduce,
                             int32_t causal, float* scores, void* ws, const kvc::WsPlan& plan, hipStream_t stream) {
  kvc::WsArgs a;
  a.bf16 = dt == KVC_BF16;
  a.B = sh->B;
  a.H = sh->H;
  a.Hkv = sh->Hkv;
  a.S = sh->S;
  a.D = sh->D;
  a.w = sh->w;
  a.q = q_win;
  a.k = k;
  a.valid = valid;
  a.chan_idx = chan_idx;
  a.d_keep = chan_idx ? d_keep : 0;
  a.reduce = reduce == KVC_REDUCE_ALL_HEADS;
  a.causal = causal != 0;
  a.scores = scores;
  a.ws = ws;
  return hip_status(kvc::launch_window_scores(a, plan, stream));
}

}  // namespace

extern "C" {

kvc_status kvc_window_scores(const kvc_shape* sh, kvc_dtype dt, const void* q_win, const void* k,
                             const uint8_t* valid, const int32_t* chan_idx, int32_t d_keep, kvc_reduce reduce,
                             int32_t causal, float* scores, void* ws, size_t* ws_bytes, hipStream_t stream) {
  return kvc_window_scores_ex(sh, dt, q_win, k, valid, chan_idx, d_keep, reduce, causal, 0, scores, ws, ws_bytes,
                              stream);
}

kvc_status kvc_window_scores_ex(const kvc_shape* sh, kvc_dtype dt, const void* q_win, const void* k,
                                const uint8_t* valid, const int32_t* chan_idx, int32_t d_keep, kvc_reduce reduce,
                                int32_t causal, int32_t cu_budget, float* scores, void* ws,
                                size_t* ws_bytes, hipStream_t stream) {
  if (!sh || !ws_bytes) return KVC_ERR_NULL;
  kvc::WsPlan plan;
  const kvc_status st = window_scores_check(sh, dt, reduce, chan_idx, d_keep, cu_budget, &plan);
  if (st != KVC_OK) return st;
  if (!ws) {
    *ws_bytes = plan.bytes;
    return KVC_OK;
  }
  if (*ws_bytes < plan.bytes) return KVC_ERR_WORKSPACE;
  if (!q_win || !k || !scores) return KVC_ERR_NULL;
  if (misaligned16(q_win) || misaligned16(k) || misaligned4(scores) || misaligned16(ws)) return KVC_ERR_ALIGN;
  return window_scores_run(sh, dt, q_win, k, valid, chan_idx, d_keep, reduce, causal, scores, ws, plan, stream);
}

kvc_status kvc_window_scores_noalloc(const kvc_shape* sh, kvc_dtype dt, const void* q_win, const void* k,
                                     const uint8_t* valid, const int32_t* chan_idx, int32_t d_keep,
                                     kvc_reduce reduce, int32_t causal, float* scores, hipStream_t stream) {
  if (!sh) return KVC_ERR_NULL;
  kvc::WsPlan plan;
  const kvc_status st = window_scores_check(sh, dt, reduce, chan_idx, d_keep, 0, &plan);
  if (st != KVC_OK) return st;
  if (plan.bytes > kvc::kNoAllocScratchBytes) return KVC_ERR_WORKSPACE;
  if (!q_win || !k || !scores) return KVC_ERR_NULL;
  if (misaligned16(q_win) || misaligned16(k) || misaligned4(scores)) return KVC_ERR_ALIGN;
  void* ws = nullptr;
  if (kvc::noalloc_scratch(&ws) != hipSuccess) return KVC_ERR_HIP;
  return window_scores_run(sh, dt, q_win, k, valid, chan_idx, d_keep, reduce, causal, scores, ws, plan, stream);
}

kvc_status kvc_scissor_update(int32_t B, int32_t Hkv, int32_t C, int32_t hist_len, int64_t step,
                              const float* probs, uint8_t* valid, uint32_t* hist, uint16_t* counts,
                              const int64_t* since, float* frac_out, const int32_t* evict_idx, int32_t n_evict,
                              hipStream_t stream) {
  if (B < 1 || Hkv < 1 || C < 1 || hist_len < 1 || hist_len > 65535 || step < 0) return KVC_ERR_SHAPE;
  if ((int64_t)B * Hkv > 0x7fffffffLL) return KVC_ERR_SHAPE;
  if (n_evict < 0 || n_evict > C) return KVC_ERR_SHAPE;
  if (C > kMaxPositions) return KVC_ERR_UNSUPPORTED;
  if (!valid) return KVC_ERR_NULL;
  if (probs && (!hist || !counts)) return KVC_ERR_NULL;
  if (frac_out && !counts) return KVC_ERR_NULL;
  if (probs && (misaligned4(probs) || misaligned4(hist))) return KVC_ERR_ALIGN;
  if ((probs || frac_out) && (reinterpret_cast<uintptr_t>(counts) & 1u)) return KVC_ERR_ALIGN;
  if (frac_out && misaligned4(frac_out)) return KVC_ERR_ALIGN;
  if (since && (reinterpret_cast<uintptr_t>(since) & 7u)) return KVC_ERR_ALIGN;
  kvc::ScissorArgs a;
  a.B = B;
  a.Hkv = Hkv;
  a.C = C;
  a.hist_len = hist_len;
  a.step = step;
  a.probs = probs;
  a.valid = valid;
  a.hist = hist;
  a.counts = counts;
  a.since = since;
  a.frac_out = frac_out;
  a.evict_idx = evict_idx;
  a.n_evict = evict_idx ? n_evict : 0;
  if (!a.probs && !a.frac_out && !a.evict_idx) return KVC_OK;
  return hip_status(kvc::launch_scissor(a, stream));
}

kvc_status kvc_scissor_refill(int32_t B, int32_t Hkv, int32_t C, int32_t hist_len, int64_t step,
                              const uint8_t* valid, const uint16_t* counts, const int64_t* since, int32_t n_protect,
                              int32_t m, int32_t* queue, void* ws, size_t* ws_bytes, hipStream_t stream) {
  if (!ws_bytes) return KVC_ERR_NULL;
  if (B < 1 || Hkv < 1 || C < 1 || hist_len < 1 || hist_len > 65535 || step < 0) return KVC_ERR_SHAPE;
  if ((int64_t)B * Hkv > 65535) return KVC_ERR_SHAPE;
  if (n_protect < 0 || n_protect >= C || m < 1 || m > C - n_protect) return KVC_ERR_SHAPE;
  if (C > kMaxPositions) return KVC_ERR_UNSUPPORTED;
  size_t off_topk = 0;
  const size_t need = kvc::scissor_refill_ws_bytes(B, Hkv, C, &off_topk);
  if (!ws) {
    *ws_bytes = need;
    return KVC_OK;
  }
  if (*ws_bytes < need) return KVC_ERR_WORKSPACE;
  if (!valid || !counts || !queue) return KVC_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(counts) & 1u) || misaligned4(queue) || misaligned16(ws) ||
      (reinterpret_cast<uintptr_t>(since) & 7u))
    return KVC_ERR_ALIGN;
  kvc::ScissorRefillArgs a;
  a.B = B;
  a.Hkv = Hkv;
  a.C = C;
  a.hist_len = hist_len;
  a.step = step;
  a.valid = valid;
  a.counts = counts;
  a.since = since;
  a.n_protect = n_protect;
  a.m = m;
  a.frac = static_cast<float*>(ws);
  a.topk_ws = static_cast<unsigned char*>(ws) + off_topk;
  a.queue = queue;
  return hip_status(kvc::launch_scissor_refill(a, stream));
}

kvc_status kvc_scissor_insert(int32_t B, int32_t Hkv, int32_t C, int32_t D, int32_t hist_len, kvc_dtype dt,
                              const int32_t* queue, int32_t m, int32_t j, int32_t fill_pos, int64_t rec,
                              const void* k_new, const void* v_new, void* k_cache, void* v_cache, uint8_t* valid,
                              uint32_t* hist, uint16_t* counts, int64_t* since, hipStream_t stream) {
  if (dt != KVC_F32 && dt != KVC_BF16) return KVC_ERR_DTYPE;
  if (B < 1 || Hkv < 1 || C < 1 || hist_len < 1 || hist_len > 65535) return KVC_ERR_SHAPE;
  if ((int64_t)B * Hkv > 0x7fffffffLL) return KVC_ERR_SHAPE;
  if (D != 64 && D != 128) return KVC_ERR_UNSUPPORTED;
  if (queue ? (m < 1 || j < 0 || j >= m) : (fill_pos < 0 || fill_pos >= C)) return KVC_ERR_SHAPE;
  if (rec < 0) return KVC_ERR_SHAPE;
  if (C > kMaxPositions) return KVC_ERR_UNSUPPORTED;
  if (!k_new || !k_cache || !valid || !hist || !counts || !since) return KVC_ERR_NULL;
  if (v_new && !v_cache) return KVC_ERR_NULL;
  if (misaligned16(k_new) || misaligned16(k_cache) || (v_new && (misaligned16(v_new) || misaligned16(v_cache))) ||
      misaligned4(hist) || (reinterpret_cast<uintptr_t>(counts) & 1u) || (queue && misaligned4(queue)) ||
      (reinterpret_cast<uintptr_t>(since) & 7u))
    return KVC_ERR_ALIGN;
  kvc::ScissorInsertArgs a;
  a.B = B;
  a.Hkv = Hkv;
  a.C = C;
  a.hist_len = hist_len;
  a.row_bytes = D * (dt == KVC_BF16 ? 2 : 4);
  a.queue = queue;
  a.m = m;
  a.j = j;
  a.fill_pos = fill_pos;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_new ? v_cache : nullptr;
  a.valid = valid;
  a.hist = hist;
  a.counts = counts;
  a.rec = rec;
  a.since = since;
  return hip_status(kvc::launch_scissor_insert(a, stream));
}

kvc_status kvc_channel_scores(const kvc_shape* sh, kvc_dtype dt, const void* q_win, const void* k,
                              float* chan_scores, void* ws, size_t* ws_bytes, hipStream_t stream) {
  if (!sh || !ws_bytes) return KVC_ERR_NULL;
  if (dt != KVC_F32 && dt != KVC_BF16) return KVC_ERR_DTYPE;
  kvc_status st = check_shape(sh, true);
  if (st != KVC_OK) return st;
  kvc::CsPlan plan;
  kvc::cs_make_plan(sh->B, sh->Hkv, sh->S, sh->D, &plan);
  if (!ws) {
    *ws_bytes = plan.bytes;
    return KVC_OK;
  }
  if (*ws_bytes < plan.bytes) return KVC_ERR_WORKSPACE;
  if (!q_win || !k || !chan_scores) return KVC_ERR_NULL;
  if (misaligned16(q_win) || misaligned16(k) || misaligned4(chan_scores) || misaligned4(ws)) return KVC_ERR_ALIGN;
  kvc::CsArgs a;
  a.bf16 = dt == KVC_BF16;
  a.B = sh->B;
  a.H = sh->H;
  a.Hkv = sh->Hkv;
  a.S = sh->S;
  a.D = sh->D;
  a.w = sh->w;
  a.q = q_win;
  a.k = k;
  a.out = chan_scores;
  a.ws = ws;
  return hip_status(kvc::launch_channel_scores(a, plan, stream));
}

kvc_status kvc_topk_select(const float* scores, int32_t rows, int32_t n, int32_t k, int32_t n_tail, int32_t* idx,
                           void* ws, size_t* ws_bytes, hipStream_t stream) {
  if (!ws_bytes) return KVC_ERR_NULL;
  if (rows < 0 || n < 1 || n_tail < 0 || n_tail > k || k > n) return KVC_ERR_SHAPE;
  if (n > kMaxPositions) return KVC_ERR_UNSUPPORTED;
  if (!ws) {
    *ws_bytes = kvc::topk_ws_bytes(rows, n);
    return KVC_OK;
  }
  if (*ws_bytes < kvc::topk_ws_bytes(rows, n)) return KVC_ERR_WORKSPACE;
  if (rows == 0 || k == 0) return KVC_OK;
  if (!scores || !idx) return KVC_ERR_NULL;
  if (misaligned4(scores) || misaligned4(idx)) return KVC_ERR_ALIGN;
  return hip_status(kvc::launch_topk(scores, rows, n, k, n_tail, idx, ws, stream));
}

kvc_status kvc_gather_compact(const kvc_shape* sh, kvc_dtype dt, const void* k, const void* v, const int32_t* idx,
                              int32_t n_keep, const int32_t* chan_idx, int32_t d_keep, void* k_out, void* v_out,
                              hipStream_t stream) {
  if (!sh) return KVC_ERR_NULL;
  if (dt != KVC_F32 && dt != KVC_BF16) return KVC_ERR_DTYPE;
  kvc_status st = check_shape(sh, false);
  if (st != KVC_OK) return st;
  if (n_keep < 0 || n_keep > sh->S) return KVC_ERR_SHAPE;
  if (chan_idx && (d_keep < 1 || d_keep > sh->D)) return KVC_ERR_SHAPE;
  if (n_keep == 0) return KVC_OK;
  if (!k || !idx || !k_out) return KVC_ERR_NULL;
  if (v && !v_out) return KVC_ERR_NULL;
  if (misaligned16(k) || misaligned16(k_out) || (v && (misaligned16(v) || misaligned16(v_out))) ||
      misaligned4(idx))
    return KVC_ERR_ALIGN;
  kvc::GatherArgs a;
  a.bf16 = dt == KVC_BF16;
  a.B = sh->B;
  a.Hkv = sh->Hkv;
  a.S = sh->S;
  a.D = sh->D;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.n_keep = n_keep;
  a.chan_idx = chan_idx;
  a.d_keep = chan_idx ? d_keep : 0;
  a.k_out = k_out;
  a.v_out = v ? v_out : nullptr;
  return hip_status(kvc::launch_gather(a, stream));
}

kvc_status kvc_gather_compress(const kvc_shape* sh, kvc_dtype dt, const void* k, const void* v, const int32_t* idx,
                               int32_t n_keep, const int32_t* chan_idx, int32_t d_keep, void* k_out, void* v_out,
                               hipStream_t stream) {
  if (!sh) return KVC_ERR_NULL;
  if (dt != KVC_F32 && dt != KVC_BF16) return KVC_ERR_DTYPE;
  kvc_status st = check_shape(sh, false);
  if (st != KVC_OK) return st;
  if (n_keep < 0 || n_keep > sh->S || d_keep < 1 || d_keep > sh->D) return KVC_ERR_SHAPE;
  if (n_keep == 0) return KVC_OK;
  if (!k || !idx || !chan_idx || !k_out) return KVC_ERR_NULL;
  if (v && !v_out) return KVC_ERR_NULL;
  const uintptr_t ea = dt == KVC_BF16 ? 1u : 3u;
  if ((reinterpret_cast<uintptr_t>(k) & ea) || (reinterpret_cast<uintptr_t>(k_out) & ea) || misaligned4(idx) ||
      misaligned4(chan_idx) || (v && (misaligned16(v) || misaligned16(v_out))))
    return KVC_ERR_ALIGN;
  if ((long long)sh->B * sh->Hkv > 65535) return KVC_ERR_UNSUPPORTED;  // grid y limit
  if (v) {
    kvc::GatherArgs g;
    g.bf16 = dt == KVC_BF16;
    g.B = sh->B;
    g.Hkv = sh->Hkv;
    g.S = sh->S;
    g.D = sh->D;
    g.k = nullptr;
    g.v = v;
    g.idx = idx;
    g.n_keep = n_keep;
    g.chan_idx = nullptr;
    g.d_keep = 0;
    g.k_out = nullptr;
    g.v_out = v_out;
    const hipError_t e = kvc::launch_gather(g, stream);
    if (e != hipSuccess) return KVC_ERR_HIP;
  }
  kvc::ChanRowsArgs a;
  a.esz = dt == KVC_BF16 ? 2 : 4;
  a.groups = sh->B * sh->Hkv;
  a.H = 0;
  a.Hkv = sh->Hkv;
  a.in = k;
  a.out = k_out;
  a.idx = idx;
  a.chan = chan_idx;
  a.n_rows = n_keep;
  a.in_rows = sh->S;
  a.in_ch = sh->D;
  a.out_ch = d_keep;
  a.d_keep = d_keep;
  a.expand = 0;
  return hip_status(kvc::launch_chan_rows(a, stream));
}

kvc_status kvc_channel_expand(int32_t B, int32_t Hkv, int32_t n, int32_t D, kvc_dtype dt, const void* k_c,
                              const int32_t* chan_idx, int32_t d_keep, void* k_full, hipStream_t stream) {
  if (dt != KVC_F32 && dt != KVC_BF16) return KVC_ERR_DTYPE;
  if (B < 1 || Hkv < 1 || n < 0) return KVC_ERR_SHAPE;
  if (D != 64 && D != 128) return KVC_ERR_UNSUPPORTED;
  if (d_keep < 1 || d_keep > D) return KVC_ERR_SHAPE;
  if (n > kMaxPositions) return KVC_ERR_UNSUPPORTED;
  if (n == 0) return KVC_OK;
  if (!k_c || !chan_idx || !k_full) return KVC_ERR_NULL;
  const uintptr_t ea = dt == KVC_BF16 ? 1u : 3u;
  if ((reinterpret_cast<uintptr_t>(k_c) & ea) || (reinterpret_cast<uintptr_t>(k_full) & ea) || misaligned4(chan_idx))
    return KVC_ERR_ALIGN;
  if ((long long)B * Hkv > 65535) return KVC_ERR_UNSUPPORTED;  // grid y limit
  kvc::ChanRowsArgs a;
  a.esz = dt == KVC_BF16 ? 2 : 4;
  a.groups = B * Hkv;
  a.H = 0;
  a.Hkv = Hkv;
  a.in = k_c;
  a.out = k_full;
  a.idx = nullptr;
  a.chan = chan_idx;
  a.n_rows = n;
  a.in_rows = n;
  a.in_ch = d_keep;
  a.out_ch = D;
  a.d_keep = d_keep;
  a.expand = 1;
  return hip_status(kvc::launch_chan_rows(a, stream));
}

kvc_status kvc_query_channels(int32_t B, int32_t H, int32_t Hkv, int32_t n, int32_t D, kvc_dtype dt, const void* q,
                              const int32_t* chan_idx, int32_t d_keep, void* q_c, hipStream_t stream) {
  if (dt != KVC_F32 && dt != KVC_BF16) return KVC_ERR_DTYPE;
  if (B < 1 || H < 1 || Hkv < 1 || n < 0 || H % Hkv != 0) return KVC_ERR_SHAPE;
  if (D != 64 && D != 128) return KVC_ERR_UNSUPPORTED;
  if (d_keep < 1 || d_keep > D) return KVC_ERR_SHAPE;
  if (n > kMaxPositions) return KVC_ERR_UNSUPPORTED;
  if (n == 0) return KVC_OK;
  if (!q || !chan_idx || !q_c) return KVC_ERR_NULL;
  const uintptr_t ea = dt == KVC_BF16 ? 1u : 3u;
  if ((reinterpret_cast<uintptr_t>(q) & ea) || (reinterpret_cast<uintptr_t>(q_c) & ea) || misaligned4(chan_idx))
    return KVC_ERR_ALIGN;
  if ((long long)B * H > 65535) return KVC_ERR_UNSUPPORTED;  // grid y limit
  kvc::ChanRowsArgs a;
  a.esz = dt == KVC_BF16 ? 2 : 4;
  a.groups = B * H;
  a.H = H;
  a.Hkv = Hkv;
  a.in = q;
  a.out = q_c;
  a.idx = nullptr;
  a.chan = chan_idx;
  a.n_rows = n;
  a.in_rows = n;
  a.in_ch = D;
  a.out_ch = d_keep;
  a.d_keep = d_keep;
  a.expand = 0;
  return hip_status(kvc::launch_chan_rows(a, stream));
}

}  // extern "C"
