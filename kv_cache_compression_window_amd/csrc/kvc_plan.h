// Host-side launch planning shared by the C-ABI entry points and the launchers.
// Plain C++ (no device code): sizes, tilings and workspace layouts.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace kvc {

// Key granularity of the window-score chunks: chunks are multiples of 128 keys
// (two 64-key tiles of the stream kernels, four 32-key blocks of the
// stored-logits kernel).
constexpr int kTileKeys = 128;

// How kvc_window_scores runs a given shape.
//  * two-pass path (rows per KV head R > 16): pass 1 computes per-row (max, sum
//    of exp2) over a chunk of keys; pass 2 combines the chunks' partials into
//    each row's log-normaliser, recomputes the logits and sums the normalised
//    probabilities over the group's rows;
//  * stored-logits path (R <= 16): pass 1 also writes the scaled logits of the
//    real rows, and a light kernel normalises and reduces them, so the keys are
//    read from HBM once.
struct WsPlan {
  bool store;       // stored-logits path
  int NW;           // waves per workgroup: one wave per 32 query rows
  int R, Rpad;      // rows per KV head (G*w) and padded rows (nrch * NW * 32)
  int nrch;         // row chunks of NW*32 rows (several only when R > 256)
  int CH, nchunks;  // keys per chunk (multiple of kTileKeys) and chunks per (b,g)
  int Spad;         // row stride of the stored logits (multiple of kTileKeys)
  size_t off_part, off_lse, off_logits, bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kMaxRows = 1024;  // G*w limit per KV head
// Size of the fixed device scratch of kvc_window_scores_noalloc (one copy per GPU).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
constexpr int kMergeLanes = 8;  // lanes of the merge kernel per (b, g, row)

// Compute units of an MI355X.  A score call is planned for a budget of them
// (`cu_budget`, 1..kNumCUs): the whole GPU by default; callers that keep several
// calls and other kernels running at once on different streams give each call a
// part, so that the calls run side by side with longer key chunks instead of
// queueing for the whole chip.
constexpr int kNumCUs = 256;

// Most waves per workgroup for a storage type and head size: eight-wave
// workgroups run two waves per SIMD, which leaves each wave 256 registers; fp32
// rows of 128 channels need more than that (their query and key fragments are
// twice the bf16 ones), so they run at most four waves (one per SIMD, up to 512
// registers each).
inline int ws_max_waves(bool fp32, int D) { return fp32 && D == 128 ? 4 : 8; }

inline bool ws_make_plan(int B, int H, int Hkv, int S, int w, int cu_budget, int max_nw, WsPlan* p) {
  const int G = H / Hkv;
  const long long R = (long long)G * w;
  if (R > kMaxRows) return false;
  p->R = (int)R;
  p->store = R <= 16;
  const long long bg = (long long)B * Hkv;
  // one wave per 32 query rows, up to 8 waves (max_nw); beyond NW*32 rows the
  // rows are processed in chunks of NW*32 by successive launches
  const int nrb = (int)((R + 31) / 32);
  p->NW = nrb <= 1 ? 1 : nrb == 2 ? 2 : nrb <= 4 ? 4 : 8;
  if (p->NW > max_nw) p->NW = max_nw;
  p->nrch = (nrb + p->NW - 1) / p->NW;
  p->Rpad = p->nrch * p->NW * 32;
  // the merge kernel indexes rows and lanes in 32-bit integers
  if (bg * p->Rpad * kMergeLanes > 0x7fffffffLL) return false;
  // workgroups to aim for: about eight waves per budgeted CU on the two-pass
  // path, two four-wave streaming workgroups per budgeted CU on the (HBM-bound)
  // stored-logits path
  const int cus = cu_budget < 1 || cu_budget > kNumCUs ? kNumCUs : cu_budget;
  long long target = (p->store ? 2LL : 8LL / p->NW) * cus;
  long long nch = (target + bg - 1) / bg;
  if (p->store) {
    // stored-logits chunks of at least 1024 keys (a quarter of the row when that
    // is shorter): fewer, longer workgroups overlap better with the work of
    // other streams and lose little alone
    long long min_keys = S / 4 < kTileKeys ? kTileKeys : S / 4;
    if (min_keys > 1024) min_keys = 1024;
    const long long by_len = S / min_keys < 1 ? 1 : S / min_keys;
    if (nch > by_len) nch = by_len;
  }
  const long long max_ch = (S + kTileKeys - 1) / kTileKeys;
  if (nch > max_ch) nch = max_ch;
  if (nch < 1) nch = 1;
  long long per = (S + nch - 1) / nch;
  per = (per + kTileKeys - 1) / kTileKeys * kTileKeys;
  p->CH = (int)per;
  p->nchunks = (int)((S + per - 1) / per);
  p->Spad = (int)((S + kTileKeys - 1) / kTileKeys * kTileKeys);
  size_t off = 0;
  p->off_part = off;
  off += align256((size_t)bg * p->Rpad * p->nchunks * 2 * sizeof(float));
  p->off_lse = off;
  off += align256((size_t)bg * p->Rpad * sizeof(float));
  p->off_logits = off;
  if (p->store) off += align256((size_t)bg * p->R * p->Spad * sizeof(float));
  p->bytes = off;
  return true;
}

// kvc_channel_scores: keys per chunk of the partial sums of k^2.
struct CsPlan {
  int CH, nchunks;
  size_t bytes;
};

inline void cs_make_plan(int B, int Hkv, int S, int D, CsPlan* p) {
  const long long bg = (long long)B * Hkv;
  long long nch = (2048 + bg - 1) / bg;
  const long long max_ch = (S + 63) / 64;
  if (nch > max_ch) nch = max_ch;
  if (nch < 1) nch = 1;
  long long per = (S + nch - 1) / nch;
  per = (per + 63) / 64 * 64;
  p->CH = (int)per;
  p->nchunks = (int)((S + per - 1) / per);
  p->bytes = align256((size_t)bg * p->nchunks * D * sizeof(float));
}

// kvc_topk_select: rows of at most kTopkResident positions are selected by one
// workgroup each (no workspace beyond a small fixed area).  Longer rows are cut
// into slices of kTopkSlice positions, one workgroup each; the workspace holds
// per row three global digit histograms and the selection state, and per slice
// the counts above and at the threshold.
constexpr int kTopkResident = 32768;
constexpr int kTopkSlice = 4096;
constexpr int kTopkBins = 2048;  // bins of the widest digit

struct TkPlan {
  int nslices;
  size_t off_hist, off_state, off_cnt, bytes;
};

inline void topk_make_plan(int rows, int n, TkPlan* p) {
  p->nslices = (n + kTopkSlice - 1) / kTopkSlice;
  size_t off = 0;
  p->off_hist = off;
  off += align256((size_t)rows * 3 * kTopkBins * sizeof(uint32_t));
  p->off_state = off;
  off += align256((size_t)rows * 8 * sizeof(uint32_t));
  p->off_cnt = off;
  off += align256((size_t)rows * p->nslices * 2 * sizeof(uint32_t));
  p->bytes = off;
}

inline size_t topk_ws_bytes(int rows, int n) {
  if (n <= kTopkResident) return 256;
  TkPlan p;
  topk_make_plan(rows, n, &p);
  return p.bytes;
}

// kvc_scissor_refill: the fraction [B*Hkv*C] f32, then the top-k's workspace.
inline size_t scissor_refill_ws_bytes(int B, int Hkv, int C, size_t* off_topk) {
  *off_topk = align256((size_t)B * Hkv * C * sizeof(float));
  return *off_topk + topk_ws_bytes(B * Hkv, C);
}

}  // namespace kvc
