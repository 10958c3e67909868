// Host-only driver of the C-ABI validation paths, built with AddressSanitizer
// and UndefinedBehaviorSanitizer (tests/test_abi_sanitize.py).  Every call here
// must be rejected (or answered as a workspace-size query) before any launch;
// the launchers of this build abort.
#include <cstdint>
#include <cstdio>

#include "kvc.h"

static int failures = 0;

static void expect(const char* what, kvc_status got, kvc_status want) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d\n", what, (int)got, (int)want);
    ++failures;
  }
}

int main() {
  void* fake = reinterpret_cast<void*>(0x100000);   // 16-byte aligned, never dereferenced
  void* odd = reinterpret_cast<void*>(0x100008);    // 8-byte aligned only
  void* odd2 = reinterpret_cast<void*>(0x100002);   // 2-byte aligned only
  size_t big = size_t(1) << 40, small = 16, q = 0;

  // status strings and the version
  for (int s = 0; s <= 8; ++s)
    if (!kvc_status_string(static_cast<kvc_status>(s))) ++failures;
  if (kvc_abi_version() != KVC_ABI_VERSION) ++failures;

  // window scores
  kvc_shape ok = {1, 32, 8, 4096, 128, 64};
  auto ws = [&](const kvc_shape* sh, int dt, const void* qp, const void* k, int reduce, void* w, size_t* n) {
    return kvc_window_scores(sh, static_cast<kvc_dtype>(dt), qp, k, nullptr, nullptr, 0,
                             static_cast<kvc_reduce>(reduce), 1, static_cast<float*>(fake), w, n, nullptr);
  };
  expect("ws null shape", ws(nullptr, 1, fake, fake, 0, fake, &big), KVC_ERR_NULL);
  expect("ws dtype", ws(&ok, 5, fake, fake, 0, fake, &big), KVC_ERR_DTYPE);
  expect("ws reduce", ws(&ok, 1, fake, fake, 2, fake, &big), KVC_ERR_DTYPE);
  kvc_shape bad_h = {1, 30, 8, 4096, 128, 64}, bad_w = {1, 32, 8, 63, 128, 64}, bad_d = {1, 32, 8, 4096, 96, 64};
  kvc_shape big_rows = {1, 64, 8, 4096, 128, 256}, overflow = {4096, 1024, 1024, 4096, 128, 64};
  expect("ws H % Hkv", ws(&bad_h, 1, fake, fake, 0, fake, &big), KVC_ERR_SHAPE);
  expect("ws w > S", ws(&bad_w, 1, fake, fake, 0, fake, &big), KVC_ERR_SHAPE);
  expect("ws D", ws(&bad_d, 1, fake, fake, 0, fake, &big), KVC_ERR_UNSUPPORTED);
  expect("ws rows", ws(&big_rows, 1, fake, fake, 0, fake, &big), KVC_ERR_UNSUPPORTED);
  expect("ws merge overflow", ws(&overflow, 1, fake, fake, 0, fake, &big), KVC_ERR_UNSUPPORTED);
  kvc_shape long_rows = {1, 32, 8, (1 << 30) + 1, 128, 64};
  expect("ws S > 2^30", ws(&long_rows, 1, fake, fake, 0, fake, &big), KVC_ERR_UNSUPPORTED);
  expect("ws size query", ws(&ok, 1, nullptr, nullptr, 0, nullptr, &q), KVC_OK);
  if (q == 0) ++failures;
  expect("ws small workspace", ws(&ok, 1, fake, fake, 0, fake, &small), KVC_ERR_WORKSPACE);
  expect("ws null q", ws(&ok, 1, nullptr, fake, 0, fake, &big), KVC_ERR_NULL);
  expect("ws misaligned k", ws(&ok, 1, fake, odd, 0, fake, &big), KVC_ERR_ALIGN);
  auto wsx = [&](int conc, void* w, size_t* n) {
    return kvc_window_scores_ex(&ok, KVC_BF16, fake, fake, nullptr, nullptr, 0, KVC_REDUCE_GROUP, 1, conc,
                                static_cast<float*>(fake), w, n, nullptr);
  };
  expect("ws_ex budget < 0", wsx(-1, fake, &big), KVC_ERR_SHAPE);
  expect("ws_ex budget > 256", wsx(257, fake, &big), KVC_ERR_SHAPE);
  expect("ws_ex size query", wsx(128, nullptr, &q), KVC_OK);
  expect("ws_ex small workspace", wsx(64, fake, &small), KVC_ERR_WORKSPACE);
  expect("ws noalloc overflow",
         kvc_window_scores_noalloc(&(const kvc_shape&)kvc_shape{64, 32, 8, 8192, 128, 1}, KVC_BF16, fake, fake,
                                   nullptr, nullptr, 0, KVC_REDUCE_GROUP, 0, static_cast<float*>(fake), nullptr),
         KVC_ERR_WORKSPACE);
  expect("ws noalloc misaligned", kvc_window_scores_noalloc(&ok, KVC_BF16, odd, fake, nullptr, nullptr, 0,
                                                            KVC_REDUCE_GROUP, 1, static_cast<float*>(fake), nullptr),
         KVC_ERR_ALIGN);

  // Scissorhands
  auto up = [&](int B, int hist, int64_t step, const float* probs, uint32_t* hist_p, uint16_t* counts,
                const int64_t* since, float* frac) {
    return kvc_scissor_update(B, 8, 4096, hist, step, probs, static_cast<uint8_t*>(fake), hist_p, counts, since, frac,
                              nullptr, 0, nullptr);
  };
  auto F = static_cast<float*>(fake);
  auto H = static_cast<uint32_t*>(fake);
  auto C = static_cast<uint16_t*>(fake);
  expect("scissor B", up(0, 400, 0, F, H, C, nullptr, nullptr), KVC_ERR_SHAPE);
  expect("scissor hist", up(8, 70000, 0, F, H, C, nullptr, nullptr), KVC_ERR_SHAPE);
  expect("scissor step", up(8, 400, -1, F, H, C, nullptr, nullptr), KVC_ERR_SHAPE);
  expect("scissor null hist", up(8, 400, 0, F, nullptr, C, nullptr, nullptr), KVC_ERR_NULL);
  expect("scissor misaligned probs", up(8, 400, 0, static_cast<float*>(odd2), H, C, nullptr, nullptr), KVC_ERR_ALIGN);
  expect("scissor misaligned since",
         up(8, 400, 3, nullptr, nullptr, C, reinterpret_cast<int64_t*>(0x100004), F), KVC_ERR_ALIGN);
  expect("scissor nothing to do", up(8, 400, 0, nullptr, nullptr, nullptr, nullptr, nullptr), KVC_OK);
  expect("refill size query",
         kvc_scissor_refill(8, 8, 4096, 400, 10, nullptr, nullptr, nullptr, 100, 64, nullptr, nullptr, &q, nullptr),
         KVC_OK);
  expect("refill protect all",
         kvc_scissor_refill(8, 8, 4096, 400, 10, static_cast<uint8_t*>(fake), C, nullptr, 4096, 1,
                            static_cast<int32_t*>(fake), fake, &big, nullptr),
         KVC_ERR_SHAPE);
  expect("insert rec",
         kvc_scissor_insert(8, 8, 4096, 128, 400, KVC_BF16, static_cast<int32_t*>(fake), 64, 3, 0, -1, fake, fake,
                            fake, fake, static_cast<uint8_t*>(fake), H, C, static_cast<int64_t*>(fake), nullptr),
         KVC_ERR_SHAPE);
  expect("insert null since",
         kvc_scissor_insert(8, 8, 4096, 128, 400, KVC_BF16, static_cast<int32_t*>(fake), 64, 3, 0, 7, fake, fake,
                            fake, fake, static_cast<uint8_t*>(fake), H, C, nullptr, nullptr),
         KVC_ERR_NULL);

  // channel scores, top-k, gathers
  expect("channel size query", kvc_channel_scores(&ok, KVC_BF16, nullptr, nullptr, nullptr, nullptr, &q, nullptr),
         KVC_OK);
  expect("channel misaligned", kvc_channel_scores(&ok, KVC_BF16, odd, fake, F, fake, &big, nullptr), KVC_ERR_ALIGN);
  expect("topk k > n", kvc_topk_select(F, 8, 100, 101, 0, static_cast<int32_t*>(fake), fake, &big, nullptr),
         KVC_ERR_SHAPE);
  expect("topk size query", kvc_topk_select(nullptr, 8, 100000, 10, 0, nullptr, nullptr, &q, nullptr), KVC_OK);
  expect("topk k = 0", kvc_topk_select(F, 8, 100, 0, 0, static_cast<int32_t*>(fake), fake, &big, nullptr), KVC_OK);
  expect("gather n_keep", kvc_gather_compact(&ok, KVC_BF16, fake, fake, static_cast<int32_t*>(fake), 5000, nullptr,
                                             0, fake, fake, nullptr),
         KVC_ERR_SHAPE);
  expect("gather misaligned", kvc_gather_compact(&ok, KVC_BF16, odd, fake, static_cast<int32_t*>(fake), 64, nullptr,
                                                 0, fake, fake, nullptr),
         KVC_ERR_ALIGN);
  expect("compress d_keep", kvc_gather_compress(&ok, KVC_BF16, fake, nullptr, static_cast<int32_t*>(fake), 64,
                                                static_cast<int32_t*>(fake), 0, fake, nullptr, nullptr),
         KVC_ERR_SHAPE);
  expect("expand D", kvc_channel_expand(1, 8, 10, 96, KVC_BF16, fake, static_cast<int32_t*>(fake), 64, fake, nullptr),
         KVC_ERR_UNSUPPORTED);
  expect("query channels H % Hkv", kvc_query_channels(1, 30, 8, 64, 128, KVC_BF16, fake,
                                                      static_cast<int32_t*>(fake), 64, fake, nullptr),
         KVC_ERR_SHAPE);

  if (failures) {
    std::printf("%d checks failed\n", failures);
    return 1;
  }
  std::printf("all checks passed\n");
  return 0;
}
