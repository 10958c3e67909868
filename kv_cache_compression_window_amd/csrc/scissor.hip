// Scissorhands low-attention history: record one decode step, bulk eviction (gfx950).
//
// Source: "Implement Scissorhands KV-cache compression & SnapKV prompt
// compression" (cold-compress PR 11).  The cache.py hunks mark a slot low when
// its attention is below that of uniform attention over the cache, and keep the
// indicators of a circular window of recent steps.  The PR description ranks
// each head's tokens by the share of their observed steps with low attention
// and evicts the largest (bulk eviction leaves holes); the review thread counts
// a token's share over the steps on which it was observed.
//
// The history is kept as bit-planes (one plane per circular slot, one bit per
// cache slot) plus a running count per slot.  A step reads and writes one plane
// and the counts instead of a [slots x history] integer tensor.
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {

namespace {

constexpr int NTH = 256;

// Low-attention fraction of one slot: its low count over its own observations,
// the recordings since its token arrived (since = recordings made before it),
// at most hist_len of them; 0 without an observation.  n_rec is the number of
// recordings made so far.  Correctly rounded, so equal ratios give equal floats.
__device__ inline float slot_fraction(int cnt, long long n_rec, long long since, int hist_len) {
  long long obs = n_rec - since;
  if (obs > hist_len) obs = hist_len;
  return obs > 0 ? (float)((double)cnt / (double)obs) : 0.0f;
}

__global__ __launch_bounds__(NTH) void scissor_record_kernel(int C, int W, int BHkv, int plane, long long n_rec,
                                                              int hist_len, const float* __restrict__ probs,
                                                              const uint8_t* __restrict__ valid,
                                                              uint32_t* __restrict__ hist,
                                                              uint16_t* __restrict__ counts,
                                                              const int64_t* __restrict__ since,
                                                              float* __restrict__ frac_out) {
  __shared__ int red[NTH / 64];
  const size_t bg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint8_t* vrow = valid + bg * C;

  // S_t: number of valid slots of this (b, g)
  int cnt = 0;
  for (int c = tid; c < C; c += NTH) cnt += vrow[c] != 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  if (lane == 0) red[wave] = cnt;
  __syncthreads();
  int S_t = 0;
#pragma unroll
  for (int wv = 0; wv < NTH / 64; ++wv) S_t += red[wv];
  const double uniform = S_t > 0 ? 1.0 / (double)S_t : 0.0;

  uint32_t* prow = hist + ((size_t)plane * BHkv + bg) * W;
  for (int c0 = 0; c0 < C; c0 += NTH) {
    const int c = c0 + tid;  // c0 is a multiple of 64, so a wave covers whole words
    const bool in = c < C;
    const bool v = in && vrow[c] != 0;
    const bool low = v && ((double)probs[bg * C + c] < uniform);
    const unsigned long long bits = __ballot(low);
    uint32_t old_bit = 0u;
    if (in) old_bit = (prow[c >> 5] >> (c & 31)) & 1u;
    if (in) {
      const int cnew = (int)counts[bg * C + c] + (int)low - (int)old_bit;
      counts[bg * C + c] = (uint16_t)cnew;
      if (frac_out)
        frac_out[bg * C + c] = v ? slot_fraction(cnew, n_rec, since ? since[bg * C + c] : 0, hist_len) : kNegInf;
    }
    // all lanes have read the old word before it is overwritten (ballot above
    // and the wave's single instruction stream order the reads first)
    __builtin_amdgcn_wave_barrier();
    if (in && (lane == 0 || lane == 32)) {
      const uint32_t word = (lane == 0) ? (uint32_t)bits : (uint32_t)(bits >> 32);
      prow[c >> 5] = word;
    }
  }
}

// Number of nonzero bytes of a 16-byte unit.
__device__ inline int nonzero_bytes(const uint4& u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  int n = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) n += ((w[i] >> (8 * k)) & 0xFFu) != 0u;
  return n;
}

// The same step when C is a multiple of 32 and the rows are 16-byte aligned:
// thread t owns the 32-slot words t, t + NTH, ... of its (b, g) row, loads the
// validity, probabilities, counts and old history word of a word with
// independent 16-byte loads, and writes the new word itself.
__global__ __launch_bounds__(NTH) void scissor_record_words_kernel(int C, int W, int BHkv, int plane,
                                                                    long long n_rec, int hist_len,
                                                                    const float* __restrict__ probs,
                                                                    const uint8_t* __restrict__ valid,
                                                                    uint32_t* __restrict__ hist,
                                                                    uint16_t* __restrict__ counts,
                                                                    const int64_t* __restrict__ since,
                                                                    float* __restrict__ frac_out) {
  __shared__ int red[NTH / 64];
  const size_t bg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint4* v4 = reinterpret_cast<const uint4*>(valid + bg * C);

  int cnt = 0;
  for (int wd = tid; wd < W; wd += NTH) cnt += nonzero_bytes(v4[2 * wd]) + nonzero_bytes(v4[2 * wd + 1]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  if (lane == 0) red[wave] = cnt;
  __syncthreads();
  int S_t = 0;
#pragma unroll
  for (int wv = 0; wv < NTH / 64; ++wv) S_t += red[wv];
  const double uniform = S_t > 0 ? 1.0 / (double)S_t : 0.0;

  uint32_t* prow = hist + ((size_t)plane * BHkv + bg) * W;
  const float4* p4 = reinterpret_cast<const float4*>(probs + bg * C);
  uint4* c4 = reinterpret_cast<uint4*>(counts + bg * C);
  float4* f4 = frac_out ? reinterpret_cast<float4*>(frac_out + bg * C) : nullptr;
  for (int wd = tid; wd < W; wd += NTH) {
    const uint4 va = v4[2 * wd], vb = v4[2 * wd + 1];
    float4 pr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pr[i] = p4[8 * wd + i];
    uint4 cn[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cn[i] = c4[4 * wd + i];
    const uint32_t old = prow[wd];
    const uint32_t vw[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
    uint32_t word = 0u;
    uint32_t cw[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      cw[4 * i] = cn[i].x;
      cw[4 * i + 1] = cn[i].y;
      cw[4 * i + 2] = cn[i].z;
      cw[4 * i + 3] = cn[i].w;
    }
    float fr[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const bool v = ((vw[j >> 2] >> (8 * (j & 3))) & 0xFFu) != 0u;
      const float pj = (j & 3) == 0 ? pr[j >> 2].x : (j & 3) == 1 ? pr[j >> 2].y : (j & 3) == 2 ? pr[j >> 2].z
                                                                                              : pr[j >> 2].w;
      const bool low = v && ((double)pj < uniform);
      word |= (uint32_t)low << j;
      const uint32_t sh = 16 * (j & 1);
      const int cold = (int)((cw[j >> 1] >> sh) & 0xFFFFu);
      const int cnew = cold + (int)low - (int)((old >> j) & 1u);
      cw[j >> 1] = (cw[j >> 1] & ~(0xFFFFu << sh)) | ((uint32_t)cnew << sh);
      if (f4) fr[j] = v ? slot_fraction(cnew, n_rec, since ? since[bg * C + 32 * wd + j] : 0, hist_len) : kNegInf;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) c4[4 * wd + i] = make_uint4(cw[4 * i], cw[4 * i + 1], cw[4 * i + 2], cw[4 * i + 3]);
    prow[wd] = word;
    if (f4) {
#pragma unroll
      for (int i = 0; i < 8; ++i) f4[8 * wd + i] = make_float4(fr[4 * i], fr[4 * i + 1], fr[4 * i + 2], fr[4 * i + 3]);
    }
  }
}

__global__ void scissor_evict_kernel(int C, int n_evict, const int32_t* __restrict__ evict_idx,
                                     uint8_t* __restrict__ valid) {
  const size_t bg = blockIdx.x;
  for (int e = threadIdx.x; e < n_evict; e += blockDim.x) {
    const int c = evict_idx[bg * n_evict + e];
    if (c >= 0 && c < C) valid[bg * C + c] = 0;  // out-of-range indices are ignored
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The fraction from the current counts, without a record (sampled recording:
// an eviction step need not be a recording step; the eviction queue's refill):
// the slot's fraction at valid slots, -inf at holes and at the first n_protect
// slots of every row, as the record kernels write it.
__global__ __launch_bounds__(NTH) void scissor_frac_kernel(long long total, int C, long long n_rec, int hist_len,
                                                            int n_protect, const uint8_t* __restrict__ valid,
                                                            const uint16_t* __restrict__ counts,
                                                            const int64_t* __restrict__ since,
                                                            float* __restrict__ frac_out) {
  for (long long i = (long long)blockIdx.x * NTH + threadIdx.x; i < total; i += (long long)gridDim.x * NTH)
    frac_out[i] = (valid[i] && (int)(i % C) >= n_protect)
                      ? slot_fraction(counts[i], n_rec, since ? since[i] : 0, hist_len)
                      : kNegInf;
}

// A new token into one slot per (b, g) (Scissorhands with insertion): its K and
// V rows, valid, a zero count, a cleared bit in every history plane, and `rec`
// (the recordings made before it) as the start of its observations.  The slot
// is queue[bg*m + j], or fill_pos for every row without a queue; a slot outside
// [0, C) is skipped.
__global__ __launch_bounds__(NTH) void scissor_insert_kernel(int C, int W, int BHkv, int hist_len, int units,
                                                              const int32_t* __restrict__ queue, int m, int j,
                                                              int fill_pos, const uint4* __restrict__ k_new,
                                                              const uint4* __restrict__ v_new,
                                                              uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                                              uint8_t* __restrict__ valid, uint32_t* __restrict__ hist,
                                                              uint16_t* __restrict__ counts, long long rec,
                                                              int64_t* __restrict__ since) {
  const size_t bg = blockIdx.x;
  const int tid = threadIdx.x;
  const int slot = queue ? queue[bg * m + j] : fill_pos;
  if (slot < 0 || slot >= C) return;
  for (int u = tid; u < units; u += NTH) {
    k_cache[(bg * C + slot) * units + u] = k_new[bg * units + u];
    if (v_new) v_cache[(bg * C + slot) * units + u] = v_new[bg * units + u];
  }
  const uint32_t keep = ~(1u << (slot & 31));
  for (int p = tid; p < hist_len; p += NTH) hist[((size_t)p * BHkv + bg) * W + (slot >> 5)] &= keep;
  if (tid == 0) {
    valid[bg * C + slot] = 1;
    counts[bg * C + slot] = 0;
    since[bg * C + slot] = rec;
  }
}

}  // namespace

hipError_t launch_scissor(const ScissorArgs& a, hipStream_t st) {
  const int BHkv = a.B * a.Hkv;
  const int W = (a.C + 31) / 32;
  const long long n_rec = a.step + 1;  // recordings made, the one at `step` included
  if (a.probs) {
    const int plane = (int)(a.step % a.hist_len);
    const bool words = a.C % 32 == 0 && aligned16(a.probs) && aligned16(a.valid) && aligned16(a.counts) &&
                       (!a.frac_out || aligned16(a.frac_out));
    if (words)
      scissor_record_words_kernel<<<BHkv, NTH, 0, st>>>(a.C, W, BHkv, plane, n_rec, a.hist_len, a.probs, a.valid,
                                                        a.hist, a.counts, a.since, a.frac_out);
    else
      scissor_record_kernel<<<BHkv, NTH, 0, st>>>(a.C, W, BHkv, plane, n_rec, a.hist_len, a.probs, a.valid, a.hist,
                                                  a.counts, a.since, a.frac_out);
  } else if (a.frac_out) {
    const long long total = (long long)BHkv * a.C;
    const long long blocks = (total + NTH - 1) / NTH;
    scissor_frac_kernel<<<(unsigned)(blocks < 4096 ? blocks : 4096), NTH, 0, st>>>(
        total, a.C, n_rec, a.hist_len, 0, a.valid, a.counts, a.since, a.frac_out);
  }
  if (a.evict_idx && a.n_evict > 0) scissor_evict_kernel<<<BHkv, 256, 0, st>>>(a.C, a.n_evict, a.evict_idx, a.valid);
  return hipGetLastError();
}

hipError_t launch_scissor_refill(const ScissorRefillArgs& a, hipStream_t st) {
  const long long total = (long long)a.B * a.Hkv * a.C;
  const long long blocks = (total + NTH - 1) / NTH;
  scissor_frac_kernel<<<(unsigned)(blocks < 4096 ? blocks : 4096), NTH, 0, st>>>(
      total, a.C, a.step + 1, a.hist_len, a.n_protect, a.valid, a.counts, a.since, a.frac);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk(a.frac, a.B * a.Hkv, a.C, a.m, 0, a.queue, a.topk_ws, st);
}

hipError_t launch_scissor_insert(const ScissorInsertArgs& a, hipStream_t st) {
  const int BHkv = a.B * a.Hkv;
  scissor_insert_kernel<<<BHkv, NTH, 0, st>>>(a.C, (a.C + 31) / 32, BHkv, a.hist_len, a.row_bytes / 16, a.queue, a.m,
                                              a.j, a.fill_pos, static_cast<const uint4*>(a.k_new),
                                              static_cast<const uint4*>(a.v_new), static_cast<uint4*>(a.k_cache),
                                              static_cast<uint4*>(a.v_cache), a.valid, a.hist, a.counts, a.rec,
                                              a.since);
  return hipGetLastError();
}

}  // namespace kvc
