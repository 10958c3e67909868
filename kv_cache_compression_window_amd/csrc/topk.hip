// Per-row top-k with a forced tail, kept indices in ascending order (gfx950).
//
// One workgroup per row.  Selection is a 4-digit (8-bit) MSB-first radix select
// on order-preserving uint32 keys of the scores.  It finds the exact threshold key
// T and how many keys equal to T must be taken.  A compaction pass in index order
// then emits every key above T and the lowest-indexed keys equal to T, in
// ascending position order.  That realises the lowest-index tie rule and the
// ascending output with one deterministic pass.  Rows of up to kLdsKeys eligible
// entries are cached in LDS as keys; longer rows are re-read from global memory
// (L2) at every pass.
//
// Sources: "Implement Scissorhands KV-cache compression & SnapKV prompt
// compression" (cold-compress PR 11), PR description: SnapKV keeps the
// observation window and compresses the prefix by its scores; Scissorhands evicts
// the tokens with the highest low-attention fraction.  "Add ThinK_Press"
// (kvpress PR 18): prune the least important channels.
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {

namespace {

constexpr int NTH = 1024;             // threads per row
constexpr int kLdsKeys = 32768;       // eligible entries cached in LDS
constexpr int NWAVE = NTH / 64;

// Exclusive scan of one uint32 per thread over the workgroup (fixed order).
__device__ inline uint32_t block_exclusive_scan(uint32_t x, uint32_t* sh_wave, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sh_wave[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint32_t w = (lane < NWAVE) ? sh_wave[lane] : 0u;
    uint32_t wi = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(wi, o);
      if (lane >= o) wi += y;
    }
    if (lane < NWAVE) sh_wave[lane] = wi - w;  // exclusive prefix of the waves
    if (lane == NWAVE - 1) *total = wi;
  }
  __syncthreads();
  const uint32_t r = sh_wave[wave] + incl - x;
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(NTH) void topk_kernel(const float* __restrict__ scores, int n, int k, int n_tail,
                                                    int32_t* __restrict__ idx) {
  __shared__ uint32_t keys[kLdsKeys];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_wave[NWAVE];
  __shared__ uint32_t sh_total;
  __shared__ uint32_t sh_bucket, sh_krem;

  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;
  const float* s = scores + row * (size_t)n;
  int32_t* out = idx + row * (size_t)k;
  const int E = n - n_tail;   // eligible positions
  const int kp = k - n_tail;  // slots they compete for

  for (int i = tid; i < n_tail; i += NTH) out[kp + i] = E + i;
  if (kp <= 0) return;
  if (kp >= E) {
    for (int i = tid; i < E; i += NTH) out[i] = i;
    return;
  }

  const bool cached = E <= kLdsKeys;
  if (cached)
    for (int i = tid; i < E; i += NTH) keys[i] = float_key(s[i]);
  auto key_at = [&](int i) -> uint32_t { return cached ? keys[i] : float_key(s[i]); };

  uint32_t prefix = 0u, mask = 0u;
  uint32_t krem = (uint32_t)kp;  // still to take among keys matching the prefix
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int i0 = 0; i0 < E; i0 += NTH) {
      const int i = i0 + tid;
      uint32_t u = 0u;
      bool active = false;
      if (i < E) {
        u = key_at(i);
        active = (u & mask) == prefix;
      }
      const uint32_t bkt = (u >> shift) & 255u;
      // Scores of one row often share their leading key bits, which would make
      // the lanes of a wave collide on one counter.  The first two distinct
      // buckets of the wave are therefore added once each by a leader lane;
      // the rest use one atomic per lane.
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const unsigned long long pend = __ballot(active);
        if (pend == 0ull) break;
        const int leader = __ffsll((long long)pend) - 1;
        const uint32_t lb = __shfl(bkt, leader);
        const unsigned long long same = __ballot(active && bkt == lb);
        if ((threadIdx.x & 63) == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(same));
        if (bkt == lb) active = false;
      }
      if (active) atomicAdd(&hist[bkt], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns buckets 255-4l .. 252-4l (descending)
      const int lane = tid;
      uint32_t c[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = hist[255 - 4 * lane - q];
      const uint32_t local = c[0] + c[1] + c[2] + c[3];
      uint32_t incl = local;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      const uint32_t excl = incl - local;
      const unsigned long long hit = __ballot(incl >= krem);
      const int first = __ffsll(hit) - 1;  // lowest lane whose suffix count reaches krem
      if (lane == first) {
        uint32_t cum = excl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (cum + c[q] >= krem) {
            sh_bucket = 255u - 4u * lane - q;
            sh_krem = krem - cum;
            break;
          }
          cum += c[q];
        }
      }
    }
    __syncthreads();
    prefix |= sh_bucket << shift;
    mask |= 255u << shift;
    krem = sh_krem;
    __syncthreads();
  }
  const uint32_t T = prefix;  // exact key of the kp-th largest
  const uint32_t take_eq = krem;  // keys equal to T to take, lowest index first

  // ordered compaction: thread tid owns the contiguous segment [j0, j1)
  // an odd segment length keeps the threads' LDS reads on distinct banks
  const int seg = ((E + NTH - 1) / NTH) | 1;
  const int j0 = min(E, tid * seg), j1 = min(E, j0 + seg);
  uint32_t n_gt = 0, n_eq = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t u = key_at(j);
    n_gt += u > T;
    n_eq += u == T;
  }
  const uint32_t eq_before = block_exclusive_scan(n_eq, sh_wave, &sh_total);
  const uint32_t my_eq = (eq_before >= take_eq) ? 0u : min(n_eq, take_eq - eq_before);
  const uint32_t pos0 = block_exclusive_scan(n_gt + my_eq, sh_wave, &sh_total);
  uint32_t pos = pos0, eq_taken = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t u = key_at(j);
    if (u > T || (u == T && eq_taken < my_eq)) {
      if (pos < (uint32_t)kp) out[pos] = j;  // kp is exact; the guard only keeps writes in the row
      ++pos;
      eq_taken += (u == T);
    }
  }
}

}  // namespace

hipError_t launch_topk(const float* scores, int rows, int n, int k, int n_tail, int32_t* idx, hipStream_t st) {
  topk_kernel<<<rows, NTH, 0, st>>>(scores, n, k, n_tail, idx);
  return hipGetLastError();
}

}  // namespace kvc
