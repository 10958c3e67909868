// Per-row top-k with a forced tail, kept indices in ascending order (gfx950).
//
// One workgroup of 1024 threads per row.  Scores become order-preserving uint32
// keys.  For the compaction thread t holds the keys of the KPT consecutive
// positions t*KPT .. t*KPT+KPT-1 of a tile of 1024*KPT positions, so that its
// kept positions come out in order; keys are loaded in coalesced order and
// handed to their owners through LDS.  Rows that fit one tile keep their keys in
// registers for the whole selection; longer rows (KPT = 32) are processed tile
// by tile and re-read from L2 at every sweep, in coalesced order for the
// histogram passes (which take any order).  Slots past the end of the row hold the row's minimum
// key: they sit after every real position, so the lowest-index tie rule never
// takes them, and the hot loops need no bounds test.
//
// Selection is an MSB-first radix select on  rel = key - min_key .  Digits of up
// to 11 bits are taken from bit L-1 of the key range downwards, so the first
// histogram already spreads the keys over the range they occupy (scores of one
// row usually share their leading key bits).  The first pass's histogram lives
// in LDS in two interleaved copies picked by lane, so lanes of one wave that fall
// into one bin spread over two counters; the later passes count few keys into
// one copy.  The passes yield the exact rel T of the kp-th
// largest eligible score and the number of keys equal to T that must be taken.
// The compaction then keeps every key above T and the lowest-indexed keys equal
// to T: a thread's first output slot is the exclusive scan, over the threads,
// of its counts of keys > T and == T (one scan of both counts packed into
// 16-bit halves), and it walks its own positions in order from there.  When
// every key equal to T is taken (the usual case) one count of keys >= T is
// enough.
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

constexpr int NTH = 1024;  // threads per row
constexpr int NWAVE = NTH / 64;
constexpr int DBITS = 11;  // digit width
constexpr int NBIN = 1 << DBITS;
constexpr int NCOPY = 2;   // interleaved copies of the first pass's histogram
constexpr int kSplitCopies = 8;  // interleaved copies of the sliced kernels' histograms

static_assert(NBIN == 2 * NTH, "each thread owns two bins when the threshold bin is searched");

// Padded LDS index used to hand keys loaded in coalesced order (thread t takes
// positions t, t+1024, ...) to the thread that owns them (t*KPT .. t*KPT+KPT-1):
// one spare word per 32 keeps both the writes and the reads free of bank
// conflicts.
__device__ inline int xpose_idx(int p) { return p + (p >> 5); }
constexpr int kXposeWords = 33 * NTH;  // padded size of a 32-key-per-thread tile

// The first pass's histogram has LDS of its own, so it is cleared while the keys
// are loaded.  The hand-over area is free once the keys are in registers: the
// later passes, which count few keys, have one-copy histograms at its end
// (cleared after the first pass's counting), and the second pass lists the keys
// it counts (those in the first pass's threshold bin) at its start; the third
// pass reads that list instead of every key of the row.
struct TopkShared {
  uint32_t xpose[kXposeWords];
  alignas(16) uint32_t hist[NBIN * NCOPY];
  alignas(16) uint32_t wave_tot[NWAVE];
  alignas(16) uint32_t list_tot[NWAVE];
  uint32_t red_min[NWAVE], red_max[NWAVE];
  uint32_t bucket, krem, bcount;
};

constexpr int kNarrowHist0 = kXposeWords - 2 * NBIN;  // second pass; the third at + NBIN
constexpr int kListCap = kNarrowHist0;
static_assert(kListCap > 4 * NTH, "room for the candidate list");
static_assert(NBIN * NCOPY == 4 * NTH && 2 * NBIN == 4 * NTH, "one 16-byte clear per thread per histogram set");

// Inclusive prefix sum over the 64 lanes of a wave: DPP shifts within rows of
// 16 lanes, then the broadcasts of lane 15 and lane 31 into the later rows.
__device__ inline uint32_t wave_inclusive_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

__device__ inline uint32_t wave_min(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, (uint32_t)__shfl_xor(x, o));
  return x;
}

__device__ inline uint32_t wave_max(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, (uint32_t)__shfl_xor(x, o));
  return x;
}

// Sum of the per-wave totals (already in LDS) of the waves before `wave`.
__device__ inline uint32_t waves_before(const uint32_t* tot, int wave) {
  const uint4* wt = reinterpret_cast<const uint4*>(tot);
  uint32_t before = 0u;
#pragma unroll
  for (int q = 0; q < NWAVE / 4; ++q) {
    const uint4 x = wt[q];
    before += (4 * q < wave ? x.x : 0u) + (4 * q + 1 < wave ? x.y : 0u) + (4 * q + 2 < wave ? x.z : 0u) +
              (4 * q + 3 < wave ? x.w : 0u);
  }
  return before;
}

// Exclusive scan of one value per thread over the workgroup, in thread order,
// and the workgroup total.  The LDS it uses is free again when it returns.
__device__ inline uint32_t block_exclusive_scan(TopkShared& sh, uint32_t x, int lane, int wave, uint32_t* total) {
  const uint32_t winc = wave_inclusive_scan(x);
  if (lane == 63) sh.wave_tot[wave] = winc;
  __syncthreads();
  const uint32_t r = waves_before(sh.wave_tot, wave) + winc - x;
  *total = waves_before(sh.wave_tot, NWAVE);
  __syncthreads();
  return r;
}

// After a histogram pass: the bin where the count of keys, summed from the top
// bin down, reaches krem.  Thread t owns bins 2047-2t and 2046-2t, so a scan in
// thread order is a suffix sum over the bins and exactly one thread sees it
// cross krem.  Leaves the bin, the rank still to take inside it and the bin's
// count in sh.bucket, sh.krem and sh.bcount.
// `wide`: the histogram has NCOPY interleaved copies per bin (the first pass);
// otherwise one counter per bin in the first NBIN words (the later passes, which
// count few keys).
__device__ inline void find_bin(TopkShared& sh, const uint32_t* hist, uint32_t krem, int tid, int lane, int wave,
                                bool wide) {
  const int b_hi = NBIN - 1 - 2 * tid, b_lo = b_hi - 1;
  uint32_t c_hi, c_lo;
  if (wide) {
    static_assert(NCOPY == 2, "two copies of bins b_lo (even) and b_hi in one 16-byte word");
    const uint4 h = reinterpret_cast<const uint4*>(hist)[b_lo >> 1];
    c_lo = h.x + h.y;
    c_hi = h.z + h.w;
  } else {
    const uint2 h = reinterpret_cast<const uint2*>(hist)[b_lo >> 1];  // bins b_lo (even) and b_hi
    c_lo = h.x;
    c_hi = h.y;
  }
  const uint32_t local = c_hi + c_lo;
  const uint32_t winc = wave_inclusive_scan(local);
  if (lane == 63) sh.wave_tot[wave] = winc;
  __syncthreads();
  const uint32_t incl = waves_before(sh.wave_tot, wave) + winc, excl = incl - local;
  if (excl < krem && incl >= krem) {
    if (excl + c_hi >= krem) {
      sh.bucket = (uint32_t)b_hi;
      sh.krem = krem - excl;
      sh.bcount = c_hi;
    } else {
      sh.bucket = (uint32_t)b_lo;
      sh.krem = krem - excl - c_hi;
      sh.bcount = c_lo;
    }
  }
  __syncthreads();
}

template <int KPT, bool RESIDENT>
__global__ __launch_bounds__(NTH) void topk_kernel(const float* __restrict__ scores, int n, int k, int n_tail,
                                                    int32_t* __restrict__ idx) {
  constexpr int TILE = NTH * KPT;
  __shared__ TopkShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  const int ntiles = RESIDENT ? 1 : (E + TILE - 1) / TILE;
  uint32_t u[KPT];
  // Keys of tile t in coalesced order (slot i of thread t holds position
  // t*TILE + i*NTH + tid; positions past E read position E-1, a duplicate that
  // leaves the key range unchanged).  The histogram passes take any order.
  auto load_coalesced = [&](int t) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) u[i] = float_key(s[min(t * TILE + i * NTH + tid, E - 1)]);
  };
  // Keys of tile t in owner order (slot i of thread t holds position
  // t*TILE + tid*KPT + i): loaded in coalesced order and handed over through LDS.
  auto load_owned = [&](int t) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int p = j * NTH + tid;
      sh.xpose[xpose_idx(p)] = float_key(s[min(t * TILE + p, E - 1)]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i) u[i] = sh.xpose[xpose_idx(tid * KPT + i)];
    __syncthreads();
  };

  // key range of the eligible positions
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  if constexpr (RESIDENT) {
    // coalesced loads, handed over through LDS
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int p = j * NTH + tid;
      const uint32_t key = float_key(s[min(p, E - 1)]);
      kmin = min(kmin, key);
      kmax = max(kmax, key);
      sh.xpose[xpose_idx(p)] = key;
    }
  } else {
    for (int t = 0; t < ntiles; ++t) {
      load_coalesced(t);
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        kmin = min(kmin, u[i]);
        kmax = max(kmax, u[i]);
      }
    }
  }
  // one barrier for the hand-over, the key range and the first histogram's clear
  kmin = wave_min(kmin);
  kmax = wave_max(kmax);
  if (lane == 0) {
    sh.red_min[wave] = kmin;
    sh.red_max[wave] = kmax;
  }
  reinterpret_cast<uint4*>(sh.hist)[tid] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  if constexpr (RESIDENT) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) u[i] = sh.xpose[xpose_idx(tid * KPT + i)];
  }
  kmin = sh.red_min[0];
  kmax = sh.red_max[0];
#pragma unroll
  for (int v = 1; v < NWAVE; ++v) {
    kmin = min(kmin, sh.red_min[v]);
    kmax = max(kmax, sh.red_max[v]);
  }
  const uint32_t range = kmax - kmin;
  const int L = range == 0u ? 0 : 32 - __clz(range);  // bit length of every rel
  const int npass = (L + DBITS - 1) / DBITS;

  // from here on u holds rel = key - kmin (same order as the keys); slots past
  // the row hold 0, the smallest rel
  auto to_rel_owned = [&](int t) {
    const int nv = E - (t * TILE + tid * KPT);
#pragma unroll
    for (int i = 0; i < KPT; ++i) u[i] -= kmin;
    if (nv < KPT) {
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        if (i >= nv) u[i] = 0u;
    }
  };
  // tiles of the non-resident passes (coalesced order)
  auto load_rel_coalesced = [&](int t) {
    load_coalesced(t);
#pragma unroll
    for (int i = 0; i < KPT; ++i) u[i] -= kmin;
    if (t == ntiles - 1) {
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        if (t * TILE + i * NTH + tid >= E) u[i] = 0u;
    }
  };
  // tiles of the non-resident compaction (owner order)
  auto load_rel_owned = [&](int t) {
    load_owned(t);
    to_rel_owned(t);
  };
  if constexpr (RESIDENT) to_rel_owned(0);

  const int cp = lane & (NCOPY - 1);
  uint32_t prefix = 0u;                            // fixed high bits of rel(T)
  uint32_t krem = (uint32_t)kp;                    // still to take among the keys matching the prefix
  uint32_t last_count = (uint32_t)(ntiles * TILE);  // keys equal to T (all of them when npass == 0)
  uint32_t* list = sh.xpose;  // free once the keys are in registers
  bool from_list = false;
  int nlist = 0;
  for (int pass = 0; pass < npass; ++pass) {
    const int hi = L - DBITS * pass;       // bits [hi, 32) of rel are fixed
    const int shift = max(0, hi - DBITS);  // this digit is bits [shift, hi)
    const uint32_t fixed = hi >= 32 ? 0u : ~0u << hi;
    const bool wide = pass == 0;
    const bool listing = RESIDENT && pass == 1;  // the second pass lists the keys it counts
    uint32_t* hist = wide ? sh.hist : sh.xpose + kNarrowHist0 + (pass - 1) * NBIN;
    uint32_t mask = 0u;  // listing: the slots counted
    if (from_list) {
      for (int j = tid; j < nlist; j += NTH) {
        const uint32_t x = list[j];
        if ((x & fixed) == prefix) atomicAdd(&hist[(x >> shift) & (NBIN - 1)], 1u);
      }
    } else {
      for (int t = 0; t < ntiles; ++t) {
        if constexpr (!RESIDENT) load_rel_coalesced(t);
        if (wide) {
#pragma unroll
          for (int i = 0; i < KPT; ++i) atomicAdd(&hist[((u[i] >> shift) & (NBIN - 1)) * NCOPY + cp], 1u);
        } else {
#pragma unroll
          for (int i = 0; i < KPT; ++i) {
            if ((u[i] & fixed) == prefix) {
              atomicAdd(&hist[(u[i] >> shift) & (NBIN - 1)], 1u);
              mask |= 1u << i;
            }
          }
        }
      }
    }
    uint32_t cnt = 0u, winc = 0u;
    if (listing) {
      cnt = (uint32_t)__popc(mask);
      winc = wave_inclusive_scan(cnt);
      if (lane == 63) sh.list_tot[wave] = winc;
    }
    __syncthreads();
    if (wide) {
      // every thread has its keys in registers: the later passes' histograms
      // (in the hand-over area) are cleared here, visible after find_bin's barriers
      reinterpret_cast<uint4*>(sh.xpose + kNarrowHist0)[tid] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (listing) {
      const uint32_t total = waves_before(sh.list_tot, NWAVE);
      nlist = (int)total;
      from_list = total <= (uint32_t)kListCap;
      if (from_list) {
        uint32_t pos = waves_before(sh.list_tot, wave) + winc - cnt;
#pragma unroll
        for (int i = 0; i < KPT; ++i)
          if ((mask >> i) & 1u) list[pos++] = u[i];
      }
    }
    find_bin(sh, hist, krem, tid, lane, wave, wide);  // its barriers publish the clears and the list
    prefix |= sh.bucket << shift;
    krem = sh.krem;
    last_count = sh.bcount;
  }
  const uint32_t T = prefix;      // rel of the kp-th largest eligible score
  const uint32_t take_eq = krem;  // keys equal to T to take, lowest positions first
  // When T is 0 the pad slots count among the keys equal to T.  They come after
  // every real position, so they are never taken, but they keep last_count above
  // take_eq and so select the general compaction.
  const bool all_eq = last_count == take_eq;

  uint32_t gt_carry = 0u, eq_carry = 0u;  // counts of earlier tiles
  for (int t = 0; t < ntiles; ++t) {
    if constexpr (!RESIDENT) load_rel_owned(t);
    const int p0 = t * TILE + tid * KPT;
    if (all_eq) {
      uint32_t c = 0u;
#pragma unroll
      for (int i = 0; i < KPT; ++i) c += u[i] >= T;
      uint32_t tot;
      uint32_t pos = gt_carry + block_exclusive_scan(sh, c, lane, wave, &tot);
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        if (u[i] >= T) {
          if (pos < (uint32_t)kp) out[pos] = p0 + i;  // pos < kp holds; the guard keeps writes in the row
          ++pos;
        }
      }
      gt_carry += tot;
    } else {
      uint32_t c = 0u;
#pragma unroll
      for (int i = 0; i < KPT; ++i) c += (u[i] > T ? 1u : 0u) + (u[i] == T ? 0x10000u : 0u);
      uint32_t tot;
      const uint32_t ex = block_exclusive_scan(sh, c, lane, wave, &tot);
      // a tile holds at most 32768 keys, so neither 16-bit half carries
      uint32_t gt_before = gt_carry + (ex & 0xFFFFu), eq_before = eq_carry + (ex >> 16);
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const bool gt = u[i] > T, eq = u[i] == T;
        if (gt || (eq && eq_before < take_eq)) {
          const uint32_t pos = gt_before + min(eq_before, take_eq);
          if (pos < (uint32_t)kp) out[pos] = p0 + i;  // pos < kp holds; the guard keeps writes in the row
        }
        gt_before += gt;
        eq_before += eq;
      }
      gt_carry += tot & 0xFFFFu;
      eq_carry += tot >> 16;
    }
  }
}

// ---------------------------------------------------------------------------
// Rows longer than one resident tile: slices of kTopkSlice positions, one
// 256-thread workgroup each, in six launches per call:
//   zero   the three global digit histograms of every row; write the tail;
//   hist q (q = 0, 1, 2)  find the bin of digit q-1 in its global histogram
//          (so every slice knows the selected high bits), then count digit q of
//          the slice's keys that carry those bits into LDS and add the nonzero
//          bins to the row's global histogram;
//   count  find the last bin: the threshold key T and the number of keys equal
//          to T to take; count the slice's keys above and at T;
//   write  the slice's first output slot is the sum of the counts of the
//          earlier slices; its kept positions follow in order.
// The digits are fixed (key bits 31..21, 20..10, 9..0), so three passes always
// reach the exact T.  Slice 0 of each pass leaves the selection state in the
// workspace for the next launch.
// ---------------------------------------------------------------------------
constexpr int SNT = 256;
constexpr int SWAVE = SNT / 64;
constexpr int SKPT = kTopkSlice / SNT;  // keys per thread
static_assert(SKPT * SNT == kTopkSlice, "slices split evenly over the threads");
static_assert(kTopkBins == NBIN, "the widest digit has 11 bits");

__host__ __device__ constexpr int split_shift(int q) { return q == 0 ? 21 : q == 1 ? 10 : 0; }
__host__ __device__ constexpr int split_bits(int q) { return q == 2 ? 10 : 11; }

// Scan and reduction scratch of a slice workgroup.
struct SplitScan {
  uint32_t wave_tot[SWAVE];
  uint32_t bucket, krem, red[2 * SWAVE];
};

// Inclusive scan over the 256 threads in thread order.
__device__ inline uint32_t split_inclusive_scan(SplitScan& sh, uint32_t x, int lane, int wave) {
  const uint32_t winc = wave_inclusive_scan(x);
  if (lane == 63) sh.wave_tot[wave] = winc;
  __syncthreads();
  uint32_t before = 0u;
#pragma unroll
  for (int v = 0; v < SWAVE; ++v) before += v < wave ? sh.wave_tot[v] : 0u;
  __syncthreads();
  return before + winc;
}

// After digit pass q with its global histogram gh (nb bins): the bin where the
// count, summed from the top bin down, reaches krem, and the rank still to take
// inside it.  Thread t owns bins nb-1-bpt*t .. nb-bpt-bpt*t (descending), so
// the scan in thread order is the suffix sum and one thread sees it cross krem.
__device__ inline void split_find_bin(SplitScan& sh, const uint32_t* gh, int nb, uint32_t krem, int tid, int lane,
                                      int wave, uint32_t* bucket, uint32_t* krem_out) {
  const int bpt = nb / SNT;
  uint32_t c[NBIN / SNT];
  uint32_t local = 0u;
#pragma unroll
  for (int j = 0; j < NBIN / SNT; ++j) {
    c[j] = j < bpt ? gh[nb - 1 - bpt * tid - j] : 0u;
    local += c[j];
  }
  const uint32_t incl = split_inclusive_scan(sh, local, lane, wave);
  const uint32_t excl = incl - local;
  if (excl < krem && incl >= krem) {
    uint32_t acc = excl;
#pragma unroll
    for (int j = 0; j < NBIN / SNT; ++j) {
      if (j < bpt && acc < krem && acc + c[j] >= krem) {
        sh.bucket = (uint32_t)(nb - 1 - bpt * tid - j);
        sh.krem = krem - acc;
      }
      acc += c[j];
    }
  }
  __syncthreads();
  *bucket = sh.bucket;
  *krem_out = sh.krem;
  __syncthreads();
}

__global__ __launch_bounds__(SNT) void topk_split_zero_kernel(uint32_t* __restrict__ hist, int32_t* __restrict__ idx,
                                                              int k, int kp, int E, int n_tail) {
  const size_t row = blockIdx.x;
  uint4* gh = reinterpret_cast<uint4*>(hist + row * 3 * kTopkBins);
  for (int i = threadIdx.x; i < 3 * kTopkBins / 4; i += SNT) gh[i] = make_uint4(0u, 0u, 0u, 0u);
  int32_t* out = idx + row * (size_t)k;
  for (int i = threadIdx.x; i < n_tail; i += SNT) out[kp + i] = E + i;
}

template <int PASS>
__global__ __launch_bounds__(SNT) void topk_split_hist_kernel(const float* __restrict__ scores, int n, int E, int kp,
                                                              uint32_t* __restrict__ hist,
                                                              uint32_t* __restrict__ state) {
  __shared__ SplitScan sh;
  __shared__ __attribute__((aligned(16))) uint32_t lds_hist[NBIN * kSplitCopies];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t row = blockIdx.y;
  const int slice = blockIdx.x;
  const float* s = scores + row * (size_t)n;
  uint32_t* gh = hist + row * 3 * kTopkBins;
  uint32_t* st = state + row * 8;

  uint32_t prefix = 0u, krem = (uint32_t)kp;  // selected high bits, rank still to take
  if constexpr (PASS >= 1) {
    if constexpr (PASS == 2) {
      prefix = st[0];
      krem = st[1];
    }
    uint32_t b, kr;
    split_find_bin(sh, gh + (PASS - 1) * kTopkBins, 1 << split_bits(PASS - 1), krem, tid, lane, wave, &b, &kr);
    prefix |= b << split_shift(PASS - 1);
    krem = kr;
    if (slice == 0 && tid == 0) {
      st[2 * (PASS - 1)] = prefix;
      st[2 * (PASS - 1) + 1] = krem;
    }
  }
  constexpr int NB = 1 << split_bits(PASS), SHIFT = split_shift(PASS);
  constexpr uint32_t HI = PASS == 0 ? 0u : ~0u << (SHIFT + split_bits(PASS));  // bits fixed before this pass
#pragma unroll
  for (int j = 0; j < NB * kSplitCopies / 4 / SNT; ++j)
    reinterpret_cast<uint4*>(lds_hist)[j * SNT + tid] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  const int base = slice * kTopkSlice;
  const int cp = lane & (kSplitCopies - 1);
  uint32_t key[SKPT];
#pragma unroll
  for (int j = 0; j < SKPT; ++j) key[j] = float_key(s[min(base + j * SNT + tid, E - 1)]);
#pragma unroll
  for (int j = 0; j < SKPT; ++j)
    if (base + j * SNT + tid < E && (key[j] & HI) == prefix)
      atomicAdd(&lds_hist[((key[j] >> SHIFT) & (NB - 1)) * kSplitCopies + cp], 1u);
  __syncthreads();
  for (int b = tid; b < NB; b += SNT) {
    const uint4* h = reinterpret_cast<const uint4*>(&lds_hist[b * kSplitCopies]);
    const uint4 h0 = h[0], h1 = h[1];
    const uint32_t c = h0.x + h0.y + h0.z + h0.w + h1.x + h1.y + h1.z + h1.w;
    if (c) atomicAdd(&gh[PASS * kTopkBins + b], c);
  }
}

__global__ __launch_bounds__(SNT) void topk_split_count_kernel(const float* __restrict__ scores, int n, int E,
                                                               const uint32_t* __restrict__ hist,
                                                               uint32_t* __restrict__ state,
                                                               uint32_t* __restrict__ cnt, int nslices) {
  __shared__ SplitScan sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t row = blockIdx.y;
  const int slice = blockIdx.x;
  const float* s = scores + row * (size_t)n;
  uint32_t* st = state + row * 8;
  uint32_t b, take_eq;
  split_find_bin(sh, hist + row * 3 * kTopkBins + 2 * kTopkBins, 1 << split_bits(2), st[3], tid, lane, wave, &b,
                 &take_eq);
  const uint32_t T = st[2] | b;  // key of the kp-th largest eligible score
  if (slice == 0 && tid == 0) {
    st[4] = T;
    st[5] = take_eq;
  }
  const int base = slice * kTopkSlice;
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int j = 0; j < SKPT; ++j) {
    const int p = base + j * SNT + tid;
    const uint32_t key = float_key(s[min(p, E - 1)]);
    gt += (p < E && key > T) ? 1u : 0u;
    eq += (p < E && key == T) ? 1u : 0u;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    gt += (uint32_t)__shfl_xor(gt, o);
    eq += (uint32_t)__shfl_xor(eq, o);
  }
  if (lane == 0) {
    sh.red[2 * wave] = gt;
    sh.red[2 * wave + 1] = eq;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t g = 0u, e = 0u;
#pragma unroll
    for (int v = 0; v < SWAVE; ++v) {
      g += sh.red[2 * v];
      e += sh.red[2 * v + 1];
    }
    cnt[(row * nslices + slice) * 2] = g;
    cnt[(row * nslices + slice) * 2 + 1] = e;
  }
}

__global__ __launch_bounds__(SNT) void topk_split_write_kernel(const float* __restrict__ scores, int n, int E, int k,
                                                               int kp, const uint32_t* __restrict__ state,
                                                               const uint32_t* __restrict__ cnt, int nslices,
                                                               int32_t* __restrict__ idx) {
  __shared__ SplitScan sh;
  __shared__ uint32_t lds_xpose[kTopkSlice + kTopkSlice / 32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t row = blockIdx.y;
  const int slice = blockIdx.x;
  const float* s = scores + row * (size_t)n;
  int32_t* out = idx + row * (size_t)k;
  const uint32_t T = state[row * 8 + 4], take_eq = state[row * 8 + 5];

  // counts of the earlier slices
  uint32_t gt_b = 0u, eq_b = 0u;
  for (int i = tid; i < slice; i += SNT) {
    gt_b += cnt[(row * nslices + i) * 2];
    eq_b += cnt[(row * nslices + i) * 2 + 1];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    gt_b += (uint32_t)__shfl_xor(gt_b, o);
    eq_b += (uint32_t)__shfl_xor(eq_b, o);
  }
  if (lane == 0) {
    sh.red[2 * wave] = gt_b;
    sh.red[2 * wave + 1] = eq_b;
  }
  // the slice's keys, loaded in coalesced order and handed to their owners
  // (thread t takes positions base + 16t .. base + 16t + 15)
  const int base = slice * kTopkSlice;
#pragma unroll
  for (int j = 0; j < SKPT; ++j) {
    const int q = j * SNT + tid;
    lds_xpose[xpose_idx(q)] = float_key(s[min(base + q, E - 1)]);
  }
  __syncthreads();
  gt_b = 0u;
  eq_b = 0u;
#pragma unroll
  for (int v = 0; v < SWAVE; ++v) {
    gt_b += sh.red[2 * v];
    eq_b += sh.red[2 * v + 1];
  }
  const int p0 = base + tid * SKPT;
  uint32_t u[SKPT];
#pragma unroll
  for (int i = 0; i < SKPT; ++i) u[i] = lds_xpose[xpose_idx(tid * SKPT + i)];
  uint32_t c = 0u;
#pragma unroll
  for (int i = 0; i < SKPT; ++i) {
    const bool ok = p0 + i < E;
    c += (ok && u[i] > T ? 1u : 0u) + (ok && u[i] == T ? 0x10000u : 0u);
  }
  // a slice holds at most 4096 keys, so neither 16-bit half carries
  const uint32_t ex = split_inclusive_scan(sh, c, lane, wave) - c;
  gt_b += ex & 0xFFFFu;
  eq_b += ex >> 16;
#pragma unroll
  for (int i = 0; i < SKPT; ++i) {
    const bool ok = p0 + i < E;
    const bool gt = ok && u[i] > T, eq = ok && u[i] == T;
    if (gt || (eq && eq_b < take_eq)) {
      const uint32_t pos = gt_b + min(eq_b, take_eq);
      if (pos < (uint32_t)kp) out[pos] = p0 + i;  // pos < kp holds; the guard keeps writes in the row
    }
    gt_b += gt;
    eq_b += eq;
  }
}

}  // namespace

hipError_t launch_topk(const float* scores, int rows, int n, int k, int n_tail, int32_t* idx, void* ws,
                       hipStream_t st) {
  const int E = n - n_tail;
  const int kp = k - n_tail;
  if (E > kTopkResident && kp > 0 && kp < E && rows <= 65535) {
    TkPlan plan;
    topk_make_plan(rows, n, &plan);
    unsigned char* w = static_cast<unsigned char*>(ws);
    uint32_t* hist = reinterpret_cast<uint32_t*>(w + plan.off_hist);
    uint32_t* state = reinterpret_cast<uint32_t*>(w + plan.off_state);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(w + plan.off_cnt);
    const int ns = (E + kTopkSlice - 1) / kTopkSlice;  // at most plan.nslices
    const dim3 g(ns, rows);
    topk_split_zero_kernel<<<rows, SNT, 0, st>>>(hist, idx, k, kp, E, n_tail);
    topk_split_hist_kernel<0><<<g, SNT, 0, st>>>(scores, n, E, kp, hist, state);
    topk_split_hist_kernel<1><<<g, SNT, 0, st>>>(scores, n, E, kp, hist, state);
    topk_split_hist_kernel<2><<<g, SNT, 0, st>>>(scores, n, E, kp, hist, state);
    topk_split_count_kernel<<<g, SNT, 0, st>>>(scores, n, E, hist, state, cnt, plan.nslices);
    topk_split_write_kernel<<<g, SNT, 0, st>>>(scores, n, E, k, kp, state, cnt, plan.nslices, idx);
    return hipGetLastError();
  }
  if (E <= NTH * 4)
    topk_kernel<4, true><<<rows, NTH, 0, st>>>(scores, n, k, n_tail, idx);
  else if (E <= NTH * 8)
    topk_kernel<8, true><<<rows, NTH, 0, st>>>(scores, n, k, n_tail, idx);
  else if (E <= NTH * 16)
    topk_kernel<16, true><<<rows, NTH, 0, st>>>(scores, n, k, n_tail, idx);
  else if (E <= NTH * 32)
    topk_kernel<32, true><<<rows, NTH, 0, st>>>(scores, n, k, n_tail, idx);
  else
    topk_kernel<32, false><<<rows, NTH, 0, st>>>(scores, n, k, n_tail, idx);
  return hipGetLastError();
}

}  // namespace kvc
