// Observation-window attention scores for one layer (gfx950).
//
// Computes, per KV head g of sequence b, the window attention of the G*w query
// rows of its group against all S keys, softmax-normalised per row, and the sum
// of the probabilities over the rows of the group (or over all heads).  Sources:
// "Add TOVA press" (kvpress PR 12: only the window rows [batch, heads,
// window_size, seq_len] are needed; TOVA averages them over heads) and
// "Implement Scissorhands KV-cache compression & SnapKV prompt compression"
// (cold-compress PR 11: the callback receives attention mean-pooled over the
// grouped queries; SnapKV scores the prefix with the observation window).
//
// Layout: the rows of KV head g are the query rows (h, i) for h in the group and
// i < w.  They are contiguous in q_win, so row r = (h - g*G)*w + i is at
// q_win + ((b*Hkv + g)*R + r)*D.
//
// Rows per KV head R = G*w > 16: two passes over the keys, each a 32x32x16 bf16
// (or 32x32x2 fp32) MFMA contraction of 32-row query blocks with 32-key blocks:
//   stats   MFMA A = key block, B = query block.  Each lane holds 16 keys of one
//           query row, so the row's running max and sum of exp2 stay in the lane.
//           Writes (max, sum) per row and key chunk.
//   scores  first combines the chunk partials of its rows into a base-2
//           log-normaliser per row.  MFMA A = query block, B = key block.  Each
//           lane holds 16 rows of one key, so the column sums of
//           exp2(l*c - lse2) stay in the lane; the partial sums of the waves are
//           added in a fixed order in LDS.
//   all_heads    (TOVA) sums the group sums over the KV heads and repeats them.
// Multi-wave workgroups (one wave per 32 query rows, up to 256 rows per launch;
// 128 for fp32 rows of 128 channels) run a continuous stream of 32-key blocks: while the exp work of block b runs
// on the VALU, the MFMAs of block b+1 run on the matrix cores and the K
// fragments of block b+2 are read from LDS.  64-key K tiles pass through a
// three-tile LDS ring (the next tile is already resident when a tile ends), fed
// by up to three tiles of staging registers requested ahead.  One-wave
// workgroups serve 16 < R <= 32 with a simple two-stage loop.
//
// R <= 16 (TOVA with w = 1, Scissorhands decode): the stored-logits path reads
// the keys once.  The four-wave logits kernel streams the keys, writes the
// scaled logits of the real rows and per-chunk (max, sum) partials; the finish
// kernel merges the partials and sums the normalised probabilities (from_logits
// and the separate merge serve more than 1024 merged rows).
// All sums run in a fixed order, so the results are deterministic.
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {

namespace {

// Staging registers use a native vector type: a 16-byte struct copied from
// global memory to LDS would be turned into a memcpy through a stack object.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct WsParams {
  const void* q;
  const void* k;
  const uint8_t* valid;
  const int32_t* chan_idx;
  int Hkv, S, w, R, Rpad, d_keep, causal, CH, nchunks, Spad, rows_total;
  int row0;        // first row of the current row chunk
  int accumulate;  // scores pass: add to the scores already written
  int lse_from_part;  // scores pass: merge the chunk partials itself (no merge launch)
  float c;         // log2(e) / sqrt(D)
  float out_scale; // scores: 1/(G*w) for GROUP, 1 for ALL_HEADS (normalised later)
  float2* part;    // [nchunks][B*Hkv*Rpad] (max, sum of exp2) in base-2 units
  float* lse;      // [B*Hkv*Rpad] base-2 log-normaliser (+inf for empty or padded rows)
  float* logits;   // [B*Hkv*R*Spad] scaled logits (stored-logits path)
  float* scores;   // [B*Hkv*S]
};

template <typename T, int D>
struct TileGeom {
  static constexpr int E = sizeof(T);
  static constexpr int HALF = D / 2;                 // channels per lane half
  static constexpr int NSTEP = HALF / Mfma<T>::KPL;  // MFMA steps per block
  static constexpr int ROWB = D * E;                 // bytes per key row
  static constexpr int LSTRIDE = ROWB + 16;          // padded LDS row stride
  static constexpr int UPR = ROWB / 16;              // 16-byte units per row
  static constexpr int FRAGU = HALF * E / 16;        // 16-byte units per lane fragment
};

template <typename T, int D>
union Frag {
  uint4 u[TileGeom<T, D>::FRAGU];
  typename Mfma<T>::op_t o[TileGeom<T, D>::NSTEP];
};

// Keys per LDS tile of the stream kernels.
template <typename T, int D, int NW>
struct StreamTK {
  static constexpr int value = 64;
};

// Tiles of staging registers of the stream kernels: K tiles are requested that
// many tiles ahead of the LDS ring, within about 24 registers per thread.  SHORT
// (a workgroup streams at most kShortChunkTiles tiles): two sets instead of
// three.  Measured on MI355X at 16 tiles per workgroup (SnapKV 32k) the third set
// costs 4% of a score call, at 64 (ThinK 128k) it gains 3%: a short chunk spends
// a larger share of its time in the start-up burst, which more requests only
// lengthen, and a long one gains from the deeper prefetch.
constexpr int kShortChunkTiles = 16;

template <typename T, int D, int NW, bool SHORT>
struct StreamNSTG {
  static constexpr int UPT = StreamTK<T, D, NW>::value * D * (int)sizeof(T) / 16 / (NW * 64);
  static constexpr int value = UPT <= 2 ? (SHORT ? 2 : 3) : UPT <= 3 ? 2 : 1;
};

// Buffer descriptor word 3 for raw (unswizzled, stride 0) buffers on gfx9.
constexpr int kRawBufferFlags = 0x00020000;

// Cache policy of the K staging loads (the buffer loads' cache-policy operand:
// 1 sc0, 2 non-temporal).  A K tile is read once per workgroup, so neither pass
// gains from the per-CU cache; the statistics pass reads K with sc0 but not
// non-temporal: the scores pass reads the same keys right after it and finds part
// of them in the shared caches.  The scores pass is K's last use, so its loads
// are non-temporal and leave the caches to the other streams' data.  Measured on
// MI355X against no hints: the SnapKV 32k call alone 1.6% faster and the ThinK
// 128k layer +2.8% tokens/s; non-temporal loads in the statistics pass cost the
// SnapKV 32k layer 2.5%.
constexpr int kStatsCpol = 1;
constexpr int kScoresCpol = 2;

// K tile staging: contiguous global rows -> registers -> padded LDS rows.
// Loads go through a buffer descriptor whose base is the tile's first key and
// whose size ends at `end`, the end of the workgroup's key chunk (saturated at
// 2^32 - 1 bytes), so the only per-tile address work is scalar, rows past the
// chunk read nothing (zero: past S those keys are masked, and tiles never
// straddle an inner chunk boundary), and a tile wholly past the chunk costs no
// memory traffic.  The vector offsets are per-thread constants; CPOL is the
// cache policy above.
template <typename T, int D, int NT, int TK, int CPOL = 0>
struct Stager {
  using G_ = TileGeom<T, D>;
  static constexpr int UPT = TK * G_::UPR / NT;
  static_assert((TK * G_::UPR) % NT == 0, "tile units must split evenly");
  static_assert(TK <= NT, "one validity byte per thread");
  u32x4_t pre[UPT];
  uint8_t pre_valid;

  // Every thread issues the same loads whatever the tile, so the compiler can
  // count them; without a validity mask the byte comes from the key data and is
  // ignored.
  __device__ inline void load(const unsigned char* kbase, const uint8_t* vrow, int base, int end, int tid) {
    const int left = max(end - base, 0);
    const unsigned long long kbytes = (unsigned long long)left * G_::ROWB;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(kbase) + (size_t)base * G_::ROWB, (short)0,
        (int)(unsigned)(kbytes < 0xFFFFFFFFull ? kbytes : 0xFFFFFFFFull), kRawBufferFlags);
#pragma unroll
    for (int i = 0; i < UPT; ++i) pre[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, (tid + i * NT) * 16, 0, CPOL);
    const __amdgpu_buffer_rsrc_t rv =
        vrow ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vrow) + base, (short)0, left, kRawBufferFlags)
             : rk;
    pre_valid = __builtin_amdgcn_raw_buffer_load_b8(rv, tid % TK, 0, CPOL);
  }
  __device__ inline void store(unsigned char* lds_k, uint8_t* lds_v, int tid, bool has_valid) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      const int row = u / G_::UPR, cu = u % G_::UPR;
      *reinterpret_cast<u32x4_t*>(lds_k + row * G_::LSTRIDE + cu * 16) = pre[i];
    }
    if (has_valid && tid < TK) lds_v[tid] = pre_valid;
  }
};


template <typename T, int D>
__device__ inline void read_frag(Frag<T, D>& f, const unsigned char* tile, int key_in_tile, int half) {
  using G_ = TileGeom<T, D>;
  const uint4* src = reinterpret_cast<const uint4*>(tile + key_in_tile * G_::LSTRIDE + half * G_::HALF * G_::E);
#pragma unroll
  for (int u = 0; u < G_::FRAGU; ++u) f.u[u] = src[u];
}

template <typename T, int D>
__device__ inline f32x16_t mma_block(const Frag<T, D>& a, const Frag<T, D>& b) {
  f32x16_t acc = {};
#pragma unroll
  for (int s = 0; s < TileGeom<T, D>::NSTEP; ++s) acc = Mfma<T>::run(a.o[s], b.o[s], acc);
  return acc;
}

// Query fragment of one row (zero for padded rows); channels not in the keep
// mask are zeroed.
template <typename T, int D>
__device__ inline void load_query(Frag<T, D>& qf, const WsParams& p, size_t bg, int r, int half,
                                  const uint32_t* keep) {
  using M = Mfma<T>;
  using G_ = TileGeom<T, D>;
  if (r < p.R) {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned char*>(p.q) +
                                                      ((bg * p.R + r) * D + half * G_::HALF) * G_::E);
#pragma unroll
    for (int u = 0; u < G_::FRAGU; ++u) qf.u[u] = src[u];
    if (keep) {
#pragma unroll
      for (int s = 0; s < G_::NSTEP; ++s) {
#pragma unroll
        for (int e = 0; e < M::KPL; ++e) {
          const int d = half * G_::HALF + s * M::KPL + e;
          if (!((keep[d >> 5] >> (d & 31)) & 1u)) {
            if constexpr (M::KPL == 1) qf.o[s] = 0.0f;
            else qf.o[s][e] = (__bf16)0.0f;
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < G_::FRAGU; ++u) qf.u[u] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// Query fragments of the 32 rows rowblk .. rowblk+31 of (b, g), through the
// wave's LDS slot.  The rows are contiguous in q_win, so the wave reads them with
// coalesced 16-byte loads (each instruction covers 1 KB of consecutive rows, not
// one 16-byte piece of each of 64 rows), writes them to padded LDS rows and reads
// its fragment back; the wave's LDS operations run in order.  Rows past R are
// zero; channels not in the keep mask are zeroed.
template <typename T, int D>
__device__ inline void load_query_rows(Frag<T, D>& qf, const WsParams& p, size_t bg, int rowblk, int lane, int half,
                                       const uint32_t* keep, unsigned char* slot) {
  using M = Mfma<T>;
  using G_ = TileGeom<T, D>;
  constexpr int UPL = 32 * G_::ROWB / 16 / 64;  // 16-byte units per lane
  const unsigned char* src =
      reinterpret_cast<const unsigned char*>(p.q) + (bg * p.R + (size_t)rowblk) * (size_t)G_::ROWB;
  u32x4_t d[UPL];
#pragma unroll
  for (int u = 0; u < UPL; ++u) {
    const int off = u * 1024 + lane * 16;
    d[u] = (rowblk + off / G_::ROWB < p.R) ? *reinterpret_cast<const u32x4_t*>(src + off) : u32x4_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < UPL; ++u) {
    const int off = u * 1024 + lane * 16;
    *reinterpret_cast<u32x4_t*>(slot + (off / G_::ROWB) * G_::LSTRIDE + off % G_::ROWB) = d[u];
  }
  __builtin_amdgcn_wave_barrier();
  read_frag<T, D>(qf, slot, lane & 31, half);
  __builtin_amdgcn_wave_barrier();
  if (keep) {
#pragma unroll
    for (int s = 0; s < G_::NSTEP; ++s) {
#pragma unroll
      for (int e = 0; e < M::KPL; ++e) {
        const int dch = half * G_::HALF + s * M::KPL + e;
        if (!((keep[dch >> 5] >> (dch & 31)) & 1u)) {
          if constexpr (M::KPL == 1) qf.o[s] = 0.0f;
          else qf.o[s][e] = (__bf16)0.0f;
        }
      }
    }
  }
}

// Bit mask of the kept key channels of (b, g) (ThinK), built in LDS.
template <int D, int NT>
__device__ inline const uint32_t* build_keep(uint32_t* lds_keep, const WsParams& p, size_t bg, int tid) {
  if (!p.chan_idx) return nullptr;
  if (tid < D / 32) lds_keep[tid] = 0u;
  __syncthreads();
  for (int i = tid; i < p.d_keep; i += NT) {
    const int ch = p.chan_idx[bg * p.d_keep + i];
    if (ch >= 0 && ch < D) atomicOr(&lds_keep[ch >> 5], 1u << (ch & 31));
  }
  __syncthreads();
  return lds_keep;
}

// Minus the log-normalisers of the 16 rows held by a lane's accumulator
// registers (scores pass layout: rows are the accumulator rows).
__device__ inline void load_neg_lse(float (&nb)[16], const WsParams& p, size_t bg, int rowblk, int half) {
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4) {
    const float4 l4 = *reinterpret_cast<const float4*>(p.lse + bg * p.Rpad + rowblk + 8 * v4 + 4 * half);
    nb[4 * v4 + 0] = -l4.x;
    nb[4 * v4 + 1] = -l4.y;
    nb[4 * v4 + 2] = -l4.z;
    nb[4 * v4 + 3] = -l4.w;
  }
}

// The same values merged here from the chunk partials of the statistics pass
// (the scores pass then needs no merge launch before it): lane (col, half) folds
// chunks half, half+2, ... of row rowblk+col, the two lane halves are merged,
// and every lane fetches its 16 accumulator rows from the lanes that hold them.
// Rows past R, and rows with no allowed key, get +inf.
__device__ inline void neg_lse_from_part(float (&nb)[16], const WsParams& p, size_t bg, int rowblk, int lane,
                                         int half) {
  const int r = rowblk + (lane & 31);
  const float2* part = p.part + bg * p.Rpad + r;
  float m = kNegInf, z = 0.0f;
  int c = half;
  for (; c + 6 < p.nchunks; c += 8) {  // four partials requested together
    float2 pc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pc[i] = part[(size_t)(c + 2 * i) * p.rows_total];
#pragma unroll
    for (int i = 0; i < 4; ++i) lse2_merge(m, z, pc[i].x, pc[i].y);
  }
  for (; c < p.nchunks; c += 2) {
    const float2 pc = part[(size_t)c * p.rows_total];
    lse2_merge(m, z, pc.x, pc.y);
  }
  lse2_merge(m, z, __shfl_xor(m, 32), __shfl_xor(z, 32));
  const float l = (r >= p.R || m == kNegInf || !(z > 0.0f)) ? kPosInf : m + log2f(z);
#pragma unroll
  for (int v = 0; v < 16; ++v) nb[v] = -__shfl(l, acc_row(v, lane));
}

// Fold the 16 logits of one (query row, 16 keys) lane slice into the lane's
// running (max, sum exp2).  Keys failing the mask must already be -inf.
__device__ inline void fold_stats(const f32x16_t& a, float c, float& m_run, float& z_run) {
  float tmax = fmaxf(a[0], a[1]);
#pragma unroll
  for (int v = 2; v < 16; v += 2) tmax = fmaxf(fmaxf(tmax, a[v]), a[v + 1]);
  const float mn = fmaxf(m_run, tmax * c);
  const float nmn = -mn;
  float zs[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) zs[v] = fast_exp2(fmaf(a[v], c, nmn));
#pragma unroll
  for (int v = 4; v < 16; ++v) zs[v & 3] += fast_exp2(fmaf(a[v], c, nmn));
  const float znew = z_run * fast_exp2(m_run - mn) + ((zs[0] + zs[1]) + (zs[2] + zs[3]));
  const bool live = mn != kNegInf;  // a slice with every key masked changes nothing
  z_run = live ? znew : z_run;
  m_run = live ? mn : m_run;
}

// The same fold without a running maximum, for the streaming statistics pass:
// (m, z) is kept as a reference m and z = sum of exp2(l*c - m) over the keys so
// far, which describes the same log-normaliser m + log2(z) whatever m is.  The
// reference moves only when the new sum would leave [0, 2^64): an unset
// reference (first allowed key), a key far above it, or a long run of large
// terms.  Then the slice's maximum (or the old reference, if larger) becomes the
// reference and the sum is rescaled; a sum still at 2^32 or more is brought into
// [1, 2) by a power of two, moved exactly into the reference.  The common case
// costs one fma, one exp2 and one add per logit.
__device__ inline void fold_stats_ref(const f32x16_t& a, float c, float& m_ref, float& z_run) {
  const float nm = -m_ref;
  float zs[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) zs[v] = fast_exp2(fmaf(a[v], c, nm));
#pragma unroll
  for (int v = 4; v < 16; ++v) zs[v & 3] += fast_exp2(fmaf(a[v], c, nm));
  const float znew = z_run + ((zs[0] + zs[1]) + (zs[2] + zs[3]));
  if (znew < 0x1p64f) {  // false for +inf and NaN (unset reference)
    z_run = znew;
    return;
  }
  float tmax = fmaxf(a[0], a[1]);
#pragma unroll
  for (int v = 2; v < 16; v += 2) tmax = fmaxf(fmaxf(tmax, a[v]), a[v + 1]);
  float mn = fmaxf(m_ref, tmax * c);
  if (mn == kNegInf) return;  // every key so far masked: the sum stays 0
  const float nmn = -mn;
#pragma unroll
  for (int v = 0; v < 4; ++v) zs[v] = fast_exp2(fmaf(a[v], c, nmn));
#pragma unroll
  for (int v = 4; v < 16; ++v) zs[v & 3] += fast_exp2(fmaf(a[v], c, nmn));
  float z = z_run * fast_exp2(m_ref - mn) + ((zs[0] + zs[1]) + (zs[2] + zs[3]));
  if (!(z < 0x1p32f)) {
    const int e = (int)((__float_as_uint(z) >> 23) & 0xFFu) - 127;  // z is finite and >= 2^32
    z = __uint_as_float(__float_as_uint(z) - ((uint32_t)e << 23));
    mn += (float)e;
  }
  m_ref = mn;
  z_run = z;
}

// Mask the stats-layout slice: keys above `lim` or holes become -inf.  The keys
// of registers 4*v4 .. 4*v4+3 are consecutive, so their validity bytes come in one
// 32-bit LDS word.
__device__ inline void mask_stats(f32x16_t& a, int key_base, int lim, const uint8_t* lv, bool has_valid, int half) {
#pragma unroll
  for (int v4 = 0; v4 < 4; ++v4) {
    const int kk0 = 8 * v4 + 4 * half;
    const uint32_t vw = has_valid ? *reinterpret_cast<const uint32_t*>(lv + kk0) : 0x01010101u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = (key_base + kk0 + e <= lim) & (((vw >> (8 * e)) & 0xFFu) != 0u);
      a[4 * v4 + e] = ok ? a[4 * v4 + e] : kNegInf;
    }
  }
}

template <int NMFMA, int NVALU>
__device__ inline void interleave_hint() {
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);
  }
}

template <bool B>
using bool_t = std::integral_constant<bool, B>;

// ---------------------------------------------------------------------------
// Stream kernels (NW = 2, 4, 8 waves; one 32-row block per wave)
// ---------------------------------------------------------------------------

// The shared skeleton: prologue (two tiles into LDS, the next NSTG into the
// staging registers), tile loop with the three-tile LDS ring, and the block
// stream.  `mfma(kf)` runs the contraction of one block, `epi(acc, t, kb,
// masked)` its VALU work, `post(t)` runs after the barrier ending tile t.
template <typename T, int D, int NW, bool SHORT, int CPOL, typename Mma, typename Epi, typename Post>
__device__ inline void stream_blocks(const unsigned char* kbase, const uint8_t* vrow, int key0, int key1,
                                     int ntiles, bool has_valid, int tid, int col, int half, int S, int w,
                                     int causal,
                                     unsigned char (*lds_k)[StreamTK<T, D, NW>::value * TileGeom<T, D>::LSTRIDE],
                                     uint8_t (*lds_v)[StreamTK<T, D, NW>::value], Mma mfma, Epi epi, Post post) {
  constexpr int NT = NW * 64;
  constexpr int TK = StreamTK<T, D, NW>::value;
  constexpr int NSTG = StreamNSTG<T, D, NW, SHORT>::value;
  constexpr int KB = TK / 32;
  static_assert(KB % 2 == 0, "fragment double buffer alternates within a tile");
  using G_ = TileGeom<T, D>;
  using Stg = Stager<T, D, NT, TK, CPOL>;

  static_assert(NSTG >= 1 && NSTG <= 3, "one to three staging sets");
  Stg s0, s1, s2;  // the staging sets (s1, s2 unused with fewer)
  {
    // Tiles 0 and 1 (into the LDS ring) and tile 2 (into the first staging set,
    // stored at the end of tile 0) are requested together, in one memory round
    // trip with the caller's query loads; only tiles 0 and 1 are waited for
    // before the first barrier.  The other staging tiles follow once the ring
    // is filled: at the start of a pass every workgroup waits for its first
    // tiles at once, and requesting more then only lengthens that burst.
    // The loads are unconditional (a tile past the chunk reads nothing: its
    // descriptor is empty), so the compiler can count them exactly and the
    // first tile waits only for what it uses.
    Stg p0, p1;
    p0.load(kbase, vrow, key0, key1, tid);
    p1.load(kbase, vrow, key0 + TK, key1, tid);
    __builtin_amdgcn_sched_barrier(0);  // tile 2 after tiles 0 and 1: their stores wait for them only
    s0.load(kbase, vrow, key0 + 2 * TK, key1, tid);
    if (ntiles > 0) p0.store(lds_k[0], lds_v[0], tid, has_valid);
    if (ntiles > 1) p1.store(lds_k[1], lds_v[1], tid, has_valid);
  }
  __syncthreads();
  if (ntiles <= 0) return;
  if constexpr (NSTG > 1) s1.load(kbase, vrow, key0 + 3 * TK, key1, tid);
  if constexpr (NSTG > 2) s2.load(kbase, vrow, key0 + 4 * TK, key1, tid);

  Frag<T, D> kf[2];
  read_frag<T, D>(kf[0], lds_k[0], col, half);
  read_frag<T, D>(kf[1], lds_k[0], 32 + col, half);
  f32x16_t acc = mfma(kf[0]);

  // tile t; `st` holds tile t+2 and is refilled with tile t+2+NSTG.  FULL: both
  // tiles exist, so the store and the load are unconditional.
  auto tile = [&](int t, Stg& st, auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int base = key0 + t * TK;
    const bool masked = has_valid || (base + TK > S) || (causal && base + TK - 1 > S - w);
    const unsigned char* next_tile = lds_k[(t + 1) % 3];
    const unsigned char* this_tile = lds_k[t % 3];

    auto run = [&](auto masked_tag, auto last_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      constexpr bool LAST = decltype(last_tag)::value;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int cur = kb & 1;
        // K fragment of block kb+2 (possibly in the next tile) into the buffer
        // the MFMAs of block kb have consumed
        if (!LAST || kb + 2 < KB) {
          const unsigned char* src = (kb + 2 < KB) ? this_tile : next_tile;
          read_frag<T, D>(kf[cur], src, ((kb + 2) % KB) * 32 + col, half);
        }
        f32x16_t nxt;
        if (!LAST || kb + 1 < KB) nxt = mfma(kf[cur ^ 1]);
        epi(acc, t, kb, MASKED);
        if constexpr (!MASKED) interleave_hint<G_::NSTEP, 6>();
        __builtin_amdgcn_sched_barrier(0);
        if (!LAST || kb + 1 < KB) acc = nxt;
      }
    };
    if (t + 1 < ntiles) {
      if (masked) run(bool_t<true>(), bool_t<false>());
      else run(bool_t<false>(), bool_t<false>());
    } else {
      if (masked) run(bool_t<true>(), bool_t<true>());
      else run(bool_t<false>(), bool_t<true>());
    }

    if (FULL || t + 2 < ntiles) st.store(lds_k[(t + 2) % 3], lds_v[(t + 2) % 3], tid, has_valid);
    __syncthreads();
    post(t);
    st.load(kbase, vrow, base + (2 + NSTG) * TK, key1, tid);  // past the chunk: an empty descriptor, nothing read
  };
  int t = 0;
  for (; t + 2 * NSTG + 1 < ntiles; t += NSTG) {  // steady state
    tile(t, s0, bool_t<true>());
    if constexpr (NSTG > 1) tile(t + 1, s1, bool_t<true>());
    if constexpr (NSTG > 2) tile(t + 2, s2, bool_t<true>());
  }
  for (; t < ntiles; t += NSTG) {
    tile(t, s0, bool_t<false>());
    if constexpr (NSTG > 1)
      if (t + 1 < ntiles) tile(t + 1, s1, bool_t<false>());
    if constexpr (NSTG > 2)
      if (t + 2 < ntiles) tile(t + 2, s2, bool_t<false>());
  }
}

// ---------------------------------------------------------------------------
// ThinK with at most 64 of 128 bf16 key channels kept: the passes contract on
// the kept channels only.  K tiles are staged as usual (coalesced 16-byte
// loads) into a two-tile ring of full rows; one tile later every thread builds
// a 16-byte unit of a compacted row (8 kept channels, 2-byte LDS reads) into the
// three-tile ring the MFMAs read, 64 channels per key.  The query rows are
// compacted in the same channel order.
// ---------------------------------------------------------------------------

// Byte offsets, within a 128-channel bf16 row, of the 8 kept channels that make
// up this thread's 16-byte unit of a compacted row (unit tid % 8).
struct ChOff {
  int off[8];
};

// The kept channels in ascending order (from the keep mask, so a repeated entry
// counts once), padded with channel 0 up to 64; returns how many are kept.  The
// list must have been zeroed before build_keep's first barrier.
__device__ inline int kept_channel_list(uint16_t* lds_ch, const uint32_t* keep, int tid) {
  if (tid < 128) {
    const int wd = tid >> 5, b = tid & 31;
    if ((keep[wd] >> b) & 1u) {
      int rank = __popc(keep[wd] & ((1u << b) - 1u));
      for (int i = 0; i < wd; ++i) rank += __popc(keep[i]);
      if (rank < 64) lds_ch[rank] = (uint16_t)tid;
    }
  }
  __syncthreads();
  return __popc(keep[0]) + __popc(keep[1]) + __popc(keep[2]) + __popc(keep[3]);
}

// Query fragments of the 32 rows rowblk .. rowblk+31 of (b, g) on the kept
// channels: the rows go through the wave's LDS slot as in load_query_rows, and
// compacted channel i of a row is its channel lds_ch[i] (zero past n_kept).
__device__ inline void load_query_rows_kept(Frag<__bf16, 64>& qf, const WsParams& p, size_t bg, int rowblk, int lane,
                                            int half, const uint16_t* lds_ch, int n_kept, unsigned char* slot) {
  using GL = TileGeom<__bf16, 128>;
  constexpr int UPL = 32 * GL::ROWB / 16 / 64;
  const unsigned char* src =
      reinterpret_cast<const unsigned char*>(p.q) + (bg * p.R + (size_t)rowblk) * (size_t)GL::ROWB;
  u32x4_t d[UPL];
#pragma unroll
  for (int u = 0; u < UPL; ++u) {
    const int off = u * 1024 + lane * 16;
    d[u] = (rowblk + off / GL::ROWB < p.R) ? *reinterpret_cast<const u32x4_t*>(src + off) : u32x4_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < UPL; ++u) {
    const int off = u * 1024 + lane * 16;
    *reinterpret_cast<u32x4_t*>(slot + (off / GL::ROWB) * GL::LSTRIDE + off % GL::ROWB) = d[u];
  }
  __builtin_amdgcn_wave_barrier();
  const unsigned char* row = slot + (lane & 31) * GL::LSTRIDE;
  uint32_t w[16];  // this lane's compacted channels half*32 .. half*32+31, two per word
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int i0 = half * 32 + 2 * j, i1 = i0 + 1;
    const uint32_t lo = i0 < n_kept ? *reinterpret_cast<const uint16_t*>(row + 2 * lds_ch[i0]) : 0u;
    const uint32_t hi = i1 < n_kept ? *reinterpret_cast<const uint16_t*>(row + 2 * lds_ch[i1]) : 0u;
    w[j] = lo | (hi << 16);
  }
  __builtin_amdgcn_wave_barrier();
  static_assert(sizeof(qf.u) == sizeof(w), "32 bf16 per lane");
  __builtin_memcpy(&qf.u[0], w, sizeof(w));
}

constexpr int kRawStride = TileGeom<__bf16, 128>::LSTRIDE;  // full 128-channel rows
constexpr int kKeptStride = TileGeom<__bf16, 64>::LSTRIDE;  // compacted 64-channel rows

// Compact one staged tile: this thread's units (key u/8, unit u%8) of the
// 64-key tile, and the tile's validity bytes.
template <int NT>
__device__ inline void gather_kept_tile(const unsigned char* raw, const uint8_t* raw_v, unsigned char* kept,
                                        uint8_t* kept_v, int tid, const ChOff& ch, bool has_valid) {
  constexpr int UPT = 64 * 8 / NT;
  static_assert(UPT * NT == 64 * 8 && NT % 8 == 0, "units split evenly; a thread keeps its unit column");
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + i * NT;
    const unsigned char* r = raw + (u >> 3) * kRawStride;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = *reinterpret_cast<const uint16_t*>(r + ch.off[2 * q]);
      const uint32_t hi = *reinterpret_cast<const uint16_t*>(r + ch.off[2 * q + 1]);
      w[q] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4_t*>(kept + (u >> 3) * kKeptStride + (u & 7) * 16) = u32x4_t{w[0], w[1], w[2], w[3]};
  }
  if (has_valid && tid < 64) kept_v[tid] = raw_v[tid];
}

// The stream skeleton of stream_blocks on compacted keys: staged tiles go to
// the two-slot ring of full rows one tile earlier, and at the end of tile t
// the staged tile t+2 is compacted into the ring slot the MFMAs read, behind
// the same barrier (so the pipeline takes one more tile of staging ahead).
template <int NW, bool SHORT, int CPOL, typename Mma, typename Epi, typename Post>
__device__ inline void stream_blocks_kept(const unsigned char* kbase, const uint8_t* vrow, int key0, int key1,
                                          int ntiles, bool has_valid, int tid, int col, int half, int S, int w,
                                          int causal, unsigned char (*lds_raw)[64 * kRawStride],
                                          uint8_t (*lds_rv)[64], unsigned char (*lds_k)[64 * kKeptStride],
                                          uint8_t (*lds_v)[64], const ChOff& ch, Mma mfma, Epi epi, Post post) {
  using T = __bf16;
  constexpr int D = 64;
  constexpr int NT = NW * 64;
  constexpr int TK = 64;
  static_assert(StreamTK<T, 128, NW>::value == TK && StreamTK<T, D, NW>::value == TK, "64-key tiles");
  constexpr int NSTG = StreamNSTG<T, 128, NW, SHORT>::value;
  constexpr int KB = TK / 32;
  using G_ = TileGeom<T, D>;
  using Stg = Stager<T, 128, NT, TK, CPOL>;
  static_assert(NSTG >= 1 && NSTG <= 3, "one to three staging sets");

  Stg s0, s1, s2;
  {
    // staged tiles 0 and 1 compacted behind the first barrier; staged tile 2
    // stored behind the second (the gather of tile 0 is still reading its slot)
    Stg p0, p1, p2;
    p0.load(kbase, vrow, key0, key1, tid);
    p1.load(kbase, vrow, key0 + TK, key1, tid);
    __builtin_amdgcn_sched_barrier(0);
    p2.load(kbase, vrow, key0 + 2 * TK, key1, tid);
    s0.load(kbase, vrow, key0 + 3 * TK, key1, tid);
    if (ntiles > 0) p0.store(lds_raw[0], lds_rv[0], tid, has_valid);
    if (ntiles > 1) p1.store(lds_raw[1], lds_rv[1], tid, has_valid);
    __syncthreads();
    if (ntiles > 0) gather_kept_tile<NT>(lds_raw[0], lds_rv[0], lds_k[0], lds_v[0], tid, ch, has_valid);
    if (ntiles > 1) gather_kept_tile<NT>(lds_raw[1], lds_rv[1], lds_k[1], lds_v[1], tid, ch, has_valid);
    __syncthreads();
    if (ntiles > 2) p2.store(lds_raw[0], lds_rv[0], tid, has_valid);
  }
  __syncthreads();
  if (ntiles <= 0) return;
  if constexpr (NSTG > 1) s1.load(kbase, vrow, key0 + 4 * TK, key1, tid);
  if constexpr (NSTG > 2) s2.load(kbase, vrow, key0 + 5 * TK, key1, tid);

  Frag<T, D> kf[2];
  read_frag<T, D>(kf[0], lds_k[0], col, half);
  read_frag<T, D>(kf[1], lds_k[0], 32 + col, half);
  f32x16_t acc = mfma(kf[0]);

  // tile t; `st` holds staged tile t+3 and is refilled with tile t+3+NSTG
  auto tile = [&](int t, Stg& st, auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int base = key0 + t * TK;
    const bool masked = has_valid || (base + TK > S) || (causal && base + TK - 1 > S - w);
    const unsigned char* next_tile = lds_k[(t + 1) % 3];
    const unsigned char* this_tile = lds_k[t % 3];

    auto run = [&](auto masked_tag, auto last_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      constexpr bool LAST = decltype(last_tag)::value;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int cur = kb & 1;
        if (!LAST || kb + 2 < KB) {
          const unsigned char* src = (kb + 2 < KB) ? this_tile : next_tile;
          read_frag<T, D>(kf[cur], src, ((kb + 2) % KB) * 32 + col, half);
        }
        f32x16_t nxt;
        if (!LAST || kb + 1 < KB) nxt = mfma(kf[cur ^ 1]);
        epi(acc, t, kb, MASKED);
        if constexpr (!MASKED) interleave_hint<G_::NSTEP, 6>();
        __builtin_amdgcn_sched_barrier(0);
        if (!LAST || kb + 1 < KB) acc = nxt;
      }
    };
    if (t + 1 < ntiles) {
      if (masked) run(bool_t<true>(), bool_t<false>());
      else run(bool_t<false>(), bool_t<false>());
    } else {
      if (masked) run(bool_t<true>(), bool_t<true>());
      else run(bool_t<false>(), bool_t<true>());
    }

    if (FULL || t + 3 < ntiles) st.store(lds_raw[(t + 1) & 1], lds_rv[(t + 1) & 1], tid, has_valid);
    if (FULL || t + 2 < ntiles)
      gather_kept_tile<NT>(lds_raw[t & 1], lds_rv[t & 1], lds_k[(t + 2) % 3], lds_v[(t + 2) % 3], tid, ch,
                           has_valid);
    __syncthreads();
    post(t);
    st.load(kbase, vrow, base + (3 + NSTG) * TK, key1, tid);  // past the chunk: an empty descriptor, nothing read
  };
  int t = 0;
  for (; t + 2 * NSTG + 2 < ntiles; t += NSTG) {  // steady state
    tile(t, s0, bool_t<true>());
    if constexpr (NSTG > 1) tile(t + 1, s1, bool_t<true>());
    if constexpr (NSTG > 2) tile(t + 2, s2, bool_t<true>());
  }
  for (; t < ntiles; t += NSTG) {
    tile(t, s0, bool_t<false>());
    if constexpr (NSTG > 1)
      if (t + 1 < ntiles) tile(t + 1, s1, bool_t<false>());
    if constexpr (NSTG > 2)
      if (t + 2 < ntiles) tile(t + 2, s2, bool_t<false>());
  }
}

// GATHER (bf16, D = 128, at most 64 kept channels): the contraction runs on the
// kept channels only (DC = 64) through stream_blocks_kept.
template <typename T, int D, int NW, bool SHORT, bool GATHER>
__global__ __launch_bounds__(NW * 64) void ws_stats_stream_kernel(WsParams p) {
  static_assert(!GATHER || (sizeof(T) == 2 && D == 128), "compaction of 128 bf16 channels to 64");
  constexpr int DC = GATHER ? 64 : D;
  using GL = TileGeom<T, D>;   // stored rows
  using G_ = TileGeom<T, DC>;  // the ring the MFMAs read
  constexpr int NT = NW * 64;
  constexpr int TK = StreamTK<T, DC, NW>::value;

  __shared__ __attribute__((aligned(16))) unsigned char lds_k[3][TK * G_::LSTRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_valid[3][TK];
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[GATHER ? 2 : 1][GATHER ? 64 * kRawStride : 16];
  __shared__ uint8_t lds_rv[GATHER ? 2 : 1][64];
  // query staging slots (bf16 only: fp32 rows would not fit next to the ring)
  constexpr bool QLDS = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) unsigned char lds_q[QLDS ? NW : 1][QLDS ? 32 * GL::LSTRIDE : 16];
  __shared__ uint32_t lds_keep[D / 32];
  __shared__ uint16_t lds_ch[GATHER ? 64 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
  const int chunk = blockIdx.x;
  const size_t bg = (size_t)blockIdx.z * p.Hkv + blockIdx.y;
  const int key0 = chunk * p.CH;
  const int key1 = min(p.S, key0 + p.CH);
  const int ntiles = (key1 - key0 + TK - 1) / TK;
  const bool has_valid = p.valid != nullptr;
  const uint8_t* vrow = has_valid ? p.valid + bg * p.S : nullptr;

  if constexpr (GATHER)
    if (tid < 64) lds_ch[tid] = 0;
  const uint32_t* keep = build_keep<D, NT>(lds_keep, p, bg, tid);
  const int r = p.row0 + wave * 32 + col;  // this lane's query row
  Frag<T, DC> qf;
  ChOff choff;
  if constexpr (GATHER) {
    const int n_kept = kept_channel_list(lds_ch, keep, tid);
    load_query_rows_kept(qf, p, bg, p.row0 + wave * 32, lane, half, lds_ch, n_kept, lds_q[wave]);
#pragma unroll
    for (int e = 0; e < 8; ++e) choff.off[e] = 2 * lds_ch[(tid & 7) * 8 + e];
  } else if constexpr (QLDS) {
    load_query_rows<T, D>(qf, p, bg, p.row0 + wave * 32, lane, half, keep, lds_q[wave]);
  } else {
    load_query<T, D>(qf, p, bg, r, half, keep);
  }
  int lim = p.S - 1;
  if (p.causal && r < p.R) lim = min(p.S - 1, p.S - p.w + r % p.w);
  float m_run = kNegInf, z_run = 0.0f;

  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) + bg * (size_t)p.S * GL::ROWB;
  auto mfma = [&](const Frag<T, DC>& kf) { return mma_block<T, DC>(kf, qf); };
  auto epi = [&](f32x16_t& a, int t, int kb, bool masked) {
    if (masked) mask_stats(a, key0 + t * TK + kb * 32, lim, &lds_valid[t % 3][kb * 32], has_valid, half);
    fold_stats_ref(a, p.c, m_run, z_run);
  };
  if constexpr (GATHER)
    stream_blocks_kept<NW, SHORT, kStatsCpol>(kbase, vrow, key0, key1, ntiles, has_valid, tid, col, half, p.S, p.w,
                                              p.causal, lds_raw, lds_rv, lds_k, lds_valid, choff, mfma, epi,
                                              [](int) {});
  else
    stream_blocks<T, D, NW, SHORT, kStatsCpol>(kbase, vrow, key0, key1, ntiles, has_valid, tid, col, half, p.S, p.w,
                                               p.causal, lds_k, lds_valid, mfma, epi, [](int) {});

  const float m2 = __shfl_xor(m_run, 32);
  const float z2 = __shfl_xor(z_run, 32);
  lse2_merge(m_run, z_run, m2, z2);
  if (half == 0) p.part[(size_t)chunk * p.rows_total + bg * p.Rpad + r] = make_float2(m_run, z_run);
}

template <typename T, int D, int NW, bool SHORT, bool GATHER>
__global__ __launch_bounds__(NW * 64) void ws_scores_stream_kernel(WsParams p) {
  static_assert(!GATHER || (sizeof(T) == 2 && D == 128), "compaction of 128 bf16 channels to 64");
  constexpr int DC = GATHER ? 64 : D;
  using GL = TileGeom<T, D>;   // stored rows
  using G_ = TileGeom<T, DC>;  // the ring the MFMAs read
  constexpr int NT = NW * 64;
  constexpr int TK = StreamTK<T, DC, NW>::value;

  __shared__ __attribute__((aligned(16))) unsigned char lds_k[3][TK * G_::LSTRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_valid[3][TK];
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[GATHER ? 2 : 1][GATHER ? 64 * kRawStride : 16];
  __shared__ uint8_t lds_rv[GATHER ? 2 : 1][64];
  __shared__ float lds_red[3][2 * NW][TK];
  // query staging slots (bf16 only: fp32 rows would not fit next to the ring)
  constexpr bool QLDS = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) unsigned char lds_q[QLDS ? NW : 1][QLDS ? 32 * GL::LSTRIDE : 16];
  __shared__ uint32_t lds_keep[D / 32];
  __shared__ uint16_t lds_ch[GATHER ? 64 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
  const int chunk = blockIdx.x;
  const size_t bg = (size_t)blockIdx.z * p.Hkv + blockIdx.y;
  const int key0 = chunk * p.CH;
  const int key1 = min(p.S, key0 + p.CH);
  const int ntiles = (key1 - key0 + TK - 1) / TK;
  const bool has_valid = p.valid != nullptr;
  const uint8_t* vrow = has_valid ? p.valid + bg * p.S : nullptr;

  if constexpr (GATHER)
    if (tid < 64) lds_ch[tid] = 0;
  const uint32_t* keep = build_keep<D, NT>(lds_keep, p, bg, tid);
  const int rowblk = p.row0 + wave * 32;
  Frag<T, DC> qf;
  ChOff choff;
  if constexpr (GATHER) {
    const int n_kept = kept_channel_list(lds_ch, keep, tid);
    load_query_rows_kept(qf, p, bg, rowblk, lane, half, lds_ch, n_kept, lds_q[wave]);
#pragma unroll
    for (int e = 0; e < 8; ++e) choff.off[e] = 2 * lds_ch[(tid & 7) * 8 + e];
  } else if constexpr (QLDS) {
    load_query_rows<T, D>(qf, p, bg, rowblk, lane, half, keep, lds_q[wave]);
  } else {
    load_query<T, D>(qf, p, bg, rowblk + col, half, keep);
  }
  float nb[16];
  if (p.lse_from_part) neg_lse_from_part(nb, p, bg, rowblk, lane, half);
  else load_neg_lse(nb, p, bg, rowblk, half);

  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) + bg * (size_t)p.S * GL::ROWB;
  auto mfma = [&](const Frag<T, DC>& kf) { return mma_block<T, DC>(qf, kf); };
  auto epi = [&](f32x16_t& a, int t, int kb, bool masked) {
    float cs[4];
    if (masked) {
      const int key = key0 + t * TK + kb * 32 + col;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = rowblk + acc_row(v, lane);
        const int i = (r < p.R) ? (r % p.w) : 0;
        const float e = fast_exp2(fmaf(a[v], p.c, nb[v]));
        const float x = (!p.causal || key <= p.S - p.w + i) ? e : 0.0f;
        cs[v & 3] = v < 4 ? x : cs[v & 3] + x;
      }
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) cs[v] = fast_exp2(fmaf(a[v], p.c, nb[v]));
#pragma unroll
      for (int v = 4; v < 16; ++v) cs[v & 3] += fast_exp2(fmaf(a[v], p.c, nb[v]));
    }
    // both lane halves publish their partial (16 of the 32 rows each)
    lds_red[t % 3][2 * wave + half][kb * 32 + col] = (cs[0] + cs[1]) + (cs[2] + cs[3]);
  };
  // after the barrier ending tile t: add the partials of every wave and lane half
  // in a fixed order; holes score 0
  auto post = [&](int t) {
    if (tid < TK) {
      const int key = key0 + t * TK + tid;
      if (key < key1) {
        float s = 0.0f;
#pragma unroll
        for (int h = 0; h < 2 * NW; ++h) s += lds_red[t % 3][h][tid];
        if (has_valid && !lds_valid[t % 3][tid]) s = 0.0f;
        s *= p.out_scale;
        float* dst = p.scores + bg * p.S + key;
        *dst = p.accumulate ? *dst + s : s;
      }
    }
  };
  if constexpr (GATHER)
    stream_blocks_kept<NW, SHORT, kScoresCpol>(kbase, vrow, key0, key1, ntiles, has_valid, tid, col, half, p.S, p.w,
                                               p.causal, lds_raw, lds_rv, lds_k, lds_valid, choff, mfma, epi, post);
  else
    stream_blocks<T, D, NW, SHORT, kScoresCpol>(kbase, vrow, key0, key1, ntiles, has_valid, tid, col, half, p.S, p.w,
                                                p.causal, lds_k, lds_valid, mfma, epi, post);
}

// ---------------------------------------------------------------------------
// One-wave kernels (at most 32 rows): two-stage staging, block by block
// ---------------------------------------------------------------------------
constexpr int kWaveTK = 64;

template <typename T, int D, bool STORE>
__global__ __launch_bounds__(64) void ws_stats_wave_kernel(WsParams p) {
  using G_ = TileGeom<T, D>;
  constexpr int TK = kWaveTK, KB = TK / 32;
  __shared__ __attribute__((aligned(16))) unsigned char lds_k[2][TK * G_::LSTRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_valid[2][TK];
  __shared__ uint32_t lds_keep[D / 32];

  const int tid = threadIdx.x, lane = tid, half = lane >> 5, col = lane & 31;
  const int chunk = blockIdx.x;
  const size_t bg = (size_t)blockIdx.z * p.Hkv + blockIdx.y;
  const int key0 = chunk * p.CH;
  const int key1 = min(p.S, key0 + p.CH);
  const int ntiles = (key1 - key0 + TK - 1) / TK;
  const bool has_valid = p.valid != nullptr;
  const uint8_t* vrow = has_valid ? p.valid + bg * p.S : nullptr;

  const uint32_t* keep = build_keep<D, 64>(lds_keep, p, bg, tid);
  const int r = col;
  Frag<T, D> qf;
  load_query<T, D>(qf, p, bg, r, half, keep);
  int lim = p.S - 1;
  if (p.causal && r < p.R) lim = min(p.S - 1, p.S - p.w + r % p.w);
  float m_run = kNegInf, z_run = 0.0f;

  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) + bg * (size_t)p.S * G_::ROWB;
  Stager<T, D, 64, TK> stg;
  if (ntiles > 0) {
    stg.load(kbase, vrow, key0, key1, tid);
    stg.store(lds_k[0], lds_valid[0], tid, has_valid);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int base = key0 + t * TK;
    if (t + 1 < ntiles) stg.load(kbase, vrow, base + TK, key1, tid);
    const bool masked = has_valid || (base + TK > p.S) || (p.causal && base + TK - 1 > p.S - p.w);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      Frag<T, D> kf;
      read_frag<T, D>(kf, lds_k[buf], kb * 32 + col, half);
      f32x16_t a = mma_block<T, D>(kf, qf);
      if (masked) mask_stats(a, base + kb * 32, lim, &lds_valid[buf][kb * 32], has_valid, half);
      if constexpr (STORE) {
        if (r < p.R) {
          float* dst = p.logits + (bg * p.R + r) * (size_t)p.Spad + base + kb * 32 + 4 * half;
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) {
            float4 o;
            o.x = a[4 * v4 + 0] * p.c;
            o.y = a[4 * v4 + 1] * p.c;
            o.z = a[4 * v4 + 2] * p.c;
            o.w = a[4 * v4 + 3] * p.c;
            *reinterpret_cast<float4*>(dst + 8 * v4) = o;
          }
        }
      }
      fold_stats(a, p.c, m_run, z_run);
    }
    if (t + 1 < ntiles) stg.store(lds_k[buf ^ 1], lds_valid[buf ^ 1], tid, has_valid);
    __syncthreads();
  }
  const float m2 = __shfl_xor(m_run, 32);
  const float z2 = __shfl_xor(z_run, 32);
  lse2_merge(m_run, z_run, m2, z2);
  if (half == 0) p.part[(size_t)chunk * p.rows_total + bg * p.Rpad + r] = make_float2(m_run, z_run);
}

template <typename T, int D>
__global__ __launch_bounds__(64) void ws_scores_wave_kernel(WsParams p) {
  using G_ = TileGeom<T, D>;
  constexpr int TK = kWaveTK, KB = TK / 32;
  __shared__ __attribute__((aligned(16))) unsigned char lds_k[2][TK * G_::LSTRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_valid[2][TK];
  __shared__ float lds_red[2][2][TK];
  __shared__ uint32_t lds_keep[D / 32];

  const int tid = threadIdx.x, lane = tid, half = lane >> 5, col = lane & 31;
  const int chunk = blockIdx.x;
  const size_t bg = (size_t)blockIdx.z * p.Hkv + blockIdx.y;
  const int key0 = chunk * p.CH;
  const int key1 = min(p.S, key0 + p.CH);
  const int ntiles = (key1 - key0 + TK - 1) / TK;
  const bool has_valid = p.valid != nullptr;
  const uint8_t* vrow = has_valid ? p.valid + bg * p.S : nullptr;

  const uint32_t* keep = build_keep<D, 64>(lds_keep, p, bg, tid);
  Frag<T, D> qf;
  load_query<T, D>(qf, p, bg, col, half, keep);
  float nb[16];
  if (p.lse_from_part) neg_lse_from_part(nb, p, bg, p.row0, lane, half);
  else load_neg_lse(nb, p, bg, 0, half);

  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) + bg * (size_t)p.S * G_::ROWB;
  Stager<T, D, 64, TK> stg;
  if (ntiles > 0) {
    stg.load(kbase, vrow, key0, key1, tid);
    stg.store(lds_k[0], lds_valid[0], tid, has_valid);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int base = key0 + t * TK;
    if (t + 1 < ntiles) stg.load(kbase, vrow, base + TK, key1, tid);
    const bool causal_tile = p.causal && base + TK - 1 > p.S - p.w;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      Frag<T, D> kf;
      read_frag<T, D>(kf, lds_k[buf], kb * 32 + col, half);
      f32x16_t a = mma_block<T, D>(qf, kf);
      float cs[4] = {0.f, 0.f, 0.f, 0.f};
      const int key = base + kb * 32 + col;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = fast_exp2(fmaf(a[v], p.c, nb[v]));
        const int rr = acc_row(v, lane);
        cs[v & 3] += (!causal_tile || rr >= p.R || key <= p.S - p.w + rr % p.w) ? e : 0.0f;
      }
      lds_red[buf][half][kb * 32 + col] = (cs[0] + cs[1]) + (cs[2] + cs[3]);
    }
    if (t + 1 < ntiles) stg.store(lds_k[buf ^ 1], lds_valid[buf ^ 1], tid, has_valid);
    __syncthreads();
    {
      const int key = base + tid;
      if (key < key1) {
        float s = lds_red[buf][0][tid] + lds_red[buf][1][tid];
        if (has_valid && !lds_valid[buf][tid]) s = 0.0f;
        p.scores[bg * p.S + key] = s * p.out_scale;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Stored-logits kernels (at most 16 rows per KV head: TOVA and decode steps)
//
// This path is bound by reading K once.  Four independent waves per workgroup
// stream interleaved 32-key blocks of a chunk.  A wave reads a block with
// coalesced 16-byte loads (each instruction covers 1 KB of consecutive rows),
// NBUF blocks ahead, and hands it to the MFMA fragment layout through its own
// padded LDS slot (the wave's LDS operations run in order, so no barrier is
// needed).  MFMA A = key block, B = query block, so the lane of column r holds
// 16 keys of row r: it keeps row r's running (max, sum of exp2) and writes the
// scaled logits of its keys.  The finish kernel merges the chunk statistics and
// reduces the normalised logits.
// ---------------------------------------------------------------------------
constexpr int kLogNW = 4;          // waves per workgroup
constexpr int kFinishRows = 1024;  // rows the finish kernel merges in LDS

// One 32-key block in coalesced order: unit u of the lane is the 16 bytes at
// offset u*1024 + lane*16 of the block; v is the validity byte of key lane%32.
template <typename T, int D>
struct KBlock {
  static constexpr int UPL = 32 * TileGeom<T, D>::ROWB / 16 / 64;  // units per lane
  u32x4_t d[UPL];
  uint8_t v;
};

template <typename T, int D>
struct LogitsNBUF {
  static constexpr int value = KBlock<T, D>::UPL <= 4 ? 3 : KBlock<T, D>::UPL <= 8 ? 2 : 1;
};

template <typename T, int D>
__global__ __launch_bounds__(kLogNW * 64) void ws_logits_kernel(WsParams p) {
  using G_ = TileGeom<T, D>;
  using KB = KBlock<T, D>;
  constexpr int NBUF = LogitsNBUF<T, D>::value;
  __shared__ uint32_t lds_keep[D / 32];
  __shared__ float2 lds_st[kLogNW][32];
  __shared__ __attribute__((aligned(16))) unsigned char lds_k[kLogNW][32 * G_::LSTRIDE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, col = lane & 31;
  const int chunk = blockIdx.x;
  const size_t bg = (size_t)blockIdx.z * p.Hkv + blockIdx.y;
  const int key0 = chunk * p.CH;
  const int key1 = min(p.S, key0 + p.CH);
  const int nblk = (key1 - key0 + 31) / 32;
  const int nb = nblk > wave ? (nblk - wave + kLogNW - 1) / kLogNW : 0;  // this wave's blocks
  const bool has_valid = p.valid != nullptr;
  const uint8_t* vrow = has_valid ? p.valid + bg * p.S : nullptr;

  const uint32_t* keep = build_keep<D, kLogNW * 64>(lds_keep, p, bg, tid);
  const int r = col;  // this lane's query row
  Frag<T, D> qf;
  load_query<T, D>(qf, p, bg, r, half, keep);
  int lim = p.S - 1;
  if (p.causal && r < p.R) lim = min(p.S - 1, p.S - p.w + r % p.w);
  float m_run = kNegInf, z_run = 0.0f;

  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) + bg * (size_t)p.S * G_::ROWB;
  unsigned char* slot = lds_k[wave];
  auto blk_key = [&](int i) { return key0 + (wave + i * kLogNW) * 32; };
  // Unconditional loads: rows past S read row S-1 instead (never used), and
  // without a validity mask the byte comes from the key data and is ignored.
  // The keys are read once, so the loads are non-temporal: the stream does not
  // push the logits, statistics and other streams' data out of the caches.
  auto load_blk = [&](KB& b, int i) {
    const int kb0 = blk_key(i);
#pragma unroll
    for (int u = 0; u < KB::UPL; ++u) {
      const int off = u * 1024 + lane * 16;
      const int key = min(kb0 + off / G_::ROWB, p.S - 1);
      b.d[u] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(kbase + (size_t)key * G_::ROWB + off % G_::ROWB));
    }
    const uint8_t* vsrc = vrow ? vrow : kbase;
    b.v = vsrc[min(kb0 + col, p.S - 1)];
  };
  auto process = [&](const KB& b, int i) {
    const int kb0 = blk_key(i);
    // coalesced units -> padded rows of the wave's LDS slot -> fragments
#pragma unroll
    for (int u = 0; u < KB::UPL; ++u) {
      const int off = u * 1024 + lane * 16;
      *reinterpret_cast<u32x4_t*>(slot + (off / G_::ROWB) * G_::LSTRIDE + off % G_::ROWB) = b.d[u];
    }
    __builtin_amdgcn_wave_barrier();
    Frag<T, D> kf;
    read_frag<T, D>(kf, slot, col, half);
    __builtin_amdgcn_wave_barrier();
    f32x16_t a = mma_block<T, D>(kf, qf);
    const bool masked = has_valid || kb0 + 32 > key1 || (p.causal && kb0 + 31 > p.S - p.w);
    if (masked) {
      const uint32_t vmask = has_valid ? (uint32_t)__ballot(b.v != 0) : 0xFFFFFFFFu;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = acc_row(v, lane);
        const bool ok = (kb0 + kk <= lim) & (kb0 + kk < key1) & (((vmask >> kk) & 1u) != 0u);
        a[v] = ok ? a[v] : kNegInf;
      }
    }
    if (r < p.R) {
      float* dst = p.logits + (bg * p.R + r) * (size_t)p.Spad + kb0 + 4 * half;
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        *reinterpret_cast<float4*>(dst + 8 * v4) =
            make_float4(a[4 * v4] * p.c, a[4 * v4 + 1] * p.c, a[4 * v4 + 2] * p.c, a[4 * v4 + 3] * p.c);
    }
    fold_stats(a, p.c, m_run, z_run);
  };

  KB kb[NBUF];
#pragma unroll
  for (int j = 0; j < NBUF; ++j) load_blk(kb[j], j);
  int i = 0;
  for (; i + 2 * NBUF <= nb; i += NBUF) {  // steady state: no conditional loads
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      process(kb[j], i + j);
      load_blk(kb[j], i + j + NBUF);
    }
  }
  for (; i < nb; i += NBUF) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      if (i + j < nb) {
        process(kb[j], i + j);
        if (i + j + NBUF < nb) load_blk(kb[j], i + j + NBUF);
      }
    }
  }

  // row statistics: lane halves, then the waves in order
  lse2_merge(m_run, z_run, __shfl_xor(m_run, 32), __shfl_xor(z_run, 32));
  if (half == 0) lds_st[wave][col] = make_float2(m_run, z_run);
  __syncthreads();
  if (tid < 32) {
    float m = lds_st[0][tid].x, z = lds_st[0][tid].y;
#pragma unroll
    for (int wv = 1; wv < kLogNW; ++wv) lse2_merge(m, z, lds_st[wv][tid].x, lds_st[wv][tid].y);
    p.part[(size_t)chunk * p.rows_total + bg * p.Rpad + tid] = make_float2(m, z);
  }
}

// Stored-logits finish: merge the chunk statistics of the rows needed (the R
// rows of one KV head, or of every KV head of the sequence for ALL_HEADS) into
// LDS, in chunk order, then s[b,g,j] = scale * sum over the rows of
// exp2(logit - lse2).  Rows with no allowed key contribute 0.
// Each thread owns KPT consecutive keys (one load per row: 16 bytes for GROUP,
// whose workgroups cover 1024 keys of one KV head; 4 bytes for ALL_HEADS, whose
// workgroups cover 256 keys and loop over the KV heads).  The logits of the
// first KV head are requested before the statistics are merged, and those of
// KV head g+1 while head g is summed, so a workgroup waits on memory about once
// per KV head instead of once per row.  RM: the rows per KV head rounded up to
// 4, 8 or 16 (R <= 16 on this path).
constexpr int kFinThreads = 256;

template <int KPT>
struct FinVec {
  float v[KPT];
};

template <int RM, int KPT>
__global__ __launch_bounds__(kFinThreads) void ws_finish_logits_kernel(WsParams p, int all_heads, float scale) {
  static_assert(KPT == 1 || KPT == 4, "one or four keys per thread");
  __shared__ float lds_lse[kFinishRows];
  const int b = blockIdx.z;
  const int g0 = all_heads ? 0 : blockIdx.y;
  const int ng = all_heads ? p.Hkv : 1;
  const int nrows = ng * p.R;
  const int j0 = (blockIdx.x * kFinThreads + threadIdx.x) * KPT;
  // j0 < S <= Spad and both are multiples of KPT, so the row's load stays inside
  // the padded logits row (values past S are never stored)
  const bool live = j0 < p.S;

  auto load_head = [&](FinVec<KPT> (&lg)[RM], int gi) {
    const float* src = p.logits + (((size_t)b * p.Hkv + g0 + gi) * p.R) * (size_t)p.Spad + j0;
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (live && r < p.R) {
        if constexpr (KPT == 4) {
          const float4 x = *reinterpret_cast<const float4*>(src + (size_t)r * p.Spad);
          lg[r].v[0] = x.x;
          lg[r].v[1] = x.y;
          lg[r].v[2] = x.z;
          lg[r].v[3] = x.w;
        } else {
          lg[r].v[0] = src[(size_t)r * p.Spad];
        }
      }
    }
  };
  FinVec<KPT> lg[RM];
  load_head(lg, 0);

  for (int t = threadIdx.x; t < nrows; t += kFinThreads) {
    const int g = g0 + t / p.R, r = t % p.R;
    const size_t row = ((size_t)b * p.Hkv + g) * p.Rpad + r;
    float m = kNegInf, z = 0.0f;
#pragma unroll 8
    for (int c = 0; c < p.nchunks; ++c) {
      const float2 pc = p.part[(size_t)c * p.rows_total + row];
      lse2_merge(m, z, pc.x, pc.y);
    }
    lds_lse[t] = (m == kNegInf || !(z > 0.0f)) ? kPosInf : m + log2f(z);
  }
  __syncthreads();
  if (!live) return;

  float s[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) s[e] = 0.0f;
  for (int gi = 0; gi < ng; ++gi) {
    FinVec<KPT> nx[RM];
    if (gi + 1 < ng) load_head(nx, gi + 1);
    float sg[KPT];
#pragma unroll
    for (int e = 0; e < KPT; ++e) sg[e] = 0.0f;
#pragma unroll
    for (int r = 0; r < RM; ++r) {
      if (r < p.R) {
        const float l = lds_lse[gi * p.R + r];
#pragma unroll
        for (int e = 0; e < KPT; ++e) sg[e] += fast_exp2(lg[r].v[e] - l);
      }
    }
#pragma unroll
    for (int e = 0; e < KPT; ++e) s[e] += sg[e];
    if (gi + 1 < ng) {
#pragma unroll
      for (int r = 0; r < RM; ++r) lg[r] = nx[r];
    }
  }
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const int j = j0 + e;
    if (j >= p.S) break;
    const float v = s[e] * scale;
    if (all_heads) {
      for (int g = 0; g < p.Hkv; ++g) p.scores[((size_t)b * p.Hkv + g) * p.S + j] = v;
    } else {
      p.scores[((size_t)b * p.Hkv + g0) * p.S + j] = v;
    }
  }
}

// Per row: combine the chunk partials into lse2 = M + log2(sum over chunks of
// z_c * exp2(m_c - M)), M the largest chunk reference.  Eight lanes per row:
// lane j folds chunks j, j+8, ... (requested together, so a row costs one
// memory round trip for up to 32 chunks), then a butterfly over the eight lanes
// merges the lane results in a fixed order.  Rows past R (padding) and rows with
// no allowed key get +inf, so their probabilities are 0.

__global__ __launch_bounds__(256) void ws_merge_kernel(const float2* __restrict__ part, float* __restrict__ lse,
                                                       int rows_total, int Rpad, int R, int nchunks) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int row = gid / kMergeLanes, j = gid % kMergeLanes;
  const bool ok = row < rows_total;
  float m = kNegInf, z = 0.0f;
  for (int c0 = 0; c0 < nchunks; c0 += 4 * kMergeLanes) {
    float2 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + j + i * kMergeLanes;
      v[i] = (ok && c < nchunks) ? part[(size_t)c * rows_total + row] : make_float2(kNegInf, 0.0f);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) lse2_merge(m, z, v[i].x, v[i].y);
  }
#pragma unroll
  for (int off = 1; off < kMergeLanes; off <<= 1) {
    const float m2 = __shfl_xor(m, off), z2 = __shfl_xor(z, off);
    lse2_merge(m, z, m2, z2);  // commutative, so every lane of the row ends with the same value
  }
  if (!ok || j != 0) return;
  const int r = row % Rpad;
  lse[row] = (r >= R || m == kNegInf || !(z > 0.0f)) ? kPosInf : m + log2f(z);
}

// Stored-logits path: s[b,g,j] = scale * sum over the rows of exp2(logit - lse2).
__global__ void ws_from_logits_kernel(const float* __restrict__ logits, const float* __restrict__ lse,
                                      float* __restrict__ scores, int Hkv, int S, int Spad, int R, int Rpad,
                                      int all_heads, float scale) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= S) return;
  const int b = blockIdx.z;
  if (!all_heads) {
    const size_t bg = (size_t)b * Hkv + blockIdx.y;
    float s = 0.0f;
    for (int r = 0; r < R; ++r) s += fast_exp2(logits[(bg * R + r) * Spad + j] - lse[bg * Rpad + r]);
    scores[bg * S + j] = s * scale;
  } else {
    float s = 0.0f;
    for (int g = 0; g < Hkv; ++g) {
      const size_t bg = (size_t)b * Hkv + g;
      float sg = 0.0f;
      for (int r = 0; r < R; ++r) sg += fast_exp2(logits[(bg * R + r) * Spad + j] - lse[bg * Rpad + r]);
      s += sg;
    }
    s *= scale;
    for (int g = 0; g < Hkv; ++g) scores[((size_t)b * Hkv + g) * S + j] = s;
  }
}

// TOVA on the two-pass path: scores hold per-KV-head sums; replace every KV
// head's entry by the scaled sum over the KV heads.
__global__ void ws_all_heads_kernel(float* __restrict__ scores, int Hkv, int S, float scale) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= S) return;
  const size_t b = blockIdx.z;
  float s = 0.0f;
  for (int g = 0; g < Hkv; ++g) s += scores[(b * Hkv + g) * S + j];
  s *= scale;
  for (int g = 0; g < Hkv; ++g) scores[(b * Hkv + g) * S + j] = s;
}

// GATHER: the stream kernels on ThinK's kept channels (bf16, D = 128, at most 64
// kept); the one-wave kernels keep the masked 128-channel contraction.
template <typename T, int D, bool GATHER = false>
void launch_pass(const WsParams& p, const WsPlan& plan, dim3 grid, hipStream_t st, bool scores_pass) {
  switch (plan.NW) {
    case 1:
      if (scores_pass) ws_scores_wave_kernel<T, D><<<grid, 64, 0, st>>>(p);
      else if (plan.store) ws_stats_wave_kernel<T, D, true><<<grid, 64, 0, st>>>(p);
      else ws_stats_wave_kernel<T, D, false><<<grid, 64, 0, st>>>(p);
      break;
    case 2:
      if (scores_pass) ws_scores_stream_kernel<T, D, 2, false, GATHER><<<grid, 128, 0, st>>>(p);
      else ws_stats_stream_kernel<T, D, 2, false, GATHER><<<grid, 128, 0, st>>>(p);
      break;
    case 4:
      if (scores_pass) ws_scores_stream_kernel<T, D, 4, false, GATHER><<<grid, 256, 0, st>>>(p);
      else ws_stats_stream_kernel<T, D, 4, false, GATHER><<<grid, 256, 0, st>>>(p);
      break;
    default:
      // eight waves (never for fp32 rows of 128 channels: ws_max_waves): the
      // staging depth follows the number of tiles per workgroup
      if constexpr (!(sizeof(T) == 4 && D == 128)) {
        if (plan.CH <= kShortChunkTiles * StreamTK<T, D, 8>::value) {
          if (scores_pass) ws_scores_stream_kernel<T, D, 8, true, GATHER><<<grid, 512, 0, st>>>(p);
          else ws_stats_stream_kernel<T, D, 8, true, GATHER><<<grid, 512, 0, st>>>(p);
        } else {
          if (scores_pass) ws_scores_stream_kernel<T, D, 8, false, GATHER><<<grid, 512, 0, st>>>(p);
          else ws_stats_stream_kernel<T, D, 8, false, GATHER><<<grid, 512, 0, st>>>(p);
        }
      }
      break;
  }
}

}  // namespace

hipError_t launch_window_scores(const WsArgs& a, const WsPlan& plan, hipStream_t st) {
  WsParams p;
  p.q = a.q;
  p.k = a.k;
  p.valid = a.valid;
  p.chan_idx = a.chan_idx;
  p.Hkv = a.Hkv;
  p.S = a.S;
  p.w = a.w;
  p.R = plan.R;
  p.Rpad = plan.Rpad;
  p.d_keep = a.d_keep;
  p.causal = (a.causal && a.w > 1) ? 1 : 0;
  p.CH = plan.CH;
  p.nchunks = plan.nchunks;
  p.Spad = plan.Spad;
  p.rows_total = a.B * a.Hkv * plan.Rpad;
  p.row0 = 0;
  p.accumulate = 0;
  p.lse_from_part = 0;
  p.c = kLog2e / sqrtf((float)a.D);
  const int G = a.H / a.Hkv;
  p.out_scale = a.reduce ? 1.0f : 1.0f / (float)(G * a.w);
  unsigned char* ws = static_cast<unsigned char*>(a.ws);
  p.part = reinterpret_cast<float2*>(ws + plan.off_part);
  p.lse = reinterpret_cast<float*>(ws + plan.off_lse);
  p.logits = reinterpret_cast<float*>(ws + plan.off_logits);
  p.scores = a.scores;

  const dim3 grid(plan.nchunks, a.Hkv, a.B);
  const bool bf = a.bf16 != 0;
  // ThinK with at most 64 kept channels: contract on the kept channels only
  const bool gather = bf && a.D == 128 && a.chan_idx != nullptr && a.d_keep <= 64;
  auto run = [&](bool scores_pass) {
    if (gather) launch_pass<__bf16, 128, true>(p, plan, grid, st, scores_pass);
    else if (bf && a.D == 128) launch_pass<__bf16, 128>(p, plan, grid, st, scores_pass);
    else if (bf && a.D == 64) launch_pass<__bf16, 64>(p, plan, grid, st, scores_pass);
    else if (!bf && a.D == 128) launch_pass<float, 128>(p, plan, grid, st, scores_pass);
    else launch_pass<float, 64>(p, plan, grid, st, scores_pass);
  };
  const int rows_per_launch = plan.NW * 32;

  if (plan.store && (!a.reduce || a.Hkv * plan.R <= kFinishRows)) {
    // stored-logits path: one launch writes the logits and the chunk statistics,
    // one launch merges them and reduces
    if (bf && a.D == 128) ws_logits_kernel<__bf16, 128><<<grid, kLogNW * 64, 0, st>>>(p);
    else if (bf) ws_logits_kernel<__bf16, 64><<<grid, kLogNW * 64, 0, st>>>(p);
    else if (a.D == 128) ws_logits_kernel<float, 128><<<grid, kLogNW * 64, 0, st>>>(p);
    else ws_logits_kernel<float, 64><<<grid, kLogNW * 64, 0, st>>>(p);
    const int all = a.reduce ? 1 : 0;
    const float fscale = all ? 1.0f / (float)(a.H * a.w) : p.out_scale;
    if (all) {
      const dim3 g2((a.S + kFinThreads - 1) / kFinThreads, 1, a.B);
      if (plan.R <= 4) ws_finish_logits_kernel<4, 1><<<g2, kFinThreads, 0, st>>>(p, all, fscale);
      else if (plan.R <= 8) ws_finish_logits_kernel<8, 1><<<g2, kFinThreads, 0, st>>>(p, all, fscale);
      else ws_finish_logits_kernel<16, 1><<<g2, kFinThreads, 0, st>>>(p, all, fscale);
    } else {
      const dim3 g2((a.S + 4 * kFinThreads - 1) / (4 * kFinThreads), a.Hkv, a.B);
      if (plan.R <= 4) ws_finish_logits_kernel<4, 4><<<g2, kFinThreads, 0, st>>>(p, all, fscale);
      else if (plan.R <= 8) ws_finish_logits_kernel<8, 4><<<g2, kFinThreads, 0, st>>>(p, all, fscale);
      else ws_finish_logits_kernel<16, 4><<<g2, kFinThreads, 0, st>>>(p, all, fscale);
    }
    return hipGetLastError();
  }
  for (int c = 0; c < plan.nrch; ++c) {  // row statistics
    p.row0 = c * rows_per_launch;
    run(false);
  }
  // the scores passes merge the row statistics themselves; the stored-logits
  // path's reduction kernel reads the merged normalisers
  p.lse_from_part = plan.store ? 0 : 1;
  if (plan.store)
    ws_merge_kernel<<<(p.rows_total * kMergeLanes + 255) / 256, 256, 0, st>>>(p.part, p.lse, p.rows_total,
                                                                              plan.Rpad, plan.R, plan.nchunks);
  const float scale_all = 1.0f / (float)(a.H * a.w);
  if (plan.store) {
    const dim3 g2((a.S + 255) / 256, a.reduce ? 1 : a.Hkv, a.B);
    ws_from_logits_kernel<<<g2, 256, 0, st>>>(p.logits, p.lse, p.scores, a.Hkv, a.S, plan.Spad, plan.R, plan.Rpad,
                                              a.reduce, a.reduce ? scale_all : p.out_scale);
  } else {
    for (int c = 0; c < plan.nrch; ++c) {  // scores, row chunk by row chunk
      p.row0 = c * rows_per_launch;
      p.accumulate = c > 0;
      run(true);
    }
    if (a.reduce) {
      const dim3 g3((a.S + 255) / 256, 1, a.B);
      ws_all_heads_kernel<<<g3, 256, 0, st>>>(p.scores, a.Hkv, a.S, scale_all);
    }
  }
  return hipGetLastError();
}

}  // namespace kvc
