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
// Kernels:
//   pass 1  MFMA A = key block (32 keys), B = query block (32 rows); each lane
//           holds 16 keys of one query row, so the per-row running max and
//           sum of exp2 stay in the lane.  It writes (max, sum) per row and chunk.
//           The stored-logits variant also writes the scaled logits.
//   merge   combines the chunk partials into a base-2 log-normaliser per row.
//   pass 2  MFMA A = query block, B = key block; each lane holds 16 rows of one
//           key, so the column sums of exp2(l*c - lse2) stay in the lane.  The
//           waves' sums are added in a fixed order in LDS and written as scores.
//   from_logits  (stored-logits path) normalises the stored logits and sums them.
//   all_heads    (TOVA) sums the group sums over the KV heads and repeats them.
// All sums are in a fixed order, so the results are deterministic.
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {

namespace {

constexpr int TK = kTileKeys;  // keys per tile
constexpr int KB = TK / 32;    // 32-key blocks per tile

enum { MODE_STATS = 0, MODE_STATS_STORE = 1, MODE_SCORES = 2 };

struct WsParams {
  const void* q;
  const void* k;
  const uint8_t* valid;
  const int32_t* chan_idx;
  int Hkv, S, w, R, Rpad, d_keep, causal, CH, nchunks, Spad;
  float c;            // log2(e) / sqrt(D)
  float out_scale;    // pass 2: 1/(G*w) for GROUP, 1 for ALL_HEADS (normalised later)
  float2* part;       // [B*Hkv*Rpad*nchunks] (max, sum of exp2) in base-2 units
  float* lse;         // [B*Hkv*Rpad] base-2 log-normaliser (+inf for empty/padded rows)
  float* logits;      // [B*Hkv*R*Spad] scaled logits (stored-logits path)
  float* scores;      // [B*Hkv*S]
};

template <typename T, int D>
struct TileGeom {
  static constexpr int E = sizeof(T);
  static constexpr int HALF = D / 2;               // channels per lane half
  static constexpr int NSTEP = HALF / Mfma<T>::KPL;  // MFMA steps per block
  static constexpr int ROWB = D * E;               // bytes per key row
  static constexpr int LSTRIDE = ROWB + 16;        // padded LDS row stride
  static constexpr int UPR = ROWB / 16;            // 16-byte units per row
  static constexpr int FRAGU = HALF * E / 16;      // 16-byte units per lane fragment
};

template <typename T, int D>
union Frag {
  uint4 u[TileGeom<T, D>::FRAGU];
  typename Mfma<T>::op_t o[TileGeom<T, D>::NSTEP];
};

template <typename T, int D, int NW, int RB, int MODE>
__global__ __launch_bounds__(NW * 64) void ws_pass_kernel(WsParams p) {
  using M = Mfma<T>;
  using G_ = TileGeom<T, D>;
  constexpr int NT = NW * 64;
  constexpr int UPT = TK * G_::UPR / NT;
  static_assert((TK * G_::UPR) % NT == 0, "tile units must split evenly");
  constexpr bool STATS = MODE != MODE_SCORES;

  __shared__ __attribute__((aligned(16))) unsigned char lds_k[2][TK * G_::LSTRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t lds_valid[2][TK];
  __shared__ float lds_red[2][NW][TK];
  __shared__ uint32_t lds_keep[D / 32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int chunk = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const size_t bg = (size_t)b * p.Hkv + g;
  const int key0 = chunk * p.CH;
  const int key1 = min(p.S, key0 + p.CH);
  const int ntiles = (key1 - key0 + TK - 1) / TK;
  const bool has_valid = p.valid != nullptr;

  // ---- kept key channels (ThinK) as a bit mask --------------------------------
  if (p.chan_idx) {
    if (tid < D / 32) lds_keep[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < p.d_keep; i += NT) {
      const int ch = p.chan_idx[bg * p.d_keep + i];
      if (ch >= 0 && ch < D) atomicOr(&lds_keep[ch >> 5], 1u << (ch & 31));
    }
    __syncthreads();
  }

  // ---- query fragments of this wave's row blocks (kept in registers) ----------
  Frag<T, D> qf[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = (wave * RB + rb) * 32 + col;
    if (r < p.R) {
      const uint4* src = reinterpret_cast<const uint4*>(
          reinterpret_cast<const unsigned char*>(p.q) + ((bg * p.R + r) * D + half * G_::HALF) * G_::E);
#pragma unroll
      for (int u = 0; u < G_::FRAGU; ++u) qf[rb].u[u] = src[u];
      if (p.chan_idx) {
#pragma unroll
        for (int s = 0; s < G_::NSTEP; ++s) {
#pragma unroll
          for (int e = 0; e < M::KPL; ++e) {
            const int d = half * G_::HALF + s * M::KPL + e;
            if (!((lds_keep[d >> 5] >> (d & 31)) & 1u)) {
              if constexpr (M::KPL == 1) qf[rb].o[s] = 0.0f;
              else qf[rb].o[s][e] = (__bf16)0.0f;
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < G_::FRAGU; ++u) qf[rb].u[u] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  // ---- per-lane state ----------------------------------------------------------
  float m_run[RB], z_run[RB];  // pass 1: running max (base-2 units) and sum of exp2
  int win_row[RB];             // pass 1: window row of this lane's query row
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = kNegInf;
    z_run[rb] = 0.0f;
    const int r = (wave * RB + rb) * 32 + col;
    win_row[rb] = (r < p.R) ? (r % p.w) : 0;
  }
  float nb[RB][16];  // pass 2: minus the log-normaliser of each accumulator row
  if constexpr (!STATS) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        nb[rb][v] = -p.lse[bg * p.Rpad + (wave * RB + rb) * 32 + acc_row(v, lane)];
  }

  // ---- tile loader: contiguous global rows -> padded LDS rows -------------------
  uint4 pre[UPT];
  uint8_t pre_valid = 0;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) + bg * (size_t)p.S * G_::ROWB;
  auto load_tile = [&](int t) {
    const int base = key0 + t * TK;
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      const int row = u / G_::UPR, cu = u % G_::UPR;
      const int key = base + row;
      if (key < key1)
        pre[i] = *reinterpret_cast<const uint4*>(kbase + (size_t)key * G_::ROWB + cu * 16);
      else
        pre[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (has_valid && tid < TK) {
      const int key = base + tid;
      pre_valid = (key < key1) ? p.valid[bg * p.S + key] : (uint8_t)0;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      const int row = u / G_::UPR, cu = u % G_::UPR;
      *reinterpret_cast<uint4*>(&lds_k[buf][row * G_::LSTRIDE + cu * 16]) = pre[i];
    }
    if (has_valid && tid < TK) lds_valid[buf][tid] = pre_valid;
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int base = key0 + t * TK;
    if (t + 1 < ntiles) load_tile(t + 1);
    // Masking is needed only on tiles with holes, a ragged end, or keys past the
    // causal limit of the first window row (S - w).
    const bool need_mask = has_valid || (base + TK > p.S) || (p.causal && p.w > 1 && base + TK - 1 > p.S - p.w);

    if constexpr (STATS) {
      f32x16_t acc[KB][RB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        Frag<T, D> kf;
        const unsigned char* rowp = &lds_k[buf][(kb * 32 + col) * G_::LSTRIDE + half * G_::HALF * G_::E];
#pragma unroll
        for (int u = 0; u < G_::FRAGU; ++u) kf.u[u] = reinterpret_cast<const uint4*>(rowp)[u];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          f32x16_t a = {};
#pragma unroll
          for (int s = 0; s < G_::NSTEP; ++s) a = M::run(kf.o[s], qf[rb].o[s], a);
          acc[kb][rb] = a;
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (need_mask) {
          // Branch-free: the keys of accumulator registers 4*v4 .. 4*v4+3 are four
          // consecutive keys, so their validity bytes come in one 32-bit LDS word.
          const int lim = min(p.S - 1, p.causal ? (p.S - p.w + win_row[rb]) : (p.S - 1));
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
              const int kk0 = kb * 32 + 8 * v4 + 4 * half;
              const uint32_t vw =
                  has_valid ? *reinterpret_cast<const uint32_t*>(&lds_valid[buf][kk0]) : 0x01010101u;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const bool ok = (base + kk0 + e <= lim) & (((vw >> (8 * e)) & 0xFFu) != 0u);
                acc[kb][rb][4 * v4 + e] = ok ? acc[kb][rb][4 * v4 + e] : kNegInf;
              }
            }
        }
        if constexpr (MODE == MODE_STATS_STORE) {
          const int r = (wave * RB + rb) * 32 + col;
          if (r < p.R) {
            float* dst = p.logits + (bg * p.R + r) * (size_t)p.Spad + base;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int v4 = 0; v4 < 4; ++v4) {
                float4 o;
                o.x = acc[kb][rb][4 * v4 + 0] * p.c;
                o.y = acc[kb][rb][4 * v4 + 1] * p.c;
                o.z = acc[kb][rb][4 * v4 + 2] * p.c;
                o.w = acc[kb][rb][4 * v4 + 3] * p.c;
                *reinterpret_cast<float4*>(dst + kb * 32 + 8 * v4 + 4 * half) = o;
              }
          }
        }
        float tmax = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, acc[kb][rb][v]);
        const float mn = fmaxf(m_run[rb], tmax * p.c);
        if (mn != kNegInf) {
          float zs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) zs[v & 3] += fast_exp2(fmaf(acc[kb][rb][v], p.c, -mn));
          z_run[rb] = z_run[rb] * fast_exp2(m_run[rb] - mn) + ((zs[0] + zs[1]) + (zs[2] + zs[3]));
          m_run[rb] = mn;
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        Frag<T, D> kf;
        const unsigned char* rowp = &lds_k[buf][(kb * 32 + col) * G_::LSTRIDE + half * G_::HALF * G_::E];
#pragma unroll
        for (int u = 0; u < G_::FRAGU; ++u) kf.u[u] = reinterpret_cast<const uint4*>(rowp)[u];
        float cs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          f32x16_t a = {};
#pragma unroll
          for (int s = 0; s < G_::NSTEP; ++s) a = M::run(qf[rb].o[s], kf.o[s], a);
          if (need_mask && p.causal && p.w > 1) {
            const int key = base + kb * 32 + col;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int r = (wave * RB + rb) * 32 + acc_row(v, lane);
              const int i = (r < p.R) ? (r % p.w) : 0;
              float e = fast_exp2(fmaf(a[v], p.c, nb[rb][v]));
              cs[v & 3] += (key <= p.S - p.w + i) ? e : 0.0f;
            }
          } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) cs[v & 3] += fast_exp2(fmaf(a[v], p.c, nb[rb][v]));
          }
        }
        float csum = (cs[0] + cs[1]) + (cs[2] + cs[3]);
        csum += __shfl_xor(csum, 32);
        if (has_valid && !lds_valid[buf][kb * 32 + col]) csum = 0.0f;
        if (half == 0) lds_red[buf][wave][kb * 32 + col] = csum;
      }
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();

    if constexpr (!STATS) {
      if (tid < TK) {
        const int key = base + tid;
        if (key < key1) {
          float s = 0.0f;
#pragma unroll
          for (int wv = 0; wv < NW; ++wv) s += lds_red[buf][wv][tid];
          p.scores[bg * p.S + key] = s * p.out_scale;
        }
      }
    }
  }

  if constexpr (STATS) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float m2 = __shfl_xor(m_run[rb], 32);
      const float z2 = __shfl_xor(z_run[rb], 32);
      lse2_merge(m_run[rb], z_run[rb], m2, z2);
      if (half == 0) {
        const int r = (wave * RB + rb) * 32 + col;
        p.part[(bg * p.Rpad + r) * p.nchunks + chunk] = make_float2(m_run[rb], z_run[rb]);
      }
    }
  }
}

// Per row: combine the chunk partials into lse2 = max + log2(sum).  Rows past R
// (padding) and rows with no allowed key get +inf, so their probabilities are 0.
__global__ void ws_merge_kernel(const float2* __restrict__ part, float* __restrict__ lse, int total,
                                int Rpad, int R, int nchunks) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int r = idx % Rpad;
  if (r >= R) {
    lse[idx] = kPosInf;
    return;
  }
  float m = kNegInf, z = 0.0f;
  for (int c = 0; c < nchunks; ++c) {
    const float2 pc = part[(size_t)idx * nchunks + c];
    lse2_merge(m, z, pc.x, pc.y);
  }
  lse[idx] = (m == kNegInf || !(z > 0.0f)) ? kPosInf : m + log2f(z);
}

// Stored-logits path: s[b,g,j] = scale * sum over the rows of exp2(logit - lse2).
__global__ void ws_from_logits_kernel(const float* __restrict__ logits, const float* __restrict__ lse,
                                      float* __restrict__ scores, int Hkv, int S, int Spad, int R,
                                      int Rpad, int all_heads, float scale) {
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

template <typename T, int D, int NW, int RB>
void launch_passes(const WsParams& p, const WsPlan& plan, dim3 grid, hipStream_t st) {
  if (plan.store) {
    if constexpr (NW == 1 && RB == 1) ws_pass_kernel<T, D, 1, 1, MODE_STATS_STORE><<<grid, 64, 0, st>>>(p);
  } else {
    ws_pass_kernel<T, D, NW, RB, MODE_STATS><<<grid, NW * 64, 0, st>>>(p);
  }
}

template <typename T, int D, int NW, int RB>
void launch_scores(const WsParams& p, dim3 grid, hipStream_t st) {
  ws_pass_kernel<T, D, NW, RB, MODE_SCORES><<<grid, NW * 64, 0, st>>>(p);
}

template <typename T, int D>
void dispatch(const WsParams& p, const WsPlan& plan, dim3 grid, hipStream_t st, bool scores_pass) {
  const int key = plan.NW * 10 + plan.RB;
#define KVC_WS_CASE(NW_, RB_)                                         \
  case NW_ * 10 + RB_:                                                \
    if (scores_pass) launch_scores<T, D, NW_, RB_>(p, grid, st);      \
    else launch_passes<T, D, NW_, RB_>(p, plan, grid, st);            \
    break;
  switch (key) {
    KVC_WS_CASE(1, 1)
    KVC_WS_CASE(2, 1)
    KVC_WS_CASE(4, 1)
    KVC_WS_CASE(4, 2)
    KVC_WS_CASE(4, 4)
    default: break;
  }
#undef KVC_WS_CASE
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
  auto run = [&](bool scores_pass) {
    if (bf && a.D == 128) dispatch<__bf16, 128>(p, plan, grid, st, scores_pass);
    else if (bf && a.D == 64) dispatch<__bf16, 64>(p, plan, grid, st, scores_pass);
    else if (!bf && a.D == 128) dispatch<float, 128>(p, plan, grid, st, scores_pass);
    else dispatch<float, 64>(p, plan, grid, st, scores_pass);
  };

  run(false);  // pass 1
  const int total = a.B * a.Hkv * plan.Rpad;
  ws_merge_kernel<<<(total + 255) / 256, 256, 0, st>>>(p.part, p.lse, total, plan.Rpad, plan.R, plan.nchunks);
  const float scale_all = 1.0f / (float)(a.H * a.w);
  if (plan.store) {
    const dim3 g2((a.S + 255) / 256, a.reduce ? 1 : a.Hkv, a.B);
    ws_from_logits_kernel<<<g2, 256, 0, st>>>(p.logits, p.lse, p.scores, a.Hkv, a.S, plan.Spad, plan.R,
                                              plan.Rpad, a.reduce, a.reduce ? scale_all : p.out_scale);
  } else {
    run(true);  // pass 2
    if (a.reduce) {
      const dim3 g3((a.S + 255) / 256, 1, a.B);
      ws_all_heads_kernel<<<g3, 256, 0, st>>>(p.scores, a.Hkv, a.S, scale_all);
    }
  }
  return hipGetLastError();
}

}  // namespace kvc
