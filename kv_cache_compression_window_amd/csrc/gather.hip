// Gather-compact of the kept K/V rows (gfx950).
//
// k_out[b,g,r,:] = k[b,g,idx[b,g,r],:] with the unkept key channels written as
// +0.0, and v_out likewise without channel pruning.  Source: "Add ThinK_Press"
// (kvpress PR 18), option 3a: put zeros in the key cache.
//
// A thread moves one 16-byte unit (four in mid-sized gathers) of the kept rows of K
// and the same units of V (V only when k is NULL: the kept-channel key cache is
// then written by the channel gathers).
// Consecutive threads cover consecutive units of a row, so every kept row is
// read as whole 128-byte lines and the output is written densely.  Output
// stores are non-temporal: the compacted cache is not read again by this layer.
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {

namespace {

constexpr int NTH = 256;

// UT 16-byte units per thread (UT rows' worth of the thread's unit column):
// every index is requested first, then every K and V load, then the stores, so a
// thread has 2*UT loads in flight.  Mid-sized gathers take UT = 4 (a quarter of
// the workgroups, which then share the GPU better with other streams' kernels);
// large and tiny ones UT = 1.
template <int ESZ, int D, int UT>
__global__ __launch_bounds__(NTH) void gather_kernel(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                                     const int32_t* __restrict__ idx, int S, int n_keep,
                                                     const int32_t* __restrict__ chan_idx, int d_keep,
                                                     uint4* __restrict__ k_out, uint4* __restrict__ v_out,
                                                     int Hkv) {
  constexpr int UPR = D * ESZ / 16;  // 16-byte units per row
  constexpr int EPU = 16 / ESZ;      // elements per unit
  static_assert(NTH % UPR == 0, "a thread keeps its unit column");
  __shared__ uint32_t keep[D / 32];
  const size_t bg = (size_t)blockIdx.z * Hkv + blockIdx.y;
  const int tid = threadIdx.x;
  if (chan_idx) {
    if (tid < D / 32) keep[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < d_keep; i += NTH) {
      const int ch = chan_idx[bg * d_keep + i];
      if (ch >= 0 && ch < D) atomicOr(&keep[ch >> 5], 1u << (ch & 31));
    }
    __syncthreads();
  }
  const int cu = tid % UPR;
  size_t in_off[UT], out_off[UT];
  bool ok[UT];
#pragma unroll
  for (int j = 0; j < UT; ++j) {
    const long long u = ((long long)blockIdx.x * UT + j) * NTH + tid;
    const int r = (int)(u / UPR);
    ok[j] = r < n_keep;
    // indices are caller data: clamp so that a bad index cannot read out of bounds
    const int src = ok[j] ? min(max(idx[bg * n_keep + r], 0), S - 1) : 0;
    in_off[j] = (bg * S + src) * UPR + cu;
    out_off[j] = (bg * n_keep + (ok[j] ? r : 0)) * UPR + cu;
  }
  uint4 vv[UT], kk[UT];
#pragma unroll
  for (int j = 0; j < UT; ++j) {
    if (v && ok[j]) vv[j] = v[in_off[j]];
    if (k && ok[j]) kk[j] = k[in_off[j]];
  }
#pragma unroll
  for (int j = 0; j < UT; ++j) {
    if (!ok[j]) continue;
    if (v) {
      __builtin_nontemporal_store(vv[j].x, &v_out[out_off[j]].x);
      __builtin_nontemporal_store(vv[j].y, &v_out[out_off[j]].y);
      __builtin_nontemporal_store(vv[j].z, &v_out[out_off[j]].z);
      __builtin_nontemporal_store(vv[j].w, &v_out[out_off[j]].w);
    }
    if (!k) continue;  // V only
    uint4 kv = kk[j];
    if (chan_idx) {
      uint32_t w[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        const int d = cu * EPU + e;
        if (!((keep[d >> 5] >> (d & 31)) & 1u)) {
          if constexpr (ESZ == 4) {
            w[e] = 0u;
          } else {
            w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
          }
        }
      }
      kv = make_uint4(w[0], w[1], w[2], w[3]);
    }
    __builtin_nontemporal_store(kv.x, &k_out[out_off[j]].x);
    __builtin_nontemporal_store(kv.y, &k_out[out_off[j]].y);
    __builtin_nontemporal_store(kv.z, &k_out[out_off[j]].z);
    __builtin_nontemporal_store(kv.w, &k_out[out_off[j]].w);
  }
}

// Gathers of 2^18 to 2^20 16-byte units per call take four units per thread
// (still 256 or more workgroups); smaller ones keep one, for parallelism.
constexpr long long kFourUnitsMin = 1LL << 18;
constexpr long long kFourUnitsMax = 1LL << 20;

template <int ESZ, int D>
void run(const GatherArgs& a, hipStream_t st) {
  constexpr int UPR = D * ESZ / 16;
  const long long units = (long long)a.n_keep * UPR;
  const auto* k = static_cast<const uint4*>(a.k);
  const auto* v = static_cast<const uint4*>(a.v);
  auto* ko = static_cast<uint4*>(a.k_out);
  auto* vo = static_cast<uint4*>(a.v_out);
  const long long total = units * a.Hkv * a.B;
  if (total >= kFourUnitsMin && total <= kFourUnitsMax) {
    const dim3 grid((unsigned)((units + 4 * NTH - 1) / (4 * NTH)), a.Hkv, a.B);
    gather_kernel<ESZ, D, 4><<<grid, NTH, 0, st>>>(k, v, a.idx, a.S, a.n_keep, a.chan_idx, a.d_keep, ko, vo, a.Hkv);
  } else {
    const dim3 grid((unsigned)((units + NTH - 1) / NTH), a.Hkv, a.B);
    gather_kernel<ESZ, D, 1><<<grid, NTH, 0, st>>>(k, v, a.idx, a.S, a.n_keep, a.chan_idx, a.d_keep, ko, vo, a.Hkv);
  }
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, hipStream_t st) {
  if (a.bf16 && a.D == 128) run<2, 128>(a, st);
  else if (a.bf16) run<2, 64>(a, st);
  else if (a.D == 128) run<4, 128>(a, st);
  else run<4, 64>(a, st);
  return hipGetLastError();
}

}  // namespace kvc
