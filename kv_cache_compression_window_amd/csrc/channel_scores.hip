// ThinK per-channel key scores (gfx950).
//
// chan_scores[b,g,d] = (sum over the group's query heads and window rows of q^2)
//                    * (sum over all S keys of k^2).
// Source: "Add ThinK_Press" (kvpress PR 18): the factorised score
// query_norm * key_norm, shape (bsz, heads, head_dim).  It equals the squared
// and summed channel_attn, so that tensor is never materialised.
//
// Kernel 1 streams K once: every workgroup sums k^2 over a chunk of keys of one
// (b, g).  The threads' partial sums are added in a fixed order through LDS.
// Kernel 2 adds the chunk partials and the query squares in a fixed order and
// multiplies them.  There are no float atomics, so the result is deterministic.
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {

namespace {

constexpr int NTH = 256;

template <typename T>
__device__ inline void unit_squares(const uint4& u, float* out);

template <>
__device__ inline void unit_squares<__bf16>(const uint4& u, float* out) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(w[i] << 16);
    const float hi = __uint_as_float(w[i] & 0xFFFF0000u);
    out[2 * i] = lo * lo;
    out[2 * i + 1] = hi * hi;
  }
}

template <>
__device__ inline void unit_squares<float>(const uint4& u, float* out) {
  const float f[4] = {__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)};
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = f[i] * f[i];
}

template <typename T, int D>
__global__ __launch_bounds__(NTH) void key_sq_partial_kernel(const uint4* __restrict__ k, int S, int CH, int nchunks,
                                                              int Hkv, float* __restrict__ part) {
  constexpr int E = sizeof(T);
  constexpr int UPR = D * E / 16;   // units per key row
  constexpr int EPU = 16 / E;       // elements per unit
  constexpr int RL = NTH / UPR;     // rows handled in parallel
  __shared__ float red[RL][D + 1];
  const size_t bg = (size_t)blockIdx.z * Hkv + blockIdx.y;
  const int chunk = blockIdx.x;
  const int key0 = chunk * CH, key1 = min(S, key0 + CH);
  const int tid = threadIdx.x;
  const int cu = tid % UPR, rl = tid / UPR;
  float acc[EPU];
#pragma unroll
  for (int e = 0; e < EPU; ++e) acc[e] = 0.0f;
  const uint4* base = k + bg * (size_t)S * UPR + cu;
  int j = key0 + rl;
  for (; j + 3 * RL < key1; j += 4 * RL) {
    uint4 x[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = base[(size_t)(j + q * RL) * UPR];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float sq[EPU];
      unit_squares<T>(x[q], sq);
#pragma unroll
      for (int e = 0; e < EPU; ++e) acc[e] += sq[e];
    }
  }
  for (; j < key1; j += RL) {
    float sq[EPU];
    unit_squares<T>(base[(size_t)j * UPR], sq);
#pragma unroll
    for (int e = 0; e < EPU; ++e) acc[e] += sq[e];
  }
#pragma unroll
  for (int e = 0; e < EPU; ++e) red[rl][cu * EPU + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.0f;
    for (int r = 0; r < RL; ++r) s += red[r][tid];
    part[(bg * nchunks + chunk) * D + tid] = s;
  }
}

// One workgroup per (b, g): thread (slice s, channel d) adds the chunks and
// query rows congruent to s modulo FS with up to 16 loads in flight, then the
// FS slices are added in slice order.
constexpr int FTH = 1024;

template <typename T, int D>
__global__ __launch_bounds__(FTH) void channel_finish_kernel(const float* __restrict__ part, int nchunks,
                                                             const T* __restrict__ q, int R, float* __restrict__ out) {
  constexpr int FS = FTH / D;
  __shared__ float red_k[FS][D], red_q[FS][D];
  const size_t bg = blockIdx.x;
  const int d = threadIdx.x % D, sl = threadIdx.x / D;
  float ks = 0.0f;
#pragma unroll 16
  for (int c = sl; c < nchunks; c += FS) ks += part[(bg * nchunks + c) * D + d];
  float qs = 0.0f;
#pragma unroll 16
  for (int r = sl; r < R; r += FS) {
    const float x = (float)q[(bg * R + r) * D + d];
    qs += x * x;
  }
  red_k[sl][d] = ks;
  red_q[sl][d] = qs;
  __syncthreads();
  if (sl == 0) {
    float k2 = 0.0f, q2 = 0.0f;
#pragma unroll
    for (int i = 0; i < FS; ++i) {
      k2 += red_k[i][d];
      q2 += red_q[i][d];
    }
    out[bg * D + d] = q2 * k2;
  }
}

template <typename T, int D>
void run(const CsArgs& a, const CsPlan& plan, hipStream_t st) {
  float* part = static_cast<float*>(a.ws);
  const dim3 grid(plan.nchunks, a.Hkv, a.B);
  key_sq_partial_kernel<T, D><<<grid, NTH, 0, st>>>(static_cast<const uint4*>(a.k), a.S, plan.CH, plan.nchunks,
                                                    a.Hkv, part);
  const int R = (a.H / a.Hkv) * a.w;
  channel_finish_kernel<T, D><<<a.B * a.Hkv, FTH, 0, st>>>(part, plan.nchunks, static_cast<const T*>(a.q), R, a.out);
}

}  // namespace

hipError_t launch_channel_scores(const CsArgs& a, const CsPlan& plan, hipStream_t st) {
  if (a.bf16 && a.D == 128) run<__bf16, 128>(a, plan, st);
  else if (a.bf16) run<__bf16, 64>(a, plan, st);
  else if (a.D == 128) run<float, 128>(a, plan, st);
  else run<float, 64>(a, plan, st);
  return hipGetLastError();
}

}  // namespace kvc
