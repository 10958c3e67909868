// Hardware ceilings measured next to the path by bench.py (libkvc_bench.so,
// not part of libkvc): the rate of a plain streaming read from HBM and the rate
// of v_exp_f32.  Neither computes anything of the method.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Every 16-byte unit of the buffer is read once (four independent loads in
// flight per thread); one word per thread is written so the loads stay.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src, size_t n16,
                                                          unsigned* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4_t a = {0u, 0u, 0u, 0u}, b = a, c = a, d = a;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    a ^= __builtin_nontemporal_load(src + i);
    b ^= __builtin_nontemporal_load(src + i + stride);
    c ^= __builtin_nontemporal_load(src + i + 2 * stride);
    d ^= __builtin_nontemporal_load(src + i + 3 * stride);
  }
  for (; i < n16; i += stride) a ^= __builtin_nontemporal_load(src + i);
  const u32x4_t s = a ^ b ^ c ^ d;
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s.x ^ s.y ^ s.z ^ s.w;
}

// Eight independent exp2 chains per thread, `iters` rounds.
__global__ __launch_bounds__(512) void exp_rate_kernel(float* __restrict__ out, int iters) {
  float a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = 0.01f * j + 1e-6f * threadIdx.x;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = __builtin_amdgcn_exp2f(-a[j]);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += a[j];
  out[(size_t)blockIdx.x * 512 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, 16-byte aligned) from `buf`; `out` holds
// blocks*256 words.  Returns 0 or the launch error.
int kvc_bench_stream_read(const void* buf, size_t bytes, unsigned* out, int blocks, hipStream_t stream) {
  stream_read_kernel<<<blocks, 256, 0, stream>>>(static_cast<const u32x4_t*>(buf), bytes / 16, out);
  return (int)hipGetLastError();
}

// 8 * iters exp2 per thread over blocks x 512 threads; `out` holds blocks*512 floats.
int kvc_bench_exp_rate(float* out, int blocks, int iters, hipStream_t stream) {
  exp_rate_kernel<<<blocks, 512, 0, stream>>>(out, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
