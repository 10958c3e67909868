// Key-channel compression for ThinK's stored cache (gfx950).
//
// Source: "Add ThinK_Press" (kvpress PR 18), review thread, the three storage
// options for pruned key channels: 3a writes zeros into the key cache (that is
// kvc_gather_compact with chan_idx); 3b stores only the kept channels and adds
// the zeros back when the cache is used; 3c stores only the kept channels and
// prunes the query the same way, so that q_c . k_c equals q . k with the pruned
// channels zeroed.  This file holds the three row-wise channel gathers those
// options need:
//   compress  out[g, r, j] = in[g, idx[g, r], chan[g, j]]      (kept rows, kept channels)
//   queries   out[g, r, j] = in[g, r, chan[map(g), j]]          (g a query head, map(g) its KV head)
//   expand    out[g, r, c] = in[g, r, j] where chan[g, j] == c, else +0.0
// All three move bits: no arithmetic on the values.
//
// One wave per output row, one lane per output channel (two for 128 channels);
// the channel map of the block's group is built once in LDS.  A block holds
// four waves and covers 32 rows of one group.
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {

namespace {

constexpr int NTH = 256;
constexpr int ROWS_PER_BLOCK = 32;
constexpr int MAXC = 128;  // channels per row, at most

template <typename E>
__global__ __launch_bounds__(NTH) void chan_rows_kernel(ChanRowsArgs a) {
  __shared__ int smap[MAXC];  // source channel of each output channel (-1: write zero)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t g = blockIdx.y;
  // channel row of this group: a query head maps to its KV head
  const size_t m = a.H ? (g / a.H) * a.Hkv + (g % a.H) / (a.H / a.Hkv) : g;
  const int32_t* chan = a.chan + m * a.d_keep;
  if (a.expand) {
    if (tid < a.out_ch) smap[tid] = -1;
    __syncthreads();
    // the largest j wins when an entry repeats (entries are meant distinct)
    for (int j = tid; j < a.d_keep; j += NTH) {
      const int c = chan[j];
      if (c >= 0 && c < a.out_ch) atomicMax(&smap[c], j);
    }
  } else {
    for (int j = tid; j < a.out_ch; j += NTH) {
      const int c = chan[j];
      smap[j] = (c >= 0 && c < a.in_ch) ? c : -1;
    }
  }
  __syncthreads();

  const E* in = static_cast<const E*>(a.in);
  E* out = static_cast<E*>(a.out);
  const int r_end = min(a.n_rows, (int)(blockIdx.x + 1) * ROWS_PER_BLOCK);
  for (int r = blockIdx.x * ROWS_PER_BLOCK + wave; r < r_end; r += NTH / 64) {
    // kept positions are caller data: clamp so that a bad index cannot read out of bounds
    const int src = a.idx ? min(max(a.idx[g * a.n_rows + r], 0), a.in_rows - 1) : r;
    const E* row_in = in + (g * a.in_rows + src) * a.in_ch;
    E* row_out = out + (g * a.n_rows + r) * a.out_ch;
#pragma unroll
    for (int h = 0; h < MAXC / 64; ++h) {
      const int c = lane + 64 * h;
      if (c < a.out_ch) {
        const int s = smap[c];
        row_out[c] = s >= 0 ? row_in[s] : E(0);
      }
    }
  }
}

}  // namespace

hipError_t launch_chan_rows(const ChanRowsArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.n_rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK), (unsigned)a.groups);
  if (a.esz == 2) chan_rows_kernel<uint16_t><<<grid, NTH, 0, st>>>(a);
  else chan_rows_kernel<uint32_t><<<grid, NTH, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvc
