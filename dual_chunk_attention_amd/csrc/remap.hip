// Position remap and regime key intervals.
// DCA feature page, "Section C design" table (keys at j mod c; intra query at i mod c; succ query
// at (i mod c) + c) with this library's readings: the inter query is clamped to c - 1 and succ
// holds only previous-chunk keys closer than c.  The page-literal modes follow the table as
// printed (succ = the whole previous chunk, inter = older chunks with the query at c) or put the
// inter query at 2c (Upstream Sync page, entry "opencoti F5 dca").  The Upstream Sync page ("opencoti F5 dca")
// fills positions densely and leaves masks NULL for contiguous caches; here the masks become one
// inclusive key interval per (row, regime):
//   intra [c*q(i), i],  succ [i-c+1, c*q(i)-1],  inter [0, i-c]          (baseline)
//   intra [c*q(i), i],  succ [c*(q(i)-1), c*q(i)-1],  inter [0, c*(q(i)-1)-1]   (page modes)
// each clipped to [0, min(i, n_kv-1)].
#include "common.h"

namespace dca {
namespace {

__global__ void remap_kernel(const int32_t* __restrict__ q_pos, int64_t rows, int32_t chunk,
                             int32_t mode, int32_t n_kv, int32_t* __restrict__ pos_q,
                             int32_t* __restrict__ pos_k, int32_t* __restrict__ bounds) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < rows; x += stride) {
    const int64_t c = chunk;
    const int64_t i = q_pos[x];
    const int64_t ci = floordiv64(i, c);
    const int64_t loc = i - ci * c;
    if (pos_q) {
      pos_q[x] = (int32_t)loc;
      pos_q[rows + x] = (int32_t)(loc + c);
      pos_q[2 * rows + x] = (int32_t)(mode == 0 ? c - 1 : mode * c);
    }
    if (bounds) {
      const int64_t last = i < (int64_t)n_kv - 1 ? i : (int64_t)n_kv - 1;
      // page modes: succ = the whole previous chunk, inter = every older chunk
      const int64_t succ_lo = mode == 0 ? i - c + 1 : (ci - 1) * c;
      const int64_t inter_hi = mode == 0 ? i - c : (ci - 1) * c - 1;
      int64_t lo[3] = {ci * c, succ_lo, 0};
      int64_t hi[3] = {last, ci * c - 1, inter_hi};
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        int64_t a = lo[r] < 0 ? 0 : lo[r];
        int64_t b = hi[r] < last ? hi[r] : last;
        const bool empty = a > b;
        bounds[(r * rows + x) * 2 + 0] = empty ? 0 : (int32_t)a;
        bounds[(r * rows + x) * 2 + 1] = empty ? -1 : (int32_t)b;
      }
    }
  }
  if (pos_k) {
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n_kv; j += stride)
      pos_k[j] = (int32_t)(j % chunk);
  }
}

}  // namespace

hipError_t launch_remap(const int32_t* q_pos, int64_t rows, int32_t chunk, int32_t mode,
                        int32_t n_kv, int32_t* pos_q, int32_t* pos_k, int32_t* bounds,
                        hipStream_t stream) {
  int64_t work = rows > n_kv ? rows : n_kv;
  if (!pos_k) work = rows;
  if (work <= 0) return hipSuccess;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(remap_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, q_pos, rows,
                     chunk, mode, n_kv, pos_q, pos_k, bounds);
  return hipGetLastError();
}

}  // namespace dca
