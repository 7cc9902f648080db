// Exact N-way LSE merge of normalised partials.
// DCA feature page, "Implementation progress + Section-D simplification": M = max_r lse_r,
// w_r = exp(lse_r - M), O = sum_r w_r O_r / sum_r w_r; "Section C2b": an empty part
// (lse = -inf) has weight exactly 0; Upstream Sync entry 0110: a zero weight sum gives 0.
// One wave per row; every lane owns D/64 columns.  The part loop reads lse_p once per lane
// (broadcast) and skips the O read of empty parts, so a -inf part's O is never touched.
#include "common.h"

namespace dca {
namespace {

__device__ __forceinline__ const float* part_o(const MergeArgs& a, int p, int64_t row) {
  return (a.strided ? a.o_base + (int64_t)p * a.o_part_stride : a.o_ptr[p]) + row * a.D;
}
__device__ __forceinline__ float part_lse(const MergeArgs& a, int p, int64_t row) {
  return (a.strided ? a.lse_base + (int64_t)p * a.lse_part_stride : a.lse_ptr[p])[row];
}

template <typename OutT>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  float M = -INFINITY;
  for (int p = lane; p < a.n_parts; p += 64) M = fmaxf(M, part_lse(a, p, row));
  M = wave_max(M);
  OutT* out = (OutT*)a.o_out + row * a.D;
  if (M == -INFINITY) {
    for (int d = lane; d < a.D; d += 64) out[d] = from_f32<OutT>(0.0f);
    if (a.lse_out && lane == 0) a.lse_out[row] = -INFINITY;
    return;
  }
  float W = 0.0f;
  for (int p = lane; p < a.n_parts; p += 64) {
    const float l = part_lse(a, p, row);
    if (l != -INFINITY) W += expf(l - M);
  }
  W = wave_sum(W);
  const float inv = 1.0f / W;
  float acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = 0.0f;
  for (int p = 0; p < a.n_parts; ++p) {
    const float l = part_lse(a, p, row);
    if (l == -INFINITY) continue;
    const float w = expf(l - M);
    const float* o = part_o(a, p, row);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int d = lane + 64 * k;
      if (d < a.D) acc[k] = fmaf(w, o[d], acc[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int d = lane + 64 * k;
    if (d < a.D) out[d] = from_f32<OutT>(acc[k] * inv);
  }
  if (a.lse_out && lane == 0) a.lse_out[row] = M + logf(W);
}

// Many parts per row (split-KV partials): one workgroup per (row, slice of 256 dims).  Non-empty
// parts are compacted in index order, split over the 4 waves (lane: 4 dims, 16-byte loads, four
// parts in flight), and the wave sums are added in a fixed order.
constexpr int kMaxManyParts = 2048;

template <typename OutT>
__global__ __launch_bounds__(256) void merge_many_kernel(MergeArgs a) {
  __shared__ float s_l[kMaxManyParts];
  __shared__ float s_w[kMaxManyParts];
  __shared__ int s_idx[kMaxManyParts];
  __shared__ float s_acc[3][256];
  __shared__ float s_M, s_W;
  __shared__ int s_cnt;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t row = blockIdx.x;
  for (int p = tid; p < a.n_parts; p += 256) s_l[p] = part_lse(a, p, row);
  __syncthreads();
  if (wv == 0) {
    float M = -INFINITY;
    for (int p = lane; p < a.n_parts; p += 64) M = fmaxf(M, s_l[p]);
    M = wave_max(M);
    int cnt = 0;
    float W = 0.0f;
    for (int p0 = 0; p0 < a.n_parts; p0 += 64) {
      const int p = p0 + lane;
      const float l = p < a.n_parts ? s_l[p] : -INFINITY;
      const bool ne = l != -INFINITY;
      const uint64_t m = __ballot(ne);
      const int before = __popcll(m & ((1ull << lane) - 1ull));
      if (ne) {
        const float wgt = expf(l - M);
        s_idx[cnt + before] = p;
        s_w[cnt + before] = wgt;
        W += wgt;
      }
      cnt += __popcll(m);
    }
    W = wave_sum(W);
    if (lane == 0) {
      s_M = M;
      s_W = W;
      s_cnt = cnt;
    }
  }
  __syncthreads();
  const int cnt = s_cnt;
  OutT* out = (OutT*)a.o_out + row * a.D;
  const int d = blockIdx.y * 256 + 4 * lane;   // the lane's 4 dims (D is a multiple of 4)
  const bool live = d < a.D;
  if (cnt == 0) {
    if (wv == 0 && live) {
#pragma unroll
      for (int k = 0; k < 4; ++k) out[d + k] = from_f32<OutT>(0.0f);
    }
    if (a.lse_out && blockIdx.y == 0 && tid == 0) a.lse_out[row] = -INFINITY;
    return;
  }
  f32x4 acc = f32x4{};
  if (live) {
    int e = wv;
    for (; e + 12 < cnt; e += 16) {
      f32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = *(const f32x4*)(part_o(a, s_idx[e + 4 * k], row) + d);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float wgt = s_w[e + 4 * k];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = fmaf(wgt, v[k][c], acc[c]);
      }
    }
    for (; e < cnt; e += 4) {
      const f32x4 v = *(const f32x4*)(part_o(a, s_idx[e], row) + d);
      const float wgt = s_w[e];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = fmaf(wgt, v[c], acc[c]);
    }
  }
  if (wv > 0 && live) *(f32x4*)&s_acc[wv - 1][4 * lane] = acc;
  __syncthreads();
  if (wv == 0 && live) {
    const float inv = 1.0f / s_W;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      out[d + c] = from_f32<OutT>((((acc[c] + s_acc[0][4 * lane + c]) + s_acc[1][4 * lane + c]) +
                                   s_acc[2][4 * lane + c]) * inv);
  }
  if (a.lse_out && blockIdx.y == 0 && tid == 0) a.lse_out[row] = s_M + logf(s_W);
}

}  // namespace

int merge_many_max_parts() { return kMaxManyParts; }

hipError_t launch_merge_many(const MergeArgs& a, bool out_bf16, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (a.n_parts > kMaxManyParts || a.D > 1024 || a.D % 4) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.rows, (unsigned)((a.D + 255) / 256));
  if (out_bf16)
    hipLaunchKernelGGL(merge_many_kernel<bf16>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(merge_many_kernel<float>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, bool out_bf16, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  dim3 grid((unsigned)((a.rows + 3) / 4));
  if (out_bf16)
    hipLaunchKernelGGL(merge_kernel<bf16>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(merge_kernel<float>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dca
