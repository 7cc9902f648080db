// One regime's attention pass for fp32 data (any head_dim <= 1024): one wave per
// (query row, query head, regime).  DCA feature page, "Implementation progress + Section-D
// simplification": each pass emits normalised O and lse = m + ln(rowsum); "Section C2b": an
// empty regime gives O = 0, lse = -inf.  Scores use the rotated query/key dims [0, n_rot) and the
// raw dims [n_rot, D); values are the raw keys (K = V).  The online softmax runs in fp32.
#include "common.h"

namespace dca {
namespace {

__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)a.B * a.T;
  const int64_t total = rows * a.Hq * 3;
  if (wid >= total) return;
  const int r = (int)(wid % 3);
  const int64_t rh = wid / 3;            // (b*T + t)*Hq + h
  const int h = (int)(rh % a.Hq);
  const int64_t row = rh / a.Hq;
  const int b = (int)(row / a.T);
  if (!a.o[r]) return;
  const int G = a.Hq / a.Hkv;
  const int g = h / G;
  const int lo = max(a.bounds[(r * rows + row) * 2 + 0], 0);   // never read outside the cache
  const int hi = min(a.bounds[(r * rows + row) * 2 + 1], a.n_kv - 1);
  const float* qr = (const float*)a.q_rot[r] + rh * a.q_rot_hs;
  const float* qt = (const float*)a.q_tail + rh * a.q_tail_hs;
  float q[16], acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int d = lane + 64 * k;
    q[k] = d < a.n_rot ? qr[d] : (d < a.D ? qt[d - a.n_rot] : 0.0f);
    acc[k] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int j = lo; j <= hi; ++j) {
    const int64_t kv = ((int64_t)b * a.n_kv + j) * a.Hkv + g;
    const float* kr = (const float*)a.k_rot + kv * a.k_rot_hs;
    const float* kw = (const float*)a.k_raw + kv * a.D;
    float part = 0.0f;
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int d = lane + 64 * k;
      v[k] = d < a.D ? kw[d] : 0.0f;
      const float kk = d < a.n_rot ? kr[d] : v[k];
      part = fmaf(q[k], kk, part);
    }
    const float s = wave_sum(part) * a.scale;
    const float m_new = fmaxf(m, s);
    const float alpha = expf(m - m_new);   // m = -inf -> 0
    const float p = expf(s - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = fmaf(p, v[k], acc[k] * alpha);
    m = m_new;
  }
  float* o = a.o[r] + rh * a.D;
  const bool empty = !(l > 0.0f);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int d = lane + 64 * k;
    if (d < a.D) o[d] = empty ? 0.0f : acc[k] / l;
  }
  if (lane == 0) a.lse[r][rh] = empty ? -INFINITY : m + logf(l);
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream) {
  const int64_t waves = (int64_t)a.B * a.T * a.Hq * 3;
  if (waves <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dca
