// Partial ("proportional") RoPE at explicit positions.
// DCA feature page: "DCA algorithm" (only the rotary dims are remapped, the rest pass through),
// "Why llamafile is sufficient" (per-pair freq_factors fed to the rope), "Section C2b" (keys
// rotated once, queries three times).  Pair f couples dims f and f + n_rot/2; its angle is
// p * theta^(-2f/n_rot) / freq_factors[f], formed and reduced in fp64; the rotation itself is
// fp32 and rounds to nearest-even on a bf16 store.  The optional magnitude factor (YaRN's
// attention factor, "Runtime knobs") multiplies the rotated dims: it scales cos and sin in fp64.
#include "common.h"

namespace dca {
namespace {

constexpr int kRopeRows = 4;   // rows per block

template <typename T, typename TO>
__global__ __launch_bounds__(256) void rope_kernel(RopeArgs a) {
  __shared__ double w_s[512];
  const int half = a.n_rot / 2;
  for (int f = threadIdx.x; f < half; f += blockDim.x) {
    double w = pow(a.theta, -2.0 * (double)f / (double)a.n_rot);
    if (a.freq_factors) w /= (double)a.freq_factors[f];
    w_s[f] = w;
  }
  __syncthreads();
  const int z = blockIdx.z;
  const T* __restrict__ x = (const T*)a.x;
  TO* __restrict__ y = (TO*)a.y + (int64_t)z * a.y_plane_stride;
  const int64_t row0 = (int64_t)blockIdx.x * kRopeRows;
  const int n = kRopeRows * half;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int64_t row = row0 + e / half;
    const int f = e % half;
    if (row >= a.rows) continue;
    int64_t p;
    if (a.pos) {
      p = a.pos[(int64_t)z * a.pos_plane_stride + row];
    } else {
      p = (row % a.pos_mod_rows) % a.chunk;
    }
    double sd, cd;
    sincos((double)p * w_s[f], &sd, &cd);
    const float cs = (float)(a.mag * cd), sn = (float)(a.mag * sd);
    for (int h = 0; h < a.n_heads; ++h) {
      const T* xr = x + row * a.x_row_stride + (int64_t)h * a.x_head_stride;
      TO* yr = y + row * a.y_row_stride + (int64_t)h * a.y_head_stride;
      const float x0 = to_f32(xr[f]);
      const float x1 = to_f32(xr[f + half]);
      yr[f] = from_f32<TO>(fmaf(x0, cs, -x1 * sn));
      yr[f + half] = from_f32<TO>(fmaf(x0, sn, x1 * cs));
    }
  }
  if (a.copy_tail && sizeof(T) == sizeof(TO)) {
    const int tail = a.head_dim - a.n_rot;
    const int m = kRopeRows * a.n_heads * tail;
    for (int e = threadIdx.x; e < m; e += blockDim.x) {
      const int64_t row = row0 + e / (a.n_heads * tail);
      const int rem = e % (a.n_heads * tail);
      const int h = rem / tail, d = a.n_rot + rem % tail;
      if (row >= a.rows) continue;
      const T v = x[row * a.x_row_stride + (int64_t)h * a.x_head_stride + d];
      y[row * a.y_row_stride + (int64_t)h * a.y_head_stride + d] = *(const TO*)&v;
    }
  }
}

// Vectorised form for the common case (n_rot/2 a multiple of 8 and at most 128, rows and heads at
// 16-byte boundaries): a block takes R rows (8, or 1 when there are few rows) for every plane and
// head.  The cos/sin of its
// rows, planes and pairs are formed once into LDS (fp64 angles, the same arithmetic as above), so
// that each input row is read once for all planes and every thread then moves 8 pairs with
// 16-byte loads and stores.  Results are bit-identical to rope_kernel.
constexpr int kRopeMaxHalf8 = 128;
constexpr int kRopeMaxPlanes = 3;

__device__ __forceinline__ void load8(const bf16* p, float* v) {
  const bf16x8 t = *(const bf16x8*)p;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)t[e];
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const f32x4 t0 = *(const f32x4*)p, t1 = *(const f32x4*)(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = t0[e];
    v[e + 4] = t1[e];
  }
}
__device__ __forceinline__ void store8(bf16* p, const float* v) {
  bf16x8 t;
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = (bf16)v[e];
  *(bf16x8*)p = t;
}
__device__ __forceinline__ void store8(f16* p, const float* v) {
  f16x8 t;
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = (f16)v[e];
  *(f16x8*)p = t;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
  *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

template <typename T, typename TO, int R>
__global__ __launch_bounds__(256) void rope8_kernel(RopeArgs a) {
  __shared__ double w_s[kRopeMaxHalf8];
  __shared__ float2 tab[kRopeMaxPlanes][R][kRopeMaxHalf8];
  const int half = a.n_rot / 2;
  const int64_t row0 = (int64_t)blockIdx.x * R;
  for (int f = threadIdx.x; f < half; f += blockDim.x) {
    double w = pow(a.theta, -2.0 * (double)f / (double)a.n_rot);
    if (a.freq_factors) w /= (double)a.freq_factors[f];
    w_s[f] = w;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.planes * R * half; e += blockDim.x) {
    const int z = e / (R * half), r = (e / half) % R, f = e % half;
    const int64_t row = row0 + r;
    if (row >= a.rows) continue;
    const int64_t p = a.pos ? (int64_t)a.pos[(int64_t)z * a.pos_plane_stride + row]
                            : (row % a.pos_mod_rows) % a.chunk;
    double sd, cd;
    sincos((double)p * w_s[f], &sd, &cd);
    tab[z][r][f] = make_float2((float)(a.mag * cd), (float)(a.mag * sd));
  }
  __syncthreads();
  const T* __restrict__ x = (const T*)a.x;
  const int g8 = half / 8;
  const int per_row = a.n_heads * g8;
  for (int e = threadIdx.x; e < R * per_row; e += blockDim.x) {
    const int r = e / per_row, h = (e % per_row) / g8, f0 = 8 * (e % g8);
    const int64_t row = row0 + r;
    if (row >= a.rows) continue;
    const T* xr = x + row * a.x_row_stride + (int64_t)h * a.x_head_stride;
    float x0[8], x1[8];
    load8(xr + f0, x0);
    load8(xr + f0 + half, x1);
    for (int z = 0; z < a.planes; ++z) {
      TO* yr = (TO*)a.y + (int64_t)z * a.y_plane_stride + row * a.y_row_stride + (int64_t)h * a.y_head_stride;
      float y0[8], y1[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float2 c = tab[z][r][f0 + k];
        y0[k] = fmaf(x0[k], c.x, -x1[k] * c.y);
        y1[k] = fmaf(x0[k], c.y, x1[k] * c.x);
      }
      store8(yr + f0, y0);
      store8(yr + f0 + half, y1);
    }
  }
  if (a.copy_tail && sizeof(T) == sizeof(TO)) {
    const int tail = a.head_dim - a.n_rot;
    const int m = R * a.n_heads * tail;
    for (int e = threadIdx.x; e < m; e += blockDim.x) {
      const int64_t row = row0 + e / (a.n_heads * tail);
      const int rem = e % (a.n_heads * tail);
      const int h = rem / tail, d = a.n_rot + rem % tail;
      if (row >= a.rows) continue;
      const T v = x[row * a.x_row_stride + (int64_t)h * a.x_head_stride + d];
      ((TO*)a.y)[row * a.y_row_stride + (int64_t)h * a.y_head_stride + d] = *(const TO*)&v;
    }
  }
}

__global__ void rope_tables_kernel(float2* lo, float2* hi, int32_t n_hi, int32_t n_rot,
                                   double theta, const float* ff, double mag) {
  const int half = n_rot / 2;
  const int64_t total = (int64_t)(64 + n_hi) * half;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / half;
    const int f = (int)(e % half);
    double w = pow(theta, -2.0 * (double)f / (double)n_rot);
    if (ff) w /= (double)ff[f];
    const double p = r < 64 ? (double)r : 64.0 * (double)(r - 64);
    double sd, cd;
    sincos(p * w, &sd, &cd);
    if (r < 64) lo[r * half + f] = make_float2((float)(mag * cd), (float)(mag * sd));
    else hi[(r - 64) * half + f] = make_float2((float)cd, (float)sd);
  }
}

// The vectorised kernel applies when every 8-pair group of a row and head starts at a 16-byte
// boundary in the input and the output.
bool rope8_applies(const RopeArgs& a, bool bf16_data) {
  const int half = a.n_rot / 2;
  if (half % 8 || half > kRopeMaxHalf8 || a.planes > kRopeMaxPlanes) return false;
  const int64_t ein = bf16_data ? 2 : 4, eout = bf16_data ? 2 : 4;
  const bool in_ok = ((uintptr_t)a.x % 16 == 0) && (a.x_row_stride * ein) % 16 == 0 &&
                     (a.x_head_stride * ein) % 16 == 0;
  const bool out_ok = ((uintptr_t)a.y % 16 == 0) && (a.y_row_stride * eout) % 16 == 0 &&
                      (a.y_head_stride * eout) % 16 == 0 && (a.planes == 1 || (a.y_plane_stride * eout) % 16 == 0);
  return in_ok && out_ok;
}

template <int R>
void launch_rope8(const RopeArgs& a, bool bf16_data, hipStream_t stream) {
  const dim3 grid((unsigned)((a.rows + R - 1) / R));
  if (bf16_data && a.out_f16)
    hipLaunchKernelGGL((rope8_kernel<bf16, f16, R>), grid, dim3(256), 0, stream, a);
  else if (bf16_data)
    hipLaunchKernelGGL((rope8_kernel<bf16, bf16, R>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((rope8_kernel<float, float, R>), grid, dim3(256), 0, stream, a);
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, bool bf16_data, hipStream_t stream) {
  if (a.rows <= 0 || a.planes <= 0) return hipSuccess;
  if (rope8_applies(a, bf16_data)) {
    if (a.rows >= 2048)
      launch_rope8<8>(a, bf16_data, stream);
    else   // few rows (decode): one row per block, so that the fp64 angles spread over more blocks
      launch_rope8<1>(a, bf16_data, stream);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((a.rows + kRopeRows - 1) / kRopeRows), 1, (unsigned)a.planes);
  if (bf16_data && a.out_f16)
    hipLaunchKernelGGL((rope_kernel<bf16, f16>), grid, dim3(256), 0, stream, a);
  else if (bf16_data)
    hipLaunchKernelGGL((rope_kernel<bf16, bf16>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((rope_kernel<float, float>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_rope_tables(float2* lo, float2* hi, int32_t n_hi, int32_t n_rot, double theta,
                              const float* freq_factors, double mag, hipStream_t stream) {
  int64_t total = (int64_t)(64 + n_hi) * (n_rot / 2);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(rope_tables_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, lo, hi,
                     n_hi, n_rot, theta, freq_factors, mag);
  return hipGetLastError();
}

}  // namespace dca
