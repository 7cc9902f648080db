// Split-KV regime passes for decode over a q8_0 key cache, on gfx950.
//
// Same math as the bf16 decode passes (DCA feature page, "DCA algorithm", "Implementation
// progress + Section-D simplification", "Section C2b"), over keys stored as q8_0 blocks: every 32
// consecutive dims of a (key, KV head) row share one fp16 scale d, and the value of a dim is
// d * q with q its int8 code (the pages run DCA over such caches, reading the codes inside the
// kernel: Upstream Sync entry "0119-p0-dcaon-scalar-inregister").  The cache is read once, at
// 544 bytes per key and head instead of 1024:
//  * Each workgroup (4 waves) handles one (query row, KV head, span of keys) as in the bf16
//    passes.  64-key tiles of codes (32 KiB) and scales (2 KiB) come in by direct global->LDS
//    loads, double buffered.
//  * Wave w turns the codes of keys [16w, 16w+16) into fp16 values d*q (one rounding) in a 64 KiB
//    fp16 tile laid out like the bf16 passes' tile; from there the score and value operands are
//    read exactly as in those passes, and both products run as fp16 MFMA 16x16x32 (the query's
//    raw dims are converted from bf16 to fp16 once per row, the probabilities are fp16).
//  * The rotary dims of a key are rotated in registers at j mod c from the fp64-built cos/sin
//    tables (lo[p & 63] composed with hi[p >> 6]), as in the bf16 passes.
//  * Codes to fp16: with u = q + 128 (the byte xor 0x80), the fp16 bit pattern 0x6400 | u is
//    1024 + u exactly, so (that - 1152) is q exactly and one fp16 multiply by d gives d*q.
#include "common.h"

namespace dca {
namespace {

constexpr int kD = 512;
constexpr int kTile = 64;
constexpr int kCodeBytes = kTile * kD;          // 32 KiB of int8 codes per tile
constexpr int kScaleBytes = kTile * kD / 32 * 2;  // 2 KiB of fp16 scales per tile
constexpr int kStageBytes = kCodeBytes + kScaleBytes;
constexpr int kF16Bytes = kTile * kD * 2;       // 64 KiB fp16 tile
constexpr float kTau = 8.0f;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// 16-byte chunk swizzle of an fp16 tile row (conflict-free 16-row b128 reads and 4-row transpose
// reads on gfx950's 256-byte bank window), the same as the bf16 passes' tile.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// eight int8 codes (two words) times the fp16 scale d -> eight fp16 values d*q
__device__ __forceinline__ f16x8 dequant8(uint32_t lo, uint32_t hi, _Float16 d) {
  const uint32_t ul = lo ^ 0x80808080u, uh = hi ^ 0x80808080u;
  const f16x2 dd = {d, d};
  const f16x2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
  f16x2 h[4];
  h[0] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, ul, 0x04010400u));
  h[1] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, ul, 0x04030402u));
  h[2] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, uh, 0x04010400u));
  h[3] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, uh, 0x04030402u));
  f16x8 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 v = (h[i] - off) * dd;
    out[2 * i] = v[0];
    out[2 * i + 1] = v[1];
  }
  return out;
}

__global__ __launch_bounds__(256, 1) void attn_decode_q8_kernel(DecodeArgs da) {
  const AttnArgs& a = da.base;
  __shared__ __attribute__((aligned(1024))) char stage[2 * kStageBytes];
  __shared__ __attribute__((aligned(1024))) char kbuf[kF16Bytes];
  __shared__ __attribute__((aligned(16))) _Float16 pbuf[16 * kTile];   // P[head][key]
  __shared__ __attribute__((aligned(1024))) float2 hbuf[2][128];         // hi table row of a tile
  __shared__ float smax[4][16], ssum[4][16], wsum[4][16];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t stage_lds = (uint32_t)(uintptr_t)(lds_char*)stage;
  const uint32_t hbuf_lds = (uint32_t)(uintptr_t)(lds_char*)&hbuf[0][0];
  const int hcol = l & 15, gq = l >> 4;   // column (query head) and 16-lane group
  const int G = a.Hq / a.Hkv;
  const int64_t rows = (int64_t)a.B * a.T;
  const int span = blockIdx.x;
  const int64_t btg = blockIdx.y;
  const int g = (int)(btg % a.Hkv);
  const int64_t bt = btg / a.Hkv;
  const int b = (int)(bt / a.T);
  const int span_lo = span * da.span;
  const int span_hi = min(span_lo + da.span, a.n_kv) - 1;
  const bool head_ok = hcol < G;
  const int64_t rowhead = bt * a.Hq + (int64_t)g * G + (head_ok ? hcol : 0);

  const int8_t* codes_b = (const int8_t*)a.k_raw + ((int64_t)b * a.n_kv * a.Hkv + g) * kD;
  const uint16_t* scales_b = da.k_scales + ((int64_t)b * a.n_kv * a.Hkv + g) * (kD / 32);
  const int half_rot = a.n_rot / 2;   // 64
  const float scale_log2 = a.scale * kLog2e;

  // query fragments (fp16): B operand lane l holds Q[head hcol][32 s + 8 gq .. +7]; the raw dims
  // come in as bf16 and are converted once
  f16x8 q[16];
  {
    const bf16* qt = (const bf16*)a.q_tail + rowhead * a.q_tail_hs + 8 * gq;
#pragma unroll
    for (int s = 4; s < 16; ++s) {
      const bf16x8 v = *(const bf16x8*)(qt + 32 * s - 128);
      f16x8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = head_ok ? (_Float16)(float)v[e] : (_Float16)0.0f;
      q[s] = h;
    }
  }
  // LDS offsets.  QK operand: key row 16w + hcol, chunk 4s + gq.
  const int qrow = 16 * w + hcol;
  int qk_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) qk_off[u] = qrow * 1024 + 16 * ((4 * u + gq) ^ swz(qrow));
  const int j16 = l & 15;

  // Key rotation from the tables (see the bf16 passes): with c a multiple of 64 the lane's lo
  // entries stay in registers and the tile's hi row travels to LDS with the tile's loads.
  const bool tab_tile = da.chunk % 64 == 0;
  const int n_hi = (da.chunk + 63) / 64;
  float2 lo_q[16];
  if (tab_tile) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) lo_q[8 * s + e] = da.rot_lo[qrow * half_rot + 32 * s + 8 * gq + e];
  }

  for (int r = 0; r < 3; ++r) {
    if (!(da.regime_mask & (1 << r))) continue;
    const int slot = da.slot0[r] + span;
    float* lse_out = da.lse_part + (int64_t)slot * rows * a.Hq;
    const int lo_r = max(a.bounds[(r * rows + bt) * 2 + 0], 0);
    const int hi_r = min(a.bounds[(r * rows + bt) * 2 + 1], a.n_kv - 1);
    const int lo = max(lo_r, span_lo), hi = min(hi_r, span_hi);
    if (lo > hi) {
      if (tid < G) lse_out[bt * a.Hq + (int64_t)g * G + tid] = -INFINITY;
      continue;
    }
    {
      const bf16* qr = (const bf16*)a.q_rot[r] + rowhead * a.q_rot_hs + 8 * gq;   // fp16 bits
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 v = *(const bf16x8*)(qr + 32 * s);
        q[s] = head_ok ? __builtin_bit_cast(f16x8, v) : f16x8{};
      }
    }
    f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{};
    // l_part: exact row sum (LSE); w_part: sum of the fp16 weights the PV product uses (O's
    // normaliser, so that weights and normaliser agree)
    float m_used = -INFINITY, l_part = 0.0f, w_part = 0.0f;

    const int kt0 = lo / kTile, kt1 = hi / kTile;
    // tile k0..k0+63 by direct global->LDS loads into stage buf: wave w the code rows 16w..16w+15
    // (two 512-byte rows per load), waves 0 and 1 the scale rows 0..31 and 32..63 (lane l the
    // half l%2 of row l/2); rows past the cache re-read its last key (their scores are masked)
    auto issue = [&](int buf, int k0) {
      const uint32_t base = stage_lds + buf * kStageBytes;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 16 * wu + 2 * i + (l >> 5);
        const int key = min(max(k0 + row, 0), a.n_kv - 1);
        dma16(codes_b + (int64_t)key * a.Hkv * kD + 16 * (l & 31), base + (16 * wu + 2 * i) * 512);
      }
      if (wu < 2) {
        const int row = 32 * wu + (l >> 1);
        const int key = min(max(k0 + row, 0), a.n_kv - 1);
        dma16(scales_b + (int64_t)key * a.Hkv * (kD / 32) + 8 * (l & 1), base + kCodeBytes + wu * 1024);
      }
      if (tab_tile && wu == 3) {   // hi row of the tile (lanes 32..63 fetch the next row, unused)
        const int hr = min((int)((int64_t)k0 % da.chunk >> 6) + (l >> 5), n_hi - 1);
        dma16(da.rot_hi + (int64_t)hr * half_rot + 2 * (l & 31), hbuf_lds + buf * 1024);
      }
    };
    issue(0, kt0 * kTile);
    wait_vm0();
    __syncthreads();

    for (int kt = kt0; kt <= kt1; ++kt) {
      const int cur = (kt - kt0) & 1;
      const int k0 = kt * kTile;
      if (kt < kt1) issue(cur ^ 1, k0 + kTile);
      const int key = k0 + qrow;

      // ---- codes of keys [16w, 16w+16) -> fp16 tile rows (lane l: dims 8l..8l+7 of a row) -----
      {
        const char* st = stage + cur * kStageBytes;
#pragma unroll 4
        for (int i = 0; i < 16; ++i) {
          const int row = 16 * w + i;
          const uint2 c8 = *(const uint2*)(st + row * 512 + 8 * l);
          const _Float16 d = __builtin_bit_cast(_Float16, *(const uint16_t*)(st + kCodeBytes + row * 32 + 2 * (l >> 2)));
          *(f16x8*)(kbuf + row * 1024 + 16 * (l ^ swz(row))) = dequant8(c8.x, c8.y, d);
        }
      }
      const char* kb = kbuf;

      // ---- S^T for keys [16w, 16w+16) (the wave's own rows: no barrier needed) ----------------
      f16x8 kf[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) kf[s] = *(const f16x8*)(kb + qk_off[s & 3] + 256 * (s >> 2));
      {
        // rotate the rotary pairs (f, f + 64) of the lane's key by (cos, sin) of pos * w_f,
        // composed from the lo and hi tables by the angle-addition formulas
        auto rotate = [&](auto lo_of, auto hi_of) {
#pragma unroll
          for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int f = 32 * s + 8 * gq + e;
              const float2 A = lo_of(8 * s + e, f), Bv = hi_of(f);
              const float cs = A.x * Bv.x - A.y * Bv.y;
              const float sn = A.y * Bv.x + A.x * Bv.y;
              const float x0 = (float)kf[s][e], x1 = (float)kf[s + 2][e];
              kf[s][e] = (_Float16)fmaf(x0, cs, -x1 * sn);
              kf[s + 2][e] = (_Float16)fmaf(x0, sn, x1 * cs);
            }
          }
        };
        if (tab_tile) {
          const float2* th = &hbuf[cur][0];
          rotate([&](int i, int) { return lo_q[i]; }, [&](int f) { return th[f]; });
        } else {
          const int64_t pos = (int64_t)min(key, a.n_kv - 1) % da.chunk;
          const float2* tlo = da.rot_lo + (pos & 63) * half_rot;
          const float2* thi = da.rot_hi + (pos >> 6) * half_rot;
          rotate([&](int, int f) { return tlo[f]; }, [&](int f) { return thi[f]; });
        }
      }
      f32x4 sacc = f32x4{};
#pragma unroll
      for (int s = 0; s < 16; ++s) sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[s], q[s], sacc, 0, 0, 0);
      // C layout: reg e = key 16w + 4 gq + e, column = head hcol
      float sv[4];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = k0 + 16 * w + 4 * gq + e;
        sv[e] = (kk < lo || kk > hi) ? -INFINITY : sacc[e] * scale_log2;
        mx = fmaxf(mx, sv[e]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (gq == 0) smax[w][hcol] = mx;
      __syncthreads();   // also: every wave's fp16 rows are in the tile before the PV reads
      const float tmax = fmaxf(fmaxf(smax[0][hcol], smax[1][hcol]), fmaxf(smax[2][hcol], smax[3][hcol]));
      const bool need = tmax > m_used + kTau;
      if (__ballot(need)) {
        const float m_new = need ? tmax : m_used;
        const float alpha = need ? exp2f(m_used - m_new) : 1.0f;
        l_part *= alpha;
        w_part *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
        m_used = m_new;
      }
      _Float16 pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = sv[e] == -INFINITY ? 0.0f : exp2f(sv[e] - m_used);
        l_part += p;
        pv[e] = (_Float16)p;
        w_part += (float)pv[e];
      }
      *(uint2*)(pbuf + hcol * kTile + 16 * w + 4 * gq) = __builtin_bit_cast(uint2, pv);
      __syncthreads();

      // ---- O^T += V^T P^T for dims [128w, 128w+128) --------------------------------------
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const f16x8 pb = *(const f16x8*)(pbuf + hcol * kTile + 32 * ks + 8 * gq);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          bf16x4 v[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int row = 32 * ks + 8 * gq + 4 * e + (j16 >> 2);
            const int c = 16 * w + 2 * dt + ((j16 >> 1) & 1);
            const int off = row * 1024 + 16 * (c ^ swz(row)) + 8 * (j16 & 1);
            v[e] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(kb + off));
          }
          bf16x8 vf;
          vf[0] = v[0][0]; vf[1] = v[0][1]; vf[2] = v[0][2]; vf[3] = v[0][3];
          vf[4] = v[1][0]; vf[5] = v[1][1]; vf[6] = v[1][2]; vf[7] = v[1][3];
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, vf), pb, o[dt], 0, 0, 0);
        }
      }
      wait_vm0();
      __syncthreads();
    }

    // ---- combine the row sums of the 4 waves and store the partial ----------------------------
    float ls = l_part, ws = w_part;
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    ws += __shfl_xor(ws, 16, 64);
    ws += __shfl_xor(ws, 32, 64);
    if (gq == 0) {
      ssum[w][hcol] = ls;
      wsum[w][hcol] = ws;
    }
    __syncthreads();
    const float l_tot = (ssum[0][hcol] + ssum[1][hcol]) + (ssum[2][hcol] + ssum[3][hcol]);
    const float w_tot = (wsum[0][hcol] + wsum[1][hcol]) + (wsum[2][hcol] + wsum[3][hcol]);
    const bool nonempty = l_tot > 0.0f && w_tot > 0.0f;
    const float inv = nonempty ? 1.0f / w_tot : 0.0f;
    if (head_ok) {
      float* orow = da.o_part + ((int64_t)slot * rows * a.Hq + rowhead) * kD + 128 * w + 4 * gq;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *(f32x4*)(orow + 16 * dt) = o[dt] * inv;
      if (gq == 0 && w == 0) lse_out[rowhead] = nonempty ? (m_used + log2f(l_tot)) * kLn2 : -INFINITY;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_attn_decode_q8(const DecodeArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.base.B * a.base.T;
  if (rows <= 0 || a.n_spans <= 0) return hipSuccess;
  if (!a.rot_lo || !a.base.rot_f16 || (a.base.n_kv > 0 && (!a.k_scales || !a.base.k_raw)))
    return hipErrorInvalidValue;
  dim3 grid((unsigned)a.n_spans, (unsigned)(rows * a.base.Hkv)), block(256);
  hipLaunchKernelGGL(attn_decode_q8_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace dca
