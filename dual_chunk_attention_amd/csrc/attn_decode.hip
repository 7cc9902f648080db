// Split-KV regime passes for bf16 decode (few query tokens per sequence) on gfx950.
//
// Same math as the prefill passes (DCA feature page, "DCA algorithm", "Implementation progress
// + Section-D simplification", "Section C2b"): per query row and regime, softmax over the
// regime's key interval with the regime-rotated query, values = raw keys, normalised O and
// natural-log lse, (0, -inf) when empty.  Decode is bound by reading the cache, so:
//  * Keys are read exactly once: the rotary dims are rotated in registers at j mod c from
//    cos/sin tables formed in fp64 (lo[p & 63][f] composed with hi[p >> 6][f] by the angle
//    addition formulas) instead of being read from a pre-rotated copy.  (When the caller passes
//    pre-rotated keys instead, those are read.)
//  * The cache of one (sequence, KV head) is split into spans of `span` keys; each workgroup
//    handles one (query row, KV head, span) and writes one partial per regime that meets its
//    span; the partials are merged by the N-way LSE merge.  A regime that misses the span
//    writes lse = -inf only.
//  * 4 waves cooperate on 64-key tiles staged by direct global->LDS loads (double buffered):
//    wave w computes S^T = K Q^T for keys [16w, 16w+16) with MFMA 16x16x32 (the G query heads of
//    the KV head are the 16 columns, padded), the per-head maximum is exchanged through LDS,
//    P goes to LDS as bf16, and wave w computes O^T = V^T P^T for head dims [128w, 128w+128)
//    with V^T fragments from the LDS transpose read.
#include "common.h"

namespace dca {
namespace {

constexpr int kD = 512;
constexpr int kTile = 64;
constexpr int kTileBytes = kTile * kD * 2;   // 64 KiB
constexpr float kTau = 8.0f;

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// 16-byte chunk swizzle of a tile row, conflict-free on gfx950 (256-byte bank window) for the
// 16-row b128 reads and the 4-row transpose reads below.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

template <bool ROT16>
__device__ __forceinline__ f32x4 mfma16_rot(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  if constexpr (ROT16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
}

// ROTATE: rotate the keys in registers (K read once); ROT16: rotary operands are fp16.
template <bool ROTATE, bool ROT16>
__global__ __launch_bounds__(256, 1) void attn_decode_kernel(DecodeArgs da) {
  const AttnArgs& a = da.base;
  __shared__ __attribute__((aligned(1024))) char kbuf[2 * kTileBytes];
  __shared__ __attribute__((aligned(16))) bf16 pbuf[16 * kTile];     // P[head][key]
  __shared__ __attribute__((aligned(1024))) float2 hbuf[2][128];      // hi table row of a tile
  __shared__ float smax[4][16], ssum[4][16], wsum[4][16];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(w);   // the wave index in a scalar register
  const uint32_t kbuf_lds = (uint32_t)(uintptr_t)(lds_char*)kbuf;
  const uint32_t hbuf_lds = (uint32_t)(uintptr_t)(lds_char*)&hbuf[0][0];
  const int hcol = l & 15, gq = l >> 4;   // column (query head) and 16-lane group
  const int G = a.Hq / a.Hkv;
  const int64_t rows = (int64_t)a.B * a.T;
  const int span = blockIdx.x;
  const int64_t btg = blockIdx.y;
  const int g = (int)(btg % a.Hkv);
  const int64_t bt = btg / a.Hkv;
  const int b = (int)(bt / a.T);
  const int key_end = da.key0 + da.n_rows;   // one past the region's last cell
  const int span_lo = da.key0 + span * da.span;
  const int span_hi = min(span_lo + da.span, key_end) - 1;
  const bool head_ok = hcol < G;
  const int64_t rowhead = bt * a.Hq + (int64_t)g * G + (head_ok ? hcol : 0);

  // rows of the region: cell j at row j - key0
  const bf16* kraw_b = (const bf16*)a.k_raw + ((int64_t)b * da.n_rows * a.Hkv + g) * kD;
  const bf16* krot_b =
      ROTATE ? nullptr : (const bf16*)a.k_rot + ((int64_t)b * da.n_rows * a.Hkv + g) * a.k_rot_hs;
  const int half_rot = a.n_rot / 2;   // 64
  const float scale_log2 = a.scale * kLog2e;

  // query fragments: B operand lane l holds Q[head hcol][32 s + 8 gq .. +7]
  bf16x8 q[16];
  {
    const bf16* qt = (const bf16*)a.q_tail + rowhead * a.q_tail_hs + 8 * gq;
#pragma unroll
    for (int s = 4; s < 16; ++s) {
      bf16x8 v = *(const bf16x8*)(qt + 32 * s - 128);
      q[s] = head_ok ? v : bf16x8{};
    }
  }
  // LDS offsets.  QK operand: key row 16w + hcol, chunk 4s + gq.
  const int qrow = 16 * w + hcol;
  int qk_off[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) qk_off[u] = qrow * 1024 + 16 * ((4 * u + gq) ^ swz(qrow));
  // PV operand (transpose read): rows 32 ks + 8 gq + 4 e + j/4, dims 128 w + 16 dt + 4 (j%4).
  const int j16 = l & 15;

  // Key rotation from the tables.  With c a multiple of 64, the 64 keys of an aligned tile sit at
  // positions p0 + row (p0 = k0 mod c, a multiple of 64): the lane's lo entries (row qrow) are the
  // same for every tile and stay in registers, and the tile's single hi row travels to LDS with
  // the tile's loads.  Other chunk sizes read both tables per key.
  const bool tab_tile = ROTATE && da.chunk % 64 == 0;
  const int n_hi = (da.chunk + 63) / 64;
  float2 lo_q[16];
  if (tab_tile) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) lo_q[8 * s + e] = da.rot_lo[qrow * half_rot + 32 * s + 8 * gq + e];
  }

  // byte offset of the lane's 16-byte chunk of each of the wave's tile rows 16w..16w+15 from the
  // tile's first key, for tiles wholly inside the region (computed once: with one wave per SIMD
  // every instruction of the per-load address arithmetic is an issue slot of the wave)
  const int64_t key_bytes = (int64_t)a.Hkv * kD * 2;
  uint32_t row_off[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 16 * wu + i;
    row_off[i] = (uint32_t)(row * key_bytes + 16 * (l ^ swz(row)));
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
      const bf16* qr = (const bf16*)a.q_rot[r] + rowhead * a.q_rot_hs + 8 * gq;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 v = *(const bf16x8*)(qr + 32 * s);
        q[s] = head_ok ? v : bf16x8{};
      }
    }
    f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{};
    // l_part: exact row sum (LSE); w_part: sum of the bf16 weights the PV product uses (O's
    // normaliser, so that weights and normaliser agree)
    float m_used = -INFINITY, l_part = 0.0f, w_part = 0.0f;

    const int kt0 = lo / kTile, kt1 = hi / kTile;
    // tile k0..k0+63 by direct global->LDS loads: wave w fills rows 16w..16w+15, lane l the
    // physical chunk l of a row with logical chunk l ^ swz(row); rows outside the region re-read
    // its first or last cell (their scores are masked)
    auto issue = [&](int buf, int k0) {
      const uint32_t base = kbuf_lds + buf * kTileBytes;
      if (k0 >= da.key0 && k0 <= key_end - kTile) {   // the whole tile inside the region
        const char* src = uniform_ptr((const char*)kraw_b + (int64_t)(k0 - da.key0) * key_bytes);
#pragma unroll
        for (int i = 0; i < 16; ++i) dma16_off<true>(src, row_off[i], base + (16 * wu + i) * 1024);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 16 * wu + i;
          const int key = min(max(k0 + row, da.key0), key_end - 1);
          const char* src = uniform_ptr((const char*)kraw_b + (int64_t)(key - da.key0) * key_bytes);
          dma16<true>(src + 16 * (l ^ swz(row)), base + row * 1024);
        }
      }
      if (tab_tile && wu == 0) {   // hi row of the tile (lanes 32..63 fetch the next row, unused)
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
      const char* kb = kbuf + cur * kTileBytes;
      const int key = k0 + qrow;

      // ---- S^T for keys [16w, 16w+16) --------------------------------------------------
      bf16x8 kf[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) kf[s] = *(const bf16x8*)(kb + qk_off[s & 3] + 256 * (s >> 2));
      if (ROTATE) {
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
              const float y0 = fmaf(x0, cs, -x1 * sn), y1 = fmaf(x0, sn, x1 * cs);
              if constexpr (ROT16) {
                kf[s][e] = __builtin_bit_cast(bf16, (f16)y0);
                kf[s + 2][e] = __builtin_bit_cast(bf16, (f16)y1);
              } else {
                kf[s][e] = (bf16)y0;
                kf[s + 2][e] = (bf16)y1;
              }
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
      } else {
        const int krow = min(max(key, da.key0), key_end - 1) - da.key0;
        const bf16* kr = krot_b + (int64_t)krow * a.Hkv * a.k_rot_hs + 8 * gq;  // 2-byte elements
#pragma unroll
        for (int s = 0; s < 4; ++s) kf[s] = *(const bf16x8*)(kr + 32 * s);
      }
      f32x4 sacc = f32x4{};
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        if (s < 4)
          sacc = mfma16_rot<ROT16>(kf[s], q[s], sacc);
        else
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s], q[s], sacc, 0, 0, 0);
      }
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
      __syncthreads();
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
      bf16x4 pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p = sv[e] == -INFINITY ? 0.0f : exp2f(sv[e] - m_used);
        l_part += p;
        pv[e] = (bf16)p;
        w_part += (float)pv[e];
      }
      *(bf16x4*)(pbuf + hcol * kTile + 16 * w + 4 * gq) = pv;
      __syncthreads();

      // ---- O^T += V^T P^T for dims [128w, 128w+128) --------------------------------------
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 pb = *(const bf16x8*)(pbuf + hcol * kTile + 32 * ks + 8 * gq);
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
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb, o[dt], 0, 0, 0);
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

hipError_t launch_attn_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.base.B * a.base.T;
  if (rows <= 0 || a.n_spans <= 0) return hipSuccess;
  dim3 grid((unsigned)a.n_spans, (unsigned)(rows * a.base.Hkv)), block(256);
  const bool r16 = a.base.rot_f16 != 0;
  if (a.rot_lo && r16)
    hipLaunchKernelGGL((attn_decode_kernel<true, true>), grid, block, 0, stream, a);
  else if (a.rot_lo)
    hipLaunchKernelGGL((attn_decode_kernel<true, false>), grid, block, 0, stream, a);
  else if (r16)
    hipLaunchKernelGGL((attn_decode_kernel<false, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attn_decode_kernel<false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace dca
