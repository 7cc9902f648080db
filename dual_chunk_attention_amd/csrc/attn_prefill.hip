// Regime flash-attention passes for bf16 prefill on gfx950 (MFMA 32x32x16).
//
// What it computes (DCA feature page, "DCA algorithm" and "Implementation progress +
// Section-D simplification"): for every query row and each requested regime r, the softmax
// attention over that row's regime key interval [lo, hi] with scores
//   s = scale * (<q_r[0:128], k_rot[0:128]> + <q[128:512], k[128:512]>)
// (q_r rotated at the regime position, k_rot rotated at j mod c) and values v = k (raw, K = V),
// written as normalised O_r (fp32) and lse_r = m + ln(sum e^(s-m)); an empty interval gives
// O_r = 0, lse_r = -inf ("Section C2b"; Upstream Sync entry 0110).
//
// Work decomposition (one workgroup of 4 waves per (sequence b, KV head g, query block)):
//  * The 128 rows of a workgroup are QB = 128/G query positions x the G query heads that share
//    KV head g (GQA), so every K tile staged in LDS serves all of them.  Wave w owns rows
//    [32w, 32w+32); lane l owns row l%32 in both halves of the wave.
//  * Scores are computed transposed, S^T = K Q^T: K is the MFMA A operand (read from LDS), Q^T
//    the B operand, kept in 128 VGPRs for the whole pass.  In the 32x32 result layout a lane
//    holds 16 keys of its own row, so the row max/sum needs one cross-half exchange.
//  * O^T = V^T P^T: the score registers, converted to bf16, are already the B operand (the key
//    order inside the MFMA k-slots is permuted identically on both operands); V^T fragments come
//    from the key-major K tile through the LDS transpose read.  O (512 x 32 per wave) lives in
//    the 256 accumulation registers.
//  * The rotary dims of q_r and k_rot may be fp16 (ROT16): their MFMA k-steps then use the fp16
//    instruction, whose 11-bit mantissa keeps the rounding of rotated operands 8x below bf16's.
//  * K tiles of 32 keys are staged by direct global->LDS 16-byte loads into a double buffer:
//    kqk[32][512] holds rotated dims 0..127 and raw dims 128..511 (QK operand), vlo[32][128]
//    holds raw dims 0..127 (the rest of the V operand).  16-byte chunks are XOR-swizzled per row
//    so that both the 16-row b128 reads and the 4-row transpose reads are bank-conflict free.
//  * Online softmax in the log2 domain against a per-row reference maximum: the first tile with a
//    valid key sets it, and it only moves when a later tile exceeds it by more than 64 (so exp2
//    arguments stay <= 64, P and the fp32 sums cannot overflow).  A move flushes the wave's
//    accumulated O into its own fp32 output rows (rescaled) and restarts O from zero, so O is
//    never rescaled inside the 256 accumulation registers; the epilogue adds the flushed part.
//  * Workgroups are launched latest query block first (longest causal work first).
#include "common.h"

namespace dca {
namespace {

constexpr int kD = 512;
constexpr int kRot = 128;
constexpr int kNK = 32;                          // keys per tile
constexpr int kKqkBytes = kNK * kD * 2;          // 32 KiB
constexpr int kVloBytes = kNK * kRot * 2;        // 8 KiB
constexpr int kStageBytes = kKqkBytes + kVloBytes;
constexpr float kTau = 64.0f;                    // reference-move threshold (log2 units)

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// 16-byte chunk swizzle of a tile row (gfx950 LDS conflicts within 256-byte windows): rows
// r..r+15 map one logical chunk to 16 distinct slots (the 16-lane b128 reads of the QK operand),
// and rows 4k..4k+3 map a chunk pair to distinct 32-byte slots (the 32-lane transpose reads).
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }


// LDS fragments in flight ahead of the MFMA that consumes them (S^T and O^T products)
constexpr int kDepthK = 4;
constexpr int kDepthV = 3;
// direct-to-LDS loads per wave and tile
constexpr int kDmaParts = 10;

template <bool ROT16>
__device__ __forceinline__ f32x16 mfma_rot(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  if constexpr (ROT16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
}

template <int G, bool ROT16>
__global__ __launch_bounds__(256, 1) void attn_prefill_kernel(AttnArgs a, int n_qblocks) {
  constexpr int QB = 128 / G;  // query positions per workgroup
  __shared__ __attribute__((aligned(1024))) char smem[2 * kStageBytes];
  __shared__ int s_lo[3][QB], s_hi[3][QB];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, n = l & 31, half = l >> 5;
  const int per = a.B * a.Hkv;
  const int qb = n_qblocks - 1 - (int)(blockIdx.x / per);
  const int bg = (int)(blockIdx.x % per);
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int64_t rows = (int64_t)a.B * a.T;
  const float scale_log2 = a.scale * kLog2e;

  // ---- per-position intervals of the three regimes ---------------------------------------
  for (int e = tid; e < 3 * QB; e += 256) {
    const int r = e / QB, p = e % QB;
    const int t = qb * QB + p;
    int lo = 0, hi = -1;
    if (t < a.T) {
      lo = max(a.bounds[(r * rows + (int64_t)b * a.T + t) * 2 + 0], 0);
      hi = min(a.bounds[(r * rows + (int64_t)b * a.T + t) * 2 + 1], a.n_kv - 1);
    }
    s_lo[r][p] = lo;
    s_hi[r][p] = hi;
  }

  // ---- this lane's query row -----------------------------------------------------------------
  const int rho = 32 * w + n;
  const int pos_in_blk = rho / G, hh = rho % G;
  const int t = qb * QB + pos_in_blk;
  const bool row_valid = t < a.T;
  const int tt = row_valid ? t : a.T - 1;
  const int64_t rowhead = ((int64_t)b * a.T + tt) * a.Hq + (int64_t)g * G + hh;

  bf16x8 q[32];
  {
    const bf16* qt = (const bf16*)a.q_tail + rowhead * a.q_tail_hs + 8 * half;
#pragma unroll
    for (int s = 8; s < 32; ++s) q[s] = *(const bf16x8*)(qt + 16 * s - kRot);
  }

  // LDS read offsets (bytes).  QK operand: row n, chunk c = 2s + half at (c ^ swz(n)):
  // byte n*1024 + 256*(s>>3) + qk_off[s & 7].
  int qk_off[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) qk_off[u] = n * 1024 + 16 * ((2 * u + half) ^ swz(n));
  // V^T operand (transpose read) for k-step ks, dim tile dt, half e of the 8 k-slots:
  // row 16ks + 8e + 4half + jj (jj = (l%16)/4), dims 32dt + 16grp + 4(l%4), i.e. chunk
  // 4dt + c0 (c0 = 2grp + (l/2)%2) at byte 8(l%2).  swz(row) = 4jj + (2e + half), so the
  // swizzled chunk is 4(dt ^ jj) + (c0 ^ (2e + half)).
  const int j16 = l & 15, grp = (l >> 4) & 1, jj = j16 >> 2;
  const int rho_l = 4 * half + jj;
  const int c0 = 2 * grp + ((j16 >> 1) & 1);
  int v_e[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) v_e[e] = 16 * (c0 ^ (2 * e + half)) + 8 * (j16 & 1);
  int v_dt[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) v_dt[u] = 64 * (u ^ jj);

  __syncthreads();

  const int64_t kv_stride = (int64_t)a.Hkv;
  const bf16* kraw_b = (const bf16*)a.k_raw + ((int64_t)b * a.n_kv * kv_stride + g) * kD;
  const char* krot_b = (const char*)a.k_rot + ((int64_t)b * a.n_kv * kv_stride + g) * a.k_rot_hs * 2;

  // per-regime pointers without indexing the argument arrays at run time
  auto o_of = [&](int r) { return r == 0 ? a.o[0] : r == 1 ? a.o[1] : a.o[2]; };
  for (int r = 0; r < 3; ++r) {
    if (!a.o[r]) continue;
    // union of the rows' intervals and the range where no row needs masking
    int umin = 0x7fffffff, umax = -1, fmax_lo = -0x7fffffff, fmin_hi = 0x7fffffff;
    for (int p = 0; p < QB; ++p) {
      const int lo = s_lo[r][p], hi = s_hi[r][p];
      if (lo <= hi) {
        umin = min(umin, lo);
        umax = max(umax, hi);
      }
      fmax_lo = max(fmax_lo, lo);
      fmin_hi = min(fmin_hi, hi);
    }
    const int my_lo = s_lo[r][pos_in_blk], my_hi = s_hi[r][pos_in_blk];

    {
      const bf16* qr = (const bf16*)a.q_rot[r] + rowhead * a.q_rot_hs + 8 * half;
#pragma unroll
      for (int s = 0; s < 8; ++s) q[s] = *(const bf16x8*)(qr + 16 * s);
    }
    f32x16 o[16];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) o[dt] = f32x16{};
    // online-softmax state of the lane's row.  l_part: sum of the exact p (for the LSE); w_part:
    // sum of the bf16-rounded p that the PV product uses (O is normalised by it, so a dominant
    // key's value comes out exactly)
    float m_used = -INFINITY, l_part = 0.0f, w_part = 0.0f;
    bool flushed = false;
    // the regime's fp32 output rows, which also take O out of the registers on a reference move
    float* const frow = o_of(r) + rowhead * kD + 4 * half;

    if (umin <= umax) {
      const int kt0 = max(umin, 0) / kNK, kt1 = min(umax, a.n_kv - 1) / kNK;
      // K tile k0..k0+31 by direct global->LDS loads.  Row `row` lane l fills physical chunk l
      // with logical chunk l ^ swz(row); since swz < 16 that is a rotary chunk exactly for lanes
      // 0..15.  Byte offsets from the tile base are loop-invariant except in the cache's last
      // tile, where rows past the end re-read the last key (their scores are masked).
      const int64_t krow_bytes = (int64_t)kv_stride * kD * 2, rrow_bytes = (int64_t)kv_stride * a.k_rot_hs * 2;
      const bool rot_lane = l < 16;
      const int lane_row_bytes = (int)(rot_lane ? rrow_bytes : krow_bytes);
      // LDS destinations as 32-bit addresses, wave-uniform (scalar registers)
      const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_char*)smem;
      const int wu = __builtin_amdgcn_readfirstlane(w);
      // part j (0..9) of the loads of tile k0..k0+31 into stage buf: parts 0..7 fill kqk row
      // 8w+j, parts 8..9 fill four vlo rows each
      auto issue_part = [&](int buf, int k0, int j) {
        const uint32_t kqk = smem_lds + buf * kStageBytes;
        const uint32_t vlo = kqk + kKqkBytes;
        // tile bases are wave-uniform: scalar registers, selected per lane
        const char* raw_t = uniform_ptr((const char*)kraw_b + (int64_t)k0 * krow_bytes);
        const char* rot_t = uniform_ptr(krot_b + (int64_t)k0 * rrow_bytes);
        const int last = a.n_kv - 1 - k0;
        const bool tail = last < kNK - 1;
        if (j < 8) {
          const int row = 8 * w + j;
          const int rr = tail ? min(row, last) : row;
          const char* lane_t = rot_lane ? rot_t : raw_t;
          dma16(lane_t + (uint32_t)(rr * lane_row_bytes + 16 * (l ^ swz(row))), kqk + (8 * wu + j) * 1024);
        } else {
          const int i = j - 8;
          const int row = 8 * w + 4 * i + (l >> 4);
          const int rr = tail ? min(row, last) : row;
          dma16(raw_t + (uint32_t)(rr * (int)krow_bytes + 16 * ((l & 15) ^ swz(row))),
                vlo + (8 * wu + 4 * i) * 256);
        }
      };
      auto issue = [&](int buf, int k0) {
#pragma unroll
        for (int j = 0; j < kDmaParts; ++j) issue_part(buf, k0, j);
      };

      issue(0, kt0 * kNK);
      wait_vm0();
      __syncthreads();

      for (int kt = kt0; kt <= kt1; ++kt) {
        const int cur = (kt - kt0) & 1;
        const int k0 = kt * kNK;
        // the next tile's loads, into the other stage (free since the last barrier)
        if (kt < kt1) issue(cur ^ 1, k0 + kNK);
        const char* kqk = smem + cur * kStageBytes;
        const char* vlo = kqk + kKqkBytes;

        // ---- S^T = K Q^T over all 512 dims --------------------------------------------------
        // software pipelined: the fragment of step s+kDepthK is requested right after the MFMA of
        // step s, and scheduling fences keep that order (one wave per SIMD: the LDS latency is
        // hidden only by the reads in flight)
        f32x16 sacc = f32x16{};
        {
          bf16x8 kf[kDepthK];
          auto kld = [&](int s) { return *(const bf16x8*)(kqk + qk_off[s & 7] + 256 * (s >> 3)); };
#pragma unroll
          for (int j = 0; j < kDepthK; ++j) kf[j] = kld(j);
#pragma unroll
          for (int s = 0; s < 32; ++s) {
            if (s < 8)
              sacc = mfma_rot<ROT16>(kf[s % kDepthK], q[s], sacc);
            else
              sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s % kDepthK], q[s], sacc, 0, 0, 0);
            if (s + kDepthK < 32) kf[s % kDepthK] = kld(s + kDepthK);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // ---- mask, row max, lazy rescale, probabilities --------------------------------------
        // raw scores: the scale (log2 domain) is applied once to the row max and fused into the
        // exponent's FMA
        const bool full = fmax_lo <= k0 && k0 + kNK - 1 <= fmin_hi;   // same for the workgroup
        float sv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) sv[e] = sacc[e];
        if (!full) {
          const int lo_eff = my_lo - k0, hi_eff = my_hi - k0;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int kk = 8 * (e >> 2) + 4 * half + (e & 3);
            if (kk < lo_eff || kk > hi_eff) sv[e] = -INFINITY;
          }
        }
        float mx = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
#pragma unroll
        for (int e = 3; e < 15; e += 2) mx = fmaxf(fmaxf(mx, sv[e]), sv[e + 1]);
        mx = fmaxf(mx, sv[15]);
        {
          auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                      false, false);
          mx = fmaxf(__uint_as_float(sw2[0]), __uint_as_float(sw2[1])) * scale_log2;
        }
        // first valid key of a row: take its tile maximum as the reference (O is still 0)
        if (m_used == -INFINITY) m_used = mx;
        // a later tile exceeding the reference by more than kTau: move the accumulated state of
        // the wave's rows into their fp32 output rows (rescaled to the new reference) and
        // restart O from zero; with kTau = 64 this is practically never taken
        const bool need = mx > m_used + kTau;
        if (__ballot(need)) {
          const float m_new = need ? mx : m_used;
          const float alpha = exp2f(m_used - m_new);
          if (row_valid && m_used != -INFINITY) {
            float* orow = frow;
#pragma unroll
            for (int dt = 0; dt < 16; ++dt) {
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) {
                f32x4 v;
                v[0] = o[dt][4 * q4 + 0];
                v[1] = o[dt][4 * q4 + 1];
                v[2] = o[dt][4 * q4 + 2];
                v[3] = o[dt][4 * q4 + 3];
                f32x4* dst = (f32x4*)(orow + 32 * dt + 8 * q4);
                if (flushed) v += *dst;
                *dst = v * alpha;
              }
            }
            flushed = true;
            wait_vm0();   // the output rows are re-read by a later flush
          }
#pragma unroll
          for (int dt = 0; dt < 16; ++dt) o[dt] = f32x16{};
          l_part *= alpha;
          w_part *= alpha;
          m_used = m_new;
        }
        // p = exp2(s * scale_log2 - m_used): a masked score (-inf) gives 0; a row without any
        // valid key so far has m_used = -inf and only masked scores, so any finite reference
        // gives the same zeros.  The exponents are <= kTau, so the raw v_exp_f32 suffices.
        const float neg_m = m_used == -INFINITY ? 0.0f : -m_used;
        bf16x8 pk[2];
        float psum = 0.0f, wsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], scale_log2, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e + 1], scale_log2, neg_m));
          const bf16x2 pb = {(bf16)p0, (bf16)p1};
          psum += p0;
          psum += p1;
          // sum of the bf16-rounded weights the PV product uses (exact products by one)
          wsum = __builtin_amdgcn_fdot2_f32_bf16(pb, bf16x2{(bf16)1.0f, (bf16)1.0f}, wsum, false);
          pk[e >> 3][e & 7] = pb[0];
          pk[e >> 3][(e & 7) + 1] = pb[1];
        }
        l_part += psum;
        w_part += wsum;

        // ---- O^T += V^T P^T, software pipelined like S^T -------------------------------------
        {
          auto vload = [&](int i) {
            const int ks = i >> 4, dt = i & 15;
            const bool lo_part = dt < 4;
            const char* base = lo_part ? vlo : kqk;
            const int stride = lo_part ? 256 : 1024;
            const int off = rho_l * stride + v_dt[dt & 3] + 256 * (dt >> 2);
            const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)(base + off + v_e[0] + (16 * ks) * stride));
            const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)(base + off + v_e[1] + (16 * ks + 8) * stride));
            bf16x8 vv;
            vv[0] = v0[0]; vv[1] = v0[1]; vv[2] = v0[2]; vv[3] = v0[3];
            vv[4] = v1[0]; vv[5] = v1[1]; vv[6] = v1[2]; vv[7] = v1[3];
            return vv;
          };
          bf16x8 vf[kDepthV];
#pragma unroll
          for (int j = 0; j < kDepthV; ++j) vf[j] = vload(j);
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            o[i & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % kDepthV], pk[i >> 4], o[i & 15], 0, 0, 0);
            if (i + kDepthV < 32) vf[i % kDepthV] = vload(i + kDepthV);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        wait_vm0();
        __syncthreads();
      }
    }

    // ---- end of the regime -----------------------------------------------------------------
    // normaliser and natural-log lse from the row totals of both halves of the wave
    float l_tot, w_tot;
    {
      auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part),
                                                  false, false);
      l_tot = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
      auto sw3 = __builtin_amdgcn_permlane32_swap(__float_as_uint(w_part), __float_as_uint(w_part),
                                                  false, false);
      w_tot = __uint_as_float(sw3[0]) + __uint_as_float(sw3[1]);
    }
    const bool nonempty = l_tot > 0.0f && w_tot > 0.0f;
    const float inv = nonempty ? 1.0f / w_tot : 0.0f;
    const float lse = nonempty ? (m_used + log2f(l_tot)) * kLn2 : -INFINITY;
    if (row_valid) {
      // this regime's normalised fp32 partial
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v;
          v[0] = o[dt][4 * q4 + 0];
          v[1] = o[dt][4 * q4 + 1];
          v[2] = o[dt][4 * q4 + 2];
          v[3] = o[dt][4 * q4 + 3];
          f32x4* src = (f32x4*)(frow + 32 * dt + 8 * q4);
          if (flushed) v += *src;
          v *= inv;
          *src = v;
        }
      }
      if (half == 0) a.lse[r][rowhead] = lse;
    }
  }
}

template <bool ROT16>
hipError_t launch_prefill(const AttnArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int QB = 128 / G;
  const int n_qblocks = (a.T + QB - 1) / QB;
  const int64_t blocks = (int64_t)n_qblocks * a.B * a.Hkv;
  if (blocks <= 0) return hipSuccess;
  dim3 grid((unsigned)blocks), block(256);
#define DCA_PREFILL_LAUNCH(GG)                                                                   \
  case GG:                                                                                       \
    hipLaunchKernelGGL((attn_prefill_kernel<GG, ROT16>), grid, block, 0, stream, a, n_qblocks);  \
    break;
  switch (G) {
    DCA_PREFILL_LAUNCH(1)
    DCA_PREFILL_LAUNCH(2)
    DCA_PREFILL_LAUNCH(4)
    DCA_PREFILL_LAUNCH(8)
    DCA_PREFILL_LAUNCH(16)
    default: return hipErrorInvalidValue;
  }
#undef DCA_PREFILL_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill_bf16(const AttnArgs& a, hipStream_t stream) {
  return a.rot_f16 ? launch_prefill<true>(a, stream) : launch_prefill<false>(a, stream);
}

}  // namespace dca
