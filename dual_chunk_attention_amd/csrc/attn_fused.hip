// Fused bf16 prefill: the three regimes of every query row under one online softmax, on gfx950.
//
// What it computes (DCA feature page, "DCA algorithm" and "Implementation progress + Section-D
// simplification"; the single pass is the fused-kernel entry of the Upstream Sync page): for every
// query row, the softmax attention over the union of its three regime key intervals, where a key
// of regime r is scored against the query rotated at that regime's position,
//   s = scale * (<q_r[0:128], k_rot[0:128]> + <q[128:512], k[128:512]>),
// k_rot rotated at j mod c, values v = k (raw, K = V).  Output: the normalised O and the
// natural-log lse = m + ln(sum e^(s-m)); a row without keys gives O = 0, lse = -inf.
//
// Work decomposition (one workgroup of 4 waves per (sequence b, KV head g, query block of 128
// rows = 128/G positions x the G query heads of g)); wave w owns rows [32w, 32w+32):
//  * Scores S^T = K Q^T with MFMA 32x32x16: K fragments from LDS (A operand), Q^T held in 128
//    VGPRs (B operand); the rotary k-steps use the fp16 instruction on fp16 rotated operands.  In
//    the 32x32 result a lane holds 16 keys of its row, so a row max needs one cross-half exchange.
//  * O^T = V^T P^T: the bf16 probabilities in registers are already the B operand (the key order
//    in the MFMA k-slots is permuted the same way on both operands); V^T fragments come from the
//    key-major tile through the LDS transpose read.  O (512 x 32 fp32) lives in the 256
//    accumulation registers for the whole pass.
//  * Three LDS stages: the loads of tile i+2 (direct global->LDS) go out between the score MFMAs
//    of tile i, so a tile has two tile times to arrive.  The probabilities of the second half of a
//    tile's keys are formed between the O^T MFMAs of its first half.
//  * The key tiles of the three regimes form one sequence (intra, succ, inter); at a regime change
//    only the rotary Q fragments are reloaded.
//  * Reference maximum per row: the first tile with a valid key sets it; later tiles take no row
//    maximum at all.  The pass keeps its result while every row's sums of p stay below 2^80 (then
//    every exponent stayed below 80 and O is far from overflow; the arithmetic is that of any
//    other reference).  A pass whose sums do not (rare; an inf or NaN included) raises a flag of
//    the workgroup; after its tile sequence a flagged workgroup runs the sequence twice more: once
//    with each row's reference following every tile's maximum (its exponents stay <= 0; its O is
//    discarded), which leaves the exact row maxima, and once more in full against them.  O never
//    leaves the registers before the end, and the pass needs no scratch memory.
//  * At the end each wave stages its normalised O through the (then free) LDS stages and stores
//    whole row segments.
//  * Workgroups are launched latest query block first (longest causal work first).
#include <type_traits>

#include "common.h"

namespace dca {
namespace {

constexpr int kD = 512;
constexpr int kRot = 128;
constexpr int kNK = 32;                          // keys per tile
constexpr int kRawBytes = kNK * kD * 2;          // 32 KiB: raw dims 0..511, 1 KiB rows
constexpr int kRotBytes = kNK * kRot * 2;        // 8 KiB: rotated dims 0..127, 256-byte rows
constexpr int kStageBytes = kRawBytes + kRotBytes;
constexpr int kStages = 3;
constexpr float kSumMax = 0x1p80f;               // bound on a row's sums of p in pass 0
constexpr int kDepthK = 4;                       // K fragments in flight ahead of their MFMA
constexpr int kDepthV = 3;                       // V^T fragments in flight ahead of their MFMA

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// 16-byte chunk swizzle of a tile row (gfx950 LDS conflicts within 256-byte windows): rows
// r..r+15 map one logical chunk to 16 distinct slots (the 16-lane b128 reads of the QK operand),
// and rows 4k..4k+3 map a chunk pair to distinct 32-byte slots (the transpose reads).  It only
// permutes the 16 chunks of a 256-byte window.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// a value the compiler cannot see through, so that address arithmetic on it is redone where it is
// used instead of being hoisted out of the tile loop into long-lived registers
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Two k-steps s, s+1 of the score product S^T += K Q^T (32 keys x 32 rows, 16 dims each): fp16
// for the rotary k-steps 0..7, bf16 for the rest; k-step 0 starts from zero.  Issued as inline asm
// so that the accumulator stays in VGPRs (the 256 accumulation registers hold O) and every step
// keeps its place in the issue order; with one wave per SIMD every instruction costs an issue slot,
// so the pair carries no wait states of its own.  Hazards the compiler does not see here: an MFMA
// reading a VGPR that a VALU instruction wrote needs two wait states; the operands come from LDS
// reads, Q's global loads and earlier MFMAs only, and the build checks the generated code for a
// VALU write of an operand within two instructions of the pair (dual_chunk_attention_amd/
// hazards.py).  Dependent MFMAs on the same accumulator need none, and the caller waits out the last
// one before the VALU reads the result.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void mfma_qk2(f32x16& acc, const bf16x8& k0, const bf16x8& q0, const bf16x8& k1,
                                         const bf16x8& q1, int s) {
  if (s == 0)
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0\n\tv_mfma_f32_32x32x16_f16 %0, %3, %4, %0"
                 : "=&v"(acc) : "v"(k0), "v"(q0), "v"(k1), "v"(q1));
  else if (s < 8)
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0\n\tv_mfma_f32_32x32x16_f16 %0, %3, %4, %0"
                 : "+v"(acc) : "v"(k0), "v"(q0), "v"(k1), "v"(q1));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %3, %4, %0"
                 : "+v"(acc) : "v"(k0), "v"(q0), "v"(k1), "v"(q1));
}
// the same pair with one direct global->LDS load (scalar base sbase + lane offset voff, LDS row
// address lds_a + lds_b): the M0 write leads, and the two MFMAs are its wait states
__device__ __forceinline__ void mfma_qk2_load(f32x16& acc, const bf16x8& k0, const bf16x8& q0, const bf16x8& k1,
                                              const bf16x8& q1, int s, const void* sbase, uint32_t voff,
                                              uint32_t lds_a, uint32_t lds_b) {
  if (s < 8)
    asm volatile("s_add_u32 m0, %5, %6\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0\n\t"
                 "v_mfma_f32_32x32x16_f16 %0, %3, %4, %0\n\tglobal_load_lds_dwordx4 %7, %8"
                 : "+v"(acc) : "v"(k0), "v"(q0), "v"(k1), "v"(q1), "s"(lds_a), "s"(lds_b), "v"(voff), "s"(sbase)
                 : "memory", "m0");
  else
    asm volatile("s_add_u32 m0, %5, %6\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
                 "v_mfma_f32_32x32x16_bf16 %0, %3, %4, %0\n\tglobal_load_lds_dwordx4 %7, %8"
                 : "+v"(acc) : "v"(k0), "v"(q0), "v"(k1), "v"(q1), "s"(lds_a), "s"(lds_b), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

template <int G>
__global__ __launch_bounds__(256, 1) void attn_fused_kernel(AttnArgs a, int n_qblocks) {
  constexpr int QB = 128 / G;  // query positions per workgroup
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];
  __shared__ int s_lo[3][QB], s_hi[3][QB];
  __shared__ int s_flag;   // some row's sums reached kSumMax: the workgroup reruns its sequence

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, n = l & 31, half = l >> 5;
  const int wu = __builtin_amdgcn_readfirstlane(w);
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
  if (tid == 0) s_flag = 0;

  // ---- this lane's query row: rho = 32w + n --------------------------------------------------
  const int rho = 32 * w + n;
  const int pos_in_blk = rho / G;
  const int t_row = qb * QB + pos_in_blk;
  const bool row_valid = t_row < a.T;
  const int64_t rowhead =
      ((int64_t)b * a.T + (row_valid ? t_row : a.T - 1)) * a.Hq + (int64_t)g * G + rho % G;

  bf16x8 q[32];
  {
    const bf16* qt = (const bf16*)a.q_tail + rowhead * a.q_tail_hs + 8 * half;
#pragma unroll
    for (int s = 8; s < 32; ++s) q[s] = *(const bf16x8*)(qt + 16 * s - kRot);
  }

  // LDS offsets (bytes) inside a stage.  QK operand of k-step s: row n, chunk 2(s%8) + half of
  // the rotated row (s < 8) or of window s/8 of the raw row (s >= 8), at that chunk ^ swz(n).
  int qk_off[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) qk_off[u] = 16 * ((2 * u + half) ^ swz(n));
  // V^T operand (transpose read) of dim tile dt, k-step ks, half e of the 8 k-slots: key row
  // 16ks + 8e + 4half + jj (jj = (l%16)/4), dims 32dt + 16grp + 4(l%4), i.e. chunk 4(dt%4) + c0
  // (c0 = 2grp + (l/2)%2) of window dt/4 at byte 8(l%2).  swz(row) = 4jj + (2e + half), so the
  // swizzled chunk is 4((dt%4) ^ jj) + (c0 ^ (2e + half)).
  const int j16 = l & 15, grp = (l >> 4) & 1, jj = j16 >> 2;
  const int c0 = 2 * grp + ((j16 >> 1) & 1);
  int v_e[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    v_e[e] = (4 * half + jj + 8 * e) * 1024 + 16 * (c0 ^ (2 * e + half)) + 8 * (j16 & 1);
  int v_dt[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) v_dt[u] = 64 * (u ^ jj);

  __syncthreads();

  // ---- the tile sequence: regimes 0, 1, 2, each over the union of its rows' intervals --------
  int st[3], kt0[3], full_lo[3], full_hi[3];
  int n_tiles = 0;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
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
    const int k_first = umin <= umax ? umin / kNK : 0;
    const int cnt = umin <= umax ? umax / kNK - k_first + 1 : 0;
    st[r] = __builtin_amdgcn_readfirstlane(n_tiles);
    kt0[r] = __builtin_amdgcn_readfirstlane(k_first);
    // keys [full_lo, full_hi] are valid for every row of the workgroup in this regime
    full_lo[r] = __builtin_amdgcn_readfirstlane(fmax_lo);
    full_hi[r] = __builtin_amdgcn_readfirstlane(fmin_hi);
    n_tiles += cnt;
  }
  n_tiles = __builtin_amdgcn_readfirstlane(n_tiles);
  // per-tile lookups as scalar selects on the tile index (no indexing of the per-regime arrays,
  // which the compiler would turn into chains of branches)
  const int st1 = st[1], st2 = st[2];
  auto sel = [&](int i, int v0, int v1, int v2) { return i >= st2 ? v2 : (i >= st1 ? v1 : v0); };
  auto regime_of = [&](int i) { return (int)(i >= st1) + (int)(i >= st2); };
  const int kb0 = kt0[0] * kNK, kb1 = (kt0[1] - st1) * kNK, kb2 = (kt0[2] - st2) * kNK;
  auto k0_of = [&](int i) { return sel(i, kb0, kb1, kb2) + kNK * i; };
  auto load_qrot = [&](int r) {
    const void* base = r == 0 ? a.q_rot[0] : r == 1 ? a.q_rot[1] : a.q_rot[2];
    const bf16* qr = (const bf16*)base + rowhead * a.q_rot_hs + 8 * half;
#pragma unroll
    for (int s = 0; s < 8; ++s) q[s] = *(const bf16x8*)(qr + 16 * s);
  };

  // ---- tile loads: part j (0..9) of tile k0..k0+31 into the stage at byte offset stg_off, by
  // direct global->LDS loads.  Parts 0..7: raw row 8w+j, lane l the physical chunk l (logical
  // chunk l ^ swz(row)); parts 8..9: four rotated rows 8w+4(j-8)+l/16 each, lane l the physical
  // chunk l%16.  Rows past the cache re-read its last key (their scores are masked).  A tile
  // wholly inside the cache (all but the last of a sequence) loads from one scalar base per tile
  // plus lane offsets computed once before the tile loop: the per-part 64-bit address arithmetic
  // it replaces cost about 280 scalar and vector instructions per tile and wave, each an issue
  // slot of the wave's only SIMD slot.
  const bf16* kraw_b = (const bf16*)a.k_raw + ((int64_t)b * a.n_kv * a.Hkv + g) * kD;
  const char* krot_b = (const char*)a.k_rot + ((int64_t)b * a.n_kv * a.Hkv + g) * a.k_rot_hs * 2;
  const int raw_row = a.Hkv * kD * 2, rot_row = a.Hkv * (int)a.k_rot_hs * 2;   // bytes per key
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_char*)smem;
  // byte offsets of the lane's 16-byte chunk of each load part from the tile's first key (tiles
  // inside the cache): parts 0..7 raw row 8w + j, parts 8..9 rotated row 8w + 4(j-8) + l/16
  uint32_t part_off[10];
#pragma unroll
  for (int j = 0; j < 10; ++j) {
    if (j < 8) {
      const int row = 8 * wu + j;
      part_off[j] = (uint32_t)(row * raw_row + 16 * (l ^ swz(row)));
    } else {
      const int row = 8 * wu + 4 * (j - 8) + (l >> 4);
      part_off[j] = (uint32_t)(row * rot_row + 16 * ((l & 15) ^ swz(row)));
    }
  }
  // the general form (any tile, rows past the cache clamped): the first two tiles and a tile
  // that reaches past the cache's end; the tiles inside the cache go through mfma_qk2_load
  auto issue_part = [&](int stg_off, int k0, int j) {
    const uint32_t raw_l = smem_lds + stg_off;
    const uint32_t rot_l = raw_l + kRawBytes;
    const int last = a.n_kv - 1 - k0;
    const bool tail = last < kNK - 1;
    const int ln = opaque(l);
    if (j < 8) {
      const int row = 8 * wu + j;
      const int rr = tail ? min(row, last) : row;
      const char* src = uniform_ptr((const char*)kraw_b + ((int64_t)k0 + rr) * raw_row);
      dma16(src + (uint32_t)(16 * (ln ^ swz(row))), raw_l + row * 1024);
    } else {
      const int row = 8 * wu + 4 * (j - 8) + (ln >> 4);
      const int rr = tail ? min(row, last) : row;
      const char* base = uniform_ptr(krot_b + (int64_t)k0 * rot_row);
      dma16(base + (uint32_t)(rr * rot_row + 16 * ((ln & 15) ^ swz(row))),
            rot_l + (8 * wu + 4 * (j - 8)) * 256);
    }
  };

  // ---- S^T of the tile in the stage at stg_off for the wave's 32 rows: K fragments 4 reads
  // ahead of their MFMA behind scheduling fences; the ten load parts of tile dma_k0 into the
  // stage at dma_off go out with MFMA pairs 1, 2, 4, 5, ..., 13, 14 (`inside`: that tile lies
  // wholly inside the cache, so the loads sit in the pairs' asm and take the precomputed lane
  // offsets; otherwise they follow the pairs in their general, clamped form); `hook(p)` runs
  // after pair p, inside its fence ---------------------------------------------------------------
  auto kld_at = [&](int stg_off, int s) {
    if (s < 8) return *(const bf16x8*)(smem + stg_off + kRawBytes + n * 256 + qk_off[s]);
    return *(const bf16x8*)(smem + stg_off + n * 1024 + 256 * (s >> 3) + qk_off[s & 7]);
  };
  auto scores = [&](auto inside, int stg_off, int dma_off, int dma_k0, auto&& hook, bf16x8* kf) {
    f32x16 acc;
    auto kld = [&](int s) { return kld_at(stg_off, s); };
    const char* rawb = uniform_ptr((const char*)kraw_b + (int64_t)dma_k0 * raw_row);
    const char* rotb = uniform_ptr(krot_b + (int64_t)dma_k0 * rot_row);
    const uint32_t lds_d = __builtin_amdgcn_readfirstlane(smem_lds + dma_off);
#pragma unroll
    for (int s = 0; s < 32; s += 2) {
      const int p = s / 2;   // load parts with pairs 1, 2, 4, 5, 7, 8, 10, 11, 13, 14
      const int j = p - 1 - p / 3;
      if (decltype(inside)::value && p % 3 != 0) {
        const uint32_t lrow = __builtin_amdgcn_readfirstlane(j < 8 ? (8 * wu + j) * 1024
                                                                    : kRawBytes + (8 * wu + 4 * (j - 8)) * 256);
        mfma_qk2_load(acc, kf[s % kDepthK], q[s], kf[(s + 1) % kDepthK], q[s + 1], s, j < 8 ? rawb : rotb,
                      part_off[j], lds_d, lrow);
      } else {
        mfma_qk2(acc, kf[s % kDepthK], q[s], kf[(s + 1) % kDepthK], q[s + 1], s);
      }
      if (s + kDepthK < 32) {
        kf[s % kDepthK] = kld(s + kDepthK);
        kf[(s + 1) % kDepthK] = kld(s + 1 + kDepthK);
      }
      if (!decltype(inside)::value && p % 3 != 0) issue_part(dma_off, dma_k0, j);
      hook(p);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the VALU reads the result next: the 12 wait states of an 8-pass MFMA's result
    asm volatile("s_nop 7\n\ts_nop 3" ::: "memory");
    return acc;
  };

  // ---- V^T fragment j = (ks, dt) = (j/16, j%16) of the tile in the stage at stg_off ---------
  auto vload = [&](int stg_off, int j) {
    const int ks = j >> 4, dt = j & 15;
    const char* p = smem + stg_off + v_dt[dt & 3] + 256 * (dt >> 2) + (16 * ks) * 1024;
    const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + v_e[0]));
    const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + v_e[1]));
    bf16x8 vv;
    vv[0] = v0[0]; vv[1] = v0[1]; vv[2] = v0[2]; vv[3] = v0[3];
    vv[4] = v1[0]; vv[5] = v1[1]; vv[6] = v1[2]; vv[7] = v1[3];
    return vv;
  };

  // Online-softmax state of the lane's row.  l_part: sum of the exact p (for the LSE); w_part:
  // sum of the bf16-rounded p that the PV product uses (O is normalised by it, so a dominant key's
  // value comes out exactly).  pass 0: the pass; 1: the reference follows every tile's maximum
  // (after a flag); 2: the pass again against the exact maxima.
  float m_used = -INFINITY, l_part = 0.0f, w_part = 0.0f;
  float neg_mu = 0.0f;   // -m_used, or 0 while the row has no reference (the exponents' bias)
  bool need_ref = true;   // some row of the wave has no reference yet (wave-uniform)
  int pass = 0;
  f32x16 o[16];

  // p = exp2(s * scale_log2 - m) for scores e, e+1 into pk: a masked score (-inf) gives 0; a row
  // without any valid key so far has m = -inf and only masked scores, so any finite reference gives
  // the same zeros.  An exponent above 128 gives inf, which the end-of-pass check of the sums
  // catches, so the raw v_exp_f32 suffices.  psum: the exact p;
  // wsum: the bf16-rounded p that the PV product uses (exact products by one).
  // Sums go to partial accumulators (psum[e/2 % 4], wsum[e/2 % 2]) so that the adds do not form
  // one long dependent chain (one wave per SIMD exposes every VALU latency).
  auto exp_pair = [&](const float* sv, int e, float neg_m, bf16x8* pk, float* psum, float* wsum) {
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], scale_log2, neg_m));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e + 1], scale_log2, neg_m));
    const bf16x2 pb = {(bf16)p0, (bf16)p1};
    // keys 0..7 of the tile start the partial sums (e < 8: psum[e/2]; e < 4: wsum[e/2])
    psum[(e >> 1) & 3] = e < 8 ? p0 + p1 : psum[(e >> 1) & 3] + (p0 + p1);
    wsum[(e >> 1) & 1] = __builtin_amdgcn_fdot2_f32_bf16(pb, bf16x2{(bf16)1.0f, (bf16)1.0f},
                                                         e < 4 ? 0.0f : wsum[(e >> 1) & 1], false);
    pk[e >> 3][e & 7] = pb[0];
    pk[e >> 3][(e & 7) + 1] = pb[1];
  };

  // The scores of tile i (raw, in sv): mask to each row's interval, reference of the row (the
  // first tile with a valid key sets it from its row maximum, O of the row being still 0), and the
  // probabilities of keys 0..15 of the tile (pk[0]).
  auto softmax_head = [&](float* sv, int i, bool full, bf16x8* pk, float& neg_m, float* psum, float* wsum) {
    const int k0 = k0_of(i);
    if (!full) {
      const int r = regime_of(i);
      const int lo_eff = s_lo[r][pos_in_blk] - k0, hi_eff = s_hi[r][pos_in_blk] - k0;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kk = 8 * (e >> 2) + 4 * half + (e & 3);
        if (kk < lo_eff || kk > hi_eff) sv[e] = -INFINITY;
      }
    }
    // the row maximum (a tree of 3-input maxima and the exchange with the row's other half), only
    // while some row of the wave has no reference yet, and in pass 1
    if (pass == 1 || need_ref) {
      float m6[6];
#pragma unroll
      for (int k = 0; k < 5; ++k) m6[k] = fmaxf(fmaxf(sv[3 * k], sv[3 * k + 1]), sv[3 * k + 2]);
      m6[5] = sv[15];
      float mx = fmaxf(fmaxf(fmaxf(m6[0], m6[1]), m6[2]), fmaxf(fmaxf(m6[3], m6[4]), m6[5]));
      auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw2[0]), __uint_as_float(sw2[1])) * scale_log2;
      m_used = (pass == 1 || m_used == -INFINITY) ? fmaxf(m_used, mx) : m_used;
      neg_mu = m_used == -INFINITY ? 0.0f : -m_used;
      need_ref = __ballot(m_used == -INFINITY) != 0;
    }
    neg_m = neg_mu;
#pragma unroll
    for (int e = 0; e < 8; e += 2) exp_pair(sv, e, neg_m, pk, psum, wsum);
  };

  // O^T += V^T P^T for the tile in the stage at stg_off, MFMA j = (ks, dt) = (j/16, j%16), V^T
  // fragments 3 reads ahead behind scheduling fences (the first three, vf, read by the caller);
  // `between(j)` runs after MFMA j
  auto values = [&](int stg_off, const bf16x8* pk, auto&& between, bf16x8* vf) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      o[j & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j % kDepthV], pk[j >> 4], o[j & 15], 0, 0, 0);
      if (j + kDepthV < 32) vf[j % kDepthV] = vload(stg_off, j + kDepthV);
      between(j);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (;;) {
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) o[dt] = f32x16{};
    l_part = w_part = 0.0f;
    if (n_tiles > 0) {
      // tiles 0 and 1 into stages 0 and 1
      const int k00 = k0_of(0), k01 = k0_of(min(1, n_tiles - 1));
#pragma unroll
      for (int j = 0; j < 10; ++j) issue_part(0, k00, j);
#pragma unroll
      for (int j = 0; j < 10; ++j) issue_part(kStageBytes, k01, j);
      load_qrot(regime_of(0));
    }
    // the Q fragments are complete before the tile loop (its wait counts cannot see the tile loads)
    wait_vm0();
    int cur_r = n_tiles > 0 ? regime_of(0) : 0;
    // byte offsets of the stages of tiles i, i+1, i+2 (rotated every tile)
    int off_c = 0, off_n = kStageBytes, off_d = 2 * kStageBytes;

    for (int i = 0; i < n_tiles; ++i) {
      // tile i has landed (the ten loads per wave of tile i+1 may still be in flight); the stage of
      // tile i+2 was last read by the previous tile
      __builtin_amdgcn_s_waitcnt(0x0F70 | 10);   // vmcnt(10), expcnt and lgkmcnt open
      __syncthreads();
      // the first K fragments go out first: the scalar work below runs in their LDS latency
      bf16x8 kf[kDepthK];
#pragma unroll
      for (int j = 0; j < kDepthK; ++j) kf[j] = kld_at(off_c, j);
      __builtin_amdgcn_sched_barrier(0);
      const int r = regime_of(i);
      if (r != cur_r) {
        // the compiler's wait counts do not see the tile loads in flight: settle everything so
        // that the score MFMAs find the new fragments without further waits
        load_qrot(r);
        wait_vm0();
        cur_r = r;
      }
      // scores of tile i, with the loads of tile i+2 (past the end: the last tile again, into a
      // stage no longer read, which keeps ten loads per wave and tile in flight)
      const int dk0 = k0_of(min(i + 2, n_tiles - 1));
      // the tile lies inside every row's interval (no masking)
      const int k0i = k0_of(i);
      const bool full = sel(i, full_lo[0], full_lo[1], full_lo[2]) <= k0i &&
                        k0i + kNK - 1 <= sel(i, full_hi[0], full_hi[1], full_hi[2]);
      // the first V^T fragments of the tile go out with the last two score pairs (their LDS
      // latency then hides under those MFMAs and the softmax)
      bf16x8 vf[kDepthV];
      auto hook = [&](int p) {
        if (p == 14) {
          vf[0] = vload(off_c, 0);
          vf[1] = vload(off_c, 1);
        }
        if (p == 15) vf[2] = vload(off_c, 2);
      };
      const f32x16 acc = a.n_kv - 1 - dk0 >= kNK - 1 ? scores(std::true_type{}, off_c, off_d, dk0, hook, kf)
                                                     : scores(std::false_type{}, off_c, off_d, dk0, hook, kf);
      float sv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) sv[e] = acc[e];
      bf16x8 pk[2];
      float neg_m, psum[4], wsum[2];
      softmax_head(sv, i, full, pk, neg_m, psum, wsum);
      // O^T of tile i; the probabilities of keys 16..31 (pk[1], first used by MFMA 16) are formed
      // after MFMAs 1, 4, 7, 10
      values(off_c, pk, [&](int j) {
        if (j < 12 && j % 3 == 1) exp_pair(sv, 8 + 2 * (j / 3), neg_m, pk, psum, wsum);
      }, vf);
      l_part += (psum[0] + psum[1]) + (psum[2] + psum[3]);
      w_part += wsum[0] + wsum[1];
      const int t_off = off_c;
      off_c = off_n;
      off_n = off_d;
      off_d = t_off;
    }
    // pass 0 keeps its result while every row's sums of p stay below kSumMax; otherwise (an inf
    // or NaN included) the workgroup raises its flag
    if (pass == 0 && __ballot(!(l_part < kSumMax && w_part < kSumMax)) != 0 && l == 0) s_flag = 1;
    // every wave's flag write and tile loads are complete; the stages may be reloaded
    wait_vm0();
    __syncthreads();
    // a flagged workgroup runs the sequence again: first for the exact row maxima, then in full
    if (pass == 2 || (pass == 0 && s_flag == 0)) break;
    ++pass;
  }

  // ---- epilogue: normaliser and natural-log lse from the row totals of both halves ----------
  float l_tot, w_tot;
  {
    auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part), __float_as_uint(l_part), false, false);
    l_tot = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
    auto sw3 = __builtin_amdgcn_permlane32_swap(__float_as_uint(w_part), __float_as_uint(w_part), false, false);
    w_tot = __uint_as_float(sw3[0]) + __uint_as_float(sw3[1]);
  }
  const bool nonempty = l_tot > 0.0f && w_tot > 0.0f;
  const float inv = nonempty ? 1.0f / w_tot : 0.0f;
  // O leaves through LDS (the stages are free now): each wave writes its 32 rows x 256 (bf16) or
  // 128 (fp32) dims of the output into its own rows of 528 bytes (16 of padding keep the writes of
  // the 32 rows of a column apart in the banks), then stores whole 512-byte row segments, 32 lanes
  // x 16 bytes per row, instead of 16-byte pieces of 32 rows per store.
  auto write_out = [&](auto bf) {
    constexpr bool BF = decltype(bf)::value;
    constexpr int kEs = BF ? 2 : 4;
    constexpr int kGroup = BF ? 8 : 4;   // dim tiles per round
    constexpr int kRowB = 528;
    char* own = smem + w * 32 * kRowB;
#pragma unroll
    for (int g0 = 0; g0 < 16; g0 += kGroup) {
#pragma unroll
      for (int dt = g0; dt < g0 + kGroup; ++dt) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v;
          v[0] = o[dt][4 * q4 + 0];
          v[1] = o[dt][4 * q4 + 1];
          v[2] = o[dt][4 * q4 + 2];
          v[3] = o[dt][4 * q4 + 3];
          v *= inv;
          char* at = own + n * kRowB + (32 * (dt - g0) + 8 * q4 + 4 * half) * kEs;
          if constexpr (BF) {
            bf16x4 vb;
            vb[0] = (bf16)v[0];
            vb[1] = (bf16)v[1];
            vb[2] = (bf16)v[2];
            vb[3] = (bf16)v[3];
            *(bf16x4*)at = vb;
          } else {
            *(f32x4*)at = v;
          }
        }
      }
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int r = 2 * it + half;   // the wave's row r: lanes 0..31 even rows, 32..63 odd
        const int rho_r = 32 * w + r;
        const int t = qb * QB + rho_r / G;
        const u32x4 seg = *(const u32x4*)(own + r * kRowB + 16 * n);
        if (t < a.T) {
          const int64_t head = ((int64_t)b * a.T + t) * a.Hq + (int64_t)g * G + rho_r % G;
          *(u32x4*)((char*)a.o_final + (head * kD + 32 * g0) * kEs + 16 * n) = seg;
        }
      }
    }
  };
  if (a.o_final_bf16)
    write_out(std::true_type{});
  else
    write_out(std::false_type{});
  if (row_valid) {
    if (half == 0) a.lse_final[rowhead] = nonempty ? (m_used + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_fused_bf16(const AttnArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int QB = 128 / G;
  const int n_qblocks = (a.T + QB - 1) / QB;
  const int64_t blocks = (int64_t)n_qblocks * a.B * a.Hkv;
  if (blocks <= 0) return hipSuccess;
  dim3 grid((unsigned)blocks), block(256);
  switch (G) {
    case 1: hipLaunchKernelGGL((attn_fused_kernel<1>), grid, block, 0, stream, a, n_qblocks); break;
    case 2: hipLaunchKernelGGL((attn_fused_kernel<2>), grid, block, 0, stream, a, n_qblocks); break;
    case 4: hipLaunchKernelGGL((attn_fused_kernel<4>), grid, block, 0, stream, a, n_qblocks); break;
    case 8: hipLaunchKernelGGL((attn_fused_kernel<8>), grid, block, 0, stream, a, n_qblocks); break;
    case 16: hipLaunchKernelGGL((attn_fused_kernel<16>), grid, block, 0, stream, a, n_qblocks); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dca
