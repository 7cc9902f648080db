// Split-KV regime passes for decode over a quantized key cache (q8_0 or q4_0), on gfx950.
//
// Same math as the bf16 decode passes (DCA feature page, "DCA algorithm", "Implementation
// progress + Section-D simplification", "Section C2b"), over keys stored in blocks of 32
// consecutive dims of a (key, KV head) row with one fp16 scale d each (the pages run DCA over such
// caches, reading the codes inside the kernel: Upstream Sync entry
// "0119-p0-dcaon-scalar-inregister").  q8_0: int8 codes q, value d * q (544 bytes per key and head
// instead of 1024).  q4_0: 4-bit codes n packed two per byte in dim order (dim 2j in the low nibble
// of byte j), value d * (n - 8) (288 bytes).
//  * Each workgroup (4 waves) handles one (query row, KV head, span of keys) as in the bf16
//    passes.  64-key tiles of codes (32 or 16 KiB) and scales (2 KiB) come in by direct
//    global->LDS loads, double buffered; two workgroups share a CU.
//  * No dequantized copy of the tile is stored.  The score operand (key rows, 8 dims per lane) is
//    read as codes and turned into fp16 d*q in registers; the value operand (8 keys of one dim per
//    lane) is read with gfx950's 8-bit transposing LDS read as exact integer codes (q4_0: one read
//    gives two dims, the low and the high nibbles), and each key's block scale multiplies its
//    probability instead (from a small transposed copy of the tile's scales).  Both products run
//    as fp16 MFMA 16x16x32 (the query's raw dims are converted from bf16 to fp16 once per row, the
//    probabilities are fp16).
//  * Code rows sit in LDS with their 16-byte chunks XOR-swizzled by the row's low 4 bits (the
//    loads pick the global chunk that belongs at each position), so that both the 16-row score
//    reads and the 8-row transposing reads hit 16 distinct chunk slots.
//  * The rotary dims of a key are rotated in registers at j mod c from the fp64-built cos/sin
//    tables, lo[p & 63] and hi[p >> 6] by angle addition.  With c a multiple of 64 (and at most 8
//    query heads per KV head: the TAB form) a 64-key tile sits at p0 + row under one hi row, and
//    <q, R(hi + lo) k> = <R(-hi) q, R(lo) k>: the workgroup turns the query's rotary pairs by
//    minus the tile's hi angles once per tile, and each key takes only its row's lo entry, which
//    the lane keeps in registers.  Otherwise each key composes both tables (the general form).
//  * Score codes to fp16, exactly: an int8 code by one sign-extending conversion; a 4-bit code n
//    by placing it under the fp16 exponent of 1024 (bit pattern 0x6400 | n = 1024 + n) and
//    subtracting 1032, or, for a high nibble taken in place, 1024 + 16 n minus 1152 = 16 (n - 8)
//    with the scale divided by 16.  One fp16 multiply by d then gives the value (one rounding).
//  * Value codes need no arithmetic: a byte under a zero high byte is the fp16 subnormal
//    byte * 2^-24, exact (q8_0: code ^ 0x80 = code + 128; q4_0: the low nibble n, the high nibble
//    in place as 16 n); the products with the weights are exact in the fp32 accumulators, and
//    the offset (128 or 8) comes back out at the end from the sum of the weights times the
//    scales, which one more MFMA per block accumulates against a ones operand.
//  * The operands of each product are read from LDS together, before the first use, so that the
//    MFMAs do not wait out one LDS round trip each.
//  * q4_0 score fragments hold their 8 dims in the order the nibble extraction yields,
//    (0, 2, 4, 6, 1, 3, 5, 7); the query fragments are stored in the same order.
#include "common.h"

namespace dca {
namespace {

constexpr int kD = 512;
constexpr int kTile = 64;
constexpr int kScaleBytes = kTile * kD / 32 * 2;  // 2 KiB of fp16 scales per tile, [key][block]
constexpr float kTau = 8.0f;
constexpr int kPad = kTile + 8;   // row stride (halves) of the weight and transposed-scale buffers

// stage layout per code width: codes [64 rows][kRow bytes], scales, the tile's hi table row
template <int BITS>
struct QLayout {
  static constexpr int kRow = kD * BITS / 8;             // 512 (q8_0) or 256 (q4_0) bytes per key
  static constexpr int kCodeBytes = kTile * kRow;
  static constexpr int kRowsPerLoad = 1024 / kRow;        // rows one 64-lane 16-byte load covers
  static constexpr int kHiRow = kCodeBytes + kScaleBytes;
  static constexpr int kStageBytes = kHiRow + 512;
};

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

// a value the compiler cannot see through, so that lane-dependent address arithmetic is redone in
// the tile loop instead of being hoisted out of it into long-lived registers
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// eight int8 codes (two words, byte i = element i) -> the exact integers as fp16: each byte is
// sign-extended and converted by an SDWA-form int16 -> fp16 conversion that writes one half of the
// destination (one instruction per code)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ f16x8 codes8(uint32_t lo, uint32_t hi) {
  uint32_t r0, r1, r2, r3;
  asm("v_cvt_f16_i16_sdwa %0, sext(%4) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
      "v_cvt_f16_i16_sdwa %1, sext(%4) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
      "v_cvt_f16_i16_sdwa %2, sext(%5) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
      "v_cvt_f16_i16_sdwa %3, sext(%5) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
      "v_cvt_f16_i16_sdwa %0, sext(%4) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1\n\t"
      "v_cvt_f16_i16_sdwa %1, sext(%4) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3\n\t"
      "v_cvt_f16_i16_sdwa %2, sext(%5) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1\n\t"
      "v_cvt_f16_i16_sdwa %3, sext(%5) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(lo), "v"(hi));
  const uint32_t r[4] = {r0, r1, r2, r3};
  return __builtin_bit_cast(f16x8, r);
}
#pragma clang diagnostic pop

// eight 4-bit codes of one word (element e at bits 4e..4e+3) -> fp16 in the order
// (0, 2, 4, 6, 1, 3, 5, 7): the low nibbles of the four bytes are the even elements, n - 8; the
// high nibbles the odd ones, taken in place as 16 (n - 8) (byte & 0xF0 under the exponent of 1024
// is 1024 + 16 n; minus 1152); each byte pair goes under the exponent by one byte permute
__device__ __forceinline__ f16x8 nibbles8(uint32_t w) {
  const uint32_t ev = w & 0x0F0F0F0Fu, od = w & 0xF0F0F0F0u;
  const f16x2 off = {(_Float16)1032.0f, (_Float16)1032.0f}, off16 = {(_Float16)1152.0f, (_Float16)1152.0f};
  f16x2 h[4];
  h[0] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, ev, 0x04010400u)) - off;
  h[1] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, ev, 0x04030402u)) - off;
  h[2] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, od, 0x04010400u)) - off16;
  h[3] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, od, 0x04030402u)) - off16;
  f16x8 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = h[i][0];
    out[2 * i + 1] = h[i][1];
  }
  return out;
}

// eight bytes (two words, byte i = element i) -> fp16 subnormals byte * 2^-24, exactly: each byte
// goes under a zero high byte by one byte permute per pair.  The value product takes its codes in
// this form (q8_0: code + 128; q4_0: n, or 16 n for a high nibble masked in place) and removes the
// offset at the end from the sum of its weights (see the value product)
__device__ __forceinline__ f16x8 bytes_sub8(uint32_t a, uint32_t b) {
  const uint32_t h[4] = {__builtin_amdgcn_perm(0u, a, 0x0C010C00u), __builtin_amdgcn_perm(0u, a, 0x0C030C02u),
                         __builtin_amdgcn_perm(0u, b, 0x0C010C00u), __builtin_amdgcn_perm(0u, b, 0x0C030C02u)};
  return __builtin_bit_cast(f16x8, h);
}

// max and sum of a value over the four 16-lane rows of the wave (lanes l, l ^ 16, l ^ 32, l ^ 48),
// by gfx950's row-swapping lane permutes (each swap hands a lane its partner row's value)
__device__ __forceinline__ float max_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Rotate the fp16 pair (x0, x1) held in half H of words a and b by (cs, sn), in place:
// (x0 cs - x1 sn, x0 sn + x1 cs), each product and sum in fp32 and one rounding to fp16 at the
// end, four mixed-precision fmas per pair (the fp16 operands are read from their halves directly)
template <int H>
__device__ __forceinline__ void rot_pair(uint32_t& a, uint32_t& b, float cs, float sn) {
  float t, u;   // t = -x1 sn, u = x1 cs
  if constexpr (H == 0)
    asm("v_fma_mix_f32 %2, %1, -%5, 0 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mix_f32 %3, %1, %4, 0 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixlo_f16 %1, %0, %5, %3 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixlo_f16 %0, %0, %4, %2 op_sel_hi:[1,0,0]"
        : "+v"(a), "+v"(b), "=&v"(t), "=&v"(u)
        : "v"(cs), "v"(sn));
  else
    asm("v_fma_mix_f32 %2, %1, -%5, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mix_f32 %3, %1, %4, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %1, %0, %5, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %0, %4, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "+v"(a), "+v"(b), "=&v"(t), "=&v"(u)
        : "v"(cs), "v"(sn));
}

// position p of a q4_0 score fragment holds element perm4(p) of its 8 dims
__device__ __forceinline__ constexpr int perm4(int p) { return 2 * (p & 3) + (p >> 2); }

template <int BITS>
__device__ __forceinline__ f16x8 order_frag(const f16x8& v) {
  if constexpr (BITS == 8) {
    return v;
  } else {
    f16x8 o;
#pragma unroll
    for (int p = 0; p < 8; ++p) o[p] = v[perm4(p)];
    return o;
  }
}

// TAB: c is a multiple of 64, so a 64-key tile's positions are p0 + row with p0 a multiple of 64
// (see the rotation notes at the top)
template <int BITS, bool TAB>
__global__ __launch_bounds__(256, 2) void attn_decode_quant_kernel(DecodeArgs da) {
  using LY = QLayout<BITS>;
  constexpr int kRow = LY::kRow, kCodeBytes = LY::kCodeBytes, kStageBytes = LY::kStageBytes;
  constexpr int kHiRow = LY::kHiRow, kRpl = LY::kRowsPerLoad;
  const AttnArgs& a = da.base;
  __shared__ __attribute__((aligned(1024))) char stage[2 * kStageBytes];
  // P[head][key] and the tile's scales [block][key], rows padded to kPad halves (bank spread)
  __shared__ __attribute__((aligned(16))) _Float16 pbuf[16 * kPad];
  __shared__ __attribute__((aligned(16))) _Float16 sT[16 * kPad];
  __shared__ __attribute__((aligned(16))) char qsm[16 * 256];          // rotated query dims, fp16
  __shared__ float smax[4][16], ssum[4][16], wsum[4][16];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t stage_lds = (uint32_t)(uintptr_t)(lds_char*)stage;
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
  const char* codes_b = (const char*)a.k_raw + ((int64_t)b * da.n_rows * a.Hkv + g) * kRow;
  const uint16_t* scales_b = da.k_scales + ((int64_t)b * da.n_rows * a.Hkv + g) * (kD / 32);
  const int half_rot = a.n_rot / 2;   // 64
  const float scale_log2 = a.scale * kLog2e;

  // query fragments (fp16): B operand lane l holds Q[head hcol][32 s + 8 gq .. +7] (q4_0: in the
  // fragment order); the raw dims come in as bf16 and are converted once into registers, the
  // rotated dims (s < 4) are read per tile from LDS (head h's 16-byte chunk c at position c ^ h)
  f16x8 q[16];
  {
    const bf16* qt = (const bf16*)a.q_tail + rowhead * a.q_tail_hs + 8 * gq;
#pragma unroll
    for (int s = 4; s < 16; ++s) {
      const bf16x8 v = *(const bf16x8*)(qt + 32 * s - 128);
      f16x8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = head_ok ? (_Float16)(float)v[e] : (_Float16)0.0f;
      q[s] = order_frag<BITS>(h);
    }
  }
  const int qrow = 16 * w + hcol;   // the lane's key row in the score product

  // Fragment position p of the rotary k-steps holds dim 32 s + 8 gq + dim_of(p).
  auto dim_of = [](int p) { return BITS == 8 ? p : perm4(p); };
  // TAB: the lane's lo entries (its key row, its 16 pairs) stay in registers
  float2 lo_q[16];
  if constexpr (TAB) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        lo_q[8 * s + e] = da.rot_lo[qrow * half_rot + 32 * s + 8 * gq + dim_of(e)];
  }

  // TAB (G <= 8): thread t turns the query pairs (f, f + 64) and (f + 1, f + 65), f = 2 (t & 31),
  // of head t >> 5 by minus the tile's hi angles and stores them in qsm (fragment order, chunk
  // swizzle)
  auto rotate_query = [&](const f16x2 x0, const f16x2 x1, const float4 hh) {
    const int t = opaque(tid);
    const int h = t >> 5, f = 2 * (t & 31);
    if (h < G) {
      const float a0 = (float)x0[0], a1 = (float)x0[1];
      const float b0 = (float)x1[0], b1 = (float)x1[1];
      const f16x2 y0 = {(_Float16)fmaf(a0, hh.x, b0 * hh.y), (_Float16)fmaf(a1, hh.z, b1 * hh.w)};
      const f16x2 y1 = {(_Float16)fmaf(b0, hh.x, -a0 * hh.y), (_Float16)fmaf(b1, hh.z, -a1 * hh.w)};
      char* c0 = qsm + h * 256 + 16 * ((f >> 3) ^ h);
      char* c1 = qsm + h * 256 + 16 * ((8 + (f >> 3)) ^ h);
      const int e = f & 7;   // even: elements e, e + 1 of the chunk
      if constexpr (BITS == 8) {
        *(f16x2*)(c0 + 2 * e) = y0;
        *(f16x2*)(c1 + 2 * e) = y1;
      } else {   // element e sits at position e / 2, element e + 1 at e / 2 + 4
        ((_Float16*)c0)[e >> 1] = y0[0];
        ((_Float16*)c0)[(e >> 1) + 4] = y0[1];
        ((_Float16*)c1)[e >> 1] = y1[0];
        ((_Float16*)c1)[(e >> 1) + 4] = y1[1];
      }
    }
  };

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
    const int kt0 = lo / kTile, kt1 = hi / kTile;
    const _Float16* qrot_r = (const _Float16*)a.q_rot[r];
    {
      // thread t: head h = t >> 4, dims 8 (t & 15) .. +7 (TAB: only the heads past G, zero)
      const int h = tid >> 4, c = tid & 15;
      if (!TAB || h >= G) {
        f16x8 v{};
        if (h < G) v = *(const f16x8*)(qrot_r + (bt * a.Hq + (int64_t)g * G + h) * a.q_rot_hs + 8 * c);
        *(f16x8*)(qsm + h * 256 + 16 * (c ^ h)) = order_frag<BITS>(v);
      }
    }
    f16x2 qx0 = {}, qx1 = {};   // TAB: the thread's unturned query pairs (see rotate_query)
    if constexpr (TAB) {
      const int h = tid >> 5, f = 2 * (tid & 31);
      if (h < G) {
        const _Float16* src = qrot_r + (bt * a.Hq + (int64_t)g * G + h) * a.q_rot_hs + f;
        qx0 = *(const f16x2*)src;
        qx1 = *(const f16x2*)(src + half_rot);
      }
      const int hr = kt0 % (da.chunk / kTile);
      rotate_query(qx0, qx1, *(const float4*)(da.rot_hi + (int64_t)hr * half_rot + f));
    }
    f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{};
    // wsb[bb]: per head, the sum over keys of the weight times the key's scale of block 4 w + bb
    // (every row of the 16x16 tile the same), which takes the codes' offset out of O at the end
    f32x4 wsb[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) wsb[bb] = f32x4{};
    // l_part: exact row sum (LSE); w_part: sum of the fp16 weights the PV product uses (O's
    // normaliser, so that weights and normaliser agree)
    float m_used = -INFINITY, l_part = 0.0f, w_part = 0.0f;

    // tile k0..k0+63 by direct global->LDS loads into stage buf: wave w the code rows
    // 16w..16w+15 (kRpl rows of kRow bytes per load; position p of row r receives global chunk
    // p ^ (r & 15)), waves 0 and 1 the scale rows 0..31 and 32..63 (lane l the slot l%2 of row
    // r = l/2, which receives the row's half (l%2) ^ bit 3 of r), lanes 0..31 of wave 2 (TAB) the
    // hi table row of the tile after it; rows outside the region re-read its first or last cell
    // (their scores are masked)
    auto issue = [&](int buf, int k0, int hr_next) {
      const uint32_t base = stage_lds + buf * kStageBytes;
      const int ln = opaque(l);
      // tile row r reads region row k0 - key0 + r, clamped to the region: r in [first, last]
      const int first = max(da.key0 - k0, 0), last = key_end - 1 - k0;
      const uint32_t key_bytes = (uint32_t)a.Hkv * kRow, key_sbytes = (uint32_t)a.Hkv * (kD / 32) * 2;
      const char* cb = uniform_ptr(codes_b + (int64_t)(k0 - da.key0) * key_bytes);
      // row 16 wu + kRpl i + hb (hb = the lane's row within the load) has swizzle key
      // kRpl i + hb = kRpl i ^ hb, so the lane's chunk offset is x ^ 16 kRpl i
      constexpr int kLanesPerRow = 64 / kRpl;
      const int hb = ln / kLanesPerRow;
      const uint32_t x = 16 * ((ln % kLanesPerRow) ^ hb);
      if (first == 0 && last >= kTile - 1) {   // whole tile inside the region: rows step by kRpl keys
        const uint32_t r0 = __umul24((uint32_t)(16 * wu + hb), key_bytes);
#pragma unroll
        for (int i = 0; i < 16 / kRpl; ++i)
          dma16_off<true>(cb, r0 + kRpl * i * key_bytes + (x ^ (16 * kRpl * i)), base + (16 * wu + kRpl * i) * kRow);
      } else {
#pragma unroll
        for (int i = 0; i < 16 / kRpl; ++i) {
          const int row = 16 * wu + kRpl * i + hb;
          dma16_off<true>(cb, __umul24((uint32_t)min(max(row, first), last), key_bytes) + (x ^ (16 * kRpl * i)),
                    base + (16 * wu + kRpl * i) * kRow);
        }
      }
      if (wu < 2) {
        const int row = 32 * wu + (ln >> 1);
        const char* sb = uniform_ptr((const char*)scales_b + (int64_t)(k0 - da.key0) * key_sbytes);
        // (not nontemporal: the scale rows of the KV heads share cache lines, which the other
        // head's workgroup reads as well)
        // LDS slot (row, half) receives the row's global half ^ bit 3 of the row, so that the
        // 16-row reads of one half spread over all banks
        dma16_off(sb, __umul24((uint32_t)min(max(row, first), last), key_sbytes) + 16 * ((ln & 1) ^ ((row >> 3) & 1)),
                  base + kCodeBytes + wu * 1024);
      }
      if (TAB && wu == 2 && ln < 32)   // hi row of the next tile (512 bytes: lanes 0..31)
        dma16_off(uniform_ptr((const char*)(da.rot_hi + (int64_t)hr_next * half_rot)), 16 * ln, base + kHiRow);
    };
    // TAB: tile kt's hi row is kt mod (c / 64); hr_ld follows the tile after the one being issued
    const int n_hi = TAB ? da.chunk / kTile : 1;
    int hr_ld = (kt0 + 1) % n_hi;
    issue(0, kt0 * kTile, hr_ld);

    for (int kt = kt0; kt <= kt1; ++kt) {
      const int cur = (kt - kt0) & 1;
      const int k0 = kt * kTile;
      // tile kt has landed (every wave's loads) and every wave is done with tile kt - 1
      wait_vm0();
      __syncthreads();
      if (kt < kt1) {
        hr_ld = hr_ld + 1 == n_hi ? 0 : hr_ld + 1;
        issue(cur ^ 1, k0 + kTile, hr_ld);
      }
      const char* st = stage + cur * kStageBytes;
      // lane-dependent offsets, recomputed per tile
      const int ln = opaque(l);
      const int lh = ln & 15, lg = ln >> 4;
      const int lrow = 16 * wu + lh;

      // ---- score operands, all read before any is used: the lane's key row of codes (dims
      // 32 s + 8 lg .. +7 for k-step s) and scales, the rotated query, the transposed scales' source
      const char* krow = st + lrow * kRow;
      f16x8 dsc[2];
      const int sh = 16 * ((lrow >> 3) & 1);   // the scale rows' half swizzle
      dsc[0] = *(const f16x8*)(st + kCodeBytes + lrow * 32 + sh);
      dsc[1] = *(const f16x8*)(st + kCodeBytes + lrow * 32 + (sh ^ 16));
      const uint2 d4 = *(const uint2*)(st + kCodeBytes + lrow * 32 + ((16 * (lg >> 1)) ^ sh) + 8 * (lg & 1));   // blocks 4lg..+3
      uint2 cw[16];   // q8_0: 8 codes; q4_0: 8 codes in .x
      if constexpr (BITS == 8) {
        // chunk (2 s + (lg >> 1)) ^ lh, bytes 8 (lg & 1): with s = 8 t + u that is byte
        // 16 ((lg >> 1) ^ (lh & 1)) + 32 (u ^ (lh >> 1)) + 256 t, so 8 addresses serve 16 reads
        const char* kb = krow + 8 * (lg & 1) + 16 * ((lg >> 1) ^ (lh & 1));
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const char* p = kb + 32 * (u ^ (lh >> 1));
          cw[u] = *(const uint2*)p;
          cw[u + 8] = *(const uint2*)(p + 256);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 16; ++s) cw[s].x = *(const uint32_t*)(krow + 4 * lg + 16 * (s ^ lh));   // chunk s, bytes 4 lg
      }
      f16x8 qs[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) qs[s] = *(const f16x8*)(qsm + lh * 256 + 16 * ((4 * s + lg) ^ lh));
      __builtin_amdgcn_sched_barrier(0);
      {
        uint16_t* t = (uint16_t*)sT + 4 * lg * kPad + lrow;
        t[0 * kPad] = (uint16_t)d4.x;
        t[1 * kPad] = (uint16_t)(d4.x >> 16);
        t[2 * kPad] = (uint16_t)d4.y;
        t[3 * kPad] = (uint16_t)(d4.y >> 16);
      }

      // ---- S^T for keys [16w, 16w+16): codes -> fp16 d*q in registers ------------------------
      // q4_0: the odd elements come as 16 (n - 8) and take d / 16 (exact for d >= 2^-10; below,
      // d / 16 is subnormal and the element's absolute error stays under 2^-25 * 128)
      f16x8 dsc16[2];
      if constexpr (BITS == 4) {
        const f16x8 r16 = {(_Float16)0.0625f, (_Float16)0.0625f, (_Float16)0.0625f, (_Float16)0.0625f,
                           (_Float16)0.0625f, (_Float16)0.0625f, (_Float16)0.0625f, (_Float16)0.0625f};
        dsc16[0] = dsc[0] * r16;
        dsc16[1] = dsc[1] * r16;
      }
      auto kfrag = [&](int s) {
        const _Float16 d = dsc[s >> 3][s & 7];
        if constexpr (BITS == 8) {
          const f16x8 dd = {d, d, d, d, d, d, d, d};
          return codes8(cw[s].x, cw[s].y) * dd;
        } else {
          const _Float16 d16 = dsc16[s >> 3][s & 7];
          const f16x8 dd = {d, d, d, d, d16, d16, d16, d16};
          return nibbles8(cw[s].x) * dd;
        }
      };
      f32x4 sacc = f32x4{};
      {
        f16x8 kr[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) kr[s] = kfrag(s);
        // rotate the rotary pairs (f, f + 64) of the lane's key by (cos, sin) of its angle (TAB:
        // the lo table entry of the key's row, the hi part is on the query; otherwise the key's
        // full position, composed from both tables by the angle-addition formulas)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          __builtin_amdgcn_sched_barrier(0);   // one half at a time: bounds the live table entries
          if constexpr (TAB) {
            struct W4 { uint32_t v[4]; };
            W4 x0 = __builtin_bit_cast(W4, kr[s]), x1 = __builtin_bit_cast(W4, kr[s + 2]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              rot_pair<0>(x0.v[j], x1.v[j], lo_q[8 * s + 2 * j].x, lo_q[8 * s + 2 * j].y);
              rot_pair<1>(x0.v[j], x1.v[j], lo_q[8 * s + 2 * j + 1].x, lo_q[8 * s + 2 * j + 1].y);
            }
            kr[s] = __builtin_bit_cast(f16x8, x0);
            kr[s + 2] = __builtin_bit_cast(f16x8, x1);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int f = 32 * s + 8 * lg + dim_of(e);
              const int pos = (int)((uint32_t)min(k0 + lrow, a.n_kv - 1) % (uint32_t)da.chunk);
              const float2 A = da.rot_lo[(pos & 63) * half_rot + f], Bv = da.rot_hi[(pos >> 6) * half_rot + f];
              const float cs = A.x * Bv.x - A.y * Bv.y;
              const float sn = A.y * Bv.x + A.x * Bv.y;
              const float x0 = (float)kr[s][e], x1 = (float)kr[s + 2][e];
              kr[s][e] = (_Float16)fmaf(x0, cs, -x1 * sn);
              kr[s + 2][e] = (_Float16)fmaf(x0, sn, x1 * cs);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 4; ++s) sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kr[s], qs[s], sacc, 0, 0, 0);
      }
#pragma unroll
      for (int s = 4; s < 16; ++s) sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kfrag(s), q[s], sacc, 0, 0, 0);
      // C layout: reg e = key 16w + 4 gq + e, column = head hcol; sv: raw scores (log2 units once
      // multiplied by scale_log2 > 0), -inf outside [lo, hi]
      float sv[4];
      if (k0 >= lo && k0 + kTile - 1 <= hi) {   // whole tile inside [lo, hi]
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[e] = sacc[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kk = k0 + 16 * wu + 4 * gq + e;
          sv[e] = (kk < lo || kk > hi) ? -INFINITY : sacc[e];
        }
      }
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = max_over_rows(mx) * scale_log2;
      if (gq == 0) smax[w][hcol] = mx;
      __syncthreads();   // also: the transposed scales are complete before the value reads, and
                         // every wave has read the rotated query of this tile
      if constexpr (TAB)
        if (kt < kt1) rotate_query(qx0, qx1, *(const float4*)(st + kHiRow + 16 * (opaque(tid) & 31)));
      // every tile holds a key of [lo, hi], so tmax is finite and so is m_used from here on:
      // masked scores give exp2(-inf) = 0
      const float tmax = fmaxf(fmaxf(smax[0][hcol], smax[1][hcol]), fmaxf(smax[2][hcol], smax[3][hcol]));
      const bool need = tmax > m_used + kTau;
      if (__ballot(need)) {
        const float m_new = need ? tmax : m_used;
        const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
        l_part *= alpha;
        w_part *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) wsb[bb] *= alpha;
        m_used = m_new;
      }
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], scale_log2, -m_used));
        l_part += p[e];
      }
      // the fp16 weights, packed in pairs; their sum (exact in fp32) by a dot with (1, 1)
      const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
      const f16x2 pv01 = {(_Float16)p[0], (_Float16)p[1]}, pv23 = {(_Float16)p[2], (_Float16)p[3]};
      w_part = __builtin_amdgcn_fdot2(pv23, one2, __builtin_amdgcn_fdot2(pv01, one2, w_part, false), false);
      *(uint2*)(pbuf + lh * kPad + 16 * wu + 4 * lg) = uint2{__builtin_bit_cast(uint32_t, pv01), __builtin_bit_cast(uint32_t, pv23)};
      __syncthreads();

      // ---- O^T += V^T P^T for dims [128w, 128w+128) ------------------------------------------
      // value operand: transposing reads of rows 32 ks + 8 lg + (lh >> 1), bytes 8 (lh & 1) of a
      // 16-byte chunk; swizzle key = the row's low 4 bits = 8 (lg & 1) + (lh >> 1).  Value chunk
      // j = 8 w + dt (q8_0) or 4 w + bb (q4_0) sits at j ^ pv_key: the wave's bits of j and the low
      // bits of j occupy disjoint bits, so their XORs are taken apart (one term per tile, one per
      // block).
      // q8_0: o[dt] holds dims 128 w + 16 dt + (4 gq .. +3); q4_0: o[2 bb] and o[2 bb + 1] hold
      // the even and odd dims 128 w + 32 bb + 8 gq + (0, 2, 4, 6) and (1, 3, 5, 7), the odd ones
      // times 16
      const int pv_row = 8 * lg + (lh >> 1);
      const int pv_key = pv_row & 15;
      const char* vrow =
          st + pv_row * kRow + 8 * (lh & 1) + 16 * (BITS == 8 ? (8 * wu) ^ (pv_key & 8) : (4 * wu) ^ (pv_key & 12));
      // operands of both halves, all read before any is used
      constexpr int kReads = BITS == 8 ? 8 : 4;
      f16x8 pb[2], d8[2][4];
      v2i cv[2][kReads];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        pb[ks] = *(const f16x8*)(pbuf + lh * kPad + 32 * ks + 8 * lg);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) d8[ks][bb] = *(const f16x8*)(sT + (4 * wu + bb) * kPad + 32 * ks + 8 * lg);
#pragma unroll
        for (int j = 0; j < kReads; ++j)
          cv[ks][j] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_v2i*)(lds_char*)(vrow + 32 * ks * kRow + 16 * (j ^ (pv_key & (BITS == 8 ? 7 : 3)))));
      }
      __builtin_amdgcn_sched_barrier(0);
      const f16x8 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                          (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          // the block's scale goes with the weights: P[h][key] * d[key][4w + bb] for keys
          // 32 ks + 8 gq .. +7; the codes enter as subnormals (code + offset) * 2^-24, so
          // O = 2^24 sum_keys (code + offset) 2^-24 p d - offset * sum_keys p d, the second sum
          // taken by one more product against ones
          const f16x8 pd = pb[ks] * d8[ks][bb];
          wsb[bb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pd, wsb[bb], 0, 0, 0);
          if constexpr (BITS == 8) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int dt = 2 * bb + h;   // chunk 8 w + dt; byte ^ 0x80 = code + 128
              o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  bytes_sub8((uint32_t)cv[ks][dt][0] ^ 0x80808080u, (uint32_t)cv[ks][dt][1] ^ 0x80808080u), pd, o[dt],
                  0, 0, 0);
            }
          } else {
            // chunk 4 w + bb = block 4 w + bb: byte i of the chunk holds dims 2 i (low nibble, n)
            // and 2 i + 1 (high nibble, taken in place as 16 n)
            const uint32_t c0 = (uint32_t)cv[ks][bb][0], c1 = (uint32_t)cv[ks][bb][1];
            o[2 * bb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                bytes_sub8(c0 & 0x0F0F0F0Fu, c1 & 0x0F0F0F0Fu), pd, o[2 * bb], 0, 0, 0);
            o[2 * bb + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                bytes_sub8(c0 & 0xF0F0F0F0u, c1 & 0xF0F0F0F0u), pd, o[2 * bb + 1], 0, 0, 0);
          }
        }
      }
    }

    // ---- combine the row sums of the 4 waves and store the partial ----------------------------
    const float ls = sum_over_rows(l_part), ws = sum_over_rows(w_part);
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
      float* orow = da.o_part + ((int64_t)slot * rows * a.Hq + rowhead) * kD + 128 * w;
      // O = (2^24 o - offset * wsb) / w: the scaling by 2^24 (2^20 for the high nibbles) is exact
      constexpr float k24 = 16777216.0f, k20 = 1048576.0f;
      if constexpr (BITS == 8) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *(f32x4*)(orow + 16 * dt + 4 * gq) = (o[dt] * k24 - wsb[dt >> 1] * 128.0f) * inv;
      } else {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const f32x4 ev = (o[2 * bb] * k24 - wsb[bb] * 8.0f) * inv, od = (o[2 * bb + 1] * k20 - wsb[bb] * 8.0f) * inv;
          *(f32x4*)(orow + 32 * bb + 8 * gq) = f32x4{ev[0], od[0], ev[1], od[1]};
          *(f32x4*)(orow + 32 * bb + 8 * gq + 4) = f32x4{ev[2], od[2], ev[3], od[3]};
        }
      }
      if (gq == 0 && w == 0) lse_out[rowhead] = nonempty ? (m_used + log2f(l_tot)) * kLn2 : -INFINITY;
    }
    __syncthreads();
  }
}

template <int BITS>
hipError_t launch_quant(const DecodeArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.base.B * a.base.T;
  if (rows <= 0 || a.n_spans <= 0) return hipSuccess;
  if (!a.rot_lo || !a.rot_hi || !a.base.rot_f16 || a.chunk <= 0 ||
      (a.base.n_kv > 0 && (!a.k_scales || !a.base.k_raw)))
    return hipErrorInvalidValue;
  dim3 grid((unsigned)a.n_spans, (unsigned)(rows * a.base.Hkv)), block(256);
  if (a.chunk % 64 == 0 && a.base.Hq <= 8 * a.base.Hkv)
    hipLaunchKernelGGL((attn_decode_quant_kernel<BITS, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((attn_decode_quant_kernel<BITS, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_decode_q8(const DecodeArgs& a, hipStream_t stream) { return launch_quant<8>(a, stream); }
hipError_t launch_attn_decode_q4(const DecodeArgs& a, hipStream_t stream) { return launch_quant<4>(a, stream); }

}  // namespace dca
