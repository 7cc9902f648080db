// Shared device helpers and launcher declarations of the DCA library (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dca {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }     // RNE

__device__ __forceinline__ int64_t floordiv64(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) q -= 1;
  return q;
}

typedef __attribute__((address_space(3))) char lds_char;

// 16-byte global->LDS load: lane l's bytes land at LDS address lds_row_addr + 16 l (the address
// must be wave-uniform).  Issued as inline asm on purpose: the compiler's wait-count model charges
// these loads to the LDS counter as well, so every LDS-read wait inside a tile loop would also
// wait for the next tile's loads to arrive from memory.  A kernel using it orders the loads
// itself (wait_vm0 + barrier before a stage is read), and no other instruction of the attention
// kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// NT = true marks the load nontemporal (data read once, such as a decode pass's key cache, which
// then does not displace reused lines from the caches).
template <bool NT = false>
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_row_addr) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_row_addr);
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
                 : "memory", "m0");
}
// The same load from a wave-uniform base (scalar registers) plus a 32-bit per-lane byte offset,
// so that no 64-bit address arithmetic is done per lane.
template <bool NT = false>
__device__ __forceinline__ void dma16_off(const void* base, uint32_t off, uint32_t lds_row_addr) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_row_addr);
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// a wave-uniform pointer, placed in scalar registers
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left open) through the builtin, so that the compiler's
// own wait placement knows that every earlier global load has completed
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wave-wide reductions over 64 lanes (fixed butterfly order, so results are deterministic).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ------------------------------------------------------------------------------------------
// Launchers (all asynchronous on `stream`).  Element strides are in elements of the tensor.
// ------------------------------------------------------------------------------------------

// Positions and regime intervals.  pos_q [3][rows], bounds [3][rows][2]; pos_k [n_kv].
hipError_t launch_remap(const int32_t* q_pos, int64_t rows, int32_t chunk, int32_t mode,
                        int32_t n_kv, int32_t* pos_q, int32_t* pos_k, int32_t* bounds,
                        hipStream_t stream);

struct RopeArgs {
  const void* x;
  int64_t x_row_stride, x_head_stride;
  void* y;
  int64_t y_row_stride, y_head_stride;
  int64_t y_plane_stride;   // between planes (grid.z); planes read pos + z*pos_plane_stride
  const int32_t* pos;       // NULL: position of row r is (r % pos_mod_rows) mod chunk
  int64_t pos_plane_stride;
  int64_t pos_mod_rows;
  int32_t chunk;
  int64_t rows;
  int32_t n_heads, n_rot, head_dim;
  int32_t copy_tail;        // copy dims [n_rot, head_dim) as well (same in/out type only)
  int32_t out_f16;          // bf16 input written as fp16 (the rotated operands of the bf16 path)
  int32_t planes;
  double theta;
  const float* freq_factors;  // [n_rot/2] or NULL
  double mag;                 // magnitude factor of the rotated dims (1 = none)
};
hipError_t launch_rope(const RopeArgs& a, bool bf16_data, hipStream_t stream);

// cos/sin tables for in-kernel key rotation: lo[64][half] of mag * (cos, sin)(l * w_f) and
// hi[n_hi][half] of (cos, sin)(64 * h * w_f), both formed from fp64 angles (their composition
// carries the magnitude factor once).
hipError_t launch_rope_tables(float2* lo, float2* hi, int32_t n_hi, int32_t n_rot, double theta,
                              const float* freq_factors, double mag, hipStream_t stream);

// N-way LSE merge.  Part p of row x: o = o_ptr[p] + x*D (pointer mode) or o_base + p*part_stride
// + x*D (strided mode); lse likewise.
struct MergeArgs {
  const float* o_ptr[8];
  const float* lse_ptr[8];
  const float* o_base;
  const float* lse_base;
  int64_t o_part_stride, lse_part_stride;
  int32_t n_parts;
  int32_t strided;
  int64_t rows;
  int32_t D;
  void* o_out;
  float* lse_out;
};
hipError_t launch_merge(const MergeArgs& a, bool out_bf16, hipStream_t stream);
// Same merge for many parts per row (up to merge_many_max_parts()), one workgroup per row.
hipError_t launch_merge_many(const MergeArgs& a, bool out_bf16, hipStream_t stream);
int merge_many_max_parts();

// One or more regime passes, fp32 data, any head_dim <= 1024: one wave per (row, head, regime).
struct AttnArgs {
  const void* q_rot[3];      // per regime: rotary dims of (b,t,h) at q_rot[r] + row_head*q_rot_hs
  int64_t q_rot_hs;
  const void* q_tail;        // dims [n_rot, D) of (b,t,h) at q_tail + row_head*q_tail_hs
  int64_t q_tail_hs;
  const void* k_rot;         // rotary dims of (b,j,g) at k_rot + ((b*N+j)*Hkv+g)*k_rot_hs
  int64_t k_rot_hs;
  const void* k_raw;         // [B,N,Hkv,D]
  const int32_t* bounds;     // [3][B*T][2]
  float* o[3];               // [B*T*Hq][D] per regime, NULL = regime skipped
  float* lse[3];
  int32_t B, T, Hq, Hkv, n_kv, D, n_rot;
  float scale;
  int32_t rot_f16;           // bf16 path: q_rot / k_rot rotary dims are fp16 (else bf16)
  // single pass over the three regimes under one online softmax (bf16 prefill): the final O and
  // lse go to o_final / lse_final; o[], lse[] are unused
  int32_t fused;
  void* o_final;             // [B*T*Hq][D], bf16 if o_final_bf16 else fp32
  int32_t o_final_bf16;
  float* lse_final;          // [B*T*Hq]
};
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream);

// bf16 prefill regime passes with MFMA; D = 512, n_rot = 128, Hq/Hkv in {1,2,4,8,16,32}.
hipError_t launch_attn_prefill_bf16(const AttnArgs& a, hipStream_t stream);
// bf16 prefill, the three regimes in one pass (a.fused set, fp16 rotary operands); D = 512,
// n_rot = 128, Hq/Hkv in {1,2,4,8,16}.
hipError_t launch_attn_fused_bf16(const AttnArgs& a, hipStream_t stream);

// bf16 split-KV decode passes.  Each (b,t,g, span of `span` keys, regime r) emits one partial
// into part slot slot0[r] + span: o_part [slot][B*T*Hq][D], lse_part [slot][B*T*Hq].
// rot_tables != NULL: keys are rotated in-kernel (k_rot unused); otherwise k_rot is read.
struct DecodeArgs {
  AttnArgs base;
  float* o_part;
  float* lse_part;
  int32_t span, n_spans;
  int32_t regime_mask;
  int32_t slot0[3];         // partial slot of (regime r, span s) is slot0[r] + s
  const float2* rot_lo;
  const float2* rot_hi;
  int32_t chunk;
  double theta;
  // quantized key cache: base.k_raw holds the codes (q8_0: int8 [B,N,Hkv,D]; q4_0: uint8
  // [B,N,Hkv,D/2], two 4-bit codes per byte) and k_scales the fp16 block scales [B,N,Hkv,D/32]
  const uint16_t* k_scales;
  // region of the cache this launch reads: k_raw (k_rot, k_scales) hold cells
  // [key0, key0 + n_rows) of every sequence (N = n_rows above); spans start at key0.  A whole
  // cache is key0 = 0, n_rows = base.n_kv.
  int32_t key0, n_rows;
};
hipError_t launch_attn_decode_bf16(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_attn_decode_q8(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_attn_decode_q4(const DecodeArgs& a, hipStream_t stream);

// reference-rate probes (calibrate.hip)
hipError_t launch_probe_mfma(int32_t n_workgroups, int32_t iters, float* sink, hipStream_t stream);
hipError_t launch_probe_read(const void* src, int64_t bytes, int32_t n_workgroups, float* sink,
                             hipStream_t stream);

}  // namespace dca
