// C ABI of the DCA library: argument validation, workspace layout and kernel dispatch.
// The operations and their sources are documented in include/dca.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <mutex>
#include <string>

#include "../../include/dca.h"
#include "../../include/dca_calibrate.h"
#include "common.h"

namespace {

thread_local std::string g_err;
thread_local hipEvent_t* g_stage_events = nullptr;

// Records stage event i on `stream` when the caller installed stage events.
hipError_t mark(int i, hipStream_t stream) {
  if (!g_stage_events) return hipSuccess;
  return hipEventRecord(g_stage_events[i], stream);
}

dca_status fail(dca_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

dca_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DCA_OK;
  return fail(DCA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kDecodeMaxT = 8;     // query tokens per sequence served by the split-KV path
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
size_t elem_size(dca_dtype t) { return t == DCA_BF16 ? 2 : 4; }

bool valid_dtype(int t) { return t == DCA_F32 || t == DCA_BF16; }

// The kernels move rows with 16-byte loads and stores (direct global->LDS loads included), so the
// tensors they stream and the workspace start at 16-byte boundaries.  NULL passes (the callers
// have already rejected a NULL that would be read).
bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }
dca_status check_aligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!al16(p)) return fail(DCA_ERR_INVALID_ARGUMENT, "pointer %p is not 16-byte aligned", p);
  return DCA_OK;
}

dca_status check_config(const dca_config* cfg, int dtype) {
  if (!cfg) return fail(DCA_ERR_INVALID_ARGUMENT, "config is NULL");
  if (!valid_dtype(dtype)) return fail(DCA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (cfg->head_dim <= 0 || cfg->head_dim > 1024)
    return fail(DCA_ERR_INVALID_ARGUMENT, "head_dim %d outside [1, 1024]", cfg->head_dim);
  if (cfg->n_rot < 2 || (cfg->n_rot & 1) || cfg->n_rot > cfg->head_dim)
    return fail(DCA_ERR_INVALID_ARGUMENT, "n_rot %d must be even and in [2, head_dim]", cfg->n_rot);
  if (cfg->n_head_q <= 0 || cfg->n_head_kv <= 0 || cfg->n_head_q % cfg->n_head_kv)
    return fail(DCA_ERR_INVALID_ARGUMENT, "n_head_q %d must be a positive multiple of n_head_kv %d",
                cfg->n_head_q, cfg->n_head_kv);
  if (cfg->chunk < 1) return fail(DCA_ERR_INVALID_ARGUMENT, "chunk %d < 1", cfg->chunk);
  if (cfg->remap_mode < DCA_REMAP_BASELINE || cfg->remap_mode > DCA_REMAP_PAGE_2C)
    return fail(DCA_ERR_INVALID_ARGUMENT, "remap_mode %d is not a dca_remap_mode", cfg->remap_mode);
  if (!(cfg->rope_theta > 0.0f) || !isfinite(cfg->rope_theta))
    return fail(DCA_ERR_INVALID_ARGUMENT, "rope_theta must be finite and > 0");
  if (!isfinite(cfg->scale)) return fail(DCA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (!(cfg->rope_attn_factor > 0.0f) || !isfinite(cfg->rope_attn_factor))
    return fail(DCA_ERR_INVALID_ARGUMENT, "rope_attn_factor must be finite and > 0");
  if (dtype == DCA_BF16) {
    const int G = cfg->n_head_q / cfg->n_head_kv;
    if (cfg->head_dim != 512 || cfg->n_rot != 128)
      return fail(DCA_ERR_UNSUPPORTED, "bf16 path needs head_dim 512 and n_rot 128 (got %d, %d)",
                  cfg->head_dim, cfg->n_rot);
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
      return fail(DCA_ERR_UNSUPPORTED, "bf16 path needs n_head_q/n_head_kv in {1,2,4,8,16} (got %d)", G);
  }
  return DCA_OK;
}

dca_status check_sizes(int32_t B, int32_t T, int32_t n_kv) {
  if (B < 0 || T < 0 || n_kv < 0)
    return fail(DCA_ERR_INVALID_ARGUMENT, "negative size (B %d, T %d, n_kv %d)", B, T, n_kv);
  return DCA_OK;
}

// Split-KV geometry: spans of >= 4096 keys, at most 512 spans per row.
void decode_split(int32_t n_kv, int32_t* span, int32_t* n_spans) {
  int64_t s = 4096;
  while ((n_kv + s - 1) / s > 512) s *= 2;
  *span = (int32_t)s;
  *n_spans = n_kv > 0 ? (int32_t)((n_kv + s - 1) / s) : 1;
}

bool use_decode(dca_dtype dtype, int32_t T) { return dtype == DCA_BF16 && T <= kDecodeMaxT; }

// Workspace of dca_attention, in order.
struct AttnWorkspace {
  size_t pos_q, bounds, qrot, krot, o_parts, lse_parts, dec_o, dec_lse, tab_lo, tab_hi, total;
  int32_t span, n_spans, n_hi;
};

AttnWorkspace attention_layout(const dca_config* cfg, dca_dtype dtype, int32_t B, int32_t T,
                               int32_t n_kv, bool split_kv = false, int32_t n_spans_override = 0) {
  AttnWorkspace w{};
  const size_t rows = (size_t)B * T;
  const size_t es = elem_size(dtype);
  const size_t D = cfg->head_dim, R = cfg->n_rot, Hq = cfg->n_head_q, Hkv = cfg->n_head_kv;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  w.pos_q = take(3 * rows * 4);
  w.bounds = take(3 * rows * 2 * 4);
  w.qrot = take(3 * rows * Hq * R * es);   // bf16 path: fp16, same size
  const bool dec = split_kv || use_decode(dtype, T);
  w.krot = take(dec ? 0 : (size_t)B * n_kv * Hkv * R * es);
  if (dec) {
    decode_split(n_kv, &w.span, &w.n_spans);
    if (n_spans_override > 0) w.n_spans = n_spans_override;
    w.n_hi = (cfg->chunk + 63) / 64;
    w.o_parts = take(0);
    w.lse_parts = take(0);
    w.dec_o = take((size_t)3 * w.n_spans * rows * Hq * D * 4);
    w.dec_lse = take((size_t)3 * w.n_spans * rows * Hq * 4);
    w.tab_lo = take((size_t)64 * (R / 2) * 8);
    w.tab_hi = take((size_t)w.n_hi * (R / 2) * 8);
  } else if (dtype == DCA_BF16) {
    // single fused pass: O stays in registers, the final O and lse go straight to the caller's
    // outputs; no scratch beyond the positions and rotated operands
    w.o_parts = take(0);
    w.lse_parts = take(0);
    w.dec_o = w.dec_lse = w.tab_lo = w.tab_hi = off;
  } else {
    w.o_parts = take(3 * rows * Hq * D * 4);
    w.lse_parts = take(3 * rows * Hq * 4);
    w.dec_o = w.dec_lse = w.tab_lo = w.tab_hi = off;
  }
  w.total = off;
  return w;
}

size_t regime_workspace(const dca_config* cfg, dca_dtype dtype, int32_t B, int32_t T, int32_t n_kv) {
  if (!use_decode(dtype, T)) return 0;
  int32_t span, n_spans;
  decode_split(n_kv, &span, &n_spans);
  const size_t rows = (size_t)B * T * cfg->n_head_q;
  return align_up((size_t)n_spans * rows * cfg->head_dim * 4) + align_up((size_t)n_spans * rows * 4);
}

dca::RopeArgs rope_args_for_q(const dca_config* cfg, const void* q, int64_t rows, void* qrot,
                              const int32_t* pos_q) {
  dca::RopeArgs ra{};
  ra.x = q;
  ra.x_row_stride = (int64_t)cfg->n_head_q * cfg->head_dim;
  ra.x_head_stride = cfg->head_dim;
  ra.y = qrot;
  ra.y_row_stride = (int64_t)cfg->n_head_q * cfg->n_rot;
  ra.y_head_stride = cfg->n_rot;
  ra.y_plane_stride = rows * cfg->n_head_q * cfg->n_rot;
  ra.pos = pos_q;
  ra.pos_plane_stride = rows;
  ra.pos_mod_rows = 1;
  ra.chunk = cfg->chunk;
  ra.rows = rows;
  ra.n_heads = cfg->n_head_q;
  ra.n_rot = cfg->n_rot;
  ra.head_dim = cfg->head_dim;
  ra.copy_tail = 0;
  ra.out_f16 = 1;   // rotated operands of the bf16 path are fp16 (ignored for fp32 data)
  ra.planes = 3;
  ra.theta = (double)cfg->rope_theta;
  ra.freq_factors = cfg->freq_factors;
  ra.mag = (double)cfg->rope_attn_factor;
  return ra;
}

// Spans of the window / tail decode: each region is cut into spans of the whole cache's span size.
void window_spans(int32_t n_win, int32_t n_tail, int32_t* span, int32_t* s_win, int32_t* s_tail) {
  int32_t n_spans;
  decode_split(n_win + n_tail, span, &n_spans);
  *s_win = (int32_t)(((int64_t)n_win + *span - 1) / *span);
  *s_tail = (int32_t)(((int64_t)n_tail + *span - 1) / *span);
}

// Address at which the kernels read caller memory: device memory as it is, pinned host memory
// (hipHostMalloc) at the device address the runtime maps it to.  Pageable host memory or an
// unknown pointer is rejected before any launch.
dca_status device_view(const void* p, const void** out, const char* what) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(DCA_ERR_INVALID_ARGUMENT, "%s: not device or pinned host memory", what);
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) {
    *out = p;
    return DCA_OK;
  }
  if (at.type == hipMemoryTypeHost) {
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess || !d) {
      (void)hipGetLastError();
      return fail(DCA_ERR_INVALID_ARGUMENT, "%s: host memory not mapped for the device", what);
    }
    *out = d;
    return DCA_OK;
  }
  return fail(DCA_ERR_INVALID_ARGUMENT, "%s: unsupported memory type %d", what, (int)at.type);
}

// ---- scratch of dca_attention_noalloc ------------------------------------------------------
// A file-scope device array serves as the workspace of the entry point that allocates nothing.
// Each GPU holds its own copy for the life of the process.  In host code `scratch` is only a
// stand-in for the symbol: its device address comes from hipGetSymbolAddress, once per device with
// that device current, and only that address is handed to kernels.
__device__ __align__(256) char scratch[DCA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

// Device address of the current device's scratch (looked up on the first call on that device).
dca_status scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DCA_ERR_UNSUPPORTED, "device %d beyond the %d devices the static scratch serves", dev, kMaxDevices);
  if (stream) {
    int sdev = -1;
    if ((e = hipStreamGetDevice(stream, &sdev)) != hipSuccess) return hip_status(e, "hipStreamGetDevice");
    if (sdev != dev)
      return fail(DCA_ERR_INVALID_ARGUMENT, "stream belongs to device %d but device %d is current", sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return hip_status(e, "hipGetSymbolAddress");
    if (!p) return fail(DCA_ERR_HIP, "hipGetSymbolAddress returned no address for the scratch");
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return DCA_OK;
}

}  // namespace

extern "C" {

const char* dca_last_error(void) { return g_err.c_str(); }

dca_status dca_set_stage_events(hipEvent_t* events, int32_t n) {
  if (events && n > 0 && n < DCA_N_STAGE_EVENTS)
    return fail(DCA_ERR_INVALID_ARGUMENT, "need %d stage events, got %d", DCA_N_STAGE_EVENTS, n);
  g_stage_events = (events && n > 0) ? events : nullptr;
  return DCA_OK;
}

dca_status dca_remap_positions(const dca_config* cfg, int32_t B, int32_t T, const int32_t* q_pos,
                               int32_t n_kv, int32_t* pos_q, int32_t* pos_k, int32_t* bounds,
                               hipStream_t stream) {
  if (!cfg) return fail(DCA_ERR_INVALID_ARGUMENT, "config is NULL");
  if (cfg->chunk < 1) return fail(DCA_ERR_INVALID_ARGUMENT, "chunk %d < 1", cfg->chunk);
  if (cfg->remap_mode < DCA_REMAP_BASELINE || cfg->remap_mode > DCA_REMAP_PAGE_2C)
    return fail(DCA_ERR_INVALID_ARGUMENT, "remap_mode %d is not a dca_remap_mode", cfg->remap_mode);
  dca_status st = check_sizes(B, T, n_kv);
  if (st) return st;
  const int64_t rows = (int64_t)B * T;
  if (rows > 0 && !q_pos && (pos_q || bounds)) return fail(DCA_ERR_INVALID_ARGUMENT, "q_pos is NULL");
  return hip_status(dca::launch_remap(q_pos, rows, cfg->chunk, cfg->remap_mode, n_kv, pos_q, pos_k, bounds, stream),
                    "remap launch");
}

dca_status dca_rope_partial(const dca_config* cfg, dca_dtype dtype, const void* x, int64_t rows,
                            int32_t n_heads, const int32_t* pos, void* y, hipStream_t stream) {
  dca_status st = check_config(cfg, DCA_F32);  // rope itself accepts any head_dim for both types
  if (st) return st;
  if (!valid_dtype(dtype)) return fail(DCA_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dtype);
  if (rows < 0 || n_heads <= 0) return fail(DCA_ERR_INVALID_ARGUMENT, "bad rows %lld / n_heads %d", (long long)rows, n_heads);
  if (rows > 0 && (!x || !y || !pos)) return fail(DCA_ERR_INVALID_ARGUMENT, "NULL pointer");
  dca::RopeArgs ra{};
  ra.x = x;
  ra.x_row_stride = (int64_t)n_heads * cfg->head_dim;
  ra.x_head_stride = cfg->head_dim;
  ra.y = y;
  ra.y_row_stride = ra.x_row_stride;
  ra.y_head_stride = cfg->head_dim;
  ra.pos = pos;
  ra.pos_mod_rows = 1;
  ra.chunk = cfg->chunk;
  ra.rows = rows;
  ra.n_heads = n_heads;
  ra.n_rot = cfg->n_rot;
  ra.head_dim = cfg->head_dim;
  ra.copy_tail = x != y;
  ra.planes = 1;
  ra.theta = (double)cfg->rope_theta;
  ra.freq_factors = cfg->freq_factors;
  ra.mag = (double)cfg->rope_attn_factor;
  return hip_status(dca::launch_rope(ra, dtype == DCA_BF16, stream), "rope launch");
}

size_t dca_attn_regime_workspace_size(const dca_config* cfg, dca_dtype dtype, int32_t B, int32_t T,
                                      int32_t n_kv) {
  if (check_config(cfg, dtype) || check_sizes(B, T, n_kv)) return 0;
  return regime_workspace(cfg, dtype, B, T, n_kv);
}

dca_status dca_attn_regime(const dca_config* cfg, dca_dtype dtype, int32_t regime, int32_t B,
                           int32_t T, const void* q_r, const int32_t* bounds, const void* k_rot,
                           const void* k_raw, int32_t n_kv, float* o_r, float* lse_r,
                           void* workspace, size_t ws_bytes, hipStream_t stream) {
  dca_status st = check_config(cfg, dtype);
  if (st) return st;
  if ((st = check_sizes(B, T, n_kv))) return st;
  if (regime < 0 || regime > 2) return fail(DCA_ERR_INVALID_ARGUMENT, "regime %d not in {0,1,2}", regime);
  const int64_t rows = (int64_t)B * T;
  if (rows == 0) return DCA_OK;
  if (!q_r || !bounds || !o_r || !lse_r || (n_kv > 0 && (!k_rot || !k_raw)))
    return fail(DCA_ERR_INVALID_ARGUMENT, "NULL pointer");
  const size_t need = regime_workspace(cfg, dtype, B, T, n_kv);
  if (ws_bytes < need || (need && !workspace))
    return fail(DCA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", ws_bytes, need);
  if (dtype == DCA_BF16 && (st = check_aligned({q_r, k_rot, k_raw, o_r, workspace}))) return st;
  const size_t es = elem_size(dtype);
  dca::AttnArgs a{};
  for (int r = 0; r < 3; ++r) a.q_rot[r] = q_r;
  a.q_rot_hs = cfg->head_dim;
  a.q_tail = (const char*)q_r + cfg->n_rot * es;
  a.q_tail_hs = cfg->head_dim;
  a.k_rot = k_rot;   // [B,n_kv,Hkv,n_rot]: the rotary dims only
  a.k_rot_hs = cfg->n_rot;
  a.k_raw = k_raw;
  a.bounds = bounds;
  a.B = B; a.T = T; a.Hq = cfg->n_head_q; a.Hkv = cfg->n_head_kv; a.n_kv = n_kv;
  a.D = cfg->head_dim; a.n_rot = cfg->n_rot; a.scale = cfg->scale;
  if (dtype == DCA_F32) {
    a.o[regime] = o_r;
    a.lse[regime] = lse_r;
    return hip_status(dca::launch_attn_f32(a, stream), "attention launch");
  }
  if (!use_decode(dtype, T)) {
    a.o[regime] = o_r;
    a.lse[regime] = lse_r;
    return hip_status(dca::launch_attn_prefill_bf16(a, stream), "prefill attention launch");
  }
  if ((int64_t)B * T * cfg->n_head_kv > 65535)
    return fail(DCA_ERR_UNSUPPORTED, "decode batch too large");
  dca::DecodeArgs da{};
  da.base = a;
  decode_split(n_kv, &da.span, &da.n_spans);
  const size_t prow = (size_t)rows * cfg->n_head_q;
  da.o_part = (float*)workspace;
  da.lse_part = (float*)((char*)workspace + align_up((size_t)da.n_spans * prow * cfg->head_dim * 4));
  da.regime_mask = 1 << regime;  // its partials fill slots [0, n_spans)
  da.chunk = cfg->chunk;
  da.key0 = 0;
  da.n_rows = n_kv;
  st = hip_status(dca::launch_attn_decode_bf16(da, stream), "decode attention launch");
  if (st) return st;
  dca::MergeArgs m{};
  m.o_base = (const float*)workspace;
  m.lse_base = da.lse_part;
  m.o_part_stride = (int64_t)prow * cfg->head_dim;
  m.lse_part_stride = (int64_t)prow;
  m.n_parts = da.n_spans;
  m.strided = 1;
  m.rows = (int64_t)prow;
  m.D = cfg->head_dim;
  m.o_out = o_r;
  m.lse_out = lse_r;
  return hip_status(dca::launch_merge_many(m, false, stream), "split merge launch");
}

dca_status dca_lse_merge(int32_t n_parts, const float* const* o_parts, const float* const* lse_parts,
                         int64_t rows, int32_t D, dca_dtype out_dtype, void* o_out, float* lse_out,
                         hipStream_t stream) {
  if (n_parts < 1 || n_parts > DCA_MAX_MERGE_PARTS)
    return fail(DCA_ERR_INVALID_ARGUMENT, "n_parts %d outside [1, %d]", n_parts, DCA_MAX_MERGE_PARTS);
  if (rows < 0 || D <= 0 || D > 1024) return fail(DCA_ERR_INVALID_ARGUMENT, "bad rows/D");
  if (!valid_dtype(out_dtype)) return fail(DCA_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)out_dtype);
  if (rows == 0) return DCA_OK;
  if (!o_parts || !lse_parts || !o_out) return fail(DCA_ERR_INVALID_ARGUMENT, "NULL pointer");
  dca::MergeArgs m{};
  for (int p = 0; p < n_parts; ++p) {
    if (!o_parts[p] || !lse_parts[p]) return fail(DCA_ERR_INVALID_ARGUMENT, "NULL part %d", p);
    m.o_ptr[p] = o_parts[p];
    m.lse_ptr[p] = lse_parts[p];
  }
  m.n_parts = n_parts;
  m.rows = rows;
  m.D = D;
  m.o_out = o_out;
  m.lse_out = lse_out;
  return hip_status(dca::launch_merge(m, out_dtype == DCA_BF16, stream), "merge launch");
}

size_t dca_attention_workspace_size(const dca_config* cfg, dca_dtype dtype, int32_t B, int32_t T,
                                    int32_t n_kv) {
  if (check_config(cfg, dtype) || check_sizes(B, T, n_kv)) return 0;
  return attention_layout(cfg, dtype, B, T, n_kv).total;
}

dca_status dca_attention(const dca_config* cfg, dca_dtype dtype, int32_t B, int32_t T,
                         const void* q, const int32_t* q_pos, const void* k, int32_t n_kv,
                         dca_dtype o_dtype, void* o, float* lse, void* workspace, size_t ws_bytes,
                         hipStream_t stream) {
  dca_status st = check_config(cfg, dtype);
  if (st) return st;
  if ((st = check_sizes(B, T, n_kv))) return st;
  if (!valid_dtype(o_dtype)) return fail(DCA_ERR_INVALID_ARGUMENT, "unknown o_dtype %d", (int)o_dtype);
  const int64_t rows = (int64_t)B * T;
  if (rows == 0) return DCA_OK;
  if (!q || !q_pos || !o || (n_kv > 0 && !k)) return fail(DCA_ERR_INVALID_ARGUMENT, "NULL pointer");
  const AttnWorkspace L = attention_layout(cfg, dtype, B, T, n_kv);
  if (ws_bytes < L.total || !workspace)
    return fail(DCA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", ws_bytes, L.total);
  const bool dec = use_decode(dtype, T);
  if (dec && rows * cfg->n_head_kv > 65535) return fail(DCA_ERR_UNSUPPORTED, "decode batch too large");
  if (dtype == DCA_BF16 && (st = check_aligned({q, k, o, workspace}))) return st;
  char* ws = (char*)workspace;
  int32_t* pos_q = (int32_t*)(ws + L.pos_q);
  int32_t* bounds = (int32_t*)(ws + L.bounds);
  void* qrot = ws + L.qrot;
  const size_t es = elem_size(dtype);
  const int64_t Hq = cfg->n_head_q, R = cfg->n_rot, D = cfg->head_dim;

  if ((st = hip_status(mark(0, stream), "stage event"))) return st;
  if ((st = hip_status(dca::launch_remap(q_pos, rows, cfg->chunk, cfg->remap_mode, n_kv, pos_q, nullptr, bounds, stream),
                       "remap launch")))
    return st;
  if ((st = hip_status(mark(1, stream), "stage event"))) return st;
  dca::RopeArgs rq = rope_args_for_q(cfg, q, rows, qrot, pos_q);
  if ((st = hip_status(dca::launch_rope(rq, dtype == DCA_BF16, stream), "rope(q) launch"))) return st;
  if ((st = hip_status(mark(2, stream), "stage event"))) return st;

  dca::AttnArgs a{};
  for (int r = 0; r < 3; ++r) a.q_rot[r] = (const char*)qrot + (size_t)r * rows * Hq * R * es;
  a.q_rot_hs = R;
  a.q_tail = (const char*)q + R * es;
  a.q_tail_hs = D;
  a.k_raw = k;
  a.bounds = bounds;
  a.B = B; a.T = T; a.Hq = cfg->n_head_q; a.Hkv = cfg->n_head_kv; a.n_kv = n_kv;
  a.D = cfg->head_dim; a.n_rot = cfg->n_rot; a.scale = cfg->scale;
  a.rot_f16 = dtype == DCA_BF16;

  if (dec) {
    float2* lo = (float2*)(ws + L.tab_lo);
    float2* hi = (float2*)(ws + L.tab_hi);
    if ((st = hip_status(dca::launch_rope_tables(lo, hi, L.n_hi, cfg->n_rot, (double)cfg->rope_theta,
                                                 cfg->freq_factors, (double)cfg->rope_attn_factor, stream),
                       "rope tables launch")))
      return st;
    if ((st = hip_status(mark(3, stream), "stage event"))) return st;
    dca::DecodeArgs da{};
    da.base = a;
    da.o_part = (float*)(ws + L.dec_o);
    da.lse_part = (float*)(ws + L.dec_lse);
    da.span = L.span;
    da.n_spans = L.n_spans;
    da.regime_mask = 7;
    for (int r = 0; r < 3; ++r) da.slot0[r] = r * L.n_spans;
    da.rot_lo = lo;
    da.rot_hi = hi;
    da.chunk = cfg->chunk;
    da.key0 = 0;
    da.n_rows = n_kv;
    if ((st = hip_status(dca::launch_attn_decode_bf16(da, stream), "decode attention launch")))
      return st;
    if ((st = hip_status(mark(4, stream), "stage event"))) return st;
    dca::MergeArgs m{};
    m.o_base = da.o_part;
    m.lse_base = da.lse_part;
    m.o_part_stride = rows * Hq * D;
    m.lse_part_stride = rows * Hq;
    m.n_parts = 3 * L.n_spans;
    m.strided = 1;
    m.rows = rows * Hq;
    m.D = cfg->head_dim;
    m.o_out = o;
    m.lse_out = lse;
    if ((st = hip_status(dca::launch_merge_many(m, o_dtype == DCA_BF16, stream), "split merge launch")))
      return st;
    return hip_status(mark(5, stream), "stage event");
  }

  // keys rotated once at j mod c (rotary dims only)
  void* krot = ws + L.krot;
  if (n_kv > 0) {
    dca::RopeArgs rk{};
    rk.x = k;
    rk.x_row_stride = (int64_t)cfg->n_head_kv * D;
    rk.x_head_stride = D;
    rk.y = krot;
    rk.y_row_stride = (int64_t)cfg->n_head_kv * R;
    rk.y_head_stride = R;
    rk.pos = nullptr;
    rk.pos_mod_rows = n_kv;
    rk.chunk = cfg->chunk;
    rk.rows = (int64_t)B * n_kv;
    rk.n_heads = cfg->n_head_kv;
    rk.n_rot = cfg->n_rot;
    rk.head_dim = cfg->head_dim;
    rk.planes = 1;
    rk.out_f16 = 1;
    rk.theta = (double)cfg->rope_theta;
    rk.freq_factors = cfg->freq_factors;
    rk.mag = (double)cfg->rope_attn_factor;
    if ((st = hip_status(dca::launch_rope(rk, dtype == DCA_BF16, stream), "rope(k) launch"))) return st;
  }
  if ((st = hip_status(mark(3, stream), "stage event"))) return st;
  a.k_rot = krot;
  a.k_rot_hs = R;
  float* op = (float*)(ws + L.o_parts);
  float* lp = (float*)(ws + L.lse_parts);
  if (dtype == DCA_BF16) {
    // one pass over the three regimes under one online softmax: no partials, no merge
    a.fused = 1;
    a.o_final = o;
    a.o_final_bf16 = o_dtype == DCA_BF16;
    a.lse_final = lse;
    if ((st = hip_status(dca::launch_attn_fused_bf16(a, stream), "prefill attention launch")))
      return st;
    if ((st = hip_status(mark(4, stream), "stage event"))) return st;
    return hip_status(mark(5, stream), "stage event");
  }
  for (int r = 0; r < 3; ++r) {
    a.o[r] = op + (size_t)r * rows * Hq * D;
    a.lse[r] = lp + (size_t)r * rows * Hq;
  }
  if (dtype == DCA_F32)
    st = hip_status(dca::launch_attn_f32(a, stream), "attention launch");
  else
    st = hip_status(dca::launch_attn_prefill_bf16(a, stream), "prefill attention launch");
  if (st) return st;
  if ((st = hip_status(mark(4, stream), "stage event"))) return st;
  dca::MergeArgs m{};
  for (int r = 0; r < 3; ++r) {
    m.o_ptr[r] = a.o[r];
    m.lse_ptr[r] = a.lse[r];
  }
  m.n_parts = 3;
  m.rows = rows * Hq;
  m.D = cfg->head_dim;
  m.o_out = o;
  m.lse_out = lse;
  if ((st = hip_status(dca::launch_merge(m, o_dtype == DCA_BF16, stream), "merge launch"))) return st;
  return hip_status(mark(5, stream), "stage event");
}

dca_status dca_attention_noalloc(const dca_config* cfg, dca_dtype dtype, int32_t B, int32_t T,
                                 const void* q, const int32_t* q_pos, const void* k, int32_t n_kv,
                                 dca_dtype o_dtype, void* o, float* lse, hipStream_t stream) {
  dca_status st = check_config(cfg, dtype);
  if (st) return st;
  if ((st = check_sizes(B, T, n_kv))) return st;
  if ((int64_t)B * T == 0) return DCA_OK;
  const size_t need = attention_layout(cfg, dtype, B, T, n_kv).total;
  if (need > (size_t)DCA_NOALLOC_SCRATCH_BYTES)
    return fail(DCA_ERR_UNSUPPORTED, "this call needs %zu bytes of scratch; the static scratch holds %zu",
                need, (size_t)DCA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_address(stream, &ws))) return st;
  return dca_attention(cfg, dtype, B, T, q, q_pos, k, n_kv, o_dtype, o, lse, ws,
                       (size_t)DCA_NOALLOC_SCRATCH_BYTES, stream);
}

// dca_attention_q8 / dca_attention_q4: the split-KV decode path over a block-quantized cache
static dca_status attention_quant(int bits, const dca_config* cfg, int32_t B, int32_t T, const void* q,
                                  const int32_t* q_pos, const void* k_codes, const uint16_t* k_scales,
                                  int32_t n_kv, dca_dtype o_dtype, void* o, float* lse, void* workspace,
                                  size_t ws_bytes, hipStream_t stream) {
  dca_status st = check_config(cfg, DCA_BF16);
  if (st) return st;
  if ((st = check_sizes(B, T, n_kv))) return st;
  if (!valid_dtype(o_dtype)) return fail(DCA_ERR_INVALID_ARGUMENT, "unknown o_dtype %d", (int)o_dtype);
  const int64_t rows = (int64_t)B * T;
  if (rows == 0) return DCA_OK;
  if (!q || !q_pos || !o || (n_kv > 0 && (!k_codes || !k_scales)))
    return fail(DCA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (rows * cfg->n_head_kv > 65535) return fail(DCA_ERR_UNSUPPORTED, "batch too large for the split-KV path");
  const AttnWorkspace L = attention_layout(cfg, DCA_BF16, B, T, n_kv, true);
  if (ws_bytes < L.total || !workspace)
    return fail(DCA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", ws_bytes, L.total);
  if ((st = check_aligned({q, k_codes, k_scales, o, workspace}))) return st;
  char* ws = (char*)workspace;
  int32_t* pos_q = (int32_t*)(ws + L.pos_q);
  int32_t* bounds = (int32_t*)(ws + L.bounds);
  void* qrot = ws + L.qrot;
  const int64_t Hq = cfg->n_head_q, R = cfg->n_rot, D = cfg->head_dim;

  if ((st = hip_status(mark(0, stream), "stage event"))) return st;
  if ((st = hip_status(dca::launch_remap(q_pos, rows, cfg->chunk, cfg->remap_mode, n_kv, pos_q, nullptr, bounds, stream),
                       "remap launch")))
    return st;
  if ((st = hip_status(mark(1, stream), "stage event"))) return st;
  dca::RopeArgs rq = rope_args_for_q(cfg, q, rows, qrot, pos_q);
  if ((st = hip_status(dca::launch_rope(rq, true, stream), "rope(q) launch"))) return st;
  if ((st = hip_status(mark(2, stream), "stage event"))) return st;
  float2* lo = (float2*)(ws + L.tab_lo);
  float2* hi = (float2*)(ws + L.tab_hi);
  if ((st = hip_status(dca::launch_rope_tables(lo, hi, L.n_hi, cfg->n_rot, (double)cfg->rope_theta,
                                               cfg->freq_factors, (double)cfg->rope_attn_factor, stream),
                       "rope tables launch")))
    return st;
  if ((st = hip_status(mark(3, stream), "stage event"))) return st;

  dca::DecodeArgs da{};
  dca::AttnArgs& a = da.base;
  for (int r = 0; r < 3; ++r) a.q_rot[r] = (const char*)qrot + (size_t)r * rows * Hq * R * 2;
  a.q_rot_hs = R;
  a.q_tail = (const char*)q + R * 2;
  a.q_tail_hs = D;
  a.k_raw = k_codes;
  a.bounds = bounds;
  a.B = B; a.T = T; a.Hq = cfg->n_head_q; a.Hkv = cfg->n_head_kv; a.n_kv = n_kv;
  a.D = cfg->head_dim; a.n_rot = cfg->n_rot; a.scale = cfg->scale;
  a.rot_f16 = 1;
  da.k_scales = k_scales;
  da.o_part = (float*)(ws + L.dec_o);
  da.lse_part = (float*)(ws + L.dec_lse);
  da.span = L.span;
  da.n_spans = L.n_spans;
  da.regime_mask = 7;
  for (int r = 0; r < 3; ++r) da.slot0[r] = r * L.n_spans;
  da.rot_lo = lo;
  da.rot_hi = hi;
  da.chunk = cfg->chunk;
  da.key0 = 0;
  da.n_rows = n_kv;
  if ((st = hip_status(bits == 8 ? dca::launch_attn_decode_q8(da, stream) : dca::launch_attn_decode_q4(da, stream),
                       "quantized decode attention launch")))
    return st;
  if ((st = hip_status(mark(4, stream), "stage event"))) return st;
  dca::MergeArgs m{};
  m.o_base = da.o_part;
  m.lse_base = da.lse_part;
  m.o_part_stride = rows * Hq * D;
  m.lse_part_stride = rows * Hq;
  m.n_parts = 3 * L.n_spans;
  m.strided = 1;
  m.rows = rows * Hq;
  m.D = cfg->head_dim;
  m.o_out = o;
  m.lse_out = lse;
  if ((st = hip_status(dca::launch_merge_many(m, o_dtype == DCA_BF16, stream), "split merge launch")))
    return st;
  return hip_status(mark(5, stream), "stage event");
}

size_t dca_attention_q8_workspace_size(const dca_config* cfg, int32_t B, int32_t T, int32_t n_kv) {
  if (check_config(cfg, DCA_BF16) || check_sizes(B, T, n_kv)) return 0;
  return attention_layout(cfg, DCA_BF16, B, T, n_kv, true).total;
}

size_t dca_attention_q4_workspace_size(const dca_config* cfg, int32_t B, int32_t T, int32_t n_kv) {
  return dca_attention_q8_workspace_size(cfg, B, T, n_kv);
}

dca_status dca_attention_q8(const dca_config* cfg, int32_t B, int32_t T, const void* q,
                            const int32_t* q_pos, const int8_t* k_codes, const uint16_t* k_scales,
                            int32_t n_kv, dca_dtype o_dtype, void* o, float* lse, void* workspace,
                            size_t ws_bytes, hipStream_t stream) {
  return attention_quant(8, cfg, B, T, q, q_pos, k_codes, k_scales, n_kv, o_dtype, o, lse, workspace,
                         ws_bytes, stream);
}

dca_status dca_attention_q4(const dca_config* cfg, int32_t B, int32_t T, const void* q,
                            const int32_t* q_pos, const uint8_t* k_codes, const uint16_t* k_scales,
                            int32_t n_kv, dca_dtype o_dtype, void* o, float* lse, void* workspace,
                            size_t ws_bytes, hipStream_t stream) {
  return attention_quant(4, cfg, B, T, q, q_pos, k_codes, k_scales, n_kv, o_dtype, o, lse, workspace,
                         ws_bytes, stream);
}

dca_status dca_probe_mfma_bf16(int32_t n_workgroups, int32_t iters, float* sink, hipStream_t stream) {
  if (!sink) return fail(DCA_ERR_INVALID_ARGUMENT, "sink is NULL");
  if (n_workgroups < 1 || n_workgroups > 65536 || iters < 1 || iters > (1 << 20))
    return fail(DCA_ERR_INVALID_ARGUMENT, "probe size out of range (%d workgroups, %d iters)",
                n_workgroups, iters);
  return hip_status(dca::launch_probe_mfma(n_workgroups, iters, sink, stream), "probe launch");
}

dca_status dca_probe_hbm_read(const void* src, int64_t bytes, int32_t n_workgroups, float* sink,
                              hipStream_t stream) {
  if (!sink || (!src && bytes > 0)) return fail(DCA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (bytes < 0 || bytes % 16 || ((uintptr_t)src & 15))
    return fail(DCA_ERR_INVALID_ARGUMENT, "bytes must be a non-negative multiple of 16, src 16-byte aligned");
  if (n_workgroups < 1 || n_workgroups > 65536)
    return fail(DCA_ERR_INVALID_ARGUMENT, "n_workgroups %d out of range", n_workgroups);
  const void* dsrc = src;
  dca_status st;
  if (bytes > 0 && (st = device_view(src, &dsrc, "probe source"))) return st;
  return hip_status(dca::launch_probe_read(dsrc, bytes, n_workgroups, sink, stream), "probe launch");
}


size_t dca_attention_window_workspace_size(const dca_config* cfg, int32_t B, int32_t T, int32_t n_win,
                                           int32_t n_tail) {
  if (check_config(cfg, DCA_BF16) || check_sizes(B, T, n_win) || check_sizes(B, T, n_tail)) return 0;
  int32_t span, sw, st;
  window_spans(n_win, n_tail, &span, &sw, &st);
  return attention_layout(cfg, DCA_BF16, B, T, n_win + n_tail, true, sw + st).total;
}

dca_status dca_attention_window(const dca_config* cfg, int32_t B, int32_t T, const void* q,
                                const int32_t* q_pos, const dca_kv_region* window,
                                const dca_kv_region* tail, dca_dtype o_dtype, void* o, float* lse,
                                void* workspace, size_t ws_bytes, hipStream_t stream) {
  dca_status st = check_config(cfg, DCA_BF16);
  if (st) return st;
  if (!window || !tail) return fail(DCA_ERR_INVALID_ARGUMENT, "region descriptor is NULL");
  const dca_kv_region* reg[2] = {window, tail};
  for (int i = 0; i < 2; ++i) {
    if (reg[i]->n < 0) return fail(DCA_ERR_INVALID_ARGUMENT, "negative region size %d", reg[i]->n);
    if (reg[i]->format < DCA_KV_BF16 || reg[i]->format > DCA_KV_Q4_0)
      return fail(DCA_ERR_INVALID_ARGUMENT, "unknown key format %d", (int)reg[i]->format);
  }
  if ((int64_t)window->n + tail->n > INT32_MAX) return fail(DCA_ERR_INVALID_ARGUMENT, "cache too long");
  const int32_t n_kv = window->n + tail->n;
  if ((st = check_sizes(B, T, n_kv))) return st;
  if (!valid_dtype(o_dtype)) return fail(DCA_ERR_INVALID_ARGUMENT, "unknown o_dtype %d", (int)o_dtype);
  const int64_t rows = (int64_t)B * T;
  if (rows == 0) return DCA_OK;
  if (!q || !q_pos || !o) return fail(DCA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (rows * cfg->n_head_kv > 65535) return fail(DCA_ERR_UNSUPPORTED, "batch too large for the split-KV path");
  for (int i = 0; i < 2; ++i)
    if (reg[i]->n > 0 && (!reg[i]->keys || (reg[i]->format != DCA_KV_BF16 && !reg[i]->scales)))
      return fail(DCA_ERR_INVALID_ARGUMENT, "NULL pointer in the %s region", i ? "tail" : "window");
  int32_t span, s_win, s_tail;
  window_spans(window->n, tail->n, &span, &s_win, &s_tail);
  const int32_t s_all = s_win + s_tail;
  const AttnWorkspace L = attention_layout(cfg, DCA_BF16, B, T, n_kv, true, s_all);
  if (ws_bytes < L.total || !workspace)
    return fail(DCA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", ws_bytes, L.total);
  if ((st = check_aligned({q, o, workspace, window->keys, window->scales, tail->keys, tail->scales})))
    return st;
  const void* keys[2] = {nullptr, nullptr};
  const void* scales[2] = {nullptr, nullptr};
  for (int i = 0; i < 2; ++i) {
    if (reg[i]->n == 0) continue;
    if ((st = device_view(reg[i]->keys, &keys[i], i ? "tail keys" : "window keys"))) return st;
    if (reg[i]->format != DCA_KV_BF16 &&
        (st = device_view(reg[i]->scales, &scales[i], i ? "tail scales" : "window scales")))
      return st;
  }
  char* ws = (char*)workspace;
  int32_t* pos_q = (int32_t*)(ws + L.pos_q);
  int32_t* bounds = (int32_t*)(ws + L.bounds);
  void* qrot = ws + L.qrot;
  const int64_t Hq = cfg->n_head_q, R = cfg->n_rot, D = cfg->head_dim;

  if ((st = hip_status(mark(0, stream), "stage event"))) return st;
  if ((st = hip_status(dca::launch_remap(q_pos, rows, cfg->chunk, cfg->remap_mode, n_kv, pos_q, nullptr, bounds, stream),
                       "remap launch")))
    return st;
  if ((st = hip_status(mark(1, stream), "stage event"))) return st;
  dca::RopeArgs rq = rope_args_for_q(cfg, q, rows, qrot, pos_q);
  if ((st = hip_status(dca::launch_rope(rq, true, stream), "rope(q) launch"))) return st;
  if ((st = hip_status(mark(2, stream), "stage event"))) return st;
  float2* lo = (float2*)(ws + L.tab_lo);
  float2* hi = (float2*)(ws + L.tab_hi);
  if ((st = hip_status(dca::launch_rope_tables(lo, hi, L.n_hi, cfg->n_rot, (double)cfg->rope_theta,
                                               cfg->freq_factors, (double)cfg->rope_attn_factor, stream),
                       "rope tables launch")))
    return st;
  if ((st = hip_status(mark(3, stream), "stage event"))) return st;

  dca::DecodeArgs da{};
  dca::AttnArgs& a = da.base;
  for (int r = 0; r < 3; ++r) a.q_rot[r] = (const char*)qrot + (size_t)r * rows * Hq * R * 2;
  a.q_rot_hs = R;
  a.q_tail = (const char*)q + R * 2;
  a.q_tail_hs = D;
  a.bounds = bounds;
  a.B = B; a.T = T; a.Hq = cfg->n_head_q; a.Hkv = cfg->n_head_kv; a.n_kv = n_kv;
  a.D = cfg->head_dim; a.n_rot = cfg->n_rot; a.scale = cfg->scale;
  a.rot_f16 = 1;
  da.o_part = (float*)(ws + L.dec_o);
  da.lse_part = (float*)(ws + L.dec_lse);
  da.span = span;
  da.regime_mask = 7;
  da.rot_lo = lo;
  da.rot_hi = hi;
  da.chunk = cfg->chunk;
  // the tail first (read over the host link when it lives in host memory), then the window; the
  // spans of region i take partial slots [r * s_all + first_span, ...) of regime r
  const int order[2] = {1, 0};
  for (int oi = 0; oi < 2; ++oi) {
    const int i = order[oi];
    if (reg[i]->n == 0) continue;
    a.k_raw = keys[i];
    da.k_scales = (const uint16_t*)scales[i];
    da.key0 = i ? window->n : 0;
    da.n_rows = reg[i]->n;
    da.n_spans = i ? s_tail : s_win;
    for (int r = 0; r < 3; ++r) da.slot0[r] = r * s_all + (i ? s_win : 0);
    hipError_t e;
    switch (reg[i]->format) {
      case DCA_KV_BF16: e = dca::launch_attn_decode_bf16(da, stream); break;
      case DCA_KV_Q8_0: e = dca::launch_attn_decode_q8(da, stream); break;
      default: e = dca::launch_attn_decode_q4(da, stream); break;
    }
    if ((st = hip_status(e, "region decode attention launch"))) return st;
  }
  if ((st = hip_status(mark(4, stream), "stage event"))) return st;
  dca::MergeArgs m{};
  m.o_base = da.o_part;
  m.lse_base = da.lse_part;
  m.o_part_stride = rows * Hq * D;
  m.lse_part_stride = rows * Hq;
  m.n_parts = 3 * s_all;
  m.strided = 1;
  m.rows = rows * Hq;
  m.D = cfg->head_dim;
  m.o_out = o;
  m.lse_out = lse;
  if ((st = hip_status(dca::launch_merge_many(m, o_dtype == DCA_BF16, stream), "split merge launch")))
    return st;
  return hip_status(mark(5, stream), "stage event");
}

}  // extern "C"