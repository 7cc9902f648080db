/*
 * dca.h -- C ABI of the Dual Chunk Attention (DCA) hot path for gfx950 (MI355X).
 *
 * Source of the method: the page "Feature -- Gemma-4 A4B Dual Chunk Attention (DCA),
 * training-free 1M context" (called "the DCA feature page" below), sections "DCA algorithm
 * (global layers only)", "Section C design" (the rope-K-once / rope-Q-thrice table),
 * "Implementation progress + Section-D simplification" (LSE-emitting attention and the
 * N-way merge) and "Section C2b" (empty-regime semantics); and the page "Protocol --
 * Upstream Sync", entries "opencoti F5 dca" and "0110 WS2 asym-band NaN guard".
 *
 * What is computed.  Positions are split into chunks of c tokens; chunk(x) = floor(x/c).
 * A query at absolute position i attends every cache cell j with 0 <= j <= i and j < n_kv.
 * Each such key falls in exactly one of three regimes:
 *     intra : chunk(j) == chunk(i)
 *     succ  : chunk(j) == chunk(i) - 1  and  i - j < c
 *     inter : i - j >= c
 * Keys are rotated once at pos_k(j) = j mod c.  The query is rotated three times:
 *     intra at (i mod c), succ at (i mod c) + c, inter at c - 1,
 * so every rotary distance (query position minus key position) lies in [0, c), and intra and
 * succ see the true distance i - j (the succ position continues the intra one across the chunk
 * seam).  The pages give the inter query position as c in one place and 2c in another; this
 * library clamps it to c - 1 so that no distance reaches c, and restricts succ to keys closer
 * than c (previous-chunk keys at distance >= c join inter).  Both are readings of the pages.
 *
 * Each regime is one softmax attention emitting O_r (normalised) and lse_r = m + ln(sum e^(s-m))
 * per row; an empty regime gives O_r = 0, lse_r = -inf.  The N-way merge
 *     M = max_r lse_r,  w_r = exp(lse_r - M),  O = sum_r w_r O_r / sum_r w_r,  lse = M + ln sum_r w_r
 * reproduces one softmax over the union of the regimes, because the regimes partition the
 * causal keys.  Scores are s = scale * <rot(q, P_r), rot(k, j mod c)>; values are the
 * un-rotated keys (K = V, no v_proj).
 *
 * RoPE ("partial", "proportional"): only dims [0, n_rot) rotate, as n_rot/2 pairs
 * (f, f + n_rot/2); dims [n_rot, head_dim) are copied bit-exactly.  For pair f the angle is
 * p * theta^(-2f/n_rot) / freq_factors[f];
 *     y_f = x_f cos a - x_{f+n_rot/2} sin a,   y_{f+n_rot/2} = x_f sin a + x_{f+n_rot/2} cos a.
 * Angles are formed in fp64 so positions up to 2^31 keep full fp32 accuracy.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers unless stated; the caller owns all memory.  The
 *    library never allocates caller-visible memory; scratch comes from a caller workspace whose
 *    size is queried first.
 *  - Layouts are row-major, last index fastest: q [B,T,Hq,D], k [B,N,Hkv,D], o [B,T,Hq,D],
 *    lse [B,T,Hq].  Query head h reads KV head h / (Hq/Hkv).
 *  - The bf16 and quantized paths move rows with 16-byte accesses: their q, k (codes and scales),
 *    o and workspace pointers must be 16-byte aligned (any allocator's base addresses are), or
 *    the call returns DCA_ERR_INVALID_ARGUMENT.  The fp32 path takes any naturally aligned
 *    pointers.
 *  - Work is enqueued on `stream` (NULL = the null stream) with no host synchronisation.
 *  - Arguments are validated on the host before anything is enqueued; a failed check returns a
 *    status, touches nothing, and leaves a message for dca_last_error().  A failing HIP call
 *    returns DCA_ERR_HIP.  Nothing aborts and no exception crosses the ABI.
 *  - Results are bit-reproducible run to run on one device (fixed reduction order, no atomics).
 *  - Calls on distinct streams with distinct workspaces may run concurrently.
 *  - Device data is not inspected on the host: a query position that is negative gives an
 *    all-empty row (O = 0, lse = -inf); keys at or beyond n_kv are never read.
 */
#ifndef DCA_H
#define DCA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dca_status {
  DCA_OK = 0,
  DCA_ERR_INVALID_ARGUMENT = 1,   /* NULL pointer, negative size, inconsistent config */
  DCA_ERR_UNSUPPORTED = 2,        /* valid but not implemented (e.g. head_dim != 512 for bf16) */
  DCA_ERR_WORKSPACE_TOO_SMALL = 3,
  DCA_ERR_HIP = 4                 /* a HIP launch or runtime call failed */
} dca_status;

typedef enum dca_dtype { DCA_F32 = 0, DCA_BF16 = 1 } dca_dtype;

typedef enum dca_regime { DCA_INTRA = 0, DCA_SUCC = 1, DCA_INTER = 2 } dca_regime;

/* Remap rules (dca_config.remap_mode).  Keys always sit at j mod c, the intra regime is the
 * query's own chunk with the query at i mod c, and the succ query sits at (i mod c) + c.
 *  DCA_REMAP_BASELINE: the rule stated at the top of this header: succ = previous-chunk keys
 *      closer than c, inter = every key at distance >= c with the query at c - 1, so every rotary
 *      distance is below c.
 *  DCA_REMAP_PAGE_C: the "Section C design" table of the DCA feature page as printed: succ =
 *      the whole previous chunk (distances up to 2c - 1), inter = every older chunk with the
 *      query at c.
 *  DCA_REMAP_PAGE_2C: as DCA_REMAP_PAGE_C with the inter query at 2c (Upstream Sync page, entry
 *      "opencoti F5 dca": the fused kernel and the dense cache fill). */
typedef enum dca_remap_mode {
  DCA_REMAP_BASELINE = 0,
  DCA_REMAP_PAGE_C = 1,
  DCA_REMAP_PAGE_2C = 2
} dca_remap_mode;

#define DCA_N_REGIMES 3
#define DCA_MAX_MERGE_PARTS 8

typedef struct dca_config {
  int32_t head_dim;     /* D, shared by K and V (K = V).  f32: any 1..1024 with D % 8 == 0 and
                           n_rot <= D; bf16: 512. */
  int32_t n_rot;        /* rotated dims; even, 2 <= n_rot <= head_dim; bf16 path: 128 */
  int32_t n_head_q;     /* Hq */
  int32_t n_head_kv;    /* Hkv; Hq % Hkv == 0 */
  int32_t chunk;        /* c >= 1 */
  int32_t remap_mode;   /* dca_remap_mode; other values: DCA_ERR_INVALID_ARGUMENT */
  float rope_theta;     /* > 0; e.g. 1e6 */
  float scale;          /* score scale, e.g. 1/sqrt(512) */
  const float* freq_factors; /* device fp32 [n_rot/2], each > 0; NULL means all 1.0 */
  float rope_attn_factor; /* YaRN magnitude factor m on the rotated dims of q and k (the pages'
                             DCA yarn factor, fed to the rope as its attention factor: DCA feature
                             page, "Runtime knobs"; measured there as no win, default 1): every
                             rotated dim is multiplied by m, so the rotary part of a score scales
                             by m^2; finite and > 0, 1 = none (DCA_ERR_INVALID_ARGUMENT otherwise) */
} dca_config;

/* Position remap and regime key intervals ("Section C design" table of the DCA feature page;
 * "opencoti F5 dca" entry of the Upstream Sync page: dense position fill, masks left NULL).
 * in : q_pos int32 [B,T] absolute query positions; n_kv cache length (cell j has position j).
 * out: pos_q int32 [3,B,T]  (regime order intra, succ, inter);
 *      pos_k int32 [n_kv]   (= j mod c, shared by the batch);
 *      bounds int32 [3,B,T,2] inclusive key interval [lo,hi] of each regime, clipped to
 *      [0, n_kv-1]; an empty regime is written as (0, -1).
 * Any output pointer may be NULL to skip that output.  Bit-exact integer arithmetic. */
dca_status dca_remap_positions(const dca_config* cfg, int32_t B, int32_t T, const int32_t* q_pos,
                               int32_t n_kv, int32_t* pos_q, int32_t* pos_k, int32_t* bounds,
                               hipStream_t stream);

/* Partial RoPE at given positions ("DCA algorithm" section: only the rotary dims are remapped;
 * "Section C2b": K rotated once, Q three times; proportional rope with freq_factors from the
 * "Why llamafile is sufficient" section).
 * x, y: [rows, n_heads, head_dim] of `dtype`; pos: int32 [rows].  y may alias x.
 * Dims >= n_rot are copied bit-exactly; rotated dims are computed in fp32 from fp64 angles and
 * rounded to nearest-even for bf16. */
dca_status dca_rope_partial(const dca_config* cfg, dca_dtype dtype, const void* x, int64_t rows,
                            int32_t n_heads, const int32_t* pos, void* y, hipStream_t stream);

/* One regime's attention pass emitting normalised O and per-row LSE ("Implementation
 * progress + Section-D simplification": the LSE-emitting attention op; "Section C2b": an
 * empty regime yields O = 0 and lse = -inf; Upstream Sync entry 0110: a zero exp-sum gives 0,
 * never 0/0).
 * q_r   : [B,T,Hq,D] queries already rotated at this regime's position (dca_rope_partial).
 * bounds: int32 [3,B,T,2] from dca_remap_positions; only slice `regime` is read.
 * k_rot : [B,n_kv,Hkv,n_rot] the rotary dims of the keys, rotated at pos_k (e.g. the first
 *         n_rot dims of a dca_rope_partial output, made contiguous).
 * k_raw : [B,n_kv,Hkv,D] un-rotated keys, which are also the values.
 * out   : o_r fp32 [B,T,Hq,D], lse_r fp32 [B,T,Hq] (natural log).
 * workspace: device scratch of at least dca_attn_regime_workspace_size() bytes (may be NULL
 * when that size is 0).  dtype selects q_r/k_rot/k_raw element type. */
dca_status dca_attn_regime(const dca_config* cfg, dca_dtype dtype, int32_t regime, int32_t B,
                           int32_t T, const void* q_r, const int32_t* bounds, const void* k_rot,
                           const void* k_raw, int32_t n_kv, float* o_r, float* lse_r,
                           void* workspace, size_t ws_bytes, hipStream_t stream);
size_t dca_attn_regime_workspace_size(const dca_config* cfg, dca_dtype dtype, int32_t B, int32_t T,
                                      int32_t n_kv);

/* Exact N-way LSE merge ("Implementation progress + Section-D simplification" of the DCA
 * feature page; the zero-weight rule of "Section C2b").
 * o_parts, lse_parts: HOST arrays of n_parts DEVICE pointers; o_parts[p] fp32 [rows, D],
 * lse_parts[p] fp32 [rows].  A part with lse = -inf has weight exactly 0 and its O is not read.
 * Rows whose parts are all -inf give O = 0, lse = -inf (no NaN).  1 <= n_parts <=
 * DCA_MAX_MERGE_PARTS.  out: o_out [rows, D] of out_dtype, lse_out fp32 [rows] (may be NULL). */
dca_status dca_lse_merge(int32_t n_parts, const float* const* o_parts,
                         const float* const* lse_parts, int64_t rows, int32_t D,
                         dca_dtype out_dtype, void* o_out, float* lse_out, hipStream_t stream);

/* The whole DCA attention of one layer: remap, rope Q thrice and K once, the three regime
 * passes, and the merge (the "build_attn_dca" body of "Section C2b", without the output
 * projection).
 * q     : [B,T,Hq,D] pre-RoPE queries of `dtype`;  q_pos: int32 [B,T].
 * k     : [B,n_kv,Hkv,D] pre-RoPE keys of `dtype`; they are the values too (K = V).
 * out   : o [B,T,Hq,D] of o_dtype; lse fp32 [B,T,Hq] (may be NULL).
 * workspace: at least dca_attention_workspace_size() bytes of device memory. */
dca_status dca_attention(const dca_config* cfg, dca_dtype dtype, int32_t B, int32_t T,
                         const void* q, const int32_t* q_pos, const void* k, int32_t n_kv,
                         dca_dtype o_dtype, void* o, float* lse, void* workspace, size_t ws_bytes,
                         hipStream_t stream);
size_t dca_attention_workspace_size(const dca_config* cfg, dca_dtype dtype, int32_t B, int32_t T,
                                    int32_t n_kv);

/* dca_attention for callers that cannot allocate memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same operation, kernels and results as
 * dca_attention, with its workspace taken from a static device array of
 * DCA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs on until the process
 * ends.  The call allocates nothing (no hipMalloc, no allocating library routine); the caller
 * still passes q, q_pos, k, o and lse.
 * A call whose workspace (dca_attention_workspace_size) exceeds DCA_NOALLOC_SCRATCH_BYTES returns
 * DCA_ERR_UNSUPPORTED before anything is enqueued (e.g. decode over 8 sequences of 256k keys fits,
 * a 32k-token prefill does not).  `stream` must belong to the current device.
 * Every call on one GPU shares that GPU's array, which keeps what the last call left there: calls
 * that overlap on one GPU (on different streams or threads) race and give undefined results;
 * calls one after the other on a stream are safe.  Other arguments and errors as dca_attention. */
#define DCA_NOALLOC_SCRATCH_BYTES (64u << 20)
dca_status dca_attention_noalloc(const dca_config* cfg, dca_dtype dtype, int32_t B, int32_t T,
                                 const void* q, const int32_t* q_pos, const void* k, int32_t n_kv,
                                 dca_dtype o_dtype, void* o, float* lse, hipStream_t stream);

/* dca_attention over a key cache stored as q8_0 blocks (the pages run DCA over q8_0 caches and
 * read the codes inside the attention kernel: Upstream Sync entries "DCA all-KV" and
 * "0119-p0-dcaon-scalar-inregister"; they give the size as about 0.53x of f16 but print no
 * layout).  Every 32 consecutive dims of one (key, KV head) row share an fp16 scale d; the key's
 * value in a dim is d * q with q the dim's int8 code; the values are also the values of the
 * attention (K = V).
 * q       : bf16 [B,T,Hq,D] pre-RoPE queries (|q| below 65504: the products run in fp16);
 *           q_pos: int32 [B,T].
 * k_codes : int8 [B,n_kv,Hkv,D], the codes in the key layout.
 * k_scales: fp16 bit patterns [B,n_kv,Hkv,D/32], the scale of each block in the same order.
 * out     : o [B,T,Hq,D] of o_dtype; lse fp32 [B,T,Hq] (may be NULL).
 * The split-KV kernel serves every T (it is meant for decode: a few query tokens per sequence);
 * B*T*n_head_kv must not exceed 65535.  head_dim 512, n_rot 128, n_head_q/n_head_kv in
 * {1,2,4,8,16}, as for bf16.  The dtype of q is bf16; the stage-event hook records as for a
 * bf16 decode.  Errors as dca_attention.
 * workspace: at least dca_attention_q8_workspace_size() bytes of device memory. */
dca_status dca_attention_q8(const dca_config* cfg, int32_t B, int32_t T, const void* q,
                            const int32_t* q_pos, const int8_t* k_codes, const uint16_t* k_scales,
                            int32_t n_kv, dca_dtype o_dtype, void* o, float* lse, void* workspace,
                            size_t ws_bytes, hipStream_t stream);
size_t dca_attention_q8_workspace_size(const dca_config* cfg, int32_t B, int32_t T, int32_t n_kv);

/* dca_attention_q8 over a key cache stored as q4_0 blocks (named with q8_0 among the scalar cache
 * types the pages read in registers inside the DCA kernel, Upstream Sync entry
 * "0119-p0-dcaon-scalar-inregister", and as the value half of their q8_0-K / q4_0-V pairs; no
 * layout printed).  Every 32 consecutive dims of one (key, KV head) row share an fp16 scale d; a
 * dim's value is d * (n - 8) with n its 4-bit code in [0, 15].
 * k_codes : uint8 [B,n_kv,Hkv,D/2]: dim 2j of a row in the low nibble of byte j, dim 2j+1 in the
 *           high nibble (this packing order is the library's; the pages fix none).
 * k_scales: fp16 bit patterns [B,n_kv,Hkv,D/32].
 * Everything else (q, outputs, limits, errors, stage events) as dca_attention_q8.
 * workspace: at least dca_attention_q4_workspace_size() bytes of device memory. */
dca_status dca_attention_q4(const dca_config* cfg, int32_t B, int32_t T, const void* q,
                            const int32_t* q_pos, const uint8_t* k_codes, const uint16_t* k_scales,
                            int32_t n_kv, dca_dtype o_dtype, void* o, float* lse, void* workspace,
                            size_t ws_bytes, hipStream_t stream);
size_t dca_attention_q4_workspace_size(const dca_config* cfg, int32_t B, int32_t T, int32_t n_kv);

/* Storage format of one region of a key cache (dca_attention_window). */
typedef enum dca_kv_format { DCA_KV_BF16 = 0, DCA_KV_Q8_0 = 1, DCA_KV_Q4_0 = 2 } dca_kv_format;

/* n consecutive cells of every sequence's key cache, in one format:
 *   DCA_KV_BF16: keys bf16 [B,n,Hkv,D], scales unused (may be NULL);
 *   DCA_KV_Q8_0: keys int8 codes [B,n,Hkv,D], scales fp16 [B,n,Hkv,D/32] (as dca_attention_q8);
 *   DCA_KV_Q4_0: keys uint8 codes [B,n,Hkv,D/2], scales fp16 [B,n,Hkv,D/32] (as dca_attention_q4).
 * The memory may be device memory or pinned host memory (hipHostMalloc or a pinned allocation of
 * the framework); the caller keeps ownership. */
typedef struct dca_kv_region {
  dca_kv_format format;
  const void* keys;
  const uint16_t* scales;
  int32_t n;
} dca_kv_region;

/* Decode over a key cache split into a window and a tail (the pages' rolling-KV residency: a
 * window of cells [0, wc) resident on the GPU and the tail [wc, n_kv) spilled to pinned host
 * memory, read by the DCA decode kernel straight from both regions, each at its own type:
 * Upstream Sync entries "0111-0113 rolling-KV spill made graceful" (the DCA streaming-tail path)
 * and "0120-p2-mixed-kv" (a more compressed type for the tail)).
 * Cells [0, window->n) come from `window`, cells [window->n, window->n + tail->n) from `tail`;
 * n_kv = window->n + tail->n, and cell j sits at position j as in dca_attention.  The result is
 * the attention over the whole cache (the split changes nothing but where the bytes are read
 * from).  A region in host memory is read over the host link by the kernels themselves, with no
 * staging copy; the library resolves its device address with the HIP runtime and rejects memory
 * the GPU cannot reach (pageable host memory) with DCA_ERR_INVALID_ARGUMENT.
 * q, q_pos, o, lse, limits and errors as dca_attention_q8 (split-KV path for every T, bf16 q).
 * workspace: at least dca_attention_window_workspace_size() bytes of device memory. */
dca_status dca_attention_window(const dca_config* cfg, int32_t B, int32_t T, const void* q,
                                const int32_t* q_pos, const dca_kv_region* window,
                                const dca_kv_region* tail, dca_dtype o_dtype, void* o, float* lse,
                                void* workspace, size_t ws_bytes, hipStream_t stream);
size_t dca_attention_window_workspace_size(const dca_config* cfg, int32_t B, int32_t T,
                                           int32_t n_win, int32_t n_tail);

/* Optional stage timing for dca_attention (measurement hook; no page defines it).  After
 * dca_set_stage_events(ev, n) with n >= DCA_N_STAGE_EVENTS, every dca_attention call made later on
 * this thread records, on its stream: ev[0] before the remap, ev[1] after the remap, ev[2] after
 * the query rotation, ev[3] after the key rotation (prefill) or the cos/sin tables (decode), ev[4]
 * after the regime passes, ev[5] after the merge.  The events are created and owned by the caller
 * (hipEventCreate); NULL or n = 0 turns the hook off.  n in (0, DCA_N_STAGE_EVENTS) is an error. */
#define DCA_N_STAGE_EVENTS 6
dca_status dca_set_stage_events(hipEvent_t* events, int32_t n);

/* Thread-local text describing the last non-OK status returned on this thread ("" if none). */
const char* dca_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DCA_H */
