/*
 * dca_oracle.c -- plain, slow, fp64 CPU oracle for Dual Chunk Attention (DCA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load this file's library.  It shares no code, header, table or constant with the
 * GPU library; the two only read the same seeded input bytes.
 *
 * Sources (page titles and sections; the pages print no numeric example):
 *  [F] "Feature -- Gemma-4 A4B Dual Chunk Attention (DCA), training-free 1M context":
 *      - "DCA algorithm (global layers only)": three regimes (intra, successive, inter), each a
 *        separately rope'd attention emitting LSE, merged by online softmax; only the rotary
 *        dims are remapped, the other dims pass through.
 *      - "Section C design": keys at j mod c, queries at (i mod c), (i mod c)+c and a clamped
 *        inter position; the regimes partition the causal triangle.
 *      - "Section-C ENGINEERING DESIGN": keys are cached un-rotated; values are the un-rotated
 *        projection (K = V on these layers, "Why llamafile is sufficient").
 *      - "Implementation progress + Section-D simplification": lse = max + log(rowsum) and the
 *        merge M = max lse_r, w_r = exp(lse_r - M), O = sum w_r O_r / sum w_r.
 *      - "Section C2b": an empty regime yields O = 0, lse = -inf and weight 0.
 *  [U] "Protocol -- Upstream Sync", entry "0110 WS2 asym-band NaN guard": a zero exp-sum gives 0.
 *
 * The remap rule this oracle fixes (readings of the pages, stated once here):
 *   chunk(x) = floor(x / c).  For a query at absolute position i and a key at cell j
 *   (cell index = position; 0 <= j <= i, j < n_kv):
 *     intra : chunk(j) == chunk(i)
 *     succ  : chunk(j) == chunk(i) - 1 and i - j < c
 *     inter : i - j >= c
 *   key position      pos_k(j)  = j mod c
 *   query positions   intra: i mod c;  succ: (i mod c) + c;  inter: c - 1
 *   The pages print the inter query position as c ([F] table) and as 2c ([U] "opencoti F5
 *   dca"); both let a distance reach c or more.  The reading here clamps it to c - 1 so that every
 *   rotary distance lies in [0, c).  The pages' succ regime covers the whole previous chunk,
 *   whose distances reach 2c - 1; the reading here keeps the succ query position (continuous
 *   with intra, so intra and succ see the true distance i - j) and moves previous-chunk keys at
 *   distance >= c into inter.
 *
 * Page-literal remap modes (mode argument; 0 is the reading above):
 *   mode 1: the [F] "Section C design" table as printed: succ holds the whole previous chunk
 *           (chunk(j) == chunk(i) - 1), inter every older chunk (chunk(j) < chunk(i) - 1), and
 *           the inter query sits at c.  Distances: intra and succ i - j (succ up to 2c - 1),
 *           inter c - (j mod c) in [1, c].
 *   mode 2: as mode 1 with the inter query at 2c ([U] entry "opencoti F5 dca", its fused kernel
 *           and the #635 cache fill).  Inter distances 2c - (j mod c) in [c + 1, 2c].
 *
 * RoPE reading: rotary dims [0, n_rot) form pairs (f, f + n_rot/2); for pair f,
 *   a = p * theta^(-2f/n_rot) / ff[f];
 *   y_f = x_f cos a - x_{f+n_rot/2} sin a;  y_{f+n_rot/2} = x_f sin a + x_{f+n_rot/2} cos a.
 *   Dims >= n_rot are copied.  Everything is fp64.
 *
 * YaRN magnitude factor (attn_factor, default 1): the pages let DCA compose with YaRN's magnitude
 * scale ("--dca-yarn-factor", fed as the rope's attention factor, [F] "Runtime knobs"; measured
 * there as no win for retrieval).  Reading: the rotated dims of every query and key are multiplied
 * by the factor, y_f = m (x_f cos a - ...), so the rotary part of each score scales by m^2; the
 * pass-through dims and the values (un-rotated keys) are untouched.
 *
 * Quantized keys (q8_0): the pages run DCA over caches of type q8_0 ([U] entries "DCA all-KV"
 * and "0119-p0-dcaon-scalar-inregister", which read the codes in registers inside the kernel) and
 * give its size as about 0.53x of f16, but print no layout.  Reading: every 32 consecutive dims of
 * one (key, KV head) row form a block with one fp16 scale d and 32 signed 8-bit codes q, and the
 * key's value in a dim is d * q (34 bytes per 32 values).  The codes are stored as int8 [..][D]
 * in the key layout and the scales as fp16 [..][D/32] in the same order.  The oracle reads the
 * value d * q exactly (fp16 -> double by the IEEE binary16 definition) and then runs the same
 * attention on it.
 *
 * Quantized keys (q4_0): the pages name q4_0 beside q8_0 among the scalar cache types read in
 * registers ([U] "0119-p0-dcaon-scalar-inregister", and the q8_0-K / q4_0-V pairs), again with no
 * layout.  Reading: every 32 consecutive dims form a block with one fp16 scale d and 32 unsigned
 * 4-bit codes n in [0, 15]; the value is d * (n - 8).  Codes are packed two per byte in dim order:
 * dim 2j in the low nibble of byte j, dim 2j + 1 in the high nibble (uint8 [..][D/2]); scales as
 * for q8_0.  This packing order is this file's reading (the pages fix none).
 *
 * Scores s_j = scale * <rot(q, P_reg(j)), rot(k_j, j mod c)>, softmax over the union of the
 * regimes, O = sum_j softmax_j * k_j (un-rotated), LSE = m + ln sum_j e^(s_j - m).
 * Query head h uses KV head h / (Hq / Hkv).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_INTRA 0
#define OR_SUCC 1
#define OR_INTER 2

static int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) q -= 1;
  return q;
}

static int64_t pos_mod(int64_t a, int64_t b) { return a - floor_div(a, b) * b; }

/* Regime of key j for a query at position i ([F] "Section C design" table, with the reading
 * above).  Returns -1 when the key is not attended (j > i, j < 0 or j >= n_kv). */
int dca_oracle_regime(int64_t i, int64_t j, int64_t c, int64_t n_kv, int mode) {
  if (j < 0 || j > i || j >= n_kv) return -1;
  int64_t ci = floor_div(i, c), cj = floor_div(j, c);
  if (cj == ci) return OR_INTRA;
  if (mode != 0) return cj == ci - 1 ? OR_SUCC : OR_INTER; /* page table: by chunk alone */
  if (cj == ci - 1 && i - j < c) return OR_SUCC;
  if (i - j >= c) return OR_INTER;
  return -2; /* unreachable: a key in an older chunk is always at distance >= c */
}

/* Remapped query position of regime r for a query at i. */
int64_t dca_oracle_query_pos(int64_t i, int64_t c, int r, int mode) {
  if (r == OR_INTRA) return pos_mod(i, c);
  if (r == OR_SUCC) return pos_mod(i, c) + c;
  if (mode == 1) return c;
  if (mode == 2) return 2 * c;
  return c - 1;
}

/* Key position of cell j. */
int64_t dca_oracle_key_pos(int64_t j, int64_t c) { return pos_mod(j, c); }

/* Positions and per-regime key intervals, found by enumerating every key with the explicit
 * regime predicate (no interval formula).  pos_q [3][n_rows], pos_k [n_kv], bounds
 * [3][n_rows][2] (inclusive lo, hi; empty = (0, -1)).  Any output may be NULL.
 * Returns 0, or -(row+1) for the first row whose regime key set is not one contiguous
 * interval, or -(n_rows+1) if the predicate reached its unreachable branch. */
int64_t dca_oracle_remap(int64_t c, int mode, int64_t n_rows, const int32_t* qpos, int64_t n_kv,
                         int32_t* pos_q, int32_t* pos_k, int32_t* bounds, int n_threads) {
  int64_t status = 0;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
  if (pos_k)
    for (int64_t j = 0; j < n_kv; ++j) pos_k[j] = (int32_t)dca_oracle_key_pos(j, c);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t row = 0; row < n_rows; ++row) {
    int64_t i = qpos[row];
    for (int r = 0; r < 3; ++r) {
      if (pos_q) pos_q[r * n_rows + row] = (int32_t)dca_oracle_query_pos(i, c, r, mode);
    }
    int64_t lo[3] = {-1, -1, -1}, hi[3] = {-1, -1, -1}, cnt[3] = {0, 0, 0};
    int bad = 0;
    int64_t jmax = i < n_kv - 1 ? i : n_kv - 1;
    for (int64_t j = 0; j <= jmax; ++j) {
      int r = dca_oracle_regime(i, j, c, n_kv, mode);
      if (r < 0) { bad = 2; continue; }
      if (cnt[r] == 0) lo[r] = j;
      hi[r] = j;
      cnt[r] += 1;
    }
    for (int r = 0; r < 3; ++r) {
      if (cnt[r] > 0 && hi[r] - lo[r] + 1 != cnt[r]) bad = bad ? bad : 1;
      if (bounds) {
        bounds[(r * n_rows + row) * 2 + 0] = cnt[r] ? (int32_t)lo[r] : 0;
        bounds[(r * n_rows + row) * 2 + 1] = cnt[r] ? (int32_t)hi[r] : -1;
      }
    }
    if (bad) {
#pragma omp critical
      {
        int64_t code = bad == 1 ? -(row + 1) : -(n_rows + 1);
        if (status == 0 || code > status) status = code;
      }
    }
  }
  return status;
}

/* Rotation of one head vector x[0..D) at position p into y (fp64), the RoPE reading above; the
 * rotated dims are multiplied by mag (the YaRN magnitude factor of the header; 1 = none). */
static void rope_one(int64_t n_rot, int64_t D, double theta, const double* ff, double mag,
                     const double* x, double p, double* y) {
  int64_t half = n_rot / 2;
  for (int64_t f = 0; f < half; ++f) {
    double w = pow(theta, -2.0 * (double)f / (double)n_rot);
    if (ff) w /= ff[f];
    double a = p * w;
    double cs = mag * cos(a), sn = mag * sin(a);
    double x0 = x[f], x1 = x[f + half];
    y[f] = x0 * cs - x1 * sn;
    y[f + half] = x0 * sn + x1 * cs;
  }
  for (int64_t d = n_rot; d < D; ++d) y[d] = x[d];
}

/* Partial RoPE of x [rows][H][D] at pos [rows] into y (fp64). */
void dca_oracle_rope(int64_t n_rot, int64_t D, double theta, const double* ff, const double* x,
                     const int64_t* pos, int64_t rows, int64_t H, double* y, double mag) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t h = 0; h < H; ++h)
      rope_one(n_rot, D, theta, ff, mag, x + (r * H + h) * D, (double)pos[r], y + (r * H + h) * D);
}

/* Element e of an input array that is fp32 (in_bf16 = 0) or bf16 bit patterns (in_bf16 = 1). */
static double load_in(const void* p, int64_t e, int in_bf16) {
  if (in_bf16) {
    uint32_t bits = (uint32_t)((const uint16_t*)p)[e] << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
  }
  return (double)((const float*)p)[e];
}

/* Value of IEEE binary16 bits: sign, 5-bit exponent (bias 15), 10-bit fraction; exponent 0 is the
 * subnormal range fraction * 2^-24, exponent 31 infinity or NaN. */
double dca_oracle_half(uint16_t h) {
  const int sign = h >> 15, ex = (h >> 10) & 31, fr = h & 1023;
  double v;
  if (ex == 0)
    v = ldexp((double)fr, -24);
  else if (ex == 31)
    v = fr ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + fr), ex - 25);
  return sign ? -v : v;
}

/* A key cache: fp32 (kind 0), bf16 bit patterns (kind 1), q8_0 (kind 2: int8 codes in p, fp16
 * scale bits in scales, one per 32 consecutive elements of a row) or q4_0 (kind 3: 4-bit codes,
 * element e in byte e / 2, low nibble for even e; same scales). */
typedef struct {
  const void* p;
  const uint16_t* scales;
  int kind;
} kv_src;

static double load_k(const kv_src* k, int64_t e) {
  if (k->kind == 2) return dca_oracle_half(k->scales[e / 32]) * (double)((const int8_t*)k->p)[e];
  if (k->kind == 3) {
    const int byte = ((const uint8_t*)k->p)[e / 2];
    const int n = (e % 2 == 0) ? (byte & 15) : (byte >> 4);
    return dca_oracle_half(k->scales[e / 32]) * (double)(n - 8);
  }
  return load_in(k->p, e, k->kind);
}

/* Dequantized values of n elements of a q8_0 cache (codes + fp16 scales), for the tests. */
void dca_oracle_dequant_q8(const int8_t* codes, const uint16_t* scales, int64_t n, double* out) {
  kv_src k = {codes, scales, 2};
  for (int64_t e = 0; e < n; ++e) out[e] = load_k(&k, e);
}

/* Dequantized values of n elements of a q4_0 cache (codes packed two per byte + fp16 scales). */
void dca_oracle_dequant_q4(const uint8_t* codes, const uint16_t* scales, int64_t n, double* out) {
  kv_src k = {codes, scales, 3};
  for (int64_t e = 0; e < n; ++e) out[e] = load_k(&k, e);
}

/* Round-to-nearest-even of a double to bf16 (through fp32, as a rotated value is formed in fp32
 * and then stored as bf16), returned as a double. */
static double round_bf16(double v) {
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* N-way LSE merge ([F] "Implementation progress + Section-D simplification"; zero weight of an
 * empty part from "Section C2b"; zero exp-sum rule from [U] entry 0110).
 * o_parts [n_parts][rows][D], lse_parts [n_parts][rows] -> o [rows][D], lse [rows]. */
void dca_oracle_merge(int64_t n_parts, const double* o_parts, const double* lse_parts,
                      int64_t rows, int64_t D, double* o, double* lse) {
  for (int64_t x = 0; x < rows; ++x) {
    double M = -INFINITY;
    for (int64_t p = 0; p < n_parts; ++p)
      if (lse_parts[p * rows + x] > M) M = lse_parts[p * rows + x];
    for (int64_t d = 0; d < D; ++d) o[x * D + d] = 0.0;
    if (M == -INFINITY) { lse[x] = -INFINITY; continue; }
    double W = 0.0;
    for (int64_t p = 0; p < n_parts; ++p) {
      double l = lse_parts[p * rows + x];
      if (l == -INFINITY) continue;
      double w = exp(l - M);
      W += w;
      for (int64_t d = 0; d < D; ++d) o[x * D + d] += w * o_parts[(p * rows + x) * D + d];
    }
    for (int64_t d = 0; d < D; ++d) o[x * D + d] /= W;
    lse[x] = M + log(W);
  }
}

/* DCA attention on selected query rows, fp64.
 *   q    [B][T][Hq][D] pre-RoPE,   qpos [B][T],   k [B][n_kv][Hkv][D] pre-RoPE (also V)
 *   sel  [n_sel] flat row indices b*T + t
 *   o    [n_sel][Hq][D],  lse [n_sel][Hq]                    -- union softmax (the definition)
 *   o_reg [3][n_sel][Hq][D], lse_reg [3][n_sel][Hq] (NULL ok) -- per-regime partials
 * rot_round = 1 rounds the rotated dims of the queries and keys to bf16 (nearest-even) before
 * the scores are formed: the contract of a caller that hands over bf16 rotated operands (used to
 * check the per-regime entry point); 0 keeps them exact.
 * Returns 0, or -1 on allocation failure, -2 on a bad argument. */
static int attention_impl(int64_t D, int64_t n_rot, int64_t Hq, int64_t Hkv, int64_t c, int mode,
                          double theta, double scale, const double* ff, int in_bf16, int rot_round,
                          int64_t B, int64_t T, const void* q, const int32_t* qpos, const kv_src* kv,
                          int64_t n_kv, int64_t n_sel, const int64_t* sel, double* o, double* lse,
                          double* o_reg, double* lse_reg, int n_threads, double mag) {
  if (!(mag > 0.0) || !isfinite(mag)) return -2;
  if (D <= 0 || n_rot <= 0 || n_rot > D || n_rot > 1024 || (n_rot & 1) || Hq <= 0 || Hkv <= 0 ||
      Hq % Hkv || c <= 0 || mode < 0 || mode > 2 || B <= 0 || T <= 0 || n_kv < 0 ||
      (kv->kind >= 2 && (D % 32 || !kv->scales)))
    return -2;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
  const int64_t G = Hq / Hkv;
  int status = 0;
  for (int64_t b = 0; b < B; ++b) {
    /* rows of this batch entry among the selection */
    int64_t nb = 0;
    for (int64_t s = 0; s < n_sel; ++s)
      if (sel[s] / T == b) ++nb;
    if (nb == 0) continue;
    /* keys of sequence b rotated at pos_k(j) = j mod c: only the rotary dims are stored */
    double* krot = (double*)malloc(sizeof(double) * (size_t)(n_kv > 0 ? n_kv : 1) * Hkv * n_rot);
    if (!krot) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n_kv; ++j) {
      double xin[1024], xout[1024];
      for (int64_t g = 0; g < Hkv; ++g) {
        for (int64_t d = 0; d < n_rot; ++d)
          xin[d] = load_k(kv, ((b * n_kv + j) * Hkv + g) * D + d);
        rope_one(n_rot, n_rot, theta, ff, mag, xin, (double)dca_oracle_key_pos(j, c), xout);
        if (rot_round == 1)
          for (int64_t d = 0; d < n_rot; ++d) xout[d] = round_bf16(xout[d]);
        memcpy(krot + (j * Hkv + g) * n_rot, xout, sizeof(double) * n_rot);
      }
    }
    int64_t work = n_sel * Hq;
#pragma omp parallel
    {
      double* s_buf = (double*)malloc(sizeof(double) * (size_t)(n_kv > 0 ? n_kv : 1));
      signed char* r_buf = (signed char*)malloc((size_t)(n_kv > 0 ? n_kv : 1));
      double* qv = (double*)malloc(sizeof(double) * D);
      double* qr = (double*)malloc(sizeof(double) * 3 * D);
      double* acc = (double*)malloc(sizeof(double) * D);
      if (!s_buf || !r_buf || !qv || !qr || !acc) {
#pragma omp critical
        status = -1;
      } else {
#pragma omp for schedule(dynamic, 1)
        for (int64_t wi = 0; wi < work; ++wi) {
          int64_t s = wi / Hq, h = wi % Hq;
          int64_t flat = sel[s];
          if (flat / T != b) continue;
          int64_t i = qpos[flat];
          int64_t g = h / G;
          for (int64_t d = 0; d < D; ++d) qv[d] = load_in(q, (flat * Hq + h) * D + d, in_bf16);
          for (int r = 0; r < 3; ++r) {
            rope_one(n_rot, D, theta, ff, mag, qv, (double)dca_oracle_query_pos(i, c, r, mode), qr + r * D);
            if (rot_round == 1)
              for (int64_t d = 0; d < n_rot; ++d) qr[r * D + d] = round_bf16(qr[r * D + d]);
          }
          int64_t jmax = i < n_kv - 1 ? i : n_kv - 1;
          /* scores of every attended key, each with its own regime's query rotation */
          for (int64_t j = 0; j <= jmax; ++j) {
            int r = dca_oracle_regime(i, j, c, n_kv, mode);
            r_buf[j] = (signed char)r;
            const double* qq = qr + (r < 0 ? 0 : r) * D;
            double dot = 0.0;
            for (int64_t d = 0; d < n_rot; ++d) dot += qq[d] * krot[(j * Hkv + g) * n_rot + d];
            for (int64_t d = n_rot; d < D; ++d)
              dot += qq[d] * load_k(kv, ((b * n_kv + j) * Hkv + g) * D + d);
            s_buf[j] = scale * dot;
          }
          /* regime set -1 = the union; then each regime alone */
          for (int set = -1; set < 3; ++set) {
            double* out_o;
            double* out_l;
            if (set < 0) {
              out_o = o + (s * Hq + h) * D;
              out_l = lse + s * Hq + h;
            } else {
              if (!o_reg || !lse_reg) break;
              out_o = o_reg + ((set * n_sel + s) * Hq + h) * D;
              out_l = lse_reg + (set * n_sel + s) * Hq + h;
            }
            double m = -INFINITY;
            for (int64_t j = 0; j <= jmax; ++j)
              if ((set < 0 || r_buf[j] == set) && s_buf[j] > m) m = s_buf[j];
            for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
            if (m == -INFINITY) { /* empty: O = 0, lse = -inf */
              memcpy(out_o, acc, sizeof(double) * D);
              *out_l = -INFINITY;
              continue;
            }
            double Z = 0.0;
            for (int64_t j = 0; j <= jmax; ++j) {
              if (set >= 0 && r_buf[j] != set) continue;
              double e = exp(s_buf[j] - m);
              Z += e;
              for (int64_t d = 0; d < D; ++d)
                acc[d] += e * load_k(kv, ((b * n_kv + j) * Hkv + g) * D + d);
            }
            for (int64_t d = 0; d < D; ++d) out_o[d] = acc[d] / Z;
            *out_l = m + log(Z);
          }
        }
      }
      free(s_buf);
      free(r_buf);
      free(qv);
      free(qr);
      free(acc);
    }
    free(krot);
    if (status) return status;
  }
  return status;
}

int dca_oracle_attention(int64_t D, int64_t n_rot, int64_t Hq, int64_t Hkv, int64_t c, int mode,
                         double theta, double scale, const double* ff, int in_bf16, int rot_round,
                         int64_t B,
                         int64_t T, const void* q, const int32_t* qpos, const void* k, int64_t n_kv,
                         int64_t n_sel, const int64_t* sel, double* o, double* lse, double* o_reg,
                         double* lse_reg, int n_threads, double attn_factor) {
  kv_src kv = {k, NULL, in_bf16};
  return attention_impl(D, n_rot, Hq, Hkv, c, mode, theta, scale, ff, in_bf16, rot_round, B, T, q,
                        qpos, &kv, n_kv, n_sel, sel, o, lse, o_reg, lse_reg, n_threads, attn_factor);
}

/* The same attention over a q8_0 key cache (codes int8 [B][n_kv][Hkv][D], scales fp16 bits
 * [B][n_kv][Hkv][D/32]); queries fp32 (q_bf16 = 0) or bf16 bit patterns (q_bf16 = 1). */
int dca_oracle_attention_q8(int64_t D, int64_t n_rot, int64_t Hq, int64_t Hkv, int64_t c, int mode,
                            double theta, double scale, const double* ff, int q_bf16, int64_t B,
                            int64_t T, const void* q, const int32_t* qpos, const int8_t* codes,
                            const uint16_t* scales, int64_t n_kv, int64_t n_sel, const int64_t* sel,
                            double* o, double* lse, double* o_reg, double* lse_reg, int n_threads,
                            double attn_factor) {
  kv_src kv = {codes, scales, 2};
  return attention_impl(D, n_rot, Hq, Hkv, c, mode, theta, scale, ff, q_bf16, 0, B, T, q, qpos,
                        &kv, n_kv, n_sel, sel, o, lse, o_reg, lse_reg, n_threads, attn_factor);
}

/* The same attention over a q4_0 key cache (codes uint8 [B][n_kv][Hkv][D/2], two per byte, scales
 * fp16 bits [B][n_kv][Hkv][D/32]). */
int dca_oracle_attention_q4(int64_t D, int64_t n_rot, int64_t Hq, int64_t Hkv, int64_t c, int mode,
                            double theta, double scale, const double* ff, int q_bf16, int64_t B,
                            int64_t T, const void* q, const int32_t* qpos, const uint8_t* codes,
                            const uint16_t* scales, int64_t n_kv, int64_t n_sel, const int64_t* sel,
                            double* o, double* lse, double* o_reg, double* lse_reg, int n_threads,
                            double attn_factor) {
  kv_src kv = {codes, scales, 3};
  return attention_impl(D, n_rot, Hq, Hkv, c, mode, theta, scale, ff, q_bf16, 0, B, T, q, qpos,
                        &kv, n_kv, n_sel, sel, o, lse, o_reg, lse_reg, n_threads, attn_factor);
}
