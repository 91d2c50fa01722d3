/*
 * CPU fp64 oracle for MLA decode over a paged latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code with the HIP library.
 *
 * What it computes (plain definition, fp64 throughout, sums in ascending
 * index order):
 *   - A cache row is 576 wide: a 512-wide latent that is also V, then a
 *     64-wide RoPE part (tokenspeed-mla package page, "Quickstart":
 *     kv_lora_rank / qk_rope_head_dim arguments; TokenSpeed MLA article,
 *     section 6: kv_cache [num_pages, page_size, D_total]).
 *   - Key j of sequence b lives in page block_table[b][j / page_size] at slot
 *     j % page_size (same article, section 6: kv_cache with block_tables).
 *   - Query token t of q_len sees keys j < n_t = clamp(L - q_len + t + 1, 0, L)
 *     where L = seq_lens[b] (causal across the q_len new tokens; bottom-right
 *     alignment is the reading taken where the pages only say "causal",
 *     article section 4, static key list).
 *   - Sliding window (TokenSpeed MLA article, section 6: the decode tests
 *     include a sliding-window mask; the pages do not spell out its
 *     convention): with window W > 0, token t sees only its last W visible
 *     keys, j in [max(0, n_t - W), n_t).  W = 0 is the plain causal mask.
 *   - s_j = softmax_scale * sum_d qv[d] * kv[d], qv = q_scale * dec(q),
 *     kv = kv_scale * dec(row).  O = sum_j softmax(s)_j * V_j (first 512),
 *     LSE = ln sum_j exp(s_j) (natural log).  A row with no visible key gets
 *     O = 0 and LSE = -inf.
 *   - Split mode (article section 2, the two-kernel split-KV scheme): the
 *     visible keys of every row are cut into consecutive chunks of
 *     `split_len` keys; each chunk yields a normalised partial O_s and
 *     lse_s; they are merged as LSE = ln sum_s exp(lse_s) and
 *     O = sum_s exp(lse_s - LSE) * O_s.  This must equal the unsplit result.
 *   - Mixed inputs (tokenspeed-mla package page, "What it is": FP16, BF16
 *     and FP8 decode; the reading taken here is bf16 queries over an FP8
 *     E4M3 cache): q is decoded as bf16 and every cache row as E4M3.
 *   - Decoders are written from the format definitions: bf16 is the top 16
 *     bits of an IEEE binary32; OCP FP8 E4M3 has bias 7, no infinities,
 *     S.1111.111 = NaN, subnormals m/8 * 2^-6.
 *
 * Parity of the split/merge and fold paths is pinned by the tests against
 * the unsplit definition, a dense brute force and closed forms.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_D_QK 576
#define ORC_D_V 512

enum { ORC_BF16 = 1, ORC_FP8_E4M3 = 2, ORC_FP16 = 3, ORC_BF16_Q_E4M3_KV = 4 };
/* element formats of q and of the cache rows for a dtype code */
static int q_format(int dtype) { return dtype == ORC_BF16_Q_E4M3_KV ? ORC_BF16 : dtype; }
static int kv_format(int dtype) { return dtype == ORC_BF16_Q_E4M3_KV ? ORC_FP8_E4M3 : dtype; }

double oracle_dec_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* IEEE binary16: bias 15, 10 fraction bits, subnormals m/1024 * 2^-14, exponent 31 = inf/NaN
 * (tokenspeed-mla package page: FP16 is one of the decode input types). */
double oracle_dec_f16(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 31) return m ? NAN : (s ? -INFINITY : INFINITY);
  if (e == 0)
    v = ldexp((double)m / 1024.0, -14);
  else
    v = ldexp(1.0 + (double)m / 1024.0, e - 15);
  return s ? -v : v;
}

double oracle_dec_e4m3(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

static void decode_row(const void* base, int dtype, size_t elem_index, int n, double scale, double* dst) {
  if (dtype == ORC_BF16) {
    const uint16_t* p = (const uint16_t*)base + elem_index;
    for (int d = 0; d < n; ++d) dst[d] = scale * oracle_dec_bf16(p[d]);
  } else if (dtype == ORC_FP16) {
    const uint16_t* p = (const uint16_t*)base + elem_index;
    for (int d = 0; d < n; ++d) dst[d] = scale * oracle_dec_f16(p[d]);
  } else {
    const uint8_t* p = (const uint8_t*)base + elem_index;
    for (int d = 0; d < n; ++d) dst[d] = scale * oracle_dec_e4m3(p[d]);
  }
}

/* Softmax over keys [j0, j1) of one query token, for all H heads at once.
 * scores: [H][j1-j0] scratch; qv: [H][576]; o: [H][512] normalised output;
 * lse: [H].  Returns 0, or -1 if a block_table entry is out of range. */
static int attend_range(const void* kv, int dtype, const int32_t* bt_row, int num_pages, int page_size,
                        int j0, int j1, int H, const double* qv, double softmax_scale, double kv_scale,
                        double* scores, double* row, double* o, double* lse, double* absv) {
  int n = j1 - j0;
  if (n <= 0) {
    for (int h = 0; h < H; ++h) {
      lse[h] = -INFINITY;
      for (int d = 0; d < ORC_D_V; ++d) o[(size_t)h * ORC_D_V + d] = 0.0;
      if (absv)
        for (int d = 0; d < ORC_D_V; ++d) absv[(size_t)h * ORC_D_V + d] = 0.0;
    }
    return 0;
  }
  /* pass 1: every score */
  for (int j = j0; j < j1; ++j) {
    int32_t page = bt_row[j / page_size];
    if (page < 0 || page >= num_pages) return -1;
    size_t e = ((size_t)page * page_size + (size_t)(j % page_size)) * ORC_D_QK;
    decode_row(kv, dtype, e, ORC_D_QK, kv_scale, row);
    for (int h = 0; h < H; ++h) {
      const double* qh = qv + (size_t)h * ORC_D_QK;
      double acc = 0.0;
      for (int d = 0; d < ORC_D_QK; ++d) acc += qh[d] * row[d];
      scores[(size_t)h * n + (j - j0)] = softmax_scale * acc;
    }
  }
  /* max and normaliser */
  for (int h = 0; h < H; ++h) {
    double mx = -INFINITY, l = 0.0;
    for (int k = 0; k < n; ++k) mx = fmax(mx, scores[(size_t)h * n + k]);
    for (int k = 0; k < n; ++k) l += exp(scores[(size_t)h * n + k] - mx);
    lse[h] = mx + log(l);
    for (int k = 0; k < n; ++k) scores[(size_t)h * n + k] = exp(scores[(size_t)h * n + k] - mx) / l;
    for (int d = 0; d < ORC_D_V; ++d) o[(size_t)h * ORC_D_V + d] = 0.0;
    if (absv)
      for (int d = 0; d < ORC_D_V; ++d) absv[(size_t)h * ORC_D_V + d] = 0.0;
  }
  /* pass 2: probability-weighted sum of V rows */
  for (int j = j0; j < j1; ++j) {
    int32_t page = bt_row[j / page_size];
    size_t e = ((size_t)page * page_size + (size_t)(j % page_size)) * ORC_D_QK;
    decode_row(kv, dtype, e, ORC_D_V, kv_scale, row);
    for (int h = 0; h < H; ++h) {
      double p = scores[(size_t)h * n + (j - j0)];
      double* oh = o + (size_t)h * ORC_D_V;
      for (int d = 0; d < ORC_D_V; ++d) oh[d] += p * row[d];
      if (absv) {
        double* ah = absv + (size_t)h * ORC_D_V;
        for (int d = 0; d < ORC_D_V; ++d) ah[d] += p * fabs(row[d]);
      }
    }
  }
  return 0;
}

/*
 * q:          [B, q_len, H, 576] bf16 / fp16 bits or e4m3 codes
 * kv:         [num_pages, page_size, 576], same format as q, except for
 *             ORC_BF16_Q_E4M3_KV: bf16 q, e4m3 cache
 * block_table:[B, max_pages] int32 (row stride max_pages)
 * seq_lens:   [B] int32
 * out:        [B, q_len, H, 512] fp64;  lse: [B, q_len, H] fp64
 * split_len:  0 = plain definition; > 0 = split/merge with chunks of that many keys
 * window:     0 = causal; > 0 = token t sees keys [max(0, n_t - window), n_t)
 * absv:       optional [B, q_len, H, 512] fp64: sum_j softmax_j * |V_j[d]|, the scale of
 *             the output's sensitivity to per-weight rounding (unsplit mode only)
 * Returns 0 on success, -1 on a block_table entry out of range, -2 on bad arguments.
 */
int oracle_mla_decode(const void* q, const void* kv, int dtype, const int32_t* block_table, int max_pages,
                      const int32_t* seq_lens, int B, int q_len, int H, int num_pages, int page_size,
                      double softmax_scale, double q_scale, double kv_scale, int split_len, int window,
                      double* out, double* lse, double* absv, int num_threads) {
  if (!q || !kv || !block_table || !seq_lens || !out || !lse) return -2;
  if (dtype != ORC_BF16 && dtype != ORC_FP8_E4M3 && dtype != ORC_FP16 && dtype != ORC_BF16_Q_E4M3_KV) return -2;
  const int qfmt = q_format(dtype), kvfmt = kv_format(dtype);
  if (B < 0 || q_len <= 0 || H <= 0 || page_size <= 0 || max_pages < 0 || split_len < 0 || window < 0) return -2;
  if (absv && split_len > 0) return -2;
  for (int b = 0; b < B; ++b) {
    if (seq_lens[b] < 0 || (seq_lens[b] + page_size - 1) / page_size > max_pages) return -2;
  }
  int status = 0;
  int npairs = B * q_len;
#ifdef _OPENMP
  if (num_threads > 0) omp_set_num_threads(num_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(min : status)
#endif
  for (int pair = 0; pair < npairs; ++pair) {
    int st = 0; /* this pair's status (the reduction copy starts at INT_MAX) */
    int b = pair / q_len, t = pair % q_len;
    int L = seq_lens[b];
    int n = L - q_len + t + 1;
    if (n < 0) n = 0;
    if (n > L) n = L;
    int lo = (window > 0 && n > window) ? n - window : 0; /* first visible key */
    int chunk = split_len > 0 ? split_len : (n - lo > 0 ? n - lo : 1);
    size_t row0 = ((size_t)b * q_len + t) * H;
    double* qv = (double*)malloc(sizeof(double) * (size_t)H * ORC_D_QK);
    double* row = (double*)malloc(sizeof(double) * ORC_D_QK);
    double* scores = (double*)malloc(sizeof(double) * (size_t)H * (size_t)(chunk > 0 ? chunk : 1));
    double* o_s = (double*)malloc(sizeof(double) * (size_t)H * ORC_D_V);
    double* lse_s = (double*)malloc(sizeof(double) * (size_t)H);
    double* o_acc = out + row0 * ORC_D_V;
    double* lse_acc = lse + row0;
    for (int h = 0; h < H; ++h) decode_row(q, qfmt, (row0 + h) * ORC_D_QK, ORC_D_QK, q_scale, qv + (size_t)h * ORC_D_QK);
    const int32_t* bt_row = block_table + (size_t)b * max_pages;
    if (split_len == 0) {
      if (attend_range(kv, kvfmt, bt_row, num_pages, page_size, lo, n, H, qv, softmax_scale, kv_scale, scores, row,
                       o_acc, lse_acc, absv ? absv + row0 * ORC_D_V : NULL) != 0)
        st = -1;
    } else {
      /* chunk partials, then the LSE-weighted merge */
      int nsplit = (n - lo + chunk - 1) / chunk;
      if (nsplit == 0) nsplit = 1;
      double* all_o = (double*)malloc(sizeof(double) * (size_t)nsplit * H * ORC_D_V);
      double* all_l = (double*)malloc(sizeof(double) * (size_t)nsplit * H);
      for (int s = 0; s < nsplit && st == 0; ++s) {
        int j0 = lo + s * chunk, j1 = j0 + chunk < n ? j0 + chunk : n;
        if (attend_range(kv, kvfmt, bt_row, num_pages, page_size, j0, j1, H, qv, softmax_scale, kv_scale, scores, row,
                         all_o + (size_t)s * H * ORC_D_V, all_l + (size_t)s * H, NULL) != 0)
          st = -1;
      }
      for (int h = 0; h < H; ++h) {
        double mx = -INFINITY, sum = 0.0;
        for (int s = 0; s < nsplit; ++s) mx = fmax(mx, all_l[(size_t)s * H + h]);
        double* oh = o_acc + (size_t)h * ORC_D_V;
        for (int d = 0; d < ORC_D_V; ++d) oh[d] = 0.0;
        if (mx == -INFINITY) {
          lse_acc[h] = -INFINITY;
          continue;
        }
        for (int s = 0; s < nsplit; ++s) sum += exp(all_l[(size_t)s * H + h] - mx);
        double L_all = mx + log(sum);
        lse_acc[h] = L_all;
        for (int s = 0; s < nsplit; ++s) {
          double w = exp(all_l[(size_t)s * H + h] - L_all);
          const double* os = all_o + ((size_t)s * H + h) * ORC_D_V;
          for (int d = 0; d < ORC_D_V; ++d) oh[d] += w * os[d];
        }
      }
      free(all_o);
      free(all_l);
    }
    free(qv);
    free(row);
    free(scores);
    free(o_s);
    free(lse_s);
    if (st < status) status = st;
  }
  return status;
}

/* Largest F with q_len % F == 0 and H * F <= tile_m (TokenSpeed MLA article,
 * section 3: query-token folding).  Returns at least 1. */
int oracle_fold_factor(int q_len, int H, int tile_m) {
  int best = 1;
  for (int F = 1; F <= q_len; ++F)
    if (q_len % F == 0 && (long)H * F <= tile_m) best = F;
  return best;
}

/* OCP E4M3 encoder used by the K/V pack + quantise check: x -> code with
 * round-to-nearest-even on the E4M3 grid and saturation to +-448; NaN -> 0x7F.
 * Written from the format definition: the representable magnitudes are
 * m/8 * 2^-6 (subnormal) and (1 + m/8) * 2^(e-7), e = 1..15 (not 15/7). */
uint8_t oracle_enc_e4m3(double x) {
  if (isnan(x)) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs(x);
  if (a >= 448.0) return sign | 0x7E;
  /* walk the 127 non-negative finite codes; pick the nearest, ties to even mantissa code */
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double v = oracle_dec_e4m3((uint8_t)c);
    double err = fabs(v - a);
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  return sign | (uint8_t)best;
}

/* Pack + quantise (the step that appends decode's cache rows): row t of the
 * output is latent[t, 0:512] || rope[t, 0:64], each element divided by
 * kv_scale and encoded as E4M3.  Inputs are bf16 bits.  If slot_mapping is
 * non-NULL the row goes to cache row slot_mapping[t] (negative = skip).
 * The quotient that decides each code is taken in IEEE fp32 (the precision
 * the quantising kernel computes in), then rounded to E4M3 exactly. */
void oracle_kv_pack_quantize_fp8(const uint16_t* latent, const uint16_t* rope, int T, double kv_scale,
                                 const int64_t* slot_mapping, uint8_t* out) {
  for (int t = 0; t < T; ++t) {
    int64_t dst = slot_mapping ? slot_mapping[t] : t;
    if (dst < 0) continue;
    uint8_t* o = out + (size_t)dst * ORC_D_QK;
    const float s = (float)kv_scale;
    for (int d = 0; d < ORC_D_V; ++d) {
      volatile float qv = (float)oracle_dec_bf16(latent[(size_t)t * ORC_D_V + d]) / s;
      o[d] = oracle_enc_e4m3((double)qv);
    }
    for (int d = 0; d < 64; ++d) {
      volatile float qv = (float)oracle_dec_bf16(rope[(size_t)t * 64 + d]) / s;
      o[ORC_D_V + d] = oracle_enc_e4m3((double)qv);
    }
  }
}
