/*
 * oracle.c -- float64 CPU reference for grouped-query attention over a KV
 * cache kept in fixed 256-position pages behind a per-stream page table.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. It shares no code,
 * header, table or constant generator with the HIP library, and the product
 * path never calls it.
 *
 * What it computes, and where the pages define it:
 *   - Each query head reads the key head it belongs to (TensorFold pull
 *     request #1373, "What changes": each tile reads its query head's key
 *     head).  The grouping itself is not spelled out; the reading used here
 *     is g = floor(h / G), G = n_q_heads / n_kv_heads.
 *   - A paged stream's key at position t lives in page PT[t / 256], slot
 *     t mod 256, head-major inside the page: element offset
 *     PT[t/256]*PS + (g*256 + t mod 256)*D + d (pull request #2011, review
 *     section "Is paged output the same as windowed output?", the base
 *     address of hpattn_p256_kernel; pull request #1373, "What changes":
 *     PTOK rows a head, PS apart).
 *   - Paged and windowed attention are the same sums over the same bytes;
 *     only addresses change (pull request #2011, same review section).  So
 *     the oracle gathers K and V into logical order and then evaluates plain
 *     softmax attention, with no blocking of any kind.
 *   - Query row i of a stream sits at absolute position first_pos + i and
 *     sees keys 0..first_pos+i inclusive (causal rows against the paged
 *     prefix: pull request #1373, prompt rows; keys past the limit land as
 *     zeros: pull request #2011 review).
 *   - Speculative verify rows may carry a per-row ancestor table (pull
 *     request #1355, follow-up checks, "Indexing": the partial and merge
 *     kernels index a row table of ancestors beside the query rows).  The
 *     pages name the table only; the reading used here is one 32-bit word
 *     per row (at most 32 rows): keys before the stream's first row stay
 *     visible, and row i sees key first_pos + j (j <= i) when bit j is set.
 *     Without the table, rows are the causal chain above.
 *   - Decode is split-K partials plus a merge (issue #1344, "Mechanism":
 *     partial then attn_merge).  oracle_attention_split and oracle_merge give
 *     the split form, in the same float64 arithmetic, for the merge self-check.
 *   - fp8 caches are OCP E4M3FN codes times a per-tensor scale (the reading
 *     of "fp8-e4m3" with a per-tensor K and V scale); bf16 caches are bf16.
 *     Decoding is exact in float64.
 *
 * All arithmetic is float64 except the fp8 store quantiser, which divides in
 * float32 (the precision the device store uses) before rounding to E4M3FN.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_PAGE_POSITIONS 256
#define ORACLE_DTYPE_BF16 0
#define ORACLE_DTYPE_E4M3 1

/* ------------------------------------------------------------------------ */
/* Codecs                                                                   */
/* ------------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
double oracle_bf16_to_f64(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
 * S.1111.111 is NaN; exponent field 0 is subnormal with scale 2^-6. */
double oracle_e4m3_to_f64(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Store quantiser: y = fl32(x / scale), clamped to the largest finite code
 * (448), then rounded to nearest E4M3FN value, ties to an even mantissa.
 * NaN input gives the NaN code. */
uint8_t oracle_e4m3_encode(float x, float scale) {
  float y32 = x / scale; /* binary32 division, as the device store does */
  double y, a, quantum, r;
  int sign, ex, m;
  if (isnan(y32)) return 0x7F;
  y = (double)y32;
  if (y > 448.0) y = 448.0;
  if (y < -448.0) y = -448.0;
  sign = signbit(y) ? 1 : 0;
  a = fabs(y);
  if (a == 0.0) return (uint8_t)(sign << 7);
  /* a = f * 2^ex with f in [0.5, 1): the binade of a is [2^(ex-1), 2^ex). */
  (void)frexp(a, &ex);
  ex -= 1; /* a in [2^ex, 2^(ex+1)) */
  if (ex < -6) ex = -6; /* subnormal range shares the quantum of binade -6 */
  quantum = ldexp(1.0, ex - 3);
  r = nearbyint(a / quantum) * quantum; /* default mode: ties to even */
  /* r is now an exact E4M3FN magnitude (r <= 448 because a <= 448). */
  if (r < ldexp(1.0, -6)) {
    m = (int)(r / ldexp(1.0, -9));
    return (uint8_t)((sign << 7) | m);
  }
  (void)frexp(r, &ex);
  ex -= 1;
  m = (int)((r / ldexp(1.0, ex) - 1.0) * 8.0);
  return (uint8_t)((sign << 7) | ((ex + 7) << 3) | m);
}

void oracle_e4m3_encode_array(const float *x, int64_t n, float scale, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i], scale);
}

void oracle_bf16_to_f64_array(const uint16_t *x, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f64(x[i]);
}

void oracle_e4m3_to_f64_array(const uint8_t *x, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_to_f64(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Addressing                                                               */
/* ------------------------------------------------------------------------ */

/* Element offset of (position t, kv head g, dim 0).
 * page_table != NULL: paged, head-major page [Hkv][256][D], pages
 *   page_stride elements apart.
 * page_table == NULL: logical rows [t][Hkv][D]. */
static int64_t oracle_offset(const int32_t *page_table, int64_t page_stride, int n_kv_heads,
                             int head_dim, int64_t t, int g) {
  if (page_table) {
    int64_t page = page_table[t / ORACLE_PAGE_POSITIONS];
    int64_t slot = t % ORACLE_PAGE_POSITIONS;
    return page * page_stride + ((int64_t)g * ORACLE_PAGE_POSITIONS + slot) * head_dim;
  }
  return (t * n_kv_heads + g) * (int64_t)head_dim;
}

static double oracle_decode(const void *base, int dtype, int64_t idx, double scale) {
  if (dtype == ORACLE_DTYPE_BF16) return oracle_bf16_to_f64(((const uint16_t *)base)[idx]);
  return oracle_e4m3_to_f64(((const uint8_t *)base)[idx]) * scale;
}

/* Write n_rows new rows (bf16 bits, [n_rows][Hkv][D]) at positions
 * first_pos.. into the cache, quantising for fp8.  Rows are independent, so
 * they are shared out over n_threads threads (0: one per online core).
 * Returns 0, or -1 on a bad argument. */
typedef struct {
  void *k_dst, *v_dst;
  int dtype;
  float k_scale, v_scale;
  const int32_t *page_table;
  int64_t page_stride;
  int n_kv_heads, head_dim;
  const uint16_t *k_rows, *v_rows;
  int64_t first_pos, lo, hi;
} oracle_store_job;

static void *oracle_store_rows(void *arg) {
  oracle_store_job *J = (oracle_store_job *)arg;
  for (int64_t i = J->lo; i < J->hi; ++i) {
    int64_t t = J->first_pos + i;
    for (int g = 0; g < J->n_kv_heads; ++g) {
      int64_t dst = oracle_offset(J->page_table, J->page_stride, J->n_kv_heads, J->head_dim, t, g);
      int64_t src = (i * J->n_kv_heads + g) * (int64_t)J->head_dim;
      for (int d = 0; d < J->head_dim; ++d) {
        if (J->dtype == ORACLE_DTYPE_BF16) {
          ((uint16_t *)J->k_dst)[dst + d] = J->k_rows[src + d];
          ((uint16_t *)J->v_dst)[dst + d] = J->v_rows[src + d];
        } else {
          float kx = (float)oracle_bf16_to_f64(J->k_rows[src + d]);
          float vx = (float)oracle_bf16_to_f64(J->v_rows[src + d]);
          ((uint8_t *)J->k_dst)[dst + d] = oracle_e4m3_encode(kx, J->k_scale);
          ((uint8_t *)J->v_dst)[dst + d] = oracle_e4m3_encode(vx, J->v_scale);
        }
      }
    }
  }
  return NULL;
}

int oracle_store(void *k_dst, void *v_dst, int dtype, float k_scale, float v_scale,
                 const int32_t *page_table, int64_t page_stride, int n_kv_heads, int head_dim,
                 const uint16_t *k_rows, const uint16_t *v_rows, int64_t first_pos,
                 int64_t n_rows, int n_threads) {
  oracle_store_job jobs[256];
  pthread_t th[256];
  int started[256];
  int i;
  if (dtype != ORACLE_DTYPE_BF16 && dtype != ORACLE_DTYPE_E4M3) return -1;
  if (n_threads <= 0) n_threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if (n_rows < 4096) n_threads = 1;
  for (i = 0; i < n_threads; ++i) {
    oracle_store_job *J = &jobs[i];
    J->k_dst = k_dst;
    J->v_dst = v_dst;
    J->dtype = dtype;
    J->k_scale = k_scale;
    J->v_scale = v_scale;
    J->page_table = page_table;
    J->page_stride = page_stride;
    J->n_kv_heads = n_kv_heads;
    J->head_dim = head_dim;
    J->k_rows = k_rows;
    J->v_rows = v_rows;
    J->first_pos = first_pos;
    J->lo = n_rows * i / n_threads;
    J->hi = n_rows * (i + 1) / n_threads;
    started[i] = pthread_create(&th[i], NULL, oracle_store_rows, J) == 0;
    if (!started[i]) oracle_store_rows(J);
  }
  for (i = 0; i < n_threads; ++i)
    if (started[i]) pthread_join(th[i], NULL);
  return 0;
}

/* Gather positions 0..n_keys-1 into logical float64 arrays [Hkv][n_keys][D]. */
int oracle_gather(const void *k_src, const void *v_src, int dtype, double k_scale,
                  double v_scale, const int32_t *page_table, int64_t page_stride,
                  int n_kv_heads, int head_dim, int64_t n_keys, double *k_out, double *v_out) {
  for (int g = 0; g < n_kv_heads; ++g)
    for (int64_t t = 0; t < n_keys; ++t) {
      int64_t src = oracle_offset(page_table, page_stride, n_kv_heads, head_dim, t, g);
      int64_t dst = ((int64_t)g * n_keys + t) * head_dim;
      for (int d = 0; d < head_dim; ++d) {
        k_out[dst + d] = oracle_decode(k_src, dtype, src + d, k_scale);
        v_out[dst + d] = oracle_decode(v_src, dtype, src + d, v_scale);
      }
    }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention                                                                */
/* ------------------------------------------------------------------------ */

typedef struct {
  const double *k, *v;     /* logical [Hkv][n_keys][D] */
  int64_t n_keys;
  int n_kv_heads, n_q_heads, head_dim;
  const uint16_t *q;       /* [rows][Hq][D] bf16 bits */
  int64_t first_pos;
  const uint32_t *tree;    /* NULL: causal chain; else one ancestor word per row */
  const int32_t *rows;     /* selected row indices */
  int n_sel;
  double sm_scale;
  int64_t split_keys;      /* 0: direct softmax; else split form */
  int64_t n_split;
  double *out;             /* direct: [n_sel][Hq][D] */
  double *m_out, *l_out, *o_out; /* split: [n_sel][Hq][n_split] and [...][D] */
  int64_t next_task;
  pthread_mutex_t lock;
} oracle_job;

/* Whether row `row` (at position first_pos + row) attends key t.  Causal
 * rows see every key up to their own position.  With an ancestor table
 * (tree-shaped speculative verify), the keys before the stream's rows stay
 * visible and among the rows' own keys first_pos + j (j <= row) only those
 * whose bit j is set in the row's word are: a draft token attends the
 * tokens on its path from the root, itself included when bit row is set. */
static int oracle_visible(const oracle_job *J, int64_t row, int64_t t) {
  int64_t j;
  if (t > J->first_pos + row) return 0;
  if (!J->tree || t < J->first_pos) return 1;
  j = t - J->first_pos;
  return (int)((J->tree[row] >> j) & 1u);
}

/* One (row, q head): z_t = sm_scale * <q, k_t> for the visible keys t, then
 * either the softmax-weighted sum of v_t, or per split j the triple
 * (m_j = max z, l_j = sum exp(z - m_j), o_j = sum exp(z - m_j) v_t). */
static void oracle_one(oracle_job *J, int64_t task, double *z, double *qd) {
  int sel = (int)(task / J->n_q_heads);
  int h = (int)(task % J->n_q_heads);
  int D = J->head_dim;
  int G = J->n_q_heads / J->n_kv_heads;
  int g = h / G;
  int64_t row = J->rows[sel];
  int64_t pos = J->first_pos + row;
  int64_t nvis = pos + 1;
  const double *K = J->k + (int64_t)g * J->n_keys * D;
  const double *V = J->v + (int64_t)g * J->n_keys * D;
  const uint16_t *qrow = J->q + (row * J->n_q_heads + h) * (int64_t)D;

  for (int d = 0; d < D; ++d) qd[d] = oracle_bf16_to_f64(qrow[d]);
  for (int64_t t = 0; t < nvis; ++t) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) s += qd[d] * K[t * D + d];
    z[t] = J->sm_scale * s;
  }

  if (J->split_keys == 0) {
    double mx = -INFINITY, den = 0.0;
    double *o = J->out + ((int64_t)sel * J->n_q_heads + h) * D;
    for (int64_t t = 0; t < nvis; ++t)
      if (oracle_visible(J, row, t) && z[t] > mx) mx = z[t];
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t t = 0; t < nvis; ++t) {
      double e;
      if (!oracle_visible(J, row, t)) continue;
      e = exp(z[t] - mx);
      den += e;
      for (int d = 0; d < D; ++d) o[d] += e * V[t * D + d];
    }
    for (int d = 0; d < D; ++d) o[d] /= den;
    return;
  }

  for (int64_t j = 0; j < J->n_split; ++j) {
    int64_t lo = j * J->split_keys;
    int64_t hi = lo + J->split_keys;
    int64_t base = ((int64_t)sel * J->n_q_heads + h) * J->n_split + j;
    double *o = J->o_out + base * D;
    double mx = -INFINITY, den = 0.0;
    if (hi > nvis) hi = nvis;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t t = lo; t < hi; ++t)
      if (oracle_visible(J, row, t) && z[t] > mx) mx = z[t];
    for (int64_t t = lo; t < hi; ++t) {
      double e;
      if (!oracle_visible(J, row, t)) continue;
      e = exp(z[t] - mx);
      den += e;
      for (int d = 0; d < D; ++d) o[d] += e * V[t * D + d];
    }
    J->m_out[base] = mx; /* -inf when the split is wholly masked for this row */
    J->l_out[base] = den;
  }
}

static void *oracle_worker(void *arg) {
  oracle_job *J = (oracle_job *)arg;
  int64_t total = (int64_t)J->n_sel * J->n_q_heads;
  double *z = (double *)malloc(sizeof(double) * (size_t)(J->n_keys > 0 ? J->n_keys : 1));
  double *qd = (double *)malloc(sizeof(double) * (size_t)J->head_dim);
  if (!z || !qd) {
    free(z);
    free(qd);
    return (void *)1;
  }
  for (;;) {
    int64_t task;
    pthread_mutex_lock(&J->lock);
    task = J->next_task++;
    pthread_mutex_unlock(&J->lock);
    if (task >= total) break;
    oracle_one(J, task, z, qd);
  }
  free(z);
  free(qd);
  return NULL;
}

static int oracle_run(oracle_job *J, int n_threads) {
  pthread_t th[256];
  int i, started = 0, rc = 0;
  if (n_threads <= 0) n_threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  J->next_task = 0;
  pthread_mutex_init(&J->lock, NULL);
  for (i = 0; i < n_threads; ++i)
    if (pthread_create(&th[i], NULL, oracle_worker, J) == 0) ++started;
  if (started == 0) {
    void *r = oracle_worker(J);
    rc = r ? -1 : 0;
  }
  for (i = 0; i < started; ++i) {
    void *r = NULL;
    pthread_join(th[i], &r);
    if (r) rc = -1;
  }
  pthread_mutex_destroy(&J->lock);
  return rc;
}

static int oracle_prepare(oracle_job *J, const void *k_src, const void *v_src, int dtype,
                          double k_scale, double v_scale, const int32_t *page_table,
                          int64_t page_stride, int n_kv_heads, int head_dim,
                          int64_t n_keys_stored, const uint16_t *q, int n_q_heads,
                          int64_t first_pos, const uint32_t *tree, const int32_t *rows,
                          int n_sel, double sm_scale,
                          double **kbuf, double **vbuf) {
  int64_t max_row = -1, need;
  int i;
  if (n_kv_heads <= 0 || n_q_heads <= 0 || head_dim <= 0 || n_q_heads % n_kv_heads) return -1;
  if (dtype != ORACLE_DTYPE_BF16 && dtype != ORACLE_DTYPE_E4M3) return -1;
  for (i = 0; i < n_sel; ++i) {
    if (rows[i] < 0) return -1;
    if (rows[i] > max_row) max_row = rows[i];
  }
  if (tree && max_row >= 32) return -1; /* one 32-bit ancestor word per row */
  need = first_pos + max_row + 1;
  if (n_sel > 0 && need > n_keys_stored) return -2;
  if (need < 1) need = 1;
  *kbuf = (double *)malloc(sizeof(double) * (size_t)need * n_kv_heads * head_dim);
  *vbuf = (double *)malloc(sizeof(double) * (size_t)need * n_kv_heads * head_dim);
  if (!*kbuf || !*vbuf) return -3;
  if (n_sel > 0)
    oracle_gather(k_src, v_src, dtype, k_scale, v_scale, page_table, page_stride, n_kv_heads,
                  head_dim, need, *kbuf, *vbuf);
  memset(J, 0, sizeof *J);
  J->k = *kbuf;
  J->v = *vbuf;
  J->n_keys = need;
  J->n_kv_heads = n_kv_heads;
  J->n_q_heads = n_q_heads;
  J->head_dim = head_dim;
  J->q = q;
  J->first_pos = first_pos;
  J->tree = tree;
  J->rows = rows;
  J->n_sel = n_sel;
  J->sm_scale = sm_scale;
  return 0;
}

/* Direct softmax attention for the selected rows of one stream.
 * out: [n_sel][n_q_heads][head_dim] float64.  Returns 0, -1 bad argument,
 * -2 a row past the stored keys, -3 out of memory. */
int oracle_attention(const void *k_src, const void *v_src, int dtype, double k_scale,
                     double v_scale, const int32_t *page_table, int64_t page_stride,
                     int n_kv_heads, int head_dim, int64_t n_keys_stored, const uint16_t *q,
                     int n_q_heads, int64_t first_pos, const uint32_t *tree,
                     const int32_t *rows, int n_sel, double sm_scale, double *out,
                     int n_threads) {
  oracle_job J;
  double *kb = NULL, *vb = NULL;
  int rc = oracle_prepare(&J, k_src, v_src, dtype, k_scale, v_scale, page_table, page_stride,
                          n_kv_heads, head_dim, n_keys_stored, q, n_q_heads, first_pos, tree,
                          rows, n_sel, sm_scale, &kb, &vb);
  if (rc == 0) {
    J.out = out;
    rc = oracle_run(&J, n_threads);
  }
  free(kb);
  free(vb);
  return rc;
}

/* Split form over consecutive blocks of split_keys keys starting at key 0.
 * m_out, l_out: [n_sel][Hq][n_split]; o_out: [n_sel][Hq][n_split][D]. */
int oracle_attention_split(const void *k_src, const void *v_src, int dtype, double k_scale,
                           double v_scale, const int32_t *page_table, int64_t page_stride,
                           int n_kv_heads, int head_dim, int64_t n_keys_stored,
                           const uint16_t *q, int n_q_heads, int64_t first_pos,
                           const uint32_t *tree, const int32_t *rows, int n_sel,
                           double sm_scale, int64_t split_keys, int64_t n_split, double *m_out,
                           double *l_out, double *o_out, int n_threads) {
  oracle_job J;
  double *kb = NULL, *vb = NULL;
  int rc;
  if (split_keys <= 0 || n_split <= 0) return -1;
  rc = oracle_prepare(&J, k_src, v_src, dtype, k_scale, v_scale, page_table, page_stride,
                      n_kv_heads, head_dim, n_keys_stored, q, n_q_heads, first_pos, tree, rows,
                      n_sel, sm_scale, &kb, &vb);
  if (rc == 0) {
    int i;
    for (i = 0; i < n_sel; ++i)
      if ((first_pos + rows[i]) >= split_keys * n_split) rc = -1; /* not enough splits */
  }
  if (rc == 0) {
    J.split_keys = split_keys;
    J.n_split = n_split;
    J.m_out = m_out;
    J.l_out = l_out;
    J.o_out = o_out;
    rc = oracle_run(&J, n_threads);
  }
  free(kb);
  free(vb);
  return rc;
}

/* Merge split triples: M = max_j m_j, w_j = exp(m_j - M),
 * out = (sum_j w_j o_j) / (sum_j w_j l_j).  A wholly masked split has
 * m_j = -inf, l_j = 0, o_j = 0 and weight exactly 0. */
int oracle_merge(const double *m_in, const double *l_in, const double *o_in, int64_t n_items,
                 int64_t n_split, int head_dim, double *out) {
  for (int64_t it = 0; it < n_items; ++it) {
    const double *m = m_in + it * n_split;
    const double *l = l_in + it * n_split;
    const double *o = o_in + it * n_split * head_dim;
    double *dst = out + it * head_dim;
    double M = -INFINITY, den = 0.0;
    for (int64_t j = 0; j < n_split; ++j)
      if (m[j] > M) M = m[j];
    if (M == -INFINITY) return -1; /* no visible key: undefined */
    for (int d = 0; d < head_dim; ++d) dst[d] = 0.0;
    for (int64_t j = 0; j < n_split; ++j) {
      double w = (m[j] == -INFINITY) ? 0.0 : exp(m[j] - M);
      den += w * l[j];
      for (int d = 0; d < head_dim; ++d) dst[d] += w * o[j * head_dim + d];
    }
    for (int d = 0; d < head_dim; ++d) dst[d] /= den;
  }
  return 0;
}
