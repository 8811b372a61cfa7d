/*
 * Oracle for DSA sparse decode attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, fp64 CPU statement
 * of what the decode path computes.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it.  It shares no source, header,
 * table or helper with the HIP library, and the HIP library never calls it.
 *
 * Source pages (cited by page title and section):
 *   [P1] "vllm.models.step5.nvidia.ops.sparse_decode_attention": module
 *        docstring, `_gate`, `sparse_decode_attention`, `sparse_decode_splits`.
 *   [P2] "vllm.models.step5.nvidia.sparse_attention": `Step5DSAAttentionImpl`
 *        (`forward`, `_forward_decode`), `Step5SplitKVFlashAttentionImpl`.
 *   [P3] "vllm.models.step5.nvidia.flashinfer_sparse":
 *        `select_and_run_decode_attention`, `_direct_sparse_decode`.
 *
 * Readings taken where the pages are silent:
 *   - region r covers tokens [r*rt, r*rt + rt) with rt = region_tokens
 *     (0 means one region per page, rt = block);
 *   - the causal mask is inclusive: token t is visible iff t <= position;
 *   - any negative region id is unused; a region whose first token lies past
 *     the position contributes nothing and its block-table entry is not read;
 *   - duplicated region ids count once per slot (a multiset);
 *   - an active row with no visible token outputs zero (then gated: still 0);
 *   - inactive rows read nothing but `active`.
 *
 * Every function below that computes floating point does so in fp64, except
 * the gate, whose precision the `_gate` section of [P1] fixes to fp32.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SDO_DIM 192     /* query/key/value head dim, [P1] `sparse_decode_attention` */
#define SDO_ROW 384     /* one cache token row: K then V, [P1] docstring */

enum { SDO_KV_BF16 = 0, SDO_KV_FP8_E4M3 = 1 };
enum {
  SDO_OK = 0,
  SDO_ERR_ARGS = -1,     /* bad sizes / null pointers */
  SDO_ERR_TABLE = -2,    /* block-table column outside the table row */
  SDO_ERR_PAGE = -3,     /* page id outside [0, num_pages): missing slab */
  SDO_ERR_NOMEM = -4
};

/* Problem description.  Pointers are host pointers.  Strides are in elements
 * of the pointed-to type.  Mirrors the argument list of
 * [P1] `sparse_decode_attention` plus the strides Python tensors carry. */
typedef struct {
  int32_t rows, heads, groups, query_len, block, R, region_tokens;
  const uint16_t *query;            /* bf16 bits [rows, heads, 192] */
  int64_t q_row_stride, q_head_stride;
  const void *cache;                /* bf16 bits or e4m3 bytes [pages, G, block, 384] */
  int32_t kv_dtype;
  int64_t c_page_stride, c_group_stride, c_token_stride;
  int64_t num_pages;                /* pages present in `cache` */
  const int32_t *regions;           /* [rows, R], < 0 unused */
  int64_t regions_row_stride;
  const int32_t *block_table;       /* [requests, table_cols] */
  int64_t table_row_stride, table_cols;
  const int32_t *positions;         /* [rows] */
  const uint8_t *active;            /* [rows] */
  float scale;                      /* softmax scale, an fp32 kernel scalar */
  int32_t clear_inactive;
  float k_scale, v_scale;           /* per-tensor dequant scales (FP8 only) */
  const uint16_t *gate;             /* bf16 bits [tokens, G*heads] or NULL */
  int64_t gate_row_stride, gate_head_stride;
} sdo_problem;

/* ---- element decoders, written from the format definitions ---------------- */

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 mantissa bits. */
double sdo_bf16_to_double(uint16_t bits) {
  int sign = bits >> 15;
  int e = (bits >> 7) & 0xFF;
  int m = bits & 0x7F;
  double v;
  if (e == 0xFF) {
    v = m ? NAN : INFINITY;
  } else if (e == 0) {
    v = ldexp((double)m, -126 - 7);                 /* subnormal */
  } else {
    v = ldexp((double)(128 + m), e - 127 - 7);      /* 1.m * 2^(e-127) */
  }
  return sign ? -v : v;
}

/* OCP float8 e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
 * no infinities, S.1111.111 is NaN, exponent 0 is subnormal m * 2^-9. */
double sdo_e4m3_to_double(uint8_t bits) {
  int sign = bits >> 7;
  int e = (bits >> 3) & 0xF;
  int m = bits & 0x7;
  double v;
  if (e == 0xF && m == 0x7) {
    v = NAN;
  } else if (e == 0) {
    v = ldexp((double)m, -6 - 3);
  } else {
    v = ldexp((double)(8 + m), e - 7 - 3);
  }
  return sign ? -v : v;
}

/* Round an fp32 value to the nearest bfloat16, ties to even. */
uint16_t sdo_f32_to_bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* Headwise sigmoid gate, [P1] `_gate`: the bf16 logit is widened to fp32,
 * sigmoid = 1 / (1 + exp(-g)) with a correctly rounded fp32 division, and the
 * result is rounded to the gate's dtype (bf16) before it multiplies the
 * output.  exp is taken correctly rounded to fp32 (evaluated in fp64, then
 * rounded), the tightest reading of the fp32 exp the page calls. */
float sdo_gate_value(uint16_t gate_bits) {
  float g = (float)sdo_bf16_to_double(gate_bits);
  float e = (float)exp(-(double)g);          /* fp32 exp */
  float den = 1.0f + e;                       /* fp32 add */
  float sig = (float)(1.0 / (double)den);     /* correctly rounded fp32 div */
  uint16_t b = sdo_f32_to_bf16_bits(sig);
  return (float)sdo_bf16_to_double(b);
}

/* [P1] `sparse_decode_splits`, exactly as the page states it for B300:
 * grow a power-of-two split count while rows*splits*2 <= 256, up to 32. */
int sdo_splits_pages(int rows) {
  int splits = 1;
  while (splits < 32 && (int64_t)rows * splits * 2 <= 256) splits *= 2;
  return splits;
}

/* ---- row semantics ---------------------------------------------------------- */

static double load_cache(const sdo_problem *p, int64_t page, int g, int off, int e) {
  int64_t idx = page * p->c_page_stride + (int64_t)g * p->c_group_stride +
                (int64_t)off * p->c_token_stride + e;
  if (p->kv_dtype == SDO_KV_BF16) return sdo_bf16_to_double(((const uint16_t *)p->cache)[idx]);
  return sdo_e4m3_to_double(((const uint8_t *)p->cache)[idx]);
}

/* A visible token of a row: where its K|V row sits in the cache. */
typedef struct { int64_t page; int32_t off; } sdo_tok;

/* Collect the visible tokens of slots [j0, j1) of row r, in slot order.
 * [P1] docstring: row r is group r % G of token r // G; the rows of one
 * request are G*query_len consecutive rows sharing a block-table row.
 * Region id rho covers tokens rho*rt .. rho*rt+rt-1; token t lives at
 * page block_table[req, t / block], offset t % block. */
static int gather_tokens(const sdo_problem *p, int r, int j0, int j1, sdo_tok *toks, int *count) {
  int rt = p->region_tokens ? p->region_tokens : p->block;
  int req = r / (p->groups * p->query_len);
  int64_t pos = p->positions[r];
  const int32_t *reg = p->regions + (int64_t)r * p->regions_row_stride;
  int n = 0;
  for (int j = j0; j < j1; ++j) {
    int32_t rho = reg[j];
    if (rho < 0) continue;                       /* -1: unused slot */
    for (int i = 0; i < rt; ++i) {
      int64_t t = (int64_t)rho * rt + i;
      if (t > pos) break;                        /* causal, inclusive */
      int64_t col = t / p->block;
      if (col >= p->table_cols) return SDO_ERR_TABLE;
      int64_t page = p->block_table[(int64_t)req * p->table_row_stride + col];
      if (page < 0 || page >= p->num_pages) return SDO_ERR_PAGE;
      toks[n].page = page;
      toks[n].off = (int32_t)(t % p->block);
      ++n;
    }
  }
  *count = n;
  return SDO_OK;
}

static double kscale(const sdo_problem *p) { return p->kv_dtype == SDO_KV_BF16 ? 1.0 : (double)p->k_scale; }
static double vscale(const sdo_problem *p) { return p->kv_dtype == SDO_KV_BF16 ? 1.0 : (double)p->v_scale; }

/* Softmax attention of one head over a token list, in fp64.  Returns the
 * log-sum-exp of the logits (-inf for an empty list) and writes the
 * normalised output (zeros for an empty list) to o[192]. */
static double attend(const sdo_problem *p, int r, int h, const sdo_tok *toks, int n,
                     double *logit, double *o) {
  int g = r % p->groups;
  const uint16_t *q = p->query + (int64_t)r * p->q_row_stride + (int64_t)h * p->q_head_stride;
  double ks = kscale(p), vs = vscale(p), scale = (double)p->scale;
  for (int d = 0; d < SDO_DIM; ++d) o[d] = 0.0;
  if (n == 0) return -INFINITY;
  double m = -INFINITY;
  for (int t = 0; t < n; ++t) {
    double dot = 0.0;
    for (int d = 0; d < SDO_DIM; ++d)
      dot += sdo_bf16_to_double(q[d]) * (load_cache(p, toks[t].page, g, toks[t].off, d) * ks);
    logit[t] = scale * dot;
    if (logit[t] > m) m = logit[t];
  }
  double l = 0.0;
  for (int t = 0; t < n; ++t) {
    double w = exp(logit[t] - m);
    l += w;
    for (int d = 0; d < SDO_DIM; ++d)
      o[d] += w * (load_cache(p, toks[t].page, g, toks[t].off, SDO_DIM + d) * vs);
  }
  for (int d = 0; d < SDO_DIM; ++d) o[d] /= l;
  return m + log(l);
}

static void apply_gate(const sdo_problem *p, int r, int h, double *o) {
  if (!p->gate) return;
  int token = r / p->groups, g = r % p->groups;
  uint16_t x = p->gate[(int64_t)token * p->gate_row_stride +
                       (int64_t)(g * p->heads + h) * p->gate_head_stride];
  double s = (double)sdo_gate_value(x);
  for (int d = 0; d < SDO_DIM; ++d) o[d] *= s;
}

static int check(const sdo_problem *p, int row_begin, int row_end) {
  if (!p || p->heads < 1 || p->groups < 1 || p->query_len < 1 || p->block < 1 || p->R < 0)
    return SDO_ERR_ARGS;
  int rt = p->region_tokens ? p->region_tokens : p->block;
  if (rt < 1 || p->rows < 0 || row_begin < 0 || row_end > p->rows || row_begin > row_end)
    return SDO_ERR_ARGS;
  if (p->rows % (p->groups * p->query_len)) return SDO_ERR_ARGS;
  return SDO_OK;
}

/* The definition: for rows [row_begin, row_end), out (contiguous fp64
 * [row_end-row_begin, heads, 192], row row_begin first) receives the exact
 * softmax attention of each head over the multiset of selected, causally
 * visible tokens, gated if a gate is given.  Inactive rows are zeroed when
 * clear_inactive is set and left untouched otherwise.  No splitting. */
int sdo_decode(const sdo_problem *p, double *out, int row_begin, int row_end) {
  int rc = check(p, row_begin, row_end);
  if (rc) return rc;
  int rt = p->region_tokens ? p->region_tokens : p->block;
  int64_t cap = (int64_t)p->R * rt + 1;
  sdo_tok *toks = (sdo_tok *)malloc(sizeof(sdo_tok) * cap);
  double *logit = (double *)malloc(sizeof(double) * cap);
  if (!toks || !logit) { free(toks); free(logit); return SDO_ERR_NOMEM; }
  for (int r = row_begin; r < row_end; ++r) {
    double *orow = out + (int64_t)(r - row_begin) * p->heads * SDO_DIM;
    if (!p->active[r]) {
      if (p->clear_inactive) memset(orow, 0, sizeof(double) * p->heads * SDO_DIM);
      continue;
    }
    int n = 0;
    rc = gather_tokens(p, r, 0, p->R, toks, &n);
    if (rc) break;
    for (int h = 0; h < p->heads; ++h) {
      double *o = orow + (int64_t)h * SDO_DIM;
      attend(p, r, h, toks, n, logit, o);
      apply_gate(p, r, h, o);
    }
  }
  free(toks);
  free(logit);
  return rc;
}

/* The split-and-combine organisation the [P1] module docstring describes:
 * the row's live slots (id >= 0) are dealt to `splits` splits by balanced
 * live rank (split s takes ranks k with floor(k*splits/L) == s, "each split
 * still covers only the row's live regions"), each split produces a
 * normalised partial output and its log-sum-exp, and the combine merges the
 * partials with weights exp(lse_s - max lse), then gates.  An empty split
 * has lse = -inf.  Mathematically equal to `sdo_decode`; kept separate so
 * that the equality can be checked. */
int sdo_decode_split(const sdo_problem *p, int splits, double *out, int row_begin, int row_end) {
  int rc = check(p, row_begin, row_end);
  if (rc) return rc;
  if (splits < 1) return SDO_ERR_ARGS;
  int rt = p->region_tokens ? p->region_tokens : p->block;
  int64_t cap = (int64_t)p->R * rt + 1;
  sdo_tok *toks = (sdo_tok *)malloc(sizeof(sdo_tok) * cap);
  double *logit = (double *)malloc(sizeof(double) * cap);
  double *part = (double *)malloc(sizeof(double) * (size_t)splits * SDO_DIM);
  double *lse = (double *)malloc(sizeof(double) * (size_t)splits);
  int *live = (int *)malloc(sizeof(int) * (size_t)(p->R + 1));
  if (!toks || !logit || !part || !lse || !live) {
    free(toks); free(logit); free(part); free(lse); free(live);
    return SDO_ERR_NOMEM;
  }
  for (int r = row_begin; r < row_end && rc == SDO_OK; ++r) {
    double *orow = out + (int64_t)(r - row_begin) * p->heads * SDO_DIM;
    if (!p->active[r]) {
      if (p->clear_inactive) memset(orow, 0, sizeof(double) * p->heads * SDO_DIM);
      continue;
    }
    const int32_t *reg = p->regions + (int64_t)r * p->regions_row_stride;
    int L = 0;
    for (int j = 0; j < p->R; ++j)
      if (reg[j] >= 0) live[L++] = j;
    for (int h = 0; h < p->heads && rc == SDO_OK; ++h) {
      for (int s = 0; s < splits; ++s) {
        /* gather the tokens of the live slots whose rank falls in split s */
        int n = 0;
        for (int k = 0; k < L; ++k) {
          if ((int64_t)k * splits / L != s) continue;
          int c = 0;
          rc = gather_tokens(p, r, live[k], live[k] + 1, toks + n, &c);
          if (rc) break;
          n += c;
        }
        if (rc) break;
        lse[s] = attend(p, r, h, toks, n, logit, part + (int64_t)s * SDO_DIM);
      }
      if (rc) break;
      double M = -INFINITY;
      for (int s = 0; s < splits; ++s)
        if (lse[s] > M) M = lse[s];
      double *o = orow + (int64_t)h * SDO_DIM;
      for (int d = 0; d < SDO_DIM; ++d) o[d] = 0.0;
      if (M != -INFINITY) {
        double wsum = 0.0;
        for (int s = 0; s < splits; ++s) {
          double w = exp(lse[s] - M);
          wsum += w;
          for (int d = 0; d < SDO_DIM; ++d) o[d] += w * part[(int64_t)s * SDO_DIM + d];
        }
        for (int d = 0; d < SDO_DIM; ++d) o[d] /= wsum;
      }
      apply_gate(p, r, h, o);
    }
  }
  free(toks); free(logit); free(part); free(lse); free(live);
  return rc;
}

/* ---- gated sliding-window decode ------------------------------------------
 * [P2] `Step5SplitKVFlashAttentionImpl.forward_with_headwise_gate`: the
 * non-DSA layers attend, per decode token, over a causal sliding window of
 * `window` tokens (window = sliding_window[0] + 1, right edge 0), reading the
 * same packed [pages, G, block, 384] cache through K and V views
 * (`_split_kv_cache`), with the query heads of each KV group packed together
 * (GQA), and apply the headwise sigmoid gate to the result.  The batch is
 * uniform: requests * query_len tokens, query_len tokens per request.
 * Readings: token j (0-based) of a request whose sequence length is L sits at
 * position L - query_len + j, the convention [P3] `decode_logits` writes out
 * for query_len > 1; it sees tokens max(0, pos - window + 1) .. pos.  Rows
 * fold (token, KV group) as in the sparse path: row r is group r % G of
 * token r / G. */
typedef struct {
  int32_t tokens, heads, groups, query_len, block, window;
  const uint16_t *query;            /* bf16 bits, row view [tokens*G, heads, 192] */
  int64_t q_row_stride, q_head_stride;
  const uint16_t *cache;            /* bf16 bits [pages, G, block, 384] */
  int64_t c_page_stride, c_group_stride, c_token_stride;
  int64_t num_pages;
  const int32_t *block_table;       /* [requests, table_cols] */
  int64_t table_row_stride, table_cols;
  const int32_t *seq_lens;          /* [requests] */
  float scale;
  const uint16_t *gate;             /* bf16 bits [tokens, G*heads] or NULL */
  int64_t gate_row_stride, gate_head_stride;
} sdo_swa_problem;

/* Rows [row_begin, row_end) into out (contiguous fp64 [n, heads, 192]): the
 * exact softmax attention of each head over its window, gated if a gate is
 * given.  A row whose window holds no token (position < 0) outputs zero. */
int sdo_swa_decode(const sdo_swa_problem *s, double *out, int row_begin, int row_end) {
  if (!s || s->heads < 1 || s->groups < 1 || s->query_len < 1 || s->block < 1 || s->window < 1 ||
      s->tokens < 0 || s->tokens % s->query_len)
    return SDO_ERR_ARGS;
  int rows = s->tokens * s->groups;
  if (row_begin < 0 || row_end > rows || row_begin > row_end) return SDO_ERR_ARGS;
  /* the fields `attend` and `apply_gate` read */
  sdo_problem p;
  memset(&p, 0, sizeof(p));
  p.rows = rows;
  p.heads = s->heads;
  p.groups = s->groups;
  p.query_len = s->query_len;
  p.block = s->block;
  p.query = s->query;
  p.q_row_stride = s->q_row_stride;
  p.q_head_stride = s->q_head_stride;
  p.cache = s->cache;
  p.kv_dtype = SDO_KV_BF16;
  p.c_page_stride = s->c_page_stride;
  p.c_group_stride = s->c_group_stride;
  p.c_token_stride = s->c_token_stride;
  p.scale = s->scale;
  p.gate = s->gate;
  p.gate_row_stride = s->gate_row_stride;
  p.gate_head_stride = s->gate_head_stride;
  sdo_tok *toks = (sdo_tok *)malloc(sizeof(sdo_tok) * (size_t)s->window);
  double *logit = (double *)malloc(sizeof(double) * (size_t)s->window);
  if (!toks || !logit) { free(toks); free(logit); return SDO_ERR_NOMEM; }
  int rc = SDO_OK;
  for (int r = row_begin; r < row_end && rc == SDO_OK; ++r) {
    int token = r / s->groups;
    int req = token / s->query_len, j = token % s->query_len;
    int64_t pos = (int64_t)s->seq_lens[req] - s->query_len + j;
    int64_t first = pos - s->window + 1;
    if (first < 0) first = 0;
    int n = 0;
    for (int64_t t = first; t <= pos; ++t) {
      int64_t col = t / s->block;
      if (col >= s->table_cols) { rc = SDO_ERR_TABLE; break; }
      int64_t page = s->block_table[(int64_t)req * s->table_row_stride + col];
      if (page < 0 || page >= s->num_pages) { rc = SDO_ERR_PAGE; break; }
      toks[n].page = page;
      toks[n].off = (int32_t)(t % s->block);
      ++n;
    }
    if (rc) break;
    double *orow = out + (int64_t)(r - row_begin) * s->heads * SDO_DIM;
    for (int h = 0; h < s->heads; ++h) {
      double *o = orow + (int64_t)h * SDO_DIM;
      attend(&p, r, h, toks, n, logit, o);
      apply_gate(&p, r, h, o);
    }
  }
  free(toks);
  free(logit);
  return rc;
}

/* ---- region selection ------------------------------------------------------
 * [P3] `select_regions` as `select_and_run_decode_attention` and the prefill
 * loop call it (`sort=False`): per row, the `topk` regions to attend.  The
 * body is not on the pages.  Reading: the candidates of row r are regions
 * 0 .. n_r - 1 with n_r = topk_lengths[r] clamped to [0, S] (S = score
 * columns; all S without lengths); the current region is forced in when it is
 * a candidate; the other slots take the highest-scoring remaining
 * candidates, equal scores going to the lower region id (-0.0 ranks below
 * +0.0); the selected ids are written in ascending order, then -1 up to topk.
 * NaN scores are outside the contract. */
typedef struct { float s; int32_t j; } sdo_cand;

static int cand_order(const void *pa, const void *pb) {
  const sdo_cand *a = (const sdo_cand *)pa, *b = (const sdo_cand *)pb;
  if (a->s != b->s) return a->s > b->s ? -1 : 1;            /* higher score first */
  if (signbit(a->s) != signbit(b->s)) return signbit(a->s) ? 1 : -1;  /* +0 before -0 */
  return a->j < b->j ? -1 : (a->j > b->j ? 1 : 0);          /* lower id first */
}

static int id_order(const void *pa, const void *pb) {
  int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return a < b ? -1 : (a > b ? 1 : 0);
}

int sdo_select_regions(int32_t rows, int32_t S, int32_t topk, const float *scores,
                       int64_t scores_row_stride, const int32_t *current,
                       const int32_t *topk_lengths, int32_t *out, int64_t out_row_stride) {
  if (rows < 0 || S < 0 || topk < 0 || (rows > 0 && (!scores || !current || !out)))
    return SDO_ERR_ARGS;
  sdo_cand *cand = (sdo_cand *)malloc(sizeof(sdo_cand) * (size_t)(S + 1));
  int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(topk + 1));
  if (!cand || !sel) { free(cand); free(sel); return SDO_ERR_NOMEM; }
  for (int32_t r = 0; r < rows; ++r) {
    int64_t n = topk_lengths ? topk_lengths[r] : S;
    if (n < 0) n = 0;
    if (n > S) n = S;
    int32_t cur = current[r];
    int forced = cur >= 0 && cur < n && topk > 0;
    int m = 0;
    for (int32_t j = 0; j < n; ++j) {
      if (forced && j == cur) continue;
      cand[m].s = scores[(int64_t)r * scores_row_stride + j];
      cand[m].j = j;
      ++m;
    }
    qsort(cand, (size_t)m, sizeof(sdo_cand), cand_order);
    int take = topk - forced;
    if (take > m) take = m;
    int k = 0;
    if (forced) sel[k++] = cur;
    for (int i = 0; i < take; ++i) sel[k++] = cand[i].j;
    qsort(sel, (size_t)k, sizeof(int32_t), id_order);
    int32_t *o = out + (int64_t)r * out_row_stride;
    for (int i = 0; i < topk; ++i) o[i] = i < k ? sel[i] : -1;
  }
  free(cand);
  free(sel);
  return SDO_OK;
}

/* ---- decode indexer logits -------------------------------------------------
 * [P3] `decode_logits`: score every region of a row's request for the region
 * selection.  Queries are e4m3 [rows, heads, 256] (row r is group r % G of
 * token r / G, query_len tokens per request, as in the decode), weights fp32
 * [rows, heads].  The direct kernel (`decode_summary_scores`) and the paged
 * MQA-logits kernel under the fallback are not shown.  Reading: region j's
 * summary is 256 e4m3 bytes kept beside the KV in the page that holds the
 * region's tokens (page block_table[req, j / rpb], slot j % rpb, rpb =
 * regions per page), with an fp32 dequant scale s_j (the fallback's packed
 * 260-byte entry: 256 e4m3 bytes + a 4-byte scale), and
 *     score[r, j] = sum_h w[r,h] * max(0, s_j * sum_d q[r,h,d] * k_j[d])
 * for the regions 0 .. positions[r] / region_tokens of the row; the other
 * score columns are -inf.  PARITY UNPINNED: this formula is a reading; the
 * pins below fix the oracle to it, not to the pages. */
typedef struct {
  int32_t rows, heads, groups, query_len, rpb, num_regions, region_tokens;
  const uint8_t *query;             /* e4m3 [rows, heads, 256] */
  int64_t q_row_stride, q_head_stride;
  const float *weights;             /* [rows, heads] */
  int64_t w_row_stride;
  const uint8_t *summaries;         /* e4m3 [pages, rpb, 256] */
  int64_t s_page_stride, s_region_stride;
  const float *scales;              /* [pages, rpb] */
  int64_t sc_page_stride;
  int64_t num_pages;
  const int32_t *block_table;
  int64_t table_row_stride, table_cols;
  const int32_t *positions;         /* [rows] */
} sdo_logits_problem;

#define SDO_IDX_DIM 256

int sdo_indexer_logits(const sdo_logits_problem *p, double *out, int row_begin, int row_end) {
  if (!p || p->heads < 1 || p->groups < 1 || p->query_len < 1 || p->rpb < 1 ||
      p->num_regions < 0 || p->region_tokens < 1 || row_begin < 0 || row_end > p->rows ||
      row_begin > row_end || p->rows % (p->groups * p->query_len))
    return SDO_ERR_ARGS;
  for (int r = row_begin; r < row_end; ++r) {
    int req = r / (p->groups * p->query_len);
    double *o = out + (int64_t)(r - row_begin) * p->num_regions;
    int64_t pos = p->positions[r];
    int64_t len = pos < 0 ? 0 : pos / p->region_tokens + 1;
    if (len > p->num_regions) len = p->num_regions;
    for (int64_t j = 0; j < p->num_regions; ++j) {
      if (j >= len) { o[j] = -INFINITY; continue; }
      int64_t col = j / p->rpb;
      if (col >= p->table_cols) return SDO_ERR_TABLE;
      int64_t page = p->block_table[(int64_t)req * p->table_row_stride + col];
      if (page < 0 || page >= p->num_pages) return SDO_ERR_PAGE;
      int slot = (int)(j % p->rpb);
      const uint8_t *k = p->summaries + page * p->s_page_stride + (int64_t)slot * p->s_region_stride;
      double s = (double)p->scales[page * p->sc_page_stride + slot];
      double acc = 0.0;
      for (int h = 0; h < p->heads; ++h) {
        const uint8_t *q = p->query + (int64_t)r * p->q_row_stride + (int64_t)h * p->q_head_stride;
        double dot = 0.0;
        for (int d = 0; d < SDO_IDX_DIM; ++d)
          dot += sdo_e4m3_to_double(q[d]) * sdo_e4m3_to_double(k[d]);
        double x = s * dot;
        acc += (double)p->weights[(int64_t)r * p->w_row_stride + h] * (x > 0.0 ? x : 0.0);
      }
      o[j] = acc;
    }
  }
  return SDO_OK;
}
