/*
 * oracle.c -- plain CPU oracle of the packed lightning-indexer step.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Slow and obvious on purpose: each
 * (row, head, block) is computed straight from the definition, with no tiling,
 * packing or reordering.  OpenMP only splits independent (request, block) and
 * (request, row) items across threads.
 *
 * ORACLE_MUTANT (default 0) compiles in one deliberate mistake; the test suite
 * builds each mutant separately and checks that its pins reject it.  The
 * product build never defines it.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif
#define MUTANT(n) (ORACLE_MUTANT == (n))

/* ------------------------------------------------------------------------ */
/* Number formats                                                           */
/* ------------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32. */
static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, no infinities; exponent 15 with mantissa 7 is NaN.  The pages store
 * fp8 index keys with a unit scale and widen them exactly to bf16 before the
 * dot ("dropping the fp8-to-bf16 cast" is one of the injected bugs of the
 * indexer-CP page, Accuracy Tests). */
double oracle_fp8_value(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double v;
  if (MUTANT(5)) return (double)code; /* the fp8 -> bf16 cast dropped */
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9); /* subnormal: m/8 * 2^(1-7) */
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -v : v;
}

/* FP4 E2M1 code: bit 3 sign, bits 2..1 exponent with bias 1, bit 0 mantissa;
 * exponent 0 is subnormal (m * 0.5).  Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6. */
double oracle_e2m1_value(uint8_t code) {
  int sign = (code >> 3) & 1;
  int e = (code >> 1) & 3;
  int m = code & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return sign ? -v : v;
}

/* Round t >= 0 to the nearest finite non-negative E4M3 value, ties to the
 * even code, values above the largest finite (448) clamped to it.  Non-negative
 * codes 0x00..0x7E are ordered by value, so walk them. */
uint8_t oracle_e4m3_encode(float t) {
  double x = (double)t;
  int lo = 0;
  if (!(x > 0.0)) return 0;
  if (x >= 448.0) return 0x7E;
  while (lo < 0x7E && oracle_fp8_value((uint8_t)(lo + 1)) <= x) lo++;
  {
    double vlo = oracle_fp8_value((uint8_t)lo);
    double vhi = oracle_fp8_value((uint8_t)(lo + 1));
    double mid = 0.5 * (vlo + vhi); /* exact in double */
    if (x == vlo) return (uint8_t)lo;
    if (MUTANT(11)) return (uint8_t)lo; /* scale rounded toward zero */
    if (x < mid) return (uint8_t)lo;
    if (x > mid) return (uint8_t)(lo + 1);
    return (uint8_t)((lo & 1) ? lo + 1 : lo);
  }
}

/* The e2m1 code of x / s: magnitude rounded to the nearest e2m1 value, ties
 * to the even code, saturating at 6; the sign bit of x is kept, so a negative
 * value that rounds to zero stores code 0x8.  The quotient is an IEEE binary32
 * division (correctly rounded), the precision the GPU store computes in. */
uint8_t oracle_e2m1_encode(float x, float s) {
  int sign = signbit(x) ? 1 : 0;
  int mag = 0;
  if (s > 0.0f) {
    float q = fabsf(x) / s;
    if (q >= 6.0f) {
      mag = 7;
    } else {
      double vlo, vhi, mid;
      while (mag < 7 && oracle_e2m1_value((uint8_t)(mag + 1)) <= (double)q) mag++;
      vlo = oracle_e2m1_value((uint8_t)mag);
      if ((double)q != vlo) {
        vhi = oracle_e2m1_value((uint8_t)(mag + 1));
        mid = 0.5 * (vlo + vhi);
        if ((double)q > mid)
          mag = mag + 1;
        else if ((double)q == mid && ((mag & 1) || MUTANT(10)))
          mag = mag + 1; /* tie: to the even code (mutant 10: away from 0) */
      }
    }
  }
  if (MUTANT(9) && mag == 0) sign = 0; /* sign of zero codes dropped */
  return (uint8_t)((sign << 3) | mag);
}

/* ------------------------------------------------------------------------ */
/* NVFP4 store (ATOM PR 2745, Summary: "Store" and the per-key layout)      */
/* ------------------------------------------------------------------------ */

int oracle_fp4_store(const void* staging_bf16, int64_t n_tokens,
                     int64_t staging_row_stride, const int64_t* slot_mapping,
                     uint8_t* payload, uint8_t* scales, int64_t n_slots) {
  const uint16_t* st = (const uint16_t*)staging_bf16;
  int64_t t;
  if (n_tokens < 0 || n_slots < 0 || staging_row_stride < 128) return -1;
  if (n_tokens == 0) return 0;
  if (!st || !slot_mapping || !payload || !scales) return -1;
#pragma omp parallel for schedule(static)
  for (t = 0; t < n_tokens; t++) {
    int64_t slot = slot_mapping[t];
    const uint16_t* row = st + t * staging_row_stride;
    uint8_t code[128];
    int g, j, d;
    if (slot < 0 || slot >= n_slots) continue;
    for (g = 0; g < 8; g++) {
      float amax = 0.0f, s;
      uint8_t sb;
      for (j = 0; j < 16; j++) {
        float a = fabsf((float)bf16_value(row[16 * g + j]));
        if (a > amax) amax = a;
      }
      sb = oracle_e4m3_encode(amax / 6.0f); /* binary32 division */
      s = (float)oracle_fp8_value(sb);
      scales[slot * 8 + g] = sb;
      for (j = 0; j < 16; j++)
        code[16 * g + j] = oracle_e2m1_encode((float)bf16_value(row[16 * g + j]), s);
    }
    for (d = 0; d < 128; d += 2) {
      uint8_t even = code[d], odd = code[d + 1];
      payload[slot * 64 + d / 2] =
          MUTANT(12) ? (uint8_t)((even << 4) | odd) : (uint8_t)(even | (odd << 4));
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Scoring: block max of raw q . k over each row's own visible tokens       */
/* ------------------------------------------------------------------------ */

static int check_params(const oracle_params* p) {
  if (!p) return -1;
  if (p->head_dim != 128 || p->block_size != 128) return -1;
  if (p->k_format < ORACLE_K_BF16 || p->k_format > ORACLE_K_NVFP4) return -1;
  if (p->n_req < 0 || p->packed_queries < 1 || p->gqa < 1 || p->max_blocks < 0 ||
      p->n_slot_rows < 0 || p->n_pages < 0 || (int64_t)p->packed_queries * p->gqa > 65536)
    return -1;
  if (p->topk < 1 || p->init_blocks < 0 || p->local_blocks < 0 ||
      p->topk < p->init_blocks + p->local_blocks)
    return -1;
  if (p->score_mode != ORACLE_SCORE_MAX && p->score_mode != ORACLE_SCORE_LSE) return -1;
  if (p->score_mode == ORACLE_SCORE_LSE && !(p->sm_scale > 0.0f && isfinite(p->sm_scale))) return -1;
  return 0;
}

/* A request is a graph pad when its slot is outside the request table
 * (indexer-CP page, Modifications item 1: no K read for such a slot). */
static int request_slot(const oracle_params* p, int r) {
  int slot = MUTANT(6) ? r : p->req_slot[r]; /* mutant 6: K by group index */
  return (slot < 0 || slot >= p->n_slot_rows) ? -1 : slot;
}

static int clamp_len(const oracle_params* p, int32_t len) {
  int64_t cap = (int64_t)p->max_blocks * 128;
  if (len < 0) return 0;
  return (int)((int64_t)len > cap ? cap : len);
}

/* Visible length of draft row j of request r.  Mutant 1 replaces it by the
 * group's longest row: the group's block count in place of the row's, one of
 * the bugs listed on the indexer-CP page (Accuracy Tests). */
static int row_visible_len(const oracle_params* p, int r, int j) {
  int P = p->packed_queries;
  int len = clamp_len(p, p->row_len[r * P + j]);
  if (MUTANT(1)) {
    int jj;
    for (jj = 0; jj < P; jj++) {
      int l2 = clamp_len(p, p->row_len[r * P + jj]);
      if (l2 > len) len = l2;
    }
  }
  return len;
}

/* Mutant 2 only: blocks the group reads when sized by its shortest row (the
 * other listed bug); the correct oracle has no group extent at all. */
static int shortest_row_blocks(const oracle_params* p, int r) {
  int P = p->packed_queries, jj, m = -1;
  for (jj = 0; jj < P; jj++) {
    int l2 = clamp_len(p, p->row_len[r * P + jj]);
    if (m < 0 || l2 < m) m = l2;
  }
  return (m + 127) / 128;
}

/* Dequantized K value d of the token at pool slot `token`. */
static double k_value(const oracle_params* p, int64_t token, int d) {
  if (p->k_format == ORACLE_K_BF16) {
    const uint16_t* k = (const uint16_t*)p->k;
    return bf16_value(k[token * 128 + d]);
  }
  if (p->k_format == ORACLE_K_FP8_E4M3) {
    const uint8_t* k = (const uint8_t*)p->k;
    return oracle_fp8_value(k[token * 128 + d]);
  }
  {
    const uint8_t* k = (const uint8_t*)p->k;
    uint8_t byte = k[token * 64 + d / 2];
    uint8_t code = (d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
    double scale = oracle_fp8_value(p->k_scale[token * 8 + d / 16]);
    return oracle_e2m1_value(code) * scale; /* unit outer scale */
  }
}

int oracle_score_packed(const oracle_params* p) {
  int P, H, R, MB, rows, failed = 0;
  int64_t item, n_items;
  if (check_params(p)) return -1;
  P = p->packed_queries;
  H = p->gqa;
  R = p->n_req;
  MB = p->max_blocks;
  rows = P * H;
  n_items = (int64_t)R * MB;
  if (n_items == 0) return 0;
  if (!p->q || !p->k || !p->req_slot || !p->block_table || !p->row_len ||
      !p->block_scores || (p->k_format == ORACLE_K_NVFP4 && !p->k_scale))
    return -1;

#pragma omp parallel for schedule(dynamic, 16)
  for (item = 0; item < n_items; item++) {
    int r = (int)(item / MB);
    int b = (int)(item % MB);
    int slot = request_slot(p, r);
    const uint16_t* q = (const uint16_t*)p->q;
    int i, t, d;
    double* best = (double*)malloc(sizeof(double) * (size_t)rows);
    int* end = (int*)malloc(sizeof(int) * (size_t)rows);
    int64_t page = -1;
    int page_ok = 0, any = 0;
    int lse = p->score_mode == ORACLE_SCORE_LSE;
    double* sv = lse ? (double*)malloc(sizeof(double) * 128 * (size_t)rows) : NULL; /* lse: each row's token scores */
    if (!best || !end || (lse && !sv)) {
#pragma omp atomic write
      failed = 1;
      free(sv);
      free(end);
      free(best);
      continue;
    }

    /* which tokens of block b each tile row sees */
    for (i = 0; i < rows; i++) {
      int len = row_visible_len(p, r, i / H);
      int nb = (len + 127) / 128;
      best[i] = -INFINITY;
      end[i] = 0;
      if (slot < 0 || b >= nb) continue;
      if (MUTANT(2) && b >= shortest_row_blocks(p, r)) continue;
      end[i] = MUTANT(8) ? 128 : (len - 128 * b < 128 ? len - 128 * b : 128);
      any = 1;
    }
    if (any) {
      page = p->block_table[(int64_t)slot * MB + b];
      page_ok = page >= 0 && page < p->n_pages;
    }
    if (any && page_ok) {
      for (t = 0; t < 128; t++) {
        double v[128];
        int64_t token = page * 128 + t;
        int need = 0;
        for (i = 0; i < rows; i++) need |= t < end[i];
        if (!need) continue;
        for (d = 0; d < 128; d++) v[d] = k_value(p, token, d);
        for (i = 0; i < rows; i++) {
          /* tile row i is draft row i / H, head i % H */
          int64_t qrow = MUTANT(4) ? (int64_t)r * rows + (i % P) * H + i / P
                                   : (int64_t)r * rows + i;
          double s = 0.0;
          if (t >= end[i]) continue;
          for (d = 0; d < 128; d++) s += bf16_value(q[qrow * 128 + d]) * v[d];
          if (s > best[i]) best[i] = s;
          if (sv) sv[i * 128 + t] = s;
        }
      }
    }
    for (i = 0; i < rows; i++) {
      float out = (float)best[i];
      if (sv && end[i] > 0 && page_ok) {
        /* lse over the visible tokens, written from their max m:
         * ln sum exp(c s_t) = c m + ln sum exp(c (s_t - m)) */
        double c = MUTANT(14) ? 1.0 : (double)p->sm_scale; /* mutant 14: scale dropped */
        double sum = 0.0;
        for (t = 0; t < end[i]; t++) sum += exp(c * (sv[i * 128 + t] - best[i]));
        out = (float)(c * best[i] + log(sum));
      }
      if (end[i] > 0 && !page_ok) /* visible block, page id out of range (mutant 15: -inf) */
        out = MUTANT(15) ? -INFINITY : NAN;
      p->block_scores[((int64_t)r * rows + i) * MB + b] = out;
    }
    free(sv);
    free(end);
    free(best);
  }
  return failed ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Forced top-k (indexer-CP page, Modifications item 1 and Accuracy Tests)  */
/* ------------------------------------------------------------------------ */

typedef struct {
  float s;
  int id;
} cand;

/* Order: higher score first, NaN after every number, ties to the lower id. */
static int cand_cmp(const void* a, const void* b) {
  const cand* x = (const cand*)a;
  const cand* y = (const cand*)b;
  int xn = isnan(x->s), yn = isnan(y->s);
  if (xn != yn) return xn ? 1 : -1;
  if (!xn && x->s != y->s) return x->s > y->s ? -1 : 1;
  if (MUTANT(7)) return x->id < y->id ? 1 : -1; /* ties to the higher id */
  return x->id < y->id ? -1 : 1;
}

int oracle_block_topk(const oracle_params* p) {
  int P, H, R, MB, K, rows, failed = 0;
  int64_t item, n_items;
  if (check_params(p)) return -1;
  P = p->packed_queries;
  H = p->gqa;
  R = p->n_req;
  MB = p->max_blocks;
  K = p->topk;
  rows = P * H;
  n_items = (int64_t)R * rows;
  if (n_items == 0) return 0;
  if (!p->req_slot || !p->row_len || !p->block_scores || !p->topk_ids || !p->topk_scores)
    return -1;

#pragma omp parallel for schedule(dynamic, 4)
  for (item = 0; item < n_items; item++) {
    int r = (int)(item / rows);
    int i = (int)(item % rows);
    int32_t* ids = p->topk_ids + item * K;
    float* sc = p->topk_scores + item * K;
    const float* bs = p->block_scores + item * MB;
    int len, nb, b, n = 0, nforced = 0, nc = 0;
    unsigned char* sel;
    cand* c;

    for (b = 0; b < K; b++) {
      ids[b] = -1;
      sc[b] = -INFINITY;
    }
    if (request_slot(p, r) < 0) continue; /* graph pad: sentinels only */
    len = row_visible_len(p, r, i / H);
    nb = (len + 127) / 128;
    if (nb == 0) continue;

    sel = (unsigned char*)calloc((size_t)nb, 1);
    c = (cand*)malloc(sizeof(cand) * (size_t)nb);
    if (!sel || !c) {
#pragma omp atomic write
      failed = 1;
      free(sel);
      free(c);
      continue;
    }
    if (nb <= K) {
      for (b = 0; b < nb; b++) sel[b] = 1;
    } else {
      /* forced: the first init blocks and the last local blocks of this row */
      if (!MUTANT(13))
        for (b = 0; b < p->init_blocks && b < nb; b++) sel[b] = 1;
      if (!MUTANT(3))
        for (b = nb - p->local_blocks; b < nb; b++)
          if (b >= 0) sel[b] = 1;
      for (b = 0; b < nb; b++) nforced += sel[b];
      for (b = 0; b < nb; b++)
        if (!sel[b]) {
          c[nc].s = bs[b];
          c[nc].id = b;
          nc++;
        }
      qsort(c, (size_t)nc, sizeof(cand), cand_cmp);
      for (b = 0; b < K - nforced && b < nc; b++) sel[c[b].id] = 1;
    }
    for (b = 0; b < nb; b++)
      if (sel[b]) {
        ids[n] = b;
        sc[n] = bs[b];
        n++;
      }
    free(sel);
    free(c);
  }
  return failed ? -1 : 0;
}

int oracle_step(const oracle_params* p) {
  int rc = oracle_score_packed(p);
  return rc ? rc : oracle_block_topk(p);
}

/* ------------------------------------------------------------------------ */
/* Sparse attention over the selected blocks (readings in oracle.h)         */
/* ------------------------------------------------------------------------ */

/* Element i of a main K or V pool in its format (fp8: the exact widening of
 * the e4m3 code; mutant 23 uses the raw byte, the cast dropped). */
static double kv_value(const oracle_attn_params* p, const void* pool, int64_t i) {
  if (p->kv_format == ORACLE_K_FP8_E4M3) {
    uint8_t c = ((const uint8_t*)pool)[i];
    return MUTANT(23) ? (double)c : oracle_fp8_value(c);
  }
  return bf16_value(((const uint16_t*)pool)[i]);
}

int oracle_sparse_attn(const oracle_attn_params* p) {
  int P, H, G, MB, K, failed = 0;
  int64_t item, n_items;
  if (!p || (p->kv_format != ORACLE_K_BF16 && p->kv_format != ORACLE_K_FP8_E4M3)) return -1;
  if (p->head_dim != 128 || p->block_size != 128 || p->n_req < 0 || p->packed_queries < 1 ||
      p->kv_heads < 1 || p->q_per_kv < 1 || p->max_blocks < 0 || p->topk < 0 || p->n_slot_rows < 0 ||
      p->n_pages < 0 || !(p->sm_scale > 0.0f && isfinite(p->sm_scale)))
    return -1;
  P = p->packed_queries;
  H = p->kv_heads;
  G = p->q_per_kv;
  MB = p->max_blocks;
  K = p->topk;
  n_items = (int64_t)p->n_req * P * H * G;
  if (n_items == 0) return 0;
  if (!p->q || !p->req_slot || !p->row_len || !p->out || !p->lse ||
      (K > 0 && !p->topk_ids) || (MB > 0 && p->n_slot_rows > 0 && !p->block_table) ||
      (p->n_pages > 0 && (!p->k || !p->v)))
    return -1;

#pragma omp parallel for schedule(dynamic, 4)
  for (item = 0; item < n_items; item++) {
    /* item = ((row * H + h) * G + g), row = r * P + j */
    int64_t row = item / ((int64_t)H * G);
    int h = (int)((item / G) % H);
    int g = (int)(item % G);
    int r = (int)(row / P);
    int hs = MUTANT(19) ? (h + 1) % H : h; /* mutant 19: another head's selection */
    const uint16_t* q = (const uint16_t*)p->q;
    int64_t qrow = MUTANT(22) ? (row * G + g) * H + h : item; /* mutant 22: heads in the wrong order */
    float* out = p->out + item * 128;
    float* oabs = p->out_abs ? p->out_abs + item * 128 : NULL;
    unsigned char* sel;
    double* sc;
    int64_t* tok; /* (page * H + h) * 128 + t of each visible token */
    int slot, len, nb, b, t, d, e, n = 0, bad = 0;
    double m = -INFINITY, l = 0.0, o[128], oa[128];

    for (d = 0; d < 128; d++) {
      out[d] = 0.0f;
      if (oabs) oabs[d] = 0.0f;
    }
    p->lse[item] = -INFINITY;
    slot = p->req_slot[r];
    if (slot < 0 || slot >= p->n_slot_rows) continue; /* graph pad */
    {
      int64_t cap = (int64_t)MB * 128;
      int32_t raw = p->row_len[row];
      len = raw < 0 ? 0 : (int)((int64_t)raw > cap ? cap : raw);
    }
    nb = (len + 127) / 128;
    if (nb == 0) continue;

    sel = (unsigned char*)calloc((size_t)nb, 1);
    sc = (double*)malloc(sizeof(double) * (size_t)nb * 128);
    tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)nb * 128);
    if (!sel || !sc || !tok) {
#pragma omp atomic write
      failed = 1;
      free(sel);
      free(sc);
      free(tok);
      continue;
    }
    /* the selected set (only blocks the row can see matter) */
    if (MUTANT(18)) {
      for (b = 0; b < nb; b++) sel[b] = 1; /* mutant 18: selection ignored */
    } else {
      const int32_t* ids = p->topk_ids + (row * H + hs) * K;
      for (e = 0; e < K; e++)
        if (ids[e] >= 0 && ids[e] < nb) sel[ids[e]] = 1;
    }
    /* scaled scores of the visible tokens of the selected blocks */
    for (b = 0; b < nb; b++) {
      int64_t page;
      if (!sel[b]) continue;
      page = p->block_table[(int64_t)slot * MB + b];
      if (page < 0 || page >= p->n_pages) {
        bad = 1; /* the row sees at least token 128 b of this block */
        continue;
      }
      for (t = 0; t < 128; t++) {
        double s = 0.0;
        int64_t kt = (page * H + h) * 128 + t;
        if (128 * b + t >= len && !MUTANT(17)) break; /* mutant 17: length mask dropped */
        for (d = 0; d < 128; d++) s += bf16_value(q[qrow * 128 + d]) * kv_value(p, p->k, kt * 128 + d);
        sc[n] = MUTANT(16) ? s : (double)p->sm_scale * s; /* mutant 16: scale dropped */
        tok[n] = kt;
        n++;
      }
    }
    if (bad) {
      for (d = 0; d < 128; d++) {
        out[d] = NAN;
        if (oabs) oabs[d] = NAN;
      }
      p->lse[item] = NAN;
    } else if (n > 0) {
      for (e = 0; e < n; e++)
        if (sc[e] > m) m = sc[e];
      for (d = 0; d < 128; d++) o[d] = oa[d] = 0.0;
      for (e = 0; e < n; e++) {
        double w = exp(sc[e] - m);
        int64_t page_h = tok[e] / 128; /* (page * H + h) */
        int tt = (int)(tok[e] % 128);
        l += w;
        for (d = 0; d < 128; d++) {
          /* V is [page][h][token / 32][dim][token % 32]; mutant 21 reads it as [token][dim] */
          double v = kv_value(p, p->v, MUTANT(21) ? tok[e] * 128 + d : ((page_h * 4 + tt / 32) * 128 + d) * 32 + tt % 32);
          o[d] += w * v;
          oa[d] += w * fabs(v);
        }
      }
      for (d = 0; d < 128; d++) {
        out[d] = (float)(MUTANT(20) ? o[d] : o[d] / l); /* mutant 20: not normalized */
        if (oabs) oabs[d] = (float)(oa[d] / l);
      }
      p->lse[item] = (float)(m + log(l));
    }
    free(sel);
    free(sc);
    free(tok);
  }
  return failed ? -1 : 0;
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int oracle_set_threads(int n) {
#ifdef _OPENMP
  const int before = omp_get_max_threads();
  if (n > 0) omp_set_num_threads(n);
  return before;
#else
  (void)n;
  return 1;
#endif
}
