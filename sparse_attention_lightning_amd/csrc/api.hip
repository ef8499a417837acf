// api.hip -- the C-ABI entry points declared in include/idx.h.
//
// Every entry point checks its arguments on the host before touching the HIP
// runtime, so a refused call enqueues nothing and needs no device.
#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "device.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

enum Need { kScore = 1, kTopk = 2 };

int check(const idx_params* p, int need) {
  if (!p) return fail(IDX_E_NULL, "params is NULL");
  if (p->k_format < IDX_K_BF16 || p->k_format > IDX_K_NVFP4)
    return fail(IDX_E_FORMAT, "unknown k_format %d", p->k_format);
  if (p->head_dim != 128 || p->block_size != 128)
    return fail(IDX_E_SHAPE, "head_dim and block_size must be 128 (got %d, %d)", p->head_dim,
                p->block_size);
  if (p->packed_queries < 1 || p->gqa < 1)
    return fail(IDX_E_SHAPE, "packed_queries and gqa must be >= 1 (got %d, %d)",
                p->packed_queries, p->gqa);
  if ((int64_t)p->packed_queries * p->gqa > IDX_MAX_REQ_ROWS)
    return fail(IDX_E_PACK, "packed_queries * gqa = %lld exceeds %d rows a request",
                (long long)p->packed_queries * p->gqa, IDX_MAX_REQ_ROWS);
  if ((int64_t)p->n_req * p->packed_queries * p->gqa > IDX_MAX_ROWS)
    return fail(IDX_E_PACK, "n_req * packed_queries * gqa = %lld exceeds %d rows a call",
                (long long)p->n_req * p->packed_queries * p->gqa, IDX_MAX_ROWS);
  if (p->n_req < 0 || p->n_slot_rows < 0 || p->n_pages < 0)
    return fail(IDX_E_SHAPE, "negative count (n_req %d, n_slot_rows %d, n_pages %lld)",
                p->n_req, p->n_slot_rows, (long long)p->n_pages);
  if (p->n_req > IDX_MAX_REQ)
    return fail(IDX_E_SHAPE, "n_req %d exceeds %d", p->n_req, IDX_MAX_REQ);
  if (p->max_blocks < 0 || p->max_blocks > IDX_MAX_BLOCKS)
    return fail(IDX_E_SHAPE, "max_blocks %d outside [0, %d]", p->max_blocks, IDX_MAX_BLOCKS);
  if (p->reserved != 0) return fail(IDX_E_SHAPE, "reserved field must be 0");
  if (p->score_mode != IDX_SCORE_MAX && p->score_mode != IDX_SCORE_LSE)
    return fail(IDX_E_MODE, "unknown score_mode %d", p->score_mode);
  if (p->score_mode == IDX_SCORE_LSE && !(p->sm_scale > 0.0f && p->sm_scale <= 3.402823466e38f))
    return fail(IDX_E_MODE, "lse needs a finite sm_scale > 0 (got %g)", (double)p->sm_scale);
  if (p->n_pages > (int64_t)1 << 40) return fail(IDX_E_SHAPE, "n_pages %lld too large", (long long)p->n_pages);
  if (p->topk < 1 || p->init_blocks < 0 || p->local_blocks < 0 ||
      (int64_t)p->topk < (int64_t)p->init_blocks + p->local_blocks)
    return fail(IDX_E_TOPK, "need topk >= 1, init/local >= 0, topk >= init + local (got %d, %d, %d)",
                p->topk, p->init_blocks, p->local_blocks);
  // a pointer is required only where its array has elements; an empty one is
  // never dereferenced (no K page is valid when n_pages is 0)
  const int64_t rows = (int64_t)p->n_req * p->packed_queries * p->gqa;
  if (p->n_req > 0 && (!p->req_slot || !p->row_len))
    return fail(IDX_E_NULL, "req_slot and row_len are required");
  if (rows * p->max_blocks > 0 && !p->block_scores) return fail(IDX_E_NULL, "block_scores is required");
  if (need & kScore) {
    if ((rows > 0 && !p->q) || (p->n_pages > 0 && !p->k) ||
        ((int64_t)p->n_slot_rows * p->max_blocks > 0 && !p->block_table))
      return fail(IDX_E_NULL, "q, k and block_table are required for scoring");
    if (p->k_format == IDX_K_NVFP4 && p->n_pages > 0 && !p->k_scale)
      return fail(IDX_E_NULL, "k_scale is required for NVFP4 keys");
    if (!aligned16(p->q) || !aligned16(p->k))
      return fail(IDX_E_ALIGN, "q and k must be 16-byte aligned");
    if (p->k_format == IDX_K_NVFP4 && (reinterpret_cast<uintptr_t>(p->k_scale) & 1u))
      return fail(IDX_E_ALIGN, "k_scale must be 2-byte aligned");
  }
  if (need & kTopk) {
    if (rows > 0 && (!p->topk_ids || !p->topk_scores))
      return fail(IDX_E_NULL, "topk_ids and topk_scores are required for selection");
  }
  return IDX_OK;
}

idx::StepArgs args_of(const idx_params* p) {
  idx::StepArgs a{};
  a.q = p->q;
  a.k = p->k;
  a.k_scale = p->k_scale;
  a.req_slot = p->req_slot;
  a.block_table = p->block_table;
  a.row_len = p->row_len;
  a.block_scores = p->block_scores;
  a.topk_ids = p->topk_ids;
  a.topk_scores = p->topk_scores;
  a.n_pages = p->n_pages;
  a.k_format = p->k_format;
  a.n_req = p->n_req;
  a.n_slot_rows = p->n_slot_rows;
  a.P = p->packed_queries;
  a.H = p->gqa;
  a.max_blocks = p->max_blocks;
  a.topk = p->topk;
  a.init_blocks = p->init_blocks;
  a.local_blocks = p->local_blocks;
  a.score_mode = p->score_mode;
  a.sm_scale = p->sm_scale;
  return a;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(IDX_E_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return IDX_OK;
}

// The runtime's last-error slot is per thread and sticky: an earlier failure
// of some other call would otherwise be reported as this call's launch error.
void clear_stale_error() { (void)hipGetLastError(); }

int check_attn(const idx_attn_params* p) {
  if (!p) return fail(IDX_E_NULL, "params is NULL");
  if (p->head_dim != 128 || p->block_size != 128)
    return fail(IDX_E_SHAPE, "head_dim and block_size must be 128 (got %d, %d)", p->head_dim, p->block_size);
  if (p->packed_queries < 1 || p->kv_heads < 1 || p->q_per_kv < 1)
    return fail(IDX_E_SHAPE, "packed_queries, kv_heads and q_per_kv must be >= 1 (got %d, %d, %d)",
                p->packed_queries, p->kv_heads, p->q_per_kv);
  if (p->packed_queries > IDX_ATTN_MAX_DRAFT)
    return fail(IDX_E_PACK, "packed_queries %d exceeds %d draft rows", p->packed_queries, IDX_ATTN_MAX_DRAFT);
  if ((int64_t)p->packed_queries * p->q_per_kv > IDX_ATTN_MAX_ROWS)
    return fail(IDX_E_PACK, "packed_queries * q_per_kv = %lld exceeds %d rows a (request, KV head)",
                (long long)p->packed_queries * p->q_per_kv, IDX_ATTN_MAX_ROWS);
  if (p->n_req < 0 || p->n_slot_rows < 0 || p->n_pages < 0)
    return fail(IDX_E_SHAPE, "negative count (n_req %d, n_slot_rows %d, n_pages %lld)", p->n_req, p->n_slot_rows,
                (long long)p->n_pages);
  if (p->n_req > IDX_MAX_REQ) return fail(IDX_E_SHAPE, "n_req %d exceeds %d", p->n_req, IDX_MAX_REQ);
  if (p->kv_heads > 1024) return fail(IDX_E_SHAPE, "kv_heads %d exceeds 1024", p->kv_heads);
  if (p->max_blocks < 0 || p->max_blocks > IDX_MAX_BLOCKS)
    return fail(IDX_E_SHAPE, "max_blocks %d outside [0, %d]", p->max_blocks, IDX_MAX_BLOCKS);
  if (p->n_pages > ((int64_t)1 << 40) / p->kv_heads)
    return fail(IDX_E_SHAPE, "n_pages %lld too large", (long long)p->n_pages);
  if (p->topk < 1 || (int64_t)p->packed_queries * p->topk > IDX_ATTN_MAX_IDS)
    return fail(IDX_E_TOPK, "need topk >= 1 and packed_queries * topk <= %d (got %d, %d)", IDX_ATTN_MAX_IDS,
                p->topk, p->packed_queries);
  if (!(p->sm_scale > 0.0f && p->sm_scale <= 3.402823466e38f))
    return fail(IDX_E_MODE, "sm_scale must be finite and > 0 (got %g)", (double)p->sm_scale);
  if (p->kv_format != IDX_K_BF16 && p->kv_format != IDX_K_FP8_E4M3)
    return fail(IDX_E_FORMAT, "kv_format must be IDX_K_BF16 or IDX_K_FP8_E4M3 (got %d)", p->kv_format);
  return IDX_OK;
}

int64_t attn_workspace_bytes(const idx_attn_params* p, int* splits) {
  const int64_t items = (int64_t)p->n_req * p->kv_heads;
  const int64_t max_union = std::min<int64_t>((int64_t)p->packed_queries * p->topk, p->max_blocks);
  const int s = idx::attn_splits(items, max_union);
  if (splits) *splits = s;
  const int64_t rows = 16 * (int64_t)idx::attn_tiles(p->packed_queries, p->q_per_kv);
  return s > 1 ? items * s * rows * 132 * (int64_t)sizeof(float) : 0;  // one split: no partials
}

}  // namespace

extern "C" {

int64_t idx_sparse_attn_workspace(const idx_attn_params* p) {
  const int rc = check_attn(p);
  if (rc) return rc;
  g_err[0] = '\0';
  return attn_workspace_bytes(p, nullptr);
}

int idx_sparse_attn(const idx_attn_params* p, void* stream) {
  const int rc = check_attn(p);
  if (rc) return rc;
  const int64_t rows = (int64_t)p->n_req * p->packed_queries;
  if (rows > 0 && (!p->q || !p->req_slot || !p->row_len || !p->topk_ids || !p->out || !p->lse))
    return fail(IDX_E_NULL, "q, req_slot, row_len, topk_ids, out and lse are required");
  if (p->n_pages > 0 && (!p->k || !p->v)) return fail(IDX_E_NULL, "k and v are required");
  if ((int64_t)p->n_slot_rows * p->max_blocks > 0 && !p->block_table)
    return fail(IDX_E_NULL, "block_table is required");
  if (!aligned16(p->q) || !aligned16(p->k) || !aligned16(p->v) || !aligned16(p->out) || !aligned16(p->workspace))
    return fail(IDX_E_ALIGN, "q, k, v, out and workspace must be 16-byte aligned");
  int splits = 1;
  const int64_t need = attn_workspace_bytes(p, &splits);
  if (need > 0 && (!p->workspace || p->workspace_bytes < need))
    return fail(IDX_E_SHAPE, "workspace of %lld bytes is below the %lld needed", (long long)p->workspace_bytes,
                (long long)need);
  clear_stale_error();
  if (rows == 0) {
    g_err[0] = '\0';
    return IDX_OK;
  }
  idx::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(p->q);
  a.k = static_cast<const uint8_t*>(p->k);
  a.v = static_cast<const uint8_t*>(p->v);
  a.req_slot = p->req_slot;
  a.block_table = p->block_table;
  a.row_len = p->row_len;
  a.topk_ids = p->topk_ids;
  a.out = static_cast<uint16_t*>(p->out);
  a.lse = p->lse;
  a.ws = static_cast<float*>(p->workspace);
  a.n_pages = p->n_pages;
  a.n_req = p->n_req;
  a.n_slot_rows = p->n_slot_rows;
  a.P = p->packed_queries;
  a.H = p->kv_heads;
  a.G = p->q_per_kv;
  a.max_blocks = p->max_blocks;
  a.topk = p->topk;
  a.splits = splits;
  a.kv_format = p->kv_format;
  a.c2 = p->sm_scale * 1.44269504088896341f;
  return launched(idx::launch_attn(a, (hipStream_t)stream), "sparse attention");
}


const char* idx_last_error(void) { return g_err; }

int idx_score_packed(const idx_params* p, void* stream) {
  const int rc = check(p, kScore);
  if (rc) return rc;
  clear_stale_error();
  return launched(idx::launch_score(args_of(p), (hipStream_t)stream), "score");
}

int idx_block_topk(const idx_params* p, void* stream) {
  const int rc = check(p, kTopk);
  if (rc) return rc;
  clear_stale_error();
  return launched(idx::launch_topk(args_of(p), (hipStream_t)stream), "top-k");
}

int idx_step(const idx_params* p, void* stream) {
  const int rc = check(p, kScore | kTopk);
  if (rc) return rc;
  clear_stale_error();
  const idx::StepArgs a = args_of(p);
  const int r1 = launched(idx::launch_score(a, (hipStream_t)stream), "score");
  if (r1) return r1;
  return launched(idx::launch_topk(a, (hipStream_t)stream), "top-k");
}

}  // extern "C"

namespace {

// The checks of idx_fp4_store for the new keys of an NVFP4 step.
int check_new_keys(const idx_params* p, const idx_fp4_new_keys* nk) {
  if (!nk) return fail(IDX_E_NULL, "keys is NULL");
  if (p->k_format != IDX_K_NVFP4)
    return fail(IDX_E_FORMAT, "the fused store is for NVFP4 keys (k_format %d)", p->k_format);
  if (nk->n_tokens < 0) return fail(IDX_E_SHAPE, "negative n_tokens %lld", (long long)nk->n_tokens);
  if (nk->staging_row_stride < 128 || (nk->staging_row_stride & 7))
    return fail(IDX_E_SHAPE, "staging_row_stride %lld must be >= 128 and a multiple of 8",
                (long long)nk->staging_row_stride);
  if (nk->n_tokens > ((int64_t)1 << 40)) return fail(IDX_E_SHAPE, "n_tokens too large");
  if (nk->n_tokens == 0) return IDX_OK;
  if (!nk->staging_bf16 || !nk->slot_mapping || (p->n_pages > 0 && (!p->k || !p->k_scale)))
    return fail(IDX_E_NULL, "staging, slot_mapping, k and k_scale are required");
  if (!aligned16(nk->staging_bf16) || !aligned16(p->k))
    return fail(IDX_E_ALIGN, "staging and k must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(p->k_scale) & 7u) != 0)
    return fail(IDX_E_ALIGN, "k_scale must be 8-byte aligned for the store");
  return IDX_OK;
}

// The store and the scoring of an NVFP4 step: one launch when the score
// kernel can take the keys, else a store launch first.
int score_with_keys(const idx_params* p, const idx_fp4_new_keys* nk, hipStream_t stream) {
  idx::StepArgs a = args_of(p);
  const int64_t n = nk->n_tokens;
  const bool fused = n > 0 && n <= IDX_FP4_FUSED_MAX_KEYS && (int64_t)p->packed_queries * p->gqa <= 16 &&
                     p->n_req > 0 && p->max_blocks > 0;
  if (fused) {
    a.st_staging = static_cast<const uint16_t*>(nk->staging_bf16);
    a.st_slots = nk->slot_mapping;
    a.st_n = n;
    a.st_stride = nk->staging_row_stride;
  } else if (n > 0) {
    const int r = launched(idx::launch_fp4_store(static_cast<const uint16_t*>(nk->staging_bf16), n,
                                                 nk->staging_row_stride, nk->slot_mapping,
                                                 static_cast<uint8_t*>(const_cast<void*>(p->k)),
                                                 const_cast<uint8_t*>(p->k_scale), p->n_pages * 128, stream),
                           "fp4 store");
    if (r) return r;
  }
  return launched(idx::launch_score(a, stream), "score");
}

}  // namespace

extern "C" {

int idx_score_packed_fp4(const idx_params* p, const idx_fp4_new_keys* keys, void* stream) {
  int rc = check(p, kScore);
  if (!rc) rc = check_new_keys(p, keys);
  if (rc) return rc;
  clear_stale_error();
  return score_with_keys(p, keys, (hipStream_t)stream);
}

int idx_step_fp4(const idx_params* p, const idx_fp4_new_keys* keys, void* stream) {
  int rc = check(p, kScore | kTopk);
  if (!rc) rc = check_new_keys(p, keys);
  if (rc) return rc;
  clear_stale_error();
  const int r1 = score_with_keys(p, keys, (hipStream_t)stream);
  if (r1) return r1;
  return launched(idx::launch_topk(args_of(p), (hipStream_t)stream), "top-k");
}

int idx_step_noalloc(const idx_params* p, void* stream) {
  if (p && p->block_scores)
    return fail(IDX_E_SHAPE, "idx_step_noalloc keeps the block scores itself: block_scores must be NULL");
  if (!p) return fail(IDX_E_NULL, "params is NULL");
  // the checks of idx_step, with the library's array standing in for block_scores
  idx_params q = *p;
  q.block_scores = reinterpret_cast<float*>(uintptr_t{16});  // non-NULL placeholder, never used
  const int rc = check(&q, kScore | kTopk);
  if (rc) return rc;
  const int64_t n = (int64_t)p->n_req * p->packed_queries * p->gqa * p->max_blocks;
  if (n > IDX_NOALLOC_MAX_SCORES)
    return fail(IDX_E_SHAPE, "n_req * packed_queries * gqa * max_blocks = %lld exceeds the %d block scores "
                "idx_step_noalloc holds", (long long)n, IDX_NOALLOC_MAX_SCORES);
  clear_stale_error();
  idx::StepArgs a = args_of(p);
  a.block_scores = nullptr;
  if (n > 0) {
    const hipError_t e = idx::noalloc_scores(&a.block_scores);
    if (e != hipSuccess)
      return fail(IDX_E_LAUNCH, "device address of the block-score array: %s", hipGetErrorString(e));
  }
  const int r1 = launched(idx::launch_score(a, (hipStream_t)stream), "score");
  if (r1) return r1;
  return launched(idx::launch_topk(a, (hipStream_t)stream), "top-k");
}

int idx_probe_read(const void* base, int64_t n_base_units, const int32_t* units, int64_t n_units,
                   int32_t unit_bytes, int32_t nt, uint32_t* sink, int32_t n_sink, void* stream) {
  if (unit_bytes < 1024 || unit_bytes > (1 << 20) || (unit_bytes & (unit_bytes - 1)))
    return fail(IDX_E_SHAPE, "unit_bytes %d must be a power of two in [1024, 1 << 20]", unit_bytes);
  if (n_units < 0 || n_base_units < 1 || n_sink < 1 || n_units > ((int64_t)1 << 40))
    return fail(IDX_E_SHAPE, "need n_units >= 0, n_base_units >= 1, n_sink >= 1");
  if (n_base_units > (INT64_MAX >> 21))
    return fail(IDX_E_SHAPE, "n_base_units %lld too large", (long long)n_base_units);
  if (!base || !sink)
    return fail(IDX_E_NULL, "base and sink are required");
  if (!aligned16(base)) return fail(IDX_E_ALIGN, "base must be 16-byte aligned");
  clear_stale_error();
  return launched(idx::launch_read_probe(base, n_base_units, units, n_units, unit_bytes, nt != 0, sink, n_sink,
                                         (hipStream_t)stream),
                  "read probe");
}

int idx_fp4_store(const void* staging_bf16, int64_t n_tokens, int64_t staging_row_stride,
                  const int64_t* slot_mapping, uint8_t* payload, uint8_t* scales, int64_t n_slots,
                  void* stream) {
  if (n_tokens < 0 || n_slots < 0)
    return fail(IDX_E_SHAPE, "negative count (n_tokens %lld, n_slots %lld)", (long long)n_tokens,
                (long long)n_slots);
  if (staging_row_stride < 128 || (staging_row_stride & 7))
    return fail(IDX_E_SHAPE, "staging_row_stride %lld must be >= 128 and a multiple of 8",
                (long long)staging_row_stride);
  if (n_tokens > ((int64_t)1 << 40) || n_slots > ((int64_t)1 << 40))
    return fail(IDX_E_SHAPE, "n_tokens / n_slots too large");
  if (n_tokens == 0) {
    g_err[0] = '\0';
    return IDX_OK;
  }
  if (!staging_bf16 || !slot_mapping || !payload || !scales)
    return fail(IDX_E_NULL, "staging, slot_mapping, payload and scales are required");
  if (!aligned16(staging_bf16) || !aligned16(payload))
    return fail(IDX_E_ALIGN, "staging and payload must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(scales) & 7u) != 0)
    return fail(IDX_E_ALIGN, "scales must be 8-byte aligned");
  clear_stale_error();
  return launched(idx::launch_fp4_store(static_cast<const uint16_t*>(staging_bf16), n_tokens,
                                        staging_row_stride, slot_mapping, payload, scales, n_slots,
                                        (hipStream_t)stream),
                  "fp4 store");
}

}  // extern "C"
