/*
 * oracle.h -- plain CPU oracle of the packed lightning-indexer step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this library: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no header, helper, table or constant with
 * the GPU library; the two only agree on the argument layout, which is the
 * problem statement of the pages (queries, K planes, scale plane, slot/page
 * table, per-row lengths, packed_queries, local_blocks, topk).
 *
 * Sources it follows (the pages, by title and section):
 *  - "[AMD] MiniMax-M3 indexer CP: packed scoring for EAGLE verify rows"
 *    (sglang PR 42614), Modifications item 1 and Accuracy Tests: tile row i is
 *    (draft row i / gqa, head i % gqa); each row masks with its own length and
 *    gets its own forced init/local blocks; K is addressed through the request
 *    slot table; a slot past the request table (graph padding) reads no K;
 *    selection is exact.
 *  - sglang PR 45451 ("packed decode score kernel"), Modifications: each row
 *    keeps its own length mask and the block score is the max score; its
 *    Accuracy Tests check the selected-block scores both as the max and as
 *    the lse.  The pages give no formula for the lse; the reading taken is
 *    ln sum_t exp(sm_scale * q.k_t) over the row's visible tokens of the
 *    block, with the caller's softmax scale sm_scale > 0.
 *  - ROCm/ATOM PR 2745 (NVFP4 index cache), Summary and Validation: per key a
 *    64 B e2m1 payload (two codes a byte, even element in the low nibble) and
 *    8 B of E4M3 scales, one per 16 elements, unit outer scale; the store uses
 *    scale = e4m3(amax / 6) and codes rounded half-to-even, saturating at 6.
 *
 * All arithmetic is plain loops.  Token scores are accumulated in double; the
 * block max (or the lse, in double) is rounded once to float, and selection
 * compares those floats.
 */
#ifndef SAL_ORACLE_H
#define SAL_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORACLE_K_BF16 = 0,     /* K stored as bf16, 256 B per token             */
  ORACLE_K_FP8_E4M3 = 1, /* K stored as OCP e4m3fn, 128 B per token        */
  ORACLE_K_NVFP4 = 2     /* 64 B e2m1 payload + 8 B E4M3 scales per token  */
};

enum {
  ORACLE_SCORE_MAX = 0,  /* block score: max of q.k over the visible tokens      */
  ORACLE_SCORE_LSE = 1   /* block score: ln sum exp(sm_scale * q.k) over them    */
};

/* Same field order and meaning as the GPU library's parameter block. */
typedef struct oracle_params {
  int32_t k_format;
  int32_t n_req;          /* requests, graph pads included                      */
  int32_t n_slot_rows;    /* rows of block_table                                 */
  int32_t packed_queries; /* P: draft rows per request                          */
  int32_t gqa;            /* H: index heads                                      */
  int32_t head_dim;       /* D: 128                                              */
  int32_t block_size;     /* tokens per block and per page: 128                  */
  int32_t max_blocks;     /* columns of block_table and of block_scores          */
  int32_t topk;
  int32_t init_blocks;
  int32_t local_blocks;
  int32_t score_mode;     /* ORACLE_SCORE_MAX or ORACLE_SCORE_LSE                */
  float   sm_scale;       /* lse: the softmax scale, finite and > 0              */
  int32_t reserved;
  int64_t n_pages;        /* pages in the K pool                                 */
  const void*    q;        /* bf16 [n_req*P][H][D]                               */
  const void*    k;        /* [n_pages*block_size][bytes per token]              */
  const uint8_t* k_scale;  /* NVFP4: [n_pages*block_size][D/16]; else unused      */
  const int32_t* req_slot; /* [n_req]                                            */
  const int32_t* block_table; /* [n_slot_rows][max_blocks]                       */
  const int32_t* row_len;  /* [n_req*P]                                          */
  float*   block_scores;   /* [n_req*P][H][max_blocks]                           */
  int32_t* topk_ids;       /* [n_req*P][H][topk]                                 */
  float*   topk_scores;    /* [n_req*P][H][topk]                                 */
} oracle_params;

/* Every entry point returns 0, or -1 when it refuses its arguments or an
 * allocation fails (its outputs are then incomplete). */

/* Block max (or lse) of every (row, head, block); -inf past the row's own
 * block count, NaN for a visible block whose page id is outside [0, n_pages). */
int oracle_score_packed(const oracle_params* p);
/* Forced top-k over block_scores; ids ascending, padded with -1 / -inf. */
int oracle_block_topk(const oracle_params* p);
/* oracle_score_packed followed by oracle_block_topk. */
int oracle_step(const oracle_params* p);

/* NVFP4 store: quantize bf16 staging rows into payload/scale planes at
 * slot_mapping[t]; a negative slot or one >= n_slots is skipped. */
int oracle_fp4_store(const void* staging_bf16, int64_t n_tokens,
                     int64_t staging_row_stride, const int64_t* slot_mapping,
                     uint8_t* payload, uint8_t* scales, int64_t n_slots);

/*
 * Sparse attention over the selected blocks (the step after selection: the
 * sparse kernel whose tests the sglang PR 45451 Accuracy Tests run beside the
 * packed scorer, and the fused verify kernel timed in the ROCm/ATOM PR 2745
 * Validation).  The pages fix none of its shapes; the readings taken:
 *  - grouped-query attention with kv_heads = the indexer's gqa index heads
 *    (index head h selects the blocks of KV head h) and q_per_kv query heads
 *    per KV head, head dimension 128;
 *  - query head g of KV head h of draft row j attends over the tokens of the
 *    blocks in topk_ids[row][h][.] (ids outside [0, max_blocks) ignored, an id
 *    listed twice counts once) that the row sees: position 128 b + t < the
 *    row's length, the same causal length as the indexer;
 *  - K and V are paged like the index K (page = block = 128 tokens, the same
 *    request slots and block table), bf16 or OCP fp8 e4m3 with unit scale
 *    (the index cache's fp8 format), K as [n_pages][kv_heads][128
 *    tokens][128] and V as [n_pages][kv_heads][4][128 dims][32 tokens] (each
 *    32-token quarter of a page-head transposed);
 *  - out = sum_t softmax_t(sm_scale * q.k_t) v_t and lse = ln sum_t
 *    exp(sm_scale * q.k_t); a row that sees no selected token gets out = 0 and
 *    lse = -inf, as do graph pads; a row that sees a token of a block whose
 *    page id is outside [0, n_pages) gets NaN in both.
 * Everything in double, rounded once to float at the end.
 */
typedef struct oracle_attn_params {
  int32_t n_req;          /* requests, graph pads included                      */
  int32_t n_slot_rows;
  int32_t packed_queries; /* P: draft rows per request                          */
  int32_t kv_heads;       /* H: KV heads = index heads                          */
  int32_t q_per_kv;       /* G: query heads per KV head                         */
  int32_t head_dim;       /* 128                                                 */
  int32_t block_size;     /* 128                                                 */
  int32_t max_blocks;
  int32_t topk;           /* ids per (draft row, KV head)                       */
  float   sm_scale;
  int32_t kv_format;      /* ORACLE_K_BF16 or ORACLE_K_FP8_E4M3                  */
  int64_t n_pages;
  const void*    q;        /* bf16 [n_req*P][H][G][128]                          */
  const void*    k;        /* [n_pages][H][128 tokens][128] bf16 or fp8          */
  const void*    v;        /* [n_pages][H][4][128 dims][32 tokens] bf16 or fp8   */
  const int32_t* req_slot;    /* [n_req]                                         */
  const int32_t* block_table; /* [n_slot_rows][max_blocks]                       */
  const int32_t* row_len;     /* [n_req*P]                                       */
  const int32_t* topk_ids;    /* [n_req*P][H][topk]                              */
  float* out;              /* [n_req*P][H][G][128]                               */
  float* lse;              /* [n_req*P][H][G]                                    */
  float* out_abs;          /* optional, like out: sum_t softmax_t |v_t|, the
                              scale of out's rounding error                      */
} oracle_attn_params;

int oracle_sparse_attn(const oracle_attn_params* p);

/* OpenMP threads the oracle's parallel loops use. */
int oracle_threads(void);
/* Threads for the calling thread's later calls (n > 0); returns the count before. */
int oracle_set_threads(int n);

/* The oracle's own format steps, exported so the tests can pin them. */
double  oracle_fp8_value(uint8_t code);          /* OCP e4m3fn -> value          */
double  oracle_e2m1_value(uint8_t code);         /* 4-bit e2m1 code -> value     */
uint8_t oracle_e4m3_encode(float t);             /* t >= 0: RNE, satfinite 448    */
uint8_t oracle_e2m1_encode(float x, float s);    /* code of x / s, sign kept      */

#ifdef __cplusplus
}
#endif
#endif
