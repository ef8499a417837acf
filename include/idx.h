/*
 * idx.h -- C-ABI of the MI355X (gfx950) packed lightning-indexer step.
 *
 * The step scores, for every request, its packed query rows (draft row x
 * index head) against the request's paged index-K cache, reduces each
 * 128-token block to one score under each row's own length (the max, or the
 * log-sum-exp), and selects the top-k blocks per (row, head) with the init
 * and local-window blocks always selected.  Sources (by page title and
 * section):
 *
 *  [P1] sglang PR 45451, "packed decode score kernel", Modifications: a
 *       request's rows share one 16-row dot tile so each K tile loads once;
 *       each row keeps its own length mask; the packed form applies when
 *       packed_queries x gqa <= 16 (wider packs and the many query rows of
 *       a prefill chunk, which ATOM PR 2745's Summary scores with a prefill
 *       block scorer, are cut into several tiles here).
 *  [P2] sglang PR 42614, "[AMD] MiniMax-M3 indexer CP: packed scoring for
 *       EAGLE verify rows", Modifications item 1: tile row i is (draft row
 *       i / gqa, head i % gqa); K is read up to the group's longest row while
 *       masks and forced init/local blocks use each row's own length; a slot
 *       past the request table (graph padding) reads no K.  Accuracy Tests:
 *       selection is exact; K is addressed through a permuted, gapped slot
 *       table.  [P1] Accuracy Tests: the selected-block scores are tested
 *       both as the max and as the lse of the block.
 *  [P3] ROCm/ATOM PR 2745, "NVFP4 index cache", Summary: per key (D = 128)
 *       a 64 B e2m1 payload, two codes a byte with the even element in the
 *       low nibble, and 8 B of E4M3 scales, one per 16 elements, unit outer
 *       scale; the store quantizes with scale = e4m3(amax / 6) and codes
 *       rounded half-to-even, saturating at 6.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller.  The library
 *    allocates no memory and keeps no state between calls, except a
 *    thread-local copy of the last error message and, per device, how many
 *    workgroups of each kernel fit at once (queried on first use).  Calls
 *    from several host threads are safe; calls on one stream run in order.
 *  - `stream` is a hipStream_t (NULL = the null stream).  A call checks its
 *    arguments on the host, enqueues its kernels on `stream` and returns
 *    without synchronising.  0 = enqueued; a negative IDX_E_* code other than
 *    IDX_E_LAUNCH = refused on the host, nothing enqueued.  IDX_E_LAUNCH = the
 *    runtime rejected a launch; for a call that makes several launches
 *    (idx_step) the launches before the rejected one stay enqueued.
 *  - A call makes no allocation, memset, copy or synchronisation, and its
 *    launch shapes depend only on the host-side sizes, so it may be captured
 *    into a HIP graph; a replay reads whatever the captured buffers then hold
 *    (new queries, lengths, slots, page ids: the fixed-shape loop that graph
 *    pads exist for [P2]).
 *  - A pointer whose array has no elements (n_req = 0, max_blocks = 0,
 *    n_pages = 0, n_slot_rows = 0 ...) may be NULL: it is never dereferenced.
 *    A call over zero rows, or over rows with no blocks, is accepted and
 *    writes what its outputs hold (sentinels where a row has no block).
 *  - Sizes that live in device memory (row lengths, page ids, slots) cannot be
 *    checked on the host; the kernels clamp or reject them as stated below and
 *    never access memory outside the extents passed in.
 *  - Calls on one stream run in order; the library adds no synchronisation
 *    between streams.
 */
#ifndef SAL_IDX_H
#define SAL_IDX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  IDX_OK = 0,
  IDX_E_NULL = -1,   /* a required pointer is NULL                                  */
  IDX_E_FORMAT = -2, /* unknown k_format                                            */
  IDX_E_SHAPE = -3,  /* head_dim / block_size != 128, or a count out of range        */
  IDX_E_PACK = -4,   /* packed_queries * gqa > IDX_MAX_REQ_ROWS, or n_req * packed_queries * gqa > IDX_MAX_ROWS */
  IDX_E_TOPK = -5,   /* topk < 1, init/local < 0, or topk < init_blocks + local_blocks */
  IDX_E_LAUNCH = -6, /* the HIP runtime rejected a kernel launch                      */
  IDX_E_ALIGN = -7,  /* a pointer below its required alignment (see each call)       */
  IDX_E_MODE = -8    /* unknown score_mode, or an lse sm_scale that is not finite > 0 */
};

enum {
  IDX_SCORE_MAX = 0, /* block score: max over the block's visible tokens of q.k        */
  IDX_SCORE_LSE = 1  /* block score: ln sum over those tokens of exp(sm_scale * q.k)    */
};

enum {
  IDX_K_BF16 = 0,     /* K row: 128 bf16 (256 B)                                        */
  IDX_K_FP8_E4M3 = 1, /* K row: 128 OCP e4m3fn bytes (128 B), unit scale               */
  IDX_K_NVFP4 = 2     /* K row: 64 B e2m1 payload; scale row: 8 E4M3 bytes [P3]         */
};

/* Largest max_blocks: 1,048,576-token contexts, the context length the
 * pages serve with (sglang PR 45451, Reproduce: --context-length). */
#define IDX_MAX_BLOCKS 8192
/* Largest n_req (graph pads included) one call accepts. */
#define IDX_MAX_REQ 8192
/* Largest packed_queries * gqa (rows of one request).  Up to 16 rows a
 * request's rows form one tile that reads each K page once [P1]; above that
 * (wide packs, the query rows of a prefill chunk) they are scored in tiles
 * of 16 rows, 64 rows sharing each K page. */
#define IDX_MAX_REQ_ROWS 65536
/* Largest n_req * packed_queries * gqa (rows of one call). */
#define IDX_MAX_ROWS (1 << 24)

/*
 * Parameters of one indexer step (one layer, all requests of the batch).
 *
 * Shapes, with P = packed_queries, H = gqa, R = n_req (graph pads included),
 * MB = max_blocks, D = head_dim = 128, B = block_size = 128:
 *   q            bf16  [R*P][H][D]   row-major; tile row i of request r is
 *                                    q[(r*P + i/H)*H + i%H], i.e. the R*P*H
 *                                    rows in order [P2].
 *   k            bf16 or fp8: [n_pages*B][D] elements; NVFP4: [n_pages*B][64]
 *                bytes.  Token t of page p is row p*B + t.  Page = block.
 *   k_scale      NVFP4 only: uint8 [n_pages*B][D/16] E4M3 scales; else ignored.
 *   req_slot     int32 [R]: the request's row in block_table.  A slot < 0 or
 *                >= n_slot_rows marks a graph pad: no K is read and its
 *                outputs are sentinels [P2].
 *   block_table  int32 [n_slot_rows][MB]: page id of each 128-token block.
 *                A page id outside [0, n_pages) is not read; every row that
 *                sees that block gets a NaN block score.
 *   row_len      int32 [R*P]: tokens visible to each draft row.  Negative
 *                values count as 0, values above MB*B as MB*B.
 *   block_scores fp32 [R*P][H][MB]: for block b of a row with nb =
 *                ceil(row_len/B) blocks, a reduction over that block's
 *                visible tokens of the raw dot q.k (fp32 accumulation):
 *                IDX_SCORE_MAX: the max; IDX_SCORE_LSE: the natural log of
 *                the sum of exp(sm_scale * q.k), in fp32 from the block's max
 *                (the [P1] Accuracy Tests name both reductions).  -inf for
 *                b >= nb and for graph pads.
 *   topk_ids     int32 [R*P][H][topk]: selected block ids, ascending, padded
 *                with -1.  If nb <= topk every block is selected; otherwise
 *                blocks [0, init_blocks) and [nb - local_blocks, nb) are
 *                always selected and the rest go by score, higher first, ties
 *                to the lower id, NaN below every number.
 *   topk_scores  fp32 [R*P][H][topk]: block_scores of each selected id, -inf
 *                padding.
 */
typedef struct idx_params {
  int32_t k_format;       /* IDX_K_*                                        */
  int32_t n_req;          /* requests in the launch, graph pads included, <= IDX_MAX_REQ */
  int32_t n_slot_rows;    /* rows of block_table (the request table)         */
  int32_t packed_queries; /* draft rows per request, >= 1                    */
  int32_t gqa;            /* index heads, >= 1; packed_queries*gqa <= IDX_MAX_REQ_ROWS */
  int32_t head_dim;       /* must be 128                                     */
  int32_t block_size;     /* must be 128                                     */
  int32_t max_blocks;     /* columns of block_table / block_scores, 0..IDX_MAX_BLOCKS */
  int32_t topk;           /* >= 1                                            */
  int32_t init_blocks;    /* forced leading blocks, >= 0                     */
  int32_t local_blocks;   /* forced trailing blocks, >= 0                    */
  int32_t score_mode;     /* IDX_SCORE_MAX or IDX_SCORE_LSE                  */
  float sm_scale;         /* IDX_SCORE_LSE: finite, > 0; ignored for MAX     */
  int32_t reserved;       /* must be 0                                       */
  int64_t n_pages;        /* pages in the K pool, >= 0                       */
  const void* q;
  const void* k;
  const uint8_t* k_scale;
  const int32_t* req_slot;
  const int32_t* block_table;
  const int32_t* row_len;
  float* block_scores;
  int32_t* topk_ids;
  float* topk_scores;
} idx_params;

/*
 * NVFP4 store [P3]: quantize bf16 staging keys into the paged payload and
 * scale planes.  For token t < n_tokens, row t of `staging_bf16` (128 bf16,
 * rows `staging_row_stride` elements apart, stride >= 128) goes to slot
 * s = slot_mapping[t] (slot = page*128 + offset): payload[s][0..63] and
 * scales[s][0..7].  Per 16-element group: scale byte = E4M3 nearest to
 * amax/6 (fp32 quotient, ties to even, clamped at 448); code = e2m1 nearest
 * to x/scale, ties to the even code, saturating at 6, with x's sign bit
 * (scale 0 gives magnitude 0).  A slot < 0 or >= n_slots is skipped; other
 * slots are left untouched.  NaN/Inf inputs give unspecified bytes.
 * Pointers: staging_bf16 and payload 16-byte aligned, scales 8-byte aligned
 * (a key's eight scale bytes are written as one 8-byte store).
 */
int idx_fp4_store(const void* staging_bf16, int64_t n_tokens, int64_t staging_row_stride,
                  const int64_t* slot_mapping, uint8_t* payload, uint8_t* scales,
                  int64_t n_slots, void* stream);

/* Block scores of every (row, head, block) [P1, P2]: reads q, k, k_scale,
 * req_slot, block_table, row_len; writes block_scores (all R*P*H*MB entries).
 * topk_ids / topk_scores may be NULL. */
int idx_score_packed(const idx_params* p, void* stream);

/* Forced top-k [P2] over an existing block_scores: reads req_slot, row_len,
 * block_scores; writes topk_ids and topk_scores.  q, k, k_scale and
 * block_table may be NULL. */
int idx_block_topk(const idx_params* p, void* stream);

/* idx_score_packed then idx_block_topk on the same stream. */
int idx_step(const idx_params* p, void* stream);

/* The step's new NVFP4 keys [P3] (Summary: the store writes each new key into
 * the index cache before the decode scorer reads it): bf16 staging rows and
 * their slots, as the arguments of idx_fp4_store. */
typedef struct idx_fp4_new_keys {
  const void* staging_bf16;    /* [n_tokens][staging_row_stride] bf16, 16-byte aligned */
  int64_t n_tokens;            /* >= 0                                                 */
  int64_t staging_row_stride;  /* >= 128, a multiple of 8                              */
  const int64_t* slot_mapping; /* [n_tokens]: slot = page * 128 + offset               */
} idx_fp4_new_keys;

/* Keys the score launch stores itself; more take a store launch of their own. */
#define IDX_FP4_FUSED_MAX_KEYS 1024

/*
 * idx_fp4_store of `keys` into p->k (payload) and p->k_scale (scales), with
 * n_slots = p->n_pages * 128, followed by idx_score_packed(p), on `stream`:
 * the pool bytes and the block scores are exactly those two calls'.  For
 * NVFP4 keys (p->k_format == IDX_K_NVFP4) only.  When keys->n_tokens <=
 * IDX_FP4_FUSED_MAX_KEYS and the requests hold at most 16 rows each
 * (packed_queries * gqa <= 16), the score launch writes the keys itself (one
 * launch in all: every key is written by one workgroup early in the launch
 * and again, with the same bytes, by every workgroup whose pages hold it
 * before that workgroup reads them); otherwise a store launch precedes the
 * score launch.  p->k and p->k_scale are written, so they must be writable
 * device memory; k_scale 8-byte aligned.  Two keys with one slot leave
 * either key's bytes there, as for idx_fp4_store.  Refusals: those of both
 * calls, IDX_E_FORMAT for another k_format, IDX_E_NULL for a NULL `keys`.
 */
int idx_score_packed_fp4(const idx_params* p, const idx_fp4_new_keys* keys, void* stream);

/* idx_score_packed_fp4 then idx_block_topk on the same stream. */
int idx_step_fp4(const idx_params* p, const idx_fp4_new_keys* keys, void* stream);

/* Message describing the last refusal on the calling thread ("" if none). */
const char* idx_last_error(void);

/*
 * Sparse attention over the selected blocks: the step after selection.  The
 * pages name it ([P1] Accuracy Tests run the sparse kernel's tests beside the
 * packed scorer; [P3] Validation times the fused verify kernel on MI355X) but
 * fix none of its shapes; the readings taken:
 *  - grouped-query attention: kv_heads = the indexer's gqa index heads, index
 *    head h choosing the blocks of KV head h; q_per_kv query heads per KV
 *    head; head dimension 128;
 *  - query head g of KV head h of draft row j attends over the tokens of the
 *    blocks listed in topk_ids[row j][h][.] (the output of idx_block_topk, or
 *    any int32 list: ids < 0, ids past the row's blocks and repeats are
 *    ignored) that the row sees: position 128 b + t < row_len[row j];
 *  - K and V are paged like the index K (page = block = 128 tokens, the same
 *    req_slot and block_table), both bf16 or both OCP fp8 e4m3fn with unit
 *    scale (kv_format; the index cache's fp8 format), fp8 widened exactly to
 *    bf16 for the products;
 *  - out = sum_t softmax_t(sm_scale q.k_t) v_t (fp32 accumulation, stored as
 *    bf16), lse = ln sum_t exp(sm_scale q.k_t) (fp32).  A row that sees no
 *    selected token (length 0, nothing selected, graph pad) gets out = 0 and
 *    lse = -inf; a row that sees a token of a selected block whose page id is
 *    outside [0, n_pages) gets NaN in both.
 *
 * Shapes, with P = packed_queries, H = kv_heads, G = q_per_kv, R = n_req:
 *   q        bf16 [R*P][H][G][128]
 *   k        [n_pages][H][128 tokens][128] of kv_format: token t of page p,
 *            head h is k[p][h][t]
 *   v        [n_pages][H][4][128 dims][32 tokens] of kv_format: each 32-token
 *            quarter of a page-head's V transposed, token t, dimension d at
 *            v[p][h][t / 32][d][t % 32] (8 consecutive tokens of a dimension
 *            are one load for the PV product, and the 16 dimensions a load
 *            instruction covers are whole lines in a row)
 *   req_slot, block_table, row_len: as idx_params
 *   topk_ids int32 [R*P][H][topk]
 *   out      bf16 [R*P][H][G][128];  lse fp32 [R*P][H][G]
 *   workspace  at least idx_sparse_attn_workspace(p) bytes, 16-byte aligned,
 *            caller-owned; its contents are scratch (partial results of the
 *            splits of each (request, KV head)), needing no initialisation.
 *            When the batch fills the device without splitting, the size is 0
 *            and the workspace may be NULL.
 * Limits: P <= IDX_ATTN_MAX_DRAFT and P * G <= IDX_ATTN_MAX_ROWS (the rows
 * of one request and KV head are up to four 16-row MFMA tiles that read each
 * selected K/V page once for all of them), P * topk <= IDX_ATTN_MAX_IDS.
 * q, k, v, out 16-byte aligned.
 */
#define IDX_ATTN_MAX_ROWS 64
#define IDX_ATTN_MAX_DRAFT 16
#define IDX_ATTN_MAX_IDS 1024
#define IDX_ATTN_MAX_SPLITS 64

typedef struct idx_attn_params {
  int32_t n_req;          /* requests, graph pads included, <= IDX_MAX_REQ  */
  int32_t n_slot_rows;    /* rows of block_table                             */
  int32_t packed_queries; /* draft rows per request, >= 1                    */
  int32_t kv_heads;       /* >= 1 (the indexer's gqa)                        */
  int32_t q_per_kv;       /* query heads per KV head, >= 1                   */
  int32_t head_dim;       /* must be 128                                     */
  int32_t block_size;     /* must be 128                                     */
  int32_t max_blocks;     /* columns of block_table, 0..IDX_MAX_BLOCKS       */
  int32_t topk;           /* ids per (draft row, KV head), >= 1              */
  float sm_scale;         /* softmax scale, finite and > 0                   */
  int32_t kv_format;      /* IDX_K_BF16 or IDX_K_FP8_E4M3, K and V alike     */
  int64_t n_pages;        /* pages in the K and V pools, >= 0                */
  int64_t workspace_bytes;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* req_slot;
  const int32_t* block_table;
  const int32_t* row_len;
  const int32_t* topk_ids;
  void* out;
  float* lse;
  void* workspace;
} idx_attn_params;

/* Bytes of workspace idx_sparse_attn needs for these sizes on the current
 * device, or a negative IDX_E_* code when the sizes are refused. */
int64_t idx_sparse_attn_workspace(const idx_attn_params* p);

/* Sparse attention over the selected blocks (on `stream`: the splits'
 * partials, then their merge; one launch when nothing is split).  Refusals as the other calls, plus
 * IDX_E_PACK for P > IDX_ATTN_MAX_DRAFT or P * G > IDX_ATTN_MAX_ROWS, IDX_E_TOPK for P * topk >
 * IDX_ATTN_MAX_IDS, IDX_E_MODE for a bad sm_scale, IDX_E_FORMAT for another
 * kv_format and IDX_E_SHAPE for a workspace below idx_sparse_attn_workspace(p). */
int idx_sparse_attn(const idx_attn_params* p, void* stream);

/* Largest n_req * packed_queries * gqa * max_blocks of idx_step_noalloc: the
 * block scores of one step it can hold (16 MiB of fp32 per device). */
#define IDX_NOALLOC_MAX_SCORES (4 << 20)

/*
 * idx_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * same kernels as idx_step; the block scores they hand from scoring to
 * selection live in a library-owned device array of IDX_NOALLOC_MAX_SCORES
 * floats (16 MiB, one per device, held until the process ends), so
 * p->block_scores must be NULL and no block scores are returned.  The call
 * makes no allocation of any kind.  Refusals as for idx_step, and
 * IDX_E_SHAPE when n_req * packed_queries * gqa * max_blocks exceeds
 * IDX_NOALLOC_MAX_SCORES.  Every call on a device shares that device's array:
 * calls whose kernels overlap on one device (several streams, or several
 * host threads without ordering) race and may select from each other's
 * scores; order them on one stream.  The array needs no clearing between
 * calls (the score kernel writes every entry the top-k kernel reads).
 */
int idx_step_noalloc(const idx_params* p, void* stream);

/*
 * Measurement aid, not a step of the method: read n_units units of
 * unit_bytes bytes each from `base` with 16-byte loads and nothing else, to
 * measure how fast the part streams HBM.  Unit u is base + id * unit_bytes
 * with id = units[u] (or u when units is NULL); ids outside
 * [0, n_base_units) read unit 0.  A resident grid of workgroups (at most
 * n_sink) each take an equal contiguous share of the unit list, as the score
 * kernel shares its pages, and fold what they read into sink[workgroup].
 * unit_bytes: a power of two in [1024, 1 << 20]; base 16-byte aligned and
 * n_base_units * unit_bytes bytes long; nt != 0: non-temporal loads.
 */
int idx_probe_read(const void* base, int64_t n_base_units, const int32_t* units, int64_t n_units,
                   int32_t unit_bytes, int32_t nt, uint32_t* sink, int32_t n_sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif
