/*
 * fg.h — C ABI of the fixed-budget ragged pass over a blocked KV cache (MI355X / gfx950).
 *
 * One pass of the method, as the pages describe it:
 *   - Dynamic SplitFuse composition (DeepSpeed-FastGen paper card by Holmes et al. 2024,
 *     "Summary" and "Interesting ideas"): every forward pass runs a fixed token budget;
 *     long prompts are cut into chunks spread over passes, generation tokens and short
 *     prompts are packed in to fill the budget exactly;          -> fg_splitfuse_compose
 *   - the blocked (paged) KV cache it builds on (same card, "Key points", PagedAttention):
 *     physical blocks named by per-sequence block tables;        -> fg_blocked_cache_init,
 *                                                                   fg_kv_append
 *   - exact causal attention of every new token over its sequence's whole cached history
 *     (same card, "Key points" and "References": FlashAttention-derived kernels, an exact
 *     attention);                                                 -> fg_ragged_attention
 *
 * Conventions (all functions):
 *   - Plain pointers and sizes only.  "host" pointers are CPU memory; "device" pointers are
 *     GPU memory (hipMalloc / torch CUDA tensors).  The caller owns ALL memory: pools, Q,
 *     new K/V, outputs, device copies of descriptors, the work list and the workspace.  The
 *     library owns only the opaque fg_cache handle and its free list (host memory).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Device work is
 *     enqueued asynchronously on it.  No entry point allocates device memory or
 *     synchronises, except in validation mode (FG_VALIDATE=1, see fg_kv_append).
 *   - Every function returns fg_status and never aborts or throws across the ABI.  On an
 *     error nothing is launched and no state is changed, unless stated otherwise;
 *     fg_last_error() returns a thread-local message for the last failing call.
 *   - Asynchronous device faults surface at the caller's next synchronisation.
 *   - A handle is not thread-safe; use one per thread or lock around it.
 *
 * Data layouts (element type = the cache dtype everywhere: float or bfloat16 bits):
 *   q, out        [T][Hq][D]        T = batch num_tokens, rows in batch order
 *   k_new, v_new  [T][Hkv][D]
 *   K pool        [num_blocks][Hkv][block_size][D]          key-major inside a block
 *   V pool        [num_blocks][Hkv][block_size/g][D][g]     g = min(8, block_size): slots in
 *                                                          groups of g, each group
 *                                                          feature-major, its g slots adjacent
 * Slot s of a block holds its key's K row at K[b][h][s][:] and V row at V[b][h][s/g][:][s%g].
 * The K pool keeps keys major so that Q.K^T, which runs over the head dimension, reads D
 * contiguously.  The P.V contraction runs over keys, so each V feature keeps 8 consecutive
 * keys adjacent (one 16-byte bf16 operand load), while a single key's V row still spans only
 * 16*D bytes (16 cache lines at D = 128), which keeps the append of a decode token cheap.
 * Query head g uses KV head g / (Hq / Hkv).
 */
#ifndef FG_H
#define FG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fg_status {
  FG_OK = 0,
  FG_E_ARG = 1,          /* bad argument: null pointer, size out of range, capacity too small */
  FG_E_DESC = 2,         /* descriptor validation failed (block ids, counts, capacity) */
  FG_E_NO_BLOCKS = 3,    /* composition: there was demand but the pool could not take a token */
  FG_E_UNSUPPORTED = 4,  /* shape or dtype the kernels do not implement */
  FG_E_HIP = 5,          /* a HIP launch reported an error */
  FG_E_WORKSPACE = 6     /* workspace missing or smaller than fg_attention_plan asked for */
} fg_status;

typedef enum fg_dtype { FG_F32 = 0, FG_BF16 = 1 } fg_dtype;

/* Number of int32 per work item in the work list produced by fg_attention_plan. */
#define FG_ITEM_INTS 12
/* Query rows (tokens x query heads per KV head) of one attention work item: up to
 * FG_STREAM_ROWS rows are a stream item, longer row sets are cut into tile items of up to
 * FG_TILE_ROWS rows; a split item's workspace partial holds that many rows. */
#define FG_STREAM_ROWS 16
#define FG_TILE_ROWS 256

typedef struct fg_cache fg_cache; /* opaque, host-side */

typedef struct fg_cache_config {
  int32_t num_blocks;   /* physical blocks in each pool, >= 1 */
  int32_t block_size;   /* tokens per block: power of two in [1, 1024]; bf16 attention
                           needs >= 8 */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;     /* D: 64 or 128 (both dtypes) */
  int32_t dtype;        /* fg_dtype of pools, q, k_new, v_new and out */
} fg_cache_config;

/* One request as the scheduler sees it (host memory, caller-owned). */
typedef struct fg_seq_state {
  int64_t seq_id;      /* caller's id, copied into the batch */
  int32_t n_cached;    /* tokens whose K/V are already in the cache */
  int32_t prompt_len;  /* n_cached < prompt_len: prompt phase; otherwise one decode token */
  int32_t n_blocks;    /* blocks owned so far (in/out) */
  int32_t max_blocks;  /* capacity of blocks[]; the sequence never owns more */
  int32_t *blocks;     /* physical ids in logical order (in/out), capacity max_blocks */
  int32_t n_scheduled; /* out: tokens given to this sequence in the composed pass */
  int32_t stop_len;    /* > 0: the request is done once n_cached >= stop_len (a prompt of P
                          tokens and O generated tokens caches P + O - 1 positions); 0: never
                          done (fg_splitfuse_retire leaves it alone) */
} fg_seq_state;

/* Ragged batch descriptor.  The struct itself is always host memory; its arrays are host
 * memory for fg_splitfuse_compose / fg_attention_plan / fg_validate_batch and device memory
 * (a copy the caller made) for fg_kv_append / fg_ragged_attention. */
typedef struct fg_ragged_batch {
  int32_t num_seqs;     /* S: sequences in the pass */
  int32_t num_tokens;   /* T = sum of n_query */
  int32_t table_stride; /* int32 per block_table row */
  int32_t seq_capacity; /* compose output: capacity of the per-sequence arrays */
  int32_t *query_start; /* [S+1] prefix sums of n_query (first row of each sequence) */
  int32_t *n_query;     /* [S] new tokens of each sequence in this pass, >= 1 */
  int32_t *context_len; /* [S] tokens cached BEFORE this pass */
  int32_t *block_table; /* [S][table_stride] physical ids, -1 padded */
  int32_t *seq_index;   /* [S] index into the fg_seq_state array given to compose */
  int64_t *seq_id;      /* [S] */
} fg_ragged_batch;

typedef struct fg_attention_plan_info {
  int32_t num_work;          /* records: attention records (workgroups of the main launch,
                                padding included), then one merge record per split group */
  int32_t num_groups;        /* key-range split groups = merge records (the last ones) */
  int64_t workspace_bytes;   /* device workspace for split partials (0: none needed) */
  int32_t num_q_heads;       /* Hq the plan was made for */
  int32_t num_tokens;        /* T of the batch the plan was made for */
  int32_t num_items;         /* work items (query tile x key split, shared by the KV heads) */
  int32_t work_ints;         /* int32 the work list occupies:
                                num_items * FG_ITEM_INTS + num_work */
} fg_attention_plan_info;

/* ---- cache handle and block allocator ------------------------------------------------ */

/* Creates the host handle of a blocked KV cache whose two pools the caller allocated
 * (device memory, layouts above; sizes num_blocks*Hkv*block_size*D elements each).
 * free_ids[0..n_free) are the physical ids the allocator may hand out, in the order they
 * are handed out (ids already owned by sequences must not be listed); free_ids may be NULL
 * with n_free = -1 to mean 0..num_blocks-1 in order.  The free list is a stack: released
 * ids are handed out next, the last released first.
 * The kernels move 16 bytes per access, so both pools must be 16-byte aligned.
 * Errors: FG_E_ARG (null out/cfg, sizes out of range, an id out of range or repeated, a pool
 * not 16-byte aligned), FG_E_UNSUPPORTED (block_size/head_dim/dtype combination not
 * implemented). */
fg_status fg_blocked_cache_init(const fg_cache_config *cfg, void *k_pool, void *v_pool,
                                const int32_t *free_ids, int32_t n_free, fg_cache **out);
fg_status fg_blocked_cache_destroy(fg_cache *cache);
int32_t fg_blocked_cache_num_free(const fg_cache *cache); /* -1 on a null handle */
/* Copies the free ids in hand-out order into out[0..cap); *n_out = number of free ids. */
fg_status fg_blocked_cache_free_ids(const fg_cache *cache, int32_t *out, int32_t cap,
                                    int32_t *n_out);
/* Returns blocks of a finished sequence to the free list.  FG_E_ARG if an id is out of
 * range or already free (then nothing is released). */
fg_status fg_blocked_cache_release(fg_cache *cache, const int32_t *blocks, int32_t n);

/* ---- Dynamic SplitFuse composition (host) -------------------------------------------- */

/* Composes one pass of at most token_budget tokens over seqs[0..n_seqs):
 *   1. each sequence in its generation phase (n_cached >= prompt_len) gets 1 token, in
 *      array order;
 *   2. prompt tokens fill what is left, sequences in array (arrival) order, the last one cut
 *      so the budget is filled exactly when demand allows; a shorter pass is not padded.
 * Before a sequence gets n tokens it is given blocks up to ceil((n_cached+n)/block_size)
 * from the free list; if the pool runs dry it gets what fits (a decode: 0 or 1 token).
 * Writes the batch (sequences with n_scheduled > 0, in array order) into out's host
 * arrays, which need out->seq_capacity >= n_seqs and out->table_stride >= every
 * max_blocks.  Mutates seqs[i].blocks/n_blocks/n_scheduled and the free list only.
 * Errors: FG_E_ARG (budget < 1, null pointers, capacities), FG_E_NO_BLOCKS (demand, but
 * not a single token fitted; the batch is empty and nothing changed). */
fg_status fg_splitfuse_compose(fg_cache *cache, fg_seq_state *seqs, int32_t n_seqs,
                               int32_t token_budget, fg_ragged_batch *out);
/* After the pass ran: n_cached += n_scheduled, n_scheduled = 0, for every sequence. */
fg_status fg_splitfuse_commit(fg_seq_state *seqs, int32_t n_seqs);

/* Continuous batching (blog "1. Introduction" and the paper card's "Key points": requests
 * join and leave the running set between passes, the blocked KV cache recycling the blocks
 * of finished ones).  Call after fg_splitfuse_commit.  Every sequence with stop_len > 0 and
 * n_cached >= stop_len is retired: its blocks go back to the free list -- retired sequences
 * in array order, each one's blocks in logical order, so the last block of the last retired
 * sequence is handed out first -- and its n_blocks becomes 0.  The array is then stably
 * partitioned: live sequences first (their order kept), the retired ones after them (theirs
 * kept), so seqs[*n_live..n_seqs) are the retired entries, whose blocks storage the caller
 * may reuse for new requests.  Errors: FG_E_ARG (null pointers, a sequence with blocks but
 * no storage, a block id out of range, already free or owned twice); then nothing changed. */
fg_status fg_splitfuse_retire(fg_cache *cache, fg_seq_state *seqs, int32_t n_seqs,
                              int32_t *n_live);

/* Full O(S * table_stride) check of a host batch: prefix sums, n_query >= 1, every block a
 * valid id, no id used twice, enough blocks for context_len + n_query.  FG_E_DESC names the
 * first violation in fg_last_error(). */
fg_status fg_validate_batch(const fg_cache *cache, const fg_ragged_batch *host);

/* Full check of a work list against the host batch and plan it was made for (host only):
 * sizes consistent with the plan; every item's sequence, query tokens and key range inside
 * that sequence (an unsplit item covers keys [0, c + last token + 1); the splits of a group
 * are consecutive items whose key ranges tile that span in split order); every query token
 * of every sequence in exactly one item; each item's split partials inside workspace_bytes;
 * every (item, KV head) in exactly one attention record; every merge record naming split 0
 * of one split group.  fg_ragged_attention runs this check on device copies when FG_VALIDATE
 * is set (below).  FG_E_DESC names the first violation in fg_last_error(); FG_E_ARG for null
 * arguments.  FG_F32 caches need no work list: FG_OK. */
fg_status fg_validate_work(const fg_cache *cache, const fg_ragged_batch *host,
                           const fg_attention_plan_info *plan, const int32_t *work,
                           size_t workspace_bytes);

/* ---- device work -------------------------------------------------------------------- */

/* Appends the pass's new rows: new token i of sequence s (position context_len[s]+i) goes
 * to block block_table[s][pos / block_size], slot pos % block_size, of both pools.  A bit
 * copy; no other element of either pool is written.  `dev` arrays are device memory.
 * k_new, v_new: device [T][Hkv][D], 16-byte aligned.  Errors: FG_E_ARG (null or unaligned
 * pointers, negative sizes), FG_E_DESC (FG_VALIDATE only), FG_E_HIP.
 * Validation mode: with the environment variable FG_VALIDATE=1 (read at every call) the
 * descriptors are first copied back to the host on `stream` -- which synchronises the stream
 * -- and checked as fg_validate_batch does; on a violation nothing is launched and FG_E_DESC
 * is returned.  Without it only cheap argument checks run and block ids are clamped into the
 * pool, so a bad table cannot make the kernel write outside the pools. */
fg_status fg_kv_append(const fg_cache *cache, const fg_ragged_batch *dev, const void *k_new,
                       const void *v_new, void *stream);

/* Splits the attention of a host batch into work (host only).  Sequences with at most 16
 * query rows (rows = tokens x query heads per KV head) become key-streaming items, others
 * tiles of up to FG_TILE_ROWS rows; long key ranges are split so that about one record per
 * resident workgroup (one per compute unit) exists.  A record is one item for one KV head.  The work list, info->
 * work_ints int32 written to `work` (host), is
 *   items[num_items][FG_ITEM_INTS]   the items (layout private to this library), then
 *   codes[num_work]                  record r = codes[r]: item * Hkv + KV head, or -1 for a
 *                                    padding record; the last num_groups are the merge
 *                                    records of the split groups.
 * Records come longest first, laid out so that record r runs on XCD r % 8 of the launch
 * with all records of a (sequence, KV head) on one XCD.  With work_capacity (in int32) 0 it
 * only sizes (FG_OK); with 0 < work_capacity < work_ints it returns FG_E_ARG.  The caller
 * copies `work` to the device. */
fg_status fg_attention_plan(const fg_cache *cache, const fg_ragged_batch *host,
                            int32_t num_q_heads, int32_t num_cus,
                            fg_attention_plan_info *info, int32_t *work,
                            int32_t work_capacity);

/* Device workspace (bytes) fg_ragged_attention needs for this host batch when planned with
 * fg_attention_plan for num_q_heads and num_cus: the same figure as plan->workspace_bytes,
 * without writing a work list.  0 when the plan splits no key range.  Errors as
 * fg_attention_plan (FG_E_ARG also for a null `bytes`). */
fg_status fg_ragged_attention_workspace_size(const fg_cache *cache, const fg_ragged_batch *host,
                                             int32_t num_q_heads, int32_t num_cus,
                                             size_t *bytes);

/* Exact causal attention of every new token over its sequence's cached history (keys
 * 0 .. context_len[s] + i for new token i, which includes the rows fg_kv_append just
 * wrote): out[t][g] = sum_j softmax_j(scale * q[t][g] . K_j) V_j.  bf16 inputs: products
 * on bf16 MFMA with fp32 accumulation, P rounded to bf16 for the P.V product, output
 * rounded to nearest even; fp32 inputs: fp32 arithmetic.  `dev` arrays, q, out, work_dev
 * and workspace are device memory; `plan` is the host info fg_attention_plan returned for
 * this batch and work_dev the device copy of its work list (both unused for FG_F32).  One
 * launch runs every attention record (decode and chunk rows together); a second, small
 * launch merges split groups when the plan has any.  The workspace needs no initialisation
 * (its contents are scratch); calls sharing a workspace must be ordered on one stream.
 * Results are deterministic (no atomics; merges run in split order).  q, out and workspace
 * must be 16-byte aligned.
 * Validation mode (FG_VALIDATE=1, as for fg_kv_append): the descriptors and the work list are
 * copied back on `stream` (synchronising it) and checked with fg_validate_batch and
 * fg_validate_work before anything is launched; a violation returns FG_E_DESC.
 * Errors: FG_E_ARG, FG_E_DESC (FG_VALIDATE only), FG_E_UNSUPPORTED, FG_E_WORKSPACE, FG_E_HIP. */
fg_status fg_ragged_attention(const fg_cache *cache, const fg_ragged_batch *dev,
                              const fg_attention_plan_info *plan, const int32_t *work_dev,
                              const void *q, int32_t num_q_heads, float scale, void *out,
                              void *workspace, size_t workspace_bytes, void *stream);

/* fg_ragged_attention for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and the
 * same results, bit for bit, with the split partials kept in a fixed scratch array that the
 * library's code object holds on each device (FG_NOALLOC_WORKSPACE_BYTES per device, held
 * until the process ends) instead of a caller workspace.  The caller still passes q, out, the
 * device descriptors and the work list.  No device memory is allocated or freed by this call.
 * The scratch needs no initialisation (every byte read was written earlier in the same call).
 * Every call on a device shares that device's scratch: calls that may overlap on one device
 * (on different streams, or from different threads without ordering) race; order them on one
 * stream.  FG_VALIDATE is not honoured here (its copies and synchronisation are what such
 * callers avoid); validate with fg_validate_batch / fg_validate_work on the host instead.
 * Errors: as fg_ragged_attention; FG_E_WORKSPACE when plan->workspace_bytes exceeds
 * FG_NOALLOC_WORKSPACE_BYTES (checked before anything else runs), FG_E_HIP if the scratch's
 * device address cannot be looked up. */
#define FG_NOALLOC_WORKSPACE_BYTES (64u << 20)
fg_status fg_ragged_attention_noalloc(const fg_cache *cache, const fg_ragged_batch *dev,
                                      const fg_attention_plan_info *plan,
                                      const int32_t *work_dev, const void *q,
                                      int32_t num_q_heads, float scale, void *out,
                                      void *stream);

/* ---- diagnostics -------------------------------------------------------------------- */
/* ---- dense projections either side of attention ------------------------------------ */

/* The layer ops next to the pass (paper card "Key points": FastGen's kernels come from
 * FlashAttention and FasterTransformer): the QKV projection whose K and V rows feed
 * fg_kv_append and whose Q rows feed fg_ragged_attention, and the output projection of the
 * attention rows.  y[T][N] = x[T][K] . w[N][K]^T (w in the [out][in] layout of a linear
 * layer), all three bf16, device memory, row-major, dense and 16-byte aligned; fp32
 * accumulation, one rounding to bf16 (nearest even) per output.  This library's own bf16 MFMA
 * GEMM for gfx950 (tile shape chosen from T and N); it allocates nothing and keeps no state.
 * Errors: FG_E_ARG (null or unaligned pointer, T < 0, K or N < 1), FG_E_UNSUPPORTED (N not a
 * multiple of 128 or K not a multiple of 64), FG_E_HIP.  T = 0 does nothing. */
fg_status fg_linear_bf16(const void *x, const void *w, void *y, int32_t T, int32_t K, int32_t N,
                         void *stream);

/* The fused QKV projection (same paper card, "Key points": the FasterTransformer layer kernels):
 * one product over the stacked weights w_qkv[Nq + 2*Nkv][K] (Wq's Nq rows, then Wk's Nkv rows,
 * then Wv's) whose output columns land in three separate dense matrices, q[T][Nq], k[T][Nkv]
 * and v[T][Nkv] -- the layouts fg_ragged_attention and fg_kv_append read (Nq = query heads x
 * head dim, Nkv = KV heads x head dim).  Each output element equals the corresponding
 * fg_linear_bf16 output of that weight block, bit for bit (same kernels and summation order);
 * one launch instead of three gives the tile chooser a wider product.  Same memory and
 * arithmetic rules as fg_linear_bf16; allocates nothing.  Errors: FG_E_ARG (null or unaligned
 * pointer, T < 0, K, Nq or Nkv < 1), FG_E_UNSUPPORTED (Nq or Nkv not a multiple of 128, K not
 * a multiple of 64), FG_E_HIP.  T = 0 does nothing. */
fg_status fg_linear_qkv_bf16(const void *x, const void *w_qkv, void *q, void *k, void *v,
                             int32_t T, int32_t K, int32_t Nq, int32_t Nkv, void *stream);

const char *fg_status_string(fg_status status);
const char *fg_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FG_H */
