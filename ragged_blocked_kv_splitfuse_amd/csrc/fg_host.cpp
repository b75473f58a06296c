// Host side of the library: block allocator, Dynamic SplitFuse composition, descriptor
// validation and the attention work-list planner.  No HIP runtime calls, so it builds with a
// plain C++ compiler and runs on machines without a GPU.
//
// Composition follows DeepSpeed-FastGen paper card by Holmes et al. (2024), "Summary" and
// "Interesting ideas" (fixed token budget per pass; long prompts cut into chunks over several
// passes; short prompts and generation tokens packed to fill the budget exactly), the reading
// notes page on DeepSpeed-FastGen, method paragraph (each request split into prompt and
// generation work), and the blog's "1. Introduction" (generation must not be stalled by
// prompt processing).  The blocked cache is the PagedAttention-style cache named in the
// card's "Key points".

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "fg_internal.h"

namespace fgi {

static thread_local char g_err[512] = "";

fg_status fail(fg_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_err[0] = 0; }

int elem_bytes(int32_t dtype) { return dtype == FG_BF16 ? 2 : 4; }

}  // namespace fgi

using namespace fgi;

extern "C" {

const char *fg_last_error(void) { return g_err; }

const char *fg_status_string(fg_status st) {
  switch (st) {
    case FG_OK: return "ok";
    case FG_E_ARG: return "invalid argument";
    case FG_E_DESC: return "invalid batch descriptor";
    case FG_E_NO_BLOCKS: return "no free blocks";
    case FG_E_UNSUPPORTED: return "unsupported shape or dtype";
    case FG_E_HIP: return "HIP error";
    case FG_E_WORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

// --------------------------------------------------------------------------------------
// cache handle and allocator
// --------------------------------------------------------------------------------------

fg_status fg_blocked_cache_init(const fg_cache_config *cfg, void *k_pool, void *v_pool,
                                const int32_t *free_ids, int32_t n_free, fg_cache **out) {
  clear_error();
  if (!cfg || !out) return fail(FG_E_ARG, "cfg and out must not be null");
  *out = nullptr;
  const fg_cache_config c = *cfg;
  if (c.num_blocks < 1) return fail(FG_E_ARG, "num_blocks must be >= 1 (got %d)", c.num_blocks);
  if (c.block_size < 1 || c.block_size > 1024 || (c.block_size & (c.block_size - 1)))
    return fail(FG_E_UNSUPPORTED, "block_size must be a power of two in [1, 1024] (got %d)",
                c.block_size);
  if (c.num_kv_heads < 1) return fail(FG_E_ARG, "num_kv_heads must be >= 1");
  if (c.dtype != FG_F32 && c.dtype != FG_BF16) return fail(FG_E_ARG, "unknown dtype %d", c.dtype);
  if (c.head_dim != 64 && c.head_dim != 128)
    return fail(FG_E_UNSUPPORTED, "the kernels implement head_dim 64 or 128 (got %d)",
                c.head_dim);
  if ((reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & 15)
    return fail(FG_E_ARG, "pools must be 16-byte aligned (k_pool %p, v_pool %p)", k_pool, v_pool);
  std::vector<int32_t> ids;
  if (n_free < 0) {
    if (free_ids) return fail(FG_E_ARG, "n_free < 0 requires free_ids == NULL");
    ids.resize(c.num_blocks);
    for (int32_t i = 0; i < c.num_blocks; ++i) ids[i] = i;
  } else {
    if (n_free > 0 && !free_ids) return fail(FG_E_ARG, "free_ids is null");
    ids.assign(free_ids, free_ids + n_free);
  }
  std::vector<uint8_t> is_free(c.num_blocks, 0);
  for (int32_t b : ids) {
    if (b < 0 || b >= c.num_blocks) return fail(FG_E_ARG, "free id %d out of range", b);
    if (is_free[b]) return fail(FG_E_ARG, "free id %d listed twice", b);
    is_free[b] = 1;
  }
  fg_cache *h = new (std::nothrow) fg_cache();
  if (!h) return fail(FG_E_ARG, "out of host memory");
  h->cfg = c;
  h->k_pool = k_pool;
  h->v_pool = v_pool;
  h->bs_log2 = 0;
  while ((1 << h->bs_log2) < c.block_size) ++h->bs_log2;
  h->free_stack.assign(ids.rbegin(), ids.rend());  // ids[0] ends on top
  h->is_free = std::move(is_free);
  *out = h;
  return FG_OK;
}

fg_status fg_blocked_cache_destroy(fg_cache *cache) {
  clear_error();
  delete cache;
  return FG_OK;
}

int32_t fg_blocked_cache_num_free(const fg_cache *cache) {
  return cache ? (int32_t)cache->free_stack.size() : -1;
}

fg_status fg_blocked_cache_free_ids(const fg_cache *cache, int32_t *out, int32_t cap,
                                    int32_t *n_out) {
  clear_error();
  if (!cache || !n_out) return fail(FG_E_ARG, "null argument");
  const int32_t n = (int32_t)cache->free_stack.size();
  *n_out = n;
  if (cap > 0 && !out) return fail(FG_E_ARG, "out is null");
  for (int32_t i = 0; i < std::min(n, cap); ++i) out[i] = cache->free_stack[n - 1 - i];
  return FG_OK;
}

fg_status fg_blocked_cache_release(fg_cache *cache, const int32_t *blocks, int32_t n) {
  clear_error();
  if (!cache) return fail(FG_E_ARG, "null cache");
  if (n < 0 || (n > 0 && !blocks)) return fail(FG_E_ARG, "bad block list");
  // validate and mark in one sweep (O(n), no per-call table); a bad id undoes the marks
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = blocks[i];
    const bool bad = b < 0 || b >= cache->cfg.num_blocks || cache->is_free[b];
    if (bad) {
      for (int32_t j = 0; j < i; ++j) cache->is_free[blocks[j]] = 0;
      if (b < 0 || b >= cache->cfg.num_blocks) return fail(FG_E_ARG, "block %d out of range", b);
      return fail(FG_E_ARG, "block %d is already free", b);
    }
    cache->is_free[b] = 1;
  }
  cache->free_stack.insert(cache->free_stack.end(), blocks, blocks + n);
  return FG_OK;
}

// --------------------------------------------------------------------------------------
// Dynamic SplitFuse composition
// --------------------------------------------------------------------------------------

// Tokens sequence `s` can take (<= want); pops the blocks they need from the free list.
static int32_t grant(fg_cache *cache, fg_seq_state &s, int32_t want) {
  const int32_t bs = cache->cfg.block_size;
  const int64_t c = s.n_cached;
  want = (int32_t)std::min<int64_t>(want, (int64_t)s.max_blocks * bs - c);
  if (want <= 0) return 0;
  const int64_t need_blocks = (c + want + bs - 1) / bs;
  int64_t missing = need_blocks - s.n_blocks;
  const int64_t avail = (int64_t)cache->free_stack.size();
  if (missing > avail) {
    want = (int32_t)(((int64_t)s.n_blocks + avail) * bs - c);
    missing = avail;
    if (want <= 0) return 0;
  }
  for (int64_t i = 0; i < missing; ++i) {
    const int32_t b = cache->free_stack.back();
    cache->free_stack.pop_back();
    cache->is_free[b] = 0;
    s.blocks[s.n_blocks++] = b;
  }
  return want;
}

fg_status fg_splitfuse_compose(fg_cache *cache, fg_seq_state *seqs, int32_t n_seqs,
                               int32_t token_budget, fg_ragged_batch *out) {
  clear_error();
  if (!cache || !out) return fail(FG_E_ARG, "null cache or batch");
  if (n_seqs < 0 || (n_seqs > 0 && !seqs)) return fail(FG_E_ARG, "bad sequence array");
  if (token_budget < 1) return fail(FG_E_ARG, "token budget must be >= 1 (got %d)", token_budget);
  if (out->seq_capacity < n_seqs)
    return fail(FG_E_ARG, "batch seq_capacity %d < n_seqs %d", out->seq_capacity, n_seqs);
  if (!out->query_start || (n_seqs > 0 && (!out->n_query || !out->context_len ||
                                           !out->block_table || !out->seq_index || !out->seq_id)))
    return fail(FG_E_ARG, "batch arrays must not be null");
  const int32_t bs = cache->cfg.block_size;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const fg_seq_state &s = seqs[i];
    if (s.n_cached < 0 || s.prompt_len < 0 || s.n_blocks < 0 || s.max_blocks < 0 ||
        s.n_blocks > s.max_blocks || (s.max_blocks > 0 && !s.blocks))
      return fail(FG_E_ARG, "sequence %d: inconsistent state", i);
    if ((int64_t)s.n_blocks * bs < s.n_cached)
      return fail(FG_E_ARG, "sequence %d: %d blocks cannot hold %d cached tokens", i,
                  s.n_blocks, s.n_cached);
    if (s.max_blocks > out->table_stride)
      return fail(FG_E_ARG, "sequence %d: max_blocks %d > table_stride %d", i, s.max_blocks,
                  out->table_stride);
  }
  for (int32_t i = 0; i < n_seqs; ++i) seqs[i].n_scheduled = 0;
  int32_t left = token_budget;
  // generation tokens first: one per decoding sequence, array order
  for (int32_t i = 0; i < n_seqs && left > 0; ++i) {
    fg_seq_state &s = seqs[i];
    if (s.n_cached >= s.prompt_len) {
      const int32_t n = grant(cache, s, 1);
      s.n_scheduled = n;
      left -= n;
    }
  }
  // then prompt tokens, arrival order; the last one is cut to fill the budget
  for (int32_t i = 0; i < n_seqs && left > 0; ++i) {
    fg_seq_state &s = seqs[i];
    if (s.n_cached < s.prompt_len) {
      const int32_t n = grant(cache, s, std::min(s.prompt_len - s.n_cached, left));
      s.n_scheduled = n;
      left -= n;
    }
  }
  int32_t S = 0;
  out->query_start[0] = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const fg_seq_state &s = seqs[i];
    if (s.n_scheduled <= 0) continue;
    out->n_query[S] = s.n_scheduled;
    out->query_start[S + 1] = out->query_start[S] + s.n_scheduled;
    out->context_len[S] = s.n_cached;
    int32_t *row = out->block_table + (size_t)S * out->table_stride;
    for (int32_t k = 0; k < out->table_stride; ++k) row[k] = k < s.n_blocks ? s.blocks[k] : -1;
    out->seq_index[S] = i;
    out->seq_id[S] = s.seq_id;
    ++S;
  }
  out->num_seqs = S;
  out->num_tokens = out->query_start[S];
  if (S == 0 && n_seqs > 0)
    return fail(FG_E_NO_BLOCKS, "no sequence could be given a token: the block pool is empty");
  return FG_OK;
}

fg_status fg_splitfuse_commit(fg_seq_state *seqs, int32_t n_seqs) {
  clear_error();
  if (n_seqs < 0 || (n_seqs > 0 && !seqs)) return fail(FG_E_ARG, "bad sequence array");
  for (int32_t i = 0; i < n_seqs; ++i) {
    seqs[i].n_cached += seqs[i].n_scheduled;
    seqs[i].n_scheduled = 0;
  }
  return FG_OK;
}

static bool seq_done(const fg_seq_state &s) { return s.stop_len > 0 && s.n_cached >= s.stop_len; }

fg_status fg_splitfuse_retire(fg_cache *cache, fg_seq_state *seqs, int32_t n_seqs,
                              int32_t *n_live) {
  clear_error();
  if (!cache || !n_live) return fail(FG_E_ARG, "null cache or n_live");
  if (n_seqs < 0 || (n_seqs > 0 && !seqs)) return fail(FG_E_ARG, "bad sequence array");
  std::vector<int32_t> ids;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const fg_seq_state &s = seqs[i];
    if (!seq_done(s)) continue;
    if (s.n_blocks < 0 || (s.n_blocks > 0 && !s.blocks))
      return fail(FG_E_ARG, "sequence %d: inconsistent blocks", i);
    ids.insert(ids.end(), s.blocks, s.blocks + s.n_blocks);
  }
  // one release for all of them: it checks every id first, so an error changes nothing
  const fg_status st = fg_blocked_cache_release(cache, ids.data(), (int32_t)ids.size());
  if (st != FG_OK) return st;
  fg_seq_state *mid = std::stable_partition(
      seqs, seqs + n_seqs, [](const fg_seq_state &s) { return !seq_done(s); });
  for (fg_seq_state *p = mid; p != seqs + n_seqs; ++p) p->n_blocks = 0;
  *n_live = (int32_t)(mid - seqs);
  return FG_OK;
}

// --------------------------------------------------------------------------------------
// validation
// --------------------------------------------------------------------------------------

fg_status fg_validate_batch(const fg_cache *cache, const fg_ragged_batch *b) {
  clear_error();
  if (!cache || !b) return fail(FG_E_ARG, "null argument");
  const int32_t S = b->num_seqs, bs = cache->cfg.block_size, NB = cache->cfg.num_blocks;
  if (S < 0 || b->num_tokens < 0 || b->table_stride < 0) return fail(FG_E_DESC, "negative size");
  if (!b->query_start) return fail(FG_E_DESC, "query_start is null");
  if (S > 0 && (!b->n_query || !b->context_len || !b->block_table))
    return fail(FG_E_DESC, "descriptor arrays are null");
  if (b->query_start[0] != 0) return fail(FG_E_DESC, "query_start[0] = %d", b->query_start[0]);
  std::vector<int32_t> owner(NB, -1);
  for (int32_t s = 0; s < S; ++s) {
    const int32_t n = b->n_query[s], c = b->context_len[s];
    if (n < 1) return fail(FG_E_DESC, "sequence %d has n_query %d", s, n);
    if (c < 0) return fail(FG_E_DESC, "sequence %d has context_len %d", s, c);
    if ((int64_t)b->query_start[s + 1] != (int64_t)b->query_start[s] + n)
      return fail(FG_E_DESC, "query_start[%d] is not the prefix sum", s + 1);
    const int64_t need = ((int64_t)c + n + bs - 1) / bs;
    if (need > b->table_stride)
      return fail(FG_E_DESC, "sequence %d needs %lld blocks, table_stride %d", s,
                  (long long)need, b->table_stride);
    const int32_t *row = b->block_table + (size_t)s * b->table_stride;
    for (int64_t k = 0; k < b->table_stride; ++k) {
      const int32_t id = row[k];
      if (k < need && id < 0) return fail(FG_E_DESC, "sequence %d: block %lld missing", s, (long long)k);
      if (id < 0) continue;
      if (id >= NB) return fail(FG_E_DESC, "sequence %d: block id %d out of range", s, id);
      if (owner[id] >= 0)
        return fail(FG_E_DESC, "block %d used by sequences %d and %d", id, owner[id], s);
      owner[id] = s;
    }
  }
  if (b->query_start[S] != b->num_tokens)
    return fail(FG_E_DESC, "num_tokens %d != sum of n_query %d", b->num_tokens, b->query_start[S]);
  return FG_OK;
}

// --------------------------------------------------------------------------------------
// work-list validation and workspace sizing
// --------------------------------------------------------------------------------------

fg_status fg_validate_work(const fg_cache *cache, const fg_ragged_batch *b,
                           const fg_attention_plan_info *plan, const int32_t *work,
                           size_t workspace_bytes) {
  clear_error();
  if (!cache || !b || !plan) return fail(FG_E_ARG, "null argument");
  if (cache->cfg.dtype == FG_F32) return FG_OK;  // the fp32 kernel reads no work list
  const int32_t Hkv = cache->cfg.num_kv_heads, D = cache->cfg.head_dim;
  const int32_t Hq = plan->num_q_heads;
  if (Hq < 1 || Hq % Hkv) return fail(FG_E_DESC, "plan num_q_heads %d", Hq);
  const int32_t G = Hq / Hkv, S = b->num_seqs;
  if (plan->num_tokens != b->num_tokens)
    return fail(FG_E_DESC, "plan made for %d tokens, batch has %d", plan->num_tokens,
                b->num_tokens);
  if (S < 0 || (S > 0 && (!b->n_query || !b->context_len)))
    return fail(FG_E_DESC, "batch arrays are null");
  const int64_t NI = plan->num_items, NW = plan->num_work, NG = plan->num_groups;
  if (NI < 0 || NW < 0 || NG < 0 || NG > NW ||
      (int64_t)plan->work_ints != NI * FG_ITEM_INTS + NW)
    return fail(FG_E_DESC, "inconsistent plan sizes (items %lld, records %lld, groups %lld)",
                (long long)NI, (long long)NW, (long long)NG);
  if (plan->workspace_bytes > 0 && workspace_bytes < (size_t)plan->workspace_bytes)
    return fail(FG_E_DESC, "workspace of %zu bytes, plan needs %lld", workspace_bytes,
                (long long)plan->workspace_bytes);
  if (plan->work_ints > 0 && !work) return fail(FG_E_ARG, "work is null");
  const int64_t ws_floats = (int64_t)(workspace_bytes / 4);
  // items: ranges inside their sequence, partial slots inside the workspace
  std::vector<int64_t> seq_rows(S, 0);  // query tokens x key coverage, checked below
  for (int64_t i = 0; i < NI; ++i) {
    const int32_t *w = work + i * FG_ITEM_INTS;
    const int32_t s = w[I_SEQ], t0 = w[I_TOK0], nt = w[I_NTOK], klo = w[I_KLO], khi = w[I_KHI];
    const int32_t mode = w[I_MODE], grp = w[I_GROUP], sp = w[I_SPLIT], ns = w[I_NSPLIT];
    if (s < 0 || s >= S) return fail(FG_E_DESC, "item %lld: sequence %d of %d", (long long)i, s, S);
    const int64_t c = b->context_len[s], n = b->n_query[s];
    if (t0 < 0 || nt < 1 || t0 + (int64_t)nt > n)
      return fail(FG_E_DESC, "item %lld: tokens [%d, %d) outside [0, %lld)", (long long)i, t0,
                  t0 + nt, (long long)n);
    if (mode != MODE_STREAM && mode != MODE_TILE)
      return fail(FG_E_DESC, "item %lld: mode %d", (long long)i, mode);
    const int64_t cap = mode == MODE_STREAM ? STREAM_ROWS : TILE_ROWS;
    if ((int64_t)nt * G > cap)
      return fail(FG_E_DESC, "item %lld: %lld rows > %lld", (long long)i, (long long)nt * G,
                  (long long)cap);
    if (klo < 0 || klo % KEY_TILE || khi <= klo || khi > c + t0 + nt)
      return fail(FG_E_DESC, "item %lld: key range [%d, %d) (last row sees %lld keys)",
                  (long long)i, klo, khi, (long long)(c + t0 + nt));
    if (grp < 0) {
      if (klo != 0 || khi != c + t0 + nt || sp != 0 || ns != 1)
        return fail(FG_E_DESC, "item %lld: unsplit item must cover keys [0, %lld)", (long long)i,
                    (long long)(c + t0 + nt));
      seq_rows[s] += nt;
    } else {
      if (ns < 2 || sp < 0 || sp >= ns || (int64_t)grp + Hkv > NG)
        return fail(FG_E_DESC, "item %lld: split %d of %d, group %d of %lld", (long long)i, sp,
                    ns, grp, (long long)NG);
      const int64_t slot = slot_floats(mode, D);
      const int64_t poff = w[I_POFF];
      if (poff < 0 || poff + (int64_t)Hkv * ns * slot > ws_floats)
        return fail(FG_E_DESC, "item %lld: partials [%lld, %lld) floats outside the workspace",
                    (long long)i, (long long)poff, (long long)(poff + (int64_t)Hkv * ns * slot));
      if (sp == 0) seq_rows[s] += nt;
    }
  }
  // splits of a group: consecutive items, contiguous key ranges covering [0, last row's keys)
  for (int64_t i = 0; i < NI; ++i) {
    const int32_t *w = work + i * FG_ITEM_INTS;
    if (w[I_GROUP] < 0 || w[I_SPLIT] != 0) continue;
    const int32_t ns = w[I_NSPLIT];
    if (i + ns > NI) return fail(FG_E_DESC, "item %lld: group runs past the list", (long long)i);
    int32_t next = 0;
    for (int32_t k = 0; k < ns; ++k) {
      const int32_t *u = work + (i + k) * FG_ITEM_INTS;
      if (u[I_GROUP] != w[I_GROUP] || u[I_SPLIT] != k || u[I_NSPLIT] != ns ||
          u[I_SEQ] != w[I_SEQ] || u[I_TOK0] != w[I_TOK0] || u[I_NTOK] != w[I_NTOK] ||
          u[I_MODE] != w[I_MODE] || u[I_POFF] != w[I_POFF] || u[I_KLO] != next)
        return fail(FG_E_DESC, "item %lld: split %d of its group is inconsistent",
                    (long long)(i + k), k);
      next = u[I_KHI];
    }
    const int64_t want = (int64_t)b->context_len[w[I_SEQ]] + w[I_TOK0] + w[I_NTOK];
    if (next != want)
      return fail(FG_E_DESC, "item %lld: splits end at key %d, rows need %lld", (long long)i,
                  next, (long long)want);
  }
  for (int32_t s = 0; s < S; ++s)
    if (seq_rows[s] != b->n_query[s])
      return fail(FG_E_DESC, "sequence %d: items cover %lld of %d query tokens", s,
                  (long long)seq_rows[s], b->n_query[s]);
  // records: every (item, KV head) exactly once among the attention records; merge records
  // name split 0 of each group's head
  const int32_t *codes = work + NI * FG_ITEM_INTS;
  std::vector<uint8_t> seen((size_t)(NI * Hkv), 0);
  for (int64_t r = 0; r < NW - NG; ++r) {
    const int32_t code = codes[r];
    if (code == -1) continue;
    if (code < 0 || code >= NI * Hkv)
      return fail(FG_E_DESC, "record %lld: code %d out of range", (long long)r, code);
    if (seen[code]++) return fail(FG_E_DESC, "record %lld: code %d repeated", (long long)r, code);
  }
  for (int64_t k = 0; k < NI * Hkv; ++k)
    if (!seen[k]) return fail(FG_E_DESC, "item %lld, KV head %lld has no record",
                              (long long)(k / Hkv), (long long)(k % Hkv));
  std::vector<uint8_t> gseen((size_t)NG, 0);
  for (int64_t r = NW - NG; r < NW; ++r) {
    const int32_t code = codes[r];
    if (code < 0 || code >= NI * Hkv)
      return fail(FG_E_DESC, "merge record %lld: code %d out of range", (long long)r, code);
    const int32_t *w = work + (int64_t)(code / Hkv) * FG_ITEM_INTS;
    const int64_t g = w[I_GROUP] >= 0 ? (int64_t)w[I_GROUP] + code % Hkv : -1;
    if (g < 0 || w[I_SPLIT] != 0 || g >= NG || gseen[g]++)
      return fail(FG_E_DESC, "merge record %lld: code %d names no split group once",
                  (long long)r, code);
  }
  return FG_OK;
}

fg_status fg_ragged_attention_workspace_size(const fg_cache *cache, const fg_ragged_batch *host,
                                             int32_t num_q_heads, int32_t num_cus,
                                             size_t *bytes) {
  if (!bytes) {
    clear_error();
    return fail(FG_E_ARG, "bytes is null");
  }
  *bytes = 0;
  fg_attention_plan_info info;
  const fg_status st = fg_attention_plan(cache, host, num_q_heads, num_cus, &info, nullptr, 0);
  if (st == FG_OK) *bytes = (size_t)info.workspace_bytes;
  return st;
}

// --------------------------------------------------------------------------------------
// attention work list
// --------------------------------------------------------------------------------------


fg_status fg_attention_plan(const fg_cache *cache, const fg_ragged_batch *b,
                            int32_t num_q_heads, int32_t num_cus, fg_attention_plan_info *info,
                            int32_t *work, int32_t work_capacity) {
  clear_error();
  if (!cache || !b || !info) return fail(FG_E_ARG, "null argument");
  std::memset(info, 0, sizeof(*info));
  const int32_t Hkv = cache->cfg.num_kv_heads, D = cache->cfg.head_dim;
  if (num_q_heads < 1 || num_q_heads % Hkv)
    return fail(FG_E_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads, Hkv);
  const int32_t G = num_q_heads / Hkv;
  if (G > TILE_ROWS) return fail(FG_E_UNSUPPORTED, "more than %d query heads per KV head", TILE_ROWS);
  if (num_cus < 1) return fail(FG_E_ARG, "num_cus must be >= 1");
  if (b->num_seqs < 0 || (b->num_seqs > 0 && (!b->n_query || !b->context_len || !b->query_start)))
    return fail(FG_E_ARG, "bad batch");
  info->num_q_heads = num_q_heads;
  info->num_tokens = b->num_tokens;
  if (cache->cfg.dtype == FG_F32) return FG_OK;  // the fp32 kernel needs no work list

  const double e = elem_bytes(cache->cfg.dtype);
  // Records are planned per "shape" — one (sequence, query-token tile) — because every KV
  // head of a shape has the same cost and split; heads are expanded when writing out.
  // Cost in "HBM-byte equivalents": a streamed record moves 2*D*e bytes per key; a tile
  // record does 4*D flops per visible (row, key) pair, converted at 8 TB/s against half the
  // bf16 MFMA peak, plus its K/V reads (mostly L2 hits, weighted down).
  const double flop_to_byte = 8.0e12 / (0.5 * 2.5e15);
  std::vector<PlanItem> &base = cache->plan_base;
  base.clear();
  for (int32_t s = 0; s < b->num_seqs; ++s) {
    const int32_t c = b->context_len[s], n = b->n_query[s];
    if (n < 1 || c < 0) return fail(FG_E_DESC, "sequence %d: n_query %d, context_len %d", s, n, c);
    const int32_t tpt = (n * G <= STREAM_ROWS) ? n : TILE_ROWS / G;
    for (int32_t t0 = 0; t0 < n; t0 += tpt) {
      const int32_t nt = std::min(tpt, n - t0);
      const int32_t mode = nt * G <= STREAM_ROWS ? MODE_STREAM : MODE_TILE;
      const int32_t keys = c + t0 + nt;
      double cost;
      if (mode == MODE_STREAM) {
        cost = (double)keys * 2.0 * D * e;
      } else {
        const double pairs = (double)G * ((double)nt * (c + t0) + 0.5 * nt * (nt + 1));
        cost = pairs * 4.0 * D * flop_to_byte + 0.25 * keys * 2.0 * D * e;
      }
      base.push_back({s, 0, t0, nt, 0, keys, mode, -1, 0, 1, 0, (float)cost});
    }
  }
  double total = 0;
  for (auto &it : base) total += (double)it.cost * Hkv;
  // aim for one full wave of resident workgroups (WG_PER_CU per compute unit); finer splits
  // cost partial-result traffic and merge work.  A shape is cut into round(cost / target)
  // pieces (not the ceiling): equal shapes slightly above a multiple of the target would
  // otherwise spill a few records into a second, nearly empty wave.
  const double target = total / ((double)WG_PER_CU * num_cus);

  std::vector<PlanItem> &items = cache->plan_items;  // one entry per shape and split
  items.clear();
  int32_t groups = 0;
  int64_t poff_bytes = 0;  // split partial storage in the workspace, bytes
  for (auto &it : base) {
    const int32_t tiles = (it.khi + KEY_TILE - 1) / KEY_TILE;
    int32_t nsplit = 1;
    // Stream records are cut 2x finer: one streams at a fixed per-workgroup rate however idle
    // the chip is, so a long one can become the pass's tail, while its split partial (16 rows)
    // is cheap to write and merge.  Tile splits cost a full-tile partial and a Q reload each.
    // (With four-wave workgroups, two per CU, 8x finer stream splits paid; with one
    // eight-wave workgroup per CU they only add merge work: on the LLaMA-2 mixed pass 2x
    // leaves no split at all and the attention call takes 242 us instead of 256.)
    const double tg = it.mode == MODE_STREAM ? target / 2 : target;
    if (tg > 0 && it.cost > tg) nsplit = (int32_t)std::lround(it.cost / tg);
    // a split covers at least 4 key tiles (256 keys), a stream split one per wave
    const int32_t min_tiles = it.mode == MODE_STREAM ? std::max(4, WAVES_PER_WG) : 4;
    nsplit = std::max(1, std::min(nsplit, tiles / min_tiles));
    if (nsplit == 1) {
      items.push_back(it);
      continue;
    }
    const int32_t g0 = groups;  // heads take groups g0 .. g0 + Hkv - 1
    groups += Hkv;
    const int64_t poff = poff_bytes;  // head h's group starts at poff + h * group_bytes
    const int64_t group_bytes = (int64_t)nsplit * slot_floats(it.mode, D) * 4;
    poff_bytes += group_bytes * Hkv;
    int32_t tile = 0;
    for (int32_t k = 0; k < nsplit; ++k) {
      const int32_t nt = tiles / nsplit + (k < tiles % nsplit ? 1 : 0);
      PlanItem p = it;
      p.klo = tile * KEY_TILE;
      p.khi = std::min(it.khi, (tile + nt) * KEY_TILE);
      p.group = g0;
      p.split = k;
      p.nsplit = nsplit;
      p.poff = poff;
      p.cost = it.cost * (float)nt / (float)tiles;
      tile += nt;
      items.push_back(p);
    }
  }
  // Longest first (ties keep their order), so the long-running records start early.
  std::vector<std::pair<float, int32_t>> &order = cache->plan_order;
  order.resize(items.size());
  for (size_t i = 0; i < items.size(); ++i) order[i] = {-items[i].cost, (int32_t)i};
  std::sort(order.begin(), order.end());

  // Placement across the chip's XCDs (accelerator dies, each with its own L2).  Workgroup i of
  // a launch runs on XCD i % NUM_XCD, in launch order within the XCD.  A record of sequence s,
  // KV head h and query tile t goes to XCD (h + Hkv*(s + t)) % NUM_XCD.  With Hkv a multiple
  // of NUM_XCD that is h % NUM_XCD: all tile records of one (sequence, head) read the same
  // keys on one XCD, so their K/V comes from HBM once and from that XCD's L2 for the others,
  // and every XCD gets the same share of each item.  With fewer heads the query tiles rotate
  // over the XCDs instead, so that a single sequence still uses the whole chip.
  //
  // Within an XCD, the dispatcher hands workgroups to its four shader engines (8 CUs each) in
  // turn, one per workgroup, and in launch order: a workgroup whose shader engine has no free
  // CU holds back every later one of the XCD, even when other engines sit idle (a trace of
  // every workgroup's start and end times and hardware ids shows both).  So positions j of an
  // XCD's sequence with the same j % 4 form one engine's list,
  // and each engine's list must carry the same work: each kind of record, longest first, is
  // dealt to the four lists in snake order (0 1 2 3 3 2 1 0 ...), and each list interleaves
  // its tile and stream records in proportion, so that the workgroups resident at any time
  // mix MFMA-bound tile records with HBM-bound stream records.  Lists that run short are
  // padded at their end with null records (sequence -1) that exit at once.
  constexpr int NUM_XCD = 8, NUM_SE = 4;
  std::vector<int32_t> *lists = cache->plan_lists;  // per XCD: item * Hkv + head
  int64_t xcd_tiles[NUM_XCD] = {0};
  for (int k = 0; k < NUM_XCD; ++k) lists[k].clear();
  if ((int64_t)items.size() * Hkv > INT32_MAX) return fail(FG_E_UNSUPPORTED, "too many records");
  for (int pass = 0; pass < 2; ++pass)  // tile records first, then stream records
    for (const auto &o : order) {
      const PlanItem &p = items[o.second];
      if ((p.mode == MODE_TILE) != (pass == 0)) continue;
      const int64_t tile = p.mode == MODE_TILE ? p.tok0 / (TILE_ROWS / G) : 0;
      const int32_t rot = (int32_t)(((int64_t)Hkv * (p.s + tile)) % NUM_XCD);
      for (int32_t h = 0; h < Hkv; ++h) {
        const int x = (h + rot) % NUM_XCD;
        lists[x].push_back(o.second * Hkv + h);
        if (pass == 0) ++xcd_tiles[x];
      }
    }
  // deal each XCD's records to its shader-engine lists (tile and stream records interleaved
  // in proportion, Bresenham-style, each kind in its longest-first order)
  size_t longest = 0;
  for (int k = 0; k < NUM_XCD; ++k) {
    const std::vector<int32_t> &lst = lists[k];
    const int64_t nt = xcd_tiles[k], n = (int64_t)lst.size();
    int64_t cnt[NUM_SE][2] = {};  // records of each kind dealt to each engine
    auto engine = [](int64_t i) {  // snake order
      const int r = (int)(i % NUM_SE);
      return ((i / NUM_SE) % 2) ? NUM_SE - 1 - r : r;
    };
    for (int64_t i = 0; i < nt; ++i) ++cnt[engine(i)][1];
    for (int64_t i = 0; i < n - nt; ++i) ++cnt[engine(i)][0];
    size_t sub_len = 0;
    for (int r = 0; r < NUM_SE; ++r) {
      std::vector<int32_t> &sub = cache->plan_se[k][r];
      sub.clear();
      // tiles dealt to engine r are lst[i] for i < nt with engine(i) == r; streams likewise
      int64_t it = 0, is = 0, err = 0, ti = 0, si = nt;
      const int64_t ntr = cnt[r][1], nsr = cnt[r][0];
      while (it < ntr || is < nsr) {
        const bool take_tile = is == nsr || (it < ntr && err <= 0);
        err += take_tile ? nsr : -ntr;
        if (take_tile) {
          while (engine(ti) != r) ++ti;
          sub.push_back(lst[ti++]);
          ++it;
        } else {
          while (engine(si - nt) != r) ++si;
          sub.push_back(lst[si++]);
          ++is;
        }
      }
      sub_len = std::max(sub_len, sub.size());
    }
    longest = std::max(longest, sub_len * NUM_SE);
  }
  const int64_t n_slots = (int64_t)longest * NUM_XCD;  // main records including padding

  const int64_t ws = groups ? poff_bytes : 0;
  if ((ws / 4) > INT32_MAX) return fail(FG_E_UNSUPPORTED, "workspace beyond 8 GiB");
  const int64_t n_items = (int64_t)items.size();
  const int64_t n_ints = n_items * FG_ITEM_INTS + n_slots + groups;
  if (n_ints > INT32_MAX) return fail(FG_E_UNSUPPORTED, "too many records");
  info->num_work = (int32_t)(n_slots + groups);
  info->num_groups = groups;
  info->workspace_bytes = ws;
  info->num_items = (int32_t)n_items;
  info->work_ints = (int32_t)n_ints;
  if (work_capacity < info->work_ints) {
    if (work_capacity == 0) return FG_OK;  // sizing call
    return fail(FG_E_ARG, "work capacity %d < %d int32", work_capacity, info->work_ints);
  }
  if (n_ints == 0) return FG_OK;
  if (!work) return fail(FG_E_ARG, "work is null");

  // the items
  for (int64_t i = 0; i < n_items; ++i) {
    const PlanItem &p = items[i];
    int32_t *w = work + i * FG_ITEM_INTS;
    w[I_SEQ] = p.s;
    w[I_TOK0] = p.tok0;
    w[I_NTOK] = p.ntok;
    w[I_KLO] = p.klo;
    w[I_KHI] = p.khi;
    w[I_MODE] = p.mode;
    w[I_GROUP] = p.group;
    w[I_SPLIT] = p.split;
    w[I_NSPLIT] = p.nsplit;
    w[I_POFF] = p.group >= 0 ? (int32_t)(p.poff / 4) : 0;
    w[I_RES0] = 0;
    w[I_RES1] = 0;
  }
  // the record codes, XCD-interleaved, then the merge records (split 0 of each group)
  int32_t *codes = work + n_items * FG_ITEM_INTS;
  for (int k = 0; k < NUM_XCD; ++k)
    for (int64_t j = 0; j < (int64_t)longest; ++j) {
      const std::vector<int32_t> &sub = cache->plan_se[k][j % NUM_SE];
      const size_t m = (size_t)(j / NUM_SE);
      codes[j * NUM_XCD + k] = m < sub.size() ? sub[m] : -1;  // -1: padding
    }
  for (int64_t i = 0; i < n_items; ++i) {
    const PlanItem &p = items[i];
    if (p.group < 0 || p.split != 0) continue;
    for (int32_t h = 0; h < Hkv; ++h) codes[n_slots + p.group + h] = (int32_t)(i * Hkv + h);
  }
  return FG_OK;
}

}  // extern "C"
