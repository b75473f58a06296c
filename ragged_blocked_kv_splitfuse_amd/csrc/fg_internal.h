// Internal declarations shared by the host library and the kernel launchers.
#pragma once

#include <cstdint>
#include <vector>

#include "fg.h"

namespace fgi {
// One attention work record while planning (before it is written out).
struct PlanItem {
  int32_t s, h, tok0, ntok, klo, khi, mode, group, split, nsplit;
  int64_t poff;
  float cost;
};
}  // namespace fgi

struct fg_cache {
  fg_cache_config cfg;
  void *k_pool;
  void *v_pool;
  int32_t bs_log2;
  std::vector<int32_t> free_stack;  // top = back(); handed out from the top
  std::vector<uint8_t> is_free;     // per physical id
  // planner scratch, reused across calls so planning allocates nothing in steady state
  mutable std::vector<fgi::PlanItem> plan_base, plan_items;
  mutable std::vector<std::pair<float, int32_t>> plan_order;
  mutable std::vector<int32_t> plan_lists[8];  // per XCD record lists
  mutable std::vector<int32_t> plan_se[8][4];  // per XCD and shader engine: record order
};

namespace fgi {

// Work items written by fg_attention_plan, FG_ITEM_INTS int32 each; record code c stands for
// item c / Hkv and KV head c % Hkv.
enum ItemField {
  I_SEQ = 0,     // batch index s
  I_TOK0 = 1,    // first query token (index into the sequence's new tokens)
  I_NTOK = 2,    // query tokens in the item
  I_KLO = 3,     // first key position (multiple of KEY_TILE)
  I_KHI = 4,     // one past the last key position the item covers
  I_MODE = 5,    // MODE_STREAM or MODE_TILE
  I_GROUP = 6,   // split group of KV head 0 (head h: +h), -1 when the item covers its whole range
  I_SPLIT = 7,   // split index inside the group
  I_NSPLIT = 8,  // splits in the group
  I_POFF = 9,    // float offset of head 0's partial slot 0 in the workspace (head h: + h *
                 // NSPLIT * slot_floats)
  I_RES0 = 10,
  I_RES1 = 11
};

// MODE_STREAM: at most STREAM_ROWS query rows (decode tokens, short chunks); the waves of a
// workgroup take key tiles in turn and merge at the end.
// MODE_TILE: up to TILE_ROWS query rows; all waves share every K/V tile staged in LDS.
enum { MODE_STREAM = 0, MODE_TILE = 1 };
constexpr int STREAM_ROWS = FG_STREAM_ROWS;
constexpr int TILE_ROWS = FG_TILE_ROWS;
// A workgroup of the attention launch is WAVES_PER_WG waves; a tile record gives each wave 32
// query rows, and WG_PER_CU workgroups are resident per compute unit (two waves per SIMD).
constexpr int WAVES_PER_WG = TILE_ROWS / 32;
constexpr int WG_PER_CU = 8 / WAVES_PER_WG;
static_assert(WAVES_PER_WG == 4 || WAVES_PER_WG == 8, "4 or 8 waves per workgroup");
constexpr int KEY_TILE = 64;

constexpr int64_t slot_floats(int mode, int head_dim) {
  return (int64_t)(mode == MODE_STREAM ? STREAM_ROWS : TILE_ROWS) * (head_dim + 2);
}

fg_status fail(fg_status st, const char *fmt, ...);
void clear_error();
int elem_bytes(int32_t dtype);

}  // namespace fgi
