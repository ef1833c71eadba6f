// Internal declarations shared by the host planner and the device entry points of
// libpic.so.  Nothing here is part of the public ABI (include/pic.h is).
#pragma once

#include <stdint.h>
#include <stddef.h>

#include "pic.h"

namespace pic {

// Validated read-only view of a host plan header.
struct PlanHeader {
  const int32_t *w = nullptr;
  int32_t operator[](int i) const { return w[i]; }
  bool valid() const {
    return w != nullptr && w[PIC_H_MAGIC] == PIC_PLAN_MAGIC && w[PIC_H_WORDS] >= PIC_PLAN_HEADER_WORDS;
  }
};

// Attention tile and item records as stored in the plan (8 int32 words each).
struct AttnTile {
  int32_t req, row_begin, n_rows, tok_base, p_first, p_last;
  int32_t pad0;  // first recomputed (fresh) row of the request
  int32_t pad1;  // recomputed rows of the request
};
struct AttnItem {
  int32_t tile, kv_head, key_begin, key_end, slot, pad0, pad1, pad2;
};
struct MergeEntry {
  int32_t tile, kv_head, slot_base, n_slots;
};
struct DecItem {
  int32_t src;  // pool chunk id (>= 0) or -1 - b for the fresh rows of request b
  int32_t n_keys, use_begin, n_uses;
};
struct DecPiece {
  int32_t item, g;        // decode item and kv head
  int32_t t_begin, t_end; // keys of the item this piece scores
  int32_t rec_off;        // its records: piece_recs[rec_off .. rec_off + n_uses)
  int32_t pad0, pad1, pad2;
};
struct RopeTile {
  int32_t tok_begin, n_rows, delta;
  int32_t pos0;  // global position (within the request) of the first row
};

static_assert(sizeof(AttnTile) == 32, "plan record size");
static_assert(sizeof(AttnItem) == 32, "plan record size");
static_assert(sizeof(MergeEntry) == 16, "plan record size");
static_assert(sizeof(RopeTile) == 16, "plan record size");
static_assert(sizeof(DecItem) == 16, "plan record size");
static_assert(sizeof(DecPiece) == 32, "plan record size");
static_assert(PIC_H_RESERVED7 < PIC_PLAN_HEADER_WORDS, "header fields fit the header");

inline size_t dtype_size(int32_t dt) { return dt == PIC_BF16 ? 2 : (dt == PIC_F32 ? 4 : 0); }

// Softmax scale of the attention calls: a value <= 0 selects the default 1/sqrt(head_dim)
// (the scaled dot product of the EPIC Step 3 listing); NaN or infinity is an error.
inline bool resolve_scale(float &scale, int32_t head_dim) {
  if (scale != scale || scale == __builtin_inff() || scale == -__builtin_inff() || head_dim <= 0)
    return false;
  if (scale <= 0.f) scale = (float)(1.0 / __builtin_sqrt((double)head_dim));
  return true;
}

}  // namespace pic
