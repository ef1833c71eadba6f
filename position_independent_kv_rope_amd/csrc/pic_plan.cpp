// Host planner of libpic.so: pic_build_index and pic_strerror.
//
// Integer work only.  It produces the recompute index of LegoLink-k (EPIC walkthrough,
// link_legolink Step 1: skip chunk 0, take the first min(k, L_c) tokens of every later
// chunk, then every query token; HYPIC section 2.2 applies the same rule with k = w) and
// the launch schedules of the three device kernels:
//   * rope tiles: runs of at most PIC_ROPE_TILE_ROWS cached rows of one chunk that keep
//     their cached K (the recomputed rows are skipped, the splice overwrites them);
//   * attention tiles: PIC_ATTN_TILE_M (row, head) pairs = PIC_ATTN_TILE_M / G
//     consecutive recomputed rows of one request times the G query heads of a KV head;
//   * attention items: (tile, kv head, key range); long tiles are split along keys so
//     the grid fills the GPU, and each split writes a partial result that a merge pass
//     combines.  Items are dispatched longest first (the LPT rule HYPIC uses to balance
//     its segment workers, section 2.3) within each XCD, with the items that share K/V
//     kept on one XCD (see xcd_order).
#include <algorithm>
#include <cstring>
#include <numeric>
#include <unordered_map>
#include <vector>

#include "pic_internal.h"

namespace {

constexpr int64_t kMaxI32 = 0x7fffffff;
constexpr int32_t kKeyAlign = 64;       // attention key block
constexpr int32_t kMinSplitKeys = 1024;  // smallest key range worth a partial result
constexpr int kXcd = 8;                  // MI355X dies with a private L2 each
constexpr int64_t kSegKeys = 8192;       // longest split-KV segment
constexpr int64_t kTailKeys = 4096;      // longest item in a die's last round

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Dispatch order of the attention items for a GPU whose consecutive workgroups go
// round-robin to n_xcd dies, each with its own L2 (MI355X: 8 XCDs).  Items that read
// the same K/V (same request and KV head: a "stream") are kept on one die so they
// share its L2: streams are assigned to dies greedily by total cost (largest first,
// to the least loaded die), each die runs its items segment by segment, and position
// i of the launch takes the next item of die i % n_xcd.  When a die runs out, the
// remaining items fill its positions, longest first.  With tail_keys > 0, the items a
// die starts during its last round (its final slots_per_die * round_keys of work) have
// their first key range cut into pieces of at most tail_keys (multiples of align; a
// second range -- the fresh blocks a paged plan attaches to the first pool range of a
// tile -- stays with the first piece), kept on that die, so the launch does not end
// waiting for a few long items.  Lengths are in keys for contiguous plans and in key
// blocks for paged ones.
std::vector<pic::AttnItem> xcd_order(std::vector<pic::AttnItem> items,
                                     const std::vector<pic::AttnTile> &tiles, int n_xcd,
                                     int64_t tail_keys = 0, int64_t slots_per_die = 0,
                                     int64_t round_keys = 0, int64_t align = 1) {
  using pic::AttnItem;
  auto len = [](const AttnItem &a) {  // second range used by paged plans
    return (int64_t)a.key_end - a.key_begin + ((int64_t)a.pad1 - a.pad0);
  };
  std::stable_sort(items.begin(), items.end(),
                   [&](const AttnItem &a, const AttnItem &b) { return len(a) > len(b); });
  if (n_xcd <= 1 || items.size() < 2) return items;
  // stream id = (request, kv head)
  std::vector<int64_t> key(items.size());
  std::vector<std::pair<int64_t, int64_t>> cost;  // (stream, cost)
  {
    std::vector<int64_t> ids;
    for (size_t i = 0; i < items.size(); ++i) {
      key[i] = (int64_t)tiles[items[i].tile].req * 65536 + items[i].kv_head;
      ids.push_back(key[i]);
    }
    std::sort(ids.begin(), ids.end());
    ids.erase(std::unique(ids.begin(), ids.end()), ids.end());
    cost.resize(ids.size());
    for (size_t s = 0; s < ids.size(); ++s) cost[s] = {ids[s], 0};
    for (size_t i = 0; i < items.size(); ++i) {
      auto it = std::lower_bound(ids.begin(), ids.end(), key[i]);
      cost[it - ids.begin()].second += len(items[i]);
    }
  }
  std::vector<size_t> order(cost.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t a, size_t b) { return cost[a].second > cost[b].second; });
  std::vector<int64_t> load(n_xcd, 0);
  std::vector<std::pair<int64_t, int>> die_of;  // (stream, die)
  for (size_t s : order) {
    const int d = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    load[d] += cost[s].second;
    die_of.push_back({cost[s].first, d});
  }
  std::sort(die_of.begin(), die_of.end());
  std::vector<std::vector<AttnItem>> per_die(n_xcd);
  std::vector<std::vector<int64_t>> per_die_key(n_xcd);
  for (size_t i = 0; i < items.size(); ++i) {
    auto it = std::lower_bound(die_of.begin(), die_of.end(), std::make_pair(key[i], -1));
    per_die[it->second].push_back(items[i]);
    per_die_key[it->second].push_back(key[i]);
  }
  // within a die: segment-major (key_begin), then stream, then longest first, so the
  // items that read the same K/V rows run side by side
  for (int d = 0; d < n_xcd; ++d) {
    std::vector<size_t> idx(per_die[d].size());
    std::iota(idx.begin(), idx.end(), 0);
    const auto &v = per_die[d];
    const auto &kk = per_die_key[d];
    std::stable_sort(idx.begin(), idx.end(), [&](size_t a, size_t b) {
      if (v[a].key_begin != v[b].key_begin) return v[a].key_begin < v[b].key_begin;
      if (kk[a] != kk[b]) return kk[a] < kk[b];
      return len(v[a]) > len(v[b]);
    });
    std::vector<AttnItem> sorted;
    for (size_t i : idx) sorted.push_back(v[i]);
    if (tail_keys > 0) {
      int64_t total = 0;
      for (const AttnItem &a : sorted) total += len(a);
      const int64_t tail_from = total - slots_per_die * round_keys;
      std::vector<AttnItem> cut;
      int64_t done = 0;
      size_t first_cut = sorted.size();
      for (const AttnItem &a : sorted) {
        const int64_t n = len(a), n1 = (int64_t)a.key_end - a.key_begin;
        if (done >= tail_from && n1 > tail_keys) {
          first_cut = std::min(first_cut, cut.size());
          const int64_t pieces = (n1 + tail_keys - 1) / tail_keys;
          const int64_t step = round_up((n1 + pieces - 1) / pieces, align);
          for (int64_t b = a.key_begin; b < a.key_end; b += step) {
            AttnItem p = a;
            p.key_begin = (int32_t)b;
            p.key_end = (int32_t)std::min<int64_t>(a.key_end, b + step);
            if (b != a.key_begin) p.pad0 = p.pad1;  // the second range stays with piece 0
            cut.push_back(p);
          }
        } else {
          cut.push_back(a);
        }
        done += n;
      }
      // the pieces run segment by segment again, each stream's pieces side by side
      auto stream = [&](const AttnItem &x) {
        return (int64_t)tiles[x.tile].req * 65536 + x.kv_head;
      };
      std::stable_sort(cut.begin() + (std::ptrdiff_t)first_cut, cut.end(),
                       [&](const AttnItem &x, const AttnItem &y) {
                         if (x.key_begin != y.key_begin) return x.key_begin < y.key_begin;
                         return stream(x) < stream(y);
                       });
      sorted.swap(cut);
    }
    per_die[d].swap(sorted);
  }
  size_t n_out = 0;  // the items after the tail cut
  for (int d = 0; d < n_xcd; ++d) n_out += per_die[d].size();
  std::vector<AttnItem> out;
  out.reserve(n_out);
  std::vector<size_t> next(n_xcd, 0);
  for (size_t pos = 0; out.size() < n_out; ++pos) {
    int d = (int)(pos % n_xcd);
    if (next[d] >= per_die[d].size()) {
      // this die is done: take the longest remaining item of any die
      int best = -1;
      for (int e = 0; e < n_xcd; ++e)
        if (next[e] < per_die[e].size() &&
            (best < 0 || len(per_die[e][next[e]]) > len(per_die[best][next[best]])))
          best = e;
      d = best;
    }
    out.push_back(per_die[d][next[d]++]);
  }
  return out;
}

}  // namespace

extern "C" int pic_build_index(int32_t n_req, const int32_t *req_chunk_ptr,
                               const int32_t *chunk_lens, const int32_t *q_lens,
                               const int32_t *chunk_ids, int32_t k, int32_t pos_base,
                               int32_t h_q, int32_t h_kv, int32_t n_cu, int32_t *plan,
                               int64_t plan_cap, int64_t *plan_words) {
  using namespace pic;
  if (plan_words == nullptr || n_req < 0 || k < 0 || h_q <= 0 || h_kv <= 0) return PIC_EINVAL;
  if (h_q % h_kv != 0) return PIC_EINVAL;
  const int32_t group = h_q / h_kv;
  if (group > PIC_ATTN_TILE_M || PIC_ATTN_TILE_M % group != 0) return PIC_EUNSUPPORTED;
  if (n_req > 0 && (req_chunk_ptr == nullptr || q_lens == nullptr)) return PIC_EINVAL;
  if (n_req > 0 && req_chunk_ptr[0] != 0) return PIC_EINVAL;
  for (int32_t b = 0; b < n_req; ++b) {
    if (req_chunk_ptr[b + 1] < req_chunk_ptr[b] || q_lens[b] < 0) return PIC_EINVAL;
  }
  const int32_t n_chunks = n_req > 0 ? req_chunk_ptr[n_req] : 0;
  if (n_chunks > 0 && chunk_lens == nullptr) return PIC_EINVAL;
  for (int32_t c = 0; c < n_chunks; ++c)
    if (chunk_lens[c] < 0 || (chunk_ids != nullptr && chunk_ids[c] < 0)) return PIC_EINVAL;
  const bool paged = chunk_ids != nullptr;
  if (n_cu <= 0) n_cu = 256;
  if (paged) {  // a pool chunk has one length wherever it is used
    std::unordered_map<int32_t, int32_t> len_of;
    for (int32_t c = 0; c < n_chunks; ++c) {
      const auto ins = len_of.emplace(chunk_ids[c], chunk_lens[c]);
      if (!ins.second && ins.first->second != chunk_lens[c]) return PIC_EINVAL;
    }
  }

  // ---- offsets, token and row pointers (64-bit, then range-checked) ----
  std::vector<int32_t> chunk_off(n_chunks + n_req);
  std::vector<int32_t> req_tok_ptr(n_req + 1), req_row_ptr(n_req + 1);
  int64_t tok = 0, nrows = 0, max_tokens = 0;
  for (int32_t b = 0; b < n_req; ++b) {
    const int32_t c0 = req_chunk_ptr[b], c1 = req_chunk_ptr[b + 1];
    int64_t off = 0, r = 0;
    for (int32_t c = c0; c < c1; ++c) {
      chunk_off[c + b] = (int32_t)std::min<int64_t>(off, kMaxI32);
      if (c > c0) r += std::min<int64_t>(k, chunk_lens[c]);
      off += chunk_lens[c];
      if (off > kMaxI32) return PIC_EINVAL;
    }
    chunk_off[c1 + b] = (int32_t)off;
    const int64_t n_b = off + q_lens[b];
    r += q_lens[b];
    req_tok_ptr[b] = (int32_t)tok;
    req_row_ptr[b] = (int32_t)nrows;
    tok += n_b;
    nrows += r;
    max_tokens = std::max(max_tokens, n_b);
    if (tok > kMaxI32 || nrows > kMaxI32) return PIC_EINVAL;
  }
  req_tok_ptr[n_req] = (int32_t)tok;
  req_row_ptr[n_req] = (int32_t)nrows;

  // ---- recompute index: ascending positions per request.  Position j is recomputed
  // when it is a query position (j >= ctx) or lies in a chunk c >= 1 with
  // j - off_c < k; per chunk those are the positions off_c .. off_c + min(k, L_c) - 1 ----
  std::vector<int32_t> rows(nrows), row_tok(nrows);
  {
    int64_t r = 0;
    for (int32_t b = 0; b < n_req; ++b) {
      const int32_t c0 = req_chunk_ptr[b], c1 = req_chunk_ptr[b + 1];
      for (int32_t c = c0 + 1; c < c1; ++c) {
        const int32_t off = chunk_off[c + b];
        const int32_t m = std::min(k, chunk_lens[c]);
        for (int32_t j = 0; j < m; ++j) rows[r++] = off + j;
      }
      const int32_t ctx = chunk_off[c1 + b];
      for (int32_t j = 0; j < q_lens[b]; ++j) rows[r++] = ctx + j;
    }
    for (int32_t b = 0; b < n_req; ++b)
      for (int32_t i = req_row_ptr[b]; i < req_row_ptr[b + 1]; ++i)
        row_tok[i] = req_tok_ptr[b] + rows[i];
  }

  // ---- rope tiles: every cached row that keeps its K (delta 0 included: rotation by
  // delta skips those tiles, RoPE at the target position needs them) ----
  std::vector<RopeTile> rope;
  for (int32_t b = 0; b < n_req; ++b) {
    if (paged) break;  // the shared pool is never rotated in place
    const int32_t c0 = req_chunk_ptr[b], c1 = req_chunk_ptr[b + 1];
    for (int32_t c = c0; c < c1; ++c) {
      const int64_t delta = (int64_t)chunk_off[c + b] - pos_base;
      // the device forms delta in fp32 exactly, which holds for |delta| <= 2^24
      if (delta > (int64_t(1) << 24) || delta < -(int64_t(1) << 24)) return PIC_EUNSUPPORTED;
      const int32_t skip = (c > c0) ? std::min(k, chunk_lens[c]) : 0;
      for (int32_t t = skip; t < chunk_lens[c]; t += PIC_ROPE_TILE_ROWS) {
        RopeTile rt;
        rt.tok_begin = req_tok_ptr[b] + chunk_off[c + b] + t;
        rt.n_rows = std::min<int32_t>(PIC_ROPE_TILE_ROWS, chunk_lens[c] - t);
        rt.delta = (int32_t)delta;
        rt.pos0 = chunk_off[c + b] + t;
        rope.push_back(rt);
      }
    }
  }

  // ---- paged pool: per-chunk segment records and per-request key blocks ----
  std::vector<int32_t> segs;     // [n_chunks][8]
  std::vector<int32_t> kblocks;  // [n_kblocks][4]
  std::vector<int64_t> kb_fresh(n_req + 1, 0), kb_pool(n_req + 1, 0);  // per request starts
  if (paged) {
    segs.assign((size_t)n_chunks * 8, 0);
    for (int32_t b = 0; b < n_req; ++b) {
      const int32_t c0 = req_chunk_ptr[b], c1 = req_chunk_ptr[b + 1];
      for (int32_t c = c0; c < c1; ++c) {
        const int64_t delta = (int64_t)chunk_off[c + b] - pos_base;
        if (delta > (int64_t(1) << 24) || delta < -(int64_t(1) << 24)) return PIC_EUNSUPPORTED;
        int32_t *sg = &segs[(size_t)c * 8];
        sg[0] = chunk_off[c + b];
        sg[1] = chunk_lens[c];
        sg[2] = c > c0 ? std::min(k, chunk_lens[c]) : 0;
        sg[3] = chunk_ids[c];
        sg[4] = (int32_t)delta;
        sg[5] = b;
      }
      // fresh rows of the request (seams then queries), 64 per block
      kb_fresh[b] = (int64_t)kblocks.size() / 4;
      const int32_t r_b = req_row_ptr[b + 1] - req_row_ptr[b];
      for (int32_t r0 = 0; r0 < r_b; r0 += kKeyAlign) {
        kblocks.insert(kblocks.end(), {-1, r0, rows[req_row_ptr[b] + r0], 0});
      }
      // pool rows chunk by chunk; blocks holding only seam rows are skipped
      kb_pool[b] = (int64_t)kblocks.size() / 4;
      for (int32_t c = c0; c < c1; ++c) {
        const int32_t seam = segs[(size_t)c * 8 + 2];
        for (int32_t t0 = 0; t0 < chunk_lens[c]; t0 += kKeyAlign) {
          if (t0 + kKeyAlign <= seam) continue;
          kblocks.insert(kblocks.end(), {c, t0, chunk_off[c + b] + t0, 0});
        }
      }
      if ((int64_t)kblocks.size() / 4 > kMaxI32) return PIC_EINVAL;
    }
    kb_fresh[n_req] = kb_pool[n_req] = (int64_t)kblocks.size() / 4;
  }

  // ---- attention tiles ----
  const int32_t tile_rows = PIC_ATTN_TILE_M / group;
  std::vector<AttnTile> tiles;
  for (int32_t b = 0; b < n_req; ++b) {
    for (int32_t r0 = req_row_ptr[b]; r0 < req_row_ptr[b + 1]; r0 += tile_rows) {
      AttnTile t{};
      t.req = b;
      t.row_begin = r0;
      t.n_rows = std::min(tile_rows, req_row_ptr[b + 1] - r0);
      t.tok_base = req_tok_ptr[b];
      t.p_first = rows[r0];
      t.p_last = rows[r0 + t.n_rows - 1];
      t.pad0 = req_row_ptr[b];                       // first fresh row of the request
      t.pad1 = req_row_ptr[b + 1] - req_row_ptr[b];  // fresh rows of the request
      tiles.push_back(t);
    }
  }

  // ---- split-KV sizing ----
  // Keys are split on a global grid of seg_len keys.  All tiles of one (request, kv
  // head) stream that reach a grid segment read the same K/V rows there; dispatched
  // together on one XCD they stream those rows in lockstep, so the XCD's L2 serves
  // the re-reads.  seg_len is also capped so that small batches still fill the GPU:
  // items no longer than a half or a third of a fair share per workgroup slot,
  // whichever packs the item count (every tile's keys start at 0) closer to whole
  // rounds of the slots.
  int64_t total_cost = 0;
  for (const AttnTile &t : tiles) total_cost += (int64_t)(t.p_last + 1) * h_kv;
  const int64_t slots = (int64_t)n_cu * 2;
  auto seg_for = [&](int64_t per_slot) {
    const int64_t sl = std::max<int64_t>(kMinSplitKeys, total_cost / std::max<int64_t>(1, slots * per_slot));
    return round_up(std::min<int64_t>(sl, kSegKeys), kKeyAlign);
  };
  auto round_fill = [&](int64_t sl) {
    int64_t n = 0;
    for (const AttnTile &t : tiles) n += (int64_t)h_kv * ((t.p_last + sl) / sl);
    return (double)n / (double)(std::max<int64_t>(1, (n + slots - 1) / slots) * slots);
  };
  int64_t seg_len = seg_for(2);
  {
    const int64_t s3 = seg_for(3);
    if (s3 != seg_len && round_fill(s3) > round_fill(seg_len)) seg_len = s3;
  }

  std::vector<AttnItem> items;
  std::vector<MergeEntry> merges;
  int64_t n_partials = 0;
  if (paged) {
    // Item ranges follow a per-request grid of seg_len keys over the pool blocks; the
    // item of the first range also carries the fresh blocks (its second block range).
    const int64_t per_range = std::max<int64_t>(1, seg_len / kKeyAlign);
    for (int32_t ti = 0; ti < (int32_t)tiles.size(); ++ti) {
      const AttnTile &t = tiles[ti];
      const int32_t b = t.req;
      auto needed = [&](int64_t lo, int64_t hi) {  // blocks of [lo, hi) starting <= p_last
        int64_t n = 0;
        while (lo + n < hi && kblocks[(size_t)(lo + n) * 4 + 2] <= t.p_last) ++n;
        return n;
      };
      const int64_t n_fresh = needed(kb_fresh[b], kb_pool[b]);
      const int64_t n_pool = needed(kb_pool[b], kb_fresh[b + 1]);
      const int64_t n_ranges = std::max<int64_t>(1, (n_pool + per_range - 1) / per_range);
      for (int32_t g = 0; g < h_kv; ++g) {
        for (int64_t r = 0; r < n_ranges; ++r) {
          AttnItem it{};
          it.tile = ti;
          it.kv_head = g;
          const int64_t p0 = kb_pool[b] + r * per_range;
          const int64_t p1 = kb_pool[b] + std::min(n_pool, (r + 1) * per_range);
          // the pool range is the first range of every item (the one the last-round
          // cut shortens); the request's fresh blocks ride as the second range of the
          // first item
          if (r == 0) {
            it.key_begin = (int32_t)p0;
            it.key_end = (int32_t)std::max(p0, p1);
            it.pad0 = (int32_t)kb_fresh[b];
            it.pad1 = (int32_t)(kb_fresh[b] + n_fresh);
          } else {
            it.key_begin = (int32_t)p0;
            it.key_end = (int32_t)p1;
            it.pad0 = it.pad1 = (int32_t)p1;
          }
          items.push_back(it);
        }
      }
    }
  }
  for (int32_t ti = 0; !paged && ti < (int32_t)tiles.size(); ++ti) {
    const int64_t keys = (int64_t)tiles[ti].p_last + 1;
    const int64_t n_split = (keys + seg_len - 1) / seg_len;
    for (int32_t g = 0; g < h_kv; ++g) {
      for (int64_t s = 0; s < n_split; ++s) {
        AttnItem it{};
        it.tile = ti;
        it.kv_head = g;
        it.key_begin = (int32_t)(s * seg_len);
        it.key_end = (int32_t)std::min<int64_t>(keys, (s + 1) * seg_len);
        items.push_back(it);
      }
    }
  }
  // (split-KV slots and merge entries are assigned once the dispatch order is final)
  {
    // shorter pieces in each die's last round (keys, or key blocks for paged plans),
    // then the split-KV slots and merge entries follow the final item list (per (tile,
    // kv head): its items in key order, contiguous slots when there is more than one)
    const int64_t unit = paged ? kKeyAlign : 1;
    items = xcd_order(std::move(items), tiles, kXcd, kTailKeys / unit,
                      std::max<int64_t>(1, slots / kXcd), seg_len / unit, paged ? 1 : kKeyAlign);
    std::vector<std::vector<int32_t>> of(tiles.size() * (size_t)h_kv);
    for (int32_t i = 0; i < (int32_t)items.size(); ++i)
      of[(size_t)items[i].tile * h_kv + items[i].kv_head].push_back(i);
    merges.clear();
    n_partials = 0;
    for (size_t u = 0; u < of.size(); ++u) {
      auto &v = of[u];
      std::sort(v.begin(), v.end(),
                [&](int32_t a, int32_t b) { return items[a].key_begin < items[b].key_begin; });
      if (v.size() == 1) {
        items[v[0]].slot = -1;
      } else if (v.size() > 1) {
        for (size_t r = 0; r < v.size(); ++r) items[v[r]].slot = (int32_t)(n_partials + r);
        merges.push_back(MergeEntry{(int32_t)(u / h_kv), (int32_t)(u % h_kv),
                                    (int32_t)n_partials, (int32_t)v.size()});
        n_partials += (int64_t)v.size();
      }
    }
    if (n_partials > kMaxI32 / 2) return PIC_EINVAL;
  }

  // ---- decode items (paged plans): every pool chunk once, for all its uses ----
  // A decode step streams each pool chunk from HBM once and serves every request
  // chunk that reads it (up to PIC_DECODE_COLS / G uses per item); each request's fresh
  // rows (seams and queries) are further items.  Each (item, kv head) unit is a run of
  // PIC_DECODE_BLOCK-key blocks; the concatenated runs are cut into n_dec_wg equal
  // parts, one per resident workgroup, so every workgroup streams the same bytes.  The
  // part of a unit inside one workgroup's run is a piece; it leaves one record
  // (m, l, O of the G heads) per use, and the records of each (request, kv head) are
  // numbered contiguously for the merge.
  std::vector<DecItem> dec_items;
  std::vector<DecPiece> dec_pieces;
  std::vector<int32_t> dec_uses, dec_rec_ptr, dec_piece_recs, dec_wg_ptr;
  if (paged && group <= PIC_DECODE_COLS) {
    const int32_t per_item = PIC_DECODE_COLS / group;
    std::vector<std::pair<int32_t, int32_t>> by_id;  // (pool chunk id, global chunk index)
    for (int32_t c = 0; c < n_chunks; ++c)
      if (chunk_lens[c] > 0) by_id.push_back({chunk_ids[c], c});
    std::stable_sort(by_id.begin(), by_id.end(),
                     [](const std::pair<int32_t, int32_t> &a,
                        const std::pair<int32_t, int32_t> &b) { return a.first < b.first; });
    for (size_t i = 0; i < by_id.size();) {
      size_t j = i;
      while (j < by_id.size() && by_id[j].first == by_id[i].first) ++j;
      for (size_t u = i; u < j; u += per_item) {
        DecItem d{};
        d.src = by_id[i].first;
        d.n_keys = chunk_lens[by_id[i].second];
        d.use_begin = (int32_t)dec_uses.size();
        d.n_uses = (int32_t)std::min<size_t>(per_item, j - u);
        for (size_t v = u; v < u + (size_t)d.n_uses; ++v) dec_uses.push_back(by_id[v].second);
        dec_items.push_back(d);
      }
      i = j;
    }
    for (int32_t b = 0; b < n_req; ++b) {
      const int32_t r_b = req_row_ptr[b + 1] - req_row_ptr[b];
      if (r_b == 0) continue;
      dec_items.push_back(DecItem{-1 - b, r_b, (int32_t)dec_uses.size(), 1});
      dec_uses.push_back(-1 - b);
    }
    constexpr int32_t kB = PIC_DECODE_BLOCK;
    int64_t total = 0;  // blocks over all units
    for (const DecItem &d : dec_items) total += (int64_t)(d.n_keys + kB - 1) / kB * h_kv;
    if (total > kMaxI32 / 2) return PIC_EINVAL;
    const int64_t n_wg = std::min<int64_t>(total, (int64_t)n_cu * PIC_DECODE_WG_PER_CU);
    auto run_begin = [&](int64_t w) { return w * total / n_wg; };  // first block of run w
    // the request of each use (a pool use names its request chunk)
    std::vector<int32_t> chunk_req((size_t)n_chunks);
    for (int32_t b = 0; b < n_req; ++b)
      for (int32_t c = req_chunk_ptr[b]; c < req_chunk_ptr[b + 1]; ++c) chunk_req[c] = b;
    auto use_req = [&](int32_t use) { return use >= 0 ? chunk_req[use] : -1 - use; };
    std::vector<int64_t> n_recs((size_t)n_req * h_kv, 0);
    int64_t pos = 0, w = 0;
    dec_wg_ptr.push_back(0);
    for (size_t it = 0; it < dec_items.size(); ++it) {
      const DecItem &d = dec_items[it];
      const int64_t nb = (d.n_keys + kB - 1) / kB;
      for (int32_t g = 0; g < h_kv; ++g) {
        for (int64_t blk = 0; blk < nb;) {
          while (pos >= run_begin(w + 1)) {  // close run w
            dec_wg_ptr.push_back((int32_t)dec_pieces.size());
            ++w;
          }
          const int64_t take = std::min<int64_t>(nb - blk, run_begin(w + 1) - pos);
          DecPiece pc{};
          pc.item = (int32_t)it;
          pc.g = g;
          pc.t_begin = (int32_t)(blk * kB);
          pc.t_end = (int32_t)std::min<int64_t>(d.n_keys, (blk + take) * kB);
          pc.rec_off = (int32_t)dec_piece_recs.size();
          for (int32_t u = 0; u < d.n_uses; ++u) {  // record ids assigned below
            const int32_t b = use_req(dec_uses[d.use_begin + u]);
            dec_piece_recs.push_back(b * h_kv + g);
            ++n_recs[(size_t)b * h_kv + g];
          }
          dec_pieces.push_back(pc);
          blk += take;
          pos += take;
        }
      }
    }
    while ((int64_t)dec_wg_ptr.size() < n_wg + 1) dec_wg_ptr.push_back((int32_t)dec_pieces.size());
    dec_rec_ptr.assign((size_t)n_req * h_kv + 1, 0);
    for (size_t x = 0; x < n_recs.size(); ++x) dec_rec_ptr[x + 1] = dec_rec_ptr[x] + (int32_t)n_recs[x];
    if (dec_rec_ptr.back() > kMaxI32 / 2) return PIC_EINVAL;
    std::vector<int32_t> next(dec_rec_ptr.begin(), dec_rec_ptr.end() - 1);
    for (int32_t &r : dec_piece_recs) r = next[r]++;  // (request, kv head) -> record id
  }

  // ---- layout of the plan ----
  int64_t words = PIC_PLAN_HEADER_WORDS;
  auto place = [&words](int64_t n) {
    const int64_t at = words;
    words += round_up(n, 4);  // keep 16-byte alignment of every section
    return at;
  };
  const int64_t o_rcp = place(n_req + 1);
  const int64_t o_coff = place(n_chunks + n_req);
  const int64_t o_rtp = place(n_req + 1);
  const int64_t o_rrp = place(n_req + 1);
  const int64_t o_rows = place(nrows);
  const int64_t o_rtok = place(nrows);
  const int64_t o_rope = place((int64_t)rope.size() * 4);
  const int64_t o_tiles = place((int64_t)tiles.size() * 8);
  const int64_t o_items = place((int64_t)items.size() * 8);
  const int64_t o_merge = place((int64_t)merges.size() * 4);
  const int64_t o_segs = place((int64_t)segs.size());
  const int64_t o_kblocks = place((int64_t)kblocks.size());
  const int64_t o_dec_items = place((int64_t)dec_items.size() * 4);
  const int64_t o_dec_uses = place((int64_t)dec_uses.size());
  const int64_t o_dec_rec_ptr = place((int64_t)dec_rec_ptr.size());
  const int64_t o_dec_pieces = place((int64_t)dec_pieces.size() * 8);
  const int64_t o_dec_piece_recs = place((int64_t)dec_piece_recs.size());
  const int64_t o_dec_wg_ptr = place((int64_t)dec_wg_ptr.size());
  if (words > kMaxI32) return PIC_EINVAL;
  *plan_words = words;
  if (plan == nullptr) return PIC_OK;
  if (plan_cap < words) return PIC_ENOSPC;

  std::memset(plan, 0, sizeof(int32_t) * (size_t)words);
  int32_t *h = plan;
  h[PIC_H_MAGIC] = PIC_PLAN_MAGIC;
  h[PIC_H_WORDS] = (int32_t)words;
  h[PIC_H_N_REQ] = n_req;
  h[PIC_H_N_CHUNKS] = n_chunks;
  h[PIC_H_N_ROWS] = (int32_t)nrows;
  h[PIC_H_N_TOKENS] = (int32_t)tok;
  h[PIC_H_K] = k;
  h[PIC_H_POS_BASE] = pos_base;
  h[PIC_H_H_Q] = h_q;
  h[PIC_H_H_KV] = h_kv;
  h[PIC_H_TILE_ROWS] = tile_rows;
  h[PIC_H_N_ROPE_TILES] = (int32_t)rope.size();
  h[PIC_H_N_ATTN_TILES] = (int32_t)tiles.size();
  h[PIC_H_N_ATTN_ITEMS] = (int32_t)items.size();
  h[PIC_H_N_MERGE] = (int32_t)merges.size();
  h[PIC_H_N_PARTIALS] = (int32_t)n_partials;
  h[PIC_H_MAX_TOKENS] = (int32_t)max_tokens;
  h[PIC_H_O_REQ_CHUNK_PTR] = (int32_t)o_rcp;
  h[PIC_H_O_CHUNK_OFF] = (int32_t)o_coff;
  h[PIC_H_O_REQ_TOK_PTR] = (int32_t)o_rtp;
  h[PIC_H_O_REQ_ROW_PTR] = (int32_t)o_rrp;
  h[PIC_H_O_ROWS] = (int32_t)o_rows;
  h[PIC_H_O_ROW_TOK] = (int32_t)o_rtok;
  h[PIC_H_O_ROPE_TILES] = (int32_t)o_rope;
  h[PIC_H_O_ATTN_TILES] = (int32_t)o_tiles;
  h[PIC_H_O_ATTN_ITEMS] = (int32_t)o_items;
  h[PIC_H_O_MERGE] = (int32_t)o_merge;
  h[PIC_H_PAGED] = paged ? 1 : 0;
  h[PIC_H_O_SEGS] = (int32_t)o_segs;
  h[PIC_H_N_KBLOCKS] = (int32_t)(kblocks.size() / 4);
  h[PIC_H_O_KBLOCKS] = (int32_t)o_kblocks;
  h[PIC_H_N_DEC_ITEMS] = (int32_t)dec_items.size();
  h[PIC_H_O_DEC_ITEMS] = (int32_t)o_dec_items;
  h[PIC_H_N_DEC_USES] = (int32_t)dec_uses.size();
  h[PIC_H_O_DEC_USES] = (int32_t)o_dec_uses;
  h[PIC_H_N_DEC_RECS] = dec_rec_ptr.empty() ? 0 : dec_rec_ptr.back();
  h[PIC_H_O_DEC_REC_PTR] = (int32_t)o_dec_rec_ptr;
  h[PIC_H_N_DEC_PIECES] = (int32_t)dec_pieces.size();
  h[PIC_H_O_DEC_PIECES] = (int32_t)o_dec_pieces;
  h[PIC_H_O_DEC_PIECE_RECS] = (int32_t)o_dec_piece_recs;
  h[PIC_H_N_DEC_WG] = dec_wg_ptr.empty() ? 0 : (int32_t)dec_wg_ptr.size() - 1;
  h[PIC_H_O_DEC_WG_PTR] = (int32_t)o_dec_wg_ptr;
  if (n_req > 0) std::memcpy(h + o_rcp, req_chunk_ptr, sizeof(int32_t) * (n_req + 1));
  else h[o_rcp] = 0;
  if (!chunk_off.empty()) std::memcpy(h + o_coff, chunk_off.data(), sizeof(int32_t) * chunk_off.size());
  std::memcpy(h + o_rtp, req_tok_ptr.data(), sizeof(int32_t) * req_tok_ptr.size());
  std::memcpy(h + o_rrp, req_row_ptr.data(), sizeof(int32_t) * req_row_ptr.size());
  if (nrows) {
    std::memcpy(h + o_rows, rows.data(), sizeof(int32_t) * nrows);
    std::memcpy(h + o_rtok, row_tok.data(), sizeof(int32_t) * nrows);
  }
  if (!rope.empty()) std::memcpy(h + o_rope, rope.data(), sizeof(RopeTile) * rope.size());
  if (!tiles.empty()) std::memcpy(h + o_tiles, tiles.data(), sizeof(AttnTile) * tiles.size());
  if (!items.empty()) std::memcpy(h + o_items, items.data(), sizeof(AttnItem) * items.size());
  if (!merges.empty()) std::memcpy(h + o_merge, merges.data(), sizeof(MergeEntry) * merges.size());
  if (!segs.empty()) std::memcpy(h + o_segs, segs.data(), sizeof(int32_t) * segs.size());
  if (!kblocks.empty()) std::memcpy(h + o_kblocks, kblocks.data(), sizeof(int32_t) * kblocks.size());
  if (!dec_items.empty())
    std::memcpy(h + o_dec_items, dec_items.data(), sizeof(DecItem) * dec_items.size());
  if (!dec_uses.empty())
    std::memcpy(h + o_dec_uses, dec_uses.data(), sizeof(int32_t) * dec_uses.size());
  if (!dec_rec_ptr.empty())
    std::memcpy(h + o_dec_rec_ptr, dec_rec_ptr.data(), sizeof(int32_t) * dec_rec_ptr.size());
  if (!dec_pieces.empty())
    std::memcpy(h + o_dec_pieces, dec_pieces.data(), sizeof(DecPiece) * dec_pieces.size());
  if (!dec_piece_recs.empty())
    std::memcpy(h + o_dec_piece_recs, dec_piece_recs.data(), sizeof(int32_t) * dec_piece_recs.size());
  if (!dec_wg_ptr.empty())
    std::memcpy(h + o_dec_wg_ptr, dec_wg_ptr.data(), sizeof(int32_t) * dec_wg_ptr.size());
  return PIC_OK;
}

extern "C" const char *pic_strerror(int status) {
  switch (status) {
    case PIC_OK: return "ok";
    case PIC_EINVAL: return "invalid argument";
    case PIC_ENOSPC: return "output buffer too small";
    case PIC_EUNSUPPORTED: return "unsupported configuration";
    case PIC_EDEVICE: return "HIP runtime error";
    default: return "unknown status";
  }
}
