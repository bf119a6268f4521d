// Host-side work partitioning for the fused varlen paged-attention launch.
//
// A step's sequences fall into two kinds ("11.2 连续批处理与 PagedAttention",
// section 11.2.2: prefill rows and decode rows share one packed step):
//  * q_len == 1 (decode) and short q_len tiles: one item per (tile, kv head,
//    key split).  Long contexts are split over the key axis so that the
//    launch has enough items to fill 256 CUs even when the step holds few
//    sequences; the splits are merged afterwards.
//  * q_len > 1 (prefill / chunked prefill, causal offset = cached prefix:
//    "Continuous Batching 深入实现", section "一个 chunked prefill 请求怎么组织
//    attention"): tiles of query positions x the kv head's query heads; a wide
//    tile holds 64 columns (64 / G positions), a narrow one 16.
// Items are ordered wide first, then by decreasing key count, so the longest
// work starts first and short items fill the tail.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "pkv_internal.h"

namespace {

using pkv::Item;
using pkv::Merge;

constexpr int kDefaultTargetItems = 8192;
constexpr int kDefaultMinSplit = 256;

int round_up32(int64_t x) { return (int)((x + 31) / 32 * 32); }

}  // namespace

extern "C" int pkv_plan(const int32_t *h_cu, const int32_t *h_seq_lens,
                        int32_t num_seqs, int32_t num_rows, int32_t Hq,
                        int32_t Hkv, int32_t head_dim,
                        const int32_t *h_bt, int32_t bt_stride,
                        int64_t num_blocks, const pkv_plan_options_t *opts,
                        void *h_staging, size_t h_staging_bytes, void *ws,
                        size_t ws_bytes, pkv_plan_t *plan,
                        pkv_stream_t stream) {
  if (!plan || num_seqs < 0 || num_rows < 0) return PKV_EINVAL;
  if (num_seqs > 0 && (!h_cu || !h_seq_lens)) return PKV_EINVAL;
  std::memset(plan, 0, sizeof(*plan));
  if (head_dim != pkv::kHeadDim) return PKV_EUNSUPPORTED;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return PKV_EUNSUPPORTED;
  const int G = Hq / Hkv;
  const int log2G = pkv::log2_exact(G);
  if (log2G < 0 || G > 16) return PKV_EUNSUPPORTED;

  // ---- validate the host copies of the metadata
  if (num_seqs == 0 ? num_rows != 0 : h_cu[0] != 0) return PKV_EINVAL;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t ql = (int64_t)h_cu[s + 1] - h_cu[s];
    if (ql < 0) return PKV_EINVAL;
    if (h_seq_lens[s] < ql) return PKV_EINVAL;
  }
  if (num_seqs > 0 && h_cu[num_seqs] != num_rows) return PKV_EINVAL;
  if (h_bt) {
    if (bt_stride <= 0 || num_blocks <= 0) return PKV_EINVAL;
    for (int s = 0; s < num_seqs; ++s) {
      if (h_cu[s + 1] == h_cu[s]) continue;
      const int64_t need = ((int64_t)h_seq_lens[s] + pkv::kBlock - 1) / pkv::kBlock;
      if (need > bt_stride) return PKV_ERANGE;
      const int32_t *row = h_bt + (int64_t)s * bt_stride;
      for (int64_t i = 0; i < need; ++i)
        if (row[i] < 0 || row[i] >= num_blocks) return PKV_ERANGE;
    }
  }

  const int target = (opts && opts->target_items > 0) ? opts->target_items : kDefaultTargetItems;
  int min_split = (opts && opts->min_split_keys > 0) ? opts->min_split_keys : kDefaultMinSplit;
  min_split = round_up32(std::max(32, min_split));
  const int wide_opt = opts ? opts->wide_tiles : -1;
  const int narrow_pos = pkv::kTileCols / G;  // positions per narrow tile
  const int wide_pos = pkv::kWideCols / G;    // positions per wide tile

  // ---- tiles: (seq, t0, np, pos0, keys) per kv head
  struct Tile { int32_t seq, t0, np, pos0, keys; bool wide; };
  std::vector<Tile> tiles;
  int64_t narrow_keys = 0, kv_keys = 0, pairs = 0;
  bool any_prefill = false;
  for (int s = 0; s < num_seqs; ++s) if (h_cu[s + 1] - h_cu[s] > 1) any_prefill = true;
  const bool use_wide = wide_opt == 1 || (wide_opt < 0 && any_prefill);
  for (int s = 0; s < num_seqs; ++s) {
    const int ql = h_cu[s + 1] - h_cu[s];
    if (ql == 0) continue;
    const int c = h_seq_lens[s] - ql;
    kv_keys += h_seq_lens[s];
    pairs += (int64_t)ql * c + (int64_t)ql * (ql + 1) / 2;
    int j = 0;
    while (j < ql) {
      const int left = ql - j;
      const bool wide = use_wide && left > narrow_pos;
      const int np = std::min(left, wide ? wide_pos : narrow_pos);
      Tile t{s, h_cu[s] + j, np, c + j, c + j + np, wide};
      if (!wide) narrow_keys += t.keys;
      tiles.push_back(t);
      j += np;
    }
  }
  // key-split length for narrow tiles
  int split = round_up32((narrow_keys * Hkv + target - 1) / std::max(1, target));
  split = std::max(split, min_split);

  std::vector<Item> items;
  std::vector<Merge> merges;
  int64_t part_cols = 0;
  int n_wide = 0;
  for (const Tile &t : tiles) {
    const int ncols = t.np * G;
    const int nsplit = t.wide ? 1 : (int)((t.keys + split - 1) / split);
    for (int h = 0; h < Hkv; ++h) {
      int64_t base = -1;
      if (nsplit > 1) {
        base = part_cols;
        part_cols += (int64_t)nsplit * ncols;
        for (int col = 0; col < ncols; ++col) {
          const int pc = col >> log2G, ho = col & (G - 1);
          merges.push_back(Merge{(t.t0 + pc) * Hq + h * G + ho, (int32_t)(base + col), nsplit, ncols});
        }
      }
      for (int k = 0; k < nsplit; ++k) {
        const int k0 = k * split;
        const int k1 = k + 1 == nsplit ? t.keys : k0 + split;
        items.push_back(Item{t.seq, h, t.t0, t.np, t.pos0, k0, k1,
                             nsplit > 1 ? (int32_t)(base + (int64_t)k * ncols) : -1});
      }
      if (t.wide) ++n_wide;
    }
  }
  if (part_cols > INT32_MAX || (int64_t)items.size() > INT32_MAX / 2) return PKV_ERANGE;
  // wide items first, then longest first (stable: equal lengths keep order)
  std::stable_sort(items.begin(), items.end(), [&](const Item &a, const Item &b) {
    const bool wa = a.np * G > pkv::kTileCols, wb = b.np * G > pkv::kTileCols;
    if (wa != wb) return wa;
    return (a.k1 - a.k0) > (b.k1 - b.k0);
  });

  // ---- sizes
  plan->num_seqs = num_seqs;
  plan->num_rows = num_rows;
  plan->num_q_heads = Hq;
  plan->num_kv_heads = Hkv;
  plan->head_dim = head_dim;
  plan->num_items = (int32_t)items.size();
  plan->num_wide_items = n_wide;
  plan->num_merge = (int32_t)merges.size();
  plan->num_part_cols = (int32_t)part_cols;
  plan->split_keys = split;
  plan->kv_keys = kv_keys;
  plan->visible_pairs = pairs;
  const size_t items_b = pkv::align_up(items.size() * sizeof(Item));
  const size_t merge_b = pkv::align_up(merges.size() * sizeof(Merge));
  plan->items_off = 0;
  plan->merge_off = (int64_t)items_b;
  plan->ml_off = (int64_t)(items_b + merge_b);
  plan->o_off = plan->ml_off + (int64_t)pkv::align_up((size_t)part_cols * 8);
  plan->ws_bytes = (size_t)plan->o_off + (size_t)part_cols * pkv::kHeadDim * 4;
  plan->host_bytes = items_b + merge_b;
  if (!h_staging) return PKV_OK;  // size query
  if (h_staging_bytes < plan->host_bytes) return PKV_EWORKSPACE;
  if (ws && ws_bytes < plan->ws_bytes) return PKV_EWORKSPACE;

  char *hs = static_cast<char *>(h_staging);
  if (!items.empty()) std::memcpy(hs, items.data(), items.size() * sizeof(Item));
  if (!merges.empty()) std::memcpy(hs + items_b, merges.data(), merges.size() * sizeof(Merge));
  if (ws && plan->host_bytes > 0) {
    hipError_t e = hipMemcpyAsync(ws, h_staging, plan->host_bytes, hipMemcpyHostToDevice,
                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return PKV_EHIP;
  }
  return PKV_OK;
}
