// Host-side work partitioning for the fused varlen paged-attention launch.
//
// A step's rows fall into two kinds ("11.2 连续批处理与 PagedAttention",
// section 11.2.2: prefill rows and decode rows share one packed step):
//  * q_len > 1 (prefill / chunked prefill, causal offset = cached prefix:
//    "Continuous Batching 深入实现", section "一个 chunked prefill 请求怎么组织
//    attention"): tiles of query positions x the kv head's query heads.  A
//    wide tile (256 columns: 256/G positions x G heads) is computed by a
//    whole workgroup of eight wavefronts sharing K/V through LDS.  The
//    launch has a fixed set of persistent workgroups; the wide tiles are
//    dealt to them in pairs of equal cost (tiles j and n - 1 - j of one
//    sequence and kv head), longest first, each to the least loaded
//    workgroup (with the estimated time of its narrow share as its starting
//    load), tiles of kv head h to the workgroups on XCD h % 8, so a head's
//    keys and values are fetched from HBM into one L2.
//  * Decode rows and the short tails of prefill rows: narrow (<= 16 column)
//    units (tile, kv head), each a stream of 32-key chunks.  All chunks of all
//    units are dealt out in equal contiguous shares to a fixed number of
//    wavefronts ("stream-K" style): wavefront w takes chunks
//    [w*C/W, (w+1)*C/W) of the concatenated units, so a long context is cut
//    across several wavefronts and several short ones share one, and every
//    wavefront streams the same number of bytes.  A unit cut into several
//    segments writes partial results that a merge launch combines.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "pkv_internal.h"

namespace {

using pkv::Item;
using pkv::Merge;

// six per CU of 256: measured on MI355X decode steps, 3-4% faster than one
// per SIMD (1024) or two per SIMD (2048)
constexpr int kDefaultNarrowWaves = 1536;
constexpr int kDefaultMinWaveKeys = 512;
constexpr int kDefaultWorkgroups = 256;    // one per CU on an MI355X
constexpr int kXcds = 8;                   // consecutive workgroups go to the XCDs in turn

// Cost model of the launch with wide tiles, in CU-microseconds (measured on
// MI355X): a wide tile costs ~0.8 us per 32-key chunk plus ~3 us for its
// start, first and last steps and epilogue (per-tile timestamps: 0.77-0.83
// us per chunk on long tiles, ~2.2 us of setup and epilogue; against 0.9 +
// 2.0, trace step 20 191 -> 186 us, step 0 111 -> 110 us, the whole trace
// within its noise).
// The narrow streams (32-key chunks of 16 KiB of K and V) move ~5 GB/s per
// wavefront until their sum nears the HBM rate they can reach, and bend
// over smoothly there (timed per workgroup on trace steps: 1088 wavefronts
// 5.5 TB/s, 1216 5.8, 1344 and 1664 6.1); a 12-norm of the two bounds
// follows that bend.  The ceiling is taken at 7.0 TB/s since the append's
// and the outputs' writes no longer land under the streams (a sweep of
// 5.7-8.5 TB/s over the 200-iteration trace: 7.0 the fastest, ~1% ahead of
// 6.1, within the runs' noise elsewhere).
constexpr double kWideChunkUs = 0.8;
constexpr double kWideTileUs = 3.0;
constexpr double kNarrowWaveBytesPerUs = 5.0e3;
constexpr double kNarrowHbmBytesPerUs = 7.0e6;
constexpr double kChunkBytes = 16384.0;

// time of the narrow shares when W wavefronts (eight per workgroup) share
// total_chunks
double narrow_share_us(int64_t total_chunks, int64_t W) {
  const double waves = (double)W * kNarrowWaveBytesPerUs;
  const double rate = waves / std::pow(1.0 + std::pow(waves / kNarrowHbmBytesPerUs, 12.0), 1.0 / 12.0);
  const double longest = (double)((total_chunks + W - 1) / W) * kChunkBytes / kNarrowWaveBytesPerUs;
  return std::max(longest, (double)total_chunks * kChunkBytes / rate);
}

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

  const int min_wave_keys = (opts && opts->min_wave_keys > 0) ? opts->min_wave_keys : kDefaultMinWaveKeys;
  const int wide_opt = opts ? opts->wide_tiles : -1;
  const int narrow_pos = pkv::kTileCols / G;  // positions per narrow tile
  const int wide_pos = pkv::kWideCols / G;    // positions per wide tile

  // ---- tiles: (seq, t0, np, pos0, keys)
  struct Tile { int32_t seq, t0, np, pos0, keys; bool wide; };
  std::vector<Tile> wide_tiles, narrow_tiles;
  int64_t kv_keys = 0, pairs = 0;
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
      (wide ? wide_tiles : narrow_tiles).push_back(t);
      j += np;
    }
  }

  // ---- the append's row groups (consecutive packed rows, at most 16): the
  // rows a sequence appends into one block (a run) are never cut, so every
  // block this step fills is written by one workgroup in whole lines;
  // runs pack into groups in packed order (decode rows 16 to a group)
  std::vector<int32_t> app;  // (first row, rows) pairs
  {
    int32_t g0 = 0, gn = 0;
    for (int s = 0; s < num_seqs; ++s) {
      const int ql = h_cu[s + 1] - h_cu[s];
      const int c = h_seq_lens[s] - ql;
      for (int j = 0; j < ql;) {
        const int run = std::min(ql - j, pkv::kBlock - (c + j) % pkv::kBlock);
        if (gn + run > pkv::kBlock) {
          app.push_back(g0);
          app.push_back(gn);
          gn = 0;
        }
        if (gn == 0) g0 = h_cu[s] + j;
        gn += run;
        j += run;
      }
    }
    if (gn > 0) {
      app.push_back(g0);
      app.push_back(gn);
    }
  }

  std::vector<Item> items;
  std::vector<Merge> merges;
  std::vector<int32_t> wave_off;
  int64_t part_cols = 0;

  // wide tiles: one item per (tile, kv head); dealt to workgroups below
  for (const Tile &t : wide_tiles)
    for (int h = 0; h < Hkv; ++h) items.push_back(Item{t.seq, h, t.t0, t.np, t.pos0, 0, t.keys, -1});
  const int n_wide = (int)items.size();

  // narrow units (tile, kv head) in order; chunk counts
  const int64_t n_units = (int64_t)narrow_tiles.size() * Hkv;
  int64_t total_chunks = 0;
  for (const Tile &t : narrow_tiles) total_chunks += (int64_t)Hkv * ((t.keys + 31) / 32);

  // Narrow wavefronts.  Alone they are one per SIMD.  Beside wide tiles
  // they travel in rows of eight workgroups of eight wavefronts, whose CUs
  // afterwards join the wide tiles; the rows get the share of the chip the
  // narrow work is estimated to need.
  const int max_wg = (opts && opts->workgroups > 0) ? opts->workgroups : kDefaultWorkgroups;
  if (max_wg % kXcds != 0 || max_wg > kDefaultWorkgroups) return PKV_EINVAL;
  const int max_rows = max_wg / kXcds;
  double wide_us = 0;
  for (int i = 0; i < n_wide; ++i) wide_us += kWideChunkUs * ((items[i].k1 + 31) / 32) + kWideTileUs;
  int narrow_rows = 0;
  int want_waves = kDefaultNarrowWaves;
  if (n_wide > 0 && total_chunks > 0) {
    // the fewest rows with the least estimated launch time: the narrow rows
    // take their wide tiles after their shares, the grid shares the rest
    double best = 0;
    for (int r = 1; r <= max_rows; ++r) {
      const double share = narrow_share_us(total_chunks, 64 * (int64_t)r);
      const double t = std::max(share, (wide_us + 8.0 * r * share) / (8.0 * max_rows));
      if (r == 1 || t < best * (1.0 - 1e-6)) {
        best = t;
        narrow_rows = r;
      }
    }
    want_waves = 64 * narrow_rows;
  }
  if (opts && opts->narrow_waves > 0) want_waves = opts->narrow_waves;
  if (n_wide > 0) want_waves = std::min(want_waves, 64 * max_rows);
  int W = 0;
  int wave_keys = 0;
  if (total_chunks > 0) {
    const int64_t by_size = (total_chunks * 32 + min_wave_keys - 1) / min_wave_keys;
    W = (int)std::max<int64_t>(1, std::min<int64_t>(want_waves, by_size));
    wave_keys = (int)((total_chunks + W - 1) / W * 32);
    if (n_wide > 0) narrow_rows = (W + 63) / 64;
  }

  // Persistent workgroups and their wide-tile lists.
  int n_wg = 0;
  std::vector<int32_t> wg_list;
  if (n_wide > 0) {
    const int rows = std::min(max_rows, narrow_rows + (n_wide + kXcds - 1) / kXcds);
    n_wg = rows * kXcds;
    // starting load: the narrow share of a narrow workgroup (eight wavefronts)
    const double share_us = W > 0 ? narrow_share_us(total_chunks, W) : 0.0;
    std::vector<double> load(n_wg, 0.0);
    for (int j = 0; j < n_wg; ++j) {
      if (pkv::mixed_row(rows, narrow_rows, j / kXcds).narrow) load[j] = share_us;
    }
    // tiles of kv head h go to XCD h % 8 when every XCD gets whole heads
    const bool affine = Hkv % kXcds == 0;
    // Dealing units: the n tiles of one (sequence, kv head) cost a + b j
    // (causal: each takes 256/G more keys than the one before), so tiles j
    // and n - 1 - j always sum to the same cost; they go to a workgroup as
    // a pair, the longer first.  Equal-cost units keep their order
    // (sequence, kv head, j), so the workgroups of an XCD take a prompt's
    // pairs side by side and stream its keys and values nearly in step
    // through one L2, one or two prompts at a time (dealt one tile at a
    // time, longest first, the XCD's L2 held every prompt of its kv head at
    // once and refetched their keys: 1.29 x the algorithmic bytes on four
    // fresh 2048-token prompts).
    // Only with at least two tiles per workgroup: with fewer, every tile of
    // a head runs at once on its XCD (sharing its keys through L2 anyway)
    // and pairs would leave workgroups idle (a 2048-token chunk after a
    // 30,720-token prefix: 32 tiles per kv head on 32 CUs, 894 -> 1518 us
    // as pairs).  Costs are compared as whole chunk and tile counts, so
    // equal pairs tie exactly and keep their order.
    const bool deal_pairs = (int64_t)n_wide >= 2 * (int64_t)n_wg;
    struct Unit { int a, b, chunks, tiles; double c; };  // items (b < 0: none), cost
    auto chunks = [&](int i) { return (items[i].k1 + 31) / 32; };
    std::vector<Unit> units;
    for (int t0 = 0; t0 < (int)wide_tiles.size();) {
      int t1 = t0;
      while (t1 < (int)wide_tiles.size() && wide_tiles[t1].seq == wide_tiles[t0].seq) ++t1;
      const int n = t1 - t0;
      for (int h = 0; h < Hkv; ++h) {
        for (int k = 0; k < (n + 1) / 2; ++k) {
          const int lo = (t0 + k) * Hkv + h, hi = (t1 - 1 - k) * Hkv + h;
          if (lo == hi || !deal_pairs) {
            units.push_back(Unit{hi, -1, chunks(hi), 1, kWideChunkUs * chunks(hi) + kWideTileUs});
            if (lo != hi) units.push_back(Unit{lo, -1, chunks(lo), 1, kWideChunkUs * chunks(lo) + kWideTileUs});
          } else {
            const int c = chunks(hi) + chunks(lo);
            units.push_back(Unit{hi, lo, c, 2, kWideChunkUs * c + 2 * kWideTileUs});
          }
        }
      }
      t0 = t1;
    }
    std::stable_sort(units.begin(), units.end(), [](const Unit &x, const Unit &y) {
      return x.chunks != y.chunks ? x.chunks > y.chunks : x.tiles > y.tiles;
    });
    std::vector<std::vector<int>> lists(n_wg);
    for (const Unit &u : units) {
      int best = -1;
      for (int j = affine ? items[u.a].kvh % kXcds : 0; j < n_wg; j += affine ? kXcds : 1)
        if (best < 0 || load[j] < load[best]) best = j;
      load[best] += u.c;
      lists[best].push_back(u.a);
      if (u.b >= 0) lists[best].push_back(u.b);
    }
    std::vector<Item> wide(items.begin(), items.begin() + n_wide);
    wg_list.push_back(0);
    int k = 0;
    for (int j = 0; j < n_wg; ++j) {
      for (int i : lists[j]) items[k++] = wide[i];
      wg_list.push_back(k);
    }
  }
  auto unit_tile = [&](int64_t u) -> const Tile & { return narrow_tiles[u / Hkv]; };
  auto unit_chunks = [&](int64_t u) -> int { return (unit_tile(u).keys + 31) / 32; };
  // pass 1: segments per unit (chunk boundaries of the wave shares)
  std::vector<int32_t> nseg(n_units, 0);
  {
    int64_t u = 0, done = 0;  // chunks of unit u already dealt
    for (int w = 0; w < W; ++w) {
      int64_t room = total_chunks / W + (w < total_chunks % W ? 1 : 0);
      while (room > 0 && u < n_units) {
        const int64_t take = std::min<int64_t>(room, unit_chunks(u) - done);
        ++nseg[u];
        done += take;
        room -= take;
        if (done == unit_chunks(u)) { ++u; done = 0; }
      }
    }
  }
  // partial columns and merge entries for cut units
  std::vector<int64_t> part_base(n_units, -1);
  for (int64_t u = 0; u < n_units; ++u) {
    if (nseg[u] <= 1) continue;
    const Tile &t = unit_tile(u);
    const int h = (int)(u % Hkv);
    const int ncols = t.np * G;
    part_base[u] = part_cols;
    part_cols += (int64_t)nseg[u] * ncols;
    for (int col = 0; col < ncols; ++col) {
      const int pc = col >> log2G, ho = col & (G - 1);
      merges.push_back(Merge{(t.t0 + pc) * Hq + h * G + ho, (int32_t)(part_base[u] + col), nseg[u], ncols});
    }
  }
  // pass 2: emit each wave's segments as items, in wave order
  {
    int64_t u = 0, done = 0;
    int seg = 0;
    wave_off.push_back(0);
    for (int w = 0; w < W; ++w) {
      int64_t room = total_chunks / W + (w < total_chunks % W ? 1 : 0);
      while (room > 0 && u < n_units) {
        const Tile &t = unit_tile(u);
        const int64_t take = std::min<int64_t>(room, unit_chunks(u) - done);
        const int k0 = (int)(done * 32);
        const int k1 = (int)std::min<int64_t>(t.keys, (done + take) * 32);
        const int32_t part = part_base[u] < 0 ? -1 : (int32_t)(part_base[u] + (int64_t)seg * t.np * G);
        items.push_back(Item{t.seq, (int32_t)(u % Hkv), t.t0, t.np, t.pos0, k0, k1, part});
        ++seg;
        done += take;
        room -= take;
        if (done == unit_chunks(u)) { ++u; done = 0; seg = 0; }
      }
      wave_off.push_back((int32_t)(items.size() - n_wide));
    }
  }
  if (part_cols > INT32_MAX || (int64_t)items.size() > INT32_MAX / 2) return PKV_ERANGE;

  // ---- sizes
  plan->num_seqs = num_seqs;
  plan->num_rows = num_rows;
  plan->num_q_heads = Hq;
  plan->num_kv_heads = Hkv;
  plan->head_dim = head_dim;
  plan->num_items = (int32_t)items.size();
  plan->num_wide_items = n_wide;
  plan->narrow_rows = narrow_rows;
  plan->num_waves = W;
  plan->num_merge = (int32_t)merges.size();
  plan->num_part_cols = (int32_t)part_cols;
  plan->wave_keys = wave_keys;
  plan->kv_keys = kv_keys;
  plan->visible_pairs = pairs;
  plan->num_workgroups = n_wg;
  plan->num_append_groups = (int32_t)(app.size() / 2);
  const size_t items_b = pkv::align_up(items.size() * sizeof(Item));
  const size_t waves_b = pkv::align_up(wave_off.size() * sizeof(int32_t));
  const size_t merge_b = pkv::align_up(merges.size() * sizeof(Merge));
  const size_t wg_b = pkv::align_up(wg_list.size() * sizeof(int32_t));
  const size_t app_b = pkv::align_up(app.size() * sizeof(int32_t));
  // a zero (block, head) tile: loads of table entries outside [0, num_blocks)
  // are pointed at it
  const size_t zero_b = (size_t)pkv::kBlock * pkv::kHeadDim * 2;
  plan->items_off = 0;
  plan->waves_off = (int64_t)items_b;
  plan->merge_off = (int64_t)(items_b + waves_b);
  plan->wg_off = (int64_t)(items_b + waves_b + merge_b);
  plan->append_off = plan->wg_off + (int64_t)wg_b;
  plan->zero_off = plan->append_off + (int64_t)app_b;
  plan->ml_off = plan->zero_off + (int64_t)zero_b;
  plan->o_off = plan->ml_off + (int64_t)pkv::align_up((size_t)part_cols * 8);
  plan->ws_bytes = (size_t)plan->o_off + (size_t)part_cols * pkv::kHeadDim * 4;
  plan->host_bytes = items_b + waves_b + merge_b + wg_b + app_b + zero_b;
  if (!h_staging) return PKV_OK;  // size query
  if (h_staging_bytes < plan->host_bytes) return PKV_EWORKSPACE;
  if (ws && ws_bytes < plan->ws_bytes) return PKV_EWORKSPACE;

  char *hs = static_cast<char *>(h_staging);
  if (!items.empty()) std::memcpy(hs, items.data(), items.size() * sizeof(Item));
  if (!wave_off.empty()) std::memcpy(hs + items_b, wave_off.data(), wave_off.size() * sizeof(int32_t));
  if (!merges.empty()) std::memcpy(hs + items_b + waves_b, merges.data(), merges.size() * sizeof(Merge));
  if (!wg_list.empty()) std::memcpy(hs + plan->wg_off, wg_list.data(), wg_list.size() * sizeof(int32_t));
  if (!app.empty()) std::memcpy(hs + plan->append_off, app.data(), app.size() * sizeof(int32_t));
  std::memset(hs + plan->zero_off, 0, zero_b);
  if (ws && plan->host_bytes > 0) {
    hipError_t e = hipMemcpyAsync(ws, h_staging, plan->host_bytes, hipMemcpyHostToDevice,
                                  static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return PKV_EHIP;
  }
  return PKV_OK;
}
