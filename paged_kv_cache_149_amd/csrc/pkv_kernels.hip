// HIP kernels for one packed, ragged attention step over a paged KV cache,
// written for CDNA4 (gfx950, wave64, bf16 MFMA).
//
//   slot_mapping_kernel     slot translation b*16 + p%16
//                           ("连续批处理与 PagedAttention 原理", "block table 与地址映射")
//   append_kernel           bit copy of the step's new K/V rows into their slots
//                           (optionally translating the slots first)
//   attention_kernel        narrow items only (decode rows, short tiles)
//   attention_mixed_kernel  persistent workgroups walking lists of wide
//                           prefill tiles (eight wavefronts sharing K/V
//                           through LDS), some first walking narrow items
//   merge_kernel            log-sum-exp merge of key-split partial results
//
// Attention: a tile of query columns (positions x the GQA group's query
// heads, all reading the same kv head) against a key range of one sequence,
// 32 keys (two paged blocks) per step:
//   S^T = K Q^T  (v_mfma_f32_16x16x32_bf16, M = keys, N = columns, K = dims)
//   softmax per column in the base-2 domain, fp32
//   O^T += V^T P^T (same MFMA, M = dims, N = columns, K = keys)
// Operand layouts of the 16x16x32 MFMA (lane l, r = l % 16, g = l / 16):
//   A[m][k]: lane holds A[r][8g .. 8g+7];  B[k][n]: lane holds B[8g .. 8g+7][r]
//   C[m][n]: lane holds C[4g .. 4g+3][r]
// Keys are assigned to the rows of the two S^T tiles so that lane group g's
// eight C values are keys 8g .. 8g+7 of the step, exactly the slots it needs
// as the B operand (P^T) of the P.V product.  The V tile of a block holds
// its tokens in two halves of 8, each dimension-major (8 tokens contiguous
// per dimension), so the V^T A operand is one 16-byte load per lane; K tiles hold 32-dimension groups,
// each token-major, so the K A operand is one 16-byte load per lane per 32
// dimensions and every load reads whole cache lines.  Narrow items load
// their operands straight from HBM in MFMA layout; wide tiles stage each
// chunk once per workgroup in LDS, in the same layout.
#include <hip/hip_runtime.h>
#include <type_traits>

#include <algorithm>
#include <cfloat>
#include <mutex>

#include "pkv_internal.h"

namespace {

using pkv::Item;
using pkv::Merge;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int D = pkv::kHeadDim;
constexpr int TILE = pkv::kBlock * pkv::kHeadDim;  // elements of a (block, head) tile
// K tiles hold the dimensions in groups of 32, each group token-major: a
// 16-byte load per lane over 16 keys x 32 dimensions reads whole cache
// lines (one 32-dimension MFMA step of 16 keys is 1 KiB contiguous).
constexpr int kKGroup = 32;
constexpr int kKGroupElems = pkv::kBlock * kKGroup;
constexpr int kXcdCount = 8;  // XCDs of an MI355X; consecutive workgroups go to them in turn
// V tiles hold the block's tokens in two halves of 8, each half
// dimension-major: element (o, d) at (o / 8) * 8 * 128 + d * 8 + o % 8, so a
// lane's V^T operand (8 consecutive keys of one dimension) is one 16-byte
// load, and a row appended alone touches 64 of the tile's 32-byte sectors
// (two dimensions per sector) rather than 128.
constexpr int kVHalf = 8;                       // tokens per half
constexpr int kVHalfElems = kVHalf * pkv::kHeadDim;  // elements per half (1024)

__device__ inline float neg_inf() { return -__builtin_huge_valf(); }

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ inline u32x4 load16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Streaming load of cache data that is read once per launch: the
// non-temporal hint keeps it from displacing reusable lines.
__device__ inline u32x4 load16_stream(const uint16_t *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Wave-uniform read-only load through the scalar data cache (s_load).
typedef const __attribute__((address_space(4))) int32_t const_i32;
__device__ inline int32_t sload(const int32_t *p, int64_t i) { return ((const_i32 *)p)[i]; }

// fp32 -> bf16 (round to nearest even), packed two per dword; low half first
// two floats to bf16 (nearest even), lo in the low half: one v_cvt_pk_bf16_f32
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
// acc + (the two bf16 halves of w), exactly as rounded: a dot product with (1, 1)
__device__ inline float sum_bf16x2(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                         acc, false);
}
__device__ inline float max3(float a, float b, float c) { return __builtin_fmaxf(__builtin_fmaxf(a, b), c); }

// Max / sum over lanes l and l^16 (resp. l^32) with gfx950's
// v_permlane16/32_swap on a copy of the value: VALU only, no LDS round trip.
// Written as one asm block: the builtins' results are folded incorrectly
// when both operands hold the same value, and the s_nop's cover the VALU
// write -> permlane read hazard that inline asm hides from the compiler.
#define PKV_XLANE(name, perm, op)                                                        \
  __device__ __forceinline__ float name(float v) {                                      \
    float t;                                                                            \
    asm volatile("v_mov_b32 %1, %0\n\ts_nop 1\n\t" perm " %0, %1\n\ts_nop 1\n\t" op \
                 " %0, %0, %1"                                                          \
                 : "+v"(v), "=&v"(t));                                                  \
    return v;                                                                           \
  }
PKV_XLANE(xmax16, "v_permlane16_swap_b32", "v_max_f32")
PKV_XLANE(xmax32, "v_permlane32_swap_b32", "v_max_f32")
PKV_XLANE(xsum16, "v_permlane16_swap_b32", "v_add_f32")
PKV_XLANE(xsum32, "v_permlane32_swap_b32", "v_add_f32")
#undef PKV_XLANE

__device__ inline float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ inline float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// slot translation
// ---------------------------------------------------------------------------
// Slot of packed row t: find its sequence s (last s with cu[s] <= t; cu[S] =
// T > t), its position seq_lens[s] - q_len_s + (t - cu[s]), then
// block_table[s][pos / 16] * 16 + pos % 16.  -1 if the entry is unusable.
__device__ inline int64_t row_slot(const int32_t *__restrict__ cu, const int32_t *__restrict__ seq_lens,
                                   const int32_t *__restrict__ bt, int32_t bt_stride, int32_t S, int t,
                                   int64_t num_blocks) {
  int lo = 0, hi = S;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int s = lo < S ? lo : S - 1;
  const int ql = cu[s + 1] - cu[s];
  const int pos = seq_lens[s] - ql + (t - cu[s]);
  if (pos < 0 || (pos >> 4) >= bt_stride) return -1;
  const int b = bt[(int64_t)s * bt_stride + (pos >> 4)];
  if (b < 0 || b >= num_blocks) return -1;
  return (int64_t)b * pkv::kBlock + (pos & 15);
}

__global__ __launch_bounds__(256) void slot_mapping_kernel(
    const int32_t *__restrict__ cu, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ bt, int32_t bt_stride, int32_t S, int32_t T,
    int64_t num_blocks, int64_t *__restrict__ slots) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  slots[t] = row_slot(cu, seq_lens, bt, bt_stride, S, t, num_blocks);
}

// ---------------------------------------------------------------------------
// Sequence of packed row t0 (the last s with cu[s] <= t0; cu[S] = T > t0),
// found by one wavefront in rounds of 64 probes: each round narrows the
// candidates to one 64th with one coalesced load, so S + 1 entries take
// ceil(log64(S + 1)) dependent loads (two up to 4,095 sequences) where a
// binary search takes log2(S + 1).  Lane 0 always probes cu[lo] <= t0 (cu[0]
// = 0), so every ballot has a bit set; every probe is clamped into cu[0 .. S].
// ---------------------------------------------------------------------------
__device__ inline int wave_seq_of_row(const int32_t *__restrict__ cu, int S, int t0, int lane) {
  int lo = 0, len = S + 1;  // the answer lies in cu[lo .. lo + len)
  while (len > 64) {
    const int step = (len + 63) / 64;
    const bool le = lane * step < len && cu[min(lo + lane * step, S)] <= t0;
    const uint64_t m = __builtin_amdgcn_ballot_w64(le);
    const int last = m ? 63 - __builtin_clzll(m) : 0;  // m == 0 only for malformed metadata
    lo += last * step;
    len = min(step, len - last * step);
  }
  const bool le = lane < len && cu[min(lo + lane, S)] <= t0;
  const uint64_t m = __builtin_amdgcn_ballot_w64(le);
  return min(m ? lo + 63 - __builtin_clzll(m) : lo, S - 1);
}

// ---------------------------------------------------------------------------
// append: a workgroup per 16 consecutive packed rows and kHeads kv heads
// (four for large steps, one when the rows are too few to fill the GPU), a
// thread per (row, 8 dimensions) for the K and the V of each head.  All the
// rows' K and V are loaded first, so their latency overlaps the slot
// translation, which the workgroup does once for its heads.
// Slots: the first row's sequence s0 by the 64-way search above (wavefront
// 0), then a window of 64 cu entries after s0 gives every row of the group
// its sequence by counting (cu is non-decreasing, so the entries <= t form
// a prefix of the window); a row more than 63 sequence boundaries past the
// first -- only possible across empty sequences -- takes the plain binary
// search.  K rows: lanes run over dimensions, each row's 256 bytes are four
// 64-byte stores, one per 32-dimension group of the tile.  V tiles hold
// two halves of 8 tokens, each dimension-major: lanes run over rows, so each
// store instruction writes, per dimension, the consecutive slots of up to 8
// consecutive rows in each half -- whole 16-byte pieces inside any prefill
// run; decode rows touch one slot of a block each (64 sectors of the tile).
// Placement and write policy, both for the launch that follows: runs of 16
// consecutive row groups go to one XCD (the runs to the XCDs in turn), so
// the two groups that share a block write it through one L2; and the K
// stores and paired V stores are non-temporal, so the step's lines leave
// the caches during the append.  Plain stores left them to be written back
// a few at a time while the attention launch streams the pools, and a
// write under a full read stream costs several times its bytes (on the
// 200-iteration trace both changes together made the attention launches
// ~8% faster).  With the planner's row groups (pkv_paged_step) every block
// the step fills is written by one workgroup.
// ---------------------------------------------------------------------------
constexpr int kAppendRows = 16;
constexpr int kAppendRun = 16;  // consecutive row groups per XCD on large steps

template <int kAppendHeads>
__global__ __launch_bounds__(256) void append_kernel(
    const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
    const int64_t *__restrict__ slot_in,  // given slots, or null: translate
    const int32_t *__restrict__ cu, const int32_t *__restrict__ seq_lens,
    const int32_t *__restrict__ bt, int32_t bt_stride, int32_t S, int32_t T, int32_t Hkv,
    int64_t num_blocks, int64_t *__restrict__ slot_out, uint16_t *__restrict__ kc,
    uint16_t *__restrict__ vc, int32_t run, const int2 *__restrict__ groups, int32_t ngroups) {
  __shared__ int64_t srow[kAppendRows];
  __shared__ uint32_t vrow[kAppendHeads][kAppendRows][D / 2 + 1];  // +1: rows start in different banks
  // runs of `run` consecutive row groups on one XCD, the runs dealt to the
  // XCDs in turn (workgroups go to the XCDs in turn; gridDim.x is a
  // multiple of 8 runs): a block that two groups of a run share is written
  // through one L2, whose partial lines then merge before they reach HBM
  const int place = blockIdx.x / kXcdCount;  // this workgroup's place on its XCD
  const int grp = ((place / run) * kXcdCount + blockIdx.x % kXcdCount) * run + place % run;
  // rows t0 .. t0 + n - 1: the planner's group grp, else 16 rows from 16 grp
  int t0, n;
  if (groups) {
    if (grp >= ngroups) return;  // padding of the grid
    const int2 gd = groups[grp];
    t0 = gd.x;
    // a list that does not fit the batch (not the plan's) touches no row
    // outside it
    if (t0 < 0 || t0 >= T) return;
    n = min(min(gd.y, kAppendRows), T - t0);
    if (n <= 0) return;
  } else {
    t0 = grp * kAppendRows;
    if (t0 >= T) return;  // padding of the grid
    n = min(kAppendRows, T - t0);
  }
  const int h0 = blockIdx.y * kAppendHeads;
  const int nh = min(kAppendHeads, Hkv - h0);
  const int tid = threadIdx.x;
  const int ri = tid >> 4, d0 = 8 * (tid & 15);  // this thread's row and dimensions
  const bool row_ok = ri < n;
  // the rows' K (kept in registers) and V (staged in LDS), before the slots
  u32x4 xk[kAppendHeads];
  if (row_ok) {
    const int64_t base = ((int64_t)(t0 + ri) * Hkv + h0) * D + d0;
    u32x4 xv[kAppendHeads];
#pragma unroll
    for (int j = 0; j < kAppendHeads; ++j) {
      if (j < nh) {
        xk[j] = load16(k_new + base + j * D);
        xv[j] = load16(v_new + base + j * D);
      }
    }
#pragma unroll
    for (int j = 0; j < kAppendHeads; ++j)
      if (j < nh)
#pragma unroll
        for (int e = 0; e < 4; ++e) vrow[j][ri][d0 / 2 + e] = xv[j][e];
  }
  if (tid < 64) {
    const int lane = tid;
    if (slot_in) {
      if (lane < kAppendRows) {
        int64_t sl = -1;
        if (lane < n) {
          sl = slot_in[t0 + lane];
          if (sl < 0 || sl >= num_blocks * pkv::kBlock) sl = -1;
        }
        srow[lane] = sl;
      }
    } else {
      const int s0 = wave_seq_of_row(cu, S, t0, lane);
      // window: cu[s0 + 1 + l] (clamped at cu[S] = T, which no row reaches)
      const int w = cu[min(s0 + 1 + lane, S)];
      int cnt = 0;  // lane i < 16: window entries <= row t0 + i
#pragma unroll
      for (int i = 0; i < kAppendRows; ++i) {
        const int c = __builtin_popcountll(__builtin_amdgcn_ballot_w64(w <= t0 + i));
        if (lane == i) cnt = c;
      }
      const int cu_s0 = cu[s0];
      // cu[s] and cu[s + 1] of this lane's row, from the window
      const int lo_e = __shfl(w, max(cnt - 1, 0)), hi_e = __shfl(w, min(cnt, 63));
      if (lane < kAppendRows) {
        const int t = t0 + lane;
        int64_t sl = -1;
        if (lane < n) {
          if (cnt < 64) {
            const int sq = min(s0 + cnt, S - 1);  // S - 1 unless the metadata is malformed
            const int c_lo = cnt == 0 ? cu_s0 : lo_e;
            const int pos = seq_lens[sq] - (hi_e - c_lo) + (t - c_lo);
            if (pos >= 0 && (pos >> 4) < bt_stride) {
              const int b = bt[(int64_t)sq * bt_stride + (pos >> 4)];
              if (b >= 0 && b < num_blocks) sl = (int64_t)b * pkv::kBlock + (pos & 15);
            }
          } else {
            sl = row_slot(cu, seq_lens, bt, bt_stride, S, t, num_blocks);
          }
          if (blockIdx.y == 0) slot_out[t] = sl;
        }
        srow[lane] = sl;
      }
    }
  }
  __syncthreads();
  {  // K: lanes over dimensions
    const int64_t sl = srow[ri];
    if (row_ok && sl >= 0) {
      uint16_t *kp = kc + ((sl >> 4) * Hkv + h0) * TILE + (d0 / kKGroup) * kKGroupElems + (sl & 15) * kKGroup +
                     d0 % kKGroup;
#pragma unroll
      for (int j = 0; j < kAppendHeads; ++j)
        if (j < nh) __builtin_nontemporal_store(xk[j], reinterpret_cast<u32x4 *>(kp + j * TILE));
    }
  }
  // V, halves of 8 tokens, dimension-major: lanes over (row pair, dimension),
  // pairs fastest, so a wavefront's stores cover 8 dimensions x 16 tokens --
  // 128 contiguous bytes per half when the rows fill a block in order; a
  // pair of consecutive, 4-byte-aligned slots (never split between halves)
  // is one 4-byte store
  const int p = tid & 7;  // this thread's row pair, the same in every round below
  const int r0 = 2 * p, r1 = r0 + 1;
  const int64_t s0 = r0 < n ? srow[r0] : -1, s1 = r1 < n ? srow[r1] : -1;
  const bool pair = s0 >= 0 && s1 == s0 + 1 && (s0 & 1) == 0;
#pragma unroll
  for (int k = 0; k < kAppendHeads * kAppendRows * D / 2 / 256; ++k) {
    const int u = tid + 256 * k, d = (u >> 3) & (D - 1), j = u >> 10;
    if (j >= nh) continue;
    const uint32_t w0 = vrow[j][r0][d >> 1], w1 = vrow[j][r1][d >> 1];
    const uint32_t a0 = d & 1 ? w0 >> 16 : w0 & 0xFFFF, a1 = d & 1 ? w1 >> 16 : w1 & 0xFFFF;
    uint16_t *vh = vc + (int64_t)(h0 + j) * TILE + (int64_t)d * kVHalf;
    // slot sl's element of this dimension
    auto at = [&](int64_t sl) { return vh + (sl >> 4) * Hkv * TILE + ((sl & 15) >> 3) * kVHalfElems + (sl & 7); };
    if (pair) {
      __builtin_nontemporal_store(a0 | (a1 << 16), reinterpret_cast<uint32_t *>(at(s0)));
    } else {
      // lone slots (decode rows, run edges) stay plain: non-temporal, each
      // would leave for HBM at once as a partial line (append 7.5 us slower
      // per trace step)
      if (s0 >= 0) *at(s0) = (uint16_t)a0;
      if (s1 >= 0) *at(s1) = (uint16_t)a1;
    }
  }
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------
struct AttnArgs {
  const uint16_t *q;
  const uint16_t *kc;
  const uint16_t *vc;
  const int32_t *bt;
  uint16_t *out;
  const Item *items;
  const int32_t *waves;  // item offsets of the narrow wavefronts (after the wide items)
  float2 *part_ml;
  float *part_o;
  const uint16_t *zero;  // one all-zero (block, head) tile
  const int32_t *wg_list;  // launch with wide tiles: item offsets of each workgroup's list
  int32_t num_wg;        // launch with wide tiles: persistent workgroups
  int32_t narrow_rows;   // launch with wide tiles: rows of eight workgroups walking narrow shares first
  int32_t nt_out;        // wide-tile outputs as non-temporal stores (the launch also streams decode items)
  int64_t num_blocks;
  int32_t bt_stride;
  int32_t num_items;
  int32_t num_wide;
  int32_t num_waves;
  int32_t Hq;
  int32_t Hkv;
  int32_t log2G;
  float scale_log2;  // scale * log2(e)
};

struct Chunk {
  u32x4 k[8];  // [m-tile][32-dim step]
  u32x4 v[8];  // [16-dim tile]
  bool bad0;   // first block id out of range (wave-uniform)
  bool bad1;   // second block needed and out of range (wave-uniform)
};

// Run one item with NT column tiles of 16 (NT = 1: up to 16 columns, NT = 4:
// up to 64).  Everything indexed [nt] is per column tile.
template <int NT>
__device__ __forceinline__ void run_item(const AttnArgs &a, const Item &it) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int r = lane & 15;
  const int G = 1 << a.log2G;
  const int Hq = a.Hq;

  // ---- columns owned by this lane: column r of each tile
  bool col_ok[NT];
  int col_pos[NT];
  int64_t col_qoff[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = nt * 16 + r;
    const int pc = col >> a.log2G;
    const int ho = col & (G - 1);
    col_ok[nt] = pc < it.np;
    col_pos[nt] = it.pos0 + pc;
    col_qoff[nt] = ((int64_t)(it.t0 + pc) * Hq + it.kvh * G + ho) * D;
  }

  // ---- Q^T operand (B of S^T = K Q^T): dims 32c + 8g .. +7 of column r
  u32x4 qb[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      qb[nt][c] = col_ok[nt] ? load16(a.q + col_qoff[nt] + 32 * c + 8 * g) : u32x4{0, 0, 0, 0};

  f32x4 acc[NT][8];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = neg_inf();
    l_run[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- block ids are wave-uniform: scalar loads, fetched ahead of use
  const int32_t *btrow = a.bt + (int64_t)it.seq * a.bt_stride;
  const int kb0 = it.k0 >> 4;
  // one past the last table entry the item may read (never past the row)
  const int kb_end = min((it.k1 + 15) >> 4, a.bt_stride);
  auto block_id = [&](int lb) -> int { return lb < kb_end ? sload(btrow, lb) : -1; };

  const int nchunks = (it.k1 - it.k0 + 31) >> 5;
  const int64_t head_off = (int64_t)it.kvh * TILE;
  const int64_t blk_stride = (int64_t)a.Hkv * TILE;

  // per-lane constant parts of the operand addresses
  const int ka = r >> 2, kbb = r & 3;               // K row r -> key 8*ka + 4*mt + kbb
  const int k_sel = ka >> 1;                         // which block of the pair
  const int k_row_off = (8 * (ka & 1) + kbb) * kKGroup + 8 * g;  // + 4*mt*kKGroup + c*kKGroupElems
  const int v_sel = g >> 1;
  const int v_off = r * kVHalf + kVHalfElems * (g & 1);  // + 16*dt*8

  // Chunk cc covers keys k0 + 32cc .. +31 in logical blocks kb0 + 2cc and
  // kb0 + 2cc + 1.  When the second block is not needed it aliases the
  // first (same cache lines): every key past k1 is masked out of the scores
  // and its value zeroed, so its contents never matter.
  auto load_chunk = [&](int cc, int b0, int b1, Chunk &ch) {
    const int key0 = it.k0 + 32 * cc;
    const bool need1 = key0 + 16 < it.k1;
    const bool ok0 = b0 >= 0 && b0 < a.num_blocks;
    const bool ok1 = b1 >= 0 && b1 < a.num_blocks;
    // addresses are always in bounds: an id outside [0, num_blocks) reads
    // block 0 and is zeroed at compute time.  Every path issues the same 16
    // loads, so the wait for this chunk can leave the next one in flight.
    const int64_t t0 = (ok0 ? (int64_t)b0 * blk_stride : 0) + head_off;
    const int64_t t1 = need1 && ok1 ? (int64_t)b1 * blk_stride + head_off : t0;
    const uint16_t *kp = a.kc + (k_sel ? t1 : t0) + k_row_off;
    const uint16_t *vp = a.vc + (v_sel ? t1 : t0) + v_off;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int c = 0; c < 4; ++c) ch.k[mt * 4 + c] = load16_stream(kp + 4 * mt * kKGroup + c * kKGroupElems);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) ch.v[dt] = load16_stream(vp + dt * 16 * kVHalf);
    ch.bad0 = !ok0;
    ch.bad1 = need1 && !ok1;
  };

  auto compute_chunk = [&](int cc, Chunk &ch) {
    const int key0 = it.k0 + 32 * cc;
    const int kl = key0 + 8 * g;  // key of this lane's slot 0
    if (ch.bad0 || ch.bad1) {
      // table entry outside [0, num_blocks): that block's keys and values are 0
      const bool kz = k_sel ? ch.bad1 : ch.bad0;
      const bool vz = v_sel ? ch.bad1 : ch.bad0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (kz) ch.k[i] = u32x4{0, 0, 0, 0};
        if (vz) ch.v[i] = u32x4{0, 0, 0, 0};
      }
    }
    if (key0 + 32 > it.k1) {
      // keys past the range may hold stale data: zero their V so 0 * garbage
      // cannot reach the accumulator
      const int nv = it.k1 - kl;
      u32x4 keep;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        keep[i] = (2 * i < nv ? 0x0000FFFFu : 0u) | (2 * i + 1 < nv ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) ch.v[dt] &= keep;
    }
    // Only a chunk that reaches past k1 or past the tile's first position
    // can hold keys some column must not see; inside the others every key
    // is visible to every column.  Columns past the tile (no query) see
    // whatever they see: their results are never written.
    const bool edge = key0 + 32 > it.k1 || key0 + 31 > it.pos0;
    u32x4 pb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s0 = mfma(ch.k[c], qb[nt][c], s0);
        s1 = mfma(ch.k[4 + c], qb[nt][c], s1);
      }
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = s0[i];
        sv[4 + i] = s1[i];
      }
      if (edge) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = kl + j;
          sv[j] = key < it.k1 && key <= col_pos[nt] ? sv[j] : neg_inf();
        }
      }
      float mx = neg_inf();
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, sv[j]);
      // raw scores until here: the scale (> 0) commutes with the maximum
      mx = xmax32(xmax16(mx)) * a.scale_log2;
      const float m_new = fmaxf(m_run[nt], mx);
      const float m_use = m_new == neg_inf() ? 0.f : m_new;
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = pack_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i], a.scale_log2, -m_use)),
                                     __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i + 1], a.scale_log2, -m_use)));
        pb[nt][i] = w;
        lsum += bf16_lo(w) + bf16_hi(w);
      }
      // rescale only when some column's maximum moved (wave-uniform test)
      if (__builtin_amdgcn_ballot_w64(m_new != m_run[nt])) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_use);
        l_run[nt] = l_run[nt] * alpha + lsum;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[nt][dt] *= alpha;
      } else {
        l_run[nt] += lsum;
      }
      m_run[nt] = m_new;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt][dt] = mfma(ch.v[dt], pb[nt], acc[nt][dt]);
  };

  // ---- main loop: one chunk of K/V loads in flight ahead of the math,
  // block ids two chunks ahead.  The loop body always issues both
  // prefetches (the tail is peeled), so every wait leaves the next chunk's
  // 16 loads outstanding.
  Chunk bufA, bufB;
  load_chunk(0, block_id(kb0), block_id(kb0 + 1), bufA);
  int nb0 = block_id(kb0 + 2), nb1 = block_id(kb0 + 3);
  int cc = 0;
  for (; cc + 2 < nchunks; cc += 2) {
    load_chunk(cc + 1, nb0, nb1, bufB);
    nb0 = block_id(kb0 + 2 * cc + 4);
    nb1 = block_id(kb0 + 2 * cc + 5);
    compute_chunk(cc, bufA);
    load_chunk(cc + 2, nb0, nb1, bufA);
    nb0 = block_id(kb0 + 2 * cc + 6);
    nb1 = block_id(kb0 + 2 * cc + 7);
    compute_chunk(cc + 1, bufB);
  }
  if (cc + 1 < nchunks) {
    load_chunk(cc + 1, nb0, nb1, bufB);
    compute_chunk(cc, bufA);
    compute_chunk(cc + 1, bufB);
  } else {
    compute_chunk(cc, bufA);
  }

  // ---- epilogue
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float l_tot = xsum32(xsum16(l_run[nt]));
    if (!col_ok[nt]) continue;
    const int col = nt * 16 + r;
    if (it.part < 0) {
      const float inv = 1.f / l_tot;
      uint16_t *op = a.out + col_qoff[nt] + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 v = acc[nt][dt] * inv;
        u32x2 w;
        w[0] = pack_bf16(v[0], v[1]);
        w[1] = pack_bf16(v[2], v[3]);
        *reinterpret_cast<u32x2 *>(op + 16 * dt) = w;
      }
    } else {
      const int64_t pcol = (int64_t)it.part + col;
      float *po = a.part_o + pcol * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4 *>(po + 16 * dt) = acc[nt][dt];
      if (g == 0) a.part_ml[pcol] = make_float2(m_run[nt], l_tot);
    }
  }
}

__device__ __forceinline__ Item load_item(const AttnArgs &a, int idx) {
  Item it;
  const int32_t *src = reinterpret_cast<const int32_t *>(a.items + idx);
  it.seq = sload(src, 0);
  it.kvh = sload(src, 1);
  it.t0 = sload(src, 2);
  it.np = sload(src, 3);
  it.pos0 = sload(src, 4);
  it.k0 = sload(src, 5);
  it.k1 = sload(src, 6);
  it.part = sload(src, 7);
  return it;
}

// ---------------------------------------------------------------------------
// Narrow wavefront stream.  A narrow wavefront's items (consecutive segments
// of the concatenated (tile, kv head) key streams) are walked as ONE stream
// of 32-key chunks: the chunk after the current one is always in flight,
// also when it belongs to the next item, so an item boundary costs no load
// latency.  Each chunk carries the Q^T operand of its item (4 KiB, reread
// from cache per chunk), so nothing of an item is held across the boundary
// but its accumulator.
//
// Finished items' outputs are not stored as they finish: they are parked in
// the wavefront's 16 KiB of LDS (64 records of 256 bytes, a bf16 output
// column per record, an fp32 partial column in two) and written out when the
// records run out and at the end of the stream.  The vector memory counter
// retires loads and stores in issue order, and a store takes long to retire
// under a full read stream, so every store issued between the chunk loads
// held up the next chunk's wait (measured on MI355X: eight stores per item
// cost about one chunk time per item, a tenth of a step at 16 items per
// wavefront).  Record j's destination lives in lane j's registers.
// ---------------------------------------------------------------------------
constexpr int kStashRecs = 64;     // records per wavefront (one per lane)
constexpr int kStashRecVec = 16;   // u32x4 per record (256 bytes)
constexpr int kStashVec = kStashRecs * kStashRecVec;  // u32x4 per wavefront (16 KiB)
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) int lds_int;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

struct StreamChunk {
  u32x4 q[4];  // Q^T operand of the chunk's item: dims 32c + 8g .. +7 of column r
  u32x4 k[8];
  u32x4 v[8];
  Item it;     // the chunk's item (wave-uniform)
  int cc;      // chunk index within the item
  bool last;   // last chunk of the item
  bool bad0, bad1;
};

__device__ __forceinline__ int item_chunks(const Item &it) { return it.k1 > it.k0 ? (it.k1 - it.k0 + 31) >> 5 : 0; }


// prog: the workgroup's eight progress words in LDS (zeroed before any
// wavefront enters), slot: this wavefront's index in the workgroup; none for
// one-wavefront workgroups.
__device__ __forceinline__ void narrow_stream(const AttnArgs &a, int i0, int i1, lds_u32x4 *stash,
                                              volatile lds_int *prog = nullptr, int slot = 0) {
  if (i0 >= i1) return;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int r = lane & 15;
  const int log2G = a.log2G;
  const int G = 1 << log2G;
  const int Hq = a.Hq;
  const int pc = r >> log2G;  // position (within the tile) of this lane's column r
  const int ho = r & (G - 1);  // query head (within the group) of column r

  // ---- chunks of the whole stream: every item's count, summed over the wave
  int total = 0;
  for (int b = i0; b < i1; b += 64) {
    int n = 0;
    if (b + lane < i1) {
      const Item *p = a.items + b + lane;
      n = p->k1 > p->k0 ? (p->k1 - p->k0 + 31) >> 5 : 0;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o);
    total += __builtin_amdgcn_readfirstlane(n);
  }
  if (total == 0) return;

  // per-lane constant parts of the K/V operand addresses (as in run_item)
  const int ka = r >> 2, kbb = r & 3;
  const int k_sel = ka >> 1;
  const int k_row_off = (8 * (ka & 1) + kbb) * kKGroup + 8 * g;
  const int v_sel = g >> 1;
  const int v_off = r * kVHalf + kVHalfElems * (g & 1);
  const int64_t blk_stride = (int64_t)a.Hkv * TILE;

  // ---- load cursor (wave-uniform): item li (fields itL, nchL chunks), its
  // chunk lc, the block ids of that chunk's two blocks, and the next item's
  // fields, fetched one item ahead
  int li = i0, lc = 0;
  Item itL = load_item(a, li), itN = itL;
  int nchL = item_chunks(itL);
  while (nchL == 0 && ++li < i1) {
    itL = load_item(a, li);
    nchL = item_chunks(itL);
  }
  if (li + 1 < i1) itN = load_item(a, li + 1);
  auto block_id = [&](const Item &it, int j) -> int {
    const int lb = (it.k0 >> 4) + j;
    const int kb_end = min((it.k1 + 15) >> 4, a.bt_stride);
    return lb < kb_end ? sload(a.bt + (int64_t)it.seq * a.bt_stride, lb) : -1;
  };
  int nb0 = block_id(itL, 0), nb1 = block_id(itL, 1);

  // move the cursor one chunk on; block ids of the new position are fetched
  // here, a chunk before they are needed
  auto advance = [&]() {
    if (++lc == nchL) {
      lc = 0;
      do {
        if (++li >= i1) break;
        itL = itN;
        if (li + 1 < i1) itN = load_item(a, li + 1);
        nchL = item_chunks(itL);
      } while (nchL == 0);
    }
    if (li < i1) {
      nb0 = block_id(itL, 2 * lc);
      nb1 = block_id(itL, 2 * lc + 1);
    }
  };

  // Issue the 20 loads of the cursor's chunk (4 of Q, 8 of K, 8 of V).  The
  // same loads on every path, so each wait leaves the next chunk in flight.
  auto issue = [&](StreamChunk &ch) {
    const Item &it = itL;
    ch.it = it;
    ch.cc = lc;
    ch.last = lc + 1 == nchL;
    const int key0 = it.k0 + 32 * lc;
    const bool need1 = key0 + 16 < it.k1;
    const bool ok0 = nb0 >= 0 && nb0 < a.num_blocks;
    const bool ok1 = nb1 >= 0 && nb1 < a.num_blocks;
    const int64_t head_off = (int64_t)it.kvh * TILE;
    const int64_t t0 = (ok0 ? (int64_t)nb0 * blk_stride : 0) + head_off;
    const int64_t t1 = need1 && ok1 ? (int64_t)nb1 * blk_stride + head_off : t0;
    // columns past the tile read the zero tile
    const uint16_t *qp = pc < it.np ? a.q + ((int64_t)(it.t0 + pc) * Hq + it.kvh * G + ho) * D + 8 * g
                                    : a.zero + 8 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) ch.q[c] = load16(qp + 32 * c);
    const uint16_t *kp = a.kc + (k_sel ? t1 : t0) + k_row_off;
    const uint16_t *vp = a.vc + (v_sel ? t1 : t0) + v_off;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int c = 0; c < 4; ++c) ch.k[mt * 4 + c] = load16_stream(kp + 4 * mt * kKGroup + c * kKGroupElems);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) ch.v[dt] = load16_stream(vp + dt * 16 * kVHalf);
    ch.bad0 = !ok0;
    ch.bad1 = need1 && !ok1;
  };

  f32x4 acc[8];
  float m_run = neg_inf(), l_run = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- parked outputs: records [0, nrec); lane j holds record j's
  // destination: a row-head index (bf16 output, 256 bytes) or, where bit j
  // of pmask is set, 2 * partial column + half (fp32, 2 x 256 bytes); where
  // bit j of mlmask is set, also that partial column's (max, sum)
  int nrec = 0;
  uint64_t pmask = 0, mlmask = 0;
  uint32_t rec_idx = 0;
  float rec_m = 0.f, rec_l = 0.f;
  auto flush = [&]() {
    for (int q = 0; q < nrec; q += 4) {
      const int j = q + (lane >> 4), piece = lane & 15;
      const uint32_t idx = (uint32_t)__shfl((int)rec_idx, j);
      if (j < nrec) {
        const u32x4 d = stash[j * kStashRecVec + piece];
        char *dst = (pmask >> j) & 1
                        ? reinterpret_cast<char *>(a.part_o) + (int64_t)(idx >> 1) * (D * 4) + (idx & 1) * 256
                        : reinterpret_cast<char *>(a.out) + (int64_t)idx * (D * 2);
        // final outputs non-temporal (they would otherwise be written back
        // under a later launch's read stream); partials stay cached for the
        // merge that reads them next
        if ((pmask >> j) & 1)
          *reinterpret_cast<u32x4 *>(dst + 16 * piece) = d;
        else
          __builtin_nontemporal_store(d, reinterpret_cast<u32x4 *>(dst + 16 * piece));
      }
    }
    if (lane < nrec && ((mlmask >> lane) & 1)) a.part_ml[rec_idx >> 1] = make_float2(rec_m, rec_l);
    nrec = 0;
    pmask = mlmask = 0;
  };

  auto finish = [&](const Item &it) {
    const float l_tot = xsum32(xsum16(l_run));
    const int ncols = max(0, min(it.np << log2G, 16));  // columns r < ncols hold a query
    const bool part = it.part >= 0;
    const int need = part ? 2 * ncols : ncols;
    if (nrec + need > kStashRecs) flush();
    const int jr = lane - nrec;  // this lane's record within the item
    if (part) {
      // fp32 partial of column r: records nrec + 2r (dims 0..63), nrec + 2r + 1
      if (r < ncols) {
        lds_u32x4 *rec = stash + (nrec + 2 * r) * kStashRecVec + g;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) rec[4 * dt] = __builtin_bit_cast(u32x4, acc[dt]);
      }
      const int c = jr >> 1;
      const float cm = __shfl(m_run, c), cl = __shfl(l_tot, c);
      if (jr >= 0 && jr < need) {
        rec_idx = (uint32_t)(2 * (it.part + c) + (jr & 1));
        if ((jr & 1) == 0) {
          rec_m = cm;
          rec_l = cl;
        }
      }
      if (need > 0) {  // need <= 32 and nrec + need <= 64 here
        const uint64_t bits = ((1ull << need) - 1) << nrec;
        pmask |= bits;
        mlmask |= bits & (0x5555555555555555ull << nrec);
      }
    } else {
      if (r < ncols) {
        const float inv = 1.f / l_tot;
        lds_u32x2 *rec = reinterpret_cast<lds_u32x2 *>(stash + (nrec + r) * kStashRecVec) + g;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const f32x4 v = acc[dt] * inv;
          u32x2 w;
          w[0] = pack_bf16(v[0], v[1]);
          w[1] = pack_bf16(v[2], v[3]);
          rec[4 * dt] = w;
        }
      }
      if (jr >= 0 && jr < need)
        rec_idx = (uint32_t)((it.t0 + (jr >> log2G)) * Hq + it.kvh * G + (jr & (G - 1)));
    }
    nrec += need;
    m_run = neg_inf();
    l_run = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  auto compute = [&](StreamChunk &ch) {
    const Item &it = ch.it;
    const int key0 = it.k0 + 32 * ch.cc;
    const int kl = key0 + 8 * g;  // key of this lane's slot 0
    if (ch.bad0 || ch.bad1) {
      // table entry outside [0, num_blocks): that block's keys and values are 0
      const bool kz = k_sel ? ch.bad1 : ch.bad0;
      const bool vz = v_sel ? ch.bad1 : ch.bad0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (kz) ch.k[i] = u32x4{0, 0, 0, 0};
        if (vz) ch.v[i] = u32x4{0, 0, 0, 0};
      }
    }
    if (key0 + 32 > it.k1) {
      // keys past the range may hold stale data: zero their V
      const int nv = it.k1 - kl;
      u32x4 keep;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        keep[i] = (2 * i < nv ? 0x0000FFFFu : 0u) | (2 * i + 1 < nv ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) ch.v[dt] &= keep;
    }
    const bool edge = key0 + 32 > it.k1 || key0 + 31 > it.pos0;
    const int col_pos = it.pos0 + pc;
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      s0 = mfma(ch.k[c], ch.q[c], s0);
      s1 = mfma(ch.k[4 + c], ch.q[c], s1);
    }
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = s0[i];
      sv[4 + i] = s1[i];
    }
    if (edge) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = kl + j;
        sv[j] = key < it.k1 && key <= col_pos ? sv[j] : neg_inf();
      }
    }
    float mx = neg_inf();
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, sv[j]);
    // raw scores until here: the scale (> 0) commutes with the maximum
    mx = xmax32(xmax16(mx)) * a.scale_log2;
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == neg_inf() ? 0.f : m_new;
    float lsum = 0.f;
    u32x4 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = pack_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i], a.scale_log2, -m_use)),
                                   __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i + 1], a.scale_log2, -m_use)));
      pb[i] = w;
      lsum += bf16_lo(w) + bf16_hi(w);
    }
    // rescale only when some column's maximum moved (wave-uniform test)
    if (__builtin_amdgcn_ballot_w64(m_new != m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[dt] *= alpha;
    } else {
      l_run += lsum;
    }
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = mfma(ch.v[dt], pb, acc[dt]);
    if (ch.last) finish(it);
  };

  // ---- the stream: the next chunk's loads are issued before each chunk's
  // math; the tail is peeled so the loop body always issues
  StreamChunk A, B;
  issue(A);
  advance();
  int sidx = 0;
  for (; sidx + 2 < total; sidx += 2) {
    issue(B);
    advance();
    // Two wavefronts of a workgroup share each SIMD (slots s and s ^ 4).
    // Left alone, the older one is served first and ends its equal share
    // far earlier (on a decode-heavy trace step the younger ones ended 1.76x
    // later); each posts its progress every two chunks and takes a higher
    // priority while it trails its partner, so the pair ends together.
    int other = 0;
    if (prog) {
      prog[slot] = sidx;
      other = __builtin_amdgcn_readfirstlane(prog[slot ^ 4]);
    }
    compute(A);
    if (prog) {
      if (sidx < other) __builtin_amdgcn_s_setprio(2);
      else __builtin_amdgcn_s_setprio(0);
    }
    issue(A);
    advance();
    compute(B);
  }
  if (sidx + 1 < total) {
    issue(B);
    advance();
    compute(A);
    compute(B);
  } else {
    compute(A);
  }
  flush();
}

// ---------------------------------------------------------------------------
// Wide prefill tiles.  A tile covers one (sequence, kv head) and up to 256/G
// query positions: 256 columns (positions x the group's query heads).  A
// persistent workgroup of eight wavefronts walks a list of tiles;
// wavefront w owns columns [32w, 32w + 32) of each, two wavefronts per
// SIMD, one's softmax issued beside the other's matrix work (on gfx950 the
// two still take about the sum of their times).  Keys and values
// stream in 32-key chunks (16 KiB), each staged once per workgroup in LDS by
// direct global->LDS loads, laid out in MFMA operand order: region R (1 KiB)
// holds, at byte 16*l, the 16 bytes lane l needs -- K operand (m-tile R/4,
// 32-dim step R%4) for R < 8, V^T operand (16-dim tile R-8) for R >= 8.
// Wavefront w loads regions 2w, 2w+1 of every chunk.  The chunks of all the
// workgroup's tiles form one stream through a ring of eight buffers that
// keeps five chunks' loads in flight, so the next tile's first chunks land
// while the current tile finishes.
// ---------------------------------------------------------------------------
constexpr int kChunkVec = 1024;  // u32x4 per chunk buffer (16 KiB)
constexpr int kNbuf = 8;         // chunk buffers in the ring (128 KiB)
typedef __attribute__((address_space(3))) void lds_void_t;

// The ring of chunk buffers.
__shared__ __attribute__((aligned(16))) u32x4 lds_chunks[kNbuf * kChunkVec];

// Operand regions of a staged chunk, lane `lane`'s 16 bytes each: the K
// operands (regions 0..7) and, separately, the V^T operands (regions 8..15),
// so the V reads can land while the scores are computed.  Issued as plain
// ds_read_b128 instructions: the caller has already waited for the chunk's
// loads (vmcnt) and passed the workgroup barrier, which the compiler's own
// wait insertion cannot see across three rotating buffers; the caller
// waits on lgkmcnt before using the results.
#define PKV_DS_READ(dst, off) asm volatile("ds_read_b128 %0, %1 offset:" #off : "=v"(dst) : "v"(addr))
__device__ __forceinline__ uint32_t lds_lane_addr(const u32x4 *buf, int lane) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) u32x4 *)buf + lane);
}
__device__ __forceinline__ void lds_read_k(uint32_t addr, u32x4 (&k)[8]) {
  PKV_DS_READ(k[0], 0);
  PKV_DS_READ(k[1], 1024);
  PKV_DS_READ(k[2], 2048);
  PKV_DS_READ(k[3], 3072);
  PKV_DS_READ(k[4], 4096);
  PKV_DS_READ(k[5], 5120);
  PKV_DS_READ(k[6], 6144);
  PKV_DS_READ(k[7], 7168);
}
__device__ __forceinline__ void lds_read_v(uint32_t addr, u32x4 (&v)[8]) {
  PKV_DS_READ(v[0], 8192);
  PKV_DS_READ(v[1], 9216);
  PKV_DS_READ(v[2], 10240);
  PKV_DS_READ(v[3], 11264);
  PKV_DS_READ(v[4], 12288);
  PKV_DS_READ(v[5], 13312);
  PKV_DS_READ(v[6], 14336);
  PKV_DS_READ(v[7], 15360);
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Waits that also hand the eight operand registers just read through to
// their users, so no use can be scheduled above the wait.  lgkmcnt(8): all
// but the last eight LDS reads issued have returned (they return in order).
#define PKV_OPS8(x) "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7])
__device__ __forceinline__ void wait_lds_for(u32x4 (&x)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : PKV_OPS8(x)::"memory");
}
__device__ __forceinline__ void wait_lds_but8_for(u32x4 (&x)[8]) {
  asm volatile("s_waitcnt lgkmcnt(8)" : PKV_OPS8(x)::"memory");
}
#undef PKV_OPS8
#undef PKV_DS_READ

// The Q^T operands of a wide tile are loaded by plain global_load_dwordx4
// instructions in asm, so the compiler does not place waits for them (its
// loop analysis would wait for every chunk load in flight); the caller waits
// with an explicit count and then hands the registers through an empty asm
// statement, so no use can be scheduled above the wait.  Each register is
// tied in and out, so the load writes the registers the operands live in.
#define PKV_GLOAD(x, off) asm volatile("global_load_dwordx4 %0, %1, off offset:" #off : "+v"(x) : "v"(p) : "memory")
template <int NT>
__device__ __forceinline__ void q_load(u32x4 (&q)[NT][4], const uint16_t *const (&ptr)[NT]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const uint16_t *p = ptr[nt];
    PKV_GLOAD(q[nt][0], 0);
    PKV_GLOAD(q[nt][1], 64);
    PKV_GLOAD(q[nt][2], 128);
    PKV_GLOAD(q[nt][3], 192);
  }
}
#undef PKV_GLOAD
template <int NT>
__device__ __forceinline__ void q_ready(u32x4 (&q)[NT][4]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) asm volatile("" : "+v"(q[nt][0]), "+v"(q[nt][1]), "+v"(q[nt][2]), "+v"(q[nt][3]));
}

template <int kVm>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt vmcnt(kVm), expcnt and lgkmcnt left at their maxima (no wait)
  __builtin_amdgcn_s_waitcnt((kVm & 0xF) | (7 << 4) | (15 << 8) | ((kVm >> 4) << 14));
}

// Wide tiles of the stream: wave-uniform description (keys start at 0).
struct WideTile {
  int32_t seq, kvh, t0, np, pos0, k1;
  int32_t nch;     // 32-key chunks (at least one)
  int32_t kb_end;  // one past the last block-table entry the tile reads
};

__device__ __forceinline__ WideTile wide_tile(const AttnArgs &a, int idx) {
  const Item it = load_item(a, idx);
  WideTile d;
  d.seq = it.seq;
  d.kvh = it.kvh;
  d.t0 = it.t0;
  d.np = it.np;
  d.pos0 = it.pos0;
  d.k1 = it.k1;
  d.nch = max(1, (it.k1 + 31) >> 5);
  d.kb_end = min((it.k1 + 15) >> 4, a.bt_stride);
  return d;
}

// A column's probabilities (relative to its reference) may sum to this
// much: every one of them then stays finite in fp32.  The output
// accumulators sum probability x value and can still overflow when values
// are large (beyond ~2^27 at this bound), so they are checked as well: a
// wavefront with a column sum past the bound, or any sum or accumulator
// that is not finite, recomputes its columns.
constexpr float kRedoSum = 0x1p100f;

// The wide tiles items[i0, i1) of one persistent workgroup.  Scores leave
// the matrix cores unscaled; each exponential's argument is one fp32 FMA,
// score * (scale * log2(e)) - reference, so Q enters the products exactly
// as stored, whatever the size of the logits.
__device__ __forceinline__ void run_wide_list(const AttnArgs &a, int i0, int i1) {
  constexpr int WV = pkv::kWideWaves;
  constexpr int NT = pkv::kWideCols / (16 * WV);  // MFMA column tiles per wavefront
  constexpr int RPW = 16 / WV;                    // operand regions loaded per wavefront
  constexpr int kAhead = kNbuf - 3;               // chunks whose loads are issued ahead
  static_assert(NT * 16 * WV == pkv::kWideCols && RPW == 2, "wide tile shape");
  constexpr int kLoadsPerIssue = RPW;            // loads per chunk issue and wavefront
  static_assert((kNbuf & (kNbuf - 1)) == 0 && kAhead == 5, "ring of eight, waits below");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int r = lane & 15;
  const int G = 1 << a.log2G;
  const int WP = (pkv::kWideCols / WV) >> a.log2G;  // positions per wavefront
  const float c2 = a.scale_log2;
  const uint32_t nblk = (uint32_t)a.num_blocks;

  // Wavefronts 0-3 load the K regions of each chunk, wavefronts 4-7 the V^T
  // regions, two each.  A lane's two regions lie in the same block of the
  // chunk (sel) at a fixed offset (lane_off) and region distance.
  const bool kside = w < 4;
  const uint16_t *cache = kside ? a.kc : a.vc;
  int sel, lane_off;
  {
    const int ka = r >> 2, kbb = r & 3;
    const int R0 = w * RPW;
    if (kside) {  // region R: m-tile R/4 (keys +4), 32-dim group R%4
      sel = ka >> 1;
      lane_off = (8 * (ka & 1) + kbb) * kKGroup + 8 * g + 4 * (R0 >> 2) * kKGroup + (R0 & 3) * kKGroupElems;
    } else {      // region R: 16-dim tile R-8
      sel = g >> 1;
      lane_off = r * kVHalf + kVHalfElems * (g & 1) + (R0 - 8) * 16 * kVHalf;
    }
  }
  auto slot = [&](int c) -> u32x4 * { return lds_chunks + (c & (kNbuf - 1)) * kChunkVec; };

  // ---- the chunk stream: every chunk of every tile of the list, in order,
  // then all-zero chunks.  The cursor (tile ci, chunk ccc) issues stream
  // chunk n_issued into ring slot n_issued % kNbuf.  Table entries outside
  // [0, num_blocks), blocks past a tile, and the chunks after the list read
  // the all-zero tile.  The table entries of the next issue (e0, e1) and
  // the descriptor of the cursor's next tile (nd) are fetched one issue
  // ahead, so no issue waits on a scalar load.  Every call issues exactly
  // kLoadsPerIssue loads, so the loads in flight behind any chunk are known
  // on every path.
  int ci = i0, ccc = 0, n_issued = 0;
  WideTile cd = wide_tile(a, i0);
  WideTile nd = i0 + 1 < i1 ? wide_tile(a, i0 + 1) : cd;
  // The next issue's two table entries (clamped to the tile's last one,
  // kb_end >= 1, so both loads always issue) and whether each is real; the
  // selection happens at the issue, so no step waits for these loads.
  int e0, e1;
  bool ok0, ok1;
  auto fetch_ids = [&]() {
    const int32_t *btrow = a.bt + (int64_t)cd.seq * a.bt_stride;
    const bool live = ci < i1;
    e0 = sload(btrow, min(2 * ccc, cd.kb_end - 1));
    e1 = sload(btrow, min(2 * ccc + 1, cd.kb_end - 1));
    ok0 = live && 2 * ccc < cd.kb_end;
    ok1 = live && 2 * ccc + 1 < cd.kb_end;
  };
  fetch_ids();
  auto issue_next = [&]() {
    const uint32_t hoff = (uint32_t)cd.kvh;
    auto tile = [&](int b) -> const uint16_t * {
      return (uint32_t)b < nblk ? cache + (uint64_t)((uint32_t)b * (uint32_t)a.Hkv + hoff) * TILE : a.zero;
    };
    const int b0 = ok0 ? e0 : -1, b1 = ok1 ? e1 : -1;
    const uint16_t *src = (sel ? tile(b1) : tile(b0)) + lane_off;
    u32x4 *dst = slot(n_issued) + w * RPW * 64;
    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)dst, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(src + (kside ? kKGroupElems : 16 * kVHalf), (lds_void_t *)(dst + 64), 16, 0,
                                     0);
    ++n_issued;
    const bool live = ci < i1;
    if (__builtin_expect(live && ccc + 1 >= cd.nch, 0)) {  // the cursor's tile is done
      ccc = 0;
      ++ci;
      cd = nd;
      if (ci + 1 < i1) nd = wide_tile(a, ci + 1);
    } else {
      ++ccc;  // past the list it only feeds clamped, unused table reads
    }
    fetch_ids();
  };
  auto barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // Two groups of four wavefronts (one of each per SIMD) run half a step
  // apart for the whole list.  A wavefront alternates a vector phase V(c) --
  // the probabilities of chunk c, while the K operands of chunk c+1 land --
  // with a matrix phase M(c+1) -- S^T tiles of chunk c+1 and O^T += V^T P^T
  // of chunk c.  Group 1 passes one extra barrier first (group 0 one extra
  // at the end), so it runs V(c) while group 0 runs M(c+1) and M(c+1) while
  // group 0 runs V(c+1): each SIMD's matrix core works for one wavefront
  // while the other computes exponentials.  A tile of n chunks takes n + 1
  // steps of two barriers; chunk c (stream index) occupies its slot from the
  // barrier before group 0's V(c-1) to group 1's M(c+1), and the load issued
  // at a step goes kAhead chunks ahead, into the slot of a chunk three steps
  // older -- also across tile boundaries, where the stream simply goes on.
  const int grp = w >> 2;
  for (int c = 0; c < kAhead; ++c) issue_next();
  if (grp == 1) barrier();

  int g_base = 0;        // stream index of the current tile's first chunk
  uint64_t redo = 0;     // list positions < 64 whose columns need recomputing
  bool redo_all = false; // a later position does (recompute every tile)
  WideTile dn = wide_tile(a, i0);  // the next tile's descriptor, fetched a tile ahead

  // Q^T operands of a tile; columns past the tile read the zero tile.  The
  // next tile's are loaded as soon as the last S^T tiles of the current one
  // have been issued, so they land during its last steps and epilogue, and
  // waiting for them does not wait for the chunk loads issued after them.
  // q_mark: the stream's issue count when they were issued.
  u32x4 qb[NT][4];
  for (int nt = 0; nt < NT; ++nt)
    for (int c = 0; c < 4; ++c) qb[nt][c] = u32x4{0u, 0u, 0u, 0u};
  int q_mark = 0;
  const uint16_t *qnext[NT];  // this lane's Q^T operand addresses in the next tile
  auto q_addresses = [&](const WideTile &t) {
    const int tnp = max(0, min(WP, t.np - w * WP));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = nt * 16 + r;
      const int pc = col >> a.log2G;
      qnext[nt] =
          (pc < tnp ? a.q + ((int64_t)(t.t0 + w * WP + pc) * a.Hq + t.kvh * G + (col & (G - 1))) * D : a.zero) +
          8 * g;
    }
  };
  // (the addresses are formed here, from a descriptor fetched a tile
  // earlier, so no tile start waits for its scalar loads)
  auto load_q = [&]() {
    q_addresses(dn);
    q_load(qb, qnext);
    q_mark = n_issued;
  };
  load_q();
  for (int i = i0; i < i1; ++i) {
    const WideTile d = dn;
    const bool next_q = i + 1 < i1;
    const int wpos0 = d.pos0 + w * WP;  // first position of this wavefront
    const int wnp = max(0, min(WP, d.np - w * WP));
    const int wlast = wpos0 + wnp - 1;
    const int ncomp = wnp > 0 ? min(d.nch, (wlast >> 5) + 1) : 0;

    bool col_ok[NT];
    int col_pos[NT];
    int64_t col_qoff[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = nt * 16 + r;
      const int pc = col >> a.log2G;
      const int ho = col & (G - 1);
      col_ok[nt] = pc < wnp;
      col_pos[nt] = wpos0 + pc;
      col_qoff[nt] = ((int64_t)(d.t0 + w * WP + pc) * a.Hq + d.kvh * G + ho) * D;
    }

    // Probabilities are taken relative to a fixed per-column reference: the
    // column's maximum score in the tile's first chunk (key 0 is in it).
    // fp32 and bf16 keep 8 exponent bits, so later scores may exceed it by
    // up to 100 (log2 units) without overflow and nothing is rescaled -- the
    // accumulators never leave the matrix cores inside the loop.  Past the
    // first chunk no maximum is tracked: a probability above kRedoSum makes
    // its column's sum exceed it too, so a wavefront with a column sum past
    // kRedoSum (or not finite) recomputes its columns after the list
    // (exactly, with the running-maximum softmax of the narrow path).
    f32x4 acc[NT][8];
    float neg_ref[NT];  // -(reference) in log2 units
    float l_part[NT];   // this lane's sum of its rounded probabilities
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      l_part[nt] = 0.f;
      neg_ref[nt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    u32x4 kop[8], vop[8];
    f32x4 sc[NT][2];
    u32x4 pb[NT];

    // kInterior (modes 1 and 2): 1 <= c - 1 and c < ncomp, so both halves
    // run; mode 1 also has chunk c - 1 free of masking (the caller's range
    // guarantees either), so the conditions fold away.
    auto phase_m = [&](int c, auto steady) {
      constexpr bool kSteady = decltype(steady)::value == 1;
      constexpr bool kInterior = decltype(steady)::value != 0;
      const bool do_qk = kInterior || (c >= 0 && c < ncomp);
      const bool do_pv = kInterior || (c >= 1 && c - 1 < ncomp);
      if (!do_qk && !do_pv) return;
      __builtin_amdgcn_s_setprio(1);
      // the V^T operands of chunk c-1 land while the S^T tiles are computed
      if (do_pv) {
        lds_read_v(lds_lane_addr(slot(g_base + c - 1), lane), vop);
        wait_lds_but8_for(kop);
      } else {
        wait_lds_for(kop);
      }
      if (do_qk) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sc[nt][0] = sc[nt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            sc[nt][0] = mfma(kop[k], qb[nt][k], sc[nt][0]);
            sc[nt][1] = mfma(kop[4 + k], qb[nt][k], sc[nt][1]);
          }
      }
      if (do_pv) {
        wait_lds_for(vop);
        const int key0 = 32 * (c - 1);
        if (!kSteady && key0 + 32 > d.k1) {
          // keys past the tile may hold stale data: zero their values
          const int nv = d.k1 - (key0 + 8 * g);
          u32x4 keep;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            keep[e] = (2 * e < nv ? 0x0000FFFFu : 0u) | (2 * e + 1 < nv ? 0xFFFF0000u : 0u);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) vop[dt] &= keep;
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[nt][dt] = mfma(vop[dt], pb[nt], acc[nt][dt]);
      }
      __builtin_amdgcn_s_setprio(0);
    };

    // kInterior: 1 <= c and c + 1 < ncomp; kSteady: also no masking in chunk c
    auto phase_v = [&](int c, auto steady) {
      constexpr bool kSteady = decltype(steady)::value == 1;
      constexpr bool kInterior = decltype(steady)::value != 0;
      // reads for the next matrix phase first, so they land during the softmax
      if (kInterior || c + 1 < ncomp) lds_read_k(lds_lane_addr(slot(g_base + c + 1), lane), kop);
      if (!kInterior && (c < 0 || c >= ncomp)) return;
      const int key0 = 32 * c;
      const int kl = key0 + 8 * g;
      float sv[NT][8];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[nt][e] = sc[nt][0][e];
          sv[nt][4 + e] = sc[nt][1][e];
        }
      // causal masking is needed only where a key can lie past a column's
      // position (or past the tile, or on empty columns)
      if (!kSteady && (key0 + 31 > wpos0 || wnp < WP || key0 + 32 > d.k1)) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int key = kl + j;
            sv[nt][j] = (col_ok[nt] && key < d.k1 && key <= col_pos[nt]) ? sv[nt][j] : neg_inf();
          }
      }
      if (!kInterior && c == 0) {
        // the reference: the column's maximum over the first chunk
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float m = max3(max3(sv[nt][0], sv[nt][1], sv[nt][2]), max3(sv[nt][3], sv[nt][4], sv[nt][5]),
                               __builtin_fmaxf(sv[nt][6], sv[nt][7]));
          const float mx = xmax32(xmax16(m));
          neg_ref[nt] = mx == neg_inf() ? 0.f : -mx * c2;
        }
      }
      // exponent (log2 units) relative to the reference
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = __builtin_fmaf(sv[nt][2 * e], c2, neg_ref[nt]);
          const float x1 = __builtin_fmaf(sv[nt][2 * e + 1], c2, neg_ref[nt]);
          pb[nt][e] = pack_bf16(__builtin_amdgcn_exp2f(x0), __builtin_amdgcn_exp2f(x1));
          l_part[nt] = sum_bf16x2(pb[nt][e], l_part[nt]);
        }
    };

    // Each step: every LDS read of this wavefront is done (its slot may be
    // refilled) and its loads of the tile's chunk s have landed -- the
    // stream's next kAhead - 1 chunks, issued after it, may still fly.
    // Loads complete in order, so the count to wait for is the loads issued
    // after the chunk's: kLoadsPerIssue per later chunk, plus the latest Q
    // loads when they came later (earlier Q loads left uncounted only make
    // the wait stricter; stores never make it weaker).
    auto wait_chunk = [&](int s) {
      wait_lds();
      // every step issues one chunk, so kAhead - 1 chunks were issued after
      // chunk s; anything else (not expected) waits for everything
      static_assert(kLoadsPerIssue * (kAhead - 1) + 4 * NT == 16, "wait counts below");
      if (__builtin_expect(n_issued - 1 - (g_base + s) == kAhead - 1, 1)) {
        if (q_mark > g_base + s) wait_vmcnt<16>();
        else wait_vmcnt<8>();
      } else {
        wait_vmcnt<0>();
      }
    };
    // the tile's Q loads have landed: every load issued after them may fly
    auto wait_q = [&]() {
      switch (n_issued - q_mark) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<kLoadsPerIssue>(); break;
        case 2: wait_vmcnt<2 * kLoadsPerIssue>(); break;
        case 3: wait_vmcnt<3 * kLoadsPerIssue>(); break;
        case 4: wait_vmcnt<4 * kLoadsPerIssue>(); break;
        case 5: wait_vmcnt<5 * kLoadsPerIssue>(); break;
        case 6: wait_vmcnt<6 * kLoadsPerIssue>(); break;
        default: wait_vmcnt<7 * kLoadsPerIssue>(); break;
      }
      q_ready(qb);
    };
    constexpr std::integral_constant<int, 0> kAny{};
    constexpr std::integral_constant<int, 1> kSteadyStep{};
    constexpr std::integral_constant<int, 2> kMaskedStep{};
    // step 0 (a tile has at least one chunk)
    wait_chunk(0);
    barrier();
    issue_next();
    // the next tile's descriptor: issued beside the table entries that the
    // next step's issue waits for anyway, so no wait covers only its latency
    if (next_q) dn = wide_tile(a, i + 1);
    phase_v(-1, kAny);
    barrier();
    wait_q();
    phase_m(0, kAny);
    const int s_next_q = next_q ? max(ncomp, 1) : -1;  // after the tile's last S^T tiles (phase_m(ncomp - 1))
    auto step = [&](int s, auto steady) {
      constexpr bool kInterior = decltype(steady)::value != 0;
      if (!kInterior && s == s_next_q) load_q();
      if (kInterior) {
        // The tile's Q loads were waited for at step 0 and the next tile's
        // are not issued yet, so every load issued before them has landed
        // and only the kAhead - 1 later chunks' loads may still fly.
        wait_lds();
        wait_vmcnt<kLoadsPerIssue * (kAhead - 1)>();
      } else if (s < d.nch) {
        wait_chunk(s);
      } else {
        wait_lds();
      }
      barrier();
      if (kInterior || s < d.nch) issue_next();
      phase_v(s - 1, steady);
      barrier();
      phase_m(s, steady);
    };
    // Steady steps: s in [2, s_hi) -- chunk s - 1 is neither the first nor
    // masked (the wavefront has all its positions, every key of the chunk
    // lies at or before its first position and inside the tile) and chunk s
    // still has S^T tiles.  Masked interior steps: s in [s_hi, ncomp), the
    // same with the masks tested at run time.  The first step and those past
    // the wavefront's last S^T tiles take the general path.
    const int s_hi = wnp < WP ? 0 : min(ncomp, min((wpos0 + 1) >> 5, d.k1 >> 5) + 1);
    int s = 1;
    for (; s < min(2, d.nch + 1); ++s) step(s, kAny);
    for (; s < s_hi; ++s) step(s, kSteadyStep);
    for (; s < ncomp; ++s) step(s, kMaskedStep);  // interior steps whose chunk needs masking
    for (; s <= d.nch; ++s) step(s, kAny);

    // column sums over the four lane groups
    float l_tot[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) l_tot[nt] = xsum32(xsum16(l_part[nt]));

    // did a column outgrow its reference, or an output accumulator
    // overflow?  (rare: recomputed after the list.)  0 * x is 0 for every
    // finite x and NaN otherwise, so one FMA per accumulator tests them all
    // with nothing to overflow.
    {
      bool grew = false;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float z = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int e = 0; e < 4; ++e) z = __builtin_fmaf(acc[nt][dt][e], 0.f, z);
        grew |= !(l_tot[nt] <= kRedoSum) || z != 0.f;
      }
      if (__builtin_amdgcn_ballot_w64(grew)) {
        if (i - i0 < 64) redo |= 1ull << (i - i0);
        else redo_all = true;
      }
    }

    // epilogue: O / l.  When the launch also streams decode items the
    // stores are non-temporal: output lines written while HBM streams reads
    // cost several times their bytes, and the hint took about 5% off a
    // decode-heavy trace step; with prefill tiles alone it only cost time,
    // so there the stores stay plain.  Lane (r, g) holds dims 16 dt + 4 g .. +3 of column r;
    // one v_permlane16_swap per dword pair of chunks dt = 2k, 2k + 1
    // hands it 8 consecutive dims instead (g = 0: 32k + 0..7, g = 2:
    // 32k + 8.., g = 1: 32k + 16.., g = 3: 32k + 24..), so each 16-byte
    // store covers 64 contiguous bytes of a column across its four lanes:
    // half the line pieces of 8-byte stores, which cost the CU's memory
    // pipeline far more than their bytes.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float inv = 1.f / l_tot[nt];
      const int col = nt * 16 + r;
      const int pc = col >> a.log2G;
      uint16_t *const op =
          a.out + ((int64_t)(d.t0 + w * WP + pc) * a.Hq + d.kvh * G + (col & (G - 1))) * D + 16 * (g & 1) + 8 * (g >> 1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 v0 = acc[nt][2 * k] * inv, v1 = acc[nt][2 * k + 1] * inv;
        uint32_t x0 = pack_bf16(v0[0], v0[1]), x1 = pack_bf16(v0[2], v0[3]);
        uint32_t y0 = pack_bf16(v1[0], v1[1]), y1 = pack_bf16(v1[2], v1[3]);
        asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3\n\ts_nop 1"
                     : "+v"(x0), "+v"(y0), "+v"(x1), "+v"(y1));
        if (pc < wnp) {
          u32x4 *dst = reinterpret_cast<u32x4 *>(op + 32 * k);
          const u32x4 val = u32x4{x0, x1, y0, y1};
          // In asm, since a non-temporal store beside a plain one is merged
          // into one plain store.  The compiler's counted waits do not see
          // it, which only makes them wait longer; the s_nop covers a VALU
          // write to the data registers of a 16-byte store.
          if (a.nt_out)
            asm volatile("global_store_dwordx4 %0, %1, off nt\n\ts_nop 1" ::"v"(dst), "v"(val) : "memory");
          else
            *dst = val;
        }
      }
    }
    g_base += d.nch;
  }
  if (grp == 0) barrier();
  // the stream's trailing zero chunks land before the workgroup's LDS is
  // released
  wait_vmcnt<0>();

  // Recompute the columns of any tile that outgrew its references, as
  // narrow items (up to 16 columns each, keys from HBM, running maximum);
  // they overwrite the tile's output.  No barriers: wavefronts are
  // independent from here on.
  if (redo == 0 && !redo_all) return;
  for (int i = i0; i < i1; ++i) {
    if (!redo_all && !(i - i0 < 64 && ((redo >> (i - i0)) & 1))) continue;
    const WideTile d = wide_tile(a, i);
    const int wnp = max(0, min(WP, d.np - w * WP));
    const int per = pkv::kTileCols >> a.log2G;  // positions per narrow item
    for (int p = 0; p < wnp; p += per) {
      Item it;
      it.seq = d.seq;
      it.kvh = d.kvh;
      it.t0 = d.t0 + w * WP + p;
      it.np = min(per, wnp - p);
      it.pos0 = d.pos0 + w * WP + p;
      it.k0 = 0;
      it.k1 = it.pos0 + it.np;
      it.part = -1;
      run_item<1>(a, it);
    }
  }
}

// Narrow tiles only (decode rows and prefill tails): two waves per SIMD.
// Workgroup w walks the items of narrow wavefront w in order.
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attention_kernel(AttnArgs a) {
  const int w = blockIdx.x;
  if (w >= a.num_waves) return;
  __shared__ u32x4 stash[kStashVec];
  narrow_stream(a, sload(a.waves, w), sload(a.waves, w + 1), (lds_u32x4 *)stash);
}

// Launch with wide tiles: a fixed grid of persistent workgroups in rows of
// eight (consecutive workgroups go to the eight XCDs in turn).  The narrow
// rows (spread evenly over the grid) first walk their wavefronts' narrow
// shares -- bandwidth-bound streams beside the other CUs' matrix-bound wide
// tiles -- and then, like every other workgroup, the wide tiles of their
// list; the lists are balanced and keep each kv head's tiles on one XCD.
__global__ __launch_bounds__(64 * pkv::kWideWaves) void attention_mixed_kernel(AttnArgs a) {
  static_assert(pkv::kWideWaves == 8, "rows of eight workgroups of eight wavefronts");
  const int j = blockIdx.x;
  if (j >= a.num_wg) return;
  const pkv::RowRole role = pkv::mixed_row(a.num_wg / 8, a.narrow_rows, j / 8);
  if (role.narrow) {
    const int w = (role.ord * 8 + j % 8) * 8 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // each wavefront parks its finished outputs in its own 16 KiB of the
    // chunk ring, which the wide loop below only fills after the barrier
    static_assert(pkv::kWideWaves * kStashVec <= kNbuf * kChunkVec, "stashes fit in the ring");
    __shared__ int prog[8];
    if ((threadIdx.x & 63) == 0) prog[threadIdx.x >> 6] = 0;
    __syncthreads();
    if (w < a.num_waves)
      narrow_stream(a, a.num_wide + sload(a.waves, w), a.num_wide + sload(a.waves, w + 1),
                    (lds_u32x4 *)lds_chunks + (threadIdx.x >> 6) * kStashVec, (volatile lds_int *)prog,
                    threadIdx.x >> 6);
    __builtin_amdgcn_s_setprio(0);
    // nothing of the narrow walk stays in flight: the wide loop's own waits
    // are then the only ones its tile loop needs
    wait_vmcnt<0>();
    __syncthreads();
  }
  const int i0 = sload(a.wg_list, j);
  const int i1 = sload(a.wg_list, j + 1);
  if (i0 < i1) run_wide_list(a, i0, i1);
}

// ---------------------------------------------------------------------------
// whole-block copies and host swaps: a workgroup per (listed block, K or V);
// 256 threads move the block's num_kv_heads tiles (4 KiB each) with 16-byte
// loads and stores, eight in flight per thread.  Ids outside [0, num_blocks)
// are skipped.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void copy_slab(const u32x4 *__restrict__ s, u32x4 *__restrict__ d, int nvec) {
  for (int i0 = 0; i0 < nvec; i0 += 256 * 8) {
    u32x4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 256 + (int)threadIdx.x;
      if (i < nvec) x[u] = __builtin_nontemporal_load(s + i);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 256 + (int)threadIdx.x;
      if (i < nvec) __builtin_nontemporal_store(x[u], d + i);
    }
  }
}

// pairs[2p] -> pairs[2p + 1]
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint16_t *kc, uint16_t *vc, const int32_t *__restrict__ pairs,
                                                          int32_t n, int64_t num_blocks, int32_t Hkv) {
  const int p = blockIdx.x;
  if (p >= n) return;
  const int64_t src = sload(pairs, 2 * (int64_t)p), dst = sload(pairs, 2 * (int64_t)p + 1);
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  uint16_t *base = blockIdx.y ? vc : kc;
  const int64_t slab = (int64_t)Hkv * TILE;
  copy_slab(reinterpret_cast<const u32x4 *>(base + src * slab), reinterpret_cast<u32x4 *>(base + dst * slab),
            (int)(slab / 8));
}

// host[p][side][Hkv * TILE] <-> block blocks[p] of the K (side 0) / V (side 1) pool
template <bool kOut>
__global__ __launch_bounds__(256) void swap_kernel(uint16_t *kc, uint16_t *vc, const int32_t *__restrict__ blocks,
                                                   int32_t n, int64_t num_blocks, int32_t Hkv, uint16_t *host) {
  const int p = blockIdx.x;
  if (p >= n) return;
  const int64_t b = sload(blocks, p);
  if (b < 0 || b >= num_blocks) return;
  uint16_t *base = blockIdx.y ? vc : kc;
  const int64_t slab = (int64_t)Hkv * TILE;
  uint16_t *dev = base + b * slab;
  uint16_t *hst = host + ((int64_t)p * 2 + blockIdx.y) * slab;
  if (kOut)
    copy_slab(reinterpret_cast<const u32x4 *>(dev), reinterpret_cast<u32x4 *>(hst), (int)(slab / 8));
  else
    copy_slab(reinterpret_cast<const u32x4 *>(hst), reinterpret_cast<u32x4 *>(dev), (int)(slab / 8));
}

// ---------------------------------------------------------------------------
// merge of key-split partials: one wavefront per (row, head), four per
// workgroup.  Lane k first holds split k's (max, sum) -- 64 splits at a time
// -- so the maximum and the normaliser are wave reductions of one load per
// lane; then lane l owns dimensions 2l, 2l + 1 and adds the splits' partial
// outputs with their weights (read across the lanes), four loads in flight.
// ---------------------------------------------------------------------------
constexpr int kMergeWaves = 4;
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(const Merge *__restrict__ merges, int32_t n,
                                                                 const float2 *__restrict__ ml,
                                                                 const float *__restrict__ po,
                                                                 uint16_t *__restrict__ out) {
  const int idx = blockIdx.x * kMergeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (idx >= n) return;
  const int lane = threadIdx.x & 63;
  const int32_t *e = reinterpret_cast<const int32_t *>(merges + idx);
  const int out_row = __builtin_amdgcn_readfirstlane(e[0]);
  const int first = __builtin_amdgcn_readfirstlane(e[1]);
  const int nsplit = __builtin_amdgcn_readfirstlane(e[2]);
  const int stride = __builtin_amdgcn_readfirstlane(e[3]);
  // the maximum over all splits
  float M = neg_inf();
  float2 mine = make_float2(neg_inf(), 0.f);  // this lane's split of the first 64
  for (int k0 = 0; k0 < nsplit; k0 += 64) {
    float2 v = make_float2(neg_inf(), 0.f);
    if (k0 + lane < nsplit) v = ml[first + (int64_t)(k0 + lane) * stride];
    if (k0 == 0) mine = v;
    M = fmaxf(M, wave_max(v.x));
  }
  float ax = 0.f, ay = 0.f, L = 0.f;
  for (int k0 = 0; k0 < nsplit; k0 += 64) {
    float2 v = mine;
    if (k0 > 0) v = k0 + lane < nsplit ? ml[first + (int64_t)(k0 + lane) * stride] : make_float2(neg_inf(), 0.f);
    const float wk = k0 + lane < nsplit ? __builtin_amdgcn_exp2f(v.x - M) : 0.f;
    L += wave_sum(wk * v.y);
    const int nk = min(64, nsplit - k0);
    int k = 0;
    for (; k + 4 <= nk; k += 4) {
      float2 o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        o[u] = *reinterpret_cast<const float2 *>(po + ((int64_t)first + (int64_t)(k0 + k + u) * stride) * D + 2 * lane);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wk), k + u));
        ax += w * o[u].x;
        ay += w * o[u].y;
      }
    }
    for (; k < nk; ++k) {
      const float2 o = *reinterpret_cast<const float2 *>(po + ((int64_t)first + (int64_t)(k0 + k) * stride) * D + 2 * lane);
      const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wk), k));
      ax += w * o.x;
      ay += w * o.y;
    }
  }
  const float inv = 1.f / L;
  // non-temporal: the row is not read again by this step
  __builtin_nontemporal_store(pack_bf16(ax * inv, ay * inv), reinterpret_cast<uint32_t *>(out + (int64_t)out_row * D) + lane);
}

inline hipStream_t as_stream(pkv_stream_t s) { return static_cast<hipStream_t>(s); }

inline int launch_status() { return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP; }

// The softmax scale must be a positive, finite number: the kernels take
// maxima of raw scores and scale them afterwards, which only a positive
// scale commutes with.
inline bool valid_scale(float scale) { return scale > 0.f && scale <= FLT_MAX; }

// Four kv heads per append workgroup once the 16-row groups alone give 256
// workgroups or more; one otherwise, so a small step still spreads over the
// GPU (64 decode rows: 32 workgroups instead of 8).
void launch_append(const uint16_t *k_new, const uint16_t *v_new, const int64_t *slot_in, const int32_t *cu,
                   const int32_t *seq_lens, const int32_t *bt, int32_t bt_stride, int32_t S, int32_t T, int32_t Hkv,
                   int64_t num_blocks, int64_t *slot_out, uint16_t *kc, uint16_t *vc, hipStream_t stream,
                   const int2 *plan_groups = nullptr, int32_t num_plan_groups = 0) {
  const unsigned real_groups =
      plan_groups ? (unsigned)num_plan_groups : (unsigned)((T + kAppendRows - 1) / kAppendRows);
  // runs of 16 groups per XCD once there are 8 runs; plain turns below (a
  // grid padded to 128 groups would cost a 64-row decode step ~0.6 us)
  const int run = real_groups >= (unsigned)(kXcdCount * kAppendRun) ? kAppendRun : 1;
  const unsigned unit = kXcdCount * run;
  const unsigned groups = (real_groups + unit - 1) / unit * unit;
  if (real_groups >= 256) {
    hipLaunchKernelGGL(append_kernel<4>, dim3(groups, (Hkv + 3) / 4), dim3(256), 0, stream, k_new, v_new, slot_in, cu,
                       seq_lens, bt, bt_stride, S, T, Hkv, num_blocks, slot_out, kc, vc, run, plan_groups,
                       num_plan_groups);
  } else {
    hipLaunchKernelGGL(append_kernel<1>, dim3(groups, Hkv), dim3(256), 0, stream, k_new, v_new, slot_in, cu, seq_lens,
                       bt, bt_stride, S, T, Hkv, num_blocks, slot_out, kc, vc, run, plan_groups, num_plan_groups);
  }
}

int check_plan(const pkv_plan_t *plan, size_t ws_bytes, const void *ws) {
  if (!plan) return PKV_EINVAL;
  if (plan->head_dim != D || plan->num_q_heads <= 0 || plan->num_kv_heads <= 0) return PKV_EINVAL;
  if (plan->num_items > 0 && !ws) return PKV_EINVAL;
  if (ws_bytes < plan->ws_bytes) return PKV_EWORKSPACE;
  if (plan->zero_off < 0 || (size_t)plan->zero_off + (size_t)pkv::kBlock * D * 2 > plan->ws_bytes)
    return PKV_EINVAL;
  return PKV_OK;
}

// ---------------------------------------------------------------------------
// The fixed workspace of pkv_paged_step_static: a device array inside the
// library, one copy per GPU, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it only stands for the
// symbol); it looks up each device's address once, with that device
// current, and uses that address for copies and kernel arguments.
// ---------------------------------------------------------------------------
constexpr size_t kStaticWsBytes = (size_t)PKV_STATIC_WS_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticWsBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, looked up on first use.
int scratch_address(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERANGE;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return PKV_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char *pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_ERANGE: return "value out of range";
    case PKV_EUNSUPPORTED: return "unsupported shape";
    case PKV_EWORKSPACE: return "workspace too small";
    case PKV_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int pkv_version(void) { return 103; }

int pkv_slot_mapping(const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                     const int32_t *block_tables, int32_t bt_stride, int32_t num_seqs,
                     int32_t num_rows, int64_t num_blocks, int64_t *slot_mapping,
                     pkv_stream_t stream) {
  if (num_seqs < 0 || num_rows < 0 || bt_stride < 0) return PKV_EINVAL;
  if (num_rows == 0) return PKV_OK;
  if (num_seqs == 0 || !cu_seqlens_q || !seq_lens || !block_tables || !slot_mapping)
    return PKV_EINVAL;
  const int grid = (num_rows + 255) / 256;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(grid), dim3(256), 0, as_stream(stream),
                     cu_seqlens_q, seq_lens, block_tables, bt_stride, num_seqs, num_rows,
                     num_blocks, slot_mapping);
  return launch_status();
}

int pkv_paged_kv_append(const pkv_bf16 *k_new, const pkv_bf16 *v_new,
                        const int64_t *slot_mapping, int32_t num_rows, pkv_bf16 *k_cache,
                        pkv_bf16 *v_cache, int64_t num_blocks, int32_t num_kv_heads,
                        int32_t head_dim, pkv_stream_t stream) {
  if (num_rows < 0 || num_kv_heads <= 0 || num_blocks < 0) return PKV_EINVAL;
  if (head_dim != D) return PKV_EUNSUPPORTED;
  if (num_rows == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PKV_EINVAL;
  launch_append(k_new, v_new, slot_mapping, nullptr, nullptr, nullptr, 0, 0, num_rows, num_kv_heads, num_blocks,
                nullptr, k_cache, v_cache, as_stream(stream));
  return launch_status();
}

int pkv_varlen_attention_main(const pkv_bf16 *q, const pkv_bf16 *k_cache,
                              const pkv_bf16 *v_cache, const int32_t *block_tables,
                              int32_t bt_stride, int64_t num_blocks, float scale,
                              const pkv_plan_t *plan, void *ws, size_t ws_bytes, pkv_bf16 *out,
                              pkv_stream_t stream) {
  int st = check_plan(plan, ws_bytes, ws);
  if (st != PKV_OK) return st;
  if (!valid_scale(scale)) return PKV_EINVAL;
  if (plan->num_items == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !out || bt_stride <= 0 || num_blocks <= 0)
    return PKV_EINVAL;
  // (block, kv head) tiles are indexed in 32 bits
  if (num_blocks > (int64_t)UINT32_MAX / plan->num_kv_heads) return PKV_ERANGE;
  const int G = plan->num_q_heads / plan->num_kv_heads;
  AttnArgs a;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.bt = block_tables;
  a.out = out;
  char *w = static_cast<char *>(ws);
  a.items = reinterpret_cast<const Item *>(w + plan->items_off);
  a.waves = reinterpret_cast<const int32_t *>(w + plan->waves_off);
  a.part_ml = reinterpret_cast<float2 *>(w + plan->ml_off);
  a.part_o = reinterpret_cast<float *>(w + plan->o_off);
  a.zero = reinterpret_cast<const uint16_t *>(w + plan->zero_off);
  a.wg_list = nullptr;
  a.num_wg = 0;
  a.narrow_rows = plan->narrow_rows;
  a.nt_out = plan->num_waves > 0;
  a.num_blocks = num_blocks;
  a.bt_stride = bt_stride;
  a.num_items = plan->num_items;
  a.num_wide = plan->num_wide_items;
  a.num_waves = plan->num_waves;
  a.Hq = plan->num_q_heads;
  a.Hkv = plan->num_kv_heads;
  a.log2G = pkv::log2_exact(G);
  a.scale_log2 = scale * 1.4426950408889634f;
  if (a.log2G < 0) return PKV_EUNSUPPORTED;
  if (plan->num_wide_items > 0) {
    const int nwg = plan->num_workgroups;
    if (nwg <= 0 || nwg % 8 != 0 || nwg > 256 || plan->narrow_rows < 0 || plan->narrow_rows > nwg / 8 ||
        (int64_t)plan->narrow_rows * 64 < plan->num_waves || plan->wg_off < 0 ||
        (size_t)plan->wg_off + (size_t)(nwg + 1) * 4 > plan->ws_bytes)
      return PKV_EINVAL;
    a.wg_list = reinterpret_cast<const int32_t *>(w + plan->wg_off);
    a.num_wg = nwg;
    hipLaunchKernelGGL(attention_mixed_kernel, dim3((unsigned)nwg), dim3(64 * pkv::kWideWaves), 0,
                       as_stream(stream), a);
  } else if (plan->num_waves > 0)
    hipLaunchKernelGGL(attention_kernel, dim3(plan->num_waves), dim3(64), 0, as_stream(stream), a);
  return launch_status();
}

int pkv_split_kv_reduce(const pkv_plan_t *plan, const void *ws, size_t ws_bytes, pkv_bf16 *out,
                        pkv_stream_t stream) {
  int st = check_plan(plan, ws_bytes, ws);
  if (st != PKV_OK) return st;
  if (plan->num_merge == 0) return PKV_OK;
  if (!out) return PKV_EINVAL;
  const char *w = static_cast<const char *>(ws);
  hipLaunchKernelGGL(merge_kernel, dim3((plan->num_merge + kMergeWaves - 1) / kMergeWaves), dim3(64 * kMergeWaves), 0,
                     as_stream(stream),
                     reinterpret_cast<const Merge *>(w + plan->merge_off), plan->num_merge,
                     reinterpret_cast<const float2 *>(w + plan->ml_off),
                     reinterpret_cast<const float *>(w + plan->o_off), out);
  return launch_status();
}

int pkv_paged_varlen_attention(const pkv_bf16 *q, const pkv_bf16 *k_cache,
                               const pkv_bf16 *v_cache, const int32_t *block_tables,
                               int32_t bt_stride, int64_t num_blocks, float scale,
                               const pkv_plan_t *plan, void *ws, size_t ws_bytes, pkv_bf16 *out,
                               pkv_stream_t stream) {
  int st = pkv_varlen_attention_main(q, k_cache, v_cache, block_tables, bt_stride, num_blocks,
                                     scale, plan, ws, ws_bytes, out, stream);
  if (st != PKV_OK) return st;
  return pkv_split_kv_reduce(plan, ws, ws_bytes, out, stream);
}

int pkv_copy_blocks(pkv_bf16 *k_cache, pkv_bf16 *v_cache, int64_t num_blocks, int32_t num_kv_heads,
                    int32_t head_dim, const int32_t *block_pairs, int32_t num_pairs, pkv_stream_t stream) {
  if (num_pairs < 0 || num_blocks < 0 || num_kv_heads <= 0) return PKV_EINVAL;
  if (head_dim != D) return PKV_EUNSUPPORTED;
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_pairs) return PKV_EINVAL;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2), dim3(256), 0, as_stream(stream), k_cache, v_cache,
                     block_pairs, num_pairs, num_blocks, num_kv_heads);
  return launch_status();
}

namespace {
// the device address of a pinned (page-locked, device-mapped) host buffer
int device_view(void *host, uint16_t **dev) {
  void *d = nullptr;
  if (!host || hipHostGetDevicePointer(&d, host, 0) != hipSuccess || !d) {
    (void)hipGetLastError();
    return PKV_EINVAL;
  }
  *dev = static_cast<uint16_t *>(d);
  return PKV_OK;
}
}  // namespace

int pkv_swap_out(const pkv_bf16 *k_cache, const pkv_bf16 *v_cache, int64_t num_blocks, int32_t num_kv_heads,
                 int32_t head_dim, const int32_t *blocks, int32_t num, void *host_dst, pkv_stream_t stream) {
  if (num < 0 || num_blocks < 0 || num_kv_heads <= 0) return PKV_EINVAL;
  if (head_dim != D) return PKV_EUNSUPPORTED;
  if (num == 0) return PKV_OK;
  if (!k_cache || !v_cache || !blocks) return PKV_EINVAL;
  uint16_t *hst;
  const int st = device_view(host_dst, &hst);
  if (st != PKV_OK) return st;
  hipLaunchKernelGGL(swap_kernel<true>, dim3(num, 2), dim3(256), 0, as_stream(stream),
                     const_cast<uint16_t *>(k_cache), const_cast<uint16_t *>(v_cache), blocks, num, num_blocks,
                     num_kv_heads, hst);
  return launch_status();
}

int pkv_swap_in(const void *host_src, const int32_t *blocks, int32_t num, pkv_bf16 *k_cache, pkv_bf16 *v_cache,
                int64_t num_blocks, int32_t num_kv_heads, int32_t head_dim, pkv_stream_t stream) {
  if (num < 0 || num_blocks < 0 || num_kv_heads <= 0) return PKV_EINVAL;
  if (head_dim != D) return PKV_EUNSUPPORTED;
  if (num == 0) return PKV_OK;
  if (!k_cache || !v_cache || !blocks) return PKV_EINVAL;
  uint16_t *hst;
  const int st = device_view(const_cast<void *>(host_src), &hst);
  if (st != PKV_OK) return st;
  hipLaunchKernelGGL(swap_kernel<false>, dim3(num, 2), dim3(256), 0, as_stream(stream), k_cache, v_cache, blocks,
                     num, num_blocks, num_kv_heads, hst);
  return launch_status();
}

int pkv_slot_append(const pkv_bf16 *k_new, const pkv_bf16 *v_new, const int32_t *cu_seqlens_q,
                    const int32_t *seq_lens, const int32_t *block_tables, int32_t bt_stride,
                    int32_t num_seqs, int32_t num_rows, int64_t num_blocks, int64_t *slot_mapping,
                    pkv_bf16 *k_cache, pkv_bf16 *v_cache, int32_t num_kv_heads, int32_t head_dim,
                    pkv_stream_t stream) {
  if (num_seqs < 0 || num_rows < 0 || bt_stride < 0 || num_blocks < 0 || num_kv_heads <= 0)
    return PKV_EINVAL;
  if (head_dim != D) return PKV_EUNSUPPORTED;
  if (num_rows == 0) return PKV_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !cu_seqlens_q || !seq_lens || !block_tables ||
      !slot_mapping || num_seqs == 0)
    return PKV_EINVAL;
  launch_append(k_new, v_new, nullptr, cu_seqlens_q, seq_lens, block_tables, bt_stride, num_seqs, num_rows,
                num_kv_heads, num_blocks, slot_mapping, k_cache, v_cache, as_stream(stream));
  return launch_status();
}

int pkv_paged_step(const pkv_bf16 *q, const pkv_bf16 *k_new, const pkv_bf16 *v_new,
                   pkv_bf16 *k_cache, pkv_bf16 *v_cache, const int32_t *cu_seqlens_q,
                   const int32_t *seq_lens, const int32_t *block_tables, int32_t bt_stride,
                   int64_t num_blocks, int64_t *slot_mapping, float scale,
                   const pkv_plan_t *plan, void *ws, size_t ws_bytes, pkv_bf16 *out,
                   pkv_stream_t stream) {
  if (!plan || !valid_scale(scale)) return PKV_EINVAL;
  const int st = pkv_slot_append_planned(k_new, v_new, cu_seqlens_q, seq_lens, block_tables, bt_stride, num_blocks,
                                         slot_mapping, k_cache, v_cache, plan, ws, ws_bytes, stream);
  if (st != PKV_OK) return st;
  return pkv_paged_varlen_attention(q, k_cache, v_cache, block_tables, bt_stride, num_blocks,
                                    scale, plan, ws, ws_bytes, out, stream);
}

int pkv_slot_append_planned(const pkv_bf16 *k_new, const pkv_bf16 *v_new, const int32_t *cu_seqlens_q,
                            const int32_t *seq_lens, const int32_t *block_tables, int32_t bt_stride,
                            int64_t num_blocks, int64_t *slot_mapping, pkv_bf16 *k_cache, pkv_bf16 *v_cache,
                            const pkv_plan_t *plan, const void *ws, size_t ws_bytes, pkv_stream_t stream) {
  if (!plan) return PKV_EINVAL;
  // pkv_slot_append's checks, then its kernel on the plan's row groups
  const int32_t S = plan->num_seqs, T = plan->num_rows, Hkv = plan->num_kv_heads;
  if (S < 0 || T < 0 || bt_stride < 0 || num_blocks < 0 || Hkv <= 0) return PKV_EINVAL;
  if (plan->head_dim != D) return PKV_EUNSUPPORTED;
  if (T > 0) {
    if (!k_new || !v_new || !k_cache || !v_cache || !cu_seqlens_q || !seq_lens || !block_tables ||
        !slot_mapping || S == 0 || !ws)
      return PKV_EINVAL;
    const int32_t ng = plan->num_append_groups;
    if (ng <= 0 || ng > T || plan->append_off < 0 || (size_t)plan->append_off + (size_t)ng * 8 > plan->ws_bytes)
      return PKV_EINVAL;
    if (ws_bytes < plan->ws_bytes) return PKV_EWORKSPACE;
    launch_append(k_new, v_new, nullptr, cu_seqlens_q, seq_lens, block_tables, bt_stride, S, T, Hkv, num_blocks,
                  slot_mapping, k_cache, v_cache, as_stream(stream),
                  reinterpret_cast<const int2 *>(static_cast<const char *>(ws) + plan->append_off), ng);
    return launch_status();
  }
  return PKV_OK;
}

int pkv_paged_step_static(const pkv_bf16 *q, const pkv_bf16 *k_new, const pkv_bf16 *v_new,
                          pkv_bf16 *k_cache, pkv_bf16 *v_cache, const int32_t *cu_seqlens_q,
                          const int32_t *seq_lens, const int32_t *block_tables, int32_t bt_stride,
                          int64_t num_blocks, int64_t *slot_mapping, float scale,
                          const pkv_plan_t *plan, const void *h_staging, pkv_bf16 *out,
                          pkv_stream_t stream) {
  // everything that needs no device is checked first
  if (!plan || !valid_scale(scale)) return PKV_EINVAL;
  if (plan->ws_bytes > kStaticWsBytes || plan->host_bytes > plan->ws_bytes) return PKV_EWORKSPACE;
  if (plan->host_bytes > 0 && !h_staging) return PKV_EINVAL;
  void *ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != PKV_OK) return st;
  // the plan's item lists, merge entries and zero tile; the partial results
  // behind them are written by the attention launch before the merge reads
  // them, so nothing else needs clearing
  if (plan->host_bytes > 0 &&
      hipMemcpyAsync(ws, h_staging, plan->host_bytes, hipMemcpyHostToDevice, as_stream(stream)) != hipSuccess)
    return PKV_EHIP;
  return pkv_paged_step(q, k_new, v_new, k_cache, v_cache, cu_seqlens_q, seq_lens, block_tables, bt_stride,
                        num_blocks, slot_mapping, scale, plan, ws, kStaticWsBytes, out, stream);
}

}  // extern "C"
