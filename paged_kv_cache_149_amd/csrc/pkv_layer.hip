// The weight layers of one packed layer around the paged step, written for
// CDNA4 (gfx950, wave64, bf16 MFMA): the projections run over all packed
// rows at once, attention per request ("11.2 连续批处理与 PagedAttention",
// section 11.2.2, selective batching: X[7, 4096] x W_Q -> Q[7, 4096]; and
// "continuous batching" (k4i.top), section "把 prefill 和 decode 打包在一起":
// Q = X W_Q, K = X W_K, V = X W_V over the packed rows, RoPE by each row's
// own position id).
//
//   linear_kernel<false>  y[m][n] = sum_k x[m][k] w[n][k]   (bf16 in, fp32
//                         accumulate, bf16 out, nearest even)
//   linear_kernel<true>   the fused QKV projection: the same product with
//                         w = [query heads; key heads; value heads] x 128
//                         rows, RoPE applied to query and key heads by each
//                         row's position, written as q [T][Hq][128],
//                         k_new and v_new [T][Hkv][128]
//
// Weights are [out features][in features], so an output feature's weights
// and an input row are both contiguous over the inner dimension and every
// MFMA operand is one 16-byte piece of a row.  A workgroup of eight
// wavefronts (two per SIMD, so one's matrix work hides the other's LDS
// reads) computes a tile of 256 rows x 256 features (two heads) in 64-deep
// stages staged through LDS (double buffered: the next stage's global loads
// are issued as the current one starts and stored to the other buffer after
// its first 32-deep half); wavefront w owns rows
// 64 (w % 4) .. +63 and the 128 features of head w / 4, as D^T = W X^T with
// v_mfma_f32_16x16x32_bf16:
//   A operand (features): lane l holds W[16j + l%16][8(l/16) .. +7]
//   B operand (rows):     lane l holds X[16i + l%16][8(l/16) .. +7]
//   D[feature][row]:      lane l holds features 16j + 4(l/16) .. +3 of row
//                         16i + l%16 -- four consecutive outputs of one row
// so feature d and its RoPE partner d + 64 (tiles j and j + 4) sit in the
// same lane, and the rotation needs no data exchange.
#include <hip/hip_runtime.h>

#include <type_traits>

#include <cfloat>
#include <cmath>
#include <cstdint>

#include "pkv_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBMMax = 256;           // rows per tile, largest form (64 per row wavefront)
constexpr int kBN = 256;              // features per tile (two heads of 128)
constexpr int kHead = 128;            // features per wavefront (one head)
constexpr int kBK = 64;               // inner dimension per stage
constexpr int kRow = kBK + 8;         // LDS row pitch, bf16: 144 bytes, so the 16 rows of a
                                      // fragment read start in 16 different bank quads
constexpr int kStage = (kBMMax + kBN) * kRow;  // bf16 per stage buffer (largest form)
constexpr int kThreads = 512;
constexpr int kXcds = 8;
constexpr int kCUs = 256;             // compute units of an MI355X
constexpr int kGroupRows = 8;         // row tiles per group of the tile order

__device__ inline f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// two floats to bf16 (nearest even), lo in the low half
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

struct LinearArgs {
  const uint16_t *x;  // [M][K]
  const uint16_t *w;  // [N][K]
  uint16_t *y;        // [M][N] (plain product)
  int32_t M, N, K;
  int32_t tiles_m;        // row tiles
  int32_t tiles_per_xcd;  // tiles dealt to each XCD (grid = 8 x this)
  // fused QKV projection
  uint16_t *q, *k, *v;
  const int32_t *cu, *seq_lens;
  int32_t S, Hq, Hkv;
  double rope_log2_step;  // log2(theta) * 2 / 128: pair i turns by p * 2^(-i * step) radians
};

// position of packed row t: its sequence s (last s with cu[s] <= t), then
// seq_lens[s] - q_len_s + (t - cu[s])
__device__ inline int row_position(const int32_t *__restrict__ cu, const int32_t *__restrict__ seq_lens, int S,
                                   int t) {
  int lo = 0, hi = S;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int s = lo < S ? lo : S - 1;
  return seq_lens[s] - (cu[s + 1] - cu[s]) + (t - cu[s]);
}

// Row positions for few-row kernels without a chain of dependent global
// loads at the end: each lane of one wavefront loads entries lane and
// lane + 64 of cu_seqlens and seq_lens when the kernel starts (their latency
// hides behind the kernel's main loop); before the epilogue they go to LDS
// and each row's sequence is found there.  Holds the tables of up to
// kPosSeqs sequences; more fall back to row_position.
constexpr int kPosSeqs = 127;
struct RowTables {
  int32_t cu0, cu1, sl0, sl1;  // this lane's entries lane and lane + 64 (clamped)
};
__device__ inline RowTables row_tables_load(const int32_t *__restrict__ cu, const int32_t *__restrict__ seq_lens,
                                            int S, int lane) {
  RowTables t;
  if (S >= 1 && S <= kPosSeqs) {
    t.cu0 = cu[min(lane, S)];
    t.cu1 = cu[min(lane + 64, S)];
    t.sl0 = seq_lens[min(lane, S - 1)];
    t.sl1 = seq_lens[min(lane + 64, S - 1)];
  } else {
    t.cu0 = t.cu1 = t.sl0 = t.sl1 = 0;
  }
  return t;
}
// lcu, lsl: 128 entries each in LDS, written here by the calling wavefront
// (entries past S are clamped copies); then row t's position
__device__ inline void row_tables_store(const RowTables &t, int32_t *lcu, int32_t *lsl, int lane) {
  lcu[lane] = t.cu0;
  lcu[lane + 64] = t.cu1;
  lsl[lane] = t.sl0;
  lsl[lane + 64] = t.sl1;
}
__device__ inline int row_position_lds(const int32_t *lcu, const int32_t *lsl, int S, int t) {
  int lo = 0, hi = S;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (lcu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int s = lo < S ? lo : S - 1;
  return lsl[s] - (lcu[s + 1] - lcu[s]) + (t - lcu[s]);
}

// Turns per position of pair i: theta^(-2i/128) / (2 pi) = 2^(-i * step) /
// (2 pi), in double: at position p ~ 3e4 the angle is ~5e3 turns, and a
// float's 2^-24 relative error there would already move it by ~2e-3 rad.
__device__ inline double rope_turns_per_pos(int i, double step) {
  return exp2(-(double)i * step) * 0.15915494309189533577;
}

// cos and sin of p * f turns: the product in double, reduced to [-1/2, 1/2]
// turns, then taken back to radians in float.
__device__ inline void rope_cos_sin(double p, double f, float &c, float &s) {
  const double turns = p * f;
  const float a = (float)(turns - rint(turns)) * 6.283185307179586f;
  c = __cosf(a);
  s = __sinf(a);
}

// kWaveRows rows per wavefront: 64 (tiles of 256 rows) when there are rows
// enough to fill the chip with tiles, else 32 (tiles of 128 rows, twice the
// workgroups for the same work, at more LDS reads per product).
template <bool kRope, int kWaveRows>
__global__ __launch_bounds__(kThreads) void linear_kernel(LinearArgs g) {
  constexpr int kBM = 4 * kWaveRows;
  constexpr int kRowTiles = kWaveRows / 16;
  constexpr int kStageT = (kBM + kBN) * kRow;
  constexpr int kXPieces = kBM * 8 / kThreads;  // 16-byte pieces of the row tile per thread
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kStage];
  // blocks go to the XCDs in turn: XCD x takes tiles x * tiles_per_xcd ..,
  // rows fastest, so the blocks resident on one XCD share their weight tile
  const int b = blockIdx.x;
  const int t = (b % kXcds) * g.tiles_per_xcd + b / kXcds;
  const int tiles_n = (g.N + kBN - 1) / kBN;
  if (t >= g.tiles_m * tiles_n) return;
  // tiles in groups of kGroupRows row tiles x every feature tile, rows
  // fastest: a round of 32 workgroups on one XCD covers 8 row tiles x 4
  // feature tiles, so each row tile and each weight tile is read by several
  // workgroups of the XCD at once and mostly hits its L2
  const int grp = t / (kGroupRows * tiles_n), first_m = grp * kGroupRows;
  const int gm = min(g.tiles_m - first_m, kGroupRows), in_grp = t % (kGroupRows * tiles_n);
  const int m_tile = first_m + in_grp % gm, n_tile = in_grp / gm;
  const int m0 = m_tile * kBM, n0 = n_tile * kBN;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = lane & 15, gq = lane >> 4;
  // wavefront wv: rows kWaveRows (wv % 4) .., features (head) 128 (wv / 4) ..
  const int wm = wv & 3, wn = wv >> 2;

  // Stage loads: thread tid moves 16-byte pieces c = tid + 512u, row c / 8,
  // column piece c % 8 -- of the row tile (rows past M read as zero) and
  // four of the weight tile (rows past N read as zero).
  u32x4 px[kXPieces], pw[4];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < kXPieces; ++u) {
      const int c = tid + kThreads * u, row = c >> 3, col = c & 7;
      px[u] = m0 + row < g.M ? *reinterpret_cast<const u32x4 *>(g.x + (int64_t)(m0 + row) * g.K + k0 + 8 * col)
                             : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + kThreads * u, row = c >> 3, col = c & 7;
      pw[u] = n0 + row < g.N ? *reinterpret_cast<const u32x4 *>(g.w + (int64_t)(n0 + row) * g.K + k0 + 8 * col)
                             : u32x4{0, 0, 0, 0};
    }
  };
  auto stash = [&](int buf) {
    uint16_t *xs = lds + buf * kStageT, *ws = xs + kBM * kRow;
#pragma unroll
    for (int u = 0; u < kXPieces; ++u) {
      const int c = tid + kThreads * u, row = c >> 3, col = c & 7;
      *reinterpret_cast<u32x4 *>(xs + row * kRow + 8 * col) = px[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = tid + kThreads * u, row = c >> 3, col = c & 7;
      *reinterpret_cast<u32x4 *>(ws + row * kRow + 8 * col) = pw[u];
    }
  };

  f32x4 acc[kRowTiles][8];
#pragma unroll
  for (int i = 0; i < kRowTiles; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = g.K / kBK;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int buf = s & 1;
    if (s + 1 < nk) fetch((s + 1) * kBK);
    const uint16_t *xs = lds + buf * kStageT, *ws = xs + kBM * kRow;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      u32x4 wf[8], xf[kRowTiles];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        wf[j] = *reinterpret_cast<const u32x4 *>(ws + (kHead * wn + 16 * j + r) * kRow + 32 * sub + 8 * gq);
#pragma unroll
      for (int i = 0; i < kRowTiles; ++i)
        xf[i] = *reinterpret_cast<const u32x4 *>(xs + (kWaveRows * wm + 16 * i + r) * kRow + 32 * sub + 8 * gq);
#pragma unroll
      for (int i = 0; i < kRowTiles; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma(wf[j], xf[i], acc[i][j]);
      // the next stage goes into the other buffer (last read before the
      // previous barrier) while the second half's products run: measured
      // 7-8% faster than storing it after both halves
      if (sub == 0 && s + 1 < nk) stash(buf ^ 1);
    }
    __syncthreads();
  }

  const int nw = n0 + kHead * wn;  // this wavefront's first feature
  if (nw >= g.N) return;           // past N (N an odd multiple of 128)
  if (!kRope) {
#pragma unroll
    for (int i = 0; i < kRowTiles; ++i) {
      const int m = m0 + kWaveRows * wm + 16 * i + r;
      if (m >= g.M) continue;
      uint16_t *yr = g.y + (int64_t)m * g.N + nw + 4 * gq;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<u32x2 *>(yr + 16 * j) =
            u32x2{pack_bf16(acc[i][j][0], acc[i][j][1]), pack_bf16(acc[i][j][2], acc[i][j][3])};
    }
    return;
  }

  // fused QKV: this wavefront's head of the stacked weight is query head
  // head, key head head - Hq or value head head - Hq - Hkv
  const int head = nw / kHead;
  uint16_t *dst;
  int H, hh;
  if (head < g.Hq) {
    dst = g.q; H = g.Hq; hh = head;
  } else if (head < g.Hq + g.Hkv) {
    dst = g.k; H = g.Hkv; hh = head - g.Hq;
  } else {
    dst = g.v; H = g.Hkv; hh = head - g.Hq - g.Hkv;
  }
  const bool rotate = head < g.Hq + g.Hkv;
  // this lane's pairs are i = 16j + 4(l/16) + e, j, e < 4
  double f[4][4];
  if (rotate) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) f[j][e] = rope_turns_per_pos(16 * j + 4 * gq + e, g.rope_log2_step);
  }
#pragma unroll
  for (int i = 0; i < kRowTiles; ++i) {
    const int m = m0 + kWaveRows * wm + 16 * i + r;
    if (m >= g.M) continue;
    f32x4 o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = acc[i][j];
    if (rotate) {
      const double p = (double)row_position(g.cu, g.seq_lens, g.S, m);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float c, s;
          rope_cos_sin(p, f[j][e], c, s);
          const float x1 = acc[i][j][e], x2 = acc[i][j + 4][e];
          o[j][e] = x1 * c - x2 * s;
          o[j + 4][e] = x2 * c + x1 * s;
        }
    }
    uint16_t *dr = dst + ((int64_t)m * H + hh) * kHead + 4 * gq;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<u32x2 *>(dr + 16 * j) = u32x2{pack_bf16(o[j][0], o[j][1]), pack_bf16(o[j][2], o[j][3])};
  }
}

// Few rows (M <= 64, a decode step): the product is bound by streaming the
// weights once, so the work is cut fine.  Workgroup b takes, for all rows,
// with RoPE 32 features -- 16 of head b / 4 starting at 16 (b % 4) and
// their partners 64 further, so a rotation needs no exchange -- else 16
// consecutive features; its kWaves wavefronts each take an equal slice of
// the inner dimension, loading their MFMA operands straight from memory (the
// weights once, the few rows from L2), eight 32-deep steps in flight, and
// the slices are summed through LDS.  Same D^T = W X^T layout as above, with
// j = 0 the first 16 features and j = 1 their partners.  The rows are read
// once per workgroup, so the 16-feature form (twice the workgroups, twice
// the row reads per weight byte) pays only where the 32-feature one leaves
// CUs idle: a 4096-wide layer's output projection takes 256 workgroups of
// eight wavefronts (25 vs 30 us on MI355X), while its QKV projection keeps
// 192 workgroups of 32 features (34.6 vs 48.6 us with 384 of 16).  An inner
// dimension that is a multiple of 256 takes the LDS-staged form below
// instead; this one covers the rest (multiples of 128).
constexpr int kSkinnyRows = 64;
constexpr int kSkinnyAhead = 8;

template <bool kRope, int kWaves>
__global__ __launch_bounds__(64 * kWaves) void linear_skinny_kernel(LinearArgs g) {
  constexpr int NJ = kRope ? 2 : 1;  // 16-feature tiles: the features, and with RoPE their partners
  __shared__ __attribute__((aligned(16))) float red[kWaves - 1][64][16 * NJ];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, r = lane & 15, gq = lane >> 4;
  const int f0 = kRope ? kHead * (b >> 2) + 16 * (b & 3) : 16 * b;  // first feature; partners at f0 + 64
  const int kq = g.K / kWaves, kbeg = wv * kq;
  const uint16_t *wrow[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) wrow[j] = g.w + (int64_t)(f0 + 64 * j + r) * g.K + 8 * gq;
  f32x4 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // rows past M read row M - 1 (their results are never stored), so every
  // load is unconditional and the loads of kSkinnyAhead steps stay in flight
  const uint16_t *xrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xrow[i] = g.x + (int64_t)min(16 * i + r, g.M - 1) * g.K + 8 * gq;
  auto load_step = [&](int k, u32x4 (&wa)[NJ], u32x4 (&xb)[4]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) wa[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wrow[j] + k));
#pragma unroll
    for (int i = 0; i < 4; ++i) xb[i] = *reinterpret_cast<const u32x4 *>(xrow[i] + k);
  };
  auto mma = [&](const u32x4 (&wa)[NJ], const u32x4 (&xb)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma(wa[j], xb[i], acc[i][j]);
  };
  const int nsteps = kq / 32;
  const int ngroups = nsteps / kSkinnyAhead;
  u32x4 wa[kSkinnyAhead][NJ], xb[kSkinnyAhead][4];
  if (ngroups > 0) {
#pragma unroll
    for (int a = 0; a < kSkinnyAhead; ++a) load_step(kbeg + 32 * a, wa[a], xb[a]);
    // every group but the last: use each slot, then refill it one group on
    for (int gi = 0; gi + 1 < ngroups; ++gi) {
#pragma unroll
      for (int a = 0; a < kSkinnyAhead; ++a) {
        mma(wa[a], xb[a]);
        load_step(kbeg + 32 * ((gi + 1) * kSkinnyAhead + a), wa[a], xb[a]);
      }
    }
#pragma unroll
    for (int a = 0; a < kSkinnyAhead; ++a) mma(wa[a], xb[a]);
  }
  for (int st = ngroups * kSkinnyAhead; st < nsteps; ++st) {
    load_step(kbeg + 32 * st, wa[0], xb[0]);
    mma(wa[0], xb[0]);
  }
  // sum the slices: wavefronts 1.. park theirs in LDS, wavefront 0 adds
  if (wv > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        *reinterpret_cast<f32x4 *>(&red[wv - 1][16 * i + r][16 * j + 4 * gq]) = acc[i][j];
  }
  __syncthreads();
  if (wv > 0) return;
#pragma unroll 1
  for (int q = 0; q < kWaves - 1; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] += *reinterpret_cast<const f32x4 *>(&red[q][16 * i + r][16 * j + 4 * gq]);

  uint16_t *dst = g.y;
  int64_t row_stride = g.N, col0 = f0;
  bool rotate = false;
  double f[4];
  if (kRope) {
    const int head = f0 / kHead;
    int H, hh;
    if (head < g.Hq) {
      dst = g.q; H = g.Hq; hh = head;
    } else if (head < g.Hq + g.Hkv) {
      dst = g.k; H = g.Hkv; hh = head - g.Hq;
    } else {
      dst = g.v; H = g.Hkv; hh = head - g.Hq - g.Hkv;
    }
    row_stride = (int64_t)H * kHead;
    col0 = (int64_t)hh * kHead + (f0 % kHead);
    rotate = head < g.Hq + g.Hkv;
    if (rotate) {
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = rope_turns_per_pos(16 * (b & 3) + 4 * gq + e, g.rope_log2_step);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 16 * i + r;
    if (m >= g.M) continue;
    uint16_t *dr = dst + (int64_t)m * row_stride + col0 + 4 * gq;
    f32x4 o0 = acc[i][0];
    if constexpr (kRope) {
      f32x4 o1 = acc[i][1];
      if (rotate) {
        const double p = (double)row_position(g.cu, g.seq_lens, g.S, m);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float c, sn;
          rope_cos_sin(p, f[e], c, sn);
          o0[e] = acc[i][0][e] * c - acc[i][1][e] * sn;
          o1[e] = acc[i][1][e] * c + acc[i][0][e] * sn;
        }
      }
      *reinterpret_cast<u32x2 *>(dr + 64) = u32x2{pack_bf16(o1[0], o1[1]), pack_bf16(o1[2], o1[3])};
    }
    *reinterpret_cast<u32x2 *>(dr) = u32x2{pack_bf16(o0[0], o0[1]), pack_bf16(o0[2], o0[3])};
  }
}

// Few rows (M <= 64) with an inner dimension a multiple of 256: the same
// split of the features as above, eight wavefronts per workgroup, but the
// operands go through LDS.  Read straight into MFMA operands, every load of
// the rows takes 64 bytes from each of 16 rows, and the rows' L2 traffic
// (all of the rows for every workgroup) runs at that scattered pattern's
// rate, about half of what 1 KiB contiguous loads reach.  Here the
// workgroup copies each 256-deep chunk of the rows (64 rows x 512 bytes)
// into an LDS ring by direct global->LDS loads of 1 KiB contiguous each (two
// rows), and the chunk's weight rows (16 per feature tile) beside them the
// same way; the wavefronts read their operands from there.  A row's 16-byte
// pieces are stored XOR-swizzled by the row's low four bits, so the 16 rows
// of one operand read fall on distinct banks.  Wavefront w takes feature
// tile w % NJ and 32-deep steps of each chunk by k-group w / NJ; the
// k-groups' sums meet in LDS, and four wavefronts finish a row tile each.
// The ring holds three chunks: the one being read, and two in flight.  At
// 64 rows and hidden 4096 on MI355X: QKV with RoPE 35.6 -> 27.2 us, the
// output projection 25.3 -> 18.5 us against the form above (before the
// whole-row weight copies and the shared epilogue).
constexpr int kXChunk = 256;                  // inner dimension per staged chunk
constexpr int kXChunkVec = 64 * kXChunk / 8;  // u32x4 of a chunk's rows (32 KiB)
constexpr int kXRing = 3;                     // chunk buffers

template <int kVm>
__device__ __forceinline__ void layer_wait_vmcnt() {
  // s_waitcnt vmcnt(kVm), expcnt and lgkmcnt left at their maxima (no wait)
  __builtin_amdgcn_s_waitcnt((kVm & 0xF) | (7 << 4) | (15 << 8) | ((kVm >> 4) << 14));
}

template <bool kRope>
__device__ __forceinline__ void skinny_lds_product(const LinearArgs &g) {
  typedef __attribute__((address_space(3))) void lds_void_t;
  constexpr int NJ = kRope ? 2 : 1;           // feature tiles: the features, and with RoPE their partners 64 further
  constexpr int KG = 8 / NJ;                  // k-groups
  constexpr int SPW = NJ;                     // 32-deep steps per wavefront and chunk (8 per chunk / KG)
  constexpr int kSlotVec = kXChunkVec + NJ * 8 * 64;  // u32x4 per ring slot: rows, then weight regions
  constexpr int kLoads = 4 + NJ;              // global->LDS loads per wavefront and chunk
  __shared__ __attribute__((aligned(16))) u32x4 ring[kXRing * kSlotVec];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, r = lane & 15, gq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int jt = w % NJ, kg = w / NJ;
  const int f0 = kRope ? kHead * (b >> 2) + 16 * (b & 3) : 16 * b;  // first feature; partners at f0 + 64
  const int nch = g.K / kXChunk;

  // this wavefront's copies of a chunk: rows 8w + 2q and 8w + 2q + 1 (q < 4),
  // lane l taking piece (l % 32) ^ (row % 16) of row 8w + 2q + l / 32 (rows
  // past M read row M - 1: never stored); the weights the same way, 16
  // feature rows per tile: copy e = NJ w + q (q < NJ) takes feature rows
  // 2 (e % 8) and 2 (e % 8) + 1 of tile e / 8 (features f0 + 64 tile + row),
  // so every copy reads whole 512-byte row pieces (64-byte pieces of 16
  // rows cost ~10% more)
  const uint16_t *xsrc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 8 * w + 2 * q + (lane >> 5);
    xsrc[q] = g.x + (int64_t)min(row, g.M - 1) * g.K + 8 * ((lane & 31) ^ (row & 15));
  }
  const uint16_t *wsrc[NJ];
#pragma unroll
  for (int q = 0; q < NJ; ++q) {
    const int e = NJ * w + q;
    const int row = 2 * (e & 7) + (lane >> 5);
    wsrc[q] = g.w + (int64_t)(f0 + 64 * (e >> 3) + row) * g.K + 8 * ((lane & 31) ^ row);
  }
  auto issue = [&](int c, int slot) {
    u32x4 *base = ring + slot * kSlotVec;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds(xsrc[q] + kXChunk * c, (lds_void_t *)(base + w * 4 * 64 + 64 * q), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < NJ; ++q)
      __builtin_amdgcn_global_load_lds(wsrc[q] + kXChunk * c, (lds_void_t *)(base + kXChunkVec + (NJ * w + q) * 64),
                                       16, 0, 0);
  };
  // LDS byte addresses (slot 0) of this lane's operands of step t: piece
  // 4 st + gq of row r (row tile 0), and of feature row r of tile jt, each
  // stored at (4 st + gq) ^ r
  uint32_t xaddr[SPW], waddr[SPW];
#pragma unroll
  for (int t = 0; t < SPW; ++t) {
    const int st = kg * SPW + t;
    const __attribute__((address_space(3))) u32x4 *lds = (const __attribute__((address_space(3))) u32x4 *)ring;
    xaddr[t] = (uint32_t)(uintptr_t)(lds + r * 32 + ((4 * st + gq) ^ r));
    waddr[t] = (uint32_t)(uintptr_t)(lds + kXChunkVec + jt * 512 + r * 32 + ((4 * st + gq) ^ r));
  }
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the rows' sequence tables, for RoPE's positions (wavefront 0)
  __shared__ int32_t pos_cu[128], pos_sl[128];
  RowTables rtab{};
  if (kRope && w == 0) rtab = row_tables_load(g.cu, g.seq_lens, g.S, lane);
  auto compute = [&](int slot) {
    const uint32_t off = (uint32_t)(slot * kSlotVec * 16);
    u32x4 xb[SPW][4], wv[SPW];
#pragma unroll
    for (int t = 0; t < SPW; ++t) {
      const uint32_t xa = xaddr[t] + off, wa = waddr[t] + off;
      asm volatile("ds_read_b128 %0, %1 offset:0" : "=v"(wv[t]) : "v"(wa));
      asm volatile("ds_read_b128 %0, %1 offset:0" : "=v"(xb[t][0]) : "v"(xa));
      asm volatile("ds_read_b128 %0, %1 offset:8192" : "=v"(xb[t][1]) : "v"(xa));
      asm volatile("ds_read_b128 %0, %1 offset:16384" : "=v"(xb[t][2]) : "v"(xa));
      asm volatile("ds_read_b128 %0, %1 offset:24576" : "=v"(xb[t][3]) : "v"(xa));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int t = 0; t < SPW; ++t) {
      asm volatile("" : "+v"(wv[t]));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        asm volatile("" : "+v"(xb[t][i]));
        acc[i] = mfma(wv[t], xb[t][i], acc[i]);
      }
    }
  };
  auto barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Chunk c is copied into slot c % 3 two chunks ahead, after the barrier
  // that follows everyone's reads of chunk c - 1 (the slot's previous
  // chunk).  Loads complete in order: at chunk c only chunk c + 1's
  // kLoads loads may still fly behind it.  (Weights further ahead than the
  // rows, in a ring of their own, measured no faster.)
  issue(0, 0);
  if (nch > 1) issue(1, 1);
  int slot = 0;
  for (int c = 0; c < nch; ++c) {
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 < nch) layer_wait_vmcnt<kLoads>(); else layer_wait_vmcnt<0>();
    barrier();
    if (c + 2 < nch) issue(c + 2, slot == 0 ? 2 : slot - 1);
    compute(slot);
    slot = slot == kXRing - 1 ? 0 : slot + 1;
  }
  // sum the k-groups and finish: every wavefront parks its partial sums in
  // the (now idle) ring, then wavefront i (i < 4) adds up row tile i of
  // both feature tiles and rotates and stores it, so the epilogue's work is
  // spread over four wavefronts
  barrier();
  f32x4 *red = reinterpret_cast<f32x4 *>(ring);
  auto red_at = [&](int grp, int tile, int i) -> f32x4 & { return red[((grp * NJ + tile) * 4 + i) * 64 + lane]; };
#pragma unroll
  for (int i = 0; i < 4; ++i) red_at(kg, jt, i) = acc[i];
  if (kRope && w == 0 && g.S >= 1 && g.S <= kPosSeqs) row_tables_store(rtab, pos_cu, pos_sl, lane);
  barrier();
  if (w >= 4) return;
  const int i = w;  // this wavefront's row tile
  const int m = 16 * i + r;
  f32x4 o0 = red_at(0, 0, i), o1 = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (kRope) o1 = red_at(0, 1, i);
#pragma unroll
  for (int q = 1; q < KG; ++q) {
    o0 += red_at(q, 0, i);
    if constexpr (kRope) o1 += red_at(q, 1, i);
  }
  if (m >= g.M) return;

  uint16_t *dst = g.y;
  int64_t row_stride = g.N, col0 = f0;
  if constexpr (kRope) {
    const int head = f0 / kHead;
    int H, hh;
    if (head < g.Hq) {
      dst = g.q; H = g.Hq; hh = head;
    } else if (head < g.Hq + g.Hkv) {
      dst = g.k; H = g.Hkv; hh = head - g.Hq;
    } else {
      dst = g.v; H = g.Hkv; hh = head - g.Hq - g.Hkv;
    }
    row_stride = (int64_t)H * kHead;
    col0 = (int64_t)hh * kHead + (f0 % kHead);
    if (head < g.Hq + g.Hkv) {  // queries and keys are rotated, values not
      const bool lds_pos = g.S >= 1 && g.S <= kPosSeqs;
      const double p = (double)(lds_pos ? row_position_lds(pos_cu, pos_sl, g.S, m)
                                        : row_position(g.cu, g.seq_lens, g.S, m));
      const f32x4 a0 = o0, a1 = o1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float c, sn;
        rope_cos_sin(p, rope_turns_per_pos(16 * (b & 3) + 4 * gq + e, g.rope_log2_step), c, sn);
        o0[e] = a0[e] * c - a1[e] * sn;
        o1[e] = a1[e] * c + a0[e] * sn;
      }
    }
  }
  uint16_t *dr = dst + (int64_t)m * row_stride + col0 + 4 * gq;
  if constexpr (kRope) *reinterpret_cast<u32x2 *>(dr + 64) = u32x2{pack_bf16(o1[0], o1[1]), pack_bf16(o1[2], o1[3])};
  *reinterpret_cast<u32x2 *>(dr) = u32x2{pack_bf16(o0[0], o0[1]), pack_bf16(o0[2], o0[3])};
}

template <bool kRope>
__global__ __launch_bounds__(512) void linear_skinny_lds_kernel(LinearArgs g) {
  skinny_lds_product<kRope>(g);
}

inline hipStream_t as_stream(pkv_stream_t s) { return static_cast<hipStream_t>(s); }

int launch_linear(LinearArgs g, bool rope, pkv_stream_t stream) {
  if (g.M <= kSkinnyRows && g.K % kXChunk == 0) {
    if (rope)
      hipLaunchKernelGGL((linear_skinny_lds_kernel<true>), dim3((unsigned)(g.N / 32)), dim3(512), 0,
                         as_stream(stream), g);
    else
      hipLaunchKernelGGL((linear_skinny_lds_kernel<false>), dim3((unsigned)(g.N / 16)), dim3(512), 0,
                         as_stream(stream), g);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
  }
  if (g.M <= kSkinnyRows && g.K % 128 == 0) {
    if (rope) {
      hipLaunchKernelGGL((linear_skinny_kernel<true, 4>), dim3((unsigned)(g.N / 32)), dim3(256), 0,
                         as_stream(stream), g);
    } else if (g.N / 16 <= kCUs && g.K % 256 == 0) {
      // every workgroup resident at once, one per CU
      hipLaunchKernelGGL((linear_skinny_kernel<false, 8>), dim3((unsigned)(g.N / 16)), dim3(512), 0,
                         as_stream(stream), g);
    } else {
      hipLaunchKernelGGL((linear_skinny_kernel<false, 4>), dim3((unsigned)(g.N / 16)), dim3(256), 0,
                         as_stream(stream), g);
    }
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
  }
  // 256-row or 128-row tiles, whichever takes fewer rounds of one
  // workgroup per CU, a 128-row tile costing ~0.6 of a 256-row one (half
  // the products at more LDS reads per product, measured on MI355X)
  const int64_t tiles_n = (g.N + kBN - 1) / kBN;
  const int64_t rounds_big = ((g.M + 255) / 256 * tiles_n + kCUs - 1) / kCUs;
  const int64_t rounds_small = ((g.M + 127) / 128 * tiles_n + kCUs - 1) / kCUs;
  const bool big = 10 * rounds_big <= 6 * rounds_small;
  const int bm = big ? 256 : 128;
  g.tiles_m = (g.M + bm - 1) / bm;
  const int64_t tiles = (int64_t)g.tiles_m * tiles_n;
  if (tiles == 0) return PKV_OK;
  g.tiles_per_xcd = (int32_t)((tiles + kXcds - 1) / kXcds);
  if ((int64_t)g.tiles_per_xcd * kXcds > INT32_MAX) return PKV_ERANGE;
  const dim3 grid((unsigned)(g.tiles_per_xcd * kXcds));
  if (rope && big)
    hipLaunchKernelGGL((linear_kernel<true, 64>), grid, dim3(kThreads), 0, as_stream(stream), g);
  else if (rope)
    hipLaunchKernelGGL((linear_kernel<true, 32>), grid, dim3(kThreads), 0, as_stream(stream), g);
  else if (big)
    hipLaunchKernelGGL((linear_kernel<false, 64>), grid, dim3(kThreads), 0, as_stream(stream), g);
  else
    hipLaunchKernelGGL((linear_kernel<false, 32>), grid, dim3(kThreads), 0, as_stream(stream), g);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // namespace

extern "C" {

int pkv_linear(const pkv_bf16 *x, const pkv_bf16 *w, int32_t M, int32_t N, int32_t K, pkv_bf16 *y,
               pkv_stream_t stream) {
  if (M < 0 || N < 0 || K < 0) return PKV_EINVAL;
  if (N % kHead != 0 || K % kBK != 0) return PKV_EUNSUPPORTED;
  if (M == 0 || N == 0) return PKV_OK;
  if (K == 0) return PKV_EUNSUPPORTED;
  if (!x || !w || !y) return PKV_EINVAL;
  LinearArgs g{};
  g.x = x;
  g.w = w;
  g.y = y;
  g.M = M;
  g.N = N;
  g.K = K;
  return launch_linear(g, false, stream);
}

int pkv_qkv_rope(const pkv_bf16 *x, const pkv_bf16 *w_qkv, int32_t num_rows, int32_t hidden,
                 const int32_t *cu_seqlens_q, const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                 int32_t num_kv_heads, float rope_theta, pkv_bf16 *q, pkv_bf16 *k_new, pkv_bf16 *v_new,
                 pkv_stream_t stream) {
  if (num_rows < 0 || hidden <= 0 || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0) return PKV_EINVAL;
  if (hidden % kBK != 0) return PKV_EUNSUPPORTED;
  if (!(rope_theta > 1.f) || !std::isfinite(rope_theta)) return PKV_EINVAL;
  if (num_rows == 0) return PKV_OK;
  if (!x || !w_qkv || !cu_seqlens_q || !seq_lens || !q || !k_new || !v_new || num_seqs == 0) return PKV_EINVAL;
  LinearArgs g{};
  g.x = x;
  g.w = w_qkv;
  g.M = num_rows;
  g.N = (num_q_heads + 2 * num_kv_heads) * pkv::kHeadDim;
  g.K = hidden;
  g.q = q;
  g.k = k_new;
  g.v = v_new;
  g.cu = cu_seqlens_q;
  g.seq_lens = seq_lens;
  g.S = num_seqs;
  g.Hq = num_q_heads;
  g.Hkv = num_kv_heads;
  g.rope_log2_step = std::log2((double)rope_theta) * 2.0 / pkv::kHeadDim;
  return launch_linear(g, true, stream);
}

int pkv_layer_forward(const pkv_bf16 *x, const pkv_bf16 *w_qkv, const pkv_bf16 *w_o, int32_t hidden,
                      pkv_bf16 *k_cache, pkv_bf16 *v_cache, const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                      const int32_t *block_tables, int32_t bt_stride, int64_t num_blocks, int64_t *slot_mapping,
                      float scale, float rope_theta, const pkv_plan_t *plan, void *ws, size_t ws_bytes,
                      pkv_bf16 *q, pkv_bf16 *k_new, pkv_bf16 *v_new, pkv_bf16 *attn, pkv_bf16 *y,
                      pkv_stream_t stream) {
  // the scale is checked by pkv_paged_step too; here it is checked before
  // the projection is launched
  if (!plan || !(scale > 0.f && scale <= FLT_MAX)) return PKV_EINVAL;
  // the output projection's features are the hidden size: checked before
  // anything is launched
  if (hidden <= 0 || hidden % kHead != 0) return PKV_EUNSUPPORTED;
  if ((plan->num_q_heads * pkv::kHeadDim) % kBK != 0) return PKV_EUNSUPPORTED;
  int st = pkv_qkv_rope(x, w_qkv, plan->num_rows, hidden, cu_seqlens_q, seq_lens, plan->num_seqs,
                        plan->num_q_heads, plan->num_kv_heads, rope_theta, q, k_new, v_new, stream);
  if (st != PKV_OK) return st;
  st = pkv_paged_step(q, k_new, v_new, k_cache, v_cache, cu_seqlens_q, seq_lens, block_tables, bt_stride,
                      num_blocks, slot_mapping, scale, plan, ws, ws_bytes, attn, stream);
  if (st != PKV_OK) return st;
  return pkv_linear(attn, w_o, plan->num_rows, hidden, plan->num_q_heads * pkv::kHeadDim, y, stream);
}

}  // extern "C"
