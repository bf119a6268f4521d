/*
 * pkv.h -- C ABI of libpkv: one packed, ragged attention step over a paged
 * KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The step (one transformer layer's attention in one scheduler iteration):
 *   1. slot translation: every packed query row gets the physical slot of its
 *      position, slot = block_table[s][pos / 16] * 16 + pos % 16
 *      ("连续批处理与 PagedAttention 原理", section "block table 与地址映射");
 *   2. append: the step's new K/V rows are written into their slots
 *      ("continuous batching" (k4i.top), section "与 KV cache 的关系": a chunk's
 *      new KV entries are written to the cache, later chunks read them back);
 *   3. plan: the ragged batch is cut into work items (decode rows split over
 *      the key axis, prefill rows tiled over query positions), on the host;
 *   4. attention: each row attends to its own request's keys under the
 *      block-diagonal causal mask M_ij = 0 iff req(i) = req(j) and j <= i
 *      ("continuous batching" (k4i.top), section "防止跨请求 attention"),
 *      out = softmax(scale * q K^T + M) V, with the request boundaries given
 *      by cu_seqlens of shape [requests + 1] ("11.2 连续批处理与 PagedAttention",
 *      section 11.2.2) and GQA: query head h reads kv head h / (Hq / Hkv);
 *   5. merge: key-split partial results are combined (log-sum-exp merge).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless the name starts with h_ (host).
 * - The caller owns every buffer; the library never allocates or frees
 *   device or host memory and keeps no state between calls.
 * - bf16 tensors are passed as pkv_bf16 (the 16-bit pattern).
 * - `stream` is a hipStream_t (NULL = the null stream).  Every device call is
 *   asynchronous on that stream; the return value only reports host-side
 *   argument validation and launch errors.
 * - Integer metadata is int32; slots are int64.
 * - Supported shapes: head_dim 128, block size 16, Hq % Hkv == 0 with
 *   Hq / Hkv in {1, 2, 4, 8, 16}.  Anything else returns PKV_EUNSUPPORTED.
 *
 * Paged pool layout (the pages fix only the slot translation and that a
 * block's 16 tokens are contiguous; they leave the tensor layout open):
 *   k_cache : bf16[num_blocks][Hkv][4][16][32]  4 KiB tiles: four groups of
 *             32 dimensions, each group token-major
 *   v_cache : bf16[num_blocks][Hkv][2][128][8]  4 KiB tiles: two halves of
 *             8 tokens, each half dimension-major
 * Slot x is block x / 16, offset x % 16.  Key element (o, d) of a tile sits
 * at (d / 32) * 512 + o * 32 + d % 32; value element (o, d) at
 * (o / 8) * 1024 + d * 8 + o % 8.  (Both orders let a 16-byte-per-lane load
 * over 16 tokens read whole cache lines in the operand order of the bf16
 * MFMAs; the halves make a lone appended token touch 64 of the value tile's
 * 32-byte sectors, not 128.)
 *
 * Packed tensors:
 *   q        : bf16[T][Hq][128]      k_new, v_new : bf16[T][Hkv][128]
 *   out      : bf16[T][Hq][128]      slot_mapping : int64[T]
 *   cu_seqlens_q : int32[S + 1], cu[0] = 0, non-decreasing, cu[S] = T
 *   seq_lens : int32[S], keys visible to the sequence's last row AFTER this
 *              step's rows are appended (cached prefix + q_len); row j of
 *              sequence s sits at position seq_lens[s] - q_len_s + j
 *   block_tables : int32[S][bt_stride]; entries past the sequence's last
 *              needed block (ceil(seq_lens[s] / 16)) are never read.
 * Sequences with q_len = 0 are allowed and contribute nothing.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t pkv_bf16;
typedef void *pkv_stream_t; /* hipStream_t */

#define PKV_BLOCK_SIZE 16
#define PKV_HEAD_DIM 128
#define PKV_ITEM_INTS 8
#define PKV_MERGE_INTS 4

enum pkv_status {
  PKV_OK = 0,
  PKV_EINVAL = 1,        /* malformed argument (null pointer, bad metadata) */
  PKV_ERANGE = 2,        /* a size or index does not fit (e.g. block id) */
  PKV_EUNSUPPORTED = 3,  /* head_dim / GQA ratio outside the supported set */
  PKV_EWORKSPACE = 4,    /* workspace or host staging buffer too small */
  PKV_EHIP = 5           /* the HIP runtime reported an error */
};

/* Static description of a status code. */
const char *pkv_status_string(int status);

/* Library ABI version (major * 100 + minor). */
int pkv_version(void);

/* ---------------------------------------------------------------------------
 * Slot translation ("连续批处理与 PagedAttention 原理", section "block table
 * 与地址映射": logical block p / 16 -> physical block b -> offset b*16 + p%16).
 * For every packed row t of sequence s at position pos:
 *   slot_mapping[t] = block_tables[s * bt_stride + pos / 16] * 16 + pos % 16
 * A row whose table entry is outside [0, num_blocks) gets slot -1 (the append
 * then skips it).  Errors: PKV_EINVAL for null pointers or negative sizes,
 * PKV_EHIP on launch failure.  Metadata is not otherwise validated on the
 * device; validate it on the host with pkv_plan.
 * ------------------------------------------------------------------------- */
int pkv_slot_mapping(const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                     const int32_t *block_tables, int32_t bt_stride,
                     int32_t num_seqs, int32_t num_rows, int64_t num_blocks,
                     int64_t *slot_mapping, pkv_stream_t stream);

/* ---------------------------------------------------------------------------
 * Paged KV append ("continuous batching" (k4i.top), section "与 KV cache 的关
 * 系"; "11.2 连续批处理与 PagedAttention", section 11.2.2: the new K and V are
 * appended to their request's cache).  Bit-exact copy of k_new[t] and
 * v_new[t] (all kv heads) into slot slot_mapping[t] of k_cache / v_cache in
 * the layout above.  Rows whose slot is negative or >= num_blocks * 16 are
 * skipped.  Two rows with the same slot race (undefined).  Errors as for
 * pkv_slot_mapping.
 * ------------------------------------------------------------------------- */
int pkv_paged_kv_append(const pkv_bf16 *k_new, const pkv_bf16 *v_new,
                        const int64_t *slot_mapping, int32_t num_rows,
                        pkv_bf16 *k_cache, pkv_bf16 *v_cache,
                        int64_t num_blocks, int32_t num_kv_heads,
                        int32_t head_dim, pkv_stream_t stream);

/* ---------------------------------------------------------------------------
 * Slot translation and append in one launch: computes slot_mapping exactly
 * as pkv_slot_mapping (and writes it: device int64[num_rows]) and copies
 * each row's K/V into its slot exactly as pkv_paged_kv_append.  Errors as
 * for pkv_slot_mapping; PKV_EUNSUPPORTED for head_dim != 128.
 * ------------------------------------------------------------------------- */
int pkv_slot_append(const pkv_bf16 *k_new, const pkv_bf16 *v_new,
                    const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                    const int32_t *block_tables, int32_t bt_stride,
                    int32_t num_seqs, int32_t num_rows, int64_t num_blocks,
                    int64_t *slot_mapping, pkv_bf16 *k_cache, pkv_bf16 *v_cache,
                    int32_t num_kv_heads, int32_t head_dim, pkv_stream_t stream);

/* ---------------------------------------------------------------------------
 * Work partitioning (host).  Rows of sequences with q_len > 1 (prefill and
 * chunked prefill, whose causal offset is the cached prefix: "Continuous
 * Batching 深入实现", section "一个 chunked prefill 请求怎么组织 attention")
 * become tiles of query positions x the kv head's query heads; a wide tile
 * (256 columns: up to 256/G positions) is computed by one whole workgroup.
 * The launch has a fixed set of persistent workgroups (rows of eight, one
 * per CU); each walks a list of wide tiles that the plan deals out longest
 * first to the least loaded workgroup -- with at least two tiles per
 * workgroup as pairs of equal cost (tiles j and n - 1 - j of one sequence
 * and kv head), the longer first -- tiles of kv head h to the workgroups
 * of XCD h % 8 when Hkv is a multiple of 8.  Everything else -- decode rows and
 * short tiles ("11.2 连续批处理与 PagedAttention", section 11.2.2: attention
 * runs per request inside one launch) -- is a (tile, kv head) unit whose
 * keys stream through the cache; all units' 32-key chunks are dealt out in
 * equal contiguous shares to a fixed number of wavefronts, splitting a unit
 * wherever a share ends, so every wavefront streams the same number of
 * bytes however ragged the contexts are.  Split units are merged afterwards.
 * The plan also cuts the packed rows into the append's row groups (at most
 * 16 consecutive rows; the rows one sequence appends into one block never
 * split), which pkv_slot_append_planned and pkv_paged_step use.
 *
 * The plan is written to h_staging (host memory; pinned memory lets the copy
 * run asynchronously) and, when ws is not NULL, copied to ws with
 * hipMemcpyAsync on `stream`.  h_staging must stay untouched until that copy
 * has executed.  One plan serves every layer of a step (same metadata).
 *
 * Size query: with h_staging == NULL the call only fills plan->ws_bytes and
 * plan->host_bytes.  With ws == NULL the plan is built on the host only.
 * Validation (host copies): cu[0] == 0, cu non-decreasing, num_rows = cu[S],
 * 0 <= q_len_s <= seq_lens[s]; with h_block_tables given, every entry a
 * sequence needs must lie in [0, num_blocks).  Errors: PKV_EINVAL,
 * PKV_ERANGE, PKV_EUNSUPPORTED, PKV_EWORKSPACE (plan->ws_bytes /
 * plan->host_bytes then hold the sizes needed), PKV_EHIP.
 * ------------------------------------------------------------------------- */
typedef struct pkv_plan_options {
  int32_t narrow_waves;   /* wavefronts sharing the decode work (0 = default:
                             1536; with wide tiles, 64 per row of narrow
                             workgroups, rows sized to the estimated share of
                             the narrow work; at most 2048 with wide tiles) */
  int32_t min_wave_keys;  /* smallest share per wavefront, keys (0 = default) */
  int32_t wide_tiles;     /* -1 auto, 0 never, 1 always use wide prefill tiles */
  int32_t workgroups;     /* persistent workgroups of a launch with wide tiles
                             (0 = default: 256, one per CU of an MI355X; a
                             multiple of 8, at most 256) */
} pkv_plan_options_t;

typedef struct pkv_plan {
  int32_t num_seqs, num_rows, num_q_heads, num_kv_heads, head_dim;
  int32_t num_items;      /* attention work items */
  int32_t num_wide_items; /* wide tiles: items [0, num_wide_items), grouped by workgroup */
  int32_t num_waves;      /* wavefronts walking the remaining items */
  int32_t num_merge;      /* merge entries (one per split output row x head) */
  int32_t num_part_cols;  /* partial-result columns in the workspace */
  int32_t wave_keys;      /* keys per wavefront share */
  int32_t narrow_rows;    /* launch with wide tiles: rows of eight workgroups
                             (at most 32) whose wavefronts first walk the
                             narrow shares */
  int64_t items_off, waves_off, merge_off, ml_off, o_off; /* byte offsets into ws */
  int64_t zero_off;       /* byte offset of a 4 KiB all-zero tile in ws */
  size_t ws_bytes;        /* workspace bytes this plan uses */
  size_t host_bytes;      /* host staging bytes this plan uses */
  int64_t kv_keys;        /* sum over sequences of visible keys (accounting) */
  int64_t visible_pairs;  /* sum over rows of visible keys (accounting) */
  int32_t num_workgroups; /* workgroups of a launch with wide tiles (0 if none) */
  int32_t num_append_groups; /* row groups of the step's append */
  int64_t wg_off;         /* byte offset in ws of int32[num_workgroups + 1]:
                             workgroup j's wide tiles are items
                             [list[j], list[j + 1]) */
  int64_t append_off;     /* byte offset in ws of int32[2 * num_append_groups]:
                             group g is rows [list[2g], list[2g] + list[2g + 1])
                             of the packed batch, at most 16; the groups cover
                             every row once, in order, and the rows a sequence
                             appends into one block lie in one group */
} pkv_plan_t;

int pkv_plan(const int32_t *h_cu_seqlens_q, const int32_t *h_seq_lens,
             int32_t num_seqs, int32_t num_rows, int32_t num_q_heads,
             int32_t num_kv_heads, int32_t head_dim,
             const int32_t *h_block_tables, int32_t bt_stride,
             int64_t num_blocks, const pkv_plan_options_t *opts,
             void *h_staging, size_t h_staging_bytes, void *ws,
             size_t ws_bytes, pkv_plan_t *plan, pkv_stream_t stream);

/* ---------------------------------------------------------------------------
 * Fused varlen paged attention, main launch.  One grid walks the plan's
 * items; decode items and prefill tiles share the launch.  For each row t
 * of sequence s at position pos and query head h:
 *   out[t][h] = sum_{i <= pos} softmax_i(scale * q[t][h] . K_s[i][g]) V_s[i][g]
 * with g = h / (Hq / Hkv) and K_s / V_s read from the pool through the
 * block table ("continuous batching" (k4i.top), section "与 KV cache 的关系",
 * the decode formula with [K_cache; k_t]; visible set of section "为什么
 * packed forward 等价").  Rows whose keys were split write fp32 partial
 * results (running max, sum, unnormalised output) into ws; every other row
 * writes out directly.  Accumulation is fp32; probabilities are rounded to
 * bf16 for the P.V product and the normaliser sums those rounded values;
 * out is rounded to bf16 (nearest even).  q enters the products as stored:
 * prefill tiles and decode items alike apply the scale in fp32, inside each
 * exponent's argument.  Block-table entries outside
 * [0, num_blocks) read as zero keys/values.  scale must be positive and
 * finite (the kernels take maxima of raw scores and scale them afterwards,
 * which only a positive scale commutes with).  Errors: PKV_EINVAL (null
 * pointers, plan mismatch, a scale that is not positive and finite -- checked
 * before anything else), PKV_ERANGE (num_blocks x num_kv_heads above 2^32),
 * PKV_EWORKSPACE, PKV_EHIP.
 * ------------------------------------------------------------------------- */
int pkv_varlen_attention_main(const pkv_bf16 *q, const pkv_bf16 *k_cache,
                              const pkv_bf16 *v_cache,
                              const int32_t *block_tables, int32_t bt_stride,
                              int64_t num_blocks, float scale,
                              const pkv_plan_t *plan, void *ws, size_t ws_bytes,
                              pkv_bf16 *out, pkv_stream_t stream);

/* ---------------------------------------------------------------------------
 * Split-KV merge: for every row and head whose keys were split,
 *   M = max_k m_k,  out = sum_k 2^(m_k - M) o_k / sum_k 2^(m_k - M) l_k
 * (m_k in the base-2 scaled domain of the main launch), rounded to bf16.
 * The pages do not describe this step; it is the standard online-softmax
 * combination and changes nothing but rounding.  A plan with no split rows
 * launches nothing.  Errors as above.
 * ------------------------------------------------------------------------- */
int pkv_split_kv_reduce(const pkv_plan_t *plan, const void *ws,
                        size_t ws_bytes, pkv_bf16 *out, pkv_stream_t stream);

/* pkv_varlen_attention_main followed by pkv_split_kv_reduce. */
int pkv_paged_varlen_attention(const pkv_bf16 *q, const pkv_bf16 *k_cache,
                               const pkv_bf16 *v_cache,
                               const int32_t *block_tables, int32_t bt_stride,
                               int64_t num_blocks, float scale,
                               const pkv_plan_t *plan, void *ws,
                               size_t ws_bytes, pkv_bf16 *out,
                               pkv_stream_t stream);

/* ---------------------------------------------------------------------------
 * The append of pkv_slot_append on the plan's row groups (plan->append_off
 * in ws; same slots, slot_mapping written, same pool bytes): the rows one
 * sequence appends into one block share a workgroup, so every block the step
 * fills is written in whole lines ("continuous batching" (k4i.top), section
 * "与 KV cache 的关系": the step's K and V join the cache; "连续批处理与
 * PagedAttention 原理", section "block table 与地址映射" for the slots).  The
 * first launch of pkv_paged_step; the plan, the metadata and ws are the
 * step's.  Errors: PKV_EINVAL (null pointers, a plan whose row groups do not
 * fit its workspace), PKV_EWORKSPACE (ws_bytes < plan->ws_bytes),
 * PKV_EUNSUPPORTED (plan head_dim != 128), PKV_EHIP.
 * ------------------------------------------------------------------------- */
int pkv_slot_append_planned(const pkv_bf16 *k_new, const pkv_bf16 *v_new,
                            const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                            const int32_t *block_tables, int32_t bt_stride,
                            int64_t num_blocks, int64_t *slot_mapping,
                            pkv_bf16 *k_cache, pkv_bf16 *v_cache,
                            const pkv_plan_t *plan, const void *ws,
                            size_t ws_bytes, pkv_stream_t stream);

/* ---------------------------------------------------------------------------
 * The whole step on one stream: pkv_slot_append_planned (slot_mapping,
 * device int64[T], is written), then pkv_paged_varlen_attention.  Attention reads the cache after the append, so
 * each row sees its own new key.  A scale that is not positive and finite,
 * and a plan whose row groups do not fit its workspace, return PKV_EINVAL
 * before the append is launched.
 * ------------------------------------------------------------------------- */
int pkv_paged_step(const pkv_bf16 *q, const pkv_bf16 *k_new,
                   const pkv_bf16 *v_new, pkv_bf16 *k_cache,
                   pkv_bf16 *v_cache, const int32_t *cu_seqlens_q,
                   const int32_t *seq_lens, const int32_t *block_tables,
                   int32_t bt_stride, int64_t num_blocks,
                   int64_t *slot_mapping, float scale, const pkv_plan_t *plan,
                   void *ws, size_t ws_bytes, pkv_bf16 *out,
                   pkv_stream_t stream);

/* ---------------------------------------------------------------------------
 * pkv_paged_step with no workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The workspace is a fixed array of
 * PKV_STATIC_WS_BYTES (32 MiB) inside the library, one per GPU, held until
 * the process ends; the call allocates nothing (no hipMalloc, no hipFree).
 * Build the plan with pkv_plan(..., h_staging, ..., ws = NULL, ...); this
 * call copies its plan->host_bytes of h_staging (host memory the caller
 * owns; pinned lets the copy run asynchronously, and h_staging must then
 * stay untouched until the copy has executed) into the array on `stream`,
 * then runs pkv_paged_step on it.  Inputs, outputs and their meaning are
 * those of pkv_paged_step.  Every call on one GPU shares that GPU's array,
 * which keeps the last call's contents: calls on one stream are ordered,
 * but calls that overlap on one GPU (two streams, or two host threads
 * without ordering) race.  Errors: PKV_EWORKSPACE when plan->ws_bytes
 * exceeds PKV_STATIC_WS_BYTES (checked before any device call), PKV_EINVAL
 * for a null plan or staging buffer or a scale that is not positive and
 * finite, PKV_ERANGE for a device index of 64 or more, and those of
 * pkv_paged_step.
 * ------------------------------------------------------------------------- */
#define PKV_STATIC_WS_BYTES (32u << 20)
int pkv_paged_step_static(const pkv_bf16 *q, const pkv_bf16 *k_new,
                          const pkv_bf16 *v_new, pkv_bf16 *k_cache,
                          pkv_bf16 *v_cache, const int32_t *cu_seqlens_q,
                          const int32_t *seq_lens, const int32_t *block_tables,
                          int32_t bt_stride, int64_t num_blocks,
                          int64_t *slot_mapping, float scale,
                          const pkv_plan_t *plan, const void *h_staging,
                          pkv_bf16 *out, pkv_stream_t stream);

/* ===========================================================================
 * The weight layers around the step: one packed layer.
 * ======================================================================== */

/* ---------------------------------------------------------------------------
 * Linear layer over all packed rows ("11.2 连续批处理与 PagedAttention",
 * section 11.2.2: the weight layers take the step's rows of every request
 * as one matrix, X[7, 4096] x W_Q[4096, 4096] -> Q[7, 4096] in the worked
 * example; "continuous batching" (k4i.top), section "把 prefill 和 decode
 * 打包在一起": Q = X W_Q over the packed rows).
 *   y[m][n] = sum_k x[m][k] * w[n][k]
 * x: device bf16[M][K] row-major; w: device bf16[N][K] (weights stored
 * [out features][in features], the transpose of the pages' W_Q); y: device
 * bf16[M][N].  fp32 accumulation, bf16 result (nearest even).  N must be a
 * multiple of 128 and K a positive multiple of 64 (PKV_EUNSUPPORTED
 * otherwise); M is any size.  Errors: PKV_EINVAL (null pointer, negative
 * size), PKV_ERANGE (grid too large), PKV_EHIP.
 * ------------------------------------------------------------------------- */
int pkv_linear(const pkv_bf16 *x, const pkv_bf16 *w, int32_t M, int32_t N, int32_t K, pkv_bf16 *y,
               pkv_stream_t stream);

/* ---------------------------------------------------------------------------
 * Fused QKV projection with RoPE (same passages; k4i.top: RoPE sees each
 * request's own position id).  w_qkv: device bf16[(Hq + 2 Hkv) * 128][hidden],
 * the query heads' 128 rows each, then the key heads', then the value
 * heads'.  For packed row t of sequence s at position
 * p = seq_lens[s] - q_len_s + (t - cu_seqlens_q[s]) (device int32 arrays of
 * num_seqs + 1 and num_seqs entries), the projection x[t] w_qkv^T is split
 * into heads; every query and key head is rotated: for i < 64 the pair
 * (d_i, d_{i+64}) turns by the angle p * rope_theta^(-2i/128) (RoFormer's
 * rotation with the two halves of a head as the pair's parts; the pages do
 * not give the formula), values are not.  Outputs: q bf16[T][Hq][128],
 * k_new and v_new bf16[T][Hkv][128] -- the step's inputs.  hidden must be a
 * multiple of 64; rope_theta > 1 (PKV_EINVAL otherwise).
 * ------------------------------------------------------------------------- */
int pkv_qkv_rope(const pkv_bf16 *x, const pkv_bf16 *w_qkv, int32_t num_rows, int32_t hidden,
                 const int32_t *cu_seqlens_q, const int32_t *seq_lens, int32_t num_seqs, int32_t num_q_heads,
                 int32_t num_kv_heads, float rope_theta, pkv_bf16 *q, pkv_bf16 *k_new, pkv_bf16 *v_new,
                 pkv_stream_t stream);

/* ---------------------------------------------------------------------------
 * One packed attention layer on one stream ("11.2 连续批处理与
 * PagedAttention", section 11.2.2: weight layers over all rows, the new K
 * and V appended to each request's cache, attention per request, results
 * back as one [T, 4096] matrix): pkv_qkv_rope, pkv_paged_step, then
 * y = attn w_o^T with pkv_linear.  w_o: device bf16[hidden][Hq * 128].
 * The caller provides q, k_new, v_new (as above) and attn bf16[T][Hq][128];
 * y: bf16[T][hidden].  The plan, workspace, pools and metadata are those of
 * pkv_paged_step.  hidden must be a multiple of 128 (PKV_EUNSUPPORTED) and
 * scale positive and finite (PKV_EINVAL), both checked before anything is
 * launched.  Errors: those of the three calls.
 * ------------------------------------------------------------------------- */
int pkv_layer_forward(const pkv_bf16 *x, const pkv_bf16 *w_qkv, const pkv_bf16 *w_o, int32_t hidden,
                      pkv_bf16 *k_cache, pkv_bf16 *v_cache, const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                      const int32_t *block_tables, int32_t bt_stride, int64_t num_blocks, int64_t *slot_mapping,
                      float scale, float rope_theta, const pkv_plan_t *plan, void *ws, size_t ws_bytes,
                      pkv_bf16 *q, pkv_bf16 *k_new, pkv_bf16 *v_new, pkv_bf16 *attn, pkv_bf16 *y,
                      pkv_stream_t stream);

/* ===========================================================================
 * Block pool, copy-on-write and swap (the steps either side of the append).
 * ======================================================================== */

/* ---------------------------------------------------------------------------
 * Host block pool ("连续批处理与 PagedAttention 原理", section "块管理器": the
 * physical block pool records which blocks are free and a reference count
 * per block in use; its operations are allocate, free and copy-on-write.
 * "11.2 连续批处理与 PagedAttention", section 11.2.3 (sharing): several logical
 * blocks may map to one physical block; when the output sequences of one
 * request share the prompt's blocks, only a shared block that is not yet
 * full is copied before a sequence writes into it; shared full prefix
 * blocks are read-only and need no copy).
 *
 * Host memory only; no GPU call.  Free blocks form a stack: allocation pops
 * the top, a block whose count drops to zero is pushed on top, and a new pool
 * has block 0 on top, then 1, 2, ...  Not thread-safe: one pool, one thread
 * at a time.  Errors: PKV_EINVAL (null pointer, negative size, a table row
 * naming a block not in use), PKV_ERANGE (not enough free blocks, an id
 * outside the pool, more releases than references).  A call that fails
 * changes nothing.
 * ------------------------------------------------------------------------- */
typedef struct pkv_block_pool pkv_block_pool_t;

int pkv_block_pool_create(int64_t num_blocks, pkv_block_pool_t **pool);
void pkv_block_pool_destroy(pkv_block_pool_t *pool);
/* blocks an allocation can take: free ones plus evictable cached ones (-1
 * for a null pool) */
int64_t pkv_block_pool_num_free(const pkv_block_pool_t *pool);
/* registered prefix blocks, in use or evictable (-1 for a null pool) */
int64_t pkv_block_pool_num_cached(const pkv_block_pool_t *pool);
/* references to `block` (0 = free; -1 for an id outside the pool) */
int32_t pkv_block_pool_refcount(const pkv_block_pool_t *pool, int32_t block);
/* n blocks, each with one reference, written to h_blocks[0..n) */
int pkv_block_pool_allocate(pkv_block_pool_t *pool, int32_t n, int32_t *h_blocks);
/* one more reference to each listed block (a forked sequence, or a prefix
 * reused by another request, maps the same physical blocks) */
int pkv_block_pool_share(pkv_block_pool_t *pool, const int32_t *h_blocks, int32_t n);
/* one reference fewer to each listed block (repeats count); blocks that
 * reach zero become free, or evictable (queued in the order listed) if
 * registered as a prefix block */
int pkv_block_pool_release(pkv_block_pool_t *pool, const int32_t *h_blocks, int32_t n);
/* Prepare a sequence's block-table row (h_table_row, `capacity` entries)
 * for writing num_new tokens after its num_tokens: if the block that
 * position num_tokens falls in is already held and has more than one
 * reference, it is replaced in the row by a newly allocated block, the old
 * one loses this reference, and the pair (old, new) is written to
 * h_copies[0..2) (*num_copies = 1): the caller copies old -> new on the
 * device (pkv_copy_blocks) before appending.  Then every further block the
 * new tokens need is allocated into the row.  *num_copies = 0 when nothing
 * is to be copied (h_copies may then be NULL). */
int pkv_block_pool_append_slots(pkv_block_pool_t *pool, int32_t *h_table_row, int32_t capacity,
                                int32_t num_tokens, int32_t num_new, int32_t *h_copies,
                                int32_t *num_copies);

/* ---------------------------------------------------------------------------
 * Prefix caching ("11.2 连续批处理与 PagedAttention", section 11.2.4: every
 * full block gets a hash computed from its parent block's hash, its own
 * tokens and extra keys; the blocks of a finished request stay in an
 * evictable queue until a new request hits them or they are pushed out; a
 * reuse needs a token-exact match, and the key must also carry whatever
 * changes the KV or its visibility -- model and version, adapter,
 * multimodal content hash, tenant salt -- here folded by the caller into
 * one 64-bit extra_key).
 *
 * pkv_block_hash: FNV-1a, 64 bits (offset basis 0xcbf29ce484222325, prime
 * 0x100000001b3), over the little-endian bytes of parent (8), the block's
 * 16 token ids h_tokens[0..16) (4 each) and extra_key (8); block 0's parent
 * is 0.  Returns 0 for a null h_tokens.
 *
 * pkv_block_pool_match_prefix: for a prompt h_tokens[0..num_tokens), walks
 * its full blocks from block 0 -- only blocks that leave at least one
 * prompt token to compute, at most `capacity` -- and stops at the first
 * block with no registered entry whose tokens, extra key and parent entry
 * all equal the prompt's (a hash match alone is not enough).  The matched
 * blocks are written to h_table_row[0..k), each gains one reference (an
 * evictable one leaves the queue), and *num_cached_tokens = 16 k: the
 * caller appends and computes only the tokens after it
 * (pkv_block_pool_append_slots with num_tokens = 16 k).
 *
 * pkv_block_pool_register_prefix: registers the full blocks of a computed
 * sequence (tokens h_tokens[0..num_tokens), table h_table_row, every full
 * block in use) from block 0 on; a block already registered for the same
 * content is kept, an entry under the same hash holding other content is
 * replaced, and the walk stops at a block registered under another hash.
 * Registration does not change counts.
 *
 * Eviction: allocation takes free blocks first, then the evictable block
 * that was released longest ago, and drops its registration.  Release a
 * finished request's blocks last block first so that the head of a prefix,
 * which every later hit needs, is evicted last.  Errors: PKV_EINVAL for a
 * null pointer, a negative size or a table entry not in use.
 * ------------------------------------------------------------------------- */
uint64_t pkv_block_hash(uint64_t parent, const int32_t *h_tokens, uint64_t extra_key);
int pkv_block_pool_match_prefix(pkv_block_pool_t *pool, const int32_t *h_tokens, int32_t num_tokens,
                                uint64_t extra_key, int32_t *h_table_row, int32_t capacity,
                                int32_t *num_cached_tokens);
int pkv_block_pool_register_prefix(pkv_block_pool_t *pool, const int32_t *h_tokens, int32_t num_tokens,
                                   uint64_t extra_key, const int32_t *h_table_row);

/* ---------------------------------------------------------------------------
 * Copy-on-write on the device: for p in [0, num_pairs), block
 * block_pairs[2p] is copied bit for bit onto block block_pairs[2p + 1], K
 * and V, every kv head (block_pairs: device int32[num_pairs][2]).  Pairs
 * with an id outside [0, num_blocks) or src == dst are skipped; two pairs
 * with the same destination, or a destination that is another pair's
 * source, race (undefined).  Errors as for pkv_paged_kv_append.
 * ------------------------------------------------------------------------- */
int pkv_copy_blocks(pkv_bf16 *k_cache, pkv_bf16 *v_cache, int64_t num_blocks, int32_t num_kv_heads,
                    int32_t head_dim, const int32_t *block_pairs, int32_t num_pairs, pkv_stream_t stream);

/* ---------------------------------------------------------------------------
 * Swap preemption ("连续批处理与 PagedAttention 原理", section "抢占策略": the
 * KV cache of a preempted sequence is copied to CPU memory and copied back
 * when it resumes, at the cost of PCIe bandwidth and host memory;
 * "Continuous Batching 深入实现", section "Preemption 与 Recompute vs Swap").
 * pkv_swap_out copies blocks[p] (device int32[num]) of both pools into
 * host_dst + p * 2 * S, K first, then V, where S = num_kv_heads * 16 * 128
 * bf16 elements is one block of one pool, in the pools' own tile layout;
 * pkv_swap_in copies them back into blocks[p].  The host buffer must be
 * page-locked, device-mapped host memory (hipHostMalloc, or a pinned torch
 * tensor) of at least num * 2 * S * 2 bytes; the kernels read or write it
 * directly.  Ids outside [0, num_blocks) are skipped (their host slot is
 * left untouched on the way out and ignored on the way in).  Errors as for
 * pkv_paged_kv_append; PKV_EINVAL also for a host buffer that is not
 * device-mapped.
 * ------------------------------------------------------------------------- */
int pkv_swap_out(const pkv_bf16 *k_cache, const pkv_bf16 *v_cache, int64_t num_blocks, int32_t num_kv_heads,
                 int32_t head_dim, const int32_t *blocks, int32_t num, void *host_dst, pkv_stream_t stream);
int pkv_swap_in(const void *host_src, const int32_t *blocks, int32_t num, pkv_bf16 *k_cache, pkv_bf16 *v_cache,
                int64_t num_blocks, int32_t num_kv_heads, int32_t head_dim, pkv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
