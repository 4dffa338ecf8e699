// Host-side argument checks and workspace layouts of every entry point:
// plain C++ with no HIP in it, so that the same code runs inside the library
// and in a CPU build under the address and undefined-behaviour sanitizers.
// Each function returns the status the entry point returns, in the order the
// entry point checks (shape, then pointers, then dtypes, then alignment, then
// the workspace); the launch code only runs after PA_OK.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "padecode.h"
#include "pa_internal.h"

namespace pa_host {

constexpr int kPageTokens = 16;          // tokens per page (pa_shape::block_size)
constexpr int kMaxGroup = 16;            // query heads per KV head one matrix-core tile covers
constexpr int kBalancedMaxBatch = 4096;  // sequences the balanced split's workgroup scan covers
constexpr int kMaxQLen = 16;             // new tokens per sequence of the multi-token decode
constexpr int kChunkTiles = 2;           // 16-row tiles per workgroup of the wide-row kernel
constexpr int kMergeThreads = 256;       // threads per workgroup of the log-sum-exp merge
constexpr long long kInt32Max = 0x7fffffffLL;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// ---------------------------------------------------------------------------
// Single-tile decode (pa_decode, pa_decode_noalloc, and pa_decode_multi when
// group * q_len <= 16).
// ---------------------------------------------------------------------------
struct DecodeLayout {
  size_t o_off, lse_off, cnt_off, total;
  int p_max, fan, g_max;
  size_t cnt_bytes;   // bytes of counters the call uses (from cnt_off)
};

inline bool decode_shape_ok(const pa_shape* s) {
  if (!s) return false;
  if (s->batch < 0 || s->batch > 65535) return false;
  if (s->num_kv_heads < 1 || s->num_kv_heads > 65535) return false;
  if (s->num_q_heads < 1 || s->num_q_heads % s->num_kv_heads != 0) return false;
  if (s->num_q_heads / s->num_kv_heads > kMaxGroup) return false;
  if (s->head_dim != 64 && s->head_dim != 128) return false;
  if (s->block_size != kPageTokens) return false;
  if (s->max_blocks_per_seq < 1 || s->max_blocks_per_seq > (1 << 26)) return false;
  if (s->num_blocks < 1) return false;
  if (s->partition_size == PA_SPLIT_BALANCED) {
    // the workgroup-wide scan covers the batch, and line positions fit int32
    if (s->batch > kBalancedMaxBatch) return false;
    const long long line = (long long)s->batch * s->num_kv_heads * s->max_blocks_per_seq;
    return line + 4096LL * 3 < kInt32Max;   // + shares (4096 CUs at most, 3 per CU)
  }
  if (s->partition_size < 0 || s->partition_size % kPageTokens != 0) return false;
  // work units B * Hkv * partitions, and the partition and group slots, must
  // fit a 1-D grid and int32 slot numbers
  const long long parts =
      s->partition_size
          ? ((long long)s->max_blocks_per_seq * kPageTokens + s->partition_size - 1) / s->partition_size
          : 1;
  const int fan = pa::merge_fan(parts);
  const long long groups = fan ? (parts + fan - 1) / fan : 0;
  if ((long long)s->batch * s->num_kv_heads * (parts + groups) > kInt32Max) return false;
  return true;
}

// shares: the balanced split's workgroup count (ignored otherwise); q_len:
// new tokens per sequence (rows per pair = group * q_len); cnt_region: 0 to
// pack the counters first (rounded up to 256 bytes), else the partial results
// start at that fixed byte offset, so counters and partials of calls of any
// shape never overlap (the no-allocation entry point's scratch).
inline DecodeLayout decode_layout(const pa_shape* s, int shares, int q_len, size_t cnt_region = 0) {
  DecodeLayout w{0, 0, 0, 0, 1, 0, 0, 0};
  if (s->partition_size == 0) return w;
  const size_t nbg = (size_t)s->batch * s->num_kv_heads;
  size_t slots;
  if (s->partition_size == PA_SPLIT_BALANCED) {
    w.p_max = 0;
    slots = (size_t)shares + nbg;
  } else {
    const long long tokens = (long long)s->max_blocks_per_seq * kPageTokens;
    w.p_max = (int)((tokens + s->partition_size - 1) / s->partition_size);
    w.fan = pa::merge_fan(w.p_max);
    w.g_max = w.fan ? (w.p_max + w.fan - 1) / w.fan : 0;
    slots = nbg * (w.p_max + w.g_max);   // partition slots, then group slots
  }
  const size_t rows = slots * (size_t)(s->num_q_heads / s->num_kv_heads) * q_len;
  // counters first (one per (b, g), then g_max per (b, g)): every completed
  // call leaves them zero, so a later call whose counters fit in the same
  // bytes finds them zero
  w.cnt_off = 0;
  w.cnt_bytes = nbg * (1 + (size_t)w.g_max) * sizeof(uint32_t);
  w.o_off = cnt_region ? cnt_region : align_up(w.cnt_bytes, 256);
  w.lse_off = w.o_off + align_up(rows * s->head_dim * sizeof(float), 256);
  w.total = w.lse_off + align_up(rows * sizeof(float), 256);
  return w;
}

// The shape checks of a single-tile call with q_len new tokens per sequence.
inline pa_status decode_shape_status(const pa_shape* s, int q_len) {
  if (!s) return PA_ERR_NULL;
  if (!decode_shape_ok(s) || q_len < 1) return PA_ERR_SHAPE;
  const int G = s->num_q_heads / s->num_kv_heads;
  if ((long long)G * q_len > pa::kTileRows) return PA_ERR_SHAPE;
  if ((long long)s->batch * q_len * s->num_q_heads > kInt32Max) return PA_ERR_SHAPE;
  return PA_OK;
}

// Pointer, dtype and alignment checks shared by the decode entry points.
inline pa_status io_args_status(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* context_lens,
                                pa_dtype io_dtype, pa_dtype kv_dtype, const float* k_scale,
                                const float* v_scale, const void* out, const float* lse_out) {
  if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out) return PA_ERR_NULL;
  const bool io_ok = io_dtype == PA_F32 || io_dtype == PA_F16 || io_dtype == PA_BF16;
  const bool kv_ok = kv_dtype == io_dtype || (kv_dtype == PA_FP8_E4M3 && io_dtype != PA_F32);
  if (!io_ok || !kv_ok) return PA_ERR_DTYPE;
  if (kv_dtype == PA_FP8_E4M3 && (!k_scale || !v_scale)) return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return PA_ERR_ALIGN;
  if (!aligned(block_table, 4) || !aligned(context_lens, 4) || !aligned(lse_out, 4))
    return PA_ERR_ALIGN;
  return PA_OK;
}

// The workspace checks of a split call (partition_size != 0) needing `need`
// bytes. cnt_region != 0 marks the no-allocation scratch, whose counter
// region holds cnt_region bytes: calls beyond either limit are refused first.
inline pa_status workspace_status(int partition_size, size_t need, size_t cnt_bytes,
                                  size_t cnt_region, const void* workspace,
                                  size_t workspace_bytes) {
  if (partition_size == 0) return PA_OK;
  if (cnt_region && (cnt_bytes > cnt_region || need > workspace_bytes)) return PA_ERR_SCRATCH;
  if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return PA_ERR_ALIGN;
  return PA_OK;
}

// ---------------------------------------------------------------------------
// Shared-prefix decode (pa_decode_prefix): the balanced split with the first
// prefix_blocks pages read once for every sequence.
// ---------------------------------------------------------------------------
constexpr int kPrefixPieces = 8;   // pieces of one prefix unit, at most (slots per pair beyond its own)

// Workspace: one counter per (sequence, KV head), then partial slots for
// shares + pairs * (1 + kPrefixPieces) pieces of G rows each.
inline DecodeLayout prefix_layout(const pa_shape* s, int shares) {
  DecodeLayout w{0, 0, 0, 0, 0, 0, 0, 0};
  const size_t nbg = (size_t)s->batch * s->num_kv_heads;
  const size_t slots = (size_t)shares + nbg * (1 + kPrefixPieces);
  const size_t rows = slots * (size_t)(s->num_q_heads / s->num_kv_heads);
  w.cnt_bytes = nbg * sizeof(uint32_t);
  w.o_off = align_up(w.cnt_bytes, 256);
  w.lse_off = w.o_off + align_up(rows * s->head_dim * sizeof(float), 256);
  w.total = w.lse_off + align_up(rows * sizeof(float), 256);
  return w;
}

// Shape checks of pa_decode_prefix that need no device: a balanced-split
// decode shape, 0 <= prefix_blocks <= max_blocks_per_seq, and a prefix line
// whose work (H * passes * prefix_blocks positions of cost up to 4, passes =
// groups of four 16-row tiles of 16 / G sequences) fits int32 beside the
// suffix line.
inline pa_status prefix_shape_status(const pa_shape* s, int prefix_blocks) {
  const pa_status st = decode_shape_status(s, 1);
  if (st != PA_OK) return st;
  if (s->partition_size != PA_SPLIT_BALANCED) return PA_ERR_SHAPE;
  if (prefix_blocks < 0 || prefix_blocks > s->max_blocks_per_seq) return PA_ERR_SHAPE;
  const int G = s->num_q_heads / s->num_kv_heads;
  const long long mpt = pa::kTileRows / G;
  const long long ntile = (s->batch + mpt - 1) / mpt;
  const long long passes = (ntile + 3) / 4;
  const long long line = (long long)s->batch * s->num_kv_heads * s->max_blocks_per_seq;
  if (4LL * s->num_kv_heads * passes * prefix_blocks + line >= kInt32Max) return PA_ERR_SHAPE;
  return PA_OK;
}

// With `shares` workgroups: at least two (one prefix share, one suffix
// share), and partial outputs addressable with 32-bit byte offsets.
inline pa_status prefix_shares_status(const pa_shape* s, int shares) {
  if (shares < 2) return PA_ERR_SHAPE;
  const DecodeLayout w = prefix_layout(s, shares);
  if (w.lse_off - w.o_off > 0xfffffff0ull) return PA_ERR_SHAPE;
  return PA_OK;
}

// Workgroups of a single-tile launch: one per (sequence, KV head, partition)
// unit, or one per share of the balanced split.
inline unsigned decode_grid(const pa_shape* s, const DecodeLayout& w, int shares) {
  if (s->partition_size == PA_SPLIT_BALANCED) return (unsigned)shares;
  return (unsigned)((long long)s->batch * s->num_kv_heads * w.p_max);
}

// ---------------------------------------------------------------------------
// Wide-row multi-token decode (pa_decode_multi when group * q_len > 16).
// ---------------------------------------------------------------------------
struct MultiPlan {
  int rows, tiles, chunks, p_max, fan, g_max;
  int shares;   // balanced split: workgroups (one share each); 0 otherwise
  size_t cnt_off, o_off, lse_off, total;
};

// True when pa_decode_multi runs this call on the single-tile decode.
inline bool multi_fits_one_tile(const pa_shape* s, int q_len) {
  return s && s->num_kv_heads > 0 && q_len >= 1 && q_len <= kMaxQLen &&
         (long long)(s->num_q_heads / s->num_kv_heads) * q_len <= pa::kTileRows;
}

// shares: the balanced split's workgroup count (partition_size ==
// PA_SPLIT_BALANCED; ignored otherwise, and a balanced plan needs 1 .. 3 * 4096).
inline bool multi_plan(const pa_shape* s, int q_len, MultiPlan* out, int shares = 0) {
  if (!s) return false;
  if (q_len < 1 || q_len > kMaxQLen) return false;
  if (s->batch < 0 || s->batch > 65535) return false;
  if (s->num_kv_heads < 1 || s->num_kv_heads > 65535) return false;
  if (s->num_q_heads < 1 || s->num_q_heads % s->num_kv_heads != 0) return false;
  const int G = s->num_q_heads / s->num_kv_heads;
  if (G > kMaxGroup) return false;
  if ((long long)s->batch * q_len * s->num_q_heads > kInt32Max) return false;
  if (s->head_dim != 64 && s->head_dim != 128) return false;
  if (s->block_size != kPageTokens) return false;
  if (s->max_blocks_per_seq < 1 || s->max_blocks_per_seq > (1 << 26)) return false;
  if (s->num_blocks < 1) return false;
  const bool balanced = s->partition_size == PA_SPLIT_BALANCED;
  if (balanced) {
    // the workgroup-wide scan covers the batch, and line positions fit int32
    if (s->batch > kBalancedMaxBatch || shares < 1 || shares > 3 * 4096) return false;
    const long long line = (long long)s->batch * s->num_kv_heads * s->max_blocks_per_seq;
    if (line + 4096LL * 3 >= kInt32Max) return false;
  } else if (s->partition_size < 0 || s->partition_size % kPageTokens != 0) {
    return false;
  }
  MultiPlan p;
  p.rows = G * q_len;
  p.tiles = (p.rows + 15) / 16;
  p.chunks = (p.tiles + kChunkTiles - 1) / kChunkTiles;
  p.shares = 0;
  if (balanced) {
    // counters: one per (sequence, KV head); partial slots: shares + pairs
    // (piece k of a pair goes to slot first share of the pair + pair index + k)
    const size_t nbg = (size_t)s->batch * s->num_kv_heads;
    const size_t slots = (size_t)shares + nbg;
    p.p_max = 0;
    p.fan = p.g_max = 0;
    p.shares = shares;
    p.cnt_off = 0;
    p.o_off = align_up(nbg * sizeof(uint32_t), 256);
    p.lse_off = p.o_off + align_up(slots * p.rows * s->head_dim * sizeof(float), 256);
    p.total = p.lse_off + align_up(slots * p.rows * sizeof(float), 256);
    *out = p;
    return true;
  }
  const long long tokens = (long long)s->max_blocks_per_seq * kPageTokens;
  p.p_max = s->partition_size ? (int)((tokens + s->partition_size - 1) / s->partition_size) : 1;
  const long long units = (long long)s->batch * s->num_kv_heads * p.chunks * p.p_max;
  if (units > kInt32Max) return false;
  p.fan = s->partition_size ? pa::merge_fan(p.p_max) : 0;
  p.g_max = p.fan ? (p.p_max + p.fan - 1) / p.fan : 0;
  if ((long long)s->batch * s->num_kv_heads * (p.p_max + p.g_max) > kInt32Max) return false;
  p.cnt_off = p.o_off = p.lse_off = p.total = 0;
  if (s->partition_size) {
    // counters first: [B][Hkv][chunks], then [B][Hkv][g_max][chunks]; slots:
    // partitions, then first-level groups
    const size_t nbg = (size_t)s->batch * s->num_kv_heads;
    const size_t slots = nbg * (p.p_max + p.g_max);
    p.o_off = align_up(nbg * (1 + (size_t)p.g_max) * p.chunks * sizeof(uint32_t), 256);
    p.lse_off = p.o_off + align_up(slots * p.rows * s->head_dim * sizeof(float), 256);
    p.total = p.lse_off + align_up(slots * p.rows * sizeof(float), 256);
  }
  *out = p;
  return true;
}

// Workgroups: one per (sequence, KV head, partition, row chunk), or one per
// share of the balanced split.
inline unsigned multi_grid(const pa_shape* s, const MultiPlan& p) {
  if (s->partition_size == PA_SPLIT_BALANCED) return (unsigned)p.shares;
  return (unsigned)((long long)s->batch * s->num_kv_heads * p.chunks * p.p_max);
}

// ---------------------------------------------------------------------------
// pa_kv_append: the status, and in *grid the workgroups (one per (sequence,
// KV head)) when it is PA_OK and the batch is not empty.
// ---------------------------------------------------------------------------
inline pa_status append_status(const pa_shape* s, const void* k_new, const void* v_new,
                               const int32_t* positions, const int32_t* block_table,
                               pa_dtype src_dtype, pa_dtype kv_dtype, const float* k_scale,
                               const float* v_scale, const void* k_cache, const void* v_cache,
                               unsigned* grid) {
  *grid = 0;
  if (!s) return PA_ERR_NULL;
  if (s->batch < 0 || s->num_kv_heads < 1 || s->num_kv_heads > 65535) return PA_ERR_SHAPE;
  if (s->head_dim != 64 && s->head_dim != 128) return PA_ERR_SHAPE;
  if (s->block_size != kPageTokens || s->max_blocks_per_seq < 1 ||
      s->max_blocks_per_seq > (1 << 26) || s->num_blocks < 1)
    return PA_ERR_SHAPE;
  if ((long long)s->batch * s->num_kv_heads > kInt32Max) return PA_ERR_SHAPE;
  if (!k_new || !v_new || !positions || !block_table || !k_cache || !v_cache) return PA_ERR_NULL;
  const bool src_ok = src_dtype == PA_F32 || src_dtype == PA_F16 || src_dtype == PA_BF16;
  if (!src_ok || (kv_dtype != src_dtype && kv_dtype != PA_FP8_E4M3)) return PA_ERR_DTYPE;
  if (kv_dtype == PA_FP8_E4M3 && (!k_scale || !v_scale)) return PA_ERR_NULL;
  const uintptr_t es = src_dtype == PA_F32 ? 4 : 2;
  if (!aligned(k_new, es) || !aligned(v_new, es)) return PA_ERR_ALIGN;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16)) return PA_ERR_ALIGN;
  if (!aligned(positions, 4) || !aligned(block_table, 4)) return PA_ERR_ALIGN;
  if (kv_dtype == PA_FP8_E4M3 && (!aligned(k_scale, 4) || !aligned(v_scale, 4))) return PA_ERR_ALIGN;
  *grid = (unsigned)((long long)s->batch * s->num_kv_heads);
  return PA_OK;
}

// ---------------------------------------------------------------------------
// pa_lse_merge: the status, and in *grid the workgroups of kMergeThreads
// threads, one thread per 4 output elements (0 for an empty call).
// ---------------------------------------------------------------------------
inline pa_status merge_status(int32_t num_shards, int32_t rows, int32_t head_dim,
                              const void* shard_out, const float* shard_lse, pa_dtype dtype,
                              const void* out, const float* lse_out, unsigned* grid) {
  *grid = 0;
  if (num_shards < 1 || num_shards > 65535 || rows < 0) return PA_ERR_SHAPE;
  if (head_dim < 4 || head_dim > 1024 || head_dim % 4) return PA_ERR_SHAPE;
  if (!shard_out || !shard_lse || !out) return PA_ERR_NULL;
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16) return PA_ERR_DTYPE;
  if (!aligned(shard_out, 16) || !aligned(out, 16) || !aligned(shard_lse, 4) || !aligned(lse_out, 4))
    return PA_ERR_ALIGN;
  const long long threads = (long long)rows * (head_dim / 4);
  const long long blocks = (threads + kMergeThreads - 1) / kMergeThreads;
  if (blocks > kInt32Max) return PA_ERR_SHAPE;
  *grid = (unsigned)blocks;
  return PA_OK;
}

}  // namespace pa_host
