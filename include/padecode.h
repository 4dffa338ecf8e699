/*
 * padecode.h -- C ABI of libpadecode.so: single-token decode attention over a
 * paged KV cache on MI355X (gfx950).
 *
 * The operation (stated on the pages only in words; no formula is printed):
 *  - "rvLLM: High-performance LLM inference in Rust", section "Kernel Compiler
 *    Stack": decode attention with an online softmax over a paged KV cache and
 *    grouped-query heads, one of the per-layer decode ops; section "FA3 v3
 *    Attention Kernel": split-KV spreads one long context over several
 *    workgroups; section "What's Inside": a paged KV cache in f16 or FP8;
 *    section "Optional Features": an FP8 KV cache.
 *  - "RapidLLM", feature table, row "Decode context parallelism": partial
 *    attention over disjoint KV ranges is combined by log-sum-exp.
 *  - "Litellama", section "Architecture": the per-step KV bookkeeping (block
 *    table and context lengths) is handed to the kernels.
 *
 * For each sequence b < batch and query head h < num_q_heads, with
 * G = num_q_heads / num_kv_heads, KV head g = h / G and L = context_lens[b]:
 *     s_t = scale * sum_d q[b][h][d] * K_t[d]          t = 0 .. L-1
 *     out[b][h][:] = sum_t softmax(s)_t * V_t
 *     lse[b][h]    = log sum_t exp(s_t)                (natural log)
 * where token t of sequence b lives in physical block block_table[b][t / 16],
 * slot t % 16. An fp8 cache holds codes c with value e4m3(c) * k_scale[g]
 * (resp. v_scale[g]).
 *
 * Memory layouts (all row-major, all DEVICE memory owned by the caller):
 *   q            [batch][num_q_heads][head_dim]                io_dtype
 *   out          [batch][num_q_heads][head_dim]                io_dtype
 *   k_cache      [num_blocks][num_kv_heads][head_dim/X][16][X] kv_dtype
 *                  X = 16 / sizeof(kv element): 4 (f32), 8 (f16, bf16), 16 (fp8)
 *                  i.e. every 16-byte run holds X consecutive head-dim
 *                  elements of one token.
 *   v_cache      [num_blocks][num_kv_heads][head_dim][16]      kv_dtype
 *                  i.e. each (block, head) page is stored transposed: one
 *                  row of 16 token values per head-dim element.
 *   block_table  int32 [batch][max_blocks_per_seq]
 *   context_lens int32 [batch]
 *   k_scale, v_scale  float32 [num_kv_heads] (fp8 cache only)
 *   lse_out      float32 [batch][num_q_heads] (optional, natural log)
 * One (block, KV head) page of K or of V is one contiguous 16*head_dim run.
 *
 * Errors: every argument is checked on the host before anything is enqueued;
 * a status other than PA_OK means nothing was launched. Nothing falls back to
 * another path: unsupported combinations are errors.
 *
 * Device-side metadata (context_lens, block_table) cannot be checked on the
 * host. The contract is 0 <= context_lens[b] <= 16 * max_blocks_per_seq and
 * 0 <= block_table[b][j] < num_blocks for j < ceil(context_lens[b] / 16);
 * entries past a sequence's last block are never read. The kernels never read
 * outside the caches when the contract is broken: a sequence with an
 * out-of-range length or block id gets NaN outputs instead.
 *
 * Thread safety: the library keeps no state between calls apart from what
 * the caller passes in. Calls are enqueued on `stream`; inputs must stay
 * alive and unmodified until the stream passes the call. Two calls that share
 * a workspace must be ordered on one stream.
 */
#ifndef PADECODE_H
#define PADECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E4M3 = 3 /* OCP E4M3, no infinities; S.1111.111 is NaN; max 448 */
} pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,      /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,     /* unsupported or inconsistent sizes */
  PA_ERR_DTYPE = 3,     /* unsupported io/kv dtype combination */
  PA_ERR_WORKSPACE = 4, /* workspace missing or smaller than required */
  PA_ERR_ALIGN = 5,     /* a tensor pointer is not 16-byte aligned */
  PA_ERR_HIP = 6,       /* the HIP runtime refused the launch */
  PA_ERR_CAPACITY = 7,  /* block pool: not enough free blocks (or host memory) */
  PA_ERR_STATE = 8,     /* block pool: sequence id unknown, or already present */
  PA_ERR_SCRATCH = 9    /* pa_decode_noalloc: the call needs more scratch than it holds */
} pa_status;

typedef struct {
  int32_t batch;              /* >= 0; 0 is a no-op */
  int32_t num_q_heads;        /* >= 1, a multiple of num_kv_heads */
  int32_t num_kv_heads;       /* >= 1; num_q_heads / num_kv_heads <= 16 */
  int32_t head_dim;           /* 64 or 128 */
  int32_t block_size;         /* must be 16 */
  int32_t max_blocks_per_seq; /* row stride of block_table, >= 1 */
  int32_t num_blocks;         /* physical blocks in each cache, >= 1 */
  int32_t partition_size;     /* 0: one pass per sequence;
                                 a positive multiple of 16 tokens: split-K
                                 partitions of that many tokens, merged by
                                 log-sum-exp;
                                 PA_SPLIT_BALANCED: balanced split (below) */
} pa_shape;

/* partition_size value for the balanced split. The pages of every
 * (sequence, KV head) pair, laid end to end, are cut into equal shares, one
 * per workgroup the GPU holds at once, so every compute unit reads the same
 * number of pages whatever the context lengths; a pair cut by share
 * boundaries is merged by log-sum-exp like split-K partitions ("RapidLLM",
 * feature table, row "Decode context parallelism"; "rvLLM", section "FA3 v3
 * Attention Kernel": split-KV spreads a context over workgroups). The result
 * equals the other modes' up to float rounding. Requires batch <= 4096 and
 * batch * num_kv_heads * max_blocks_per_seq < 2^31 - 12288. */
#define PA_SPLIT_BALANCED (-1)

/* Bytes of workspace pa_decode needs for this shape: 0 when
 * partition_size == 0, else room for float32 partial outputs and
 * log-sum-exps of every (sequence, query head, partition) -- for the balanced
 * split, of (shares + batch * num_kv_heads) pieces per query head of a group,
 * where shares depends on the current device's compute units -- plus one
 * counter per (sequence, KV head).
 * With fixed partitions and P = ceil(16 * max_blocks_per_seq / partition_size)
 * > 16, a sequence's partitions are merged in two levels: groups of F
 * consecutive partitions first (F the smallest integer >= 16 with F * F >= P),
 * then the groups. That adds ceil(P / F) group pieces per (sequence, query
 * head) and ceil(P / F) counters per (sequence, KV head).
 * The counters come first: the workspace's first 4 * batch * num_kv_heads *
 * (1 + groups) bytes, rounded up to 256; every completed call leaves its own
 * counters zero, and the rest is scratch that a call overwrites with partial
 * results. A call of another shape (or split mode, or q_len) lays its counters
 * over bytes that an earlier call may have used for partial results. So a
 * workspace needs pa_workspace_reset (a zero fill on a stream) before its
 * first use and before every call whose counter bytes exceed the smallest
 * counter bytes of any call since the last reset; calls of one shape and mode
 * back to back need no reset. A counter found at or above the number of
 * pieces it counts (a broken rule) makes the affected (sequence, KV head)
 * rows NaN instead of a silently wrong merge, and keeps doing so until the
 * workspace is reset; a stale counter below that number cannot be told apart
 * from a live one.
 * Returns 0 for a NULL or invalid shape. */
size_t pa_decode_workspace_bytes(const pa_shape* shape);

/* Decode attention, enqueued on `stream` (a hipStream_t; NULL = the default
 * stream).
 *   scale        softmax scale (e.g. 1/sqrt(head_dim))
 *   io_dtype     dtype of q and out: PA_F32, PA_F16 or PA_BF16
 *   kv_dtype     dtype of the caches: io_dtype, or PA_FP8_E4M3 when io_dtype
 *                is PA_F16 or PA_BF16
 *   k_scale, v_scale  required for PA_FP8_E4M3, ignored otherwise
 *   workspace    device memory of at least pa_decode_workspace_bytes(shape)
 *                bytes (ignored when partition_size == 0), 256-byte aligned
 *   lse_out      optional (NULL to skip)
 * Returns PA_OK once the work is enqueued. */
pa_status pa_decode(const pa_shape* shape, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* block_table,
                    const int32_t* context_lens, float scale, pa_dtype io_dtype,
                    pa_dtype kv_dtype, const float* k_scale,
                    const float* v_scale, void* workspace,
                    size_t workspace_bytes, void* out, float* lse_out,
                    void* stream);

/* Decode attention over a batch whose sequences begin with the same cached
 * prefix ("Litellama", section "Features", Prefix Caching: requests with a
 * common prompt prefix share its physical blocks). Same arguments, results
 * and errors as pa_decode with shape->partition_size == PA_SPLIT_BALANCED
 * (any other value: PA_ERR_SHAPE), plus
 *   prefix_blocks  0 <= prefix_blocks <= max_blocks_per_seq: the number of
 *                  leading block-table entries the rows share.
 * With P = min(prefix_blocks, floor(longest in-contract length / 16)),
 * sequence b takes its first P_b = min(P, floor(context_lens[b] / 16)) pages
 * from the shared prefix: the caller declares that block_table[b][j] is the
 * same block for every b and every j < P_b. Those pages are read once for
 * the query rows of all sequences (per 64 query rows at most, i.e. per four
 * groups of 16 / G sequences) instead of once per sequence; each
 * sequence's remaining tokens go through the balanced split as in
 * pa_decode, and the two parts are merged by log-sum-exp. The result equals
 * pa_decode's up to float rounding. The declaration is checked as the pages
 * are read: a sequence whose row differs from the row the prefix is read
 * from (a longest sequence) at some j < P_b, or whose prefix holds a block
 * id outside the pool, gets NaN outputs. A short prefix saves little: the
 * call then takes about as long as pa_decode's balanced split or a little
 * longer (every piece of a pair goes through the workspace to be merged
 * with the prefix's), so it pays when the prefix is a good part of the
 * batch's pages.
 * workspace: at least pa_decode_prefix_workspace_bytes(shape) bytes, 256-byte
 * aligned, with the same counter region (4 * batch * num_kv_heads bytes
 * first) and reset rule as pa_decode's balanced split; its partial slots are
 * (shares + 9 * batch * num_kv_heads) pieces of G rows. Calls whose partial
 * outputs would pass 4 GiB return PA_ERR_SHAPE. */
size_t pa_decode_prefix_workspace_bytes(const pa_shape* shape);
pa_status pa_decode_prefix(const pa_shape* shape, int32_t prefix_blocks, const void* q,
                           const void* k_cache, const void* v_cache, const int32_t* block_table,
                           const int32_t* context_lens, float scale, pa_dtype io_dtype,
                           pa_dtype kv_dtype, const float* k_scale, const float* v_scale,
                           void* workspace, size_t workspace_bytes, void* out, float* lse_out,
                           void* stream);

/* pa_decode for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. Same arguments, results and errors as pa_decode
 * without workspace and workspace_bytes: the split modes keep their partial
 * results and counters in a scratch array of PA_NOALLOC_SCRATCH_BYTES that
 * the library holds on each GPU it runs on until the process ends. Its first
 * PA_NOALLOC_COUNTER_BYTES hold the counters (4 bytes per (sequence, KV
 * head), plus the merge-group counters of fixed partitions beyond 16 per
 * sequence); the partial results of pa_decode_workspace_bytes's layout follow
 * them. A call that needs more than either gets PA_ERR_SCRATCH and launches
 * nothing (with 512-token partitions over 4096-token tables, head_dim 128 and
 * 7 query heads per KV head, a (sequence, KV head) pair takes 8 x 7 x 129
 * floats, so about 570 pairs fit; the balanced split needs far less). The
 * library allocates nothing in this call;
 * its first call on a GPU looks up that GPU's array and enqueues one zero
 * fill of the counter region on `stream`. Every call on a GPU shares the
 * array: calls that may overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller. partition_size 0 uses
 * no scratch. */
#define PA_NOALLOC_SCRATCH_BYTES (16u << 20)
#define PA_NOALLOC_COUNTER_BYTES (256u << 10)
pa_status pa_decode_noalloc(const pa_shape* shape, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* context_lens, float scale, pa_dtype io_dtype,
                            pa_dtype kv_dtype, const float* k_scale, const float* v_scale,
                            void* out, float* lse_out, void* stream);

/* Attention of q_len new tokens per sequence over the paged cache, causal
 * among the new tokens: the attention step of chunked prefill ("Litellama",
 * section "Features", Chunked Prefill) and of speculative verification
 * ("rvLLM: High-performance LLM inference in Rust", speculative decoding:
 * several drafted tokens checked in one target step). The new tokens' K and V
 * are already in the cache (pa_kv_append), so context_lens[b] = L counts
 * them; new token t (0 .. q_len-1) sits at position L - q_len + t and
 * attends to positions 0 .. L - q_len + t:
 *     out[b][t][h] = softmax(scale * q[b][t][h] . K^T) V   over those positions
 * A new token with no visible position (L < q_len) gets out = 0 and
 * lse = -inf; q_len = 1 is pa_decode.
 *   q, out      [batch][q_len][num_q_heads][head_dim] in io_dtype
 *   lse_out     float32 [batch][q_len][num_q_heads] (natural log) or NULL
 *   q_len       1 .. 16
 *   shape       as for pa_decode; partition_size 0, a positive multiple of
 *               16, or PA_SPLIT_BALANCED (batch <= 4096) for any q_len
 *               (G = num_q_heads / num_kv_heads; rows per (sequence, KV
 *               head) G * q_len). With PA_SPLIT_BALANCED every CU gets an
 *               equal share of the pages of all (sequence, KV head) pairs,
 *               whatever the row count
 *   workspace   pa_decode_multi_workspace_bytes(shape, q_len) bytes when
 *               partition_size != 0; same counter-first contract and
 *               two-level merge as pa_decode, with one counter per
 *               (sequence, KV head) and merge level-1 group when
 *               G * q_len <= 16 or the split is balanced, else
 *               ceil(ceil(G*q_len/16)/2) (one per chunk of 32 rows); the
 *               balanced split's size depends on the device's CU count
 * Everything else (dtypes, scales, alignment, errors) as for pa_decode. */
size_t pa_decode_multi_workspace_bytes(const pa_shape* shape, int32_t q_len);
pa_status pa_decode_multi(const pa_shape* shape, int32_t q_len, const void* q,
                          const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* context_lens,
                          float scale, pa_dtype io_dtype, pa_dtype kv_dtype,
                          const float* k_scale, const float* v_scale, void* workspace,
                          size_t workspace_bytes, void* out, float* lse_out, void* stream);

/* Paged KV append: write each sequence's new token K and V rows into its
 * block and slot of the caches, as the decode step does right before
 * attention ("rvLLM: High-performance LLM inference in Rust", section "Kernel
 * Compiler Stack", per-layer decode steps: the KV cache write follows RoPE and
 * precedes attention), into an f16/bf16/f32 or FP8 cache ("rvLLM", sections
 * "What's Inside" and "Optional Features"; "Litellama", section "Features").
 *   shape        batch, num_kv_heads, head_dim, block_size (16),
 *                max_blocks_per_seq, num_blocks as for pa_decode
 *                (num_q_heads and partition_size are not used)
 *   k_new, v_new [batch][num_kv_heads][head_dim] in src_dtype
 *                (PA_F32, PA_F16 or PA_BF16), device memory
 *   positions    int32 [batch]: the token position p to write (for a decode
 *                step, the context length before the token); p < 0 skips
 *                the sequence
 *   block_table  int32 [batch][max_blocks_per_seq], as for pa_decode
 *   kv_dtype     src_dtype (the bits are copied) or PA_FP8_E4M3: the code is
 *                round-to-nearest-even of clamp(x / scale, -448, 448) with
 *                the division in float32 and scale = k_scale[g] (v_scale[g]),
 *                NaN becoming 0x7F
 *   k_cache, v_cache  written in place, layouts as for pa_decode
 * Row p of sequence b goes to block block_table[b][p / 16], slot p % 16. A
 * position at or past 16 * max_blocks_per_seq, or a block id outside the
 * pool, writes nothing (never outside the caches). Two sequences must not
 * name the same (block, slot). Enqueued on `stream`; errors as for
 * pa_decode. */
pa_status pa_kv_append(const pa_shape* shape, const void* k_new, const void* v_new,
                       const int32_t* positions, const int32_t* block_table,
                       pa_dtype src_dtype, pa_dtype kv_dtype, const float* k_scale,
                       const float* v_scale, void* k_cache, void* v_cache,
                       void* stream);

/* Merge decode-attention results computed on disjoint position shards of
 * every sequence (decode context parallelism: "RapidLLM", feature table, row
 * "Decode context parallelism": partial attention over disjoint KV ranges is
 * combined by log-sum-exp). For each row r (a (sequence, query head) pair):
 *     M = max_s lse_s[r],  w_s = exp(lse_s[r] - M),
 *     out[r] = sum_s w_s * shard_out[s][r] / sum_s w_s,
 *     lse_out[r] = M + log sum_s w_s                       (natural log)
 * summed over s = 0 .. num_shards-1 in that order.
 *   shard_out  [num_shards][rows][head_dim] in dtype (F32, F16 or BF16),
 *              e.g. the out of one pa_decode call per shard
 *   shard_lse  float32 [num_shards][rows], natural log (pa_decode's lse_out)
 *   out        [rows][head_dim] in dtype;  lse_out float32 [rows] or NULL
 * A shard whose lse is -inf (no tokens) contributes nothing; a row with no
 * contributing shard gets out = 0 and lse = -inf; a NaN lse in any shard
 * makes that row's out and lse NaN. head_dim: a multiple of 4, 4 .. 1024;
 * shard_out and out 16-byte aligned. Enqueued on `stream`; errors as for
 * pa_decode. */
pa_status pa_lse_merge(int32_t num_shards, int32_t rows, int32_t head_dim,
                       const void* shard_out, const float* shard_lse, pa_dtype dtype,
                       void* out, float* lse_out, void* stream);

/* ---- Host block pool with hash-chained prefix reuse --------------------
 * The block manager of a paged KV cache ("rvLLM: High-performance LLM
 * inference in Rust", architecture diagram, "Block Manager (paged KV)") with
 * prefix caching ("Litellama", section "Features", Prefix Caching): block ids
 * for the block tables pa_decode and pa_kv_append read, handed out so that
 * sequences whose leading 16-token blocks hold the same tokens share the
 * same physical blocks, and blocks no sequence uses stay cached until the
 * pool needs them.
 *   * A full block is keyed by FNV-1a-64 over the 8 little-endian bytes of
 *     its parent key (the pool seed for a sequence's first block) followed
 *     by its 16 token ids as 4-byte little-endian integers. A lookup also
 *     compares parent key and tokens, so a hash collision never shares.
 *   * The free queue holds every block no sequence uses, least recently
 *     released first; initially all blocks, in id order. Taking a block from
 *     it drops the cache entry the block carried (eviction).
 * Host memory only; the pool is not thread-safe (one caller at a time).
 * Every call returns PA_ERR_NULL for a NULL pool or required pointer. */
typedef struct pa_block_pool pa_block_pool;

/* A pool of num_blocks (>= 1) block ids 0 .. num_blocks-1; *pool receives the
 * handle (NULL on error). PA_ERR_CAPACITY if host memory runs out. */
pa_status pa_pool_create(int32_t num_blocks, uint64_t seed, pa_block_pool** pool);

/* Frees the pool and everything it holds; NULL is a no-op. */
void pa_pool_destroy(pa_block_pool* pool);

/* Registers sequence seq_id with its num_tokens (>= 0) prompt tokens. The
 * longest run of leading full blocks found in the cache is shared (their
 * reference counts rise; cached blocks in the free queue leave it); the
 * remaining full blocks and a partial last block are taken from the free
 * queue, and the new full blocks enter the cache unless it already holds
 * that key. *cached_tokens (if not NULL) receives 16 x the blocks shared.
 * PA_ERR_STATE if seq_id exists; PA_ERR_CAPACITY, changing nothing, if the
 * free queue cannot supply every block the call needs. */
pa_status pa_pool_add_sequence(pa_block_pool* pool, int64_t seq_id, const int32_t* tokens,
                               int32_t num_tokens, int32_t* cached_tokens);

/* Appends one generated token: a token that starts a new block takes one
 * from the free queue (PA_ERR_CAPACITY, changing nothing, if it is empty);
 * a token that completes a block enters that block in the cache.
 * PA_ERR_STATE for an unknown seq_id. */
pa_status pa_pool_append_token(pa_block_pool* pool, int64_t seq_id, int32_t token);

/* Releases the sequence's blocks, last block first: a block whose reference
 * count reaches zero joins the back of the free queue, still cached.
 * PA_ERR_STATE for an unknown seq_id. */
pa_status pa_pool_free_sequence(pa_block_pool* pool, int64_t seq_id);

/* Number of blocks in the free queue; -1 for a NULL pool. */
int32_t pa_pool_num_free(const pa_block_pool* pool);

/* Writes the block tables of num_seqs sequences (host memory):
 * block_table[i][j] = j-th block of seq_ids[i], pad_block past its blocks,
 * int32 [num_seqs][max_blocks_per_seq]; context_lens[i] (if not NULL) = its
 * token count. PA_ERR_STATE for an unknown id, PA_ERR_SHAPE if a sequence
 * has more than max_blocks_per_seq blocks; nothing is written on error. */
pa_status pa_pool_block_table(const pa_block_pool* pool, const int64_t* seq_ids,
                              int32_t num_seqs, int32_t max_blocks_per_seq, int32_t pad_block,
                              int32_t* block_table, int32_t* context_lens);

/* The prefix of blocks the given sequences share, for pa_decode_prefix's
 * prefix_blocks over a batch of exactly these sequences (in any order):
 * the largest P such that every sequence holds the same blocks as the
 * longest one (the first among equals) at each of its own full blocks below
 * P, P at most the longest one's full blocks. 0 for num_seqs == 0.
 * PA_ERR_STATE for an unknown seq_id; PA_ERR_SHAPE for num_seqs < 0. */
pa_status pa_pool_shared_prefix(const pa_block_pool* pool, const int64_t* seq_ids,
                                int32_t num_seqs, int32_t* prefix_blocks);

/* Zero-fill a workspace on `stream` with a fill kernel (safe to capture in a
 * HIP graph). */
pa_status pa_workspace_reset(void* workspace, size_t workspace_bytes,
                             void* stream);

/* Static description of a status code; never NULL. */
const char* pa_status_str(pa_status status);

#ifdef __cplusplus
}
#endif

#endif /* PADECODE_H */
