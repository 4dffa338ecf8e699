// Attention of several new query tokens per sequence over the paged KV cache,
// causal among the new tokens, for gfx950 (MI355X): the attention step of
// chunked prefill ("Litellama", section "Features": Chunked Prefill, prompts
// split into 512-token chunks that interleave with decode requests) and of
// speculative verification ("rvLLM: High-performance LLM inference in Rust",
// speculative decoding: the target model checks several drafted tokens in one
// step). The new tokens' K and V are already in the cache, so a sequence's
// length L counts them; new token t (0 .. T-1) sees positions 0 .. L-T+t.
//
// When a pair's rows fit one matrix-core tile (G * T <= 16) the call runs on
// the decode kernels (fixed partitions or the balanced split), which take the
// same row mapping and causal masks; this kernel serves wider row sets.
//
// Same building blocks and cache layouts as single-token decode. A workgroup
// of four waves owns one (sequence b, KV head g, partition p, row chunk c)
// unit. The query rows of a (b, g) pair are its G*T (new token, head) pairs,
// row = t*G + h, cut into chunks of NT = 2 matrix-core column tiles of 16
// rows (a pair has ceil(G*T/16) tiles, so ceil(tiles/2) chunks: four tiles of
// accumulators do not fit in the registers at head_dim 128). Every wave keeps
// NT sets of accumulators, so one K/V page loaded into registers feeds all
// NT*16 rows, and the matrix-core work per byte grows with T. The
// chunks of one (b, g, p) are launched nbg workgroups apart, which keeps them
// on one XCD (workgroups go to the XCDs round-robin; nbg = B * Hkv is
// usually a multiple of 8) and close in time, so the second chunk's K/V reads
// mostly hit that XCD's L2. The chunk's query operand
// sits in LDS in lane order (one 16-byte read per lane per operand chunk),
// which keeps the registers for the accumulators. Pages go to the waves
// round-robin through the same register rings as decode; a page whose tokens
// reach past L - T (only a sequence's last two pages, always the last page of
// its wave in the unit) is masked per column: token j is visible to row
// (t, h) iff j <= L - T + t. A column with nothing visible yet keeps a zero
// state (the running max stays -inf, exponentials are taken against 0).
// Waves merge through LDS one column tile at a time; split-K partials go to
// the workspace and the last partition of each (b, g, chunk) to finish merges
// them, as for decode (two levels beyond 16 partitions). Rows with no visible
// token get out = 0, lse = -inf.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "padecode.h"
#include "pa_host.h"
#include "pa_internal.h"
#include "pa_schedule.h"
#include "pa_tiles.h"

namespace pa_mq {
using namespace pa;

constexpr int kMaxQLen = pa_host::kMaxQLen;
constexpr int kChunkTiles = pa_host::kChunkTiles;   // column tiles of 16 rows per workgroup

struct Params {
  const uint8_t* q;          // [B][T][Hq][D]
  const uint8_t* k;
  const uint8_t* v;
  const int32_t* block_table;
  const int32_t* context_lens;
  const float* k_scale;
  const float* v_scale;
  uint8_t* out;              // [B][T][Hq][D]
  float* lse_out;            // [B][T][Hq] or null
  float* ws_o;               // [slot][R][D]  partial outputs, normalised
  float* ws_lse;             // [slot][R]     base 2, in units of the scaled scores
  uint32_t* ws_cnt;          // [B][Hkv][chunks], then [B][Hkv][g_max][chunks] (first-level groups)
  float scale;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;             // G = Hq / Hkv
  int32_t q_len;             // T
  int32_t rows;              // R = G * T
  int32_t chunks;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t part_tokens;
  int32_t p_max;
  int32_t fan;               // partitions per first-level merge group (0: one level)
  int32_t g_max;             // first-level groups per (b, g); their slots follow the
                             // B * Hkv * p_max partition slots
};

// Merge the n pieces of rows row0 .. row0 + rows_c - 1 of (b, g) stored in
// workspace slots slot0 .. slot0 + n - 1 (partitions, first-level groups of
// partitions, or pieces of the balanced split) in slot order, and write the
// final output of those rows (dst < 0) or the merged piece to workspace slot
// dst. Threads take (row, 4-float quad) items kU at a time and issue the
// loads of kBatch pieces of all of them before folding any, so up to
// kU * 256 items cost one memory round trip per kBatch pieces (a 56-row pair
// at head_dim 128, 1,792 items, costs one). A piece a row sees nothing of
// (lse = -inf) adds nothing; a row that sees nothing in any piece gets out = 0
// and lse = -inf; NaN in any piece gives NaN.
template <typename IO, int D>
__device__ __forceinline__ void merge_rows(const Params& a, int b, int g, int row0, int rows_c,
                                           size_t slot0, int n, long long dst) {
  constexpr int kBatch = 4;
  constexpr int kU = 8;
  const int R = a.rows, G = a.group;
  const int items = rows_c * (D / 4);
  for (int base = 0; base < items; base += kU * kThreads) {
    int rho[kU], d[kU];
    bool on[kU], nan[kU];
    float mr[kU], wr[kU];
    f32x4 ar[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + u * kThreads + threadIdx.x;
      on[u] = i < items;
      const int r2 = i / (D / 4);
      d[u] = 4 * (i - r2 * (D / 4));
      rho[u] = on[u] ? row0 + r2 : row0;
      nan[u] = false;
      mr[u] = -INFINITY;
      wr[u] = 0.f;
      ar[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int q0 = 0; q0 < n; q0 += kBatch) {
      const int nb = min(kBatch, n - q0);
      const brsrc ro = buffer_rsrc(a.ws_o + (slot0 + q0) * R * D, (uint32_t)(nb * R * D * sizeof(float)));
      const brsrc rl = buffer_rsrc(a.ws_lse + (slot0 + q0) * R, (uint32_t)(nb * R * sizeof(float)));
      float lp[kU][kBatch];
      f32x4 ov[kU][kBatch];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t vo = (uint32_t)(((size_t)rho[u] * D + d[u]) * sizeof(float));
        const uint32_t vl = (uint32_t)(rho[u] * sizeof(float));
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          if (on[u] && q < nb) {
            lp[u][q] = ld_agent1(rl, vl, (uint32_t)(q * R * sizeof(float)));
            ov[u][q] = ld_agent4(ro, vo, (uint32_t)((size_t)q * R * D * sizeof(float)));
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          if (on[u] && q < nb) {
            const float l = lp[u][q];
            if (l != l) {
              nan[u] = true;
            } else if (l > -INFINITY) {
              const float mn = fmaxf(mr[u], l);
              const float sa = exp2_fast(mr[u] - mn), sb = exp2_fast(l - mn);
              ar[u] = ar[u] * sa + ov[u][q] * sb;
              wr[u] = wr[u] * sa + sb;
              mr[u] = mn;
            }
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (!on[u]) continue;
      f32x4 val = {0.f, 0.f, 0.f, 0.f};
      float lse2 = -INFINITY;   // base 2
      if (nan[u]) {
        val = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
        lse2 = __builtin_nanf("");
      } else if (wr[u] > 0.f) {
        val = ar[u] * __builtin_amdgcn_rcpf(wr[u]);
        lse2 = mr[u] + log2_fast(wr[u]);
      }
      if (dst < 0) {
        const int t = rho[u] / G, h = rho[u] - t * G;
        const size_t orow = ((size_t)b * a.q_len + t) * a.num_q_heads + (size_t)g * G + h;
        store_out4<IO>(a.out, orow * D + d[u], val);
        if (d[u] == 0 && a.lse_out) a.lse_out[orow] = lse2 * kLn2;
      } else {
        const brsrc wd = buffer_rsrc(a.ws_o + (size_t)dst * R * D, (uint32_t)(R * D * sizeof(float)));
        st_agent4(wd, (uint32_t)(((size_t)rho[u] * D + d[u]) * sizeof(float)), val);
        if (d[u] == 0) st_agent(a.ws_lse + (size_t)dst * R + rho[u], lse2);
      }
    }
  }
}

template <typename QC, int NT, int KQ, int D>
struct MqSmem {
  QC q[NT][KQ][64];            // query operand chunks, lane order
  float acc[kWaves][16][D + 4];
  float m[kWaves][16];
  float l[kWaves][16];
  int bad;
  int last;
};

// One wave's share of a unit: pages first, first + stride, ... (n of them)
// of sequence b and KV head g, tokens before t1, against NT column tiles whose
// query operands sit in LDS at qsm ([NT][KQ][64] chunks, lane order). lim[j]:
// the last token the lane's column of tile j may see. Pages go through the
// same register rings as decode; the steady blocks never hold the wave's last
// tail_min pages (nor its last ring depth), and every page a mask can touch
// is among those, so the steady blocks run unmasked: the causal mask reaches
// at most a sequence's last two pages, the last two of a wave with stride 1
// and the last of a wave with a larger stride. A column with nothing visible
// yet keeps a zero state (running max -inf, exponentials taken against 0).
// Leaves the wave's running max, its lanes' partial sums and the
// accumulators; bad_blk: a block id outside the pool was met (block 0 read
// instead).
// Block ids of pages first + stride * (64 * chunk + lane), clamped into the
// table row: the lane's id of one 64-page chunk.
__device__ __forceinline__ int fetch_ids(const Params& a, int b, int first, int stride, int chunk) {
  const int lane = threadIdx.x & 63;
  return a.block_table[(size_t)b * a.max_blocks_per_seq +
                       min(first + stride * (chunk * 64 + lane), a.max_blocks_per_seq - 1)];
}

// bt0: fetch_ids(a, b, first, stride, 0), loaded by the caller as early as it
// can be.
template <typename IO, typename KV, int D, int NT, bool KEEP>
__device__ __forceinline__ void stream_pages(const Params& a, int b, int g, int first, int stride, int n,
                                             int bt0, int t1, const int (&lim)[NT],
                                             const typename TileOf<IO, KV, D>::type::QC* qsm, float kmul,
                                             int tail_min, float (&mrow)[NT], float (&lrow)[NT],
                                             f32x4 (&acc)[NT][D / 16], bool& bad_blk) {
  using T = typename TileOf<IO, KV, D>::type;
  constexpr int KQ = T::kQ;
  constexpr size_t kPageBytes = (size_t)kBlock * D * ElemSize<KV>::v;
  const int lane = threadIdx.x & 63;
  const int jj = lane >> 4;

  // Block ids of the wave's pages, 64 at a time.
  auto fetch_bt = [&](int chunk) { return fetch_ids(a, b, first, stride, chunk); };
  int bt_cur = bt0;
  int bt_next = n > 64 ? fetch_bt(1) : 0;

  const gptr kbase = uniform_ptr(a.k + (size_t)g * kPageBytes);
  const gptr vbase = uniform_ptr(a.v + (size_t)g * kPageBytes);
  const size_t block_stride = (size_t)a.num_kv_heads * kPageBytes;
  const uint32_t ko = T::koff(lane), vo = T::voff(lane);

  constexpr int kKS = T::kKStages, kVS = T::kVStages;
  constexpr int dK = kKS - 1, dV = kVS - 1;
  // a V load reuses the page offset its K load recorded, so V may not run
  // ahead of K
  static_assert(kKS >= 1 && kVS >= 1 && dV <= dK, "ring depths");
  constexpr int kAhead = dK > 1 ? dK : 1;
  constexpr int kTailMax = kAhead > 2 ? kAhead : 2;
  const int tail = max(kAhead, tail_min);
  typename T::KRegs ring_k[kKS];
  typename T::VRegs ring_v[kVS];
  size_t poff[kKS];

  auto issue_k = [&](int slot, int i, auto refresh_tag) __attribute__((always_inline)) {
    if constexpr (decltype(refresh_tag)::value) {
      if (i > 0 && (i & 63) == 0) {
        bt_cur = bt_next;
        if (n > i + 64) bt_next = fetch_bt((i >> 6) + 1);
      }
    }
    int phys = __builtin_amdgcn_readlane(bt_cur, i & 63);
    if ((unsigned)phys >= (unsigned)a.num_blocks) {
      bad_blk = true;
      phys = 0;
    }
    poff[slot] = (size_t)phys * block_stride;
    T::template load_k<KEEP>(ring_k[slot], kbase + poff[slot], ko);
  };
  auto issue_v = [&](int vslot, int kslot) __attribute__((always_inline)) {
    T::template load_v<KEEP>(ring_v[vslot], vbase + poff[kslot], vo);
  };

#pragma unroll
  for (int j = 0; j < NT; ++j) {
    mrow[j] = -INFINITY;
    lrow[j] = 0.f;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One page for all NT column tiles. kMasked: the page may hold tokens at
  // or past t1, or tokens some column must not see.
  auto compute = [&](int kslot, int vslot, int i, auto masked_tag) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const int pstart = (first + stride * i) * kBlock;
    typename T::A4 va[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      va[t] = T::pvt(ring_v[vslot], t);
      if constexpr (kMasked) va[t] = T::zero_tail(va[t], jj, t1 - pstart);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      typename T::Q qop;
#pragma unroll
      for (int cc = 0; cc < KQ; ++cc) qop.c[cc] = qsm[(j * KQ + cc) * 64 + lane];
      const f32x4 s = T::scores(ring_k[kslot], qop);
      float sc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (kMasked) {
          const int tok = pstart + 4 * jj + e;
          sc[e] = (tok <= lim[j] && tok < t1) ? s[e] * kmul : -INFINITY;
        } else {
          sc[e] = s[e] * kmul;
        }
      }
      const float mx = wave_max_rows(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
      const float mnew = fmaxf(mrow[j], mx);
      float msafe = mnew;
      if constexpr (kMasked) msafe = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = exp2_fast(mrow[j] - msafe);
      float pr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pr[e] = exp2_fast(sc[e] - msafe);
      const typename T::P pk = T::pack(pr);
      lrow[j] = lrow[j] * alpha + T::psum(pk);
      mrow[j] = mnew;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int t = 0; t < D / 16; ++t) acc[j][t] *= alpha;
      }
#pragma unroll
      for (int t = 0; t < D / 16; ++t) acc[j][t] = T::pv(va[t], pk, acc[j][t]);
    }
  };
  using Full = std::integral_constant<bool, false>;
  using Tail = std::integral_constant<bool, true>;

  constexpr int kU = kKS * kVS / gcd_c(kKS, kVS);
  auto run_ring = [&](auto refresh_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < dK; ++j)
      if (j < n) issue_k(j, j, refresh_tag);
#pragma unroll
    for (int j = 0; j < dV; ++j)
      if (j < n) issue_v(j, j);
    int i0 = 0;
    for (; i0 + kU - 1 + tail < n; i0 += kU) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        issue_k((u + dK) % kKS, i0 + u + dK, refresh_tag);
        issue_v((u + dV) % kVS, (u + dV) % kKS);
        compute(u % kKS, u % kVS, i0 + u, Full{});
      }
    }
#pragma unroll
    for (int u = 0; u < kU + kTailMax; ++u) {
      const int i = i0 + u;
      if (i < n) {
        if (i + dK < n) issue_k((u + dK) % kKS, i + dK, refresh_tag);
        if (i + dV < n) issue_v((u + dV) % kVS, (u + dV) % kKS);
        compute(u % kKS, u % kVS, i, Tail{});
      }
    }
  };
  if (n > 64)
    run_ring(std::integral_constant<bool, true>{});
  else
    run_ring(std::integral_constant<bool, false>{});
}

// KEEP: the pair has three or more row chunks, so several other workgroups
// read the same pages soon after: ordinary loads, which leave them in L2 for
// those (non-temporal otherwise, as in decode). Measured on the
// Qwen2.5-7B-shaped workload: with two chunks (8 new tokens) non-temporal
// loads are 4% faster, with four (16 new tokens) ordinary loads 16% faster.
template <typename IO, typename KV, int D, int NT, bool KEEP>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
pa_multi_kernel(const Params a) {
  using T = typename TileOf<IO, KV, D>::type;
  using QC = typename T::QC;
  constexpr int KQ = T::kQ;
  constexpr bool kFp8 = std::is_same<KV, FP8>::value;
  constexpr int kRowsC = NT * 16;
  __shared__ MqSmem<QC, NT, KQ, D> sm;

  const int H = a.num_kv_heads;
  const int nbg = a.batch * H;
  const int pc = blockIdx.x / nbg;          // p * chunks + c: partition-major
  const int bg = blockIdx.x - pc * nbg;
  const int p = pc / a.chunks;
  const int c = pc - p * a.chunks;
  const int b = bg / H;
  const int g = bg - b * H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rr = lane & 15, jj = lane >> 4;
  const int G = a.group, TQ = a.q_len, R = a.rows;
  const int PT = a.part_tokens;
  const int page0 = PT > 0 ? p * (PT / kBlock) : 0;
  const int row0 = c * kRowsC;

  // Block ids of this wave's first 64 pages, before the length is known.
  const int bt0 = fetch_ids(a, b, page0 + w, kWaves, 0);

  // The chunk's query operand into LDS. Rows past R repeat row R-1: their
  // columns hold finite duplicates that are never stored.
  // (every load of the thread issued before its first LDS write)
  constexpr int kQItems = NT * KQ * 64;
  constexpr int kQPer = (kQItems + kThreads - 1) / kThreads;
  u32x4 qv[kQPer];
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int i = u * kThreads + tid;
    if (i < kQItems) {
      const int j = i / (KQ * 64);
      const int rem = i - j * (KQ * 64);
      const int cc = rem >> 6, ln = rem & 63;
      const int rho = min(row0 + 16 * j + (ln & 15), R - 1);
      const int t = rho / G, h = rho - t * G;
      const uint8_t* qrow =
          a.q + (((size_t)b * TQ + t) * a.num_q_heads + (size_t)g * G + h) * D * ElemSize<IO>::v;
      qv[u] = *reinterpret_cast<const u32x4*>(qrow + T::qoff(cc, ln >> 4));
    }
  }
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int i = u * kThreads + tid;
    if (i < kQItems) {
      const int j = i / (KQ * 64);
      const int rem = i - j * (KQ * 64);
      sm.q[j][rem >> 6][rem & 63] = __builtin_bit_cast(QC, qv[u]);
    }
  }

  const int L = a.context_lens[b];
  const bool bad_len = L < 0 || L > a.max_blocks_per_seq * kBlock;
  const int nparts = (bad_len || L == 0) ? 1 : (PT > 0 ? (L + PT - 1) / PT : 1);
  if (p >= nparts) return;
  const int rows_c = min(kRowsC, R - row0);   // rows this chunk stores
  if (bad_len || L == 0) {
    const float fill = bad_len ? __builtin_nanf("") : 0.f;
    for (int i = tid; i < rows_c * D; i += kThreads) {
      const int rho = row0 + i / D, t = rho / G, h = rho - t * G;
      store_out<IO>(a.out, (((size_t)b * TQ + t) * a.num_q_heads + (size_t)g * G + h) * D + i % D, fill);
    }
    if (a.lse_out && tid < rows_c) {
      const int rho = row0 + tid, t = rho / G, h = rho - t * G;
      a.lse_out[((size_t)b * TQ + t) * a.num_q_heads + (size_t)g * G + h] = bad_len ? fill : -INFINITY;
    }
    return;
  }

  // Last visible position of each of the lane's columns.
  int lim[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) lim[j] = L - TQ + min(row0 + 16 * j + rr, R - 1) / G;

  const int t0 = page0 * kBlock;
  const int pg_hi = PT > 0 ? page0 + PT / kBlock : a.max_blocks_per_seq;
  const int t1 = min(pg_hi * kBlock, L);
  const int npages = (t1 - t0 + kBlock - 1) / kBlock;
  const int nmine = npages > w ? (npages - w + kWaves - 1) / kWaves : 0;

  float kmul = a.scale * kLog2e;
  float vmul = 1.0f;
  if constexpr (kFp8) {
    kmul *= a.k_scale[g];
    vmul = a.v_scale[g];
  }
  __syncthreads();   // query operand in LDS
  float mrow[NT], lrow[NT];
  f32x4 acc[NT][D / 16];
  bool bad_blk = false;
  stream_pages<IO, KV, D, NT, KEEP>(a, b, g, page0 + w, kWaves, nmine, bt0, t1, lim, &sm.q[0][0][0], kmul,
                                    1, mrow, lrow, acc, bad_blk);

  // ---- merge the waves through LDS, one column tile at a time -------------
  if (tid == 0) sm.bad = 0;
  __syncthreads();
  if (bad_blk) sm.bad = 1;
  const bool split = nparts > 1;
  const size_t slot = (size_t)bg * a.p_max + p;
  const brsrc wr_slot = buffer_rsrc(a.ws_o + slot * R * D, (uint32_t)(R * D * sizeof(float)));
  bool bad = false;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const float lsum = wave_sum_rows(lrow[j]);
    if (j > 0) __syncthreads();   // the previous tile's readers are done
    if (jj == 0) {
      sm.m[w][rr] = mrow[j];
      sm.l[w][rr] = lsum;
    }
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      *reinterpret_cast<f32x4*>(&sm.acc[w][rr][16 * t + 4 * jj]) = acc[j][t];
    __syncthreads();
    if (j == 0) bad = sm.bad != 0;
    for (int i = tid; i < 16 * (D / 4); i += kThreads) {   // (row, 4-float quad)
      const int r2 = i / (D / 4), d = 4 * (i - r2 * (D / 4));
      const int rho = row0 + 16 * j + r2;
      if (rho >= R) continue;
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.m[ww][r2]);
      float W = 0.f;
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      if (M > -INFINITY) {
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
          const float e = exp2_fast(sm.m[ww][r2] - M);
          W += e * sm.l[ww][r2];
          o += e * *reinterpret_cast<const f32x4*>(&sm.acc[ww][r2][d]);
        }
      }
      f32x4 val = {0.f, 0.f, 0.f, 0.f};
      float lse2 = -INFINITY;
      if (W > 0.f) {
        val = o * (__builtin_amdgcn_rcpf(W) * vmul);
        lse2 = M + log2_fast(W);
      }
      if (bad) {
        val = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
        lse2 = __builtin_nanf("");
      }
      if (!split) {
        const int t = rho / G, h = rho - t * G;
        const size_t orow = ((size_t)b * TQ + t) * a.num_q_heads + (size_t)g * G + h;
        store_out4<IO>(a.out, orow * D + d, val);
        if (d == 0 && a.lse_out) a.lse_out[orow] = lse2 * kLn2;
      } else {
        st_agent4(wr_slot, (uint32_t)(((size_t)rho * D + d) * sizeof(float)), val);
        if (d == 0) st_agent(a.ws_lse + slot * R + rho, lse2);
      }
    }
  }
  if (!split) return;

  // ---- split-K: the last partition of (b, g, c) to finish merges ----------
  // With more than a.fan partitions the merge has two levels, as for decode:
  // the last finisher of each group of a.fan partitions merges the group's
  // rows of this chunk into a group slot, the last group merges the groups.
  size_t first = (size_t)bg * a.p_max;
  int np = nparts;
  bool reporter = p == 0;   // the piece that reports a stale count of (b, g, c)
  if (a.fan > 0 && nparts > a.fan) {
    const int grp = p / a.fan;
    const int gfirst = grp * a.fan;
    const int gn = min(a.fan, nparts - gfirst);
    const size_t gbase = (size_t)nbg * a.p_max + (size_t)bg * a.g_max;   // group slots of (b, g)
    const int c1 =
        last_to_finish(a.ws_cnt + ((size_t)nbg + (size_t)bg * a.g_max + grp) * a.chunks + c, gn, &sm.last);
    if (c1 == kCountMore) return;
    if (c1 == kCountStale) {
      // the group's first partition reports it: a NaN log-sum-exp in the
      // group slot makes the final merge's rows NaN
      if (p != gfirst) return;
      if ((int)threadIdx.x < rows_c)
        st_agent(a.ws_lse + (gbase + grp) * R + row0 + threadIdx.x, __builtin_nanf(""));
    } else {
      merge_rows<IO, D>(a, b, g, row0, rows_c, first + gfirst, gn, (long long)(gbase + grp));
    }
    first = gbase;
    np = (nparts + a.fan - 1) / a.fan;
    reporter = grp == 0;
  }
  const int c2 = last_to_finish(a.ws_cnt + (size_t)bg * a.chunks + c, np, &sm.last);
  if (c2 == kCountLast) {
    merge_rows<IO, D>(a, b, g, row0, rows_c, first, np, -1);
  } else if (c2 == kCountStale && reporter) {
    for (int i = threadIdx.x; i < rows_c * D; i += kThreads) {
      const int rho = row0 + i / D;
      const int t = rho / G, h = rho - t * G;
      const size_t orow = ((size_t)b * TQ + t) * a.num_q_heads + (size_t)g * G + h;
      store_out<IO>(a.out, orow * D + i % D, __builtin_nanf(""));
      if (i % D == 0 && a.lse_out) a.lse_out[orow] = __builtin_nanf("");
    }
  }
}


// ---------------------------------------------------------------------------
// Balanced split for rows wider than one tile (partition_size ==
// PA_SPLIT_BALANCED, G * T > 16): the work line and shares of the decode
// balanced split (pa_schedule.h: all (sequence, KV head) pairs' pages end to
// end, cut into one equal share per workgroup, one workgroup per CU), so a
// long sequence no longer holds one workgroup for its whole length. Each
// workgroup walks the pieces of its share in line order. Inside a piece its
// waves split by row chunk (two column tiles each, as above): WC waves per
// chunk take the piece's pages round-robin, the NCG = 4 / WC chunks of a pass
// run side by side, so the waves of different chunks read the same pages at
// about the same time and all but the first find them in L2 (ordinary loads
// when a page has several readers, non-temporal when it has one). Pairs with
// more than four chunks take several passes over the piece. The chunk's waves
// merge through LDS; a piece that is a whole pair writes the output, any
// other piece stores a partial result to workspace slot (first share of the
// pair) + (pair index) + (piece index), and the piece that completes the
// pair's count merges them (the same counter hand-off as the decode kernels).
// Every value the piece loop and its barriers depend on is made wave-uniform
// with readfirstlane, so every wave runs the same barriers.
// ---------------------------------------------------------------------------
struct MqBalLayout {
  unsigned q, acc, m, l, badw, misc, len, pre, total;
};
// Tiles the waves merge through LDS at once: both of a chunk, except f32 at
// head_dim 128, whose operands and accumulators would not fit beside the
// largest batch's lengths.
__host__ __device__ constexpr int mq_bal_merge_tiles(bool f32, int D) { return f32 && D == 128 ? 1 : kChunkTiles; }
// LDS of pa_multi_bal_kernel for head_dim D, qbytes of query operand per tile,
// ncg chunks per pass, mt tiles merged at once and B sequences (host and
// device).
__host__ __device__ inline MqBalLayout mq_bal_layout(int D, int qbytes, int ncg, int mt, int B) {
  MqBalLayout o;
  unsigned p = 0;
  auto al = [](unsigned x) { return (x + 15u) & ~15u; };
  o.q = p;    p = al(p + (unsigned)(ncg * kChunkTiles * qbytes));     // [chunk][tile][KQ][64]
  o.acc = p;  p = al(p + (unsigned)(mt * kWaves * 16 * (D + 4) * 4)); // [tile][wave][row][D + 4]
  o.m = p;    p = al(p + (unsigned)(mt * kWaves * 16 * 4));
  o.l = p;    p = al(p + (unsigned)(mt * kWaves * 16 * 4));
  o.badw = p; p = al(p + kWaves * 4);
  o.misc = p; p = al(p + 8 * 4);                                   // scan sums, count flag
  o.len = p;  p = al(p + (unsigned)B * 4);
  o.pre = p;  p = al(p + (unsigned)(B + 1) * 4);
  o.total = p;
  return o;
}

// One workgroup per CU, one wave per SIMD: the whole register file is the
// wave's (no waves-per-SIMD target).
template <typename IO, typename KV, int D, int WC, bool KEEP>
__global__ void __launch_bounds__(kThreads) pa_multi_bal_kernel(const Params a) {
  using T = typename TileOf<IO, KV, D>::type;
  using QC = typename T::QC;
  constexpr int KQ = T::kQ;
  constexpr int NT = kChunkTiles;      // column tiles per wave: one row chunk
  constexpr int NCG = kWaves / WC;     // chunks of one pass
  static_assert(WC == 1 || WC == 2 || WC == 4, "waves per chunk");
  constexpr bool kFp8 = std::is_same<KV, FP8>::value;
  constexpr int kMT = mq_bal_merge_tiles(std::is_same<IO, F32>::value, D);
  extern __shared__ __attribute__((aligned(16))) uint8_t mqb_lds[];
  const int B = a.batch, H = a.num_kv_heads, mbs = a.max_blocks_per_seq;
  const MqBalLayout lay = mq_bal_layout(D, KQ * 64 * (int)sizeof(QC), NCG, kMT, B);
  QC* const qsm = reinterpret_cast<QC*>(mqb_lds + lay.q);
  float* const sacc = reinterpret_cast<float*>(mqb_lds + lay.acc);
  float* const sm_m = reinterpret_cast<float*>(mqb_lds + lay.m);
  float* const sm_l = reinterpret_cast<float*>(mqb_lds + lay.l);
  int* const badw = reinterpret_cast<int*>(mqb_lds + lay.badw);
  int* const misc = reinterpret_cast<int*>(mqb_lds + lay.misc);
  int* const slen = reinterpret_cast<int*>(mqb_lds + lay.len);
  int* const spre = reinterpret_cast<int*>(mqb_lds + lay.pre);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rr = lane & 15, jj = lane >> 4;
  const int G = a.group, TQ = a.q_len, R = a.rows;
  const int NC = (R + 16 * NT - 1) / (16 * NT);   // row chunks of a pair
  const int passes = (NC + NCG - 1) / NCG;
  const int wi = w % WC, cg = w / WC;             // the wave's place in its chunk, its chunk in a pass

  // Lengths into LDS and the exclusive prefix sums of their line positions
  // (as in the decode balanced split).
  const int per = (B + kThreads - 1) / kThreads;
  const int bbeg = tid * per;
  int mine = 0;
  for (int i = 0; i < per; ++i) {
    const int bb = bbeg + i;
    if (bb < B) {
      const int L = a.context_lens[bb];
      slen[bb] = L;
      mine += line_pages(L, mbs);
    }
  }
  int incl = mine;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) misc[w] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int ww = 0; ww < kWaves; ++ww)
    if (ww < w) before += misc[ww];
  int pre = before + incl - mine;
  for (int i = 0; i < per; ++i) {
    const int bb = bbeg + i;
    if (bb < B) {
      spre[bb] = pre;
      pre += line_pages(slen[bb], mbs);
    }
  }
  if (tid == kThreads - 1) spre[B] = before + incl;
  __syncthreads();

  const int n = H * __builtin_amdgcn_readfirstlane(spre[B]);
  const int S = share_count(n, gridDim.x);
  const int wg = __builtin_amdgcn_readfirstlane(share_of_block(blockIdx.x, gridDim.x, S));
  if (wg >= S) return;
  const int x1 = __builtin_amdgcn_readfirstlane(share_start(wg + 1, n, S));
  int x = __builtin_amdgcn_readfirstlane(share_start(wg, n, S));
  // the sequence holding x
  int b = 0;
  {
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (H * __builtin_amdgcn_readfirstlane(spre[mid]) <= x) lo = mid; else hi = mid;
    }
    b = lo;
  }
  int seq_pre = __builtin_amdgcn_readfirstlane(spre[b]);

  auto row_of = [&](int bb, int gg, int rho) {
    const int t = rho / G, h = rho - t * G;
    return ((size_t)bb * TQ + t) * a.num_q_heads + (size_t)gg * G + h;
  };
  auto fill_pair = [&](int bb, int gg, float v, float lse) {
    for (int i = tid; i < R * D; i += kThreads) store_out<IO>(a.out, row_of(bb, gg, i / D) * D + i % D, v);
    if (a.lse_out)
      for (int rho = tid; rho < R; rho += kThreads) a.lse_out[row_of(bb, gg, rho)] = lse;
  };

  while (x < x1 && b < B) {
    const int L = __builtin_amdgcn_readfirstlane(slen[b]);
    const int cb = line_pages(L, mbs);
    const int seq_first = H * seq_pre;
    const LinePiece pc = line_piece(x, x1, seq_first, cb, b, H, n, S, wg);
    const int g = __builtin_amdgcn_readfirstlane(pc.g);
    const int pg_lo = __builtin_amdgcn_readfirstlane(pc.pg_lo);
    const int pg_hi = __builtin_amdgcn_readfirstlane(pc.pg_hi);
    const int k = __builtin_amdgcn_readfirstlane(pc.k);
    const int nparts = __builtin_amdgcn_readfirstlane(pc.nparts);
    const int slot0 = __builtin_amdgcn_readfirstlane(pc.slot0);
    const int x_end = __builtin_amdgcn_readfirstlane(pc.x_end);

    lds_barrier();   // the previous piece's LDS readers are done
    const bool bad_len = L < 0 || L > mbs * kBlock;
    if (bad_len || L == 0) {
      // a placeholder position: the pair lies whole in this share
      fill_pair(b, g, bad_len ? __builtin_nanf("") : 0.f, bad_len ? __builtin_nanf("") : -INFINITY);
    } else {
      float kmul = a.scale * kLog2e;
      float vmul = 1.0f;
      if constexpr (kFp8) {
        kmul *= a.k_scale[g];
        vmul = a.v_scale[g];
      }
      const int t1 = min(pg_hi * kBlock, L);
      const int np = pg_hi - pg_lo;
      const int nmine = np > wi ? (np - wi + WC - 1) / WC : 0;
      const bool split = nparts > 1;
      const size_t slot = (size_t)slot0 + k;
      const brsrc wr_slot = buffer_rsrc(a.ws_o + slot * R * D, (uint32_t)(R * D * sizeof(float)));
      for (int cp = 0; cp < passes; ++cp) {
        const int c = cp * NCG + cg;   // this wave's row chunk
        const bool active = c < NC;
        const int bt0 = fetch_ids(a, b, pg_lo + wi, WC, 0);
        if (cp > 0) lds_barrier();   // the previous pass's LDS readers are done
        // the pass's query operands into LDS; rows past R repeat row R-1
        // (finite duplicates, never stored). Every load of the thread is
        // issued before its first LDS write: one memory round trip.
        constexpr int kQItems = NCG * NT * KQ * 64;
        constexpr int kQPer = (kQItems + kThreads - 1) / kThreads;
        u32x4 qv[kQPer];
#pragma unroll
        for (int u = 0; u < kQPer; ++u) {
          const int i = u * kThreads + tid;
          if (i < kQItems) {
            const int tj = i / (KQ * 64);
            const int rem = i - tj * (KQ * 64);
            const int cc = rem >> 6, ln = rem & 63;
            const int rho = min(16 * (cp * NCG * NT + tj) + (ln & 15), R - 1);
            const uint8_t* qrow = a.q + row_of(b, g, rho) * D * ElemSize<IO>::v;
            qv[u] = *reinterpret_cast<const u32x4*>(qrow + T::qoff(cc, ln >> 4));
          }
        }
#pragma unroll
        for (int u = 0; u < kQPer; ++u)
          if (u * kThreads + tid < kQItems) qsm[u * kThreads + tid] = __builtin_bit_cast(QC, qv[u]);
        if (tid < kWaves) badw[tid] = 0;
        lds_barrier();
        int lim[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) lim[j] = L - TQ + min(16 * (NT * c + j) + rr, R - 1) / G;
        float mrow[NT], lrow[NT];
        f32x4 acc[NT][D / 16];
        bool bad_blk = false;
        stream_pages<IO, KV, D, NT, KEEP>(a, b, g, pg_lo + wi, WC, active ? nmine : 0, bt0, t1, lim,
                                          qsm + (size_t)cg * NT * KQ * 64, kmul, WC == 1 ? 2 : 1, mrow,
                                          lrow, acc, bad_blk);
        if (bad_blk && lane == 0) badw[w] = 1;
        // the WC waves of each chunk merge, kMT tiles at a time
#pragma unroll
        for (int j0 = 0; j0 < NT; j0 += kMT) {
          float lsum[kMT];
#pragma unroll
          for (int jm = 0; jm < kMT; ++jm) lsum[jm] = wave_sum_rows(lrow[j0 + jm]);
          lds_barrier();   // the previous tiles' readers are done (first: the bad flags are in)
#pragma unroll
          for (int jm = 0; jm < kMT; ++jm) {
            const int sw = jm * kWaves + w;
            if (jj == 0) {
              sm_m[sw * 16 + rr] = mrow[j0 + jm];
              sm_l[sw * 16 + rr] = lsum[jm];
            }
#pragma unroll
            for (int t = 0; t < D / 16; ++t)
              *reinterpret_cast<f32x4*>(&sacc[(sw * 16 + rr) * (D + 4) + 16 * t + 4 * jj]) = acc[j0 + jm][t];
          }
          lds_barrier();
          for (int i = tid; i < kMT * NCG * 16 * (D / 4); i += kThreads) {   // (tile, chunk, row, quad)
            const int jm = i / (NCG * 16 * (D / 4));
            const int r1 = i - jm * (NCG * 16 * (D / 4));
            const int cgi = r1 / (16 * (D / 4));
            const int rem = r1 - cgi * (16 * (D / 4));
            const int r2 = rem / (D / 4), d = 4 * (rem - r2 * (D / 4));
            const int c2 = cp * NCG + cgi;
            const int rho = 16 * (NT * c2 + j0 + jm) + r2;
            if (c2 >= NC || rho >= R) continue;
            float M = -INFINITY;
            bool bad = false;
#pragma unroll
            for (int u = 0; u < WC; ++u) {
              M = fmaxf(M, sm_m[(jm * kWaves + cgi * WC + u) * 16 + r2]);
              bad |= badw[cgi * WC + u] != 0;
            }
            const float Ms = M == -INFINITY ? 0.f : M;
            float W = 0.f;
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < WC; ++u) {
              const int sw = jm * kWaves + cgi * WC + u;
              const float e = exp2_fast(sm_m[sw * 16 + r2] - Ms);
              W += e * sm_l[sw * 16 + r2];
              o += e * *reinterpret_cast<const f32x4*>(&sacc[(sw * 16 + r2) * (D + 4) + d]);
            }
            f32x4 val = {0.f, 0.f, 0.f, 0.f};
            float lse2 = -INFINITY;
            if (W > 0.f) {
              val = o * (__builtin_amdgcn_rcpf(W) * vmul);
              lse2 = M + log2_fast(W);
            }
            if (bad) {
              val = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
              lse2 = __builtin_nanf("");
            }
            if (!split) {
              const size_t orow = row_of(b, g, rho);
              store_out4<IO>(a.out, orow * D + d, val);
              if (d == 0 && a.lse_out) a.lse_out[orow] = lse2 * kLn2;
            } else {
              st_agent4(wr_slot, (uint32_t)(((size_t)rho * D + d) * sizeof(float)), val);
              if (d == 0) st_agent(a.ws_lse + slot * R + rho, lse2);
            }
          }
        }
      }
      if (split) {
        const int c2 = last_to_finish(a.ws_cnt + (size_t)b * H + g, nparts, &misc[4]);
        if (c2 == kCountLast)
          merge_rows<IO, D>(a, b, g, 0, R, (size_t)slot0, nparts, -1);
        else if (c2 == kCountStale && k == 0)
          fill_pair(b, g, __builtin_nanf(""), __builtin_nanf(""));
      }
    }
    x = x_end;
    if (x == seq_first + H * cb) {
      ++b;
      seq_pre += cb;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
// Two tiles per chunk: rows that fit one tile run on the decode kernels.
template <typename IO, typename KV, int D>
static hipError_t launch_chunks(const Params& prm, dim3 grid, hipStream_t st) {
  if (prm.chunks <= 2)
    hipLaunchKernelGGL((pa_multi_kernel<IO, KV, D, kChunkTiles, false>), grid, dim3(kThreads), 0, st, prm);
  else
    hipLaunchKernelGGL((pa_multi_kernel<IO, KV, D, kChunkTiles, true>), grid, dim3(kThreads), 0, st, prm);
  return hipGetLastError();
}

template <typename IO, typename KV>
static hipError_t launch_d(int D, const Params& prm, dim3 grid, hipStream_t st) {
  return D == 64 ? launch_chunks<IO, KV, 64>(prm, grid, st) : launch_chunks<IO, KV, 128>(prm, grid, st);
}

// Balanced split: waves per chunk from the pair's row chunks (one chunk: all
// four waves on it, pages read once, non-temporal; two: two waves each; more:
// one wave per chunk, four chunks per pass), ordinary loads whenever several
// waves read each page.
template <typename IO, typename KV, int D, int WC>
static hipError_t launch_bal_wc(const Params& prm, dim3 grid, hipStream_t st) {
  using T = typename TileOf<IO, KV, D>::type;
  const size_t lds = mq_bal_layout(D, T::kQ * 64 * (int)sizeof(typename T::QC), kWaves / WC,
                                   mq_bal_merge_tiles(std::is_same<IO, F32>::value, D), prm.batch)
                         .total;
  hipLaunchKernelGGL((pa_multi_bal_kernel<IO, KV, D, WC, (WC < 4)>), grid, dim3(kThreads), lds, st, prm);
  return hipGetLastError();
}

template <typename IO, typename KV, int D>
static hipError_t launch_bal_d(const Params& prm, dim3 grid, hipStream_t st) {
  if (prm.chunks == 1) return launch_bal_wc<IO, KV, D, 4>(prm, grid, st);
  if (prm.chunks == 2) return launch_bal_wc<IO, KV, D, 2>(prm, grid, st);
  return launch_bal_wc<IO, KV, D, 1>(prm, grid, st);
}

template <typename IO, typename KV>
static hipError_t launch_bal(int D, const Params& prm, dim3 grid, hipStream_t st) {
  return D == 64 ? launch_bal_d<IO, KV, 64>(prm, grid, st) : launch_bal_d<IO, KV, 128>(prm, grid, st);
}

}  // namespace pa_mq

extern "C" {

size_t pa_decode_multi_workspace_bytes(const pa_shape* shape, int32_t q_len) {
  if (pa_host::multi_fits_one_tile(shape, q_len)) return pa::decode_workspace_bytes(shape, q_len);
  int shares = 0;
  if (shape && shape->partition_size == PA_SPLIT_BALANCED) {
    shares = pa::balanced_shares();
    if (shares < 0) return 0;
  }
  pa_host::MultiPlan p;
  if (!pa_host::multi_plan(shape, q_len, &p, shares)) return 0;
  return p.total;
}

pa_status pa_decode_multi(const pa_shape* shape, int32_t q_len, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* block_table,
                          const int32_t* context_lens, float scale, pa_dtype io_dtype,
                          pa_dtype kv_dtype, const float* k_scale, const float* v_scale,
                          void* workspace, size_t workspace_bytes, void* out, float* lse_out,
                          void* stream) {
  using namespace pa_mq;
  if (!shape) return PA_ERR_NULL;
  if (pa_host::multi_fits_one_tile(shape, q_len))
    return pa::decode_call(shape, q_len, q, k_cache, v_cache, block_table, context_lens, scale,
                           io_dtype, kv_dtype, k_scale, v_scale, workspace, workspace_bytes, out,
                           lse_out, stream);
  const bool balanced = shape->partition_size == PA_SPLIT_BALANCED;
  pa_host::MultiPlan pl;
  if (!pa_host::multi_plan(shape, q_len, &pl, balanced ? 1 : 0)) return PA_ERR_SHAPE;
  pa_status status = pa_host::io_args_status(q, k_cache, v_cache, block_table, context_lens, io_dtype,
                                             kv_dtype, k_scale, v_scale, out, lse_out);
  if (status != PA_OK) return status;
  if (balanced) {
    const int shares = pa::balanced_shares();
    if (shares < 0) return PA_ERR_HIP;
    if (!pa_host::multi_plan(shape, q_len, &pl, shares)) return PA_ERR_SHAPE;
  }
  status = pa_host::workspace_status(shape->partition_size, pl.total, 0, 0, workspace, workspace_bytes);
  if (status != PA_OK) return status;
  if (shape->batch == 0) return PA_OK;

  Params prm;
  prm.q = static_cast<const uint8_t*>(q);
  prm.k = static_cast<const uint8_t*>(k_cache);
  prm.v = static_cast<const uint8_t*>(v_cache);
  prm.block_table = block_table;
  prm.context_lens = context_lens;
  prm.k_scale = k_scale;
  prm.v_scale = v_scale;
  prm.out = static_cast<uint8_t*>(out);
  prm.lse_out = lse_out;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const bool split = shape->partition_size != 0;
  prm.ws_o = split ? reinterpret_cast<float*>(ws + pl.o_off) : nullptr;
  prm.ws_lse = split ? reinterpret_cast<float*>(ws + pl.lse_off) : nullptr;
  prm.ws_cnt = split ? reinterpret_cast<uint32_t*>(ws + pl.cnt_off) : nullptr;
  prm.scale = scale;
  prm.batch = shape->batch;
  prm.num_q_heads = shape->num_q_heads;
  prm.num_kv_heads = shape->num_kv_heads;
  prm.group = shape->num_q_heads / shape->num_kv_heads;
  prm.q_len = q_len;
  prm.rows = pl.rows;
  prm.chunks = pl.chunks;
  prm.max_blocks_per_seq = shape->max_blocks_per_seq;
  prm.num_blocks = shape->num_blocks;
  prm.part_tokens = shape->partition_size;
  prm.fan = pl.fan;
  prm.g_max = pl.g_max;
  prm.p_max = pl.p_max;

  const dim3 grid(pa_host::multi_grid(shape, pl), 1, 1);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int D = shape->head_dim;
  hipError_t e;
  if (balanced) {
    if (io_dtype == PA_F32)
      e = launch_bal<F32, F32>(D, prm, grid, st);
    else if (io_dtype == PA_F16)
      e = kv_dtype == PA_FP8_E4M3 ? launch_bal<F16, FP8>(D, prm, grid, st)
                                  : launch_bal<F16, F16>(D, prm, grid, st);
    else
      e = kv_dtype == PA_FP8_E4M3 ? launch_bal<BF16, FP8>(D, prm, grid, st)
                                  : launch_bal<BF16, BF16>(D, prm, grid, st);
  } else if (io_dtype == PA_F32)
    e = launch_d<F32, F32>(D, prm, grid, st);
  else if (io_dtype == PA_F16)
    e = kv_dtype == PA_FP8_E4M3 ? launch_d<F16, FP8>(D, prm, grid, st)
                                : launch_d<F16, F16>(D, prm, grid, st);
  else
    e = kv_dtype == PA_FP8_E4M3 ? launch_d<BF16, FP8>(D, prm, grid, st)
                                : launch_d<BF16, BF16>(D, prm, grid, st);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
