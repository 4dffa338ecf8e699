// Paged single-token decode attention for gfx950 (MI355X).
//
// What it computes is stated in include/padecode.h: for each sequence and
// query head, softmax(scale * q . K^T) V over the sequence's cached tokens,
// found through its block table ("rvLLM: High-performance LLM inference in
// Rust", section "Kernel Compiler Stack": online-softmax decode attention over
// a paged cache with grouped-query heads; section "FA3 v3 Attention Kernel":
// split-KV over several workgroups; "RapidLLM", feature table, row "Decode
// context parallelism": partials merged by log-sum-exp).
//
// One kernel does the whole call. A workgroup of kWaves wavefronts owns one
// (sequence b, KV head g, partition p) unit. Its waves take the unit's
// 16-token pages round-robin; per page a wave
//   1. reads the physical block id (block ids are fetched 64 pages at a time
//      into a VGPR, one chunk ahead, and read out with readlane, so page
//      addresses are wave-uniform scalars),
//   2. loads the K page and the V page straight from HBM into registers in the
//      layout the matrix cores consume (the cache layouts in padecode.h make
//      every one of these loads a contiguous run); K loads run two or three
//      pages ahead of the math and V loads one page ahead, through rings of
//      register buffers,
//   3. computes S^T[token][head] = K Q^T for the whole GQA group with MFMA
//      (query heads padded to 16 columns),
//   4. masks tokens past the unit's end, updates the running max and sum in
//      base 2 (scale * log2 e folded into one multiplier),
//   5. rounds P to the 16-bit operand type and accumulates O^T += V^T P^T with
//      MFMA; the running sum uses the same rounded P. The accumulator is
//      rescaled only when some head's running max moved.
// The waves' partial results are merged through LDS. With split-K, the
// partition's normalised output and base-2 log-sum-exp go to the workspace
// through agent-coherent stores; the last workgroup of each (b, g) to finish
// (device-scope atomic counter) reads them back with agent-coherent loads,
// merges all partitions of that sequence in a fixed order, writes the output
// and resets the counter to zero. Beyond 16 partitions per sequence the merge
// takes two levels (groups of partitions first), so that no workgroup reads
// hundreds of partials alone.
//
// fp8 (OCP E4M3) caches are widened exactly to f16/bf16 with the gfx950
// conversion instructions; k_scale folds into the score multiplier and
// v_scale into the output.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "padecode.h"
#include "pa_host.h"
#include "pa_internal.h"
#include "pa_schedule.h"
#include "pa_tiles.h"

namespace pa {

struct Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const int32_t* block_table;
  const int32_t* context_lens;
  const float* k_scale;
  const float* v_scale;
  uint8_t* out;
  float* lse_out;
  float* ws_o;       // [slot][G][D]   partial outputs, normalised
  float* ws_lse;     // [slot][G]      base 2, in units of the scaled scores
  uint32_t* ws_cnt;  // [B][Hkv] pieces (or first-level groups) of (b, g) finished so
                     // far, then [B][Hkv][g_max] partitions of each group finished
  float scale;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t part_tokens;  // 0: whole sequence in one unit
  int32_t p_max;        // fixed partitions: slots per (b, g)
  int32_t fan;          // fixed partitions: partitions per first-level merge group
                        // (0: a single merge level)
  int32_t g_max;        // first-level groups per (b, g); their slots follow the
                        // B * Hkv * p_max partition slots
  int32_t q_len;        // new tokens per sequence (1: decode)
  int32_t gq;           // query heads per KV head (group = gq * q_len rows)
  int32_t prefix_pages; // shared prefix: block-table entries every row shares (0: none)
};

// Several new tokens per sequence (MQ, the multi-token call when its rows fit
// one tile): row r of pair (b, g) is new token t = r / gq of head h = r % gq,
// stored at [b][t][g * gq + h]; token t sees positions 0 .. L - q_len + t.
template <bool MQ>
__device__ __forceinline__ size_t mq_row(const Params& a, int b, int g, int r) {
  const int t = r / a.gq, h = r - t * a.gq;
  return ((size_t)b * a.q_len + t) * a.num_q_heads + (size_t)g * a.gq + h;
}

// ---------------------------------------------------------------------------
// LDS for the cross-wave merge and the cross-partition merge.
// ---------------------------------------------------------------------------
template <int D>
struct Smem {
  // rows padded by 4 floats: the waves' float4 row writes (rows of 16 heads)
  // then fall on distinct LDS banks
  float acc[kWaves][kMaxGroup][D + 4];
  float m[kWaves][kMaxGroup];
  float l[kWaves][kMaxGroup];
  int bad;
  int last;
  int wsum[kWaves];   // balanced split: per-wave sums of the work-line scan
  int b0, pre0;       // balanced split: sequence holding the share's start
};

// One merge: the np pieces of pair (b, g) held in workspace slots slot0 ..
// slot0 + np - 1 (partitions, first-level groups of partitions, or pieces of
// the balanced split), folded into the final output of the pair's query rows
// (dst < 0) or into one piece (normalised output and base-2 log-sum-exp,
// like any other piece) in workspace slot dst.
struct MergeJob {
  int b, g, np;
  size_t slot0;
  long long dst;
};

constexpr int kMergeScratch = 12 * kThreads;   // floats: slice results of 2 * kThreads items

// Piece loads in flight per merge item (MB below): 8, or 4 for an fp8 cache,
// whose balanced kernel holds the widened operands beside the merge state
// and spilled registers at 256 per lane with 8.
template <typename KV>
constexpr int merge_batch() {
  return std::is_same<KV, FP8>::value ? 4 : 8;
}

// Run m merges (job j = jobs(j), all with a.group rows per pair). Threads take
// (job, slice, row, 4-float quad) items two at a time and issue the loads of
// up to MB pieces of both before folding either, so two jobs, or the
// two halves of a job with more items than threads, cost one memory round
// trip rather than two. A job's items fill whole waves (its item count
// rounded up to 64), so the job, and with it the base of the buffer resource
// its loads use, is uniform across a wave. When a job has more pieces than
// one batch, S slices split its pieces (slice s takes pieces s, s + S, ...)
// and are combined in order 0, 1, ... through LDS; within a slice pieces are
// folded in slot order. S is a function of the job's own piece count and row
// count only (merge_jobs gives a job with more than one batch of pieces a pass
// of its own), never of which other jobs the merging workgroup happens to
// hold, so the rounding does not depend on which workgroup merges: the result
// is bit-identical from run to run. A piece a row sees nothing of (lse =
// -inf) adds nothing, a row with nothing in any piece gets out = 0 and lse =
// -inf, and a NaN piece makes the row NaN. red: LDS scratch of kMergeScratch
// floats. Control flow is uniform across the workgroup.
// Slices for a job of np pieces alone in a pass (its items in one round),
// mb pieces a batch.
__device__ __forceinline__ int merge_slices(int np, int npad, int mb, int* shift) {
  int S = 1, sh = 0;
  while (S < 8 && S * mb < np && 2 * S * npad <= 2 * kThreads) {
    S *= 2;
    ++sh;
  }
  *shift = sh;
  return S;
}

template <typename IO, int D, int MB, typename Jobs>
__device__ __forceinline__ void merge_pass(const Params& a, float* red, int m, int S, int sshift, Jobs jobs) {
  constexpr int kQuads = D / 4;
  const int tid = threadIdx.x;
  const int npair = a.group * kQuads;
  const int npad = (npair + 63) & ~63;
  const int per_job = S * npad;
  const int total = m * per_job;
  const size_t slot_floats = (size_t)a.group * D;
  for (int base = 0; base < total; base += 2 * kThreads) {
    MergeJob J[2];
    int sl[2], h[2], dq[2], cnt[2];
    bool on[2], nan[2];
    float mr[2], wr[2];
    f32x4 ar[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // the wave's first item: per_job and npad are multiples of 64, so the
      // job and the slice are uniform across the wave (found by counting,
      // not dividing: at most 8 jobs and 8 slices)
      const int wbase = __builtin_amdgcn_readfirstlane(base + u * kThreads + (tid & ~63));
      int j = 0, rem = wbase;
      while (j < m && rem >= per_job) {
        ++j;
        rem -= per_job;
      }
      sl[u] = 0;
      while (rem >= npad) {
        ++sl[u];
        rem -= npad;
      }
      const int pair = rem + (tid & 63);
      on[u] = j < m && pair < npair;
      J[u] = jobs(j < m ? j : m - 1);
      cnt[u] = j < m && J[u].np > sl[u] ? (J[u].np - sl[u] + S - 1) >> sshift : 0;   // pieces of the slice
      h[u] = pair / kQuads;
      dq[u] = pair - h[u] * kQuads;
      nan[u] = false;
      mr[u] = -INFINITY;
      wr[u] = 0.f;
      ar[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int nmax = max(cnt[0], cnt[1]);
    for (int i0 = 0; i0 < nmax; i0 += MB) {
      float lp[2][MB];
      f32x4 ov[2][MB];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (i0 < cnt[u]) {   // uniform
          const int nb = min(MB, cnt[u] - i0);
          const size_t s0 = J[u].slot0 + sl[u] + (size_t)S * i0;   // first slot of the batch
          const uint32_t nslots = (uint32_t)((nb - 1) * S + 1);
          const brsrc ro = buffer_rsrc(a.ws_o + s0 * slot_floats, (uint32_t)(nslots * slot_floats * sizeof(float)));
          const brsrc rl = buffer_rsrc(a.ws_lse + s0 * a.group, (uint32_t)(nslots * a.group * sizeof(float)));
          const uint32_t vo = (uint32_t)((h[u] * D + 4 * dq[u]) * sizeof(float));
          const uint32_t vl = (uint32_t)(h[u] * sizeof(float));
#pragma unroll
          for (int q = 0; q < MB; ++q) {
            if (on[u] && q < nb) {
              lp[u][q] = ld_agent1(rl, vl, (uint32_t)(q * S * a.group * sizeof(float)));
              ov[u][q] = ld_agent4(ro, vo, (uint32_t)(q * S * slot_floats * sizeof(float)));
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int q = 0; q < MB; ++q) {
          if (on[u] && i0 + q < cnt[u]) {
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
    if (S > 1) {
      // one round (total <= 2 * kThreads): slice results through LDS, then
      // the slice-0 items combine the slices in order. red: [2 * kThreads]
      // float4s, then m, then w (NaN for a slice that met a NaN piece).
      float* redm = red + 8 * kThreads;
      float* redw = redm + 2 * kThreads;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int idx = u * kThreads + tid;
        if (on[u]) {
          *reinterpret_cast<f32x4*>(&red[4 * idx]) = ar[u];
          redm[idx] = mr[u];
          redw[idx] = nan[u] ? __builtin_nanf("") : wr[u];
        }
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int idx = u * kThreads + tid;
        if (on[u] && sl[u] == 0) {
          float M = -INFINITY;
          for (int s2 = 0; s2 < S; ++s2) M = fmaxf(M, redm[idx + s2 * npad]);
          const float Ms = M == -INFINITY ? 0.f : M;
          float W = 0.f;
          f32x4 A = {0.f, 0.f, 0.f, 0.f};
          for (int s2 = 0; s2 < S; ++s2) {
            const int k = idx + s2 * npad;
            const float e = exp2_fast(redm[k] - Ms);
            W += e * redw[k];
            A += e * *reinterpret_cast<const f32x4*>(&red[4 * k]);
          }
          mr[u] = M;
          wr[u] = W;
          ar[u] = A;
          nan[u] = W != W;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!on[u] || sl[u] != 0) continue;
      f32x4 val = {0.f, 0.f, 0.f, 0.f};
      float lse2 = -INFINITY;   // base 2
      if (nan[u]) {
        val = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
        lse2 = __builtin_nanf("");
      } else if (wr[u] > 0.f) {
        val = ar[u] * __builtin_amdgcn_rcpf(wr[u]);
        lse2 = mr[u] + log2_fast(wr[u]);
      }
      if (J[u].dst < 0) {
        const size_t row = mq_row<true>(a, J[u].b, J[u].g, h[u]);
        store_out4<IO>(a.out, row * D + 4 * dq[u], val);
        if (dq[u] == 0 && a.lse_out) a.lse_out[row] = lse2 * kLn2;
      } else {
        const size_t dst = (size_t)J[u].dst;
        const brsrc wd = buffer_rsrc(a.ws_o + dst * slot_floats, (uint32_t)(slot_floats * sizeof(float)));
        st_agent4(wd, (uint32_t)((h[u] * D + 4 * dq[u]) * sizeof(float)), val);
        if (dq[u] == 0) st_agent(a.ws_lse + dst * a.group + h[u], lse2);
      }
    }
  }
}

// Run m merges: jobs of at most MB pieces all in one pass (one slice each);
// otherwise every job in a pass of its own, with its own slice count.
template <typename IO, int D, int MB, typename Jobs>
__device__ __forceinline__ void merge_jobs(const Params& a, float* red, int m, int np_max, Jobs jobs) {
  if (np_max <= MB) {
    merge_pass<IO, D, MB>(a, red, m, 1, 0, jobs);
    return;
  }
  const int npad = (a.group * (D / 4) + 63) & ~63;
  for (int j = 0; j < m; ++j) {
    const MergeJob J = jobs(j);
    int sh;
    const int S = merge_slices(J.np, npad, MB, &sh);
    if (j > 0) __syncthreads();   // the previous pass's slice results in LDS are consumed
    merge_pass<IO, D, MB>(a, red, 1, S, sh, [&](int) { return J; });
  }
}

// The single merge of one pair.
template <typename IO, int D, int MB>
__device__ __forceinline__ void merge_one(const Params& a, float* red, const MergeJob& job) {
  merge_jobs<IO, D, MB>(a, red, 1, job.np, [&](int) { return job; });
}

// Every output row of pair (b, g) (and its lse) set to x by the workgroup.
template <typename IO, int D, bool MQ>
__device__ __forceinline__ void fill_rows(const Params& a, int b, int g, float x) {
  const int tid = threadIdx.x;
  for (int i = tid; i < a.group * D; i += kThreads) {
    size_t row;
    if constexpr (MQ) row = mq_row<MQ>(a, b, g, i / D);
    else row = (size_t)b * a.num_q_heads + (size_t)g * a.group + i / D;
    store_out<IO>(a.out, row * D + i % D, x);
    if (i % D == 0 && a.lse_out) a.lse_out[row] = x;
  }
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
// What the caller knows of a piece once the context length is in.
struct Piece {
  int L;        // context length of the sequence
  int pg_hi;    // one past the piece's last page (tokens past L are cut off)
  int k;        // index of the piece among the pieces of (b, g)
  int nparts;   // pieces of (b, g); 1: write the output directly; 0: no work
  int slot0;    // workspace slot of piece 0 of (b, g)
};

// One piece: pages page0 .. pg_hi - 1 of sequence b for KV head g, by the
// whole workgroup. resolve() returns the Piece; it is called after the loads
// that do not depend on it are issued. Control flow is uniform across the
// workgroup.
template <typename IO, typename KV, int D, bool MQ, typename Resolve>
__device__ __forceinline__ void decode_piece(const Params& a, Smem<D>& sm, const int b, const int g,
                                             const int page0, Resolve resolve) {
  using T = typename TileOf<IO, KV, D>::type;
  constexpr bool kFp8 = std::is_same<KV, FP8>::value;
  constexpr size_t kPageBytes = (size_t)kBlock * D * ElemSize<KV>::v;

  // The thread index passes through an empty asm statement so that the
  // per-lane offsets below are recomputed for every piece rather than hoisted
  // out of the balanced kernel's piece loop, where they would stay live (and
  // spill) across all of it.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.group;
  const int hq0 = g * G;

  const int rr = lane & 15, jj = lane >> 4;
  const bool head_ok = rr < G;

  // Issued before the context length is known (all indices stay in bounds):
  // the block ids of this wave's first 64 pages and the query operand.
  const int32_t* bt = a.block_table + (size_t)b * a.max_blocks_per_seq + w;
  const int bt_last = a.max_blocks_per_seq - 1 - w;
  auto fetch_bt = [&](int chunk) {
    return bt[min(page0 + kWaves * (chunk * 64 + lane), bt_last)];
  };
  int bt_cur = fetch_bt(0);
  typename T::Q qop;
  if constexpr (MQ)
    T::load_q(qop, (gptr)(a.q + mq_row<MQ>(a, b, g, head_ok ? rr : 0) * D * ElemSize<IO>::v), jj);
  else
    T::load_q(qop, (gptr)(a.q + ((size_t)b * a.num_q_heads + hq0 + (head_ok ? rr : 0)) * D * ElemSize<IO>::v),
              jj);

  const Piece pc = resolve();
  if (pc.nparts == 0) return;
  const int L = pc.L;
  const bool bad_len = L < 0 || L > a.max_blocks_per_seq * kBlock;
  if (bad_len || L == 0) {
    // No tokens (or an out-of-contract length): zeros, resp. NaN.
    const float fill = bad_len ? __builtin_nanf("") : 0.f;
    if constexpr (MQ) {
      for (int i = tid; i < G * D; i += kThreads)
        store_out<IO>(a.out, mq_row<MQ>(a, b, g, i / D) * D + i % D, fill);
      if (a.lse_out && tid < G) a.lse_out[mq_row<MQ>(a, b, g, tid)] = bad_len ? fill : -INFINITY;
    } else {
      for (int i = tid; i < G * D; i += kThreads)
        store_out<IO>(a.out, ((size_t)b * a.num_q_heads + hq0) * D + i, fill);
      if (a.lse_out && tid < G)
        a.lse_out[(size_t)b * a.num_q_heads + hq0 + tid] = bad_len ? fill : -INFINITY;
    }
    return;
  }
  // MQ: last position this lane's row may see
  int lim = 0;
  if constexpr (MQ) lim = L - a.q_len + (head_ok ? rr : 0) / a.gq;

  const int t0 = page0 * kBlock;
  const int t1 = min(pc.pg_hi * kBlock, L);
  const int npages = (t1 - t0 + kBlock - 1) / kBlock;
  const int nmine = npages > w ? (npages - w + kWaves - 1) / kWaves : 0;

  float kmul = a.scale * kLog2e;
  float vmul = 1.0f;
  if constexpr (kFp8) {
    kmul *= a.k_scale[g];
    vmul = a.v_scale[g];
  }

  int bt_next = nmine > 64 ? fetch_bt(1) : 0;

  const gptr kbase = uniform_ptr(a.k + (size_t)g * kPageBytes);
  const gptr vbase = uniform_ptr(a.v + (size_t)g * kPageBytes);
  const size_t block_stride = (size_t)a.num_kv_heads * kPageBytes;
  const uint32_t ko = T::koff(lane), vo = T::voff(lane);
  bool bad_blk = false;

  // Register rings: K pages are loaded kKS - 1 pages ahead of the page being
  // computed, V pages kVS - 1 ahead (V is needed only after the softmax).
  // poff[] keeps each K slot's page offset so the later V load of the same
  // page reuses it.
  constexpr int kKS = T::kKStages, kVS = T::kVStages;
  constexpr int dK = kKS - 1, dV = kVS - 1;
  static_assert(kKS >= 1 && kVS >= 1 && dV <= dK, "ring depths");
  // the steady-state block must stop short of a wave's last page
  constexpr int kAhead = dK > 1 ? dK : 1;
  typename T::KRegs ring_k[kKS];
  typename T::VRegs ring_v[kVS];
  size_t poff[kKS];

  // kRefresh: the wave has more than 64 pages, so block ids are re-fetched
  // every 64 pages inside the loop (see run_ring below).
  auto issue_k = [&](int slot, int i, auto refresh_tag) {
    if constexpr (decltype(refresh_tag)::value) {
      if (i > 0 && (i & 63) == 0) {
        bt_cur = bt_next;
        if (nmine > i + 64) bt_next = fetch_bt((i >> 6) + 1);
      }
    }
    int phys = __builtin_amdgcn_readlane(bt_cur, i & 63);
    if ((unsigned)phys >= (unsigned)a.num_blocks) {
      bad_blk = true;
      phys = 0;
    }
    poff[slot] = (size_t)phys * block_stride;
    T::load_k(ring_k[slot], kbase + poff[slot], ko);
  };
  auto issue_v = [&](int vslot, int kslot) { T::load_v(ring_v[vslot], vbase + poff[kslot], vo); };

  float m = -INFINITY, lsum = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One page of the online softmax. kMasked: the page may end before its
  // 16th token (only a wave's last page can).
  auto compute = [&](int kslot, int vslot, int i, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const f32x4 s = T::scores(ring_k[kslot], qop);
    int nvalid = kBlock;
    float sc[4];
    if constexpr (kMasked) {
      const int pos = t0 + (w + kWaves * i) * kBlock;
      nvalid = t1 - pos;
      if constexpr (MQ) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sc[e] = (4 * jj + e < nvalid && pos + 4 * jj + e <= lim) ? s[e] * kmul : -INFINITY;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[e] = (4 * jj + e < nvalid) ? s[e] * kmul : -INFINITY;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = s[e] * kmul;
    }
    const float mx = wave_max_rows(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    const float mnew = fmaxf(m, mx);
    // MQ: a row that sees nothing yet keeps a zero state (exponentials
    // against 0 instead of -inf - -inf)
    float msafe = mnew;
    if constexpr (MQ && kMasked) msafe = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = exp2_fast(m - msafe);
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = exp2_fast(sc[e] - msafe);
    const typename T::P pk = T::pack(pr);
    lsum = lsum * alpha + T::psum(pk);
    m = mnew;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int t = 0; t < D / 16; ++t) acc[t] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      typename T::A4 va = T::pvt(ring_v[vslot], t);
      if constexpr (kMasked) va = T::zero_tail(va, jj, nvalid);
      acc[t] = T::pv(va, pk, acc[t]);
    }
  };
  using Full = std::integral_constant<bool, false>;
  using Tail = std::integral_constant<bool, true>;

  // The steady-state block (kU = lcm(kKS, kVS) pages) issues unconditionally
  // and never holds a wave's last page (the only one that can be partial);
  // the peeled remainder issues and masks as needed.
  constexpr int kU = kKS * kVS / gcd_c(kKS, kVS);
  // Two copies of the loop: with no block-id fetch inside it (at most 64
  // pages per wave, the usual case) the compiler's wait counts for the ring
  // stay exact; a fetch inside the loop makes them conservative (it then
  // waits for nearly every load in flight at the top of each iteration).
  auto run_ring = [&](auto refresh_tag) {
#pragma unroll
    for (int j = 0; j < dK; ++j)
      if (j < nmine) issue_k(j, j, refresh_tag);
#pragma unroll
    for (int j = 0; j < dV; ++j)
      if (j < nmine) issue_v(j, j);
    int i0 = 0;
    for (; i0 + kU - 1 + kAhead < nmine; i0 += kU) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        issue_k((u + dK) % kKS, i0 + u + dK, refresh_tag);
        issue_v((u + dV) % kVS, (u + dV) % kKS);
        compute(u % kKS, u % kVS, i0 + u, Full{});
      }
    }
#pragma unroll
    for (int u = 0; u < kU + kAhead; ++u) {
      const int i = i0 + u;
      if (i < nmine) {
        if (i + dK < nmine) issue_k((u + dK) % kKS, i + dK, refresh_tag);
        if (i + dV < nmine) issue_v((u + dV) % kVS, (u + dV) % kKS);
        compute(u % kKS, u % kVS, i, Tail{});
      }
    }
  };
  if (nmine > 64)
    run_ring(std::integral_constant<bool, true>{});
  else
    run_ring(std::integral_constant<bool, false>{});

  // ---- merge the waves through LDS --------------------------------------
  lsum = wave_sum_rows(lsum);
  if (tid == 0) sm.bad = 0;
  __syncthreads();
  if (bad_blk) sm.bad = 1;
  if (head_ok) {
    if (jj == 0) {
      sm.m[w][rr] = m;
      sm.l[w][rr] = lsum;
    }
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      *reinterpret_cast<f32x4*>(&sm.acc[w][rr][16 * t + 4 * jj]) = acc[t];
  }
  __syncthreads();
  const bool bad = sm.bad != 0;

  const bool split = pc.nparts > 1;
  const size_t slot = (size_t)pc.slot0 + pc.k;
  const brsrc wr_slot = buffer_rsrc(a.ws_o + slot * G * D, (uint32_t)(G * D * sizeof(float)));
  for (int i = tid; i < G * (D / 4); i += kThreads) {   // (head, 4-float quad)
    const int h = i / (D / 4), d = 4 * (i - h * (D / 4));
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.m[ww][h]);
    float W = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    const float Ms = (MQ && M == -INFINITY) ? 0.f : M;   // MQ: a row may see nothing here
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float e = exp2_fast(sm.m[ww][h] - Ms);
      W += e * sm.l[ww][h];
      o += e * *reinterpret_cast<const f32x4*>(&sm.acc[ww][h][d]);
    }
    f32x4 val = o * (__builtin_amdgcn_rcpf(W) * vmul);
    float lse2 = M + log2_fast(W);
    if constexpr (MQ) {
      if (!(W > 0.f)) {
        val = f32x4{0.f, 0.f, 0.f, 0.f};
        lse2 = -INFINITY;
      }
    }
    if (bad) {
      val = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      lse2 = __builtin_nanf("");
    }
    size_t row;
    if constexpr (MQ) row = mq_row<MQ>(a, b, g, h);
    else row = (size_t)b * a.num_q_heads + hq0 + h;
    if (!split) {
      store_out4<IO>(a.out, row * D + d, val);
      if (d == 0 && a.lse_out) a.lse_out[row] = lse2 * kLn2;
    } else {
      st_agent4(wr_slot, (uint32_t)((h * D + d) * sizeof(float)), val);
      if (d == 0) st_agent(a.ws_lse + slot * G + h, lse2);
    }
  }
  if (!split) return;

  // ---- split-K: the last partition of (b, g) to finish merges ------------
  // With more than a.fan partitions (fixed partitions only) the merge has two
  // levels: the last finisher of each group of a.fan consecutive partitions
  // merges the group into a group slot, and the last group merges the group
  // slots. A single workgroup reading hundreds of partials would be held to
  // one CU's read rate.
  static_assert(sizeof(sm.acc) >= kMergeScratch * sizeof(float), "merge scratch");
  float* red = &sm.acc[0][0][0];
  const size_t nbg = (size_t)a.batch * a.num_kv_heads;
  const size_t bg = (size_t)b * a.num_kv_heads + g;
  size_t first = pc.slot0;
  int np = pc.nparts;
  bool reporter = pc.k == 0;   // the piece that reports a stale count of (b, g)
  if (a.fan > 0 && pc.nparts > a.fan) {
    const int grp = pc.k / a.fan;
    const int gfirst = grp * a.fan;
    const int gn = min(a.fan, pc.nparts - gfirst);
    first = nbg * a.p_max + bg * a.g_max;   // the group slots of (b, g)
    const int c1 = last_to_finish(a.ws_cnt + nbg + bg * a.g_max + grp, gn, &sm.last);
    if (c1 == kCountMore) return;
    if (c1 == kCountStale) {
      // one piece of the group (its first) reports it: the group slot gets a
      // NaN log-sum-exp, so the final merge makes the rows NaN, and the group
      // is counted at the second level like a merged one
      if (pc.k != gfirst) return;
      if (tid < G) st_agent(a.ws_lse + (first + grp) * G + tid, __builtin_nanf(""));
    } else {
      merge_one<IO, D, merge_batch<KV>()>(a, red,
                                          MergeJob{b, g, gn, (size_t)pc.slot0 + gfirst, (long long)(first + grp)});
    }
    np = (pc.nparts + a.fan - 1) / a.fan;
    reporter = grp == 0;
  }
  const int c2 = last_to_finish(a.ws_cnt + bg, np, &sm.last);
  if (c2 == kCountLast) {
    merge_one<IO, D, merge_batch<KV>()>(a, red, MergeJob{b, g, np, first, -1});
  } else if (c2 == kCountStale && reporter) {
    fill_rows<IO, D, MQ>(a, b, g, __builtin_nanf(""));
  }
}

// Fixed schedule: one workgroup per (sequence b, KV head g, partition p) unit
// (partition = the whole sequence when part_tokens == 0).
template <typename IO, typename KV, int D, bool MQ>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
pa_decode_kernel(const Params a) {
  __shared__ Smem<D> sm;
  // Work units are numbered partition-major, unit = p * (B * Hkv) + b * Hkv
  // + g, because the hardware hands consecutive workgroups to the eight XCDs
  // in turn: every XCD then gets an even share of each partition level, whose
  // population shrinks with p.
  const int H = a.num_kv_heads;
  const int nbg = a.batch * H;
  const int p = blockIdx.x / nbg;
  const int bg = blockIdx.x - p * nbg;
  const int b = bg / H;
  const int g = bg - b * H;
  const int PT = a.part_tokens;
  const int page0 = PT > 0 ? p * (PT / kBlock) : 0;
  decode_piece<IO, KV, D, MQ>(a, sm, b, g, page0, [&]() {
    Piece pc;
    pc.L = a.context_lens[b];
    const bool bad_len = pc.L < 0 || pc.L > a.max_blocks_per_seq * kBlock;
    const int n = (bad_len || pc.L == 0) ? 1 : (PT > 0 ? (pc.L + PT - 1) / PT : 1);
    pc.nparts = p < n ? n : 0;
    pc.k = p;
    pc.pg_hi = PT > 0 ? page0 + PT / kBlock : a.max_blocks_per_seq;
    pc.slot0 = bg * a.p_max;
    return pc;
  });
}

// ---------------------------------------------------------------------------
// Balanced schedule.
//
// The work line (pa_schedule.h) is cut into equal shares, one per workgroup
// (numbered XCD by XCD); the grid (kWgPerCu workgroups per CU) is resident
// all at once, so every CU gets the same number of pages. Each workgroup first loads the
// context lengths into LDS with the exclusive prefix sums of their line
// positions (a scan over the workgroup, batch <= kThreads * kScanPerThread);
// every later lookup of "which sequence holds line position x" is a binary
// search there. Wave w then takes the contiguous quarter [y_w, y_w+1) of the
// share and streams its pages through one register ring from the first to
// the last, across all the (sequence, KV head) pairs the quarter touches:
//   - block ids and per-position facts (tokens in the page, KV head, "last
//     position of its piece") are fetched 64 positions at a time, one chunk
//     ahead;
//   - the query rows (and fp8 scales) of the next pair are loaded while the
//     current pair is computed;
//   - at a pair's last position in the quarter the wave flushes its softmax
//     state: a pair that lies whole inside the quarter gets its output
//     written by the wave; any other piece (it continues into a neighbouring
//     quarter or share) goes to one of the wave's two LDS slots, slot 0 for
//     the piece that starts the quarter, slot 1 for the one that ends it,
//     with a record of its pair, its range of shares and whether it leads.
// After its quarter, the workgroup combines, for every leading piece of the
// share, the slots of the waves holding it (all pieces in one pass), and
// writes the output (pair inside the share) or a partial result, handed on to
// the last-finisher merge of the pair as in the fixed schedule; the pairs it
// completes are merged together in one pass.
// ---------------------------------------------------------------------------
constexpr int kScanPerThread = 16;
constexpr int kBalancedMaxBatch = pa_host::kBalancedMaxBatch;
static_assert(kBlock == pa_host::kPageTokens && kLineBlock == pa_host::kPageTokens, "page size");
static_assert(kMaxGroup == pa_host::kMaxGroup, "group limit");
static_assert(kBalancedMaxBatch <= kThreads * kScanPerThread, "the scan covers the batch");
static_assert(kMinSharePages >= kWaves, "a share gives every wave a page");

// Per-position facts in a lane's meta word.
constexpr int kMetaValid = 31;     // tokens of the page; 0: placeholder position
constexpr int kMetaEnd = 32;       // last position of its piece in the quarter
constexpr int kMetaBad = 64;       // block id outside the pool
constexpr int kMetaHeadShift = 8;  // KV head in bits 8..23
constexpr int kMetaNear = 128;     // MQ: one of the sequence's last two pages
constexpr int kMetaPfeShift = 24;  // MQ: bit 24 set for the second-to-last page

// Dynamic LDS of the balanced kernel, sized by group G, head_dim D, batch B.
// Each wave has two slots for pieces that go through the LDS merge: slot 0
// for the piece its quarter starts with (the pair began at or before the
// quarter), slot 1 for the piece it ends with (the pair goes on past it).

struct BalLayout {
  uint32_t acc, m, l, bad, pm, red, len, pre, misc, split, full, pfx, total;   // byte offsets
};
// Per (wave, slot), recorded when the wave flushes the piece it holds: the
// pair's sequence and KV head, its end line position, the output multiplier
// (v_scale, as float bits), its pieces over the shares (count, this share's
// index among them, workspace slot of the first) and flags (in use; the slot
// leads the piece, i.e. no earlier wave of the share holds the pair).
constexpr int kPmB = 0, kPmG = 1, kPmEnd = 2, kPmVmul = 3, kPmParts = 4, kPmK = 5, kPmSlot0 = 6, kPmFlags = 7;
constexpr int kPieceMeta = 8;
constexpr int kPmUsed = 1, kPmLead = 2;
__host__ __device__ inline uint32_t lds_align(uint32_t x) { return (x + 15u) & ~15u; }
// Shared prefix (pfx): the prefix shares keep one 16-row tile per wave in the
// same acc / m / l regions ([kWaves][16][D + 4], [kWaves][16]), so each wave
// gets max(2G, 16) rows; full holds the sequences' whole lengths (len then
// holds their suffixes) and pfx the prefix shares' flags and counts.
constexpr int kPfxBad = 0;                    // [kWaves][16] rows that met a bad or foreign block id
constexpr int kPfxDone = kWaves * 16;         // [2]: sequences whose count a prefix piece completed
constexpr int kPfxKey = kPfxDone + 2;         // [kWaves][2]: longest sequence, per wave
constexpr int kPfxJob = kPfxKey + 2 * kWaves; // [3][64]: pairs a workgroup merges (pair, pieces, slot0)
constexpr int kPfxInts = kPfxJob + 3 * 64;
__host__ __device__ inline BalLayout bal_layout(int G, int D, int B, bool pfx = false) {
  BalLayout o;
  uint32_t p = 0;
  const int rw = pfx && 2 * G < 16 ? 16 : 2 * G;   // rows per wave
  o.acc = p;  p = lds_align(p + 4u * kWaves * rw * (D + 4));      // [kWaves][2][G][D + 4]
  o.m = p;    p = lds_align(p + 4u * kWaves * rw);                // [kWaves][2][G]
  o.l = p;    p = lds_align(p + 4u * kWaves * rw);
  o.bad = p;  p = lds_align(p + 4u * kWaves * 2);                 // [kWaves][2]
  o.pm = p;   p = lds_align(p + 4u * kWaves * 2 * kPieceMeta);    // [kWaves][2][kPieceMeta]
  o.red = p;  p = lds_align(p + 4u * kMergeScratch);
  o.len = p;  p = lds_align(p + 4u * B);                          // [B]
  o.pre = p;  p = lds_align(p + 4u * (B + 1));                    // [B + 1]
  o.misc = p; p = lds_align(p + 4u * kWaves);                     // wsum[kWaves]
  o.split = p; p = lds_align(p + 4u * 2 * kWaves);               // [0]: completed pairs, [1]: stale ones
  o.full = p; p = lds_align(p + (pfx ? 4u * B : 0u));            // [B]
  o.pfx = p;  p = lds_align(p + (pfx ? 4u * kPfxInts : 0u));
  o.total = p;
  return o;
}

extern __shared__ __attribute__((aligned(16))) uint8_t bal_lds[];

template <int D>
struct BalSm {
  float* acc;
  float* m;
  float* l;
  int* bad;
  int* pm;
  float* red;
  int* len;
  int* pre;
  int* misc;
  int* split;   // bit c set when the workgroup completed candidate slot c's pair ([0]) or
                // found its counter stale and reports it ([1])
  int* full;    // shared prefix: whole lengths (len holds the suffixes)
  int* pfx;
  int G;
  __device__ BalSm(int G_, int B, bool pfx_ = false) : G(G_) {
    const BalLayout o = bal_layout(G_, D, B, pfx_);
    acc = reinterpret_cast<float*>(bal_lds + o.acc);
    m = reinterpret_cast<float*>(bal_lds + o.m);
    l = reinterpret_cast<float*>(bal_lds + o.l);
    bad = reinterpret_cast<int*>(bal_lds + o.bad);
    pm = reinterpret_cast<int*>(bal_lds + o.pm);
    red = reinterpret_cast<float*>(bal_lds + o.red);
    len = reinterpret_cast<int*>(bal_lds + o.len);
    pre = reinterpret_cast<int*>(bal_lds + o.pre);
    misc = reinterpret_cast<int*>(bal_lds + o.misc);
    split = reinterpret_cast<int*>(bal_lds + o.split);
    full = reinterpret_cast<int*>(bal_lds + o.full);
    pfx = reinterpret_cast<int*>(bal_lds + o.pfx);
  }
  __device__ float* acc_row(int w, int slot, int h) const { return acc + ((w * 2 + slot) * G + h) * (D + 4); }
  __device__ int mi(int w, int slot, int h) const { return (w * 2 + slot) * G + h; }
};

// The sequence holding line position x: the largest b < B with H*pre[b] <= x.
__device__ __forceinline__ int seq_of(const int* pre, int B, int H, int x) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (H * pre[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}
__device__ __forceinline__ int seq_of_uniform(const int* pre, int B, int H, int x) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (H * __builtin_amdgcn_readfirstlane(pre[mid]) <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// A uniform cursor on one piece of a quarter [., y1): the pair (b, g) and the
// pages pg_lo .. pg_hi - 1 of it that lie in the quarter.
struct QCursor {
  int b, L;
  int g, pg_lo, pg_hi;
  int pair_first, pair_end;  // the pair's line positions
};

// The piece at line position x (uniform); P: shared prefix pages (0: none).
template <int D>
__device__ __forceinline__ void qcursor_at(QCursor& c, const Params& a, const BalSm<D>& sm, int x,
                                           int y1, int P) {
  const int H = a.num_kv_heads;
  c.b = seq_of_uniform(sm.pre, a.batch, H, x);
  c.L = __builtin_amdgcn_readfirstlane(sm.len[c.b]);
  const int cb = pfx_positions(P, c.L, a.max_blocks_per_seq);
  const int sf = H * __builtin_amdgcn_readfirstlane(sm.pre[c.b]);
  c.g = (x - sf) / cb;
  c.pg_lo = x - sf - c.g * cb;
  c.pair_first = sf + c.g * cb;
  c.pair_end = c.pair_first + cb;
  c.pg_hi = c.pg_lo + (min(y1, c.pair_end) - x);
}

// The share a workgroup works on: index wg of s shares over n line positions.
struct ShareOf {
  int wg, n, s;
};


// One wave's quarter [y0, y1) of share sh.
// PFX: the line holds the pairs' suffixes (len: suffix length, -1 for an
// out-of-contract sequence), whose pages start at page (full - len) / 16 of
// the sequence, pfx_pages the prefix pages read once; with a prefix every
// piece goes through a workspace slot, since the pair's prefix pieces are
// merged with it.
template <typename IO, typename KV, int D, bool MQ, bool PFX>
__device__ __forceinline__ void decode_quarter(const Params& a, const BalSm<D>& sm, const ShareOf& sh,
                                               const int y0, const int y1, const int pfx_pages) {
  using T = typename TileOf<IO, KV, D>::type;
  constexpr bool kFp8 = std::is_same<KV, FP8>::value;
  constexpr size_t kPageBytes = (size_t)kBlock * D * ElemSize<KV>::v;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.group, H = a.num_kv_heads, mbs = a.max_blocks_per_seq, B = a.batch;
  const int rr = lane & 15, jj = lane >> 4;
  const bool head_ok = rr < G;
  const int n = y1 - y0;
  const int P = PFX ? pfx_pages : 0;
  if constexpr (PFX)
    if (n <= 0) return;   // a short suffix line leaves some quarters empty

  // ---- block ids and position facts, 64 positions per chunk ---------------
  auto fetch_chunk = [&](int c0, int& blk, int& meta) {
    const int xp = y0 + c0 + lane;
    blk = 0;
    meta = 0;
    if (xp < y1) {
      const int bl = seq_of(sm.pre, B, H, xp);
      const int L = sm.len[bl];
      const int cb = pfx_positions(P, L, mbs);
      const int sf = H * sm.pre[bl];
      const int g = (xp - sf) / cb;
      const int page = xp - sf - g * cb;
      const int pair_end = sf + (g + 1) * cb;
      const bool valid = L > 0 && L <= mbs * kBlock;
      int first = 0;   // PFX: the suffix's first page in the sequence
      if constexpr (PFX) first = valid ? (sm.full[bl] - L) / kBlock : 0;
      if (valid) blk = a.block_table[(size_t)bl * mbs + first + page];
      meta = (valid ? min(kBlock, L - page * kBlock) : 0) | (xp + 1 == min(y1, pair_end) ? kMetaEnd : 0) |
             (g << kMetaHeadShift);
      if constexpr (PFX)
        if (L < 0) meta |= kMetaBad;   // out-of-contract length: NaN rows
      if constexpr (MQ) {
        const int pfe = cb - 1 - page;   // pages from the end of the sequence
        if (valid && pfe <= 1) meta |= kMetaNear | (pfe << kMetaPfeShift);
      }
    }
  };
  int bt_cur, meta_cur, bt_nxt = 0, meta_nxt = 0;
  fetch_chunk(0, bt_cur, meta_cur);
  if (n > 64) fetch_chunk(64, bt_nxt, meta_nxt);

  // ---- the pieces, in order: the current one and the next ----------------
  QCursor cur, nxt;
  qcursor_at(cur, a, sm, y0, y1, P);
  bool has_nxt = cur.pair_end < y1;
  if (has_nxt) qcursor_at(nxt, a, sm, cur.pair_end, y1, P);
  auto q_row = [&](const QCursor& c) {
    if constexpr (MQ) return (gptr)(a.q + mq_row<MQ>(a, c.b, c.g, head_ok ? rr : 0) * D * ElemSize<IO>::v);
    else return (gptr)(a.q + ((size_t)c.b * a.num_q_heads + c.g * G + (head_ok ? rr : 0)) * D * ElemSize<IO>::v);
  };
  // MQ: new token of this lane's row, and the last position it may see in the
  // current piece's sequence
  const int t_rr = MQ ? (head_ok ? rr : 0) / a.gq : 0;
  int lim_cur = 0;
  if constexpr (MQ) lim_cur = cur.L - a.q_len + t_rr;
  typename T::Q q_cur, q_nxt;
  T::load_q(q_cur, q_row(cur), jj);
  if (has_nxt) T::load_q(q_nxt, q_row(nxt), jj);
  float kmul_cur = a.scale * kLog2e, kmul_nxt = kmul_cur, vmul_cur = 1.0f, vmul_nxt = 1.0f;
  if constexpr (kFp8) {
    const float s0 = kmul_cur;
    kmul_cur = s0 * a.k_scale[cur.g];
    vmul_cur = a.v_scale[cur.g];
    if (has_nxt) {
      kmul_nxt = s0 * a.k_scale[nxt.g];
      vmul_nxt = a.v_scale[nxt.g];
    }
  }

  const gptr kbase = uniform_ptr(a.k);
  const gptr vbase = uniform_ptr(a.v);
  const uint32_t ko = T::koff(lane), vo = T::voff(lane);

  constexpr int kKS = T::kKStages, kVS = T::kVStages;
  constexpr int dK = kKS - 1, dV = kVS - 1;
  static_assert(kKS >= 1 && kVS >= 1 && dV <= dK, "ring depths");
  constexpr int kAhead = dK > 1 ? dK : 1;
  typename T::KRegs ring_k[kKS];
  typename T::VRegs ring_v[kVS];
  size_t poff[kKS];
  int meta_k[kKS];

  auto issue_k = [&](int slot, int i, auto refresh_tag) {
    if constexpr (decltype(refresh_tag)::value) {
      if (i > 0 && (i & 63) == 0) {
        bt_cur = bt_nxt;
        meta_cur = meta_nxt;
        if (n > i + 64) fetch_chunk(i + 64, bt_nxt, meta_nxt);
      }
    }
    // Loads are issued for every position, placeholders included (they read
    // block 0 and are never used): a load under a branch would make the
    // compiler's wait counts for the whole ring conservative.
    int mk = __builtin_amdgcn_readlane(meta_cur, i & 63);
    int phys = __builtin_amdgcn_readlane(bt_cur, i & 63);
    if (!(mk & kMetaValid)) phys = 0;
    if ((unsigned)phys >= (unsigned)a.num_blocks) {
      mk |= kMetaBad;
      phys = 0;
    }
    const int g = (mk >> kMetaHeadShift) & 0xffff;
    poff[slot] = ((size_t)phys * H + g) * kPageBytes;
    T::load_k(ring_k[slot], kbase + poff[slot], ko);
    meta_k[slot] = mk;
  };
  auto issue_v = [&](int vslot, int kslot) { T::load_v(ring_v[vslot], vbase + poff[kslot], vo); };

  float m = -INFINITY, lsum = 0.f;
  bool bad = false;
  f32x4 acc[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One page of the online softmax (as in the fixed schedule).
  // pos: first position of the page in its sequence (MQ, masked pages only)
  auto page_math = [&](int kslot, int vslot, int nvalid, int pos, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const f32x4 s = T::scores(ring_k[kslot], q_cur);
    float sc[4];
    if constexpr (MQ && kMasked) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sc[e] = (4 * jj + e < nvalid && pos + 4 * jj + e <= lim_cur) ? s[e] * kmul_cur : -INFINITY;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = (!kMasked || 4 * jj + e < nvalid) ? s[e] * kmul_cur : -INFINITY;
    }
    const float mx = wave_max_rows(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    const float mnew = fmaxf(m, mx);
    float msafe = mnew;
    if constexpr (MQ && kMasked) msafe = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = exp2_fast(m - msafe);
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = exp2_fast(sc[e] - msafe);
    const typename T::P pk = T::pack(pr);
    lsum = lsum * alpha + T::psum(pk);
    m = mnew;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int t = 0; t < D / 16; ++t) acc[t] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      typename T::A4 va = T::pvt(ring_v[vslot], t);
      if constexpr (kMasked) va = T::zero_tail(va, jj, nvalid);
      acc[t] = T::pv(va, pk, acc[t]);
    }
  };

  // End of the current piece: flush the state, move to the next piece.
  auto flush = [&]() {
    const float l = wave_sum_rows(lsum);
    const bool direct = cur.pair_first >= y0 && cur.pair_end <= y1;
    if (PFX && direct) {
      // the whole suffix of the pair is here (one share, piece 0): its partial
      // goes straight to the pair's first slot; the workgroup counts it once
      // every wave's stores are complete
      const int slot = share_of(cur.pair_first, sh.n, sh.s) + (cur.b * H + cur.g) * (1 + kPfxPieces);
      if (head_ok) {
        const bool none = !(l > 0.f);
        const float inv = bad ? __builtin_nanf("") : (none ? 0.f : vmul_cur / l);
        const brsrc wr = buffer_rsrc(a.ws_o + (size_t)slot * G * D, (uint32_t)(G * D * sizeof(float)));
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
          st_agent4(wr, (uint32_t)((rr * D + 16 * t + 4 * jj) * sizeof(float)), acc[t] * inv);
        if (jj == 0)
          st_agent(a.ws_lse + (size_t)slot * G + rr,
                   bad ? __builtin_nanf("") : (none ? -INFINITY : m + log2_fast(l)));
      }
    } else if (direct) {
      const size_t row0 = (size_t)cur.b * a.num_q_heads + (size_t)cur.g * G;
      const bool bad_len = cur.L < 0 || cur.L > mbs * kBlock;
      if (bad_len || cur.L == 0) {
        const float fill = bad_len ? __builtin_nanf("") : 0.f;
        if constexpr (MQ) {
          for (int i = lane; i < G * D; i += 64)
            store_out<IO>(a.out, mq_row<MQ>(a, cur.b, cur.g, i / D) * D + i % D, fill);
          if (a.lse_out && lane < G) a.lse_out[mq_row<MQ>(a, cur.b, cur.g, lane)] = bad_len ? fill : -INFINITY;
        } else {
          for (int i = lane; i < G * D; i += 64) store_out<IO>(a.out, row0 * D + i, fill);
          if (a.lse_out && lane < G) a.lse_out[row0 + lane] = bad_len ? fill : -INFINITY;
        }
      } else if (head_ok) {
        if constexpr (MQ) {
          // a row that saw nothing (sequence shorter than q_len) gets 0, -inf
          const bool none = !(l > 0.f);
          const float inv = bad ? __builtin_nanf("") : (none ? 0.f : vmul_cur / l);
          const size_t row = mq_row<MQ>(a, cur.b, cur.g, rr);
#pragma unroll
          for (int t = 0; t < D / 16; ++t)
            store_out4<IO>(a.out, row * D + 16 * t + 4 * jj, acc[t] * inv);
          if (jj == 0 && a.lse_out)
            a.lse_out[row] = bad ? __builtin_nanf("") : (none ? -INFINITY : (m + log2_fast(l)) * kLn2);
        } else {
          const float inv = bad ? __builtin_nanf("") : vmul_cur / l;
#pragma unroll
          for (int t = 0; t < D / 16; ++t)
            store_out4<IO>(a.out, (row0 + rr) * D + 16 * t + 4 * jj, acc[t] * inv);
          if (jj == 0 && a.lse_out)
            a.lse_out[row0 + rr] = bad ? __builtin_nanf("") : (m + log2_fast(l)) * kLn2;
        }
      }
    } else {
      const int slot = cur.pair_first <= y0 ? 0 : 1;
      const int s_first = share_of(cur.pair_first, sh.n, sh.s);
      const int s_last = share_of(cur.pair_end - 1, sh.n, sh.s);
      // (PFX: the workgroup adds the pair's prefix pieces and its slot stride)
      const int parts = s_last - s_first + 1, slot0 = s_first + cur.b * H + cur.g;
      if (lane == 0) {
        int* e = sm.pm + (w * 2 + slot) * kPieceMeta;
        e[kPmB] = cur.b;
        e[kPmG] = cur.g;
        e[kPmEnd] = cur.pair_end;
        e[kPmVmul] = __builtin_bit_cast(int, vmul_cur);
        e[kPmParts] = parts;
        e[kPmK] = sh.wg - s_first;
        e[kPmSlot0] = slot0;
        e[kPmFlags] = kPmUsed | (slot == 1 || w == 0 || cur.pair_first == y0 ? kPmLead : 0);
      }
      if (head_ok) {
        float* row = sm.acc_row(w, slot, rr);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) *reinterpret_cast<f32x4*>(row + 16 * t + 4 * jj) = acc[t];
        if (jj == 0) {
          sm.m[sm.mi(w, slot, rr)] = m;
          sm.l[sm.mi(w, slot, rr)] = l;
        }
      }
      if (lane == 0) sm.bad[w * 2 + slot] = bad ? 1 : 0;
    }
    m = -INFINITY;
    lsum = 0.f;
    bad = false;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (has_nxt) {
      cur = nxt;
      q_cur = q_nxt;
      kmul_cur = kmul_nxt;
      vmul_cur = vmul_nxt;
      if constexpr (MQ) lim_cur = cur.L - a.q_len + t_rr;
      has_nxt = cur.pair_end < y1;
      if (has_nxt) {
        qcursor_at(nxt, a, sm, cur.pair_end, y1, P);
        T::load_q(q_nxt, q_row(nxt), jj);
        if constexpr (kFp8) {
          kmul_nxt = a.scale * kLog2e * a.k_scale[nxt.g];
          vmul_nxt = a.v_scale[nxt.g];
        }
      }
    }
  };

  auto compute = [&](int kslot, int vslot) {
    const int mk = meta_k[kslot];
    const int nvalid = mk & kMetaValid;
    if constexpr (PFX)
      if (nvalid == 0 && (mk & kMetaBad)) bad = true;   // placeholder of an out-of-contract length
    if (nvalid != 0) {
      if (mk & kMetaBad) bad = true;
      bool masked = nvalid != kBlock;
      int pos = 0;
      if constexpr (MQ) {
        // the last two pages of a sequence can hold positions a row may not see
        masked = masked || (mk & kMetaNear) != 0;
        pos = (line_pages(cur.L, mbs) - 1 - ((mk >> kMetaPfeShift) & 1)) * kBlock;
      }
      if (!masked)
        page_math(kslot, vslot, nvalid, pos, std::integral_constant<bool, false>{});
      else
        page_math(kslot, vslot, nvalid, pos, std::integral_constant<bool, true>{});
    }
    if (mk & kMetaEnd) flush();
  };

  // The ring, as in the fixed schedule: a steady-state block of kU positions
  // that issues unconditionally, then a peeled remainder.
  constexpr int kU = kKS * kVS / gcd_c(kKS, kVS);
  // Two copies of the loop, as in the fixed schedule: without a chunk fetch
  // inside it (quarters of at most 64 positions) the ring's wait counts stay
  // exact.
  auto run_ring = [&](auto refresh_tag) {
#pragma unroll
    for (int j = 0; j < dK; ++j)
      if (j < n) issue_k(j, j, refresh_tag);
#pragma unroll
    for (int j = 0; j < dV; ++j)
      if (j < n) issue_v(j, j);
    int i0 = 0;
    for (; i0 + kU - 1 + kAhead < n; i0 += kU) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        issue_k((u + dK) % kKS, i0 + u + dK, refresh_tag);
        issue_v((u + dV) % kVS, (u + dV) % kKS);
        compute(u % kKS, u % kVS);
      }
    }
#pragma unroll
    for (int u = 0; u < kU + kAhead; ++u) {
      const int i = i0 + u;
      if (i < n) {
        if (i + dK < n) issue_k((u + dK) % kKS, i + dK, refresh_tag);
        if (i + dV < n) issue_v((u + dV) % kVS, (u + dV) % kKS);
        compute(u % kKS, u % kVS);
      }
    }
  };
  if (n > 64)
    run_ring(std::integral_constant<bool, true>{});
  else
    run_ring(std::integral_constant<bool, false>{});
}

// Per candidate slot c = 2 * wave + slot, what the combine needs of the piece
// it leads, one value per lane c < 2 * kWaves (taken with readlane).
struct SlotFacts {
  int b, g;     // the pair
  int vmul;     // output multiplier (v_scale), float bits
  int parts;    // pieces of the pair over the shares (1: the pair is whole here)
  int slot;     // workspace slot of this piece
  int hold;     // waves holding the piece: bit wave c >> 1, and bit w of every
                // later wave whose quarter the pair reaches (its slot 0)
};

// Combine, for every piece of the share that leads in LDS (candidate slots c
// in the bit mask lead), the slots of the waves holding it, and write the
// pair's output (a pair whose pieces are all in this share) or the piece's
// partial result to its workspace slot. Uniform across the workgroup, a pass
// at a time; a thread has two item slots: with G x D/4 (row, 4-float quad)
// items of a piece at most the thread count (G <= 8 at head_dim 128) a pass
// takes two pieces, one item of each per thread, else one piece, two items
// per thread (G <= 16). Every LDS read of both slots is issued before any
// arithmetic, so a pass costs one LDS round trip.
template <typename IO, typename KV, int D, bool MQ, bool PFX>
__device__ __forceinline__ void combine_pieces(const Params& a, const BalSm<D>& sm, uint32_t lead,
                                               const SlotFacts& f) {
  constexpr bool kMayBeEmpty = MQ || PFX;   // a row may see nothing in the piece
  constexpr int kQuads = D / 4;
  static_assert(kMaxGroup * kQuads <= 2 * kThreads, "two items per thread cover a piece");
  const int tid = threadIdx.x;
  const int G = a.group;
  const int items = G * kQuads;
  const bool two_pieces = items <= kThreads;   // uniform
  for (uint32_t mk = lead; mk;) {
    // the pass's pieces (candidate slots, uniform): cs[1] == cs[0] when the
    // pass takes one
    int cs[2];
    cs[0] = __builtin_ctz(mk);
    mk &= mk - 1;
    cs[1] = cs[0];
    bool second = false;
    if (two_pieces && mk) {
      cs[1] = __builtin_ctz(mk);
      mk &= mk - 1;
      second = true;
    }
    bool on[2];
    int h[2], d[2], bd[2][kWaves];
    float mv[2][kWaves], lv[2][kWaves];
    f32x4 av[2][kWaves];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int wa = cs[u] >> 1, sa = cs[u] & 1;
      const int i = two_pieces ? tid : tid + u * kThreads;
      on[u] = i < items && (u == 0 || !two_pieces || second);
      h[u] = on[u] ? i / kQuads : 0;
      d[u] = on[u] ? 4 * (i - h[u] * kQuads) : 0;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const int sl = ww == wa ? sa : 0;
        bd[u][ww] = sm.bad[ww * 2 + sl];
        mv[u][ww] = sm.m[sm.mi(ww, sl, h[u])];
        lv[u][ww] = sm.l[sm.mi(ww, sl, h[u])];
        av[u][ww] = *reinterpret_cast<const f32x4*>(sm.acc_row(ww, sl, h[u]) + d[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!on[u]) continue;
      const int c = cs[u];
      const int b = __builtin_amdgcn_readlane(f.b, c);
      const int g = __builtin_amdgcn_readlane(f.g, c);
      const float vmul = __builtin_bit_cast(float, __builtin_amdgcn_readlane(f.vmul, c));
      const int nparts = __builtin_amdgcn_readlane(f.parts, c);
      const int wslot = __builtin_amdgcn_readlane(f.slot, c);
      const int hold = __builtin_amdgcn_readlane(f.hold, c);
      int bad = 0;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww)
        if ((hold >> ww) & 1) bad |= bd[u][ww];
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww)
        if ((hold >> ww) & 1) M = fmaxf(M, mv[u][ww]);
      float W = 0.f;
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      const float Ms = (kMayBeEmpty && M == -INFINITY) ? 0.f : M;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        if ((hold >> ww) & 1) {
          const float ex = exp2_fast(mv[u][ww] - Ms);
          W += ex * lv[u][ww];
          o += ex * av[u][ww];
        }
      }
      f32x4 val = o * (__builtin_amdgcn_rcpf(W) * vmul);
      float lse2 = M + log2_fast(W);
      if constexpr (kMayBeEmpty) {
        if (!(W > 0.f)) {
          val = f32x4{0.f, 0.f, 0.f, 0.f};
          lse2 = -INFINITY;
        }
      }
      if (bad) {
        val = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
        lse2 = __builtin_nanf("");
      }
      if (nparts == 1) {
        size_t row;
        if constexpr (MQ) row = mq_row<MQ>(a, b, g, h[u]);
        else row = (size_t)b * a.num_q_heads + g * G + h[u];
        store_out4<IO>(a.out, row * D + d[u], val);
        if (d[u] == 0 && a.lse_out) a.lse_out[row] = lse2 * kLn2;
      } else {
        const brsrc wr_slot = buffer_rsrc(a.ws_o + (size_t)wslot * G * D, (uint32_t)(G * D * sizeof(float)));
        st_agent4(wr_slot, (uint32_t)((h[u] * D + d[u]) * sizeof(float)), val);
        if (d[u] == 0) st_agent(a.ws_lse + (size_t)wslot * G + h[u], lse2);
      }
    }
  }
}

// One wave's pages q0 .. q1 - 1 of a prefix unit (KV head g), for the query
// rows of its tile: lane row rr sees the first vis pages (vis_min / vis_max:
// the least and the most over the wave's rows). Block ids are read from row
// r_star; each lane also reads its own row's id of every page it sees
// (brow's) and marks the row bad when the two differ or the id is outside
// the pool. Then the tail pages `tails` (bit l: the tile's sequence l, whose
// block id and token count lane l holds in tblk / ttok) for that sequence's
// rows alone (lane row of sequence mrow). The state (m, lsum, acc) is this
// wave's online softmax over the pages it read. KEEP: ordinary loads (other
// tiles read the same pages).
template <typename IO, typename KV, int D, bool KEEP>
__device__ __forceinline__ void prefix_stream(const Params& a, int g, int r_star, int q0, int q1,
                                              const typename TileOf<IO, KV, D>::type::Q& q, float kmul,
                                              int vis, int vis_min, int vis_max, int brow, uint64_t tails,
                                              int tblk, int ttok, int mrow, float& m, float& lsum,
                                              f32x4 (&acc)[D / 16], bool& bad) {
  using T = typename TileOf<IO, KV, D>::type;
  constexpr size_t kPageBytes = (size_t)kBlock * D * ElemSize<KV>::v;
  const int lane = threadIdx.x & 63;
  const int jj = lane >> 4;
  const int H = a.num_kv_heads, mbs = a.max_blocks_per_seq;
  const int n = q1 - q0;
  const int32_t* const ref = a.block_table + (size_t)r_star * mbs;
  const int32_t* const own = a.block_table + (size_t)brow * mbs;
  auto fetch = [&](int c0) {
    const int pp = q0 + c0 + lane;
    return pp < q1 ? ref[pp] : 0;
  };
  int bt_cur = fetch(0), bt_nxt = n > 64 ? fetch(64) : 0;

  const gptr kbase = uniform_ptr(a.k);
  const gptr vbase = uniform_ptr(a.v);
  const uint32_t ko = T::koff(lane), vo = T::voff(lane);
  constexpr int kKS = T::kKStages, kVS = T::kVStages;
  constexpr int dK = kKS - 1, dV = kVS - 1;
  static_assert(kKS >= 1 && kVS >= 1 && dV <= dK, "ring depths");
  constexpr int kAhead = dK > 1 ? dK : 1;
  typename T::KRegs ring_k[kKS];
  typename T::VRegs ring_v[kVS];
  size_t poff[kKS];
  int rid[kKS], oid[kKS];

  auto issue_k = [&](int slot, int i, auto refresh_tag) {
    if constexpr (decltype(refresh_tag)::value) {
      if (i > 0 && (i & 63) == 0) {
        bt_cur = bt_nxt;
        if (n > i + 64) bt_nxt = fetch(i + 64);
      }
    }
    const int raw = __builtin_amdgcn_readlane(bt_cur, i & 63);
    const int phys = (unsigned)raw < (unsigned)a.num_blocks ? raw : 0;
    poff[slot] = ((size_t)phys * H + g) * kPageBytes;
    T::template load_k<KEEP>(ring_k[slot], kbase + poff[slot], ko);
    rid[slot] = raw;
    oid[slot] = own[q0 + i];
  };
  auto issue_v = [&](int vslot, int kslot) { T::template load_v<KEEP>(ring_v[vslot], vbase + poff[kslot], vo); };

  auto page_math = [&](int kslot, int vslot, bool sees, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const f32x4 s = T::scores(ring_k[kslot], q);
    float sc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) sc[e] = (!kMasked || sees) ? s[e] * kmul : -INFINITY;
    const float mx = wave_max_rows(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    const float mnew = fmaxf(m, mx);
    const float msafe = (kMasked && mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = exp2_fast(m - msafe);
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = exp2_fast(sc[e] - msafe);
    const typename T::P pk = T::pack(pr);
    lsum = lsum * alpha + T::psum(pk);
    m = mnew;
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int t = 0; t < D / 16; ++t) acc[t] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < D / 16; ++t) acc[t] = T::pv(T::pvt(ring_v[vslot], t), pk, acc[t]);
  };
  auto compute = [&](int kslot, int vslot, int i) {
    const int pg_i = q0 + i;
    const bool sees = pg_i < vis;
    if (sees && ((unsigned)rid[kslot] >= (unsigned)a.num_blocks || oid[kslot] != rid[kslot])) bad = true;
    if (pg_i < vis_min)
      page_math(kslot, vslot, true, std::integral_constant<bool, false>{});
    else if (pg_i < vis_max)
      page_math(kslot, vslot, sees, std::integral_constant<bool, true>{});
  };

  auto run_ring = [&](auto refresh_tag) {
#pragma unroll
    for (int j = 0; j < dK; ++j)
      if (j < n) issue_k(j, j, refresh_tag);
#pragma unroll
    for (int j = 0; j < dV; ++j)
      if (j < n) issue_v(j, j);
    constexpr int kU = kKS * kVS / gcd_c(kKS, kVS);
    int i0 = 0;
    for (; i0 + kU - 1 + kAhead < n; i0 += kU) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        issue_k((u + dK) % kKS, i0 + u + dK, refresh_tag);
        issue_v((u + dV) % kVS, (u + dV) % kKS);
        compute(u % kKS, u % kVS, i0 + u);
      }
    }
#pragma unroll
    for (int u = 0; u < kU + kAhead; ++u) {
      const int i = i0 + u;
      if (i < n) {
        if (i + dK < n) issue_k((u + dK) % kKS, i + dK, refresh_tag);
        if (i + dV < n) issue_v((u + dV) % kVS, (u + dV) % kKS);
        compute(u % kKS, u % kVS, i);
      }
    }
  };
  if (n > 64)
    run_ring(std::integral_constant<bool, true>{});
  else
    run_ring(std::integral_constant<bool, false>{});

  // tail pages, one at a time (a few per unit): tokens past the sequence's
  // length and every other sequence's rows masked, V past it zeroed
  for (uint64_t mk = tails; mk; mk &= mk - 1) {
    const int ml = __builtin_ctzll(mk);
    const int raw = __builtin_amdgcn_readlane(tblk, ml);
    const int tok = __builtin_amdgcn_readlane(ttok, ml);
    const bool sees = mrow == ml;
    const int phys = (unsigned)raw < (unsigned)a.num_blocks ? raw : 0;
    if (sees && phys != raw) bad = true;
    const size_t off = ((size_t)phys * H + g) * kPageBytes;
    T::load_k(ring_k[0], kbase + off, ko);
    T::load_v(ring_v[0], vbase + off, vo);
    const f32x4 sv = T::scores(ring_k[0], q);
    float sc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) sc[e] = (sees && 4 * jj + e < tok) ? sv[e] * kmul : -INFINITY;
    const float mx = wave_max_rows(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
    const float mnew = fmaxf(m, mx);
    const float msafe = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = exp2_fast(m - msafe);
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = exp2_fast(sc[e] - msafe);
    const typename T::P pk = T::pack(pr);
    lsum = lsum * alpha + T::psum(pk);
    m = mnew;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      acc[t] *= alpha;
      acc[t] = T::pv(T::zero_tail(T::pvt(ring_v[0], t), jj, tok), pk, acc[t]);
    }
  }
}

// Own pieces and first slot of pair (b, g) under the shared prefix: the
// shares its suffix spans on the suffix line (n_s positions, s_n shares).
template <int D>
__device__ __forceinline__ PfxSlots pfx_pair_slots(const Params& a, const BalSm<D>& sm, const PfxGeo& pg,
                                                   int b, int g, int n_s, int s_n) {
  const int H = a.num_kv_heads;
  const int cb = pfx_positions(pg.P, sm.len[b], a.max_blocks_per_seq);
  return pfx_slots(H * sm.pre[b] + g * cb, cb, b * H + g, n_s, s_n);
}

// Prefix share k: its pieces of the prefix line in order. Per piece (unit u
// = (g, pass), pages p_lo .. p_hi - 1): the pass's nt tiles run side by side,
// wc = 4 / nt waves per tile (one wave idle when nt = 3) splitting the pages;
// the tile's waves merge through LDS into one partial result per (sequence,
// head) row, stored to the sequence's prefix slot; then one lane per sequence
// of the pass counts the piece on its pair's counter, and the pairs this
// piece completes are merged here. Control flow around the barriers depends
// only on uniform values.
template <typename IO, typename KV, int D>
__device__ __forceinline__ void prefix_share(const Params& a, const BalSm<D>& sm, const PfxGeo& pg, int k,
                                             int n_s, int s_n) {
  using T = typename TileOf<IO, KV, D>::type;
  constexpr bool kFp8 = std::is_same<KV, FP8>::value;
  constexpr int kQuads = D / 4;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rr = lane & 15, jj = lane >> 4;
  const int G = a.group, H = a.num_kv_heads, B = a.batch, mbs = a.max_blocks_per_seq;
  const int P = pg.P, mpt = pg.mpt;
  const int x1 = share_start(k + 1, pg.np, pg.sp);
  int x = share_start(k, pg.np, pg.sp);
  const brsrc wo = buffer_rsrc(a.ws_o, 0xfffffff0u);
  while (x < x1) {
    const int u = x / P;
    const int p_lo = x - u * P;
    const int p_hi = min(P, x1 - u * P);
    const int g = u / pg.passes, pass = u - g * pg.passes;
    const int nt = min(4, pg.ntile - 4 * pass);
    const int wc = nt == 1 ? 4 : (nt == 2 ? 2 : 1);
    const int tile = w / wc, wi = w - tile * wc;
    const bool active = tile < nt;
    const int span = p_hi - p_lo;
    const int q0 = p_lo + span * wi / wc, q1 = p_lo + span * (wi + 1) / wc;
    const int b_tile = (4 * pass + (active ? tile : 0)) * mpt;   // first sequence of the tile
    const int mrow = rr / G, h = rr - mrow * G;
    const int bq = b_tile + mrow;
    const bool row_ok = active && mrow < mpt && bq < B;
    int vis = P;   // rows that hold no sequence see everything (never stored)
    bool bad = false;
    if (row_ok) {
      const int L = sm.full[bq];
      const bool in = L >= 0 && L <= mbs * kBlock;
      vis = in ? min(P, L / kBlock) : 0;
      bad = !in;   // an out-of-contract length: NaN rows (it has no line positions)
    }
    float kmul = a.scale * kLog2e, vmul = 1.0f;
    if constexpr (kFp8) {
      kmul *= a.k_scale[g];
      vmul = a.v_scale[g];
    }

    // the unit's last piece also reads the tails of its sequences (suffixes
    // of one page at most), the j-th tail of a tile by its wave j % wc
    const int kk = k - share_of(u * P, pg.np, pg.sp);   // this piece among the unit's
    const int pp = pfx_pieces(pg, u);
    uint64_t tails = 0;
    int tblk = 0, ttok = 0;
    if (active && kk == pp - 1) {
      const int bm = b_tile + lane;
      bool has = false;
      if (lane < mpt && bm < B) {
        const int Sb = sm.len[bm];
        if (pfx_tail(P, Sb)) {
          has = true;
          ttok = Sb;
          tblk = a.block_table[(size_t)bm * mbs + (sm.full[bm] - Sb) / kBlock];
        }
      }
      const uint64_t hm = __ballot(has);
      const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(hm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)hm, 0u));
      tails = __ballot(has && rank % wc == wi);
    }

    float m = -INFINITY, lsum = 0.f;
    f32x4 acc[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (active && (q1 > q0 || tails != 0)) {
      int vmin = vis, vmax = row_ok ? vis : 0;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        vmin = min(vmin, __shfl_xor(vmin, d));
        vmax = max(vmax, __shfl_xor(vmax, d));
      }
      vmin = __builtin_amdgcn_readfirstlane(vmin);
      vmax = __builtin_amdgcn_readfirstlane(vmax);
      const size_t qrow = (size_t)(row_ok ? bq : b_tile) * a.num_q_heads + (size_t)g * G + (row_ok ? h : 0);
      typename T::Q q;
      T::load_q(q, (gptr)(a.q + qrow * D * ElemSize<IO>::v), jj);
      const int brow = row_ok ? bq : pg.r_star;
      const int mr = row_ok ? mrow : -1;
      if (nt > 1)
        prefix_stream<IO, KV, D, true>(a, g, pg.r_star, q0, q1, q, kmul, vis, vmin, vmax, brow, tails, tblk,
                                       ttok, mr, m, lsum, acc, bad);
      else
        prefix_stream<IO, KV, D, false>(a, g, pg.r_star, q0, q1, q, kmul, vis, vmin, vmax, brow, tails, tblk,
                                        ttok, mr, m, lsum, acc, bad);
    }
    // the wave's state into LDS: [w][16][D + 4], m / l / bad [w][16]
    const float l = wave_sum_rows(lsum);
    {
      float* row = sm.acc + (w * 16 + rr) * (D + 4);
#pragma unroll
      for (int t = 0; t < D / 16; ++t) *reinterpret_cast<f32x4*>(row + 16 * t + 4 * jj) = acc[t];
      if (jj == 0) {
        sm.m[w * 16 + rr] = m;
        sm.l[w * 16 + rr] = l;
        sm.pfx[kPfxBad + w * 16 + rr] = bad ? 1 : 0;
      }
    }
    lds_barrier();

    // one partial per (tile, row, quad) item, to the row's sequence's slot
    const int rows_t = mpt * G;
    const int items = nt * rows_t * kQuads;
    for (int i = tid; i < items; i += kThreads) {
      const int t = i / (rows_t * kQuads);
      const int r1 = i - t * rows_t * kQuads;
      const int r = r1 / kQuads, dq = r1 - r * kQuads;
      const int b = (4 * pass + t) * mpt + r / G, hh = r % G;
      if (b >= B) continue;
      float M = -INFINITY;
      int bd = 0;
      for (int v = 0; v < wc; ++v) {
        const int ww = t * wc + v;
        M = fmaxf(M, sm.m[ww * 16 + r]);
        bd |= sm.pfx[kPfxBad + ww * 16 + r];
      }
      const float Ms = M == -INFINITY ? 0.f : M;
      float W = 0.f;
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      for (int v = 0; v < wc; ++v) {
        const int ww = t * wc + v;
        const float e = exp2_fast(sm.m[ww * 16 + r] - Ms);
        W += e * sm.l[ww * 16 + r];
        o += e * *reinterpret_cast<const f32x4*>(sm.acc + (ww * 16 + r) * (D + 4) + 4 * dq);
      }
      f32x4 val = {0.f, 0.f, 0.f, 0.f};
      float lse2 = -INFINITY;
      if (bd) {
        val = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
        lse2 = __builtin_nanf("");
      } else if (W > 0.f) {
        val = o * (__builtin_amdgcn_rcpf(W) * vmul);
        lse2 = M + log2_fast(W);
      }
      const PfxSlots ps = pfx_pair_slots(a, sm, pg, b, g, n_s, s_n);
      const size_t slot = (size_t)ps.slot0 + ps.own + kk;
      st_agent4(wo, (uint32_t)(((slot * G + hh) * D + 4 * dq) * sizeof(float)), val);
      if (dq == 0) st_agent(a.ws_lse + slot * G + hh, lse2);
    }
    // the partials are complete; count this piece for every sequence of the pass
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int b_pass = 4 * pass * mpt;
    const int nseq = min(4 * mpt, B - b_pass);
    if (w == 0) {
      int outcome = kCountMore;
      bool first = false;   // the pair's first piece: its own piece 0, else this unit's piece 0
      if (lane < nseq) {
        const int b = b_pass + lane;
        const PfxSlots ps = pfx_pair_slots(a, sm, pg, b, g, n_s, s_n);
        outcome = count_piece(a.ws_cnt + (size_t)b * H + g, ps.own + pp);
        first = ps.own == 0 && kk == 0;
      }
      const uint64_t dm = __ballot(outcome == kCountLast);
      const uint64_t st = __ballot(outcome == kCountStale && first);
      if (lane == 0) {
        sm.pfx[kPfxDone] = (int)(uint32_t)dm;
        sm.pfx[kPfxDone + 1] = (int)(uint32_t)(dm >> 32);
        sm.pfx[kPfxKey] = (int)(uint32_t)st;
        sm.pfx[kPfxKey + 1] = (int)(uint32_t)(st >> 32);
      }
    }
    lds_barrier();
    // a stale counter: the pair's first piece makes its rows NaN
    const uint64_t stale = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(sm.pfx[kPfxKey + 1]) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane(sm.pfx[kPfxKey]);
    for (uint64_t mk = stale; mk; mk &= mk - 1)
      fill_rows<IO, D, false>(a, b_pass + __builtin_ctzll(mk), g, __builtin_nanf(""));
    const uint64_t done = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(sm.pfx[kPfxDone + 1]) << 32) |
                          (uint32_t)__builtin_amdgcn_readfirstlane(sm.pfx[kPfxDone]);
    if (done) {   // uniform
      const int nm = __builtin_popcountll(done);
      int npm = 0;
      for (uint64_t mk = done; mk; mk &= mk - 1) {
        const PfxSlots ps = pfx_pair_slots(a, sm, pg, b_pass + __builtin_ctzll(mk), g, n_s, s_n);
        npm = max(npm, ps.own + pp);
      }
      merge_jobs<IO, D, merge_batch<KV>()>(a, sm.red, nm, npm, [&](int j) {
        uint64_t mk = done;   // the j-th completed sequence
        for (int i = 0; i < j && i < nm - 1; ++i) mk &= mk - 1;
        const int b = b_pass + __builtin_ctzll(mk);
        const PfxSlots ps = pfx_pair_slots(a, sm, pg, b, g, n_s, s_n);
        return MergeJob{b, g, ps.own + pp, (size_t)ps.slot0, -1};
      });
    }
    __syncthreads();   // LDS state and flags are reused by the next piece
    x = u * P + p_hi;
  }
}

template <typename IO, typename KV, int D, bool MQ, bool PFX>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
pa_decode_balanced_kernel(const Params a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int B = a.batch, H = a.num_kv_heads, mbs = a.max_blocks_per_seq;
  const BalSm<D> sm(a.group, B, PFX);
  // this wave's piece slots start unused (their use is recorded when flushed)
  if (lane == 0) {
    sm.pm[(w * 2) * kPieceMeta + kPmFlags] = 0;
    sm.pm[(w * 2 + 1) * kPieceMeta + kPmFlags] = 0;
  }

  // lengths of this thread's sequences [bbeg, bbeg + per) into LDS, and the
  // exclusive prefix sums of their line positions
  const int per = (B + kThreads - 1) / kThreads;
  const int bbeg = tid * per;
  int mine = 0;
  PfxGeo pg{0, 1, 0, 0, 0, 0, 0};
  if constexpr (PFX) {
    // whole lengths, and the longest in-contract sequence (the lowest index
    // among equals): key = L * 2^32 + (2^32 - 1 - b)
    uint64_t key = 0;
    for (int i = 0; i < per; ++i) {
      const int bb = bbeg + i;
      if (bb < B) {
        const int L = a.context_lens[bb];
        sm.full[bb] = L;
        if (L >= 0 && L <= mbs * kBlock) {
          const uint64_t kb = ((uint64_t)(uint32_t)L << 32) | (uint32_t)(0xffffffffu - (uint32_t)bb);
          key = kb > key ? kb : key;
        }
      }
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)key, d);
      const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(key >> 32), d);
      const uint64_t o = ((uint64_t)hi << 32) | lo;
      key = o > key ? o : key;
    }
    if (lane == 0) {
      sm.pfx[kPfxKey + 2 * w] = (int)(uint32_t)key;
      sm.pfx[kPfxKey + 2 * w + 1] = (int)(uint32_t)(key >> 32);
    }
    __syncthreads();
    uint64_t best = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const uint64_t o = ((uint64_t)(uint32_t)sm.pfx[kPfxKey + 2 * ww + 1] << 32) | (uint32_t)sm.pfx[kPfxKey + 2 * ww];
      best = o > best ? o : best;
    }
    const int lmax = (int)(best >> 32);
    pg.P = best ? min(a.prefix_pages, lmax / kBlock) : 0;
    pg.r_star = best ? (int)(0xffffffffu - (uint32_t)best) : 0;
    // suffixes: -1 for an out-of-contract length
    for (int i = 0; i < per; ++i) {
      const int bb = bbeg + i;
      if (bb < B) {
        const int S = pfx_suffix(pg.P, sm.full[bb], mbs);
        sm.len[bb] = S;
        mine += pfx_positions(pg.P, S, mbs);
      }
    }
  } else {
    for (int i = 0; i < per; ++i) {
      const int bb = bbeg + i;
      if (bb < B) {
        const int L = a.context_lens[bb];
        sm.len[bb] = L;
        mine += line_pages(L, mbs);
      }
    }
  }
  int incl = mine;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == 63) sm.misc[w] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int ww = 0; ww < kWaves; ++ww)
    if (ww < w) before += sm.misc[ww];
  int pre = before + incl - mine;
  for (int i = 0; i < per; ++i) {
    const int bb = bbeg + i;
    if (bb < B) {
      sm.pre[bb] = pre;
      pre += pfx_positions(PFX ? pg.P : 0, sm.len[bb], mbs);
    }
  }
  if (tid == kThreads - 1) sm.pre[B] = before + incl;
  __syncthreads();

  const int total = __builtin_amdgcn_readfirstlane(sm.pre[B]);
  const int N = total * H;
  int S, wg;
  if constexpr (PFX) {
    // the prefix line, and the shares split between it and the suffix line
    pg.P = __builtin_amdgcn_readfirstlane(pg.P);
    pg.r_star = __builtin_amdgcn_readfirstlane(pg.r_star);
    const int sn = pfx_split(pg, B, H, a.group, N, (int)gridDim.x);
    const int sp = pg.sp;
    const int wall = share_of_block((int)blockIdx.x, (int)gridDim.x, sp + sn);
    if (wall >= sp + sn) return;   // uniform
    if (wall < sp) {
      prefix_share<IO, KV, D>(a, sm, pg, wall, N, sn);
      return;
    }
    S = sn;
    wg = wall - sp;
  } else {
    S = share_count(N, (int)gridDim.x);
    // shares numbered XCD by XCD (pa_schedule.h); a workgroup left without one
    // returns
    wg = share_of_block((int)blockIdx.x, (int)gridDim.x, S);
    if (wg >= S) return;   // uniform
  }
  const int x0 = share_start(wg, N, S);
  const int x1 = share_start(wg + 1, N, S);

  // this wave's quarter of the share
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto yq = [&](int ww) { return x0 + share_start(ww, x1 - x0, kWaves); };
  decode_quarter<IO, KV, D, MQ, PFX>(a, sm, ShareOf{wg, N, S}, yq(wu), yq(wu + 1), pg.P);
  __syncthreads();

  // Pieces of the share whose state went through LDS, in three steps:
  // 1. combine each one's wave slots (all pieces in one pass); write the
  //    output of whole pairs and the partial result of split ones;
  // 2. once those stores are complete, count every split piece in on its
  //    pair's counter (one lane per candidate slot, all at once);
  // 3. merge the pairs whose count this workgroup completed, all in one pass.
  int yqv[kWaves + 1];
#pragma unroll
  for (int ww = 0; ww <= kWaves; ++ww) yqv[ww] = yq(ww);
  // candidate slots c = 2 * wave + slot: lane c of every wave reads slot c's
  // record once; later steps take its fields with readlane
  const int cl = lane < 2 * kWaves ? lane : 0;
  const int* rec = sm.pm + cl * kPieceMeta;
  const int fl = rec[kPmFlags];
  int parts = rec[kPmParts];
  const int rb = rec[kPmB], rg = rec[kPmG];
  int rs0 = rec[kPmSlot0];
  if constexpr (PFX) {
    // the pair's prefix pieces follow its own, in slots of stride 1 + kPfxPieces
    parts += pfx_pieces(pg, pfx_unit(pg, rb, rg));
    rs0 += (rb * H + rg) * kPfxPieces;
  }
  const uint32_t lead = (uint32_t)__ballot(lane < 2 * kWaves && (fl & kPmLead)) & 0xffu;
  const uint32_t split = (uint32_t)__ballot(lane < 2 * kWaves && (fl & kPmLead) && parts > 1) & 0xffu;
  if (!PFX && lead == 0) return;   // uniform
  SlotFacts facts;
  facts.b = rb;
  facts.g = rg;
  facts.vmul = rec[kPmVmul];
  facts.parts = parts;
  facts.slot = rs0 + rec[kPmK];
  {
    // the waves holding the piece slot cl leads: its own, and every later
    // one whose quarter starts before the pair's end (it holds the pair in
    // its slot 0)
    const int wa = cl >> 1, pend = rec[kPmEnd];
    int hold = 1 << wa;
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww)
      if (ww > wa && pend > yqv[ww]) hold |= 1 << ww;
    facts.hold = hold;
  }
  // steps 2 and 3 for the split pieces
  auto settle_split = [&]() {
    if (wu == 0) {
      int outcome = kCountMore;
      if (lane < 2 * kWaves && ((split >> lane) & 1u))
        outcome = count_piece(a.ws_cnt + (size_t)rb * H + rg, parts);
      const uint32_t dm = (uint32_t)__ballot(outcome == kCountLast) & 0xffu;
      // a stale counter: the pair's first piece makes its rows NaN
      const uint32_t sm_ = (uint32_t)__ballot(outcome == kCountStale && rec[kPmK] == 0) & 0xffu;
      if (lane == 0) {
        sm.split[0] = (int)dm;
        sm.split[1] = (int)sm_;
      }
    }
    lds_barrier();
    const uint32_t stale = (uint32_t)__builtin_amdgcn_readfirstlane(sm.split[1]);
    for (uint32_t mk = stale; mk; mk &= mk - 1) {
      const int c = __builtin_ctz(mk);
      fill_rows<IO, D, MQ>(a, __builtin_amdgcn_readlane(rb, c), __builtin_amdgcn_readlane(rg, c),
                           __builtin_nanf(""));
    }
    // the pairs this workgroup completes, all merged in one pass
    const uint32_t done = (uint32_t)__builtin_amdgcn_readfirstlane(sm.split[0]);
    if (done == 0) return;   // uniform
    int npm = 0;
    for (uint32_t mk = done; mk; mk &= mk - 1)
      npm = max(npm, __builtin_amdgcn_readlane(parts, __builtin_ctz(mk)));
    const int m = __builtin_popcount(done);
    merge_jobs<IO, D, merge_batch<KV>()>(a, sm.red, m, npm, [&](int j) {
      uint32_t mk = done;   // the j-th completed pair
      for (int i = 0; i < j && i < m - 1; ++i) mk &= mk - 1;
      const int c = __builtin_ctz(mk);
      return MergeJob{__builtin_amdgcn_readlane(rb, c), __builtin_amdgcn_readlane(rg, c),
                      __builtin_amdgcn_readlane(parts, c), (size_t)__builtin_amdgcn_readlane(rs0, c), -1};
    });
  };
  if constexpr (!PFX) {
    combine_pieces<IO, KV, D, MQ, PFX>(a, sm, lead, facts);
    if (split == 0) return;   // uniform
    __builtin_amdgcn_s_waitcnt(0);   // this wave's partial stores are complete
    __syncthreads();
    settle_split();
  } else {
    if (lead) combine_pieces<IO, KV, D, MQ, PFX>(a, sm, lead, facts);
    __builtin_amdgcn_s_waitcnt(0);   // every partial store of this wave is complete
    __syncthreads();
    // Count every piece this workgroup holds at once, one lane each: the
    // split pieces (lanes 0 .. 7, candidate slots) and the pairs whose
    // suffix lies wholly inside a quarter (they stored their partial during
    // the stream as piece 0 of one; per quarter a contiguous range of pair
    // indices), 64 lanes a round; then merge every pair a round completed
    // in one pass.
    int qlo[kWaves], qn[kWaves];
    int ndirect = 0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const int y0 = yqv[ww], y1 = yqv[ww + 1];
      qlo[ww] = 0;
      qn[ww] = 0;
      if (y0 < y1) {
        auto pair_at = [&](int x, int* first, int* end) {
          const int b = seq_of_uniform(sm.pre, B, H, x);
          const int cb = pfx_positions(pg.P, __builtin_amdgcn_readfirstlane(sm.len[b]), mbs);
          const int sf = H * __builtin_amdgcn_readfirstlane(sm.pre[b]);
          const int g = (x - sf) / cb;
          *first = sf + g * cb;
          *end = *first + cb;
          return b * H + g;
        };
        int f0, e0, f1, e1;
        int lo = pair_at(y0, &f0, &e0);
        if (f0 < y0) ++lo;
        int hi = pair_at(y1 - 1, &f1, &e1) + 1;
        if (e1 > y1) --hi;
        qlo[ww] = lo;
        qn[ww] = max(0, hi - lo);
      }
      ndirect += qn[ww];
    }
    const int nitems = 2 * kWaves + ndirect;
    int* const jpi = sm.pfx + kPfxJob;
    int* const jnp = jpi + 64;
    int* const js0 = jnp + 64;
    for (int c0 = 0; c0 < nitems; c0 += 64) {
      if (c0 > 0) __syncthreads();   // the previous round's list and merge scratch are consumed
      if (wu == 0) {
        const int item = c0 + lane;
        int outcome = kCountMore, pi = 0, np = 0, s0 = 0;
        bool first_piece = true;
        if (item < 2 * kWaves) {
          if ((split >> lane) & 1u) {
            pi = rb * H + rg;
            np = parts;
            s0 = rs0;
            first_piece = rec[kPmK] == 0;
            outcome = count_piece(a.ws_cnt + (size_t)pi, np);
          }
        } else if (item < nitems) {
          int d = item - 2 * kWaves, ww = 0;
          while (d >= qn[ww]) d -= qn[ww++];
          pi = qlo[ww] + d;
          const int b = pi / H, g = pi - b * H;
          // sequences without line positions inside the range are the prefix pass's
          if (pfx_positions(pg.P, sm.len[b], mbs) > 0) {
            const PfxSlots ps = pfx_pair_slots(a, sm, pg, b, g, N, S);
            np = ps.own + pfx_pieces(pg, pfx_unit(pg, b, g));
            s0 = ps.slot0;
            outcome = count_piece(a.ws_cnt + (size_t)pi, np);
          }
        }
        const uint64_t dm = __ballot(outcome == kCountLast);
        // a stale counter: the pair's first piece makes its rows NaN
        const uint64_t st = __ballot(outcome == kCountStale && first_piece);
        jpi[lane] = pi;
        jnp[lane] = np;
        js0[lane] = s0;
        if (lane == 0) {
          sm.pfx[kPfxDone] = (int)(uint32_t)dm;
          sm.pfx[kPfxDone + 1] = (int)(uint32_t)(dm >> 32);
          sm.pfx[kPfxKey] = (int)(uint32_t)st;
          sm.pfx[kPfxKey + 1] = (int)(uint32_t)(st >> 32);
        }
      }
      lds_barrier();
      const uint64_t done = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(sm.pfx[kPfxDone + 1]) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane(sm.pfx[kPfxDone]);
      const uint64_t stale = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(sm.pfx[kPfxKey + 1]) << 32) |
                             (uint32_t)__builtin_amdgcn_readfirstlane(sm.pfx[kPfxKey]);
      for (uint64_t mk = stale; mk; mk &= mk - 1) {
        const int pi = __builtin_amdgcn_readfirstlane(jpi[__builtin_ctzll(mk)]);
        fill_rows<IO, D, MQ>(a, pi / H, pi % H, __builtin_nanf(""));
      }
      if (done) {   // uniform
        const int nm = __builtin_popcountll(done);
        auto job = [&](int j) {
          uint64_t mk = done;   // the j-th completed pair
          for (int i = 0; i < j && i < nm - 1; ++i) mk &= mk - 1;
          const int l = __builtin_ctzll(mk);
          const int pi = __builtin_amdgcn_readfirstlane(jpi[l]);
          return MergeJob{pi / H, pi % H, __builtin_amdgcn_readfirstlane(jnp[l]),
                          (size_t)__builtin_amdgcn_readfirstlane(js0[l]), -1};
        };
        int npm = 0;
        for (int j = 0; j < nm; ++j) npm = max(npm, job(j).np);
        merge_jobs<IO, D, merge_batch<KV>()>(a, sm.red, nm, npm, job);
      }
    }
  }
}

__global__ void fill_zero_kernel(uint8_t* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t n16 = n / 16;
  for (size_t j = i; j < n16; j += (size_t)gridDim.x * blockDim.x)
    reinterpret_cast<u32x4*>(p)[j] = u32x4{0u, 0u, 0u, 0u};
  if (i < n % 16) p[n16 * 16 + i] = 0;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
// Shares of the balanced split per CU. One share (one workgroup of four
// waves with deep register rings) per CU measured as fast as two or three on
// MI355X at streaming and faster overall: every share pays a fixed cost at
// its start (lengths, block ids, first pages) and at its end (combining the
// waves, partial results, the hand-off to the pair's merge), and fewer,
// longer shares cut pairs into fewer pieces.
constexpr int kWgPerCu = 1;

// Shares of the balanced split on the current device, or -1.
int balanced_shares() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (cus <= 0 || cus > 4096) return -1;
  return cus * kWgPerCu;
}

template <typename IO, typename KV, int D, bool MQ>
static hipError_t launch(const Params& prm, dim3 grid, bool balanced, hipStream_t stream) {
  if (balanced)
    hipLaunchKernelGGL((pa_decode_balanced_kernel<IO, KV, D, MQ, false>), grid, dim3(kThreads),
                       bal_layout(prm.group, D, prm.batch).total, stream, prm);
  else
    hipLaunchKernelGGL((pa_decode_kernel<IO, KV, D, MQ>), grid, dim3(kThreads), 0, stream, prm);
  return hipGetLastError();
}

template <typename IO, typename KV, bool MQ>
static hipError_t launch_d(int D, const Params& prm, dim3 grid, bool balanced, hipStream_t stream) {
  return D == 64 ? launch<IO, KV, 64, MQ>(prm, grid, balanced, stream)
                 : launch<IO, KV, 128, MQ>(prm, grid, balanced, stream);
}

template <typename IO, typename KV>
static hipError_t launch_prefix(int D, const Params& prm, dim3 grid, hipStream_t stream) {
  if (D == 64)
    hipLaunchKernelGGL((pa_decode_balanced_kernel<IO, KV, 64, false, true>), grid, dim3(kThreads),
                       bal_layout(prm.group, 64, prm.batch, true).total, stream, prm);
  else
    hipLaunchKernelGGL((pa_decode_balanced_kernel<IO, KV, 128, false, true>), grid, dim3(kThreads),
                       bal_layout(prm.group, 128, prm.batch, true).total, stream, prm);
  return hipGetLastError();
}
static_assert(kPfxPieces == pa_host::kPrefixPieces, "prefix slots per pair");

}  // namespace pa

namespace pa {

size_t decode_workspace_bytes(const pa_shape* shape, int q_len) {
  if (!pa_host::decode_shape_ok(shape) || q_len < 1) return 0;
  if ((long long)(shape->num_q_heads / shape->num_kv_heads) * q_len > kTileRows) return 0;
  int shares = 0;
  if (shape->partition_size == PA_SPLIT_BALANCED) {
    shares = balanced_shares();
    if (shares < 0) return 0;
  }
  return pa_host::decode_layout(shape, shares, q_len).total;
}

// cnt_region: 0 for a caller's workspace (counters packed first), else the
// fixed counter region of the no-allocation scratch (see decode_layout).
// prefix_blocks >= 0: the shared-prefix call (balanced split only).
static pa_status decode_launch(const pa_shape* shape, int q_len, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_table,
                               const int32_t* context_lens, float scale, pa_dtype io_dtype,
                               pa_dtype kv_dtype, const float* k_scale, const float* v_scale,
                               void* workspace, size_t workspace_bytes, size_t cnt_region,
                               void* out, float* lse_out, void* stream, int prefix_blocks = -1) {
  const bool prefix = prefix_blocks >= 0;
  pa_status st = prefix ? pa_host::prefix_shape_status(shape, prefix_blocks)
                        : pa_host::decode_shape_status(shape, q_len);
  if (st != PA_OK) return st;
  st = pa_host::io_args_status(q, k_cache, v_cache, block_table, context_lens, io_dtype, kv_dtype,
                               k_scale, v_scale, out, lse_out);
  if (st != PA_OK) return st;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  const bool balanced = shape->partition_size == PA_SPLIT_BALANCED;
  int shares = 0;
  if (balanced) {
    shares = balanced_shares();
    if (shares < 0) return PA_ERR_HIP;
  }
  if (prefix) {
    st = pa_host::prefix_shares_status(shape, shares);
    if (st != PA_OK) return st;
  }
  const pa_host::DecodeLayout wl = prefix ? pa_host::prefix_layout(shape, shares)
                                          : pa_host::decode_layout(shape, shares, q_len, cnt_region);
  st = pa_host::workspace_status(shape->partition_size, wl.total, wl.cnt_bytes, cnt_region, workspace,
                                 workspace_bytes);
  if (st != PA_OK) return st;
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
  prm.ws_o = split ? reinterpret_cast<float*>(ws + wl.o_off) : nullptr;
  prm.ws_lse = split ? reinterpret_cast<float*>(ws + wl.lse_off) : nullptr;
  prm.ws_cnt = split ? reinterpret_cast<uint32_t*>(ws + wl.cnt_off) : nullptr;
  prm.scale = scale;
  prm.batch = shape->batch;
  prm.num_q_heads = shape->num_q_heads;
  prm.num_kv_heads = shape->num_kv_heads;
  prm.group = G * q_len;   // rows per (sequence, KV head)
  prm.max_blocks_per_seq = shape->max_blocks_per_seq;
  prm.num_blocks = shape->num_blocks;
  prm.part_tokens = shape->partition_size;
  prm.p_max = wl.p_max;
  prm.fan = wl.fan;
  prm.g_max = wl.g_max;
  prm.q_len = q_len;
  prm.gq = G;
  prm.prefix_pages = prefix ? prefix_blocks : 0;

  // 1-D grid: one workgroup per unit, or one per share (see the kernels)
  const dim3 grid(pa_host::decode_grid(shape, wl, shares), 1, 1);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e;
  const int D = shape->head_dim;
  if (prefix) {
    if (io_dtype == PA_F32)
      e = launch_prefix<F32, F32>(D, prm, grid, hs);
    else if (io_dtype == PA_F16)
      e = kv_dtype == PA_FP8_E4M3 ? launch_prefix<F16, FP8>(D, prm, grid, hs)
                                  : launch_prefix<F16, F16>(D, prm, grid, hs);
    else
      e = kv_dtype == PA_FP8_E4M3 ? launch_prefix<BF16, FP8>(D, prm, grid, hs)
                                  : launch_prefix<BF16, BF16>(D, prm, grid, hs);
  } else if (q_len == 1) {
    if (io_dtype == PA_F32)
      e = launch_d<F32, F32, false>(D, prm, grid, balanced, hs);
    else if (io_dtype == PA_F16)
      e = kv_dtype == PA_FP8_E4M3 ? launch_d<F16, FP8, false>(D, prm, grid, balanced, hs)
                                  : launch_d<F16, F16, false>(D, prm, grid, balanced, hs);
    else
      e = kv_dtype == PA_FP8_E4M3 ? launch_d<BF16, FP8, false>(D, prm, grid, balanced, hs)
                                  : launch_d<BF16, BF16, false>(D, prm, grid, balanced, hs);
  } else {
    if (io_dtype == PA_F32)
      e = launch_d<F32, F32, true>(D, prm, grid, balanced, hs);
    else if (io_dtype == PA_F16)
      e = kv_dtype == PA_FP8_E4M3 ? launch_d<F16, FP8, true>(D, prm, grid, balanced, hs)
                                  : launch_d<F16, F16, true>(D, prm, grid, balanced, hs);
    else
      e = kv_dtype == PA_FP8_E4M3 ? launch_d<BF16, FP8, true>(D, prm, grid, balanced, hs)
                                  : launch_d<BF16, BF16, true>(D, prm, grid, balanced, hs);
  }
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status decode_call(const pa_shape* shape, int q_len, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_table,
                      const int32_t* context_lens, float scale, pa_dtype io_dtype,
                      pa_dtype kv_dtype, const float* k_scale, const float* v_scale,
                      void* workspace, size_t workspace_bytes, void* out, float* lse_out,
                      void* stream) {
  return decode_launch(shape, q_len, q, k_cache, v_cache, block_table, context_lens, scale, io_dtype,
                       kv_dtype, k_scale, v_scale, workspace, workspace_bytes, 0, out, lse_out, stream);
}

// ---------------------------------------------------------------------------
// Scratch of the no-allocation entry point: one array per GPU the library
// runs on, held until the process ends. The first kScratchCounterBytes hold
// the (sequence, KV head) and merge-group counters of every call; partial
// results follow at that fixed offset, so no call's partials ever land on
// another call's counters. The array starts zeroed (and is zero-filled once
// more when a device first uses it); every completed call leaves the counters
// it used at zero, so calls need no clearing in between.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr size_t kScratchCounterBytes = (size_t)256 << 10;
static_assert(kScratchBytes == PA_NOALLOC_SCRATCH_BYTES, "scratch size in the header");
static_assert(kScratchCounterBytes == PA_NOALLOC_COUNTER_BYTES, "counter region in the header");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The device address of this GPU's scratch (the array's name in host code is
// only a handle for hipGetSymbolAddress, never an address to pass on). On the
// first call on a device its counter region is zero-filled on `stream`.
static pa_status scratch_of_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PA_ERR_HIP;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(64), dim3(256), 0, stream, static_cast<uint8_t*>(ptr),
                       kScratchCounterBytes);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace pa

extern "C" {

size_t pa_decode_workspace_bytes(const pa_shape* shape) { return pa::decode_workspace_bytes(shape, 1); }

pa_status pa_decode(const pa_shape* shape, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* block_table,
                    const int32_t* context_lens, float scale, pa_dtype io_dtype,
                    pa_dtype kv_dtype, const float* k_scale, const float* v_scale,
                    void* workspace, size_t workspace_bytes, void* out, float* lse_out,
                    void* stream) {
  return pa::decode_call(shape, 1, q, k_cache, v_cache, block_table, context_lens, scale, io_dtype,
                         kv_dtype, k_scale, v_scale, workspace, workspace_bytes, out, lse_out, stream);
}

pa_status pa_decode_noalloc(const pa_shape* shape, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* context_lens, float scale, pa_dtype io_dtype,
                            pa_dtype kv_dtype, const float* k_scale, const float* v_scale,
                            void* out, float* lse_out, void* stream) {
  if (!shape) return PA_ERR_NULL;
  if (shape->partition_size == 0)   // one pass: no scratch at all
    return pa::decode_launch(shape, 1, q, k_cache, v_cache, block_table, context_lens, scale, io_dtype,
                             kv_dtype, k_scale, v_scale, nullptr, 0, 0, out, lse_out, stream);
  // fixed partitions: the size check needs no device, so an oversized call is
  // refused before the scratch is looked up
  if (shape->partition_size > 0 && pa_host::decode_shape_ok(shape)) {
    const pa_host::DecodeLayout wl = pa_host::decode_layout(shape, 0, 1, pa::kScratchCounterBytes);
    if (wl.cnt_bytes > pa::kScratchCounterBytes || wl.total > pa::kScratchBytes) return PA_ERR_SCRATCH;
  }
  void* ws = nullptr;
  const pa_status st = pa::scratch_of_current_device(static_cast<hipStream_t>(stream), &ws);
  if (st != PA_OK) return st;
  return pa::decode_launch(shape, 1, q, k_cache, v_cache, block_table, context_lens, scale, io_dtype,
                           kv_dtype, k_scale, v_scale, ws, pa::kScratchBytes, pa::kScratchCounterBytes,
                           out, lse_out, stream);
}

size_t pa_decode_prefix_workspace_bytes(const pa_shape* shape) {
  if (pa_host::prefix_shape_status(shape, 0) != PA_OK) return 0;
  const int shares = pa::balanced_shares();
  if (shares < 0 || pa_host::prefix_shares_status(shape, shares) != PA_OK) return 0;
  return pa_host::prefix_layout(shape, shares).total;
}

pa_status pa_decode_prefix(const pa_shape* shape, int32_t prefix_blocks, const void* q,
                           const void* k_cache, const void* v_cache, const int32_t* block_table,
                           const int32_t* context_lens, float scale, pa_dtype io_dtype,
                           pa_dtype kv_dtype, const float* k_scale, const float* v_scale,
                           void* workspace, size_t workspace_bytes, void* out, float* lse_out,
                           void* stream) {
  if (!shape) return PA_ERR_NULL;
  if (prefix_blocks < 0) return PA_ERR_SHAPE;
  return pa::decode_launch(shape, 1, q, k_cache, v_cache, block_table, context_lens, scale, io_dtype,
                           kv_dtype, k_scale, v_scale, workspace, workspace_bytes, 0, out, lse_out, stream,
                           prefix_blocks);
}

pa_status pa_workspace_reset(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return workspace_bytes == 0 ? PA_OK : PA_ERR_NULL;
  if ((uintptr_t)workspace & 15u) return PA_ERR_ALIGN;
  if (workspace_bytes == 0) return PA_OK;
  const size_t n16 = workspace_bytes / 16;
  unsigned blocks = (unsigned)((n16 + 255) / 256);
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(pa::fill_zero_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint8_t*>(workspace),
                     workspace_bytes);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

const char* pa_status_str(pa_status status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "unsupported or inconsistent shape";
    case PA_ERR_DTYPE: return "unsupported io/kv dtype combination";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_ALIGN: return "a tensor pointer is not suitably aligned";
    case PA_ERR_HIP: return "the HIP runtime refused the launch";
    case PA_ERR_CAPACITY: return "not enough free blocks in the pool";
    case PA_ERR_STATE: return "unknown or already present sequence id";
    case PA_ERR_SCRATCH: return "the call needs more scratch than the no-allocation entry point holds";
  }
  return "unknown status";
}

}  // extern "C"
