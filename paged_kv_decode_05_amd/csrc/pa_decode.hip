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
//   1. reads the physical block id (block table, kept in a VGPR and read out
//      with readlane),
//   2. loads the K page and the V page straight from HBM into registers in the
//      layout the matrix cores consume (the cache layouts in padecode.h are
//      chosen so that these loads are contiguous 16-byte or 8-byte runs),
//   3. computes S^T[token][head] = K Q^T for the whole GQA group with MFMA
//      (query heads padded to 16 columns),
//   4. masks tokens past the partition end, updates the running max / sum in
//      base 2 (scale * log2 e folded into one multiplier),
//   5. rounds P to the 16-bit operand type and accumulates O^T += V^T P^T with
//      MFMA; the running sum uses the same rounded P.
// The page loads of page i+1 are issued before page i is computed.
// The waves' partial results are merged through LDS. With split-K, the
// partition's normalised output and base-2 log-sum-exp go to the workspace,
// and the last workgroup of each (b, g) to finish (an atomic counter) merges
// all partitions of that sequence in a fixed order and writes the output, then
// resets the counter to zero.
//
// fp8 (OCP E4M3) caches are widened exactly to f16/bf16 with the gfx950
// conversion instructions; k_scale folds into the score multiplier and
// v_scale into the output.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "padecode.h"

namespace pa {

constexpr int kBlock = 16;      // tokens per page
constexpr int kMaxGroup = 16;   // query heads per KV head one MFMA tile covers
constexpr int kWaves = 4;       // wavefronts per workgroup
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Storage tags.
struct F32 {};
struct F16 {};
struct BF16 {};
struct FP8 {};

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
  float* ws_o;       // [B][Hq][p_max][D]
  float* ws_lse;     // [B][Hq][p_max]   base-2, scaled score units
  uint32_t* ws_cnt;  // [B][Hkv]
  float scale;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t part_tokens;  // 0: whole sequence in one unit
  int32_t p_max;
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float wave_max_rows(float x) {
  // lanes l, l^16, l^32, l^48 hold the same query head
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum_rows(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

template <typename T>
__device__ __forceinline__ T load_nt(const T* p) {
  return *p;
}

// ---------------------------------------------------------------------------
// Per-dtype pieces. A "family" fixes the matrix-core operand type.
//
// 16-bit family (q/out f16 or bf16): QK^T uses 16x16x32 MFMA (8 head-dim
// elements per lane per instruction), PV uses 16x16x16 (4 tokens per lane).
// fp32 family: both use 16x16x4 f32 MFMA (1 element per lane).
//
// Lane l of a wave is (r = l % 16, jj = l / 16). In the QK^T product lane l
// feeds token r of the page (A operand) and query head r (B operand); its
// k-slots are the head-dim elements of 16-byte group jj + 4*i of the K page.
// The 16x16 accumulator leaves lane l with rows 4*jj .. 4*jj+3 (tokens) of
// column r (query head), which is exactly the B operand of the PV product
// (k = token 4*jj + i, n = head r); its A operand is V^T[16*t + r][4*jj + i].
// The result O^T[16*t + 4*jj + i][head r] thus stays with the lane that owns
// head r's softmax state.
// ---------------------------------------------------------------------------

template <typename IO>
struct Op16;
template <>
struct Op16<F16> {
  typedef f16x8 A8;
  typedef f16x4 A4;
  typedef _Float16 E;
  static __device__ __forceinline__ f32x4 qk(A8 a, A8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(A4 a, A4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  // 4 fp8 codes (one dword) -> 4 exact f16 values
  static __device__ __forceinline__ A4 fp8x4(uint32_t w) {
    f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
    A4 r = {lo[0], lo[1], hi[0], hi[1]};
    return r;
  }
  static __device__ __forceinline__ float out_f(E x) { return (float)x; }
};
template <>
struct Op16<BF16> {
  typedef bf16x8 A8;
  typedef bf16x4 A4;
  typedef __bf16 E;
  static __device__ __forceinline__ f32x4 qk(A8 a, A8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(A4 a, A4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ A4 fp8x4(uint32_t w) {
    bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    A4 r = {lo[0], lo[1], hi[0], hi[1]};
    return r;
  }
  static __device__ __forceinline__ float out_f(E x) { return (float)x; }
};

template <typename T>
__device__ __forceinline__ T bitcast16(u32x4 x) {
  return __builtin_bit_cast(T, x);
}

// Register tile of one page for the 16-bit family.
//   KV16 = true: 16-bit cache. K: D/32 loads of 16 B; V: D/16 loads of 8 B.
//   KV16 = false: fp8 cache.   K: D/64 loads of 16 B; V: D/16 loads of 4 B.
template <int D, bool KV16>
struct PageRegs16 {
  static constexpr int kKLoads = KV16 ? D / 32 : D / 64;
  static constexpr int kVTiles = D / 16;
  u32x4 k[kKLoads];
  typename std::conditional<KV16, u32x2, uint32_t>::type v[kVTiles];
};

template <int D, bool KV16>
__device__ __forceinline__ void load_page16(PageRegs16<D, KV16>& r, const uint8_t* kpage,
                                            const uint8_t* vpage, int lane) {
  const int rr = lane & 15, jj = lane >> 4;
#pragma unroll
  for (int i = 0; i < PageRegs16<D, KV16>::kKLoads; ++i)
    r.k[i] = *reinterpret_cast<const u32x4*>(kpage + i * 1024 + lane * 16);
  // V^T row d = 16*t + rr holds 16 tokens; this lane wants tokens 4*jj..4*jj+3.
  constexpr int esz = KV16 ? 2 : 1;
#pragma unroll
  for (int t = 0; t < PageRegs16<D, KV16>::kVTiles; ++t) {
    const uint8_t* p = vpage + (size_t)(16 * t + rr) * (16 * esz) + jj * 4 * esz;
    if constexpr (KV16)
      r.v[t] = *reinterpret_cast<const u32x2*>(p);
    else
      r.v[t] = *reinterpret_cast<const uint32_t*>(p);
  }
}

// fp32 family page registers. K: D/16 loads of 16 B; V: D/16 loads of 16 B.
template <int D>
struct PageRegs32 {
  static constexpr int kKLoads = D / 16;
  static constexpr int kVTiles = D / 16;
  f32x4 k[kKLoads];
  f32x4 v[kVTiles];
};

template <int D>
__device__ __forceinline__ void load_page32(PageRegs32<D>& r, const uint8_t* kpage,
                                            const uint8_t* vpage, int lane) {
  const int rr = lane & 15, jj = lane >> 4;
#pragma unroll
  for (int i = 0; i < PageRegs32<D>::kKLoads; ++i)
    r.k[i] = *reinterpret_cast<const f32x4*>(kpage + i * 1024 + lane * 16);
#pragma unroll
  for (int t = 0; t < PageRegs32<D>::kVTiles; ++t)
    r.v[t] = *reinterpret_cast<const f32x4*>(vpage + (size_t)(16 * t + rr) * 64 + jj * 16);
}

// ---------------------------------------------------------------------------
// Online-softmax state of one wave: lane (rr, jj) tracks query head rr.
// ---------------------------------------------------------------------------
template <int D>
struct WaveState {
  float m;       // running max of scaled base-2 scores (same on the 4 lanes of a head)
  float l;       // this lane's share of the running sum
  f32x4 acc[D / 16];
};

// Score scaling, masking and the online-softmax update for one page.
// Returns the (unrounded) probabilities of this lane's 4 tokens in p[].
__device__ __forceinline__ void softmax_page(float& m, float& alpha, float p[4], f32x4 s,
                                             float cmul, int nvalid, int jj) {
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x = s[i] * cmul;
    sc[i] = (4 * jj + i < nvalid) ? x : -INFINITY;
  }
  float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  mx = wave_max_rows(mx);
  const float mnew = fmaxf(m, mx);
  alpha = exp2_fast(m - mnew);
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = exp2_fast(sc[i] - mnew);
  m = mnew;
}

template <typename IO, typename KV, int D>
__device__ __forceinline__ void compute_page16(WaveState<D>& st, const PageRegs16<D, std::is_same<KV, IO>::value>& r,
                                               const typename Op16<IO>::A8* qop, float cmul,
                                               int nvalid, int lane) {
  using O = Op16<IO>;
  using A8 = typename O::A8;
  using A4 = typename O::A4;
  constexpr bool kv16 = std::is_same<KV, IO>::value;
  const int jj = lane >> 4;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kv16) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c) s = O::qk(bitcast16<A8>(r.k[c]), qop[c], s);
  } else {
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      A4 a0 = O::fp8x4(r.k[c][0]), a1 = O::fp8x4(r.k[c][1]);
      A4 a2 = O::fp8x4(r.k[c][2]), a3 = O::fp8x4(r.k[c][3]);
      A8 lo = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      A8 hi = {a2[0], a2[1], a2[2], a2[3], a3[0], a3[1], a3[2], a3[3]};
      s = O::qk(lo, qop[2 * c], s);
      s = O::qk(hi, qop[2 * c + 1], s);
    }
  }
  float alpha, p[4];
  softmax_page(st.m, alpha, p, s, cmul, nvalid, jj);
  A4 pk;
#pragma unroll
  for (int i = 0; i < 4; ++i) pk[i] = (typename O::E)p[i];
  const float ps = (O::out_f(pk[0]) + O::out_f(pk[1])) + (O::out_f(pk[2]) + O::out_f(pk[3]));
  st.l = st.l * alpha + ps;
  const bool partial = nvalid < kBlock;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    A4 va;
    if constexpr (kv16) {
      va = __builtin_bit_cast(A4, r.v[t]);
    } else {
      va = O::fp8x4(r.v[t]);
    }
    if (partial) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * jj + i >= nvalid) va[i] = (typename O::E)0.0f;
    }
    st.acc[t] = O::pv(va, pk, st.acc[t] * alpha);
  }
}

template <int D>
__device__ __forceinline__ void compute_page32(WaveState<D>& st, const PageRegs32<D>& r,
                                               const f32x4* qop, float cmul, int nvalid,
                                               int lane) {
  const int jj = lane >> 4;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_16x16x4f32(r.k[c][e], qop[c][e], s, 0, 0, 0);
  }
  float alpha, p[4];
  softmax_page(st.m, alpha, p, s, cmul, nvalid, jj);
  st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
  const bool partial = nvalid < kBlock;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    f32x4 va = r.v[t];
    if (partial) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * jj + i >= nvalid) va[i] = 0.0f;
    }
    f32x4 a = st.acc[t] * alpha;
#pragma unroll
    for (int e = 0; e < 4; ++e) a = __builtin_amdgcn_mfma_f32_16x16x4f32(va[e], p[e], a, 0, 0, 0);
    st.acc[t] = a;
  }
}

// ---------------------------------------------------------------------------
// Output conversion.
// ---------------------------------------------------------------------------
template <typename IO>
__device__ __forceinline__ void store_out(uint8_t* out, size_t idx, float x);
template <>
__device__ __forceinline__ void store_out<F32>(uint8_t* out, size_t idx, float x) {
  reinterpret_cast<float*>(out)[idx] = x;
}
template <>
__device__ __forceinline__ void store_out<F16>(uint8_t* out, size_t idx, float x) {
  reinterpret_cast<_Float16*>(out)[idx] = (_Float16)x;
}
template <>
__device__ __forceinline__ void store_out<BF16>(uint8_t* out, size_t idx, float x) {
  reinterpret_cast<__bf16*>(out)[idx] = (__bf16)x;
}

template <typename IO>
struct IoSize { static constexpr int v = 2; };
template <>
struct IoSize<F32> { static constexpr int v = 4; };
template <typename KV>
struct KvSize { static constexpr int v = 2; };
template <>
struct KvSize<F32> { static constexpr int v = 4; };
template <>
struct KvSize<FP8> { static constexpr int v = 1; };

// ---------------------------------------------------------------------------
// LDS for the cross-wave merge and the cross-partition merge.
// ---------------------------------------------------------------------------
template <int D>
struct Smem {
  float acc[kWaves][kMaxGroup][D];
  float m[kWaves][kMaxGroup];
  float l[kWaves][kMaxGroup];
  int bad;
  int last;
};

// Merge the partitions of (b, g) stored in the workspace and write the final
// output of its `group` query heads. Partitions are combined in a fixed order
// (thread slice s takes p = s, s + S, ...; slices are then folded 0, 1, ...),
// so the result does not depend on which workgroup finished last.
template <typename IO, int D>
__device__ void merge_partitions(const Params& a, Smem<D>& sm, int b, int g, int nparts) {
  constexpr int kQuads = D / 4;
  constexpr int kSlices = kThreads / kQuads;
  const int tid = threadIdx.x;
  const int dq = tid % kQuads, sl = tid / kQuads;
  float* red = &sm.acc[0][0][0];            // [kSlices][D]
  float* redm = &sm.m[0][0];                // [kSlices]
  float* redw = &sm.l[0][0];                // [kSlices]
  for (int h = 0; h < a.group; ++h) {
    const int hq = g * a.group + h;
    const size_t row = (size_t)b * a.num_q_heads + hq;
    const float* lse = a.ws_lse + row * a.p_max;
    const f32x4* o = reinterpret_cast<const f32x4*>(a.ws_o + row * a.p_max * D);
    float mr = -INFINITY, wr = 0.f;
    f32x4 ar = {0.f, 0.f, 0.f, 0.f};
    for (int p = sl; p < nparts; p += kSlices) {
      const float lp = lse[p];
      const f32x4 op = o[(size_t)p * kQuads + dq];
      const float mn = fmaxf(mr, lp);
      const float sa = exp2_fast(mr - mn), sb = exp2_fast(lp - mn);
      ar = ar * sa + op * sb;
      wr = wr * sa + sb;
      mr = mn;
    }
    __syncthreads();
    *reinterpret_cast<f32x4*>(&red[sl * D + 4 * dq]) = ar;
    if (dq == 0) {
      redm[sl] = mr;
      redw[sl] = wr;
    }
    __syncthreads();
    if (tid < D) {
      float M = -INFINITY;
#pragma unroll
      for (int s = 0; s < kSlices; ++s) M = fmaxf(M, redm[s]);
      float W = 0.f, acc = 0.f;
#pragma unroll
      for (int s = 0; s < kSlices; ++s) {
        const float e = exp2_fast(redm[s] - M);
        W += e * redw[s];
        acc += e * red[s * D + tid];
      }
      store_out<IO>(a.out, row * D + tid, acc / W);
      if (tid == 0 && a.lse_out) a.lse_out[row] = (M + log2_fast(W)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <typename IO, typename KV, int D>
__global__ void __launch_bounds__(kThreads) pa_decode_kernel(const Params a) {
  __shared__ Smem<D> sm;
  constexpr bool kFam32 = std::is_same<IO, F32>::value;
  constexpr bool kFp8 = std::is_same<KV, FP8>::value;
  constexpr int kEsz = KvSize<KV>::v;
  constexpr size_t kPageBytes = (size_t)kBlock * D * kEsz;

  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.group;
  const int hq0 = g * G;

  const int L = a.context_lens[b];
  const bool bad_len = L < 0 || L > a.max_blocks_per_seq * kBlock;
  const int PT = a.part_tokens;
  const int nparts = (bad_len || L == 0) ? 1 : (PT > 0 ? (L + PT - 1) / PT : 1);
  if (p >= nparts) return;

  if (bad_len || L == 0) {
    // No tokens (or an out-of-contract length): zeros, resp. NaN.
    const float fill = bad_len ? __builtin_nanf("") : 0.f;
    for (int i = tid; i < G * D; i += kThreads)
      store_out<IO>(a.out, ((size_t)b * a.num_q_heads + hq0) * D + i, fill);
    if (a.lse_out && tid < G)
      a.lse_out[(size_t)b * a.num_q_heads + hq0 + tid] = bad_len ? fill : -INFINITY;
    return;
  }

  const int t0 = PT > 0 ? p * PT : 0;
  const int t1 = PT > 0 ? min(t0 + PT, L) : L;
  const int page0 = t0 / kBlock;
  const int npages = (t1 - t0 + kBlock - 1) / kBlock;
  const int nmine = npages > w ? (npages - w + kWaves - 1) / kWaves : 0;

  // Query operand: lane (rr, jj) feeds query head rr (zero beyond the group).
  const int rr = lane & 15, jj = lane >> 4;
  const bool head_ok = rr < G;
  const uint8_t* qrow = a.q + ((size_t)b * a.num_q_heads + hq0 + (head_ok ? rr : 0)) * D * IoSize<IO>::v;

  float kmul = a.scale * kLog2e;
  float vmul = 1.0f;
  if constexpr (kFp8) {
    kmul *= a.k_scale[g];
    vmul = a.v_scale[g];
  }

  const int32_t* bt = a.block_table + (size_t)b * a.max_blocks_per_seq + page0;
  const uint8_t* kbase = a.k + (size_t)g * kPageBytes;
  const uint8_t* vbase = a.v + (size_t)g * kPageBytes;
  const size_t block_stride = (size_t)a.num_kv_heads * kPageBytes;

  WaveState<D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) st.acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool bad_blk = false;

  // Block ids of this wave's pages: lane i holds page w + kWaves * (i + 64 * chunk).
  int btv = 0;
  auto fetch_bt = [&](int chunk) {
    const int i = chunk * 64 + lane;
    btv = i < nmine ? bt[w + kWaves * i] : 0;
  };
  auto page_ptrs = [&](int i, const uint8_t*& kp, const uint8_t*& vp) {
    int phys = __builtin_amdgcn_readlane(btv, i & 63);
    if ((unsigned)phys >= (unsigned)a.num_blocks) {
      bad_blk = true;
      phys = 0;
    }
    kp = kbase + (size_t)phys * block_stride;
    vp = vbase + (size_t)phys * block_stride;
  };
  auto nvalid_of = [&](int i) { return t1 - (t0 + (w + kWaves * i) * kBlock); };

  if constexpr (!kFam32) {
    using O = Op16<IO>;
    using A8 = typename O::A8;
    constexpr bool kv16 = !kFp8;
    A8 qop[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      // d-slots of chunk c: 16-bit cache -> 8*(jj + 4c) + e;
      // fp8 cache -> 16*(jj + 4*(c/2)) + 8*(c%2) + e.
      const int d0 = kv16 ? 8 * (jj + 4 * c) : 16 * (jj + 4 * (c / 2)) + 8 * (c % 2);
      u32x4 raw = *reinterpret_cast<const u32x4*>(qrow + d0 * 2);
      if (!head_ok) raw = u32x4{0u, 0u, 0u, 0u};
      qop[c] = bitcast16<A8>(raw);
    }
    PageRegs16<D, kv16> ra, rb;
    const uint8_t *kp, *vp;
    if (nmine > 0) {
      fetch_bt(0);
      page_ptrs(0, kp, vp);
      load_page16<D, kv16>(ra, kp, vp, lane);
    }
    for (int i = 0; i < nmine; i += 2) {
      if (i + 1 < nmine) {
        if (((i + 1) & 63) == 0) fetch_bt((i + 1) >> 6);
        page_ptrs(i + 1, kp, vp);
        load_page16<D, kv16>(rb, kp, vp, lane);
      }
      compute_page16<IO, KV, D>(st, ra, qop, kmul, nvalid_of(i), lane);
      if (i + 1 < nmine) {
        if (i + 2 < nmine) {
          if (((i + 2) & 63) == 0) fetch_bt((i + 2) >> 6);
          page_ptrs(i + 2, kp, vp);
          load_page16<D, kv16>(ra, kp, vp, lane);
        }
        compute_page16<IO, KV, D>(st, rb, qop, kmul, nvalid_of(i + 1), lane);
      }
    }
  } else {
    f32x4 qop[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      f32x4 raw = *reinterpret_cast<const f32x4*>(qrow + (size_t)4 * (jj + 4 * c) * 4);
      qop[c] = head_ok ? raw : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    PageRegs32<D> ra, rb;
    const uint8_t *kp, *vp;
    if (nmine > 0) {
      fetch_bt(0);
      page_ptrs(0, kp, vp);
      load_page32<D>(ra, kp, vp, lane);
    }
    for (int i = 0; i < nmine; i += 2) {
      if (i + 1 < nmine) {
        if (((i + 1) & 63) == 0) fetch_bt((i + 1) >> 6);
        page_ptrs(i + 1, kp, vp);
        load_page32<D>(rb, kp, vp, lane);
      }
      compute_page32<D>(st, ra, qop, kmul, nvalid_of(i), lane);
      if (i + 1 < nmine) {
        if (i + 2 < nmine) {
          if (((i + 2) & 63) == 0) fetch_bt((i + 2) >> 6);
          page_ptrs(i + 2, kp, vp);
          load_page32<D>(ra, kp, vp, lane);
        }
        compute_page32<D>(st, rb, qop, kmul, nvalid_of(i + 1), lane);
      }
    }
  }

  // ---- merge the waves through LDS --------------------------------------
  const float lsum = wave_sum_rows(st.l);
  if (tid == 0) sm.bad = 0;
  __syncthreads();
  if (bad_blk) sm.bad = 1;
  if (head_ok) {
    if (jj == 0) {
      sm.m[w][rr] = st.m;
      sm.l[w][rr] = lsum;
    }
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      *reinterpret_cast<f32x4*>(&sm.acc[w][rr][16 * t + 4 * jj]) = st.acc[t];
  }
  __syncthreads();
  const bool bad = sm.bad != 0;

  const bool split = nparts > 1;
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, d = i - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.m[ww][h]);
    float W = 0.f, o = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float e = exp2_fast(sm.m[ww][h] - M);
      W += e * sm.l[ww][h];
      o += e * sm.acc[ww][h][d];
    }
    float val = o / W * vmul;
    float lse2 = M + log2_fast(W);
    if (bad) val = lse2 = __builtin_nanf("");
    const size_t row = (size_t)b * a.num_q_heads + hq0 + h;
    if (!split) {
      store_out<IO>(a.out, row * D + d, val);
      if (d == 0 && a.lse_out) a.lse_out[row] = lse2 * kLn2;
    } else {
      a.ws_o[(row * a.p_max + p) * D + d] = val;
      if (d == 0) a.ws_lse[row * a.p_max + p] = lse2;
    }
  }
  if (!split) return;

  // ---- split-K: the last partition of (b, g) to finish merges ------------
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    uint32_t* cnt = a.ws_cnt + (size_t)b * a.num_kv_heads + g;
    const uint32_t done = atomicAdd(cnt, 1u);
    sm.last = done == (uint32_t)(nparts - 1);
  }
  __syncthreads();
  if (!sm.last) return;
  __threadfence();
  merge_partitions<IO, D>(a, sm, b, g, nparts);
  if (tid == 0) atomicExch(a.ws_cnt + (size_t)b * a.num_kv_heads + g, 0u);
}

__global__ void fill_zero_kernel(uint8_t* p, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t n16 = n / 16;
  for (size_t j = i; j < n16; j += (size_t)gridDim.x * blockDim.x)
    reinterpret_cast<u32x4*>(p)[j] = u32x4{0u, 0u, 0u, 0u};
  if (i < n % 16) p[n16 * 16 + i] = 0;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t o_off, lse_off, cnt_off, total;
  int p_max;
};

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static bool shape_ok(const pa_shape* s) {
  if (!s) return false;
  if (s->batch < 0 || s->batch > 65535) return false;
  if (s->num_kv_heads < 1 || s->num_kv_heads > 65535) return false;
  if (s->num_q_heads < 1 || s->num_q_heads % s->num_kv_heads != 0) return false;
  if (s->num_q_heads / s->num_kv_heads > kMaxGroup) return false;
  if (s->head_dim != 64 && s->head_dim != 128) return false;
  if (s->block_size != kBlock) return false;
  if (s->max_blocks_per_seq < 1 || s->max_blocks_per_seq > (1 << 26)) return false;
  if (s->num_blocks < 1) return false;
  if (s->partition_size < 0 || s->partition_size % kBlock != 0) return false;
  return true;
}

static WsLayout ws_layout(const pa_shape* s) {
  WsLayout w{0, 0, 0, 0, 1};
  if (s->partition_size == 0) return w;
  const long long tokens = (long long)s->max_blocks_per_seq * kBlock;
  w.p_max = (int)((tokens + s->partition_size - 1) / s->partition_size);
  const size_t rows = (size_t)s->batch * s->num_q_heads * w.p_max;
  w.o_off = 0;
  w.lse_off = align_up(rows * s->head_dim * sizeof(float), 256);
  w.cnt_off = w.lse_off + align_up(rows * sizeof(float), 256);
  w.total = w.cnt_off + align_up((size_t)s->batch * s->num_kv_heads * sizeof(uint32_t), 256);
  return w;
}

template <typename IO, typename KV, int D>
static hipError_t launch(const Params& prm, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((pa_decode_kernel<IO, KV, D>), grid, dim3(kThreads), 0, stream, prm);
  return hipGetLastError();
}

template <typename IO, typename KV>
static hipError_t launch_d(int D, const Params& prm, dim3 grid, hipStream_t stream) {
  return D == 64 ? launch<IO, KV, 64>(prm, grid, stream) : launch<IO, KV, 128>(prm, grid, stream);
}

static inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace pa

extern "C" {

size_t pa_decode_workspace_bytes(const pa_shape* shape) {
  if (!pa::shape_ok(shape)) return 0;
  return pa::ws_layout(shape).total;
}

pa_status pa_decode(const pa_shape* shape, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* block_table,
                    const int32_t* context_lens, float scale, pa_dtype io_dtype,
                    pa_dtype kv_dtype, const float* k_scale, const float* v_scale,
                    void* workspace, size_t workspace_bytes, void* out, float* lse_out,
                    void* stream) {
  using namespace pa;
  if (!shape) return PA_ERR_NULL;
  if (!shape_ok(shape)) return PA_ERR_SHAPE;
  if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out) return PA_ERR_NULL;
  const bool io_ok = io_dtype == PA_F32 || io_dtype == PA_F16 || io_dtype == PA_BF16;
  const bool kv_ok = kv_dtype == io_dtype || (kv_dtype == PA_FP8_E4M3 && io_dtype != PA_F32);
  if (!io_ok || !kv_ok) return PA_ERR_DTYPE;
  if (kv_dtype == PA_FP8_E4M3 && (!k_scale || !v_scale)) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return PA_ERR_ALIGN;
  if (((uintptr_t)block_table & 3u) || ((uintptr_t)context_lens & 3u) ||
      ((uintptr_t)lse_out & 3u))
    return PA_ERR_ALIGN;
  const WsLayout wl = ws_layout(shape);
  if (shape->partition_size > 0) {
    if (!workspace || workspace_bytes < wl.total) return PA_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 255u) return PA_ERR_ALIGN;
  }
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
  prm.ws_o = shape->partition_size > 0 ? reinterpret_cast<float*>(ws + wl.o_off) : nullptr;
  prm.ws_lse = shape->partition_size > 0 ? reinterpret_cast<float*>(ws + wl.lse_off) : nullptr;
  prm.ws_cnt = shape->partition_size > 0 ? reinterpret_cast<uint32_t*>(ws + wl.cnt_off) : nullptr;
  prm.scale = scale;
  prm.num_q_heads = shape->num_q_heads;
  prm.num_kv_heads = shape->num_kv_heads;
  prm.group = shape->num_q_heads / shape->num_kv_heads;
  prm.max_blocks_per_seq = shape->max_blocks_per_seq;
  prm.num_blocks = shape->num_blocks;
  prm.part_tokens = shape->partition_size;
  prm.p_max = wl.p_max;

  const dim3 grid(wl.p_max, shape->num_kv_heads, shape->batch);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  const int D = shape->head_dim;
  if (io_dtype == PA_F32)
    e = launch_d<F32, F32>(D, prm, grid, st);
  else if (io_dtype == PA_F16)
    e = kv_dtype == PA_FP8_E4M3 ? launch_d<F16, FP8>(D, prm, grid, st)
                                : launch_d<F16, F16>(D, prm, grid, st);
  else
    e = kv_dtype == PA_FP8_E4M3 ? launch_d<BF16, FP8>(D, prm, grid, st)
                                : launch_d<BF16, BF16>(D, prm, grid, st);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
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
  }
  return "unknown status";
}

}  // extern "C"
