// Building blocks shared by the paged-attention kernels for gfx950: vector
// types, storage tags, memory helpers, and the matrix-core page tiles that
// turn one 16-token K/V page and a 16-column query operand into scores and
// PV products.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

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

constexpr int gcd_c(int x, int y) { return y == 0 ? x : gcd_c(y, x % y); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Lanes l, l^16, l^32, l^48 hold the same query head. The reductions use
// gfx950's lane-swap instructions: with x in both operands,
// v_permlane16_swap returns the pair {x[l], x[l^16]} (in some order) and
// v_permlane32_swap the pair {x[l], x[l^32]}, in the vector ALU, without the
// LDS round trip a bpermute makes. max and + are commutative, so every lane
// of a head gets the same bits (and the same bits as the xor-shuffle form).
__device__ __forceinline__ float pair_max(float x, bool wide) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = wide ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                      : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum(float x, bool wide) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = wide ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                      : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ float wave_max_rows(float x) { return pair_max(pair_max(x, false), true); }
__device__ __forceinline__ float wave_sum_rows(float x) { return pair_sum(pair_sum(x, false), true); }

// Global-memory pointer every lane agrees on, kept in scalar registers, so
// loads take the saddr + 32-bit voffset form of global_load.
typedef const __attribute__((address_space(1))) uint8_t* gptr;
__device__ __forceinline__ gptr uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return (gptr)((static_cast<uint64_t>(hi) << 32) | lo);
}

template <typename V>
__device__ __forceinline__ V ld(gptr base, uint32_t off) {
  return *(const __attribute__((address_space(1))) V*)(base + off);
}
// Non-temporal load (global_load ... nt): for K/V pages, which a call reads
// once. Measured on MI355X: 6.6% faster decode on the Qwen2.5-7B-shaped
// workload, and random 4 KiB page reads 5% faster than with ordinary loads.
template <typename V>
__device__ __forceinline__ V ld_nt(gptr base, uint32_t off) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) V*)(base + off));
}
// kKeep: an ordinary load, for pages that other workgroups read again soon
template <bool kKeep, typename V>
__device__ __forceinline__ V ld_page(gptr base, uint32_t off) {
  if constexpr (kKeep) return ld<V>(base, off);
  else return ld_nt<V>(base, off);
}

// Agent-coherent (write-through / cache-revalidating) float store and load.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte agent-coherent accesses through a buffer resource (base must be
// wave-uniform): the SC1 cache-policy bit, the same one the agent-scope
// atomics above carry, on a dwordx4 buffer load/store. One such access moves
// a float4 where four scalar ones would each cost a memory transaction.
constexpr int kCpolSc1 = 16;
typedef __amdgpu_buffer_rsrc_t brsrc;
__device__ __forceinline__ brsrc buffer_rsrc(const float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 ld_agent4(brsrc r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1));
}
__device__ __forceinline__ void st_agent4(brsrc r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCpolSc1);
}
// Loads at per-lane byte offset off plus the wave-uniform byte offset soff
// (the instruction's scalar offset field: a batch of loads shares one
// per-lane offset register).
__device__ __forceinline__ f32x4 ld_agent4(brsrc r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, kCpolSc1));
}
__device__ __forceinline__ float ld_agent1(brsrc r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, kCpolSc1));
}

// Workgroup barrier that orders LDS only: each wave waits for its own LDS
// (and scalar) operations, not for its global stores, which __syncthreads()
// would wait for as well and the next LDS phase does not depend on.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Outcome of counting one piece of n on a workspace counter.
constexpr int kCountMore = 0;    // other pieces are still to come
constexpr int kCountLast = 1;    // this piece completed the count: merge, counter reset to 0
constexpr int kCountStale = 2;   // the counter held n or more before this call

// Count one piece on *cnt (one thread). A completed call leaves every counter
// at 0, so during a call a counter runs 0 .. n-1; a value of n or more can only
// be left over from a broken workspace-reuse rule. Such a piece takes its
// count back (the counter keeps its stale value, so later calls see it too
// until the workspace is reset) and reports kCountStale, and the caller makes
// the rows NaN rather than merge partial results that were never counted.
__device__ __forceinline__ int count_piece(uint32_t* cnt, int n) {
  const uint32_t done = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (done == (uint32_t)(n - 1)) {
    __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return kCountLast;
  }
  if (done >= (uint32_t)n) {
    __hip_atomic_fetch_sub(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return kCountStale;
  }
  return kCountMore;
}

// Split-K hand-off: every wave waits until its agent-coherent stores have
// completed, then one thread counts this piece on *cnt; the outcome
// (count_piece) is returned uniformly to the whole workgroup. kCountLast
// makes the workgroup the owner of the merge.
__device__ __forceinline__ int last_to_finish(uint32_t* cnt, int n, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) *flag = count_piece(cnt, n);
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*flag);
}

// ---------------------------------------------------------------------------
// Matrix-core operand types.
//
// Lane l of a wave is (r = l % 16, jj = l / 16). In the QK^T product lane l
// feeds token r of the page (A operand) and query head r (B operand); both
// operands put the same head-dim elements in the same k-slots of the lane,
// namely the elements of 16-byte K-page groups jj + 4*i. The 16x16
// accumulator leaves lane l with rows 4*jj .. 4*jj+3 (tokens) of column r
// (query head), which is exactly the B operand of the PV product (k = token
// 4*jj + i, n = head r); its A operand is V^T[16*t + r][4*jj + i]. So the
// result O^T[16*t + 4*jj + i][head r] stays with the lane that owns head r's
// softmax state.
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
  // 4 fp8 codes (one dword, lowest byte first) -> 4 exact f16 values
  static __device__ __forceinline__ A4 fp8x4(uint32_t w) {
    const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
    return A4{lo[0], lo[1], hi[0], hi[1]};
  }
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
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return A4{lo[0], lo[1], hi[0], hi[1]};
  }
};

// ---------------------------------------------------------------------------
// Page tiles: what one wave holds of one page and how it feeds the MFMAs.
//   kKoff / kVoff: per-lane byte offsets inside a K / V page (loop constants)
//   load_k()/load_v(): issue the page's K / V loads;  scores(): S^T for the page;
//   pvt(): the V^T operand of tile t (4 tokens of row 16*t + r).
// load_q() reads the query row the caller points it at. Lanes whose head
// column r lies past the group (r >= G) are pointed at the group's first row:
// an MFMA output column depends only on its own B column, so those columns
// hold finite duplicates that are never stored, and the query operand needs
// no masking after its load (a select there would make the compiler wait for
// the load at once).
// ---------------------------------------------------------------------------

// q/out f16 or bf16 with a cache of the same type.
template <typename IO, int D>
struct Tile16 {
  using O = Op16<IO>;
  typedef typename O::A8 A8;
  typedef typename O::A4 A4;
  typedef A4 P;                            // PV B operand: 4 rounded probabilities
  static constexpr int kK = D / 32;        // 16-byte K loads = QK MFMAs
  static constexpr int kT = D / 16;        // V tiles (8-byte loads)
  // register ring depths (pages in flight per wave for K and for V); a third
  // K stage at D = 128 does not fit in the 168 VGPRs of 3 waves per SIMD
  static constexpr int kKStages = D == 128 ? 2 : 4;
  static constexpr int kVStages = 2;
  struct KRegs {
    u32x4 k[kK];
  };
  struct VRegs {
    u32x2 v[kT];
  };
  typedef A8 QC;                           // one 16-byte chunk of the query operand
  static constexpr int kQ = kK;            // chunks per lane
  struct Q {
    QC c[kQ];
  };
  static __device__ __forceinline__ uint32_t koff(int lane) { return lane * 16; }
  static __device__ __forceinline__ uint32_t voff(int lane) { return (lane & 15) * 32 + (lane >> 4) * 8; }
  // byte offset in the query row of chunk c of lane group jj:
  // head-dim 8*(jj + 4c) .. +7
  static __device__ __forceinline__ uint32_t qoff(int c, int jj) { return 16 * (jj + 4 * c); }
  static __device__ __forceinline__ void load_q(Q& q, gptr qrow, int jj) {
#pragma unroll
    for (int c = 0; c < kQ; ++c) q.c[c] = __builtin_bit_cast(QC, ld<u32x4>(qrow, qoff(c, jj)));
  }
  template <bool kKeep = false>
  static __device__ __forceinline__ void load_k(KRegs& r, gptr kp, uint32_t ko) {
#pragma unroll
    for (int i = 0; i < kK; ++i) r.k[i] = ld_page<kKeep, u32x4>(kp, ko + i * 1024);
  }
  template <bool kKeep = false>
  static __device__ __forceinline__ void load_v(VRegs& r, gptr vp, uint32_t vo) {
#pragma unroll
    for (int t = 0; t < kT; ++t) r.v[t] = ld_page<kKeep, u32x2>(vp, vo + t * 512);
  }
  static __device__ __forceinline__ f32x4 scores(const KRegs& r, const Q& q) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kK; ++c) s = O::qk(__builtin_bit_cast(A8, r.k[c]), q.c[c], s);
    return s;
  }
  static __device__ __forceinline__ A4 pvt(const VRegs& r, int t) {
    return __builtin_bit_cast(A4, r.v[t]);
  }
  static __device__ __forceinline__ P pack(const float p[4]) {
    return P{(typename O::E)p[0], (typename O::E)p[1], (typename O::E)p[2], (typename O::E)p[3]};
  }
  static __device__ __forceinline__ float psum(P p) {
    return ((float)p[0] + (float)p[1]) + ((float)p[2] + (float)p[3]);
  }
  static __device__ __forceinline__ f32x4 pv(A4 a, P b, f32x4 c) { return O::pv(a, b, c); }
  static __device__ __forceinline__ A4 zero_tail(A4 a, int jj, int nvalid) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * jj + i >= nvalid) a[i] = (typename O::E)0.0f;
    return a;
  }
};

// q/out f16 or bf16 with an fp8-e4m3 cache.
template <typename IO, int D>
struct Tile8 {
  using O = Op16<IO>;
  typedef typename O::A8 A8;
  typedef typename O::A4 A4;
  typedef A4 P;
  static constexpr int kK = D / 64;        // 16-byte K loads, two QK MFMAs each
  static constexpr int kT = D / 16;        // V tiles (4-byte loads)
  static constexpr int kKStages = 4;
  static constexpr int kVStages = 2;
  struct KRegs {
    u32x4 k[kK];
  };
  struct VRegs {
    uint32_t v[kT];
  };
  typedef A8 QC;
  static constexpr int kQ = 2 * kK;
  struct Q {
    QC c[kQ];
  };
  static __device__ __forceinline__ uint32_t koff(int lane) { return lane * 16; }
  static __device__ __forceinline__ uint32_t voff(int lane) { return (lane & 15) * 16 + (lane >> 4) * 4; }
  // head-dim 16*(jj + 4*(c/2)) + 8*(c%2) .. +7
  static __device__ __forceinline__ uint32_t qoff(int c, int jj) {
    return 2 * (16 * (jj + 4 * (c / 2)) + 8 * (c % 2));
  }
  static __device__ __forceinline__ void load_q(Q& q, gptr qrow, int jj) {
#pragma unroll
    for (int c = 0; c < kQ; ++c) q.c[c] = __builtin_bit_cast(QC, ld<u32x4>(qrow, qoff(c, jj)));
  }
  template <bool kKeep = false>
  static __device__ __forceinline__ void load_k(KRegs& r, gptr kp, uint32_t ko) {
#pragma unroll
    for (int i = 0; i < kK; ++i) r.k[i] = ld_page<kKeep, u32x4>(kp, ko + i * 1024);
  }
  template <bool kKeep = false>
  static __device__ __forceinline__ void load_v(VRegs& r, gptr vp, uint32_t vo) {
#pragma unroll
    for (int t = 0; t < kT; ++t) r.v[t] = ld_page<kKeep, uint32_t>(vp, vo + t * 256);
  }
  static __device__ __forceinline__ f32x4 scores(const KRegs& r, const Q& q) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kK; ++c) {
      const A4 a0 = O::fp8x4(r.k[c][0]), a1 = O::fp8x4(r.k[c][1]);
      const A4 a2 = O::fp8x4(r.k[c][2]), a3 = O::fp8x4(r.k[c][3]);
      const A8 lo = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      const A8 hi = {a2[0], a2[1], a2[2], a2[3], a3[0], a3[1], a3[2], a3[3]};
      s = O::qk(lo, q.c[2 * c], s);
      s = O::qk(hi, q.c[2 * c + 1], s);
    }
    return s;
  }
  static __device__ __forceinline__ A4 pvt(const VRegs& r, int t) { return O::fp8x4(r.v[t]); }
  static __device__ __forceinline__ P pack(const float p[4]) {
    return Tile16<IO, D>::pack(p);
  }
  static __device__ __forceinline__ float psum(P p) { return Tile16<IO, D>::psum(p); }
  static __device__ __forceinline__ f32x4 pv(A4 a, P b, f32x4 c) { return O::pv(a, b, c); }
  static __device__ __forceinline__ A4 zero_tail(A4 a, int jj, int nvalid) {
    return Tile16<IO, D>::zero_tail(a, jj, nvalid);
  }
};

// q/out and cache f32: 16x16x4 f32 MFMAs, one element per lane per step.
template <int D>
struct Tile32 {
  typedef f32x4 A4;
  typedef f32x4 P;
  static constexpr int kK = D / 16;        // 16-byte K loads, four QK MFMAs each
  static constexpr int kT = D / 16;        // V tiles (16-byte loads)
  static constexpr int kKStages = D == 128 ? 1 : 2;
  static constexpr int kVStages = D == 128 ? 1 : 2;
  struct KRegs {
    f32x4 k[kK];
  };
  struct VRegs {
    f32x4 v[kT];
  };
  typedef f32x4 QC;
  static constexpr int kQ = kK;
  struct Q {
    QC c[kQ];
  };
  static __device__ __forceinline__ uint32_t koff(int lane) { return lane * 16; }
  static __device__ __forceinline__ uint32_t voff(int lane) { return (lane & 15) * 64 + (lane >> 4) * 16; }
  // head-dim 4*(jj + 4c) .. +3
  static __device__ __forceinline__ uint32_t qoff(int c, int jj) { return 16 * (jj + 4 * c); }
  static __device__ __forceinline__ void load_q(Q& q, gptr qrow, int jj) {
#pragma unroll
    for (int c = 0; c < kQ; ++c) q.c[c] = ld<f32x4>(qrow, qoff(c, jj));
  }
  template <bool kKeep = false>
  static __device__ __forceinline__ void load_k(KRegs& r, gptr kp, uint32_t ko) {
#pragma unroll
    for (int i = 0; i < kK; ++i) r.k[i] = ld_page<kKeep, f32x4>(kp, ko + i * 1024);
  }
  template <bool kKeep = false>
  static __device__ __forceinline__ void load_v(VRegs& r, gptr vp, uint32_t vo) {
#pragma unroll
    for (int t = 0; t < kT; ++t) r.v[t] = ld_page<kKeep, f32x4>(vp, vo + t * 1024);
  }
  static __device__ __forceinline__ f32x4 scores(const KRegs& r, const Q& q) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kK; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(r.k[c][e], q.c[c][e], s, 0, 0, 0);
    return s;
  }
  static __device__ __forceinline__ A4 pvt(const VRegs& r, int t) { return r.v[t]; }
  static __device__ __forceinline__ P pack(const float p[4]) { return P{p[0], p[1], p[2], p[3]}; }
  static __device__ __forceinline__ float psum(P p) { return (p[0] + p[1]) + (p[2] + p[3]); }
  static __device__ __forceinline__ f32x4 pv(A4 a, P b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ A4 zero_tail(A4 a, int jj, int nvalid) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * jj + i >= nvalid) a[i] = 0.0f;
    return a;
  }
};

template <typename IO, typename KV, int D>
struct TileOf {
  typedef typename std::conditional<std::is_same<KV, FP8>::value, Tile8<IO, D>, Tile16<IO, D>>::type type;
};
template <int D>
struct TileOf<F32, F32, D> {
  typedef Tile32<D> type;
};

// ---------------------------------------------------------------------------
// Output conversion and sizes.
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
__device__ __forceinline__ void store_out4(uint8_t* out, size_t idx, f32x4 v);
template <>
__device__ __forceinline__ void store_out4<F32>(uint8_t* out, size_t idx, f32x4 v) {
  *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + idx) = v;
}
template <>
__device__ __forceinline__ void store_out4<F16>(uint8_t* out, size_t idx, f32x4 v) {
  *reinterpret_cast<f16x4*>(reinterpret_cast<_Float16*>(out) + idx) =
      f16x4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
}
template <>
__device__ __forceinline__ void store_out4<BF16>(uint8_t* out, size_t idx, f32x4 v) {
  *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(out) + idx) =
      bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
}

template <typename T> struct ElemSize { static constexpr int v = 2; };
template <> struct ElemSize<F32> { static constexpr int v = 4; };
template <> struct ElemSize<FP8> { static constexpr int v = 1; };

}  // namespace pa
