// Merge of decode-attention results computed on disjoint position shards,
// by log-sum-exp ("RapidLLM", feature table, row "Decode context
// parallelism"): for every row r (a (sequence, query head) pair), with
// natural-log lse_s[r] from shards s = 0 .. S-1,
//     M = max_s lse_s,  w_s = exp(lse_s - M),
//     out[r] = sum_s w_s o_s[r] / sum_s w_s,   lse[r] = M + log sum_s w_s.
// A shard with lse = -inf (no tokens) contributes nothing; a row with none
// gives out = 0 and lse = -inf; a NaN lse makes the row NaN.
//
// One thread per (row, 4-element quad): it walks the shards in order with a
// running maximum (base 2 inside), so the result does not depend on the
// launch; the loads of 8 shards are in flight at once. Loads are 8-byte
// (16-bit types) or 16-byte (f32) quads.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "padecode.h"
#include "pa_host.h"

namespace pa_merge {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kThreads = pa_host::kMergeThreads;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

struct F32 {};
struct F16 {};
struct BF16 {};

template <typename T>
__device__ __forceinline__ f32x4 load4(const void* p, size_t i);
template <>
__device__ __forceinline__ f32x4 load4<F32>(const void* p, size_t i) {
  return *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
}
template <>
__device__ __forceinline__ f32x4 load4<F16>(const void* p, size_t i) {
  const f16x4 v = *reinterpret_cast<const f16x4*>(static_cast<const _Float16*>(p) + i);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <>
__device__ __forceinline__ f32x4 load4<BF16>(const void* p, size_t i) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(static_cast<const __bf16*>(p) + i);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

template <typename T>
__device__ __forceinline__ void store4(void* p, size_t i, f32x4 v);
template <>
__device__ __forceinline__ void store4<F32>(void* p, size_t i, f32x4 v) {
  *reinterpret_cast<f32x4*>(static_cast<float*>(p) + i) = v;
}
template <>
__device__ __forceinline__ void store4<F16>(void* p, size_t i, f32x4 v) {
  *reinterpret_cast<f16x4*>(static_cast<_Float16*>(p) + i) =
      f16x4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
}
template <>
__device__ __forceinline__ void store4<BF16>(void* p, size_t i, f32x4 v) {
  *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p) + i) =
      bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
}

struct Params {
  const void* shard_out;   // [S][rows][D]
  const float* shard_lse;  // [S][rows]
  void* out;               // [rows][D]
  float* lse_out;          // [rows] or null
  int32_t shards, rows, D;
};

template <typename T>
__global__ void __launch_bounds__(kThreads) lse_merge_kernel(const Params a) {
  const int quads = a.D / 4;
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (long long)a.rows * quads) return;
  const int r = (int)(i / quads);
  const int dq = (int)(i - (long long)r * quads);
  float m = -INFINITY, w = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  bool nan = false;
  // kBatch shards' loads are issued before any is folded in
  constexpr int kBatch = 8;
  for (int s0 = 0; s0 < a.shards; s0 += kBatch) {
    float lv[kBatch];
    f32x4 ov[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int s = s0 + u;
      if (s < a.shards) {
        lv[u] = a.shard_lse[(size_t)s * a.rows + r];
        ov[u] = load4<T>(a.shard_out, ((size_t)s * a.rows + r) * a.D + 4 * dq);
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (s0 + u >= a.shards) break;
      const float l = lv[u];
      if (l != l) nan = true;
      if (!(l > -INFINITY)) continue;   // empty shard (or NaN, flagged above)
      const float l2 = l * kLog2e;
      const float mn = fmaxf(m, l2);
      const float sa = exp2f(m - mn), sb = exp2f(l2 - mn);
      acc = acc * sa + ov[u] * sb;
      w = w * sa + sb;
      m = mn;
    }
  }
  f32x4 val;
  float lse;
  if (nan) {
    val = f32x4{NAN, NAN, NAN, NAN};
    lse = NAN;
  } else if (w > 0.f) {
    val = f32x4{acc[0] / w, acc[1] / w, acc[2] / w, acc[3] / w};
    lse = (m + log2f(w)) * kLn2;
  } else {
    val = f32x4{0.f, 0.f, 0.f, 0.f};
    lse = -INFINITY;
  }
  store4<T>(a.out, (size_t)r * a.D + 4 * dq, val);
  if (dq == 0 && a.lse_out) a.lse_out[r] = lse;
}

}  // namespace pa_merge

extern "C" pa_status pa_lse_merge(int32_t num_shards, int32_t rows, int32_t head_dim,
                                  const void* shard_out, const float* shard_lse,
                                  pa_dtype dtype, void* out, float* lse_out, void* stream) {
  using namespace pa_merge;
  unsigned blocks = 0;
  const pa_status status = pa_host::merge_status(num_shards, rows, head_dim, shard_out, shard_lse, dtype,
                                                 out, lse_out, &blocks);
  if (status != PA_OK) return status;
  if (blocks == 0) return PA_OK;
  Params p{shard_out, shard_lse, out, lse_out, num_shards, rows, head_dim};
  const dim3 grid(blocks);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == PA_F32)
    hipLaunchKernelGGL(lse_merge_kernel<F32>, grid, dim3(kThreads), 0, st, p);
  else if (dtype == PA_F16)
    hipLaunchKernelGGL(lse_merge_kernel<F16>, grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(lse_merge_kernel<BF16>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
