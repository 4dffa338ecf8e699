// Paged KV append for gfx950: write each sequence's new token K and V rows
// into its block and slot of the paged caches, as the decode step does right
// before attention ("rvLLM: High-performance LLM inference in Rust", section
// "Kernel Compiler Stack", the per-layer decode step list: the KV cache write
// follows RoPE and precedes attention), optionally quantising to an fp8
// (OCP E4M3) cache ("rvLLM", sections "What's Inside" and "Optional
// Features"; "Litellama", section "Features": FP8 KV cache).
//
// One wavefront per (sequence, KV head); lane d writes head-dim elements
// d, d + 64. Cache layouts are those pa_decode reads (include/padecode.h):
//   k_cache[blk][g][d / X][slot][d % X]   X = 16 bytes of elements
//   v_cache[blk][g][d][slot]
// fp8: code = RNE(clamp(x / scale, -448, 448)) with the division in float32
// and the gfx950 conversion instruction doing the rounding; NaN -> 0x7F.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "padecode.h"
#include "pa_host.h"

namespace pa_append {

constexpr int kBlock = pa_host::kPageTokens;

struct F32 {};
struct F16 {};
struct BF16 {};
struct FP8 {};

template <typename T> struct Bytes { static constexpr int v = 2; };
template <> struct Bytes<F32> { static constexpr int v = 4; };
template <> struct Bytes<FP8> { static constexpr int v = 1; };

struct Params {
  const uint8_t* k_new;
  const uint8_t* v_new;
  const int32_t* positions;
  const int32_t* block_table;
  const float* k_scale;
  const float* v_scale;
  uint8_t* k_cache;
  uint8_t* v_cache;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
};

template <typename SRC>
__device__ __forceinline__ float widen(const uint8_t* p, size_t i);
template <>
__device__ __forceinline__ float widen<F32>(const uint8_t* p, size_t i) {
  return reinterpret_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float widen<F16>(const uint8_t* p, size_t i) {
  return (float)reinterpret_cast<const _Float16*>(p)[i];
}
template <>
__device__ __forceinline__ float widen<BF16>(const uint8_t* p, size_t i) {
  return (float)reinterpret_cast<const __bf16*>(p)[i];
}

// One E4M3 code: RNE of the clamped float32 value; NaN -> 0x7F.
__device__ __forceinline__ uint8_t e4m3_code(float y) {
  if (y != y) return 0x7F;
  y = y < -448.f ? -448.f : (y > 448.f ? 448.f : y);
  const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false);
  return (uint8_t)(packed & 0xFF);
}

template <typename SRC, typename KV, int D>
__global__ void __launch_bounds__(64) kv_append_kernel(const Params a) {
  constexpr int kEs = Bytes<KV>::v;
  constexpr int kX = 16 / kEs;
  const int H = a.num_kv_heads;
  const int b = blockIdx.x / H;
  const int g = blockIdx.x - b * H;
  const int lane = threadIdx.x;

  const int pos = a.positions[b];
  if (pos < 0 || pos >= a.max_blocks_per_seq * kBlock) return;   // padding / out of contract
  const int blk = a.block_table[(size_t)b * a.max_blocks_per_seq + pos / kBlock];
  if (blk < 0 || blk >= a.num_blocks) return;
  const int slot = pos % kBlock;

  const size_t src_row = ((size_t)b * H + g) * D;
  const size_t page = ((size_t)blk * H + g) * (size_t)kBlock * D;   // elements
  float ks = 1.f, vs = 1.f;
  if constexpr (std::is_same<KV, FP8>::value) {
    ks = a.k_scale[g];
    vs = a.v_scale[g];
  }
#pragma unroll
  for (int d = lane; d < D; d += 64) {
    const size_t ko = page + (size_t)(d / kX) * kBlock * kX + (size_t)slot * kX + d % kX;
    const size_t vo = page + (size_t)d * kBlock + slot;
    if constexpr (std::is_same<KV, FP8>::value) {
      a.k_cache[ko] = e4m3_code(widen<SRC>(a.k_new, src_row + d) / ks);
      a.v_cache[vo] = e4m3_code(widen<SRC>(a.v_new, src_row + d) / vs);
    } else if constexpr (kEs == 4) {
      reinterpret_cast<uint32_t*>(a.k_cache)[ko] = reinterpret_cast<const uint32_t*>(a.k_new)[src_row + d];
      reinterpret_cast<uint32_t*>(a.v_cache)[vo] = reinterpret_cast<const uint32_t*>(a.v_new)[src_row + d];
    } else {
      reinterpret_cast<uint16_t*>(a.k_cache)[ko] = reinterpret_cast<const uint16_t*>(a.k_new)[src_row + d];
      reinterpret_cast<uint16_t*>(a.v_cache)[vo] = reinterpret_cast<const uint16_t*>(a.v_new)[src_row + d];
    }
  }
}

template <typename SRC, typename KV>
static hipError_t launch(int D, const Params& p, unsigned grid, hipStream_t st) {
  if (D == 64)
    hipLaunchKernelGGL((kv_append_kernel<SRC, KV, 64>), dim3(grid), dim3(64), 0, st, p);
  else
    hipLaunchKernelGGL((kv_append_kernel<SRC, KV, 128>), dim3(grid), dim3(64), 0, st, p);
  return hipGetLastError();
}

}  // namespace pa_append

extern "C" pa_status pa_kv_append(const pa_shape* s, const void* k_new, const void* v_new,
                                  const int32_t* positions, const int32_t* block_table,
                                  pa_dtype src_dtype, pa_dtype kv_dtype, const float* k_scale,
                                  const float* v_scale, void* k_cache, void* v_cache,
                                  void* stream) {
  using namespace pa_append;
  unsigned grid = 0;
  const pa_status status = pa_host::append_status(s, k_new, v_new, positions, block_table, src_dtype,
                                                  kv_dtype, k_scale, v_scale, k_cache, v_cache, &grid);
  if (status != PA_OK) return status;
  if (grid == 0) return PA_OK;

  Params p;
  p.k_new = static_cast<const uint8_t*>(k_new);
  p.v_new = static_cast<const uint8_t*>(v_new);
  p.positions = positions;
  p.block_table = block_table;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.k_cache = static_cast<uint8_t*>(k_cache);
  p.v_cache = static_cast<uint8_t*>(v_cache);
  p.num_kv_heads = s->num_kv_heads;
  p.max_blocks_per_seq = s->max_blocks_per_seq;
  p.num_blocks = s->num_blocks;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int D = s->head_dim;
  hipError_t e;
  if (kv_dtype == PA_FP8_E4M3) {
    e = src_dtype == PA_F32   ? launch<F32, FP8>(D, p, grid, st)
        : src_dtype == PA_F16 ? launch<F16, FP8>(D, p, grid, st)
                              : launch<BF16, FP8>(D, p, grid, st);
  } else {
    e = src_dtype == PA_F32   ? launch<F32, F32>(D, p, grid, st)
        : src_dtype == PA_F16 ? launch<F16, F16>(D, p, grid, st)
                              : launch<BF16, BF16>(D, p, grid, st);
  }
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}
