// Test-only probes of gfx950 building blocks the decode kernels rely on:
//  * the lane layout of the 16x16 MFMA operands and accumulator
//    (A: lane l holds row l%16, B: lane l holds column l%16, both with the
//    same per-lane k-slots; C: lane l holds rows 4*(l/16)+i of column l%16);
//  * exactness of the E4M3 -> f16 / bf16 conversion instructions;
//  * the lane pairs gfx950's v_permlane16_swap / v_permlane32_swap return
//    when both operands hold the same register (the row reductions use them).
// Each probe is one 64-thread workgroup over small, fully in-bounds buffers.
// pa_probe_schedule runs the balanced split's work-line arithmetic (the same
// header the kernel uses) on the host, so its coverage can be checked without
// a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_schedule.h"

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// which: 0 = f16 16x16x32, 1 = bf16 16x16x32, 2 = f16 16x16x16, 3 = bf16 16x16x16,
//        4 = f32 16x16x4.  A is [16][K] row-major, B is [K][16] row-major, both in
// the operand type (f32 for which 4); C is [16][16] f32.
__global__ void mfma_probe_kernel(int which, const void* A, const void* B, float* C) {
  const int l = threadIdx.x, r = l % 16, j = l / 16;
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
  if (which == 0 || which == 1) {
    const uint16_t* a = (const uint16_t*)A;
    const uint16_t* b = (const uint16_t*)B;
    uint16_t av[8], bv[8];
    for (int i = 0; i < 8; ++i) {
      av[i] = a[r * 32 + 8 * j + i];
      bv[i] = b[(8 * j + i) * 16 + r];
    }
    if (which == 0) {
      f16x8 x = __builtin_bit_cast(f16x8, av), y = __builtin_bit_cast(f16x8, bv);
      c = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, c, 0, 0, 0);
    } else {
      bf16x8 x = __builtin_bit_cast(bf16x8, av), y = __builtin_bit_cast(bf16x8, bv);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
    }
  } else if (which == 2 || which == 3) {
    const uint16_t* a = (const uint16_t*)A;
    const uint16_t* b = (const uint16_t*)B;
    uint16_t av[4], bv[4];
    for (int i = 0; i < 4; ++i) {
      av[i] = a[r * 16 + 4 * j + i];
      bv[i] = b[(4 * j + i) * 16 + r];
    }
    if (which == 2) {
      f16x4 x = __builtin_bit_cast(f16x4, av), y = __builtin_bit_cast(f16x4, bv);
      c = __builtin_amdgcn_mfma_f32_16x16x16f16(x, y, c, 0, 0, 0);
    } else {
      bf16x4 x = __builtin_bit_cast(bf16x4, av), y = __builtin_bit_cast(bf16x4, bv);
      c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(x, y, c, 0, 0, 0);
    }
  } else {
    const float* a = (const float*)A;
    const float* b = (const float*)B;
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r * 4 + j], b[j * 16 + r], c, 0, 0, 0);
  }
  for (int i = 0; i < 4; ++i) C[(4 * j + i) * 16 + r] = c[i];
}

// codes: 256 bytes (one dword = 4 codes per lane); out16/outb: 256 16-bit words.
__global__ void fp8_probe_kernel(const uint32_t* codes, uint32_t* out16, uint32_t* outb) {
  const int l = threadIdx.x;
  const uint32_t w = codes[l];
  f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  out16[2 * l] = __builtin_bit_cast(uint32_t, lo);
  out16[2 * l + 1] = __builtin_bit_cast(uint32_t, hi);
  bf16x2 blo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 bhi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  outb[2 * l] = __builtin_bit_cast(uint32_t, blo);
  outb[2 * l + 1] = __builtin_bit_cast(uint32_t, bhi);
}

// in: 64 words; out: 4 words per lane -- the two results of the 16-lane
// swap, then the two of the 32-lane swap, each with in[l] in both operands.
__global__ void permlane_probe_kernel(const uint32_t* in, uint32_t* out) {
  const int l = threadIdx.x;
  const uint32_t x = in[l];
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  out[4 * l + 0] = a[0];
  out[4 * l + 1] = a[1];
  out[4 * l + 2] = b[0];
  out[4 * l + 3] = b[1];
}

extern "C" int pa_probe_permlane(const void* in, void* out, void* stream) {
  hipLaunchKernelGGL(permlane_probe_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (const uint32_t*)in, (uint32_t*)out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int pa_probe_mfma(int which, const void* A, const void* B, float* C, void* stream) {
  if (which < 0 || which > 4) return 1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, which, A, B, C);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int pa_probe_fp8(const void* codes, void* out16, void* outb, void* stream) {
  hipLaunchKernelGGL(fp8_probe_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (const uint32_t*)codes, (uint32_t*)out16, (uint32_t*)outb);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Streaming-read ceiling: every 16-byte word of the buffer is read once, with
// non-temporal loads (the fastest plain read measured on MI355X); the XOR of
// everything is compared with a value it practically never takes, so the
// loads stay live while almost nothing is written.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ void stream_read_kernel(const u32x4* p, size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 a0 = {0u, 0u, 0u, 0u}, a1 = a0, a2 = a0, a3 = a0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    a0 ^= __builtin_nontemporal_load(p + i);
    a1 ^= __builtin_nontemporal_load(p + i + stride);
    a2 ^= __builtin_nontemporal_load(p + i + 2 * stride);
    a3 ^= __builtin_nontemporal_load(p + i + 3 * stride);
  }
  for (; i < n16; i += stride) a0 ^= __builtin_nontemporal_load(p + i);
  const u32x4 a = a0 ^ a1 ^ a2 ^ a3;
  const uint32_t x = a.x ^ a.y ^ a.z ^ a.w;
  if (x == 0x9E3779B9u) sink[0] = x;
}

extern "C" int pa_probe_stream_read(const void* p, size_t bytes, void* sink, int blocks,
                                    void* stream) {
  if (((uintptr_t)p & 15u) || blocks < 1) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)p, bytes / 16, (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Page-read floor: the same bytes a decode call reads, as whole pages at the
// given byte offsets (one chunk of chunk_kib KiB each, a multiple of 1 KiB),
// read with non-temporal 16-byte loads and nothing else done with them. Each
// workgroup of 8 waves takes a contiguous range of the chunk list; its waves
// interleave over the range with 4 chunks in flight each. The offsets must
// leave every chunk inside the buffer (checked by the caller).
template <int KB>
__global__ void __launch_bounds__(512) page_read_kernel(const uint8_t* base, const uint64_t* offs,
                                                        int nchunks, uint32_t* sink) {
  const int nw = blockDim.x / 64, w = threadIdx.x / 64, lane = threadIdx.x & 63;
  const int c0 = (int)((long long)blockIdx.x * nchunks / gridDim.x);
  const int c1 = (int)((long long)(blockIdx.x + 1) * nchunks / gridDim.x);
  u32x4 acc = {0u, 0u, 0u, 0u};
  int c = c0 + w;
  for (; c + 3 * nw < c1; c += 4 * nw) {
    u32x4 r[4][KB];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint8_t* p = base + offs[c + d * nw];
#pragma unroll
      for (int k = 0; k < KB; ++k) r[d][k] = __builtin_nontemporal_load((const u32x4*)(p + k * 1024) + lane);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int k = 0; k < KB; ++k) acc ^= r[d][k];
  }
  for (; c < c1; c += nw) {
    const uint8_t* p = base + offs[c];
#pragma unroll
    for (int k = 0; k < KB; ++k) acc ^= __builtin_nontemporal_load((const u32x4*)(p + k * 1024) + lane);
  }
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == 0x9E3779B9u) sink[0] = x;
}

extern "C" int pa_probe_page_read(const void* base, const uint64_t* offs, int nchunks, int chunk_kib,
                                  void* sink, int blocks, void* stream) {
  if (!base || !offs || nchunks < 1 || blocks < 1 || ((uintptr_t)base & 15u)) return 1;
  if (chunk_kib == 4)
    hipLaunchKernelGGL(page_read_kernel<4>, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                       (const uint8_t*)base, offs, nchunks, (uint32_t*)sink);
  else if (chunk_kib == 2)
    hipLaunchKernelGGL(page_read_kernel<2>, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                       (const uint8_t*)base, offs, nchunks, (uint32_t*)sink);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Host-side walk of every share of the balanced split. Writes one row of 8
// ints per piece -- share, sequence, KV head, first page, end page, piece
// index, pieces of the pair, slot of piece 0 -- up to max_rows rows, and
// returns the number of pieces (or -1 for bad arguments). The start of each
// share is found by a plain linear search over the sequences.
extern "C" int pa_probe_schedule(const int* lens, int B, int H, int max_blocks, int shares,
                                 int* rows, int max_rows) {
  if (!lens || B < 1 || H < 1 || max_blocks < 1 || shares < 1) return -1;
  long long total = 0;
  for (int b = 0; b < B; ++b) total += pa::line_pages(lens[b], max_blocks);
  if (total * H > 0x7fffffffLL) return -1;
  const int N = (int)total * H;
  const int S = pa::share_count(N, shares);
  int n = 0;
  for (int wg = 0; wg < S; ++wg) {
    const int x0 = pa::share_start(wg, N, S);
    const int x1 = pa::share_start(wg + 1, N, S);
    int b = 0, pre = 0;
    while (H * (pre + pa::line_pages(lens[b], max_blocks)) <= x0) {
      pre += pa::line_pages(lens[b], max_blocks);
      ++b;
    }
    pa::walk_share(
        wg, x0, x1, b, pre, B, H, N, S, max_blocks, [&](int bb) { return lens[bb]; },
        [&](int bb, int, const pa::LinePiece& p) {
          if (rows && n < max_rows) {
            int* r = rows + 8 * n;
            r[0] = wg; r[1] = bb; r[2] = p.g; r[3] = p.pg_lo;
            r[4] = p.pg_hi; r[5] = p.k; r[6] = p.nparts; r[7] = p.slot0;
          }
          ++n;
        });
  }
  return n;
}

// Host evaluation of the work line's exact division helper (pa_schedule.h),
// element by element: out[i] = floor_div(a[i], b[i]).
extern "C" void pa_probe_floor_div(const long long* a, const long long* b, int n, int* out) {
  for (int i = 0; i < n; ++i) out[i] = pa::floor_div(a[i], b[i]);
}

// Host evaluation of the balanced split's workgroup-to-share numbering
// (pa_schedule.h): out[blk] = share_of_block(blk, grid, s) for every
// workgroup of the grid.
extern "C" void pa_probe_share_of_block(int grid, int s, int* out) {
  for (int blk = 0; blk < grid; ++blk) out[blk] = pa::share_of_block(blk, grid, s);
}
