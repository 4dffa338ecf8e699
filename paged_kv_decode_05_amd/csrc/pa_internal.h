// Entry points shared between the library's translation units (not exported).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <cmath>

#include "padecode.h"

namespace pa {

constexpr int kTileRows = 16;   // query rows one matrix-core tile holds

// Fixed partitions: up to kMergeFan partitions of a sequence are merged in
// one level; beyond that, groups of fan partitions first, fan being the
// smallest value >= kMergeFan with fan * fan >= p_max, so that neither level
// merges more than fan pieces. Returns 0 for one level.
constexpr int kMergeFan = 16;
inline int merge_fan(long long p_max) {
  if (p_max <= kMergeFan) return 0;
  long long f = (long long)std::sqrt((double)p_max);
  while (f * f < p_max) ++f;
  return (int)(f < kMergeFan ? kMergeFan : f);
}

// The decode kernels for q_len new tokens per sequence whose
// (new token, query head) rows fit one tile: group * q_len <= kTileRows.
// q_len = 1 is pa_decode itself; q and out are [batch][q_len][Hq][D] and new
// token t sees positions 0 .. L - q_len + t. Same argument rules, workspace
// contract and statuses as pa_decode.
size_t decode_workspace_bytes(const pa_shape* shape, int q_len);

// Workgroups of a balanced split on the current device (one per CU), or -1
// when the device cannot be queried.
int balanced_shares();
pa_status decode_call(const pa_shape* shape, int q_len, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_table,
                      const int32_t* context_lens, float scale, pa_dtype io_dtype,
                      pa_dtype kv_dtype, const float* k_scale, const float* v_scale,
                      void* workspace, size_t workspace_bytes, void* out, float* lse_out,
                      void* stream);

}  // namespace pa
