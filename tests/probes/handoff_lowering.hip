// Compiled (device code only, to assembly) by tests/test_handoff_lowering.py:
// the split-K hand-off helpers of the decode kernels next to the compiler's
// own release/acquire lowering at agent scope, so the test can compare the
// two instruction sequences. Never launched.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_tiles.h"

// The product's hand-off: partials stored with SC1, counted by
// last_to_finish, read back with SC1 by the last piece to finish.
__global__ void handoff_product(float* ws, uint32_t* cnt, float v, int n, float* out) {
  __shared__ int flag;
  const pa::brsrc r = pa::buffer_rsrc(ws, 4096);
  pa::st_agent4(r, threadIdx.x * 16, pa::f32x4{v, v, v, v});
  const int c = pa::last_to_finish(cnt, n, &flag);
  if (c == pa::kCountLast) {
    const pa::f32x4 x = pa::ld_agent4(r, (threadIdx.x ^ 1) * 16);
    out[threadIdx.x] = x[0] + x[3];
  }
}

// Reference: ordinary stores, then a release increment at agent scope.
__global__ void handoff_release(float* ws, uint32_t* cnt, float v) {
  ws[threadIdx.x] = v;
  __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Reference: an acquire increment at agent scope, then ordinary loads.
__global__ void handoff_acquire(float* ws, uint32_t* cnt, float* out) {
  const uint32_t c = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
  if (c == 7) out[threadIdx.x] = ws[threadIdx.x ^ 1];
}
