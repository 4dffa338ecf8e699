// The library's host code, built for the CPU alone with the address and
// undefined-behaviour sanitizers (g++, no HIP): the argument checks and
// workspace layouts of every entry point (csrc/pa_host.h), the balanced
// split's work line (csrc/pa_schedule.h) and the block pool
// (csrc/block_pool.cpp). Modes:
//   args            fixed cases with known statuses, the ones the C-ABI tests
//                   send to the library;
//   fuzz N SEED     N random shapes drawn around every limit; each layout is
//                   checked against 128-bit arithmetic of its own;
//   line N SEED     N random batches: the shares of the work line cover every
//                   position once, pieces and slots agree;
//   prefix N SEED   N random batches under a shared prefix: the prefix and
//                   suffix shares cover every page once, each pair's slots
//                   are its pieces', disjoint from every other pair's;
//   pool            block-pool operations read from stdin, one result line
//                   each (compared with the oracle's pool by the caller).
// Any failed check prints "FAIL ..." and exits 1; a sanitizer report aborts.
#define __host__
#define __device__

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "padecode.h"
#include "pa_host.h"
#include "pa_schedule.h"

typedef unsigned __int128 u128;
typedef __int128 i128;

static int g_fail = 0;
#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      printf("FAIL %s:%d %s | ", __FILE__, __LINE__, #cond); \
      printf(__VA_ARGS__);                                 \
      printf("\n");                                        \
      if (++g_fail > 20) exit(1);                          \
    }                                                      \
  } while (0)

// splitmix64
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int64_t range(int64_t lo, int64_t hi) { return lo + (int64_t)(next() % (uint64_t)(hi - lo + 1)); }
  template <size_t N>
  int32_t pick(const int64_t (&v)[N]) {
    return (int32_t)v[next() % N];
  }
};

static const void* P(uintptr_t v) { return reinterpret_cast<const void*>(v); }
static const int32_t* PI(uintptr_t v) { return reinterpret_cast<const int32_t*>(v); }
static const float* PF(uintptr_t v) { return reinterpret_cast<const float*>(v); }
constexpr uintptr_t F = 1u << 20;   // an aligned non-null value; never dereferenced

static pa_shape base_shape() {
  pa_shape s;
  s.batch = 2;
  s.num_q_heads = 8;
  s.num_kv_heads = 2;
  s.head_dim = 128;
  s.block_size = 16;
  s.max_blocks_per_seq = 32;
  s.num_blocks = 100;
  s.partition_size = 0;
  return s;
}

// The decode entry point's host path up to the launch, shares given.
static pa_status decode_host(const pa_shape* s, int q_len, uintptr_t q, uintptr_t k, uintptr_t v,
                             uintptr_t bt, uintptr_t cl, int io, int kv, uintptr_t ks, uintptr_t vs,
                             uintptr_t ws, size_t wsb, uintptr_t out, uintptr_t lse, int shares = 256) {
  pa_status st = pa_host::decode_shape_status(s, q_len);
  if (st != PA_OK) return st;
  st = pa_host::io_args_status(P(q), P(k), P(v), PI(bt), PI(cl), (pa_dtype)io, (pa_dtype)kv, PF(ks),
                               PF(vs), P(out), PF(lse));
  if (st != PA_OK) return st;
  const pa_host::DecodeLayout w = pa_host::decode_layout(s, shares, q_len);
  return pa_host::workspace_status(s->partition_size, w.total, w.cnt_bytes, 0, P(ws), wsb);
}

static pa_status multi_host(const pa_shape* s, int q_len, uintptr_t q, int io, int kv, uintptr_t ks,
                            uintptr_t vs, uintptr_t ws, size_t wsb) {
  if (!s) return PA_ERR_NULL;
  if (pa_host::multi_fits_one_tile(s, q_len))
    return decode_host(s, q_len, q, F, F, F, F, io, kv, ks, vs, ws, wsb, F, 0);
  pa_host::MultiPlan p;
  const bool balanced = s->partition_size == PA_SPLIT_BALANCED;
  if (!pa_host::multi_plan(s, q_len, &p, balanced ? 256 : 0)) return PA_ERR_SHAPE;
  pa_status st = pa_host::io_args_status(P(q), P(F), P(F), PI(F), PI(F), (pa_dtype)io, (pa_dtype)kv,
                                         PF(ks), PF(vs), P(F), nullptr);
  if (st != PA_OK) return st;
  return pa_host::workspace_status(s->partition_size, p.total, 0, 0, P(ws), wsb);
}

static int mode_args() {
  pa_shape s = base_shape();
  // decode: nulls, shapes, dtypes, alignment, workspace
  CHECK(decode_host(nullptr, 1, F, F, F, F, F, 1, 1, 0, 0, 0, 0, F, 0) == PA_ERR_NULL, "null shape");
  CHECK(decode_host(&s, 1, 0, F, F, F, F, 1, 1, 0, 0, 0, 0, F, 0) == PA_ERR_NULL, "null q");
  CHECK(decode_host(&s, 1, F, F, F, F, 0, 1, 1, 0, 0, 0, 0, F, 0) == PA_ERR_NULL, "null lens");
  CHECK(decode_host(&s, 1, F, F, F, F, F, 1, 1, 0, 0, 0, 0, 0, 0) == PA_ERR_NULL, "null out");
  CHECK(decode_host(&s, 1, F, F, F, F, F, 1, 3, 0, 0, 0, 0, F, 0) == PA_ERR_NULL, "fp8 no scales");
  struct Bad { int32_t pa_shape::*f; int32_t v; };
  const Bad bad[] = {{&pa_shape::num_q_heads, 7},     {&pa_shape::head_dim, 96},
                     {&pa_shape::head_dim, 256},      {&pa_shape::block_size, 32},
                     {&pa_shape::partition_size, 24}, {&pa_shape::partition_size, -16},
                     {&pa_shape::partition_size, -2}, {&pa_shape::max_blocks_per_seq, 0},
                     {&pa_shape::num_blocks, 0},      {&pa_shape::batch, -1},
                     {&pa_shape::num_kv_heads, 0},    {&pa_shape::batch, 70000}};
  for (const Bad& b : bad) {
    pa_shape t = base_shape();
    t.*(b.f) = b.v;
    CHECK(decode_host(&t, 1, F, F, F, F, F, 1, 1, 0, 0, 0, 0, F, 0) == PA_ERR_SHAPE, "bad shape %d", b.v);
  }
  {
    pa_shape t = base_shape();
    t.num_q_heads = 40;   // group 20
    CHECK(decode_host(&t, 1, F, F, F, F, F, 1, 1, 0, 0, 0, 0, F, 0) == PA_ERR_SHAPE, "group 20");
    t = base_shape();
    t.partition_size = PA_SPLIT_BALANCED;
    t.batch = 4097;
    CHECK(decode_host(&t, 1, F, F, F, F, F, 1, 1, 0, 0, F, 1u << 30, F, 0) == PA_ERR_SHAPE, "bal batch");
    t.batch = 4096;
    t.num_q_heads = t.num_kv_heads = 64;
    t.max_blocks_per_seq = 1 << 13;
    CHECK(decode_host(&t, 1, F, F, F, F, F, 1, 1, 0, 0, F, 1u << 30, F, 0) == PA_ERR_SHAPE, "bal line");
  }
  CHECK(decode_host(&s, 1, F, F, F, F, F, 0, 3, F, F, 0, 0, F, 0) == PA_ERR_DTYPE, "fp8 f32 io");
  CHECK(decode_host(&s, 1, F, F, F, F, F, 1, 2, 0, 0, 0, 0, F, 0) == PA_ERR_DTYPE, "f16/bf16");
  CHECK(decode_host(&s, 1, F, F, F, F, F, 3, 3, F, F, 0, 0, F, 0) == PA_ERR_DTYPE, "fp8 io");
  CHECK(decode_host(&s, 1, F, F, F, F, F, 7, 7, 0, 0, 0, 0, F, 0) == PA_ERR_DTYPE, "dtype 7");
  CHECK(decode_host(&s, 1, F + 8, F, F, F, F, 1, 1, 0, 0, 0, 0, F, 0) == PA_ERR_ALIGN, "q align");
  CHECK(decode_host(&s, 1, F, F, F, F, F, 1, 1, 0, 0, 0, 0, F + 2, 0) == PA_ERR_ALIGN, "out align");
  CHECK(decode_host(&s, 1, F, F, F, F + 2, F, 1, 1, 0, 0, 0, 0, F, 0) == PA_ERR_ALIGN, "table align");
  CHECK(decode_host(&s, 1, F, F, F, F, F, 1, 1, 0, 0, 0, 0, F, F + 2) == PA_ERR_ALIGN, "lse align");
  {
    pa_shape t = base_shape();
    t.partition_size = 512;
    const size_t need = pa_host::decode_layout(&t, 0, 1).total;
    CHECK(decode_host(&t, 1, F, F, F, F, F, 1, 1, 0, 0, 0, 0, F, 0) == PA_ERR_WORKSPACE, "no ws");
    CHECK(decode_host(&t, 1, F, F, F, F, F, 1, 1, 0, 0, F, need - 1, F, 0) == PA_ERR_WORKSPACE, "small");
    CHECK(decode_host(&t, 1, F, F, F, F, F, 1, 1, 0, 0, F + 16, need, F, 0) == PA_ERR_ALIGN, "ws align");
    CHECK(decode_host(&t, 1, F, F, F, F, F, 1, 1, 0, 0, F, need, F, 0) == PA_OK, "ws ok");
    // the workspace sizes the C-ABI tests state: B32 Hq28 Hkv4 D128, 8 partitions
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    t = base_shape();
    t.batch = 32;
    t.num_q_heads = 28;
    t.num_kv_heads = 4;
    t.max_blocks_per_seq = 256;
    t.partition_size = 512;
    CHECK(pa_host::decode_layout(&t, 0, 1).total ==
              up(32 * 28 * 8 * 128 * 4) + up(32 * 28 * 8 * 4) + up(32 * 4 * 4), "ws size B32");
    t = base_shape();
    t.partition_size = 16;   // 32 partitions: fan 16, 2 groups
    const size_t rows = 2 * 2 * (32 + 2) * 4;
    CHECK(pa_host::decode_layout(&t, 0, 1).total == up(2 * 2 * 3 * 4) + up(rows * 128 * 4) + up(rows * 4),
          "ws size two-level");
    t = base_shape();
    t.batch = 1;
    t.num_kv_heads = 1;
    t.max_blocks_per_seq = 8192;
    t.partition_size = 16;   // 8192 partitions: fan 91
    const pa_host::DecodeLayout w = pa_host::decode_layout(&t, 0, 1);
    CHECK(w.fan == 91 && w.g_max == 91, "fan %d groups %d", w.fan, w.g_max);
    // the no-allocation scratch's counter region: refused past it
    CHECK(pa_host::workspace_status(16, 100, 300, 256, P(F), 1000) == PA_ERR_SCRATCH, "scratch cnt");
    CHECK(pa_host::workspace_status(16, 2000, 100, 256, P(F), 1000) == PA_ERR_SCRATCH, "scratch size");
  }
  // multi-token
  CHECK(multi_host(nullptr, 4, F, 1, 1, 0, 0, 0, 0) == PA_ERR_NULL, "multi null");
  for (int T : {0, 17, -1}) CHECK(multi_host(&s, T, F, 1, 1, 0, 0, 0, 0) == PA_ERR_SHAPE, "multi T %d", T);
  {
    pa_shape t = base_shape();
    t.partition_size = PA_SPLIT_BALANCED;
    CHECK(multi_host(&t, 5, F, 1, 1, 0, 0, 0, 0) == PA_ERR_WORKSPACE, "multi balanced wide");
    t.batch = 4097;
    CHECK(multi_host(&t, 5, F, 1, 1, 0, 0, 0, 0) == PA_ERR_SHAPE, "multi balanced batch");
    t = base_shape();
    t.partition_size = 24;
    CHECK(multi_host(&t, 4, F, 1, 1, 0, 0, 0, 0) == PA_ERR_SHAPE, "multi ps24");
    t = base_shape();
    t.num_q_heads = 40;
    CHECK(multi_host(&t, 4, F, 1, 1, 0, 0, 0, 0) == PA_ERR_SHAPE, "multi G20");
  }
  CHECK(multi_host(&s, 4, F, 0, 3, F, F, 0, 0) == PA_ERR_DTYPE, "multi fp8 f32");
  CHECK(multi_host(&s, 4, F, 1, 3, 0, 0, 0, 0) == PA_ERR_NULL, "multi fp8 no scales");
  CHECK(multi_host(&s, 4, F + 8, 1, 1, 0, 0, 0, 0) == PA_ERR_ALIGN, "multi q align");
  {
    pa_shape t = base_shape();
    t.partition_size = 512;
    pa_host::MultiPlan p;
    CHECK(pa_host::multi_plan(&t, 4, &p), "plan");
    CHECK(multi_host(&t, 4, F, 1, 1, 0, 0, 0, 0) == PA_ERR_WORKSPACE, "multi no ws");
    CHECK(multi_host(&t, 4, F, 1, 1, 0, 0, F, p.total - 1) == PA_ERR_WORKSPACE, "multi small ws");
    CHECK(multi_host(&t, 4, F, 1, 1, 0, 0, F + 16, p.total) == PA_ERR_ALIGN, "multi ws align");
  }
  // append
  unsigned grid = 0;
  auto app = [&](const pa_shape* t, uintptr_t kn, uintptr_t pos, uintptr_t kc, int src, int kv,
                 uintptr_t ks) {
    return pa_host::append_status(t, P(kn), P(F), PI(pos), PI(F), (pa_dtype)src, (pa_dtype)kv, PF(ks),
                                  PF(ks), P(kc), P(F), &grid);
  };
  CHECK(app(nullptr, F, F, F, 1, 1, 0) == PA_ERR_NULL, "append null");
  CHECK(app(&s, 0, F, F, 1, 1, 0) == PA_ERR_NULL, "append null k");
  CHECK(app(&s, F, F, F, 1, 3, 0) == PA_ERR_NULL, "append fp8 no scales");
  {
    pa_shape t = base_shape();
    t.head_dim = 96;
    CHECK(app(&t, F, F, F, 1, 1, 0) == PA_ERR_SHAPE, "append D96");
    t = base_shape();
    t.block_size = 8;
    CHECK(app(&t, F, F, F, 1, 1, 0) == PA_ERR_SHAPE, "append bs8");
    t = base_shape();
    t.batch = 0;
    CHECK(app(&t, F, F, F, 1, 1, 0) == PA_OK && grid == 0, "append empty");
  }
  CHECK(app(&s, F, F, F, 1, 2, 0) == PA_ERR_DTYPE, "append f16 to bf16");
  CHECK(app(&s, F, F, F, 3, 3, F) == PA_ERR_DTYPE, "append fp8 rows");
  CHECK(app(&s, F + 1, F, F, 1, 1, 0) == PA_ERR_ALIGN, "append kn align");
  CHECK(app(&s, F, F, F + 8, 1, 1, 0) == PA_ERR_ALIGN, "append cache align");
  CHECK(app(&s, F, F + 2, F, 1, 1, 0) == PA_ERR_ALIGN, "append pos align");
  CHECK(app(&s, F, F, F, 1, 1, 0) == PA_OK && grid == 4, "append ok");
  // log-sum-exp merge
  auto mrg = [&](int n, int rows, int hd, uintptr_t so, uintptr_t sl, int dt, uintptr_t o) {
    return pa_host::merge_status(n, rows, hd, P(so), PF(sl), (pa_dtype)dt, P(o), nullptr, &grid);
  };
  CHECK(mrg(0, 4, 128, F, F, 1, F) == PA_ERR_SHAPE, "merge no shards");
  CHECK(mrg(2, -1, 128, F, F, 1, F) == PA_ERR_SHAPE, "merge rows");
  CHECK(mrg(2, 4, 6, F, F, 1, F) == PA_ERR_SHAPE, "merge hd%%4");
  CHECK(mrg(2, 4, 2048, F, F, 1, F) == PA_ERR_SHAPE, "merge hd big");
  CHECK(mrg(2, 4, 128, 0, F, 1, F) == PA_ERR_NULL, "merge null");
  CHECK(mrg(2, 4, 128, F, F, 3, F) == PA_ERR_DTYPE, "merge fp8");
  CHECK(mrg(2, 4, 128, F + 8, F, 1, F) == PA_ERR_ALIGN, "merge align");
  CHECK(mrg(2, 4, 128, F, F + 2, 1, F) == PA_ERR_ALIGN, "merge lse align");
  CHECK(mrg(2, 0, 128, F, F, 1, F) == PA_OK && grid == 0, "merge empty");
  CHECK(mrg(2, 0x7fffffff, 1024, F, F, 1, F) == PA_OK && grid == 0x7fffffffu + 0u, "merge max");
  // shared prefix: balanced split only, 0 <= prefix_blocks <= max_blocks_per_seq
  {
    pa_shape b = base_shape();
    b.partition_size = PA_SPLIT_BALANCED;
    CHECK(pa_host::prefix_shape_status(nullptr, 0) == PA_ERR_NULL, "prefix null");
    CHECK(pa_host::prefix_shape_status(&b, 0) == PA_OK && pa_host::prefix_shape_status(&b, 32) == PA_OK,
          "prefix ok");
    CHECK(pa_host::prefix_shape_status(&b, -1) == PA_ERR_SHAPE, "prefix negative");
    CHECK(pa_host::prefix_shape_status(&b, 33) == PA_ERR_SHAPE, "prefix beyond the table");
    pa_shape f = base_shape();
    f.partition_size = 512;
    CHECK(pa_host::prefix_shape_status(&f, 4) == PA_ERR_SHAPE, "prefix fixed partitions");
    CHECK(pa_host::prefix_shares_status(&b, 1) == PA_ERR_SHAPE && pa_host::prefix_shares_status(&b, 256) == PA_OK,
          "prefix shares");
    const pa_host::DecodeLayout w = pa_host::prefix_layout(&b, 256);
    const size_t slots = 256 + 4 * 9, rows = slots * 4;
    CHECK(w.cnt_bytes == 16 && w.o_off == 256 && w.lse_off == 256 + rows * 128 * 4 &&
              w.total == w.lse_off + (rows * 4 + 255) / 256 * 256,
          "prefix layout");
  }
  printf("args: %s\n", g_fail ? "FAILED" : "ok");
  return g_fail ? 1 : 0;
}

// A random shape around every limit the checks draw: a valid shape with
// fields near their limits, then, for half of the draws, one or two fields
// replaced by edge values (valid or not).
static pa_shape random_shape(Rng& r) {
  static const int64_t kB[] = {-1, 0, 1, 2, 3, 31, 32, 255, 4095, 4096, 4097, 65535, 65536, 0x7fffffff};
  static const int64_t kH[] = {-1, 0, 1, 2, 4, 8, 64, 65535, 65536, 0x7fffffff};
  static const int64_t kD[] = {64, 128, 64, 128, 0, 96, 256, -64};
  static const int64_t kBs[] = {16, 16, 16, 8, 32, 0};
  static const int64_t kMbs[] = {-1, 0, 1, 2, 256, 4096, 1 << 20, 1 << 26, (1 << 26) + 1, 0x7fffffff};
  static const int64_t kPs[] = {0, -1, -2, 16, 48, 256, 512, 8192, 1 << 30, 0x7ffffff0, 17, -16};
  static const int64_t kBig[] = {1, 2, 16, 255, 256, 4095, 4096, 65535};
  pa_shape s;
  // valid: sizes drawn log-uniformly so that products reach the int32 limits
  auto logu = [&](int bits) { return (int32_t)r.range(1 << 0, ((int64_t)1 << r.range(0, bits)) ); };
  s.batch = r.next() % 4 ? logu(16) : r.pick(kBig);
  if (s.batch > 65535) s.batch = 65535;
  s.num_kv_heads = r.next() % 4 ? logu(8) : r.pick(kBig);
  s.num_q_heads = s.num_kv_heads * (int32_t)r.range(1, 16);
  s.head_dim = r.next() % 2 ? 64 : 128;
  s.block_size = 16;
  s.max_blocks_per_seq = logu(26);
  s.num_blocks = (int32_t)r.range(1, 0x7fffffff);
  const int k = (int)(r.next() % 4);
  s.partition_size = k == 0 ? 0 : k == 1 ? PA_SPLIT_BALANCED : 16 * logu(20);
  if (s.partition_size == PA_SPLIT_BALANCED && r.next() % 2) s.batch = (int32_t)r.range(0, 4096);
  for (int n = (int)(r.next() % 2 ? 1 + r.next() % 2 : 0); n > 0; --n) {
    switch (r.next() % 9) {
      case 0: s.batch = r.next() % 2 ? r.pick(kB) : (int32_t)r.range(0, 70000); break;
      case 1: s.num_kv_heads = r.pick(kH); break;
      case 2: s.num_q_heads = r.next() % 2 ? (int32_t)r.range(-2, 300) : 0x7fffffff; break;
      case 3: s.head_dim = r.pick(kD); break;
      case 4: s.block_size = r.pick(kBs); break;
      case 5: s.max_blocks_per_seq = r.pick(kMbs); break;
      case 6: s.num_blocks = (int32_t)r.range(-1, 1); break;
      case 7: s.partition_size = r.pick(kPs); break;
      default: s.partition_size = (int32_t)(16 * r.range(0, 1 << 12)); break;
    }
  }
  return s;
}

static void check_layout(const pa_shape& s, int q_len, int shares) {
  const pa_host::DecodeLayout w = pa_host::decode_layout(&s, shares, q_len);
  if (s.partition_size == 0) {
    CHECK(w.total == 0 && w.p_max == 1, "one pass needs no workspace");
    return;
  }
  const u128 nbg = (u128)s.batch * s.num_kv_heads;
  u128 slots;
  if (s.partition_size == PA_SPLIT_BALANCED) {
    slots = (u128)shares + nbg;
    CHECK(slots <= 0x7fffffffu, "balanced slots fit int32");
  } else {
    const i128 tokens = (i128)s.max_blocks_per_seq * 16;
    const i128 p = (tokens + s.partition_size - 1) / s.partition_size;
    CHECK(p == w.p_max && p >= 1, "partitions %d", w.p_max);
    if (p <= 16) {
      CHECK(w.fan == 0 && w.g_max == 0, "one merge level");
    } else {
      CHECK(w.fan >= 16 && (i128)w.fan * w.fan >= p, "fan covers");
      CHECK(w.fan == 16 || (i128)(w.fan - 1) * (w.fan - 1) < p, "fan smallest");
      CHECK((i128)w.g_max * w.fan >= p && (i128)(w.g_max - 1) * w.fan < p, "groups");
    }
    slots = nbg * (u128)(w.p_max + w.g_max);
    CHECK(slots <= 0x7fffffffu, "slots fit int32");
    CHECK(nbg * (u128)w.p_max <= 0x7fffffffu, "grid fits");
    CHECK(pa_host::decode_grid(&s, w, shares) == (unsigned)(nbg * (u128)w.p_max), "grid");
  }
  const u128 rows = slots * (u128)(s.num_q_heads / s.num_kv_heads) * (u128)q_len;
  auto up = [](u128 x) { return (x + 255) / 256 * 256; };
  const u128 cnt = nbg * (1 + (u128)w.g_max) * 4;
  const u128 o = up(cnt), lse = o + up(rows * s.head_dim * 4), total = lse + up(rows * 4);
  CHECK(w.cnt_off == 0 && (u128)w.cnt_bytes == cnt, "counters");
  CHECK((u128)w.o_off == o && (u128)w.lse_off == lse && (u128)w.total == total, "layout");
  CHECK(w.o_off % 256 == 0 && w.lse_off % 256 == 0 && w.total % 256 == 0, "aligned regions");
  CHECK(total < ((u128)1 << 62), "total");
}

static int mode_fuzz(long n, uint64_t seed) {
  Rng r{seed};
  long ok_decode = 0, ok_multi = 0, ok_append = 0;
  for (long i = 0; i < n && !g_fail; ++i) {
    const pa_shape s = random_shape(r);
    const int q_len = r.next() % 4 ? (int)r.range(1, 17) : (int)r.range(-2, 40);
    const int shares = (int)r.range(1, 3 * 4096);
    const pa_status st = pa_host::decode_shape_status(&s, q_len);
    if (st == PA_OK) {
      ++ok_decode;
      const int G = s.num_q_heads / s.num_kv_heads;
      CHECK(G >= 1 && G <= 16 && G * q_len <= 16, "group %d q_len %d", G, q_len);
      CHECK((i128)s.batch * q_len * s.num_q_heads <= 0x7fffffff, "rows fit");
      if (s.partition_size == PA_SPLIT_BALANCED) {
        CHECK(s.batch <= 4096, "balanced batch");
        CHECK((i128)s.batch * s.num_kv_heads * s.max_blocks_per_seq + shares < 0x7fffffff, "line");
      }
      check_layout(s, q_len, shares);
      // the no-allocation scratch layout: partials after a fixed counter region
      if (s.partition_size > 0) {
        const pa_host::DecodeLayout w = pa_host::decode_layout(&s, 0, 1, PA_NOALLOC_COUNTER_BYTES);
        CHECK(w.o_off == PA_NOALLOC_COUNTER_BYTES && w.lse_off >= w.o_off && w.total >= w.lse_off,
              "scratch layout");
        const pa_status ws = pa_host::workspace_status(s.partition_size, w.total, w.cnt_bytes,
                                                       PA_NOALLOC_COUNTER_BYTES, P(F), PA_NOALLOC_SCRATCH_BYTES);
        CHECK((ws == PA_OK) == (w.cnt_bytes <= PA_NOALLOC_COUNTER_BYTES && w.total <= PA_NOALLOC_SCRATCH_BYTES),
              "scratch refusal");
      }
    } else {
      CHECK(st == PA_ERR_SHAPE, "status %d", st);
    }
    pa_host::MultiPlan p;
    const int msh = s.partition_size == PA_SPLIT_BALANCED ? shares : 0;
    if (pa_host::multi_plan(&s, q_len, &p, msh) && s.partition_size == PA_SPLIT_BALANCED) {
      ++ok_multi;
      const u128 nbg = (u128)s.batch * s.num_kv_heads;
      const u128 slots = (u128)shares + nbg;
      auto up = [](u128 x) { return (x + 255) / 256 * 256; };
      CHECK(s.batch <= 4096 && slots <= 0x7fffffffu, "balanced plan limits");
      CHECK((u128)p.o_off == up(nbg * 4) && (u128)p.lse_off == p.o_off + up(slots * p.rows * s.head_dim * 4) &&
                (u128)p.total == p.lse_off + up(slots * p.rows * 4),
            "balanced plan layout");
      CHECK(pa_host::multi_grid(&s, p) == (unsigned)shares, "balanced grid");
    } else if (pa_host::multi_plan(&s, q_len, &p, msh)) {
      ++ok_multi;
      const int G = s.num_q_heads / s.num_kv_heads;
      CHECK(p.rows == G * q_len && p.tiles * 16 >= p.rows && p.chunks * 2 >= p.tiles, "plan rows");
      const u128 units = (u128)s.batch * s.num_kv_heads * p.chunks * p.p_max;
      CHECK(units <= 0x7fffffffu && pa_host::multi_grid(&s, p) == (unsigned)units, "plan grid");
      if (s.partition_size) {
        const u128 nbg = (u128)s.batch * s.num_kv_heads;
        const u128 slots = nbg * (u128)(p.p_max + p.g_max);
        auto up = [](u128 x) { return (x + 255) / 256 * 256; };
        const u128 o = up(nbg * (1 + (u128)p.g_max) * p.chunks * 4);
        const u128 lse = o + up(slots * p.rows * s.head_dim * 4);
        CHECK((u128)p.o_off == o && (u128)p.lse_off == lse && (u128)p.total == lse + up(slots * p.rows * 4),
              "plan layout");
      } else {
        CHECK(p.total == 0, "plan one pass");
      }
    }
    unsigned grid = 7;
    const int src = (int)r.range(0, 4), kv = (int)r.range(0, 4);
    const pa_status as = pa_host::append_status(&s, P(F), P(F), PI(F), PI(F), (pa_dtype)src, (pa_dtype)kv,
                                                PF(F), PF(F), P(F), P(F), &grid);
    if (as == PA_OK) {
      ++ok_append;
      CHECK((u128)grid == (u128)s.batch * s.num_kv_heads, "append grid");
    } else {
      CHECK(grid == 0, "append grid on error");
    }
    const int ns = (int)r.range(-1, 70000), rows = r.next() % 2 ? (int)r.next() : (int)r.range(-1, 1000);
    const int hd = (int)r.range(-4, 1100);
    const pa_status ms = pa_host::merge_status(ns, rows, hd, P(F), PF(F), PA_F16, P(F), nullptr, &grid);
    if (ms == PA_OK) CHECK((i128)grid * 256 >= (i128)rows * (hd / 4) && (i128)(grid)*256 < (i128)rows * (hd / 4) + 256,
                           "merge grid");
  }
  printf("fuzz: %ld shapes, %ld decode, %ld multi, %ld append accepted: %s\n", n, ok_decode, ok_multi,
         ok_append, g_fail ? "FAILED" : "ok");
  return g_fail ? 1 : 0;
}

// The balanced split's work line over a random batch: walking every share
// from the start the workgroup scan would give it visits each page of each
// (sequence, KV head) pair exactly once, piece k of a pair sits in share
// first + k, and slots stay below shares + pairs.
static int mode_line(long n, uint64_t seed) {
  Rng r{seed};
  long long pages = 0, pieces = 0;
  for (long it = 0; it < n && !g_fail; ++it) {
    const int B = (int)r.range(1, it % 10 == 0 ? 4096 : 40);
    const int H = (int)r.range(1, 8);
    const int mbs = (int)r.range(1, B > 40 ? 64 : 300);
    std::vector<int> L(B);
    for (int b = 0; b < B; ++b) {
      const int k = (int)(r.next() % 8);
      L[b] = k == 0 ? 0 : k == 1 ? (int)r.range(-3, 0) : k == 2 ? mbs * 16 + (int)r.range(1, 20)
                                                                  : (int)r.range(1, mbs * 16);
    }
    std::vector<long long> pre(B + 1, 0);
    for (int b = 0; b < B; ++b) pre[b + 1] = pre[b] + pa::line_pages(L[b], mbs);
    const long long N = pre[B] * H;
    CHECK(N < 0x7fffffff, "line length");
    const int grid = (int)r.range(1, 3 * 256);
    const int S = pa::share_count((int)N, grid);
    std::vector<std::vector<uint8_t>> seen(B);
    for (int b = 0; b < B; ++b) seen[b].assign((size_t)H * pa::line_pages(L[b], mbs), 0);
    std::vector<int> shares_seen(S, 0);
    for (int blk = 0; blk < grid; ++blk) {
      const int w = pa::share_of_block(blk, grid, S);
      if (w >= S) continue;
      CHECK(shares_seen[w] == 0, "share %d taken twice", w);
      shares_seen[w] = 1;
      const int x0 = pa::share_start(w, (int)N, S), x1 = pa::share_start(w + 1, (int)N, S);
      CHECK(x1 - x0 >= 8 || S == 1, "share size");
      int b = 0;
      while (b + 1 <= B && pre[b + 1] * H <= x0) ++b;   // the scan: sequence holding x0
      pa::walk_share(w, x0, x1, b, (int)pre[b], B, H, (int)N, S, mbs, [&](int bb) { return L[bb]; },
                     [&](int bb, int Lb, const pa::LinePiece& pc) {
                       const int cb = pa::line_pages(Lb, mbs);
                       CHECK(pc.g >= 0 && pc.g < H && pc.pg_lo >= 0 && pc.pg_hi <= cb && pc.pg_lo < pc.pg_hi,
                             "piece pages");
                       CHECK(pc.k >= 0 && pc.k < pc.nparts, "piece index");
                       ++pieces;
                       pages += pc.pg_hi - pc.pg_lo;
                       CHECK(pc.slot0 + pc.k < S + B * H, "slot");
                       for (int pg = pc.pg_lo; pg < pc.pg_hi; ++pg) {
                         uint8_t& v = seen[bb][(size_t)pc.g * cb + pg];
                         CHECK(v == 0, "page visited twice");
                         v = 1;
                       }
                     });
    }
    for (int w = 0; w < S; ++w) CHECK(shares_seen[w], "share %d never taken", w);
    for (int b = 0; b < B; ++b)
      for (uint8_t v : seen[b]) CHECK(v == 1, "page never visited (b %d)", b);
  }
  printf("line: %ld batches, %lld pieces, %lld pages: %s\n", n, pieces, pages, g_fail ? "FAILED" : "ok");
  return g_fail ? 1 : 0;
}

// The shared-prefix schedule over a random batch, walked the way the kernel
// walks it: the prefix shares cover every (unit, page) once and cut no unit
// into more than kPfxPieces pieces; the suffix shares cover every suffix page
// once; each pair's slots -- its own suffix pieces, then its unit's prefix
// pieces -- are the range slot0 .. slot0 + own + pp - 1, each used once, and
// no slot is used by two pieces or lies beyond sn + B * H * (1 + kPfxPieces).
static int mode_prefix(long n, uint64_t seed) {
  Rng r{seed};
  long long ppos = 0, spos = 0, skipped = 0;
  for (long it = 0; it < n && !g_fail; ++it) {
    const int B = (int)r.range(1, it % 10 == 0 ? 4096 : 40);
    const int H = (int)r.range(1, 8);
    const int G = (int)r.range(1, 16);
    const int mbs = (int)r.range(1, B > 40 ? 64 : 400);
    const int preq = r.next() % 4 ? (int)r.range(0, mbs) : (int)r.range(0, 3);
    pa_shape shp = base_shape();
    shp.batch = B;
    shp.num_kv_heads = H;
    shp.num_q_heads = G * H;
    shp.max_blocks_per_seq = mbs;
    shp.partition_size = PA_SPLIT_BALANCED;
    if (pa_host::prefix_shape_status(&shp, preq) != PA_OK) {
      ++skipped;
      continue;
    }
    std::vector<int> L(B);
    for (int b = 0; b < B; ++b) {
      const int k = (int)(r.next() % 8);
      L[b] = k == 0 ? 0
             : k == 1 ? (int)r.range(-3, -1)
             : k == 2 ? mbs * 16 + (int)r.range(1, 20)
             : k == 3 ? 16 * preq
             : k == 4 ? std::min(mbs * 16, 16 * preq + (int)r.range(1, 40))
                      : (int)r.range(1, mbs * 16);
    }
    // the kernel's scan: the longest in-contract length, lowest index first
    int lmax = -1, rstar = 0;
    for (int b = 0; b < B; ++b)
      if (L[b] >= 0 && L[b] <= mbs * 16 && L[b] > lmax) {
        lmax = L[b];
        rstar = b;
      }
    pa::PfxGeo pg{};
    pg.P = lmax >= 0 ? std::min(preq, lmax / 16) : 0;
    pg.r_star = rstar;
    CHECK(pg.P == 0 || (pg.P * 16 <= L[rstar] && L[rstar] <= mbs * 16), "prefix pages of the read row");
    std::vector<int> S(B);
    std::vector<long long> pre(B + 1, 0);
    for (int b = 0; b < B; ++b) {
      S[b] = pa::pfx_suffix(pg.P, L[b], mbs);
      const bool in = L[b] >= 0 && L[b] <= mbs * 16;
      CHECK(in ? (S[b] >= 0 && (L[b] - S[b]) % 16 == 0 && (L[b] - S[b]) / 16 == std::min(pg.P, L[b] / 16))
               : S[b] == -1,
            "suffix of %d", L[b]);
      pre[b + 1] = pre[b] + pa::pfx_positions(pg.P, S[b], mbs);
      CHECK(pa::pfx_positions(pg.P, S[b], mbs) == (pg.P > 0 && S[b] <= 16 ? 0 : pa::line_pages(S[b], mbs)),
            "positions");
    }
    const long long N = pre[B] * H;
    const int grid = (int)r.range(2, 3 * 256);
    const int sn = pa::pfx_split(pg, B, H, G, (int)N, grid);
    const int sp = pg.sp;
    CHECK(sn >= 1 && sp + sn <= grid, "shares %d + %d of %d", sp, sn, grid);
    CHECK((sp > 0) == (pg.P > 0), "prefix shares %d with P %d", sp, pg.P);
    CHECK(pg.mpt == 16 / G && pg.ntile * pg.mpt >= B && (pg.ntile - 1) * pg.mpt < B, "tiles");
    CHECK(pg.passes * 4 >= pg.ntile && (pg.passes - 1) * 4 < pg.ntile, "passes");
    const int units = H * pg.passes;
    CHECK((long long)pg.np == (long long)units * pg.P, "prefix line");
    for (int u = 0; u < units && pg.P > 0; ++u)
      CHECK(pa::pfx_pieces(pg, u) >= 1 && pa::pfx_pieces(pg, u) <= pa::kPfxPieces, "unit %d pieces %d", u,
            pa::pfx_pieces(pg, u));
    const long long nslots = (long long)sn + (long long)B * H * (1 + pa::kPfxPieces);
    std::vector<uint8_t> used((size_t)nslots, 0);
    auto own_of = [&](int b, int g, int* slot0) {
      const int cb = pa::pfx_positions(pg.P, S[b], mbs);
      const pa::PfxSlots ps = pa::pfx_slots((int)(H * pre[b]) + g * cb, cb, b * H + g, (int)N, sn);
      *slot0 = ps.slot0;
      return ps.own;
    };
    auto use = [&](long long slot) {
      CHECK(slot >= 0 && slot < nslots, "slot %lld of %lld", slot, nslots);
      if (slot >= 0 && slot < nslots) {
        CHECK(used[(size_t)slot] == 0, "slot %lld used twice", slot);
        used[(size_t)slot] = 1;
      }
    };
    // prefix shares; the last piece of a unit reads its sequences' tails
    std::vector<uint8_t> pseen((size_t)pg.np, 0);
    std::vector<int> tail_seen((size_t)B * H, 0);
    for (int k = 0; k < sp; ++k) {
      const int x1 = pa::share_start(k + 1, pg.np, sp);
      int x = pa::share_start(k, pg.np, sp);
      while (x < x1) {
        const int u = x / pg.P, p_lo = x - u * pg.P, p_hi = std::min(pg.P, x1 - u * pg.P);
        CHECK(p_lo < p_hi, "empty prefix piece");
        for (int p = p_lo; p < p_hi; ++p) {
          uint8_t& v = pseen[(size_t)u * pg.P + p];
          CHECK(v == 0, "prefix position visited twice");
          v = 1;
        }
        ppos += p_hi - p_lo;
        const int kk = k - pa::share_of(u * pg.P, pg.np, sp);
        CHECK(kk >= 0 && kk < pa::pfx_pieces(pg, u), "piece %d of unit %d", kk, u);
        const int g = u / pg.passes, pass = u - g * pg.passes;
        const int b0 = 4 * pass * pg.mpt, nseq = std::min(4 * pg.mpt, B - b0);
        CHECK(nseq >= 1 && nseq <= 64, "sequences of a pass %d", nseq);
        for (int b = b0; b < b0 + nseq; ++b) {
          CHECK(pa::pfx_unit(pg, b, g) == u, "unit of (%d, %d)", b, g);
          int slot0;
          const int own = own_of(b, g, &slot0);
          use((long long)slot0 + own + kk);
          if (kk == pa::pfx_pieces(pg, u) - 1 && pa::pfx_tail(pg.P, S[b])) ++tail_seen[(size_t)b * H + g];
        }
        x = u * pg.P + p_hi;
      }
    }
    for (uint8_t v : pseen) CHECK(v == 1, "prefix position never visited");
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < H; ++g)
        CHECK(tail_seen[(size_t)b * H + g] == pa::pfx_tail(pg.P, S[b]), "tail of (%d, %d) read %d times", b, g,
              tail_seen[(size_t)b * H + g]);
    // the sequence holding suffix-line position x: the largest b with
    // H * pre[b] <= x (sequences without positions share their successor's
    // start and are passed over)
    auto seq_at = [&](int x) {
      int b = 0;
      while (b + 1 < B && pre[b + 1] * H <= x) ++b;
      return b;
    };
    // suffix shares, walked piece by piece as the waves of the kernel do
    std::vector<std::vector<uint8_t>> seen(B);
    for (int b = 0; b < B; ++b) seen[b].assign((size_t)H * pa::pfx_positions(pg.P, S[b], mbs), 0);
    for (int w = 0; w < sn; ++w) {
      const int x0 = pa::share_start(w, (int)N, sn), x1 = pa::share_start(w + 1, (int)N, sn);
      int x = x0;
      while (x < x1) {
        const int bb = seq_at(x);
        const int cb = pa::pfx_positions(pg.P, S[bb], mbs);
        CHECK(cb > 0, "position %d in a sequence without positions", x);
        if (cb <= 0) break;
        const int g = (x - (int)(H * pre[bb])) / cb;
        const int first = (int)(H * pre[bb]) + g * cb, end = first + cb;
        const int x_end = std::min(x1, end);
        int slot0;
        const int own = own_of(bb, g, &slot0);
        const int k = w - pa::share_of(first, (int)N, sn);
        CHECK(k >= 0 && k < own, "own piece %d of %d", k, own);
        use((long long)slot0 + k);
        spos += x_end - x;
        for (int q = x - first; q < x_end - first; ++q) {
          uint8_t& v = seen[bb][(size_t)g * cb + q];
          CHECK(v == 0, "suffix page visited twice");
          v = 1;
        }
        x = x_end;
      }
    }
    for (int b = 0; b < B; ++b)
      for (uint8_t v : seen[b]) CHECK(v == 1, "suffix page never visited (b %d)", b);
    // the pairs wholly inside a quarter of a suffix share (their partial is
    // stored by the wave and counted by the workgroup afterwards) are the
    // contiguous range of pair indices the kernel computes from the
    // quarter's ends
    auto pair_at = [&](int x, int* first, int* end) {
      const int b = seq_at(x);
      const int cb = pa::pfx_positions(pg.P, S[b], mbs);
      const int sf = (int)(H * pre[b]);
      const int g = (x - sf) / cb;
      *first = sf + g * cb;
      *end = *first + cb;
      return b * H + g;
    };
    for (int w = 0; w < sn && B <= 64; ++w) {
      const int x0 = pa::share_start(w, (int)N, sn), x1 = pa::share_start(w + 1, (int)N, sn);
      for (int q = 0; q < 4; ++q) {
        const int y0 = x0 + pa::share_start(q, x1 - x0, 4), y1 = x0 + pa::share_start(q + 1, x1 - x0, 4);
        if (y0 >= y1) continue;
        int f0, e0, f1, e1;
        int lo = pair_at(y0, &f0, &e0);
        if (f0 < y0) ++lo;
        int hi = pair_at(y1 - 1, &f1, &e1) + 1;
        if (e1 > y1) --hi;
        for (int b = 0; b < B; ++b)
          for (int g = 0; g < H; ++g) {
            const int cb = pa::pfx_positions(pg.P, S[b], mbs);
            const long long first = H * pre[b] + (long long)g * cb;
            const bool inside = cb > 0 && first >= y0 && first + cb <= y1;
            const int pi = b * H + g;
            // the kernel skips pairs without positions inside the range
            CHECK(inside == (pi >= lo && pi < hi && cb > 0), "direct range of quarter [%d, %d): pair %d", y0,
                  y1, pi);
          }
      }
    }
    // each pair's slots are exactly its own and its unit's pieces, contiguous
    long long expect = 0;
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < H; ++g) {
        int slot0;
        const int parts = own_of(b, g, &slot0) + pa::pfx_pieces(pg, pa::pfx_unit(pg, b, g));
        expect += parts;
        for (int j = 0; j < parts; ++j)
          CHECK(slot0 + j < nslots && used[(size_t)(slot0 + j)] == 1, "pair (%d, %d) slot %d unused", b, g, j);
      }
    long long total = 0;
    for (uint8_t v : used) total += v;
    CHECK(total == expect, "slots used %lld, pieces %lld", total, expect);
  }
  printf("prefix: %ld batches (%lld outside the limits), %lld prefix and %lld suffix positions: %s\n", n,
         skipped, ppos, spos, g_fail ? "FAILED" : "ok");
  return g_fail ? 1 : 0;
}

// Block-pool script: one operation per line, one result line each.
//   C nb seed | A sid n tok... | P sid tok | F sid | N | T pad mbs k sid... | S k sid... | D
static int mode_pool() {
  pa_block_pool* pool = nullptr;
  char op[4];
  while (scanf("%3s", op) == 1) {
    if (op[0] == 'C') {
      int nb;
      unsigned long long seed;
      if (scanf("%d %llu", &nb, &seed) != 2) return 2;
      if (pool) pa_pool_destroy(pool);
      pool = nullptr;
      printf("C %d\n", (int)pa_pool_create(nb, seed, &pool));
    } else if (op[0] == 'A') {
      long long sid;
      int n;
      if (scanf("%lld %d", &sid, &n) != 2 || n < 0) return 2;
      std::vector<int32_t> t(n);
      for (int i = 0; i < n; ++i)
        if (scanf("%d", &t[i]) != 1) return 2;
      int32_t cached = -1;
      const pa_status st = pa_pool_add_sequence(pool, sid, n ? t.data() : nullptr, n, &cached);
      printf("A %d %d\n", (int)st, st == PA_OK ? cached : -1);
    } else if (op[0] == 'P') {
      long long sid;
      int tok;
      if (scanf("%lld %d", &sid, &tok) != 2) return 2;
      printf("P %d\n", (int)pa_pool_append_token(pool, sid, tok));
    } else if (op[0] == 'F') {
      long long sid;
      if (scanf("%lld", &sid) != 1) return 2;
      printf("F %d\n", (int)pa_pool_free_sequence(pool, sid));
    } else if (op[0] == 'N') {
      printf("N %d\n", pa_pool_num_free(pool));
    } else if (op[0] == 'T') {
      int pad, mbs, k;
      if (scanf("%d %d %d", &pad, &mbs, &k) != 3 || k < 0 || mbs < 0) return 2;
      std::vector<int64_t> ids(k);
      for (int i = 0; i < k; ++i) {
        long long v;
        if (scanf("%lld", &v) != 1) return 2;
        ids[i] = v;
      }
      std::vector<int32_t> table((size_t)k * mbs + 1, 12345), lens(k + 1, -1);
      const pa_status st = pa_pool_block_table(pool, k ? ids.data() : nullptr, k, mbs, pad, table.data(),
                                               lens.data());
      printf("T %d", (int)st);
      if (st == PA_OK) {
        for (size_t i = 0; i < (size_t)k * mbs; ++i) printf(" %d", table[i]);
        printf(" |");
        for (int i = 0; i < k; ++i) printf(" %d", lens[i]);
      }
      printf("\n");
    } else if (op[0] == 'S') {
      int k;
      if (scanf("%d", &k) != 1 || k < 0) return 2;
      std::vector<int64_t> ids(k + 1);
      for (int i = 0; i < k; ++i) {
        long long v;
        if (scanf("%lld", &v) != 1) return 2;
        ids[i] = v;
      }
      int32_t pb = -1;
      const pa_status st = pa_pool_shared_prefix(pool, k ? ids.data() : nullptr, k, &pb);
      printf("S %d %d\n", (int)st, st == PA_OK ? pb : -1);
    } else if (op[0] == 'D') {
      pa_pool_destroy(pool);
      pool = nullptr;
      printf("D\n");
    } else {
      return 2;
    }
  }
  // null arguments never touch memory
  int32_t c = 0;
  if (pa_pool_create(0, 1, &pool) != PA_ERR_SHAPE || pa_pool_create(4, 1, nullptr) != PA_ERR_NULL ||
      pa_pool_add_sequence(nullptr, 1, nullptr, 0, &c) != PA_ERR_NULL || pa_pool_num_free(nullptr) != -1 ||
      pa_pool_block_table(nullptr, nullptr, 0, 1, 0, nullptr, nullptr) != PA_ERR_NULL ||
      pa_pool_shared_prefix(nullptr, nullptr, 0, &c) != PA_ERR_NULL)
    printf("FAIL null pool arguments\n");
  pa_pool_destroy(nullptr);
  pa_pool_destroy(pool);
  return 0;
}

int main(int argc, char** argv) {
  if (argc < 2) {
    fprintf(stderr, "usage: %s args|fuzz N SEED|line N SEED|prefix N SEED|pool\n", argv[0]);
    return 2;
  }
  const std::string m = argv[1];
  const long n = argc > 2 ? atol(argv[2]) : 1000;
  const uint64_t seed = argc > 3 ? strtoull(argv[3], nullptr, 10) : 1;
  if (m == "args") return mode_args();
  if (m == "fuzz") return mode_fuzz(n, seed);
  if (m == "line") return mode_line(n, seed);
  if (m == "prefix") return mode_prefix(n, seed);
  if (m == "pool") return mode_pool();
  fprintf(stderr, "unknown mode %s\n", m.c_str());
  return 2;
}
