// Work line of the balanced split (host and device).
//
// Every (sequence b, KV head g) pair owns line_pages(L_b) consecutive
// positions of one work line, sequences in order and, inside a sequence, KV
// heads in order; position x of pair (b, g) stands for its page x - first.
// The line of N positions is cut into S shares, one per workgroup, share w
// being [w*N/S, (w+1)*N/S) (integer quotients), so every workgroup reads the
// same number of pages, give or take one, whatever the lengths are. A share
// boundary that falls inside a pair splits that pair into pieces; the pieces
// of a pair are merged by log-sum-exp, the same merge that combines split-K
// partitions ("RapidLLM", feature table, row "Decode context parallelism").
//
// Piece k of a pair keeps its partial result in workspace slot slot0 + k with
// slot0 = (first share of the pair) + (pair index b * H + g); slots of
// different pairs never overlap because a pair's last share is at most the
// next pair's first share, and every slot is below (shares) + B * H.
#ifndef PA_SCHEDULE_H
#define PA_SCHEDULE_H

namespace pa {

constexpr int kLineBlock = 16;   // tokens per page
constexpr int kMinSharePages = 8;   // two pages for each of a workgroup's four waves

// Line positions of one (sequence, KV head) pair: its cached pages, or one
// placeholder position for an empty or out-of-contract sequence (whose output
// is written without reading the cache).
__host__ __device__ inline int line_pages(int L, int max_blocks) {
  return (L <= 0 || L > max_blocks * kLineBlock) ? 1 : (L + kLineBlock - 1) / kLineBlock;
}

// Shares for n positions and at most `shares` workgroups: fewer when the line
// is short, so that a share holds at least kMinSharePages positions.
__host__ __device__ inline int share_count(int n, int shares) {
  const int most = n / kMinSharePages;
  const int s = shares < most ? shares : most;
  return s > 1 ? s : 1;
}

// floor(a / b) for 0 <= a < 2^53, 0 < b < 2^31 and a quotient below 2^31,
// through one correctly rounded double division instead of a 64-bit integer
// division (which the GPU has no instruction for: it expands into a long
// scalar routine). Exact: a / b = q + f/b with the integer q and 0 <= f < b,
// so rounding can only lift it to q + 1 if 1/b <= ulp(a / b) / 2 <=
// (a / b) * 2^-53, i.e. if a >= 2^53; every caller stays far below (a < 2^46).
__host__ __device__ inline int floor_div(long long a, long long b) {
  return (int)((double)a / (double)b);
}

// First line position of share w of s over n positions.
__host__ __device__ inline int share_start(int w, int n, int s) {
  return floor_div((long long)w * n, s);
}

// The share holding line position x: the largest w with share_start(w) <= x.
__host__ __device__ inline int share_of(int x, int n, int s) {
  return floor_div((long long)(x + 1) * s - 1, n);
}

// The share workgroup blk of a grid of `grid` takes when the line has s
// shares, or s for a workgroup left without one. Consecutive workgroups go to
// the eight XCDs in turn, so when grid is a multiple of 8 the shares are
// numbered XCD by XCD, ceil(s / 8) consecutive shares per XCD: neighbouring
// shares (which split a pair between them and hand its partial results over)
// share an XCD and its L2, and a short line still spreads over all eight.
__host__ __device__ inline int share_of_block(int blk, int grid, int s) {
  if (grid % 8 != 0) return blk < s ? blk : s;
  const int per_xcd = (s + 7) / 8;
  const int wg = blk / 8 < per_xcd ? (blk % 8) * per_xcd + blk / 8 : s;
  return wg < s ? wg : s;
}

struct LinePiece {
  int g;        // KV head
  int pg_lo;    // first page of the piece inside the sequence
  int pg_hi;    // one past its last page
  int k;        // index of the piece among the pieces of (b, g)
  int nparts;   // pieces of (b, g)
  int slot0;    // workspace slot of piece 0 of (b, g)
  int x_end;    // line position after the piece
};

// The piece that starts at line position x of share `wg` (which ends at x1),
// inside sequence b whose pairs start at line position seq_first and take
// cb positions each; H KV heads, n positions in s shares.
__host__ __device__ inline LinePiece line_piece(int x, int x1, int seq_first, int cb, int b, int H,
                                                int n, int s, int wg) {
  LinePiece p;
  const int rel = x - seq_first;
  p.g = floor_div(rel, cb);
  p.pg_lo = rel - p.g * cb;
  const int pair_first = seq_first + p.g * cb;
  const int pair_end = pair_first + cb;
  p.x_end = x1 < pair_end ? x1 : pair_end;
  p.pg_hi = p.pg_lo + (p.x_end - x);
  const int s_first = share_of(pair_first, n, s);
  const int s_last = share_of(pair_end - 1, n, s);
  p.k = wg - s_first;
  p.nparts = s_last - s_first + 1;
  p.slot0 = s_first + b * H + p.g;
  return p;
}

// Visit the pieces of share wg = [x0, x1) in line order, starting in sequence
// b whose pairs start at line position H * pre; B sequences, n positions in
// s shares. len(b) returns context_lens[b]; visit(b, L, piece) handles one
// piece. (b < B always holds when the start is right; the test only keeps a
// wrong start from reading past the batch.)
template <typename Len, typename Visit>
__host__ __device__ inline void walk_share(int wg, int x0, int x1, int b, int pre, int B, int H,
                                           int n, int s, int max_blocks, Len len, Visit visit) {
  int x = x0;
  while (x < x1 && b < B) {
    const int L = len(b);
    const int cb = line_pages(L, max_blocks);
    const int seq_first = H * pre;
    const LinePiece pc = line_piece(x, x1, seq_first, cb, b, H, n, s, wg);
    visit(b, L, pc);
    x = pc.x_end;
    if (x == seq_first + H * cb) {
      ++b;
      pre += cb;
    }
  }
}

}  // namespace pa

#endif  // PA_SCHEDULE_H
