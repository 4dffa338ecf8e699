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

// ---------------------------------------------------------------------------
// Shared prefix ("Litellama", "Features", Prefix Caching: sequences whose
// prompts begin alike hold the same physical blocks for that beginning).
// With P shared pages, sequence b takes its first P_b = min(P, floor(L_b / 16))
// pages from the prefix and the rest, tokens 16 P_b .. L_b - 1, as its
// suffix; the suffixes form the work line above. The prefix is read once per
// pass: the batch's query rows are cut into 16-row tiles of 16 / G
// sequences, four tiles make a pass, and a unit u = g * passes + pass (KV
// head g) is the P prefix pages read for the pass's rows; units lie end to
// end on a prefix line of np positions cut into sp prefix shares, taken by
// the first sp workgroups, the suffix line by the next sn.
// A piece of a unit leaves one partial result per sequence of its pass in
// the slots of that sequence's pair: pair (b, g) owns slots slot0 .. slot0 +
// own + pp - 1 with slot0 = (first suffix share of the pair) + (b * H + g) *
// (1 + kPfxPieces), its own suffix pieces first (none for a pair without
// line positions), then the pp pieces of its unit; every slot is below
// sn + B * H * (1 + kPfxPieces).
// ---------------------------------------------------------------------------
constexpr int kPfxPieces = 8;   // pieces a unit is cut into, at most
// Weight of prefix work against suffix work in the share split.
constexpr int kPfxCostNum = 1, kPfxCostDen = 1;

struct PfxGeo {
  int P;        // shared pages read once (clamped to the longest sequence's full pages)
  int mpt;      // sequences per tile: 16 / G
  int ntile;    // tiles over the batch
  int passes;   // units per KV head
  int np;       // prefix line positions: H * passes * P
  int sp;       // prefix shares
  int r_star;   // the row the prefix block ids are read from (a longest sequence)
};

// The suffix length of a sequence of length L under P shared pages, or -1
// for a length outside 0 .. 16 * max_blocks (NaN rows).
__host__ __device__ inline int pfx_suffix(int P, int L, int max_blocks) {
  if (L < 0 || L > max_blocks * kLineBlock) return -1;
  const int pb = L / kLineBlock < P ? L / kLineBlock : P;
  return L - kLineBlock * pb;
}

// Line positions of a pair whose suffix has S tokens (-1: out of contract).
// With a prefix (P > 0) a suffix of at most one page takes none: the last
// piece of its prefix unit reads that page (its tail) for the sequence's
// rows, and an out-of-contract sequence gets its NaN rows from the prefix
// pieces, so short suffixes never become tiny pairs on the line. Without one
// it is the plain line's count (one placeholder for an empty or
// out-of-contract sequence).
__host__ __device__ inline int pfx_positions(int P, int S, int max_blocks) {
  if (P > 0 && S <= kLineBlock) return 0;
  return line_pages(S, max_blocks);
}
// 1 when the prefix pass reads the sequence's suffix as its tail page.
__host__ __device__ inline int pfx_tail(int P, int S) { return P > 0 && S > 0 && S <= kLineBlock ? 1 : 0; }

// Fill the prefix geometry for B sequences, H KV heads, G query heads per
// KV head (pg.P set), a suffix line of n positions and `grid` workgroups
// (at least 2): the shares are split between the prefix and the suffix line
// in proportion to their work, a suffix position being one page for one
// wave and a prefix position one page for each tile of its pass, of which a
// workgroup runs 4 / nt at once, with a share for every unit (up to an
// eighth of the grid); a unit stays within kPfxPieces pieces and no share of
// either line is empty. Returns sn, the suffix shares (sp + sn <=
// grid).
__host__ __device__ inline int pfx_split(PfxGeo& pg, int B, int H, int G, int n, int grid) {
  pg.mpt = 16 / G;
  pg.ntile = (B + pg.mpt - 1) / pg.mpt;
  pg.passes = (pg.ntile + 3) / 4;
  pg.np = H * pg.passes * pg.P;
  const int nt_last = pg.ntile - 4 * (pg.passes - 1);
  const int c_last = nt_last == 1 ? 1 : (nt_last == 2 ? 2 : 4);
  const long long wp = (long long)H * pg.P * (4LL * (pg.passes - 1) + c_last) * kPfxCostNum / kPfxCostDen;
  const long long tot = (long long)n + wp;
  const int st = share_count(tot < 0x7fffffffLL ? (int)tot : 0x7fffffff, grid);
  int sp = 0;
  if (pg.P > 0) {
    sp = floor_div(2LL * st * wp + tot, 2LL * tot);   // rounded share of the work
    // a unit of P positions meets at most ceil((P - 1) / len) + 1 shares of
    // len positions or more
    const int minlen = (pg.P - 1 + kPfxPieces - 2) / (kPfxPieces - 1);
    const int most = pg.np / (minlen > 1 ? minlen : 1);
    // a piece pays fixed costs (its ring's first pages, the merge of its
    // waves, a partial per sequence, the counting): one share per unit at
    // least, up to an eighth of the grid, so that no share runs many units
    // of a short prefix one after another
    const int units = H * pg.passes;
    const int least = units < grid / 8 ? units : grid / 8;
    sp = sp > least ? sp : least;
    sp = sp < most ? sp : most;
    sp = sp > grid - 1 ? grid - 1 : sp;
    sp = sp < 1 ? 1 : sp;
  }
  pg.sp = sp;
  // the suffix line keeps at least kMinSharePages positions per share, so no
  // share is empty (a pair counts every share its pages span as a piece)
  const int fit = share_count(n, grid - sp);
  const int sn = st - sp < fit ? st - sp : fit;
  return sn > 1 ? sn : 1;
}

// Own pieces and first slot of pair index `pair` = b * H + g whose suffix
// takes cb positions from line position `first` of a suffix line of n
// positions in s shares (a pair without positions: no own pieces, slots
// after every share's).
struct PfxSlots {
  int own, slot0;
};
__host__ __device__ inline PfxSlots pfx_slots(int first, int cb, int pair, int n, int s) {
  const int s_first = first < n ? share_of(first, n, s) : s;
  const int own = cb > 0 ? share_of(first + cb - 1, n, s) - s_first + 1 : 0;
  return PfxSlots{own, s_first + pair * (1 + kPfxPieces)};
}

// Pieces of unit u (0 without a prefix).
__host__ __device__ inline int pfx_pieces(const PfxGeo& pg, int u) {
  if (pg.P == 0) return 0;
  return share_of(u * pg.P + pg.P - 1, pg.np, pg.sp) - share_of(u * pg.P, pg.np, pg.sp) + 1;
}
// The unit holding pair (b, g)'s prefix rows.
__host__ __device__ inline int pfx_unit(const PfxGeo& pg, int b, int g) {
  return g * pg.passes + (b / pg.mpt) / 4;
}

}  // namespace pa

#endif  // PA_SCHEDULE_H
