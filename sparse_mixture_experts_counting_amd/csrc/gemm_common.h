// Grouped-GEMM launch parameters and the device-side tile scheduler shared by the GEMM kernels.
//
// A grouped GEMM here is: for every group g (an expert) and every row r in [offsets[g],
// offsets[g+1]), C[r, n] = sum_k A[src(r), k] B_g[n, k] (+ epilogue), with B_g = B + g * b_gstride
// an [N][K] row-major matrix (K contiguous: the [out][in] layout of a linear layer's weight, the
// layout the weights are given in).  src(r) = gather[r] /
// gather_div when a gather list is given (token of assignment perm[r]), else r.  The group sizes
// live on the device (they come out of the dispatch kernels), so the grid is sized for an upper
// bound and every block finds its tile from `offsets` itself; blocks past the real tile count exit.
#pragma once

#include "common.h"

namespace moe {

struct GemmParams {
  const void* A;            // [a_rows][K], element type of the kernel
  int a_rows;               // rows of A (bounds of the gathered reads)
  const int32_t* gather;    // NULL: A row r; else A row gather[r] / gather_div
  int gather_div;
  const int32_t* offsets;   // [G+1] on the device, or NULL for one group of M rows
  int G;
  int M;                    // rows of the single group (offsets == NULL)
  int N, K;
  const void* B0;           // [G][N][K]
  const void* B1;           // second matrix for the fused SwiGLU epilogue (same layout) or NULL
  long long b_gstride;      // elements between consecutive groups' B
  void* C;                  // output rows, [rows][ldc]
  int ldc;
  const float* bias;        // fp32 [N] added by the fp32 epilogue, or NULL
  float* part;              // split-K scratch: [ksplit][NMAT][part_rows][N] fp32, or NULL
  int ksplit;               // K chunks (set by the launcher; 1 = no split)
  int part_rows;
  int slots;                // blocks resident at once; > 0 enables splitting the last partial
                            // round of tiles over K (set by the launcher)
  int lda, ldb;             // row strides of A and B in elements (0: K)
  // K-grouped mode (kgrouped = 1, with at = bt = 1): the groups split the reduction instead of
  // the rows.  Group g reduces over rows offsets[g] .. offsets[g+1] - 1 of A [K][lda] (M columns)
  // and B [K][ldb] (N columns) and writes its own C at C + g * c_gstride; every group has all M
  // output rows.  No gather, no split.
  int kgrouped;
  long long c_gstride;
  // SwiGLU-backward epilogue (EPI_SWIGLU_BWD, two matrices: a = A B0^T, b = A B1^T): reads
  // D = dh [rows][N], writes H = silu(a) * b [rows][N] and C [rows][ldc] with da in columns
  // [0, N) and db in [N, 2N): da = dh * b * silu'(a), db = dh * silu(a).  All bf16.
  const void* D;
  void* H;
  // EPI_STORE with D set (one group, no split): C = A B^T + D, D a bf16 [rows][ldd] addend, the
  // sum rounded to bf16 once.
  // Saved-activation epilogues.  EPI_SWIGLU_SAVE: as EPI_SWIGLU, and also stores the bf16 a and b
  // beside h in the same row of C (ldc >= 3N): h in columns [0, N), a in [N, 2N), b in [2N, 3N).
  // EPI_SWIGLU_BWD_SAVED (one matrix, the GEMM gives dh): reads a = D[row * ldd + col] and
  // b = D[row * ldd + N + col] and writes da, db into C as EPI_SWIGLU_BWD does.
  int ldd;
  // Transposed B (bt != 0; one matrix, bf16 output): B_g is stored [K][N] (row stride ldb, or N),
  // i.e. N-contiguous, as a linear layer's weight is for the products that reduce over its output
  // dimension.  With bt_k1 > 0, rows k < bt_k1 come from B0 and rows k >= bt_k1 from row
  // k - bt_k1 of B1 (two matrices stacked along K).
  int bt;
  int bt_k1;
  // Transposed A (at != 0, K-grouped only, with bt): A is stored [K][M] (row stride lda).
  int at;
  // Block-sparse launch with one block per CU (set by the launcher): 8 tile counters, one per
  // XCD, zeroed on the stream before the launch; NULL for one block per tile.
  int* tickets;
};

enum {
  EPI_SWIGLU = 0,
  EPI_STORE = 1,
  EPI_STORE_F32_BIAS = 2,
  EPI_SWIGLU_BWD = 3,
  EPI_SWIGLU_SAVE = 4,
  EPI_SWIGLU_BWD_SAVED = 5
};

// Epilogues whose GEMM carries two matrices (a and b) and writes h = silu(a) * b.
constexpr bool epi_swiglu(int epi) { return epi == EPI_SWIGLU || epi == EPI_SWIGLU_SAVE; }

struct TileCoord {
  int g;        // group
  int row0;     // first output row of the tile (global row index)
  int row_end;  // end of the group's rows
  int n_tile;   // column tile index
};

// Tile bookkeeping.  Tiles are ordered group by group; inside a group n-tile by n-tile, with the
// m-tiles of one n-tile consecutive (they share the same B tile).  scan_tiles counts them (each lane
// of the wave takes a slice of the groups), tile_at maps a tile index to its coordinates.
struct TileScan {
  int total;    // number of tiles
  int g0, g1;   // this lane's groups [g0, g1)
  int mine;     // tiles in this lane's groups
  int incl;     // tiles up to and including this lane's groups
};

// Rows [rs, re) of group g.
__device__ __forceinline__ void group_range(const GemmParams& p, int g, int& rs, int& re) {
  rs = p.offsets[g];
  re = p.offsets[g + 1];
}

template <int BM>
__device__ __forceinline__ TileScan scan_tiles(const GemmParams& p, int NT) {
  TileScan s;
  if (p.offsets == nullptr) {
    s.total = ((p.M + BM - 1) / BM) * NT;
    s.g0 = s.g1 = s.mine = s.incl = 0;
    return s;
  }
  const int lane = __lane_id();
  const int per = (p.G + 63) >> 6;
  s.g0 = min(p.G, lane * per);
  s.g1 = min(p.G, s.g0 + per);
  int mine = 0;
  for (int g = s.g0; g < s.g1; ++g) {
    int rs, re;
    group_range(p, g, rs, re);
    mine += ((re - rs + BM - 1) / BM) * NT;
  }
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  s.mine = mine;
  s.incl = incl;
  s.total = __shfl(incl, 63, 64);
  return s;
}

// Tile t (< s.total) -> coordinates.  Wave-uniform t.
template <int BM>
__device__ __forceinline__ void tile_at(const GemmParams& p, int NT, const TileScan& s, int t,
                                        TileCoord& tc) {
  if (p.offsets == nullptr) {
    const int tm = (p.M + BM - 1) / BM;
    tc.g = 0;
    tc.row0 = (t % tm) * BM;
    tc.n_tile = t / tm;
    tc.row_end = p.M;
    return;
  }
  const int lane = __lane_id();
  const int excl = s.incl - s.mine;
  const uint64_t own = __ballot(t >= excl && t < s.incl);
  const int owner = __ffsll((long long)own) - 1;
  int g_found = 0, base = 0;
  if (lane == owner) {
    base = excl;
    for (int g = s.g0; g < s.g1; ++g) {
      int rs, re;
      group_range(p, g, rs, re);
      const int c = ((re - rs + BM - 1) / BM) * NT;
      if (t < base + c) {
        g_found = g;
        break;
      }
      base += c;
    }
  }
  g_found = __shfl(g_found, owner, 64);
  base = __shfl(base, owner, 64);
  int rs, re;
  group_range(p, g_found, rs, re);
  const int tm = (re - rs + BM - 1) / BM;
  const int local = t - base;
  tc.g = g_found;
  tc.row0 = rs + (local % tm) * BM;
  tc.row_end = re;
  tc.n_tile = local / tm;
}

// Blocks are handed to the 8 XCDs round-robin (block b to XCD b % 8).  Give each XCD a contiguous
// run of the n tile indices, so that the m-tiles sharing a B tile also share that XCD's L2.
__device__ __forceinline__ int xcd_order(int bid, int n) {
  const int q = n >> 3, r = n & 7, x = bid & 7, i = bid >> 3;
  return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Blocks are handed to the 8 XCDs round-robin; in each whole round of `round` blocks (a multiple of
// 8: the blocks resident at once), XCD x takes the x-th chunk of round / 8 consecutive tiles of that
// round, so consecutive tiles (those sharing a weight panel) share an L2, and every XCD gets the
// same share of every part of the tile order (equal work when tile costs vary along the order).
// Blocks past the last whole round take tiles in index order.
__device__ __forceinline__ int xcd_round_order(int bid, int n, int round) {
  if (round < 8 || bid >= n / round * round) return bid;
  const int chunk = round >> 3, x = bid & 7, k = bid >> 3;
  return (k / chunk) * round + x * chunk + k % chunk;
}

// Map block `bid` to a tile in XCD order.  Returns false when bid is past the real tile count.
template <int BM>
__device__ __forceinline__ bool find_tile(const GemmParams& p, int NT, int bid, TileCoord& tc) {
  const TileScan s = scan_tiles<BM>(p, NT);
  if (bid >= s.total) return false;
  tile_at<BM>(p, NT, s, xcd_order(bid, s.total), tc);
  return true;
}

// Host-side upper bound on the number of tiles (for the grid size).
inline int tiles_upper_bound(int rows_max, int G, bool grouped, int BM, int NT) {
  const int tm = (rows_max + BM - 1) / BM + (grouped ? G : 0);
  return tm * NT;
}

}  // namespace moe
