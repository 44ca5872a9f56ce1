// Order of the (segment, n-tile, m-tile) tiles of a grouped GEMM launch.
//
// Segments are taken in order. Inside a segment the m-tiles go in groups of
// kTileGroupM; for each group, every n-tile in turn, and inside it the
// group's m-tiles. With the launch's XCD-contiguous mapping, the ~32 tiles
// that run together on one XCD then share both their activation rows (a
// group's m-tiles) and their weight rows (an n-tile) in that XCD's L2. A
// routed expert with 1..4 m-tiles is a single group: its m-tiles that share a
// weight tile are adjacent.
#pragma once
#include <stdint.h>

namespace moe {

constexpr int kTileGroupM = 4;

// Finds (segment, n-tile, m-tile) of logical tile L; sprefix[s] is the number
// of m-tiles before segment s. Returns false past the last tile.
__device__ __forceinline__ bool decode_tile(const int32_t* sprefix, int n_seg, int n_tiles, int L,
                                            int& seg, int& nt, int& mt) {
  const int total = sprefix[n_seg] * n_tiles;
  if (L >= total) return false;
  int lo = 0, hi = n_seg - 1;
  while (lo < hi) {                       // largest seg with sprefix[seg]*n_tiles <= L
    const int mid = (lo + hi + 1) >> 1;
    if (sprefix[mid] * n_tiles <= L) lo = mid; else hi = mid - 1;
  }
  seg = lo;
  const int local = L - sprefix[seg] * n_tiles;
  const int mte = sprefix[seg + 1] - sprefix[seg];
  const int span = kTileGroupM * n_tiles;           // tiles of one full group
  const int full = mte / kTileGroupM;
  const int g = local / span;
  const int gsize = g < full ? kTileGroupM : mte - full * kTileGroupM;
  const int rem = local - g * span;
  nt = rem / gsize;
  mt = g * kTileGroupM + (rem - nt * gsize);
  return true;
}

}  // namespace moe
