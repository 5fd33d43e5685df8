// fa_sched.h -- tile scheduler: maps the 1-D hardware workgroup id to a
// (query tile, batch*head) work item.
//
// The logical grid is the one the "Learning Metal with FlashAttention" page
// dispatches (section FlashAttention: one threadgroup per query tile, head
// and batch).  On MI355X the grid is launched 1-D and remapped here:
//
// * Workgroup i is dispatched to XCD i % 8 (eight XCDs, each with its own
//   L2).  When B*H is a multiple of 8, each XCD is given a contiguous group
//   of B*H/8 heads, so the K/V tiles of a head are shared through one L2.
// * Under causal masking the query tile t needs t+1 units of key work, so
//   the heaviest tiles are handed out first (longest-processing-time order)
//   to shorten the tail.
#pragma once

namespace fa {

struct TileSched {
  int n_qtiles;       // query tiles per (batch, head)
  int bh;             // B * H
  int heads_per_xcd;  // B*H / 8 when B*H % 8 == 0, else 0 (no XCD grouping)
  int heavy_first;    // 1: tile order n_qtiles-1 .. 0 (causal)
  int head_major;     // with XCD grouping: an XCD's items run head by head (else rank by rank across its heads)
};

__host__ inline TileSched make_sched(int n_qtiles, int bh, bool causal) {
  TileSched s;
  s.n_qtiles = n_qtiles;
  s.bh = bh;
  s.heads_per_xcd = (bh % 8 == 0) ? bh / 8 : 0;
  s.heavy_first = causal ? 1 : 0;
  s.head_major = 0;
  return s;
}

__device__ __forceinline__ void sched_item(const TileSched& s, int hw, int& qtile, int& bh) {
  int rank;
  if (s.heads_per_xcd > 0) {
    const int xcd = hw & 7, slot = hw >> 3;
    if (s.head_major) {
      rank = slot % s.n_qtiles;
      bh = xcd * s.heads_per_xcd + slot / s.n_qtiles;
    } else {
      rank = slot / s.heads_per_xcd;
      bh = xcd * s.heads_per_xcd + slot % s.heads_per_xcd;
    }
  } else {
    rank = hw / s.bh;
    bh = hw % s.bh;
  }
  qtile = s.heavy_first ? s.n_qtiles - 1 - rank : rank;
}

}  // namespace fa
