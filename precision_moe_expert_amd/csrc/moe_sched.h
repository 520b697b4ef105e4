// Work scheduling shared by the grouped GEMMs: a chunk of active experts
// (Orbit announcement, 技术细节: router-selected experts grouped into
// fixed-size batches) becomes a device-built list of (expert, BM-row tile)
// entries; each work item is one tile times one N block.  The grid is
// persistent: every workgroup walks items with stride gridDim.x and exits
// when the chunk has none left, so the launch count never depends on data.
#pragma once
#include "common.h"
#include "kernels.h"

namespace moe {

struct ChunkWork {
  int a0, a1;    // active-expert index range of the chunk
  int t0;        // first tile of the chunk
  int ntiles;
  int nwork;
};

MOE_DEV bool chunk_work(const GemmArgs& p, int nblk, ChunkWork& cw) {
  if (p.chunk < 0) return false;
  const int na = *p.num_active;
  cw.a0 = p.chunk * p.chunk_experts;
  if (cw.a0 >= na) return false;
  cw.a1 = min(cw.a0 + p.chunk_experts, na);
  cw.t0 = p.tile_start[cw.a0];
  cw.ntiles = p.tile_start[cw.a1] - cw.t0;
  cw.nwork = cw.ntiles * nblk;
  return cw.nwork > 0;
}

struct Tile {
  int e;       // expert id
  int rbase;   // first permuted row
  int nrows;   // valid rows (1..BM)
  int nb;      // N block
  int a;       // index of the expert in the active list
};

// Item wk -> (tile, N block).  With tiles fastest, workgroups that run at
// the same time share an expert's weight slice; with N blocks fastest they
// share one tile of activation rows.  The host picks the order whose shared
// operand is the larger one.
MOE_DEV Tile tile_of(const GemmArgs& p, const ChunkWork& cw, int wk, int bm) {
  Tile t;
  const int nblk = cw.nwork / cw.ntiles;
  int tile;
  if (p.nb_fastest) {
    t.nb = wk % nblk;
    tile = cw.t0 + wk / nblk;
  } else {
    t.nb = wk / cw.ntiles;
    tile = cw.t0 + wk % cw.ntiles;
  }
  const i32x4 d = *reinterpret_cast<const i32x4*>(p.tiles + 4 * (int64_t)tile);
  t.e = d[0];
  t.rbase = d[1];
  t.nrows = d[2];
  t.a = d[3];
  (void)bm;
  return t;
}

// Workgroups are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8).
// Items are walked in rounds of gridDim.x; within a round of n items, XCD x
// takes the contiguous item range [x*per, (x+1)*per), per = ceil(n/8), so that
// neighbouring items (the row tiles of one expert, which read the same
// weights) share an L2.  Returns -1 for a block with nothing in this round.
// gridDim.x must be a multiple of 8.
MOE_DEV int xcd_item(int round_base, int nwork) {
  const int n = min((int)gridDim.x, nwork - round_base);
  const int per = (n + 7) >> 3;
  const int b = blockIdx.x;
  const int slot = (b & 7) * per + (b >> 3);
  return ((b >> 3) < per && slot < n) ? round_base + slot : -1;
}

}  // namespace moe
