// Item walk shared by the kernels in which one workgroup per CU walks a list of work items
// (token, head group) as one stream of 64-entry index tiles (narrow_kernel.h, roles.hip):
// the item order and the slot ids of a tile. Internal linkage: every translation unit gets
// its own copy.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dkern.h"
#include "smla_internal.h"

namespace smla {
namespace {

using namespace dk;

constexpr int kWalkTile = 64;  // index entries per tile

// Work items of this workgroup: item k is u = blockIdx + k * grid of the list (token, head
// group); the items of a token are 8 apart, so they run on one XCD and share its L2.
struct NItem {
  int t, hg;
};
__device__ __forceinline__ NItem nitem_of(const KParams &p, int k) {
  const int u = (int)blockIdx.x + k * (int)gridDim.x;
  const int per = p.n_hg;
  const int full = (p.T >> 3) * 8 * per;
  NItem it;
  if (u < full) {
    const int s = u >> 3, grp = s / per;
    it.hg = s - grp * per;
    it.t = 8 * grp + (u & 7);
  } else {
    const int r = u - full, dt = r / per;
    it.hg = r - dt * per;
    it.t = (p.T & ~7) + dt;
  }
  return it;
}

// Position in the tile stream: item k (token t, head group hg), tile j of n_tiles.
struct NCur {
  int k, j, t, hg;
};
__device__ __forceinline__ NCur ncur_at(const KParams &p, int s) {
  const int k = s / p.n_tiles;
  const NItem it = nitem_of(p, k);
  return NCur{k, s - k * p.n_tiles, it.t, it.hg};
}
__device__ __forceinline__ void ncur_next(const KParams &p, NCur &c) {
  if (++c.j == p.n_tiles) {
    c.j = 0;
    ++c.k;
    const NItem it = nitem_of(p, c.k);
    c.t = it.t;
    c.hg = it.hg;
  }
}

// Checked slot id of entry e of tile j of token t (-1 when unused or past the stream).
__device__ __forceinline__ int32_t nslot_load(const KParams &p, const NCur &c, int e,
                                              bool live_tile) {
  const int tile = c.j;
  const bool main = tile < p.main_tiles;
  const int base = (main ? tile : tile - p.main_tiles) * kWalkTile;
  const int width = main ? p.topk : p.topk_extra;
  const int t = live_tile ? c.t : 0;
  const int32_t *row = main ? p.idx + (int64_t)t * p.idx_st : p.eidx + (int64_t)t * p.eidx_st;
  return *(gi32 *)(row + min(base + e, width - 1));
}
__device__ __forceinline__ int32_t nslot_check(const KParams &p, const NCur &c, int e,
                                               bool live_tile, int32_t s32) {
  const int tile = c.j;
  const bool main = tile < p.main_tiles;
  const int base = (main ? tile : tile - p.main_tiles) * kWalkTile;
  const int width = main ? p.topk : p.topk_extra;
  const int32_t *lens = main ? p.len : p.elen;
  const int live = lens ? min(max(*(ci32 *)(lens + (live_tile ? c.t : 0)), 0), width) : width;
  const int64_t nslots = main ? p.kv.num_slots : p.ex.num_slots;
  const bool ok = live_tile && base + e < live && s32 >= 0 && (int64_t)s32 < nslots;
  return ok ? s32 : -1;
}

}  // namespace
}  // namespace smla
