// Work-group -> output-tile mapping shared by the tiled kernel families.
//
// The C matrix is cut into tiles_m x tiles_n tiles, one work-group each.  On
// MI355X the hardware hands consecutive work-group ids to the eight XCDs in
// turn (id % 8), and each XCD has its own L2.  Two remaps make work-groups
// that run at the same time on one XCD share operand panels:
//   1. XCD remap: ids landing on XCD x become one contiguous range of the
//      linear tile order (a bijection on [0, n) for any n);
//   2. grouped order: the linear order walks `group` tile-rows down a column
//      before moving right, so the tiles resident on an XCD at once form a
//      compact block (few A row-panels and few B column-panels) instead of a
//      long strip of one tile-row.
// Where grid size matters is the subject of vidyal.ai Part 2 ("The CUDA
// Programming Model": occupancy and grid size); the XCD split is MI355X's own.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355gemm {

constexpr int kNumXcd = 8;

struct TileCoord {
    int64_t tm, tn;
};

__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t n)
{
    const int64_t q = n / kNumXcd, rem = n % kNumXcd;
    const int64_t x = b % kNumXcd, i = b / kNumXcd;
    return x * q + (x < rem ? x : rem) + i;
}

__device__ __forceinline__ TileCoord grouped_tile(int64_t lin, int64_t tiles_m, int64_t tiles_n,
                                                  int64_t group)
{
    const int64_t per_group = group * tiles_n;
    const int64_t gi = lin / per_group;
    const int64_t first = gi * group;
    const int64_t rows = (tiles_m - first) < group ? (tiles_m - first) : group;
    const int64_t in = lin - gi * per_group;
    return TileCoord{first + in % rows, in / rows};
}

__device__ __forceinline__ TileCoord map_tile(int64_t tiles_m, int64_t tiles_n, int64_t group)
{
    const int64_t n = tiles_m * tiles_n;
    return grouped_tile(xcd_remap(blockIdx.x, n), tiles_m, tiles_n, group);
}

// A batch of products in one grid: the XCD remap runs over all
// tiles x batch work-groups, then the linear index splits into the product
// and the tile inside it (grouped order within the product), so each XCD
// runs a contiguous range of (product, tile) pairs.  With batch = 1 this is
// map_tile.
struct BatchTile {
    int64_t b, tm, tn;
};

__device__ __forceinline__ BatchTile map_batch_tile(int64_t tiles_m, int64_t tiles_n,
                                                    int64_t batch, int64_t group)
{
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t lin = xcd_remap(blockIdx.x, tiles * batch);
    const int64_t b = lin / tiles;
    const TileCoord t = grouped_tile(lin - b * tiles, tiles_m, tiles_n, group);
    return BatchTile{b, t.tm, t.tn};
}

}  // namespace mi355gemm
