// zs_grid.h — grid sizing of the hot kernels (plain C++, no HIP types, so that host tests can
// compile it on its own).
#pragma once

#include <stdint.h>

namespace zs {

// Hot kernels launch one block per work item (a tile, or a tile of one row): on MI355X a
// one-shot grid with one 16-byte chunk per thread streams faster than a grid-stride loop.  The
// kernels still loop, so any grid size is correct.  A dispatch holds fewer than 2^32
// work-items per dimension, so grids are capped at 2^23 blocks of up to 256 threads (2^31
// work-items); larger work counts loop inside the kernels.
#ifndef ZS_GRID_CAP
#define ZS_GRID_CAP (int64_t(1) << 23)
#endif
inline int grid_for(int64_t work, int64_t cap = ZS_GRID_CAP) {
    return int(work < 1 ? 1 : (work < cap ? work : cap));
}

}  // namespace zs
