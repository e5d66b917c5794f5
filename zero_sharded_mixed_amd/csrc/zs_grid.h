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

// Blocks resident per CU, capped through LDS.  A launch that reserves kTwoBlocksLds bytes of
// dynamic LDS per block (the kernels do not touch it) fits at most two of its blocks on a CU's
// 160 KB of LDS: two waves per SIMD for 256-thread blocks, whatever the register count allows.
// Measured on MI355X, the streams that interleave many arrays run faster with fewer waves in
// flight: Adam (4 read and 4 written arrays) 5-9% faster on the 7.5B, GPT-2 and Llama lists at
// two blocks per CU than at its register-bound 6-7 (one block: 5% slower, three: 0-2% faster);
// the reduce's one-group form (Nd >= 16 row streams) up to 5% faster than at three.  The
// copy-shaped pack and unpack are fastest at full occupancy (two blocks: 30-124% slower).
constexpr int64_t kLdsPerCu = 160 * 1024;
constexpr unsigned kTwoBlocksLds = 60 * 1024;
static_assert(2 * kTwoBlocksLds <= kLdsPerCu && 3 * kTwoBlocksLds > kLdsPerCu, "two blocks per CU");
static_assert(kTwoBlocksLds <= 64 * 1024, "within the default dynamic LDS limit of a block");

}  // namespace zs
