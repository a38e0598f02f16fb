// Workgroup -> output tile mapping shared by the window-GEMM kernels.
//
// MI355X dispatches the workgroups of a 1-D grid round-robin over its 8 XCDs,
// each with a private L2. Giving every XCD a contiguous range of logical
// tiles keeps the tiles that share a window strip (all M tiles of one N tile,
// and neighbouring N tiles whose windows overlap) in the same L2. Inside the
// range the M index runs back and forth (a serpentine), so consecutive tiles
// also share their filter block: the parity-alternating traversal of
// "Enabling Memory-efficient Im2win Convolution ...", Algorithm 1 and
// Sec. III-E.3 (read with the reversed index gridDim - 1 - blockIdx, so that
// it stays inside the grid).
#pragma once

#include <hip/hip_runtime.h>

namespace im2win {

__device__ __forceinline__ void tile_coords(int b, int G, int tiles_m, int &tm, int &tn)
{
    const int per = G >> 3, rem = G & 7;
    const int x = b & 7, i = b >> 3;
    const int t = x * per + min(x, rem) + i;   // logical tile, contiguous per XCD
    tn = t / tiles_m;
    const int mm = t - tn * tiles_m;
    tm = (tn & 1) ? tiles_m - 1 - mm : mm;
}

}  // namespace im2win
