// xcd_map.h -- workgroup -> tile mapping shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tide {

// Workgroup -> tile.  The dispatcher hands consecutive workgroup IDs to the
// 8 XCDs in turn; with one workgroup per tile, XCD x would get tiles x,
// x+8, x+16, ... .  Regrouping so that each XCD takes runs of kXcdGroup
// consecutive tiles keeps the tiles one XCD works on at a time (and so its
// L2 and the DRAM rows it opens) on neighbouring addresses.  Measured on
// the reduce-scatter: +5-7% at R = 16..64 and neutral at R = 8 (runs of 8
// against none), runs of 32 another +0.5-1% (runs of 128: -1.5% at R = 8);
// on the placement copy, runs of 32 against none: +1-5%.  The tail that does
// not fill whole groups keeps the identity mapping; a capped grid
// (workgroups striding over tiles) is left as is.
constexpr int kXcds = 8;
constexpr int kXcdGroup = 32;

__device__ __forceinline__ int64_t tile_of(int64_t b, int64_t ntiles) {
    if ((int64_t)gridDim.x != ntiles) return b;
    constexpr int64_t span = (int64_t)kXcds * kXcdGroup;
    const int64_t full = (ntiles / span) * span;
    if (b >= full) return b;
    const int64_t x = b % kXcds, i = b / kXcds;
    return (i / kXcdGroup) * span + x * kXcdGroup + (i % kXcdGroup);
}

}  // namespace tide
