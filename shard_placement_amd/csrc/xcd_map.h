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
constexpr int64_t kXcdSpan = (int64_t)kXcds * kXcdGroup;

__device__ __forceinline__ int64_t tile_of(int64_t b, int64_t ntiles) {
    if ((int64_t)gridDim.x != ntiles) return b;
    const int64_t full = (ntiles / kXcdSpan) * kXcdSpan;
    if (b >= full) return b;
    const int64_t x = b % kXcds, i = b / kXcds;
    return (i / kXcdGroup) * kXcdSpan + x * kXcdGroup + (i % kXcdGroup);
}

// Skewed launches.  The odd-numbered XCDs of the MI355X run the same
// reduce-scatter workgroup 5-9% longer than the even-numbered ones (per-tile
// timing: 9.8 vs 9.2 us at R = 8, 18.3 vs 17.4 us at R = 16, 22.7 vs 20.9 us
// at R = 32; with the tile runs rotated by one XCD the odd XCDs stay the slow
// ones, so it is the XCD, not the data), and in a launch of several rounds
// of workgroups per CU the even XCDs run out of tiles first (1.0-1.7 us
// before the launch ends, against 0.5-0.6 us for the odd ones).  A skewed
// launch gives the even XCDs runs of kXcdGroup + kXcdSkew tiles per span
// and the odd ones kXcdGroup - kXcdSkew.  The dispatcher still hands every
// XCD the same number of workgroups, so each odd XCD's last workgroups get
// no tile (-1) and exit; tiles past the last full span take one workgroup
// each, in order.  Measured against the plain runs (same buffers, one
// process, interleaved, four processes on three boxes): +0.1..0.8% on the
// Llama layer (R = 8, 4096 tiles per launch) and +0.4..1.4% on the MoE
// layer with 2275-tile launches (R = 16; its default launches are now
// one-round launches of 1792 tiles, plan.cpp); a skew of 2 read -0.3% /
// +0.5%.  Launches of about
// one round of workgroups per CU (the R = 32 and R = 64 layers: every tile
// starts at once) gain nothing, so only launches of kSkewMinTiles or more
// are skewed.  The kernel reads the skew back from its grid size; the same
// mapping with the skew as a compile-time constant read 0.5-1% slower (the
// compiler's code for the tile loop differs), and so did the plain launches
// when they ran this form.  This form holds at most 7 workgroups per CU
// (92 scalar registers) where the plain one holds 8; holding plain launches
// to 7 per CU through LDS did not reproduce the gain.
constexpr int kXcdSkew = 1;
constexpr int64_t kSkewMinTiles = 8 * kXcdSpan;

__host__ __device__ constexpr int64_t skewed_grid(int64_t ntiles) {
    return (ntiles / kXcdSpan) * kXcds * (kXcdGroup + kXcdSkew) + ntiles % kXcdSpan;
}

// Loop bound of a kernel that may run a skewed grid (more workgroups than
// tiles).
__device__ __forceinline__ int64_t walk_end(int64_t ntiles) {
    return (int64_t)gridDim.x > ntiles ? (int64_t)gridDim.x : ntiles;
}

// Workgroup -> tile (or -1) for a grid of skewed_grid(ntiles) workgroups;
// a grid of ntiles workgroups maps as tile_of, a smaller one strides.  A
// grid larger than ntiles must be skewed_grid(ntiles) with ntiles >=
// kXcdSpan (the launch code only makes it for ntiles >= kSkewMinTiles).
__device__ __forceinline__ int64_t tile_of_skewed(int64_t b, int64_t ntiles) {
    const int64_t g = gridDim.x;
    if (g < ntiles) return b;
    const uint32_t full = (uint32_t)(ntiles / kXcdSpan);
    if (g == ntiles) {
        const int64_t fullt = (int64_t)full * kXcdSpan;
        if (b >= fullt) return b;
        const int64_t x = b % kXcds, i = b / kXcds;
        return (i / kXcdGroup) * kXcdSpan + x * kXcdGroup + (i % kXcdGroup);
    }
    const uint32_t rem = (uint32_t)(ntiles - (int64_t)full * kXcdSpan);
    const uint32_t head = (uint32_t)g - rem;  // workgroups of the full spans
    const uint32_t bb = (uint32_t)b;
    if (bb >= head) return (int64_t)full * kXcdSpan + (bb - head);
    const uint32_t skew = head / (kXcds * full) - kXcdGroup;
    const uint32_t x = bb % kXcds, i = bb / kXcds;
    const uint32_t len = (x & 1) ? kXcdGroup - skew : kXcdGroup + skew;
    const uint32_t q = i / len;
    if (q >= full) return -1;  // an odd XCD's spare workgroup
    const uint32_t start = (x >> 1) * 2 * kXcdGroup + (x & 1) * (kXcdGroup + skew);
    return (int64_t)q * kXcdSpan + start + i % len;
}

}  // namespace tide
