// ag.hip -- all-gather placement for gfx950: rank-major bf16 gathered
// buffer -> per-parameter full tensors, padding rows trimmed.
//
// TIDE-AG writes each rank's shard straight into the parameter's own tensor,
// with no separate copy-out pass (Abstract of "The Endgame of FSDP
// Communication", weekinpapers.com); the gathered buffer is rank-major: each
// rank's block contiguous, blocks in rank order (kongchang.com article,
// section "The Root of FSDP2 Communication Overhead").  On one GPU
// the delivery is the placement step itself: for param p and rank r the
// clamp(d0 - r*s, 0, s) valid rows of slot r land in rows [r*s, ...) of the
// full tensor; slot padding is never read.
//
// Two engines do it:
//   tide_ag_place       a compute kernel: one short-lived workgroup per tile
//                       of up to ag_tile elements (runs of consecutive tiles
//                       per XCD, as in the reduce-scatter); 16-byte loads and stores
//                       where the destination allows it (from a 2-byte-aligned
//                       source where the slot is shifted), 4-byte or 2-byte
//                       moves otherwise.
//   tide_ag_place_sdma  host-issued copies.  engine_only = 1: one 1-D copy
//                       per (param, rank) run with the no-compute-unit copy
//                       kind, executed by the DMA engines (the pages move and
//                       place data without compute units, same Abstract).
//                       engine_only = 0: one 2-D copy per param over the
//                       ranks whose shard is full plus a 1-D copy for the
//                       partial rank, which the runtime executes with a
//                       blit kernel on the compute units.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstring>
#include <vector>

#include "plan_format.h"
#include "tide.h"
#include "xcd_map.h"

using namespace tide;

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// All buffers are device global memory: global_* instead of flat_* accesses.
#define TIDE_GLOBAL __attribute__((address_space(1)))

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
    const TIDE_GLOBAL u32x4* g = (const TIDE_GLOBAL u32x4*)(p);
    if constexpr (NT)
        return __builtin_nontemporal_load(g);
    else
        return *g;
}

template <bool NT>
__device__ __forceinline__ void st16(uint16_t* p, u32x4 v) {
    TIDE_GLOBAL u32x4* g = (TIDE_GLOBAL u32x4*)(p);
    if constexpr (NT)
        __builtin_nontemporal_store(v, g);
    else
        *g = v;
}

constexpr int kUnroll = 4;  // 16-byte vectors in flight per lane

template <bool NTL, bool NTS>
__device__ __forceinline__ void copy_vec16(const uint16_t* __restrict__ src,
                                           uint16_t* __restrict__ dst, int len) {
    constexpr int kStep = kBlock * kVec;  // elements per wave-group pass
    for (int base = 0; base < len; base += kStep * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int e = base + u * kStep + threadIdx.x * kVec;
            if (e < len) v[u] = ld16<NTL>(src + e);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int e = base + u * kStep + threadIdx.x * kVec;
            if (e < len) st16<NTS>(dst + e, v[u]);
        }
    }
}

// 4-byte moves (the two ends agree in 4-byte but not 16-byte phase): kNarrow
// words in flight per lane before any store, each instruction of a wave
// covering one contiguous run (4.9 TB/s on a misaligned layer vs 4.0 for a
// plain loop).
constexpr int kNarrow = 8;

template <typename T>
__device__ __forceinline__ void copy_narrow(const T* __restrict__ src, T* __restrict__ dst,
                                            int n) {
    const TIDE_GLOBAL T* s = (const TIDE_GLOBAL T*)(src);
    TIDE_GLOBAL T* d = (TIDE_GLOBAL T*)(dst);
    for (int base = 0; base < n; base += kBlock * kNarrow) {
        T v[kNarrow];
#pragma unroll
        for (int u = 0; u < kNarrow; ++u) {
            const int e = base + u * kBlock + threadIdx.x;
            if (e < n) v[u] = s[e];
        }
#pragma unroll
        for (int u = 0; u < kNarrow; ++u) {
            const int e = base + u * kBlock + threadIdx.x;
            if (e < n) d[e] = v[u];
        }
    }
}

__device__ __forceinline__ void copy_vec4(const uint16_t* __restrict__ src,
                                          uint16_t* __restrict__ dst, int len) {
    copy_narrow<uint32_t>(reinterpret_cast<const uint32_t*>(src),
                          reinterpret_cast<uint32_t*>(dst), len / 2);
}

// 2-byte moves: a plain strided loop measured faster than the batched form
// (4.8 vs 2.6 TB/s for a whole misaligned layer).
__device__ __forceinline__ void copy_scalar(const uint16_t* __restrict__ src,
                                            uint16_t* __restrict__ dst, int len) {
    const TIDE_GLOBAL uint16_t* s = (const TIDE_GLOBAL uint16_t*)(src);
    TIDE_GLOBAL uint16_t* d = (TIDE_GLOBAL uint16_t*)(dst);
    for (int e = threadIdx.x; e < len; e += kBlock) d[e] = s[e];
}

// Realigning copy: the destination is 16-byte aligned, the source is only
// 2-byte aligned.  gfx9 global loads take any address under the unaligned
// access mode the ROCm runtime sets, so each lane loads its 16 source bytes
// straight from the shifted address: a wave's load covers 1 KB + 2 bytes
// (nine 128-byte lines instead of eight) and its store one aligned 1 KB
// run.  Measured on a layer whose slots are all shifted by 2 bytes: 5.8-5.9
// TB/s, against 5.5-5.6 for two aligned loads per lane funnelled into
// place and 4.9 for 4-byte moves.  No byte outside the tile is read.
typedef unsigned int u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));

template <bool NT>
__device__ __forceinline__ u32x4 ld16_a2(const uint16_t* p) {
    const TIDE_GLOBAL u32x4_a2* g = (const TIDE_GLOBAL u32x4_a2*)(p);
    if constexpr (NT)
        return __builtin_nontemporal_load(g);
    else
        return *g;
}

template <bool NTL, bool NTS>
__device__ __forceinline__ void copy_shift(const uint16_t* __restrict__ src,
                                           uint16_t* __restrict__ dst, int len) {
    constexpr int kStep = kBlock * kVec;
    for (int base = 0; base < len; base += kStep * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int e = base + u * kStep + threadIdx.x * kVec;
            if (e < len) v[u] = ld16_a2<NTL>(src + e);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int e = base + u * kStep + threadIdx.x * kVec;
            if (e < len) st16<NTS>(dst + e, v[u]);
        }
    }
}

template <bool NTL, bool NTS>
__global__ __launch_bounds__(kBlock) void ag_kernel(const AgTile* __restrict__ tiles,
                                                    int64_t ntiles,
                                                    const uint16_t* __restrict__ gathered,
                                                    const uint64_t* __restrict__ full) {
    for (int64_t b = blockIdx.x; b < ntiles; b += gridDim.x) {
        const AgTile tile = tiles[tile_of(b, ntiles)];
        const uint16_t* src = gathered + tile.src;
        uint16_t* dst = reinterpret_cast<uint16_t*>(full[tile.p]) + tile.dst;
        if (tile.kind == kAgVec16)
            copy_vec16<NTL, NTS>(src, dst, tile.len);
        else if (tile.kind == kAgVec4)
            copy_vec4(src, dst, tile.len);
        else if (tile.kind == kAgShift)
            copy_shift<NTL, NTS>(src, dst, tile.len);
        else
            copy_scalar(src, dst, tile.len);
    }
}

typedef void (*AgKernel)(const AgTile*, int64_t, const uint16_t*, const uint64_t*);

AgKernel pick(uint32_t flags) {
    const bool ntl = flags & kFlagNtLoads, nts = flags & kFlagNtStores;
    if (ntl && nts) return ag_kernel<true, true>;
    if (ntl) return ag_kernel<true, false>;
    if (nts) return ag_kernel<false, true>;
    return ag_kernel<false, false>;
}

}  // namespace

extern "C" tide_status tide_ag_place(const void* h_plan, const void* d_plan,
                                     int32_t max_workgroups, tide_stream_t stream) {
    if (!h_plan || !d_plan) return TIDE_EINVAL;
    PlanHeader h;
    std::memcpy(&h, h_plan, sizeof h);
    if (h.magic != kMagic || h.version != kVersion) return TIDE_EPLAN;
    if (max_workgroups < 0) return TIDE_EINVAL;
    if (!h.has_ag) return TIDE_EUNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(d_plan) % 16) return TIDE_EALIGN;
    if (h.n_ag_tiles == 0) return TIDE_OK;

    const uint8_t* d = static_cast<const uint8_t*>(d_plan);
    const AgTile* all = reinterpret_cast<const AgTile*>(d + h.off_ag);
    const uint64_t* full = reinterpret_cast<const uint64_t*>(d + h.off_full);
    const uint16_t* gathered = reinterpret_cast<const uint16_t*>(h.gathered);
    AgKernel k = pick(h.flags);
    const int64_t per_launch = h.ag_launch_tiles > 0 ? h.ag_launch_tiles : h.n_ag_tiles;

    for (int64_t b = 0; b < h.n_ag_tiles; b += per_launch) {
        const AgTile* tiles = all + b;
        int64_t ntiles = per_launch < h.n_ag_tiles - b ? per_launch : h.n_ag_tiles - b;
        int64_t grid = ntiles;
        if (max_workgroups > 0 && grid > max_workgroups) grid = max_workgroups;
        if (grid > INT_MAX) grid = INT_MAX;
        void* args[] = {&tiles, &ntiles, &gathered, &full};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(k), dim3((unsigned)grid),
                                       dim3(kBlock), args, 0, reinterpret_cast<hipStream_t>(stream));
        if (e != hipSuccess) return TIDE_EHIP;
    }
    return TIDE_OK;
}

extern "C" tide_status tide_ag_place_sdma(const void* h_plan, int32_t engine_only,
                                          tide_stream_t stream) {
    if (!h_plan) return TIDE_EINVAL;
    PlanHeader h;
    std::memcpy(&h, h_plan, sizeof h);
    if (h.magic != kMagic || h.version != kVersion) return TIDE_EPLAN;
    if (engine_only != 0 && engine_only != 1) return TIDE_EINVAL;
    if (!h.has_ag) return TIDE_EUNSUPPORTED;
    const uint8_t* b = static_cast<const uint8_t*>(h_plan);
    const ParamDesc* ps = reinterpret_cast<const ParamDesc*>(b + h.off_params);
    const uint64_t* full = reinterpret_cast<const uint64_t*>(b + h.off_full);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const char* g = reinterpret_cast<const char*>(h.gathered);
    for (int32_t p = 0; p < h.P; ++p) {
        ParamDesc d;
        std::memcpy(&d, ps + p, sizeof d);
        if (d.n == 0) continue;
        char* dst = reinterpret_cast<char*>(full[p]);
        const int64_t nfull = d.d0 / d.s;        // ranks whose shard has s valid rows
        const int64_t rest = d.n - nfull * d.m;  // elements of the one partial rank
        if (engine_only) {
            // One 1-D copy per (param, rank) run of the runtime's no-compute-
            // unit copy kind, which the runtime normally gives to the DMA
            // engines (a 2-D copy of the same kind is always executed by a
            // blit kernel, and 1-D ones have been seen to be too).
            const int64_t nruns = nfull + (rest > 0 ? 1 : 0);
            for (int64_t r = 0; r < nruns && r < h.R; ++r) {
                const int64_t cnt = r < nfull ? d.m : rest;
                hipError_t e = hipMemcpyAsync(dst + 2 * r * d.m, g + 2 * (r * h.S + d.off),
                                              (size_t)(2 * cnt), hipMemcpyDeviceToDeviceNoCU, s);
                if (e != hipSuccess) return TIDE_EHIP;
            }
            continue;
        }
        if (nfull > 0) {
            hipError_t e = hipMemcpy2DAsync(dst, (size_t)(2 * d.m), g + 2 * d.off, (size_t)(2 * h.S),
                                            (size_t)(2 * d.m), (size_t)nfull,
                                            hipMemcpyDeviceToDevice, s);
            if (e != hipSuccess) return TIDE_EHIP;
        }
        if (rest > 0 && nfull < h.R) {
            hipError_t e = hipMemcpyAsync(dst + 2 * nfull * d.m, g + 2 * (nfull * h.S + d.off),
                                          (size_t)(2 * rest), hipMemcpyDeviceToDevice, s);
            if (e != hipSuccess) return TIDE_EHIP;
        }
    }
    return TIDE_OK;
}

extern "C" tide_status tide_ag_place_sdma_streams(const void* h_plan, const tide_stream_t* streams,
                                                  int32_t n_streams) {
    if (!h_plan || !streams || n_streams < 1 || n_streams > 64) return TIDE_EINVAL;
    PlanHeader h;
    std::memcpy(&h, h_plan, sizeof h);
    if (h.magic != kMagic || h.version != kVersion) return TIDE_EPLAN;
    if (!h.has_ag) return TIDE_EUNSUPPORTED;
    const uint8_t* b = static_cast<const uint8_t*>(h_plan);
    const ParamDesc* ps = reinterpret_cast<const ParamDesc*>(b + h.off_params);
    const uint64_t* full = reinterpret_cast<const uint64_t*>(b + h.off_full);
    const char* g = reinterpret_cast<const char*>(h.gathered);
    struct Copy {
        char* dst;
        const char* src;
        size_t bytes;
    };
    std::vector<Copy> copies;
    for (int32_t p = 0; p < h.P; ++p) {
        ParamDesc d;
        std::memcpy(&d, ps + p, sizeof d);
        if (d.n == 0) continue;
        char* dst = reinterpret_cast<char*>(full[p]);
        const int64_t nfull = d.d0 / d.s;
        const int64_t rest = d.n - nfull * d.m;
        const int64_t nruns = nfull + (rest > 0 ? 1 : 0);
        for (int64_t r = 0; r < nruns && r < h.R; ++r) {
            const int64_t cnt = r < nfull ? d.m : rest;
            copies.push_back({dst + 2 * r * d.m, g + 2 * (r * h.S + d.off), (size_t)(2 * cnt)});
        }
    }
    std::stable_sort(copies.begin(), copies.end(),
                     [](const Copy& a, const Copy& c) { return a.bytes > c.bytes; });
    std::vector<size_t> load((size_t)n_streams, 0);
    for (const Copy& c : copies) {
        size_t k = (size_t)(std::min_element(load.begin(), load.end()) - load.begin());
        load[k] += c.bytes;
        hipError_t e = hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyDeviceToDeviceNoCU,
                                      reinterpret_cast<hipStream_t>(streams[k]));
        if (e != hipSuccess) return TIDE_EHIP;
    }
    return TIDE_OK;
}
