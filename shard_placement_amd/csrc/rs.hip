// rs.hip -- fused bf16 -> fp32 dim-0-shard reduce-scatter for gfx950.
//
// TIDE-RS reads each parameter's bf16 gradient tensor where it lies and
// reduces it into fp32 shards (Abstract of "The Endgame of FSDP
// Communication", weekinpapers.com); a reduce-scatter starts from one
// whole buffer per rank and leaves each rank with the sum of its own shard
// only (kongchang.com article, section
// "The Root of FSDP2 Communication Overhead").  Here all R ranks' gradient
// tensors sit in one GPU's HBM and are read in place: no rank-major pack
// buffer, no fp32 staging copy.
//
// Work decomposition: the host plan cuts every (param, rank) shard into
// tiles (plan.cpp); one short-lived 256-lane workgroup takes one tile (or
// strides over tiles when the grid is capped), runs of 32 consecutive tiles
// going to one XCD (runs of 33 and 31 tiles on even and odd XCDs in long
// launches: xcd_map.h).  A call is cut into launches of about 160 MiB of
// traffic (the plan's launch size) so that kernels on other queues get whole
// compute units at the launch boundaries.  In a vector tile each lane owns 8
// consecutive elements: it issues one 16-byte load per rank, a batch of
// ranks in flight at once (2, 4 or 8 ranks by the rule at pick_fixed: about
// 32-56 KB of loads in flight per CU), widens bf16 -> fp32 exactly
// (bits << 16), adds in rank order 0..R-1 starting from rank 0's value (or
// pairwise, tree order), and hands its 8 results through the wave's own 2 KB
// of LDS so that each of the wave's two 16-byte-per-lane stores covers one
// contiguous 1 KB run.  Padding tiles only write +0.0f.  There is no
// inter-workgroup communication.  The path is HBM-bound (about 0.25-0.5 flop
// per byte), so there is no MFMA here.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstring>
#include <mutex>

#include "plan_format.h"
#include "stage_check.h"
#include "tide.h"
#include "xcd_map.h"

using namespace tide;

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Every buffer the kernels touch is device global memory; saying so lets
// the compiler emit global_* instead of flat_* memory instructions.
#define TIDE_GLOBAL __attribute__((address_space(1)))

template <bool NT>
__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
    const TIDE_GLOBAL u32x4* g = (const TIDE_GLOBAL u32x4*)(p);
    if constexpr (NT)
        return __builtin_nontemporal_load(g);
    else
        return *g;
}

template <bool NT>
__device__ __forceinline__ void store16(float* p, f32x4 v) {
    TIDE_GLOBAL f32x4* g = (TIDE_GLOBAL f32x4*)(p);
    if constexpr (NT)
        __builtin_nontemporal_store(v, g);
    else
        *g = v;
}

__device__ __forceinline__ uint16_t load2(const uint16_t* p) {
    return *(const TIDE_GLOBAL uint16_t*)(p);
}

__device__ __forceinline__ void store4(float* p, float v) { *(TIDE_GLOBAL float*)(p) = v; }

// bf16 is the upper half of a binary32, so widening is a shift (exact).
// A 32-bit word holds elements 2k (low half) and 2k+1 (high half).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf_one(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ void acc_init(float (&a)[8], u32x4 v) {
    a[0] = bf_lo(v.x); a[1] = bf_hi(v.x);
    a[2] = bf_lo(v.y); a[3] = bf_hi(v.y);
    a[4] = bf_lo(v.z); a[5] = bf_hi(v.z);
    a[6] = bf_lo(v.w); a[7] = bf_hi(v.w);
}

// One IEEE binary32 add per element (no multiply, so nothing to contract).
__device__ __forceinline__ void acc_add(float (&a)[8], u32x4 v) {
    a[0] = a[0] + bf_lo(v.x); a[1] = a[1] + bf_hi(v.x);
    a[2] = a[2] + bf_lo(v.y); a[3] = a[3] + bf_hi(v.y);
    a[4] = a[4] + bf_lo(v.z); a[5] = a[5] + bf_hi(v.z);
    a[6] = a[6] + bf_lo(v.w); a[7] = a[7] + bf_hi(v.w);
}

// The compute unit a workgroup runs on, for the optional census: the HW_ID
// hardware register's cu_id [11:8], sh_id [12] and se_id [15:13] fields
// and the XCC_ID register's xcc_id [3:0], packed as xcc << 8 | (HW_ID >> 8
// & 0xff).  Reading the registers has no side effect.
__device__ __forceinline__ uint32_t hw_cu_id() {
    const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);    // HW_ID
    const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 20);  // XCC_ID
    return ((xcc & 0xfu) << 8) | ((hw >> 8) & 0xffu);
}

// Optional per-tile timing: the GPU's constant-rate real-time counter read
// when the workgroup starts the tile and after all its waves have finished
// it, stored as stamps[2t], stamps[2t + 1].  The barrier only runs when
// stamps is set (a uniform kernel argument).
__device__ __forceinline__ void stamp_tile(uint64_t* stamps, int64_t t, uint64_t t_begin) {
    if (!stamps) return;
    __syncthreads();
    if (threadIdx.x == 0) {
        stamps[2 * t] = t_begin;
        stamps[2 * t + 1] = __builtin_amdgcn_s_memrealtime();
    }
}

__device__ __forceinline__ const uint16_t* src_of(const uint64_t* gp, int q) {
    return reinterpret_cast<const uint16_t*>(gp[q]);
}

// Rank q's source at element j0 + e: a uniform 64-bit base plus a 32-bit
// per-lane byte offset, so the loads use the scalar-base addressing form.
__device__ __forceinline__ const uint16_t* at(const uint64_t* gp, int q, int64_t j0, int e) {
    const char* base = reinterpret_cast<const char*>(gp[q]) + 2 * j0;
    return reinterpret_cast<const uint16_t*>(base + (uint32_t)(2 * e));
}

// Where a tile reads rank q's value of its element e.
// In place: rank q's gradient tensor of the tile's param, flat index j0 + e.
struct GradSrc {
    const uint64_t* gp;  // the param's R gradient pointers
    int64_t j0;
    __device__ __forceinline__ const uint16_t* vec(int q, int e) const { return at(gp, q, j0, e); }
    __device__ __forceinline__ const uint16_t* one(int q, int e) const {
        return src_of(gp, q) + j0 + e;
    }
};

// Staged: slot q of the output rank's staging buffer, which holds rank q's
// slice of every param at the same offsets as the rank's fp32 arena, so the
// element sits at arena offset o0 + e of every slot.
struct SlotSrc {
    const char* base;  // staging buffer of the tile's rank + 2 * o0
    int64_t stride;    // bytes from one slot to the next
    __device__ __forceinline__ const uint16_t* vec(int q, int e) const {
        return reinterpret_cast<const uint16_t*>(base + q * stride + (uint32_t)(2 * e));
    }
    __device__ __forceinline__ const uint16_t* one(int q, int e) const {
        return reinterpret_cast<const uint16_t*>(base + q * stride) + e;
    }
};

// Store a lane's 8 fp32 results so that each store instruction of the wave
// writes one contiguous 1 KB run.  Lane l holds elements [8l, 8l+8) of the
// wave's 512-element chunk; written as two 16-byte stores per lane, each
// instruction would cover every other 16 bytes, and with streaming stores
// the halves of a line reach memory separately (measured: 2.4 TB/s for
// such writes alone vs 5.7 TB/s contiguous).  The lane's results go through
// the wave's own 2 KB of LDS and come back as floats [4l, 4l+4) and
// [256+4l, 256+4l+4).  wb: the wave chunk's first element relative to out;
// len bounds the valid elements (a multiple of 8).  Only this wave touches
// its LDS slice, so a wave-level barrier orders the accesses.
template <bool NTS>
__device__ __forceinline__ void store8_contig(float* __restrict__ out, int wb, int len,
                                              const float (&a)[8], bool ok, float* lds_wave) {
    const int l = threadIdx.x & 63;
    if (ok) {
        *reinterpret_cast<f32x4*>(lds_wave + 8 * l) = f32x4{a[0], a[1], a[2], a[3]};
        *reinterpret_cast<f32x4*>(lds_wave + 8 * l + 4) = f32x4{a[4], a[5], a[6], a[7]};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(lds_wave + 4 * l);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(lds_wave + 256 + 4 * l);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (wb + 4 * l < len)
        store16<NTS>(reinterpret_cast<float*>(reinterpret_cast<char*>(out) +
                                              (uint32_t)(4 * (wb + 4 * l))), o0);
    if (wb + 256 + 4 * l < len)
        store16<NTS>(reinterpret_cast<float*>(reinterpret_cast<char*>(out) +
                                              (uint32_t)(4 * (wb + 256 + 4 * l))), o1);
}

// An output that is not 16-byte aligned takes 8 dword stores per lane (the
// compiler merges them into unaligned 16-byte stores; measured faster than
// an LDS exchange into 256-byte dword runs: 5.3 vs 5.2 TB/s).
__device__ __forceinline__ void store8_unaligned(float* __restrict__ out, int e,
                                                 const float (&a)[8], bool ok) {
    if (!ok) return;
    float* o = reinterpret_cast<float*>(reinterpret_cast<char*>(out) + (uint32_t)(4 * e));
#pragma unroll
    for (int k = 0; k < 8; ++k) store4(o + k, a[k]);
}

// Vector tile, fixed rank order.  Each lane owns U chunks of 8 elements
// (kBlock*8 apart) and issues U*RB 16-byte loads before it adds anything.
// RB ranks are loaded per batch; EXACT means R is a multiple of RB (no
// per-rank guard).  src: where the tile's R source runs are (uniform, every
// run 16-byte aligned); len % 8 == 0.  The loop bounds are uniform over the
// workgroup, so every lane of a wave reaches the LDS exchange of the
// contiguous store; a lane past len re-reads the tile's first elements
// instead of branching around its loads (its results are never stored).
template <int RB, bool EXACT, int U, bool NTL, bool NTS, class Src>
__device__ __forceinline__ void rs_vec_fixed(const Src& src, int R, int len,
                                             float* __restrict__ out, float* lds_wave) {
    constexpr int kStep = kBlock * kVec;
    const bool out16 = (reinterpret_cast<uintptr_t>(out) & 15) == 0;
    const int wave0 = (int)(threadIdx.x & ~63) * kVec;  // this wave's offset in a step
    for (int cbase = 0; cbase < len; cbase += kStep * U) {
        float a[U][8];
        bool ok[U];
        int e[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int x = cbase + u * kStep + (int)threadIdx.x * kVec;
            ok[u] = x < len;
            e[u] = ok[u] ? x : 0;
        }
        {
            u32x4 v[U][RB];
            const int nb = EXACT ? RB : (R < RB ? R : RB);
            // every load of the batch is issued (a rank past R re-reads rank
            // 0, never used): guarded loads would be issued one at a time
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int b = 0; b < RB; ++b)
                    v[u][b] = load16<NTL>(src.vec((EXACT || b < nb) ? b : 0, e[u]));
            // keep the whole batch of loads in flight before any add
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                acc_init(a[u], v[u][0]);
#pragma unroll
                for (int b = 1; b < RB; ++b)
                    if (EXACT || b < nb) acc_add(a[u], v[u][b]);
            }
        }
        for (int q0 = RB; q0 < R; q0 += RB) {
            u32x4 v[U][RB];
            const int nb = EXACT ? RB : ((R - q0) < RB ? (R - q0) : RB);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int b = 0; b < RB; ++b)
                    v[u][b] = load16<NTL>(src.vec((EXACT || b < nb) ? q0 + b : q0, e[u]));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int b = 0; b < RB; ++b)
                    if (EXACT || b < nb) acc_add(a[u], v[u][b]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (out16)
                store8_contig<NTS>(out, cbase + u * kStep + wave0, len, a[u], ok[u], lds_wave);
            else
                store8_unaligned(out, e[u], a[u], ok[u]);
        }
    }
}

// Element-wise tile (unaligned heads and tails, or sources whose 16-byte
// phases differ between ranks): one element per lane, same order.
template <class Src>
__device__ __forceinline__ void rs_scalar_fixed(const Src& src, int R, int len,
                                                float* __restrict__ out) {
    for (int e = threadIdx.x; e < len; e += kBlock) {
        float a = bf_one(load2(src.one(0, e)));
        for (int q = 1; q < R; ++q) a = a + bf_one(load2(src.one(q, e)));
        store4(out + e, a);
    }
}

// Padding rows: +0.0f (all bits clear); nothing is read.
__device__ __forceinline__ void rs_pad(int len, float* __restrict__ out) {
    for (int e = threadIdx.x; e < len; e += kBlock) store4(out + e, 0.0f);
}

// ---- tree order
//
// Pairwise over adjacent ranks, level by level, an odd last element carried
// up unchanged.  That tree is the same as: split R ranks into a left block
// of 2^k ranks (the largest power of two below R) and the rest, recursively;
// i.e. perfect pairwise blocks of sizes given by R's binary digits, largest
// first, combined right to left.  It is evaluated streaming, rank by rank,
// as a binary counter: level l holds a finished block of 2^l ranks while
// bit l of the count is set; pushing rank q merges (older block + newer)
// for every trailing one of q.  Control flow depends only on the uniform
// rank count, and every stack index is a compile-time constant, so the
// stack stays in registers.  LEVELS >= floor(log2 R) + 1.
template <int LEVELS, int W>
struct TreeStack {
    float v[LEVELS][W];

    __device__ __forceinline__ void push(const float (&x_in)[W], int count) {
        float x[W];
#pragma unroll
        for (int k = 0; k < W; ++k) x[k] = x_in[k];
        bool placed = false;
#pragma unroll
        for (int l = 0; l < LEVELS; ++l) {
            const bool carry = (count >> l) & 1;
            if (!placed && carry) {
#pragma unroll
                for (int k = 0; k < W; ++k) x[k] = v[l][k] + x[k];
            }
            if (!placed && !carry) {
#pragma unroll
                for (int k = 0; k < W; ++k) v[l][k] = x[k];
            }
            placed = placed || !carry;
        }
    }

    // After R pushes: combine the blocks named by R's set bits, smallest
    // (rightmost ranks) first, each older block on the left.
    __device__ __forceinline__ void finish(int R, float (&out)[W]) {
        bool have = false;
#pragma unroll
        for (int l = 0; l < LEVELS; ++l) {
            if ((R >> l) & 1) {
#pragma unroll
                for (int k = 0; k < W; ++k) out[k] = have ? v[l][k] + out[k] : v[l][k];
                have = true;
            }
        }
    }
};

__device__ __forceinline__ void widen8(float (&x)[8], u32x4 v) {
    x[0] = bf_lo(v.x); x[1] = bf_hi(v.x);
    x[2] = bf_lo(v.y); x[3] = bf_hi(v.y);
    x[4] = bf_lo(v.z); x[5] = bf_hi(v.z);
    x[6] = bf_lo(v.w); x[7] = bf_hi(v.w);
}

template <int LEVELS, bool NTL, bool NTS, class Src>
__device__ __forceinline__ void rs_vec_tree(const Src& src, int R, int len,
                                            float* __restrict__ out, float* lds_wave) {
    constexpr int RB = 8;
    constexpr int kStep = kBlock * kVec;
    const bool out16 = (reinterpret_cast<uintptr_t>(out) & 15) == 0;
    const int wave0 = (int)(threadIdx.x & ~63) * kVec;
    for (int cbase = 0; cbase < len; cbase += kStep) {
        const int x = cbase + (int)threadIdx.x * kVec;
        const bool ok = x < len;
        const int e = ok ? x : 0;  // lanes past len re-read the tile start
        TreeStack<LEVELS, 8> st;
        for (int q0 = 0; q0 < R; q0 += RB) {
            u32x4 v[RB];
            const int nb = (R - q0) < RB ? (R - q0) : RB;
            // the whole batch of loads in flight (a rank past R re-reads
            // rank q0, never used), then the pushes
#pragma unroll
            for (int b = 0; b < RB; ++b) v[b] = load16<NTL>(src.vec(b < nb ? q0 + b : q0, e));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < RB; ++b)
                if (b < nb) {
                    float x[8];
                    widen8(x, v[b]);
                    st.push(x, q0 + b);
                }
        }
        float a[8];
        st.finish(R, a);
        if (out16)
            store8_contig<NTS>(out, cbase + wave0, len, a, ok, lds_wave);
        else
            store8_unaligned(out, e, a, ok);
    }
}

template <int LEVELS, class Src>
__device__ __forceinline__ void rs_scalar_tree(const Src& src, int R, int len,
                                               float* __restrict__ out) {
    for (int e = threadIdx.x; e < len; e += kBlock) {
        TreeStack<LEVELS, 1> st;
        for (int q = 0; q < R; ++q) {
            float x[1] = {bf_one(load2(src.one(q, e)))};
            st.push(x, q);
        }
        float a[1];
        st.finish(R, a);
        store4(out + e, a[0]);
    }
}

template <int LEVELS, bool NTL, bool NTS>
__global__ __launch_bounds__(kBlock) void rs_tree_kernel(const RsTile* __restrict__ tiles,
                                                         int64_t ntiles,
                                                         const uint64_t* __restrict__ gptr,
                                                         const uint64_t* __restrict__ obase,
                                                         int R, uint32_t* __restrict__ census,
                                                         uint64_t* __restrict__ stamps) {
    __shared__ float lds[kBlock * kVec];
    float* lds_wave = lds + (threadIdx.x & ~63) * kVec;
    for (int64_t b = blockIdx.x; b < ntiles; b += gridDim.x) {
        const int64_t t = tile_of(b, ntiles);
        if (census && threadIdx.x == 0) census[t] = hw_cu_id();
        const uint64_t t_begin = stamps ? __builtin_amdgcn_s_memrealtime() : 0;
        const RsTile tile = tiles[t];
        float* out = reinterpret_cast<float*>(obase[tile.r]) + tile.o0;
        const GradSrc src{gptr + (int64_t)tile.p * R, tile.j0};
        if (tile.kind == kRsVec)
            rs_vec_tree<LEVELS, NTL, NTS>(src, R, tile.len, out, lds_wave);
        else if (tile.kind == kRsScalar)
            rs_scalar_tree<LEVELS>(src, R, tile.len, out);
        else
            rs_pad(tile.len, out);
        stamp_tile(stamps, t, t_begin);
    }
}

template <int RB, bool EXACT, int U, bool NTL, bool NTS>
__device__ __forceinline__ void rs_fixed_tile(const RsTile* __restrict__ tiles, int64_t t,
                                              const uint64_t* __restrict__ gptr,
                                              const uint64_t* __restrict__ obase, int R,
                                              uint32_t* __restrict__ census,
                                              uint64_t* __restrict__ stamps, float* lds_wave) {
    if (census && threadIdx.x == 0) census[t] = hw_cu_id();
    const uint64_t t_begin = stamps ? __builtin_amdgcn_s_memrealtime() : 0;
    const RsTile tile = tiles[t];
    float* out = reinterpret_cast<float*>(obase[tile.r]) + tile.o0;
    const GradSrc src{gptr + (int64_t)tile.p * R, tile.j0};
    if (tile.kind == kRsVec)
        rs_vec_fixed<RB, EXACT, U, NTL, NTS>(src, R, tile.len, out, lds_wave);
    else if (tile.kind == kRsScalar)
        rs_scalar_fixed(src, R, tile.len, out);
    else
        rs_pad(tile.len, out);
    stamp_tile(stamps, t, t_begin);
}

// SKEW: the instance for launches of skewed_grid(ntiles) workgroups, each
// taking one tile at most (xcd_map.h); the plain instance runs one
// workgroup per tile or a capped grid striding over the tiles.
template <int RB, bool EXACT, int U, bool NTL, bool NTS, bool SKEW = false>
__global__ __launch_bounds__(kBlock) void rs_fixed_kernel(const RsTile* __restrict__ tiles,
                                                          int64_t ntiles,
                                                          const uint64_t* __restrict__ gptr,
                                                          const uint64_t* __restrict__ obase,
                                                          int R, uint32_t* __restrict__ census,
                                                          uint64_t* __restrict__ stamps) {
    __shared__ float lds[kBlock * kVec];
    float* lds_wave = lds + (threadIdx.x & ~63) * kVec;
    if constexpr (SKEW) {
        for (int64_t b = blockIdx.x; b < walk_end(ntiles); b += gridDim.x) {
            const int64_t t = tile_of_skewed(b, ntiles);
            if (t < 0) continue;
            rs_fixed_tile<RB, EXACT, U, NTL, NTS>(tiles, t, gptr, obase, R, census, stamps,
                                                  lds_wave);
        }
    } else {
        for (int64_t b = blockIdx.x; b < ntiles; b += gridDim.x)
            rs_fixed_tile<RB, EXACT, U, NTL, NTS>(tiles, tile_of(b, ntiles), gptr, obase, R,
                                                  census, stamps, lds_wave);
    }
}

// ---- fold of staged slots
//
// The copy engines have moved rank q's slice of every param of rank r's
// shard into slot q of rank r's staging buffer (stage[r] + q * stride bytes,
// laid out like rank r's fp32 arena), so a tile's R runs are the slots at
// its arena offset o0.  Same tiles, rank order and bits as the in-place
// kernels.  vec_ok: every staging buffer and the slot stride are 16-byte
// aligned; a vector tile whose o0 is not a multiple of 8 goes element-wise.
__device__ __forceinline__ SlotSrc slot_src(const uint64_t* stage, int64_t stride,
                                            const RsTile& tile) {
    return SlotSrc{reinterpret_cast<const char*>(stage[tile.r]) + 2 * tile.o0, stride};
}

template <int RB, bool EXACT, int U, bool NTL, bool NTS>
__global__ __launch_bounds__(kBlock) void rs_fold_kernel(const RsTile* __restrict__ tiles,
                                                         int64_t ntiles,
                                                         const uint64_t* __restrict__ stage,
                                                         int64_t stride, int vec_ok,
                                                         const uint64_t* __restrict__ obase,
                                                         int R) {
    __shared__ float lds[kBlock * kVec];
    float* lds_wave = lds + (threadIdx.x & ~63) * kVec;
    for (int64_t b = blockIdx.x; b < ntiles; b += gridDim.x) {
        const RsTile tile = tiles[tile_of(b, ntiles)];
        float* out = reinterpret_cast<float*>(obase[tile.r]) + tile.o0;
        const SlotSrc src = slot_src(stage, stride, tile);
        if (tile.kind == kRsVec && vec_ok && (tile.o0 & 7) == 0)
            rs_vec_fixed<RB, EXACT, U, NTL, NTS>(src, R, tile.len, out, lds_wave);
        else if (tile.kind != kRsPad)
            rs_scalar_fixed(src, R, tile.len, out);
        else
            rs_pad(tile.len, out);
    }
}

template <int LEVELS, bool NTL, bool NTS>
__global__ __launch_bounds__(kBlock) void rs_fold_tree_kernel(const RsTile* __restrict__ tiles,
                                                              int64_t ntiles,
                                                              const uint64_t* __restrict__ stage,
                                                              int64_t stride, int vec_ok,
                                                              const uint64_t* __restrict__ obase,
                                                              int R) {
    __shared__ float lds[kBlock * kVec];
    float* lds_wave = lds + (threadIdx.x & ~63) * kVec;
    for (int64_t b = blockIdx.x; b < ntiles; b += gridDim.x) {
        const RsTile tile = tiles[tile_of(b, ntiles)];
        float* out = reinterpret_cast<float*>(obase[tile.r]) + tile.o0;
        const SlotSrc src = slot_src(stage, stride, tile);
        if (tile.kind == kRsVec && vec_ok && (tile.o0 & 7) == 0)
            rs_vec_tree<LEVELS, NTL, NTS>(src, R, tile.len, out, lds_wave);
        else if (tile.kind != kRsPad)
            rs_scalar_tree<LEVELS>(src, R, tile.len, out);
        else
            rs_pad(tile.len, out);
    }
}

// ---- two-phase pipeline
//
// Phase 1 reduces a range of tiles into a dense staging chunk (tile t of the
// range at stage + t * T floats, T = the plan's tile size) instead of the
// shard arenas; phase 2 moves a chunk's results to their places in the
// arenas (the stand-in for the network phase that delivers partial results
// to their owners).  Phase 1 computes exactly what the in-place kernel
// computes; phase 2 is a copy, so phase 1 then phase 2 gives its bits.
template <int RB, bool EXACT, int U, bool NTL, bool NTS>
__global__ __launch_bounds__(kBlock) void rs_dense_kernel(const RsTile* __restrict__ tiles,
                                                          int64_t ntiles,
                                                          const uint64_t* __restrict__ gptr,
                                                          float* __restrict__ stage, int64_t T,
                                                          int R) {
    __shared__ float lds[kBlock * kVec];
    float* lds_wave = lds + (threadIdx.x & ~63) * kVec;
    for (int64_t b = blockIdx.x; b < ntiles; b += gridDim.x) {
        const int64_t t = tile_of(b, ntiles);
        const RsTile tile = tiles[t];
        float* out = stage + t * T;
        const GradSrc src{gptr + (int64_t)tile.p * R, tile.j0};
        if (tile.kind == kRsVec)
            rs_vec_fixed<RB, EXACT, U, NTL, NTS>(src, R, tile.len, out, lds_wave);
        else if (tile.kind == kRsScalar)
            rs_scalar_fixed(src, R, tile.len, out);
        else
            rs_pad(tile.len, out);
    }
}

__device__ __forceinline__ f32x4 load16f(const float* p) {
    return *(const TIDE_GLOBAL f32x4*)(p);
}

template <bool NTS>
__global__ __launch_bounds__(kBlock) void rs_drain_kernel(const RsTile* __restrict__ tiles,
                                                          int64_t ntiles,
                                                          const float* __restrict__ stage,
                                                          int64_t T,
                                                          const uint64_t* __restrict__ obase) {
    for (int64_t b = blockIdx.x; b < ntiles; b += gridDim.x) {
        const int64_t t = tile_of(b, ntiles);
        const RsTile tile = tiles[t];
        const float* src = stage + t * T;
        float* dst = reinterpret_cast<float*>(obase[tile.r]) + tile.o0;
        const int len = tile.len;
        if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0 && (len & 3) == 0) {
            for (int e = threadIdx.x * 4; e < len; e += kBlock * 4)
                store16<NTS>(dst + e, load16f(src + e));
        } else {
            for (int e = threadIdx.x; e < len; e += kBlock) store4(dst + e, src[e]);
        }
    }
}

typedef void (*RsKernel)(const RsTile*, int64_t, const uint64_t*, const uint64_t*, int, uint32_t*,
                         uint64_t*);

template <int RB, bool EXACT, int U, bool SKEW = false>
RsKernel pick_nt(uint32_t flags) {
    const bool ntl = flags & kFlagNtLoads, nts = flags & kFlagNtStores;
    if (ntl && nts) return rs_fixed_kernel<RB, EXACT, U, true, true, SKEW>;
    if (ntl) return rs_fixed_kernel<RB, EXACT, U, true, false, SKEW>;
    if (nts) return rs_fixed_kernel<RB, EXACT, U, false, true, SKEW>;
    return rs_fixed_kernel<RB, EXACT, U, false, false, SKEW>;
}

// Rank batching: small power-of-two R loads every rank at once (with U
// chunks per lane when R < 8 and the tile holds them, so that up to 8 loads
// are in flight).  R a multiple of 8 loads 2 ranks per batch, or 4 when the
// launch holds two workgroups per CU (the plan's LDS reservation): about
// 32-56 KB of loads in flight per CU read fastest.  Measured on MI355X
// (same buffers, one process, two processes each): against batches of 8,
// +1.5..2.1% at R = 8, +1.0..1.6% at R = 16, +1.5..2.3% at R = 32 (2 ranks
// per batch, up to 7 workgroups per CU) and +1.6..1.9% at R = 64 (4 ranks, 2
// per CU); 2 ranks at R = 64 read 14% less, 16 ranks 1.5-3.2% less than 8.
// Any other R batches 8, the last batch re-reading a rank in place of the
// missing ones.  Chunks per lane for R < 8: as many as the tile holds, up
// to 4 (a chunk past the tile end would only re-read its start); a second
// chunk per lane at R = 8 did not help (5.6 vs 5.8 TB/s).
template <typename K, K (*PICK1)(uint32_t), K (*PICK2)(uint32_t), K (*PICK4)(uint32_t)>
K by_chunks(int32_t tile, uint32_t flags) {
    const int32_t chunks = tile / kTileQuantum;
    return chunks >= 4 ? PICK4(flags) : chunks >= 2 ? PICK2(flags) : PICK1(flags);
}

RsKernel pick_fixed(int R, uint32_t flags, int32_t tile, bool two_per_cu) {
    switch (R) {
        case 1: return by_chunks<RsKernel, pick_nt<1, true, 1>, pick_nt<1, true, 2>, pick_nt<1, true, 4>>(tile, flags);
        case 2: return by_chunks<RsKernel, pick_nt<2, true, 1>, pick_nt<2, true, 2>, pick_nt<2, true, 4>>(tile, flags);
        case 4: return by_chunks<RsKernel, pick_nt<4, true, 1>, pick_nt<4, true, 2>, pick_nt<4, true, 4>>(tile, flags);
        default: break;
    }
    if (R % 8 == 0) return two_per_cu ? pick_nt<4, true, 1>(flags) : pick_nt<2, true, 1>(flags);
    return pick_nt<8, false, 1>(flags);
}

// A launch holds two workgroups per CU when the plan reserves LDS for them.
bool holds_two_per_cu(const PlanHeader& h) { return h.rs_lds_bytes > (uint32_t)kRsStaticLds; }

// The skewed form (xcd_map.h) of the fixed-order kernel that loads 2 ranks
// per batch, for launches of kSkewMinTiles tiles or more; null where the
// plan's kernel has none (other rank counts were not measured with it).
RsKernel pick_fixed_skewed(int R, uint32_t flags, bool two_per_cu) {
    if (R % 8 == 0 && !two_per_cu) return pick_nt<2, true, 1, true>(flags);
    return nullptr;
}

template <int LEVELS>
RsKernel pick_tree_nt(uint32_t flags) {
    const bool ntl = flags & kFlagNtLoads, nts = flags & kFlagNtStores;
    if (ntl && nts) return rs_tree_kernel<LEVELS, true, true>;
    if (ntl) return rs_tree_kernel<LEVELS, true, false>;
    if (nts) return rs_tree_kernel<LEVELS, false, true>;
    return rs_tree_kernel<LEVELS, false, false>;
}

// Stack depth: 7 levels hold blocks up to 64 ranks; 13 up to kMaxRanks.
RsKernel pick_tree(int R, uint32_t flags) {
    static_assert(kMaxRanks <= 4096, "13 levels cover R <= 8191");
    if (R <= 127) return pick_tree_nt<7>(flags);
    return pick_tree_nt<13>(flags);
}

typedef void (*DenseKernel)(const RsTile*, int64_t, const uint64_t*, float*, int64_t, int);

template <int RB, bool EXACT, int U>
DenseKernel pick_dense_nt(uint32_t flags) {
    const bool ntl = flags & kFlagNtLoads, nts = flags & kFlagNtStores;
    if (ntl && nts) return rs_dense_kernel<RB, EXACT, U, true, true>;
    if (ntl) return rs_dense_kernel<RB, EXACT, U, true, false>;
    if (nts) return rs_dense_kernel<RB, EXACT, U, false, true>;
    return rs_dense_kernel<RB, EXACT, U, false, false>;
}

DenseKernel pick_dense(int R, uint32_t flags, int32_t tile, bool two_per_cu) {
    switch (R) {
        case 1: return by_chunks<DenseKernel, pick_dense_nt<1, true, 1>, pick_dense_nt<1, true, 2>, pick_dense_nt<1, true, 4>>(tile, flags);
        case 2: return by_chunks<DenseKernel, pick_dense_nt<2, true, 1>, pick_dense_nt<2, true, 2>, pick_dense_nt<2, true, 4>>(tile, flags);
        case 4: return by_chunks<DenseKernel, pick_dense_nt<4, true, 1>, pick_dense_nt<4, true, 2>, pick_dense_nt<4, true, 4>>(tile, flags);
        default: break;
    }
    if (R % 8 == 0) return two_per_cu ? pick_dense_nt<4, true, 1>(flags) : pick_dense_nt<2, true, 1>(flags);
    return pick_dense_nt<8, false, 1>(flags);
}

typedef void (*FoldKernel)(const RsTile*, int64_t, const uint64_t*, int64_t, int, const uint64_t*,
                           int);

template <int RB, bool EXACT, int U>
FoldKernel pick_fold_nt(uint32_t flags) {
    const bool ntl = flags & kFlagNtLoads, nts = flags & kFlagNtStores;
    if (ntl && nts) return rs_fold_kernel<RB, EXACT, U, true, true>;
    if (ntl) return rs_fold_kernel<RB, EXACT, U, true, false>;
    if (nts) return rs_fold_kernel<RB, EXACT, U, false, true>;
    return rs_fold_kernel<RB, EXACT, U, false, false>;
}

// Same rank batching as the in-place kernels.
FoldKernel pick_fold(int R, uint32_t flags, int32_t tile, bool two_per_cu) {
    switch (R) {
        case 1: return by_chunks<FoldKernel, pick_fold_nt<1, true, 1>, pick_fold_nt<1, true, 2>, pick_fold_nt<1, true, 4>>(tile, flags);
        case 2: return by_chunks<FoldKernel, pick_fold_nt<2, true, 1>, pick_fold_nt<2, true, 2>, pick_fold_nt<2, true, 4>>(tile, flags);
        case 4: return by_chunks<FoldKernel, pick_fold_nt<4, true, 1>, pick_fold_nt<4, true, 2>, pick_fold_nt<4, true, 4>>(tile, flags);
        default: break;
    }
    if (R % 8 == 0) return two_per_cu ? pick_fold_nt<4, true, 1>(flags) : pick_fold_nt<2, true, 1>(flags);
    return pick_fold_nt<8, false, 1>(flags);
}

template <int LEVELS>
FoldKernel pick_fold_tree_nt(uint32_t flags) {
    const bool ntl = flags & kFlagNtLoads, nts = flags & kFlagNtStores;
    if (ntl && nts) return rs_fold_tree_kernel<LEVELS, true, true>;
    if (ntl) return rs_fold_tree_kernel<LEVELS, true, false>;
    if (nts) return rs_fold_tree_kernel<LEVELS, false, true>;
    return rs_fold_tree_kernel<LEVELS, false, false>;
}

FoldKernel pick_fold_tree(int R, uint32_t flags) {
    if (R <= 127) return pick_fold_tree_nt<7>(flags);
    return pick_fold_tree_nt<13>(flags);
}

}  // namespace

namespace {

// Dynamic LDS a reduce-scatter launch requests on top of the kernel's own,
// so that each workgroup holds the plan's LDS reservation (the kernels never
// touch the extra bytes).
static_assert(sizeof(float[kBlock * kVec]) == kRsStaticLds, "the kernels' static LDS");
unsigned rs_extra_lds(const PlanHeader& h) {
    return h.rs_lds_bytes > (uint32_t)kRsStaticLds ? h.rs_lds_bytes - (uint32_t)kRsStaticLds : 0u;
}

// Launch i of the call goes to streams[i % n_streams] (one stream unless a
// caller deals the launches over several hardware queues).
tide_status launch_rs(const void* h_plan, const void* d_plan, int32_t order, int64_t tile_begin,
                      int64_t tile_count, int32_t max_workgroups, const tide_stream_t* streams,
                      int32_t n_streams, uint32_t* census = nullptr, int64_t census_len = 0,
                      uint64_t* stamps = nullptr) {
    if (!h_plan || !d_plan) return TIDE_EINVAL;
    PlanHeader h;
    std::memcpy(&h, h_plan, sizeof h);
    if (h.magic != kMagic || h.version != kVersion) return TIDE_EPLAN;
    if (order != 0 && order != 1) return TIDE_EINVAL;
    if (max_workgroups < 0) return TIDE_EINVAL;
    if (!h.has_rs) return TIDE_EUNSUPPORTED;
    if (reinterpret_cast<uintptr_t>(d_plan) % 16) return TIDE_EALIGN;
    if (tile_count < 0) tile_count = h.n_rs_tiles - tile_begin;
    if (tile_begin < 0 || tile_count < 0 || tile_begin > h.n_rs_tiles ||
        tile_count > h.n_rs_tiles - tile_begin)
        return TIDE_EINVAL;
    if (tile_count == 0) return TIDE_OK;
    if ((census || stamps) && census_len < tile_count) return TIDE_EINVAL;

    const uint8_t* d = static_cast<const uint8_t*>(d_plan);
    const RsTile* all = reinterpret_cast<const RsTile*>(d + h.off_rs);
    const uint64_t* gptr = reinterpret_cast<const uint64_t*>(d + h.off_gptr);
    const uint64_t* obase = reinterpret_cast<const uint64_t*>(d + h.off_obase);
    int R = h.R;
    RsKernel k = order == 0 ? pick_fixed(R, h.flags, h.rs_tile, holds_two_per_cu(h))
                            : pick_tree(R, h.flags);
    RsKernel ks = order == 0 && max_workgroups == 0
                      ? pick_fixed_skewed(R, h.flags, holds_two_per_cu(h))
                      : nullptr;
    const int64_t launch_tiles = order == 1 ? h.rs_launch_tiles_tree : h.rs_launch_tiles;
    const int64_t per_launch = launch_tiles > 0 ? launch_tiles : tile_count;

    // One launch per run of per_launch tiles: the launch boundaries are where
    // kernels on other hardware queues get whole compute units.
    int64_t i = 0;
    for (int64_t b = tile_begin; b < tile_begin + tile_count; b += per_launch, ++i) {
        const RsTile* tiles = all + b;
        int64_t ntiles = per_launch < tile_begin + tile_count - b ? per_launch
                                                                  : tile_begin + tile_count - b;
        const bool skew = ks && ntiles >= kSkewMinTiles && skewed_grid(ntiles) <= INT_MAX;
        int64_t grid = skew ? skewed_grid(ntiles) : ntiles;
        if (max_workgroups > 0 && grid > max_workgroups) grid = max_workgroups;
        if (grid > INT_MAX) grid = INT_MAX;
        uint32_t* cen = census ? census + (b - tile_begin) : nullptr;
        uint64_t* stp = stamps ? stamps + 2 * (b - tile_begin) : nullptr;
        void* args[] = {&tiles, &ntiles, &gptr, &obase, &R, &cen, &stp};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(skew ? ks : k),
                                       dim3((unsigned)grid),
                                       dim3(kBlock), args, rs_extra_lds(h),
                                       reinterpret_cast<hipStream_t>(streams[i % n_streams]));
        if (e != hipSuccess) return TIDE_EHIP;
    }
    return TIDE_OK;
}

}  // namespace

extern "C" tide_status tide_rs_bf16_to_fp32(const void* h_plan, const void* d_plan, int32_t order,
                                            int32_t max_workgroups, tide_stream_t stream) {
    return launch_rs(h_plan, d_plan, order, 0, -1, max_workgroups, &stream, 1);
}

extern "C" tide_status tide_rs_bf16_to_fp32_streams(const void* h_plan, const void* d_plan,
                                                    int32_t order, int32_t max_workgroups,
                                                    const tide_stream_t* streams,
                                                    int32_t n_streams) {
    if (!streams || n_streams < 1 || n_streams > 64) return TIDE_EINVAL;
    // the null stream waits for (and holds up) every blocking stream: dealing
    // launches between it and other streams would serialise them all
    if (n_streams > 1)
        for (int32_t i = 0; i < n_streams; ++i)
            if (!streams[i]) return TIDE_EINVAL;
    return launch_rs(h_plan, d_plan, order, 0, -1, max_workgroups, streams, n_streams);
}

extern "C" tide_status tide_rs_bf16_to_fp32_tiles(const void* h_plan, const void* d_plan,
                                                  int32_t order, int64_t tile_begin,
                                                  int64_t tile_count, int32_t max_workgroups,
                                                  tide_stream_t stream) {
    if (tile_count < 0) return TIDE_EINVAL;
    return launch_rs(h_plan, d_plan, order, tile_begin, tile_count, max_workgroups, &stream, 1);
}

extern "C" tide_status tide_rs_fold_staged(const void* h_plan, const void* d_plan, int32_t order,
                                           const uint64_t* h_stage, const uint64_t* d_stage,
                                           int64_t slot_stride, int32_t max_workgroups,
                                           tide_stream_t stream) {
    if (!h_plan || !d_plan || !d_stage) return TIDE_EINVAL;
    PlanHeader h;
    std::memcpy(&h, h_plan, sizeof h);
    if (h.magic != kMagic || h.version != kVersion) return TIDE_EPLAN;
    if (order != 0 && order != 1) return TIDE_EINVAL;
    if (max_workgroups < 0) return TIDE_EINVAL;
    bool vec_ok = false;
    tide_status st = check_stage(h_plan, h_stage, slot_stride, &vec_ok);
    if (st != TIDE_OK) return st;
    if (reinterpret_cast<uintptr_t>(d_plan) % 16 || reinterpret_cast<uintptr_t>(d_stage) % 8)
        return TIDE_EALIGN;
    if (h.n_rs_tiles == 0) return TIDE_OK;

    const uint8_t* d = static_cast<const uint8_t*>(d_plan);
    const RsTile* all = reinterpret_cast<const RsTile*>(d + h.off_rs);
    const uint64_t* obase = reinterpret_cast<const uint64_t*>(d + h.off_obase);
    int R = h.R;
    int vec = vec_ok ? 1 : 0;
    int64_t stride = 2 * slot_stride;
    FoldKernel k = order == 0 ? pick_fold(R, h.flags, h.rs_tile, holds_two_per_cu(h))
                              : pick_fold_tree(R, h.flags);
    const int64_t launch_tiles = order == 1 ? h.rs_launch_tiles_tree : h.rs_launch_tiles;
    const int64_t per_launch = launch_tiles > 0 ? launch_tiles : h.n_rs_tiles;
    for (int64_t b = 0; b < h.n_rs_tiles; b += per_launch) {
        const RsTile* tiles = all + b;
        int64_t ntiles = per_launch < h.n_rs_tiles - b ? per_launch : h.n_rs_tiles - b;
        int64_t grid = ntiles;
        if (max_workgroups > 0 && grid > max_workgroups) grid = max_workgroups;
        if (grid > INT_MAX) grid = INT_MAX;
        void* args[] = {&tiles, &ntiles, &d_stage, &stride, &vec, &obase, &R};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(k), dim3((unsigned)grid),
                                       dim3(kBlock), args, rs_extra_lds(h),
                                       reinterpret_cast<hipStream_t>(stream));
        if (e != hipSuccess) return TIDE_EHIP;
    }
    return TIDE_OK;
}

namespace tide {

tide_status issue_tiles_to_stage(const PlanHeader& h, const void* d_plan, int64_t tile_begin,
                                 int64_t tile_count, float* stage, int32_t max_workgroups,
                                 tide_stream_t stream) {
    const uint8_t* d = static_cast<const uint8_t*>(d_plan);
    const RsTile* all = reinterpret_cast<const RsTile*>(d + h.off_rs);
    const uint64_t* gptr = reinterpret_cast<const uint64_t*>(d + h.off_gptr);
    int R = h.R;
    int64_t T = h.rs_tile;
    DenseKernel k = pick_dense(R, h.flags, h.rs_tile, holds_two_per_cu(h));
    const int64_t per_launch = h.rs_launch_tiles > 0 ? h.rs_launch_tiles : tile_count;
    for (int64_t b = tile_begin; b < tile_begin + tile_count; b += per_launch) {
        const RsTile* tiles = all + b;
        int64_t ntiles = per_launch < tile_begin + tile_count - b ? per_launch
                                                                  : tile_begin + tile_count - b;
        int64_t grid = ntiles;
        if (max_workgroups > 0 && grid > max_workgroups) grid = max_workgroups;
        if (grid > INT_MAX) grid = INT_MAX;
        float* out = stage + (b - tile_begin) * T;
        void* args[] = {&tiles, &ntiles, &gptr, &out, &T, &R};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(k), dim3((unsigned)grid),
                                       dim3(kBlock), args, rs_extra_lds(h),
                                       reinterpret_cast<hipStream_t>(stream));
        if (e != hipSuccess) return TIDE_EHIP;
    }
    return TIDE_OK;
}

tide_status issue_stage_to_shards(const PlanHeader& h, const void* d_plan, int64_t tile_begin,
                                  int64_t tile_count, const float* stage, int32_t max_workgroups,
                                  tide_stream_t stream) {
    const uint8_t* d = static_cast<const uint8_t*>(d_plan);
    const RsTile* all = reinterpret_cast<const RsTile*>(d + h.off_rs);
    const uint64_t* obase = reinterpret_cast<const uint64_t*>(d + h.off_obase);
    int64_t T = h.rs_tile;
    const void* k = (h.flags & kFlagNtStores)
                        ? reinterpret_cast<const void*>(rs_drain_kernel<true>)
                        : reinterpret_cast<const void*>(rs_drain_kernel<false>);
    // a drain moves 8 bytes per element where the reduction moves 2R + 4:
    // launches of the same byte size hold (2R + 4) / 8 times the tiles
    int64_t per_launch = h.rs_launch_tiles > 0 ? h.rs_launch_tiles * (2 * h.R + 4) / 8 : tile_count;
    if (per_launch < 1) per_launch = 1;
    for (int64_t b = tile_begin; b < tile_begin + tile_count; b += per_launch) {
        const RsTile* tiles = all + b;
        int64_t ntiles = per_launch < tile_begin + tile_count - b ? per_launch
                                                                  : tile_begin + tile_count - b;
        int64_t grid = ntiles;
        if (max_workgroups > 0 && grid > max_workgroups) grid = max_workgroups;
        if (grid > INT_MAX) grid = INT_MAX;
        const float* src = stage + (b - tile_begin) * T;
        void* args[] = {&tiles, &ntiles, &src, &T, &obase};
        hipError_t e = hipLaunchKernel(k, dim3((unsigned)grid), dim3(kBlock), args, 0,
                                       reinterpret_cast<hipStream_t>(stream));
        if (e != hipSuccess) return TIDE_EHIP;
    }
    return TIDE_OK;
}

}  // namespace tide

extern "C" tide_status tide_rs_tiles_to_stage(const void* h_plan, const void* d_plan,
                                              int64_t tile_begin, int64_t tile_count,
                                              float* stage, int64_t stage_elems,
                                              int32_t max_workgroups, tide_stream_t stream) {
    if (!d_plan) return TIDE_EINVAL;
    PlanHeader h;
    tide_status st = check_pipeline(h_plan, d_plan, tile_begin, tile_count, stage, stage_elems,
                                    max_workgroups, &h);
    if (st != TIDE_OK) return st;
    return issue_tiles_to_stage(h, d_plan, tile_begin, tile_count, stage, max_workgroups, stream);
}

extern "C" tide_status tide_rs_stage_to_shards(const void* h_plan, const void* d_plan,
                                               int64_t tile_begin, int64_t tile_count,
                                               const float* stage, int64_t stage_elems,
                                               int32_t max_workgroups, tide_stream_t stream) {
    if (!d_plan) return TIDE_EINVAL;
    PlanHeader h;
    tide_status st = check_pipeline(h_plan, d_plan, tile_begin, tile_count, stage, stage_elems,
                                    max_workgroups, &h);
    if (st != TIDE_OK) return st;
    return issue_stage_to_shards(h, d_plan, tile_begin, tile_count, stage, max_workgroups, stream);
}

extern "C" tide_status tide_rs_bf16_to_fp32_census(const void* h_plan, const void* d_plan,
                                                   int32_t order, int32_t max_workgroups,
                                                   uint32_t* census, int64_t census_len,
                                                   tide_stream_t stream) {
    if (!census) return TIDE_EINVAL;
    return launch_rs(h_plan, d_plan, order, 0, -1, max_workgroups, &stream, 1, census, census_len);
}

extern "C" tide_status tide_rs_bf16_to_fp32_trace(const void* h_plan, const void* d_plan,
                                                  int32_t order, int32_t max_workgroups,
                                                  uint32_t* census, uint64_t* stamps,
                                                  int64_t len, tide_stream_t stream) {
    if (!census || !stamps) return TIDE_EINVAL;
    if (reinterpret_cast<uintptr_t>(census) % 4 || reinterpret_cast<uintptr_t>(stamps) % 8)
        return TIDE_EALIGN;
    return launch_rs(h_plan, d_plan, order, 0, -1, max_workgroups, &stream, 1, census, len, stamps);
}

// ---- the two phases through the library's own staging array
//
// For callers that cannot allocate device memory: the staging chunk of the
// two-phase calls is a file-scope device array instead of caller memory.
// In host code `scratch` names a host-side stand-in, not the device array:
// its device address is looked up once per device (with that device
// current) and only that address is ever handed to kernels.
namespace {

static_assert(TIDE_SCRATCH_BYTES % 256 == 0, "the staging array is whole 256-byte blocks");
static __device__ __align__(256) float scratch[TIDE_SCRATCH_BYTES / sizeof(float)];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kScratchDevices];  // device address of `scratch`, per device

// The array's address for the calling thread's current device, which must
// be the device `stream` belongs to (kernels get that device's address).
tide_status scratch_for_stream(tide_stream_t stream, float** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TIDE_EHIP;
    if (stream) {
        hipDevice_t sdev = 0;
        if (hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev) != hipSuccess)
            return TIDE_EHIP;
        if (sdev != dev) return TIDE_EINVAL;
    }
    if (dev < 0 || dev >= kScratchDevices) return TIDE_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TIDE_EHIP;
        g_scratch[dev] = static_cast<float*>(p);
    }
    *out = g_scratch[dev];
    return TIDE_OK;
}

}  // namespace

extern "C" tide_status tide_rs_two_phase_noalloc(const void* h_plan, const void* d_plan,
                                                 int64_t tile_begin, int64_t tile_count,
                                                 int32_t max_workgroups, tide_stream_t stream) {
    // every host-side check before the first HIP call
    if (!h_plan || !d_plan) return TIDE_EINVAL;
    PlanHeader h;
    std::memcpy(&h, h_plan, sizeof h);
    if (h.magic != kMagic || h.version != kVersion) return TIDE_EPLAN;
    if (!h.has_rs) return TIDE_EUNSUPPORTED;
    if (max_workgroups < 0 || tile_begin < 0 || tile_count < 0 || tile_begin > h.n_rs_tiles ||
        tile_count > h.n_rs_tiles - tile_begin)
        return TIDE_EINVAL;
    const int64_t cap = (int64_t)(TIDE_SCRATCH_BYTES / sizeof(float));
    if (h.rs_tile <= 0 || tile_count > cap / h.rs_tile) return TIDE_ENOSPACE;
    if (reinterpret_cast<uintptr_t>(d_plan) % 16) return TIDE_EALIGN;
    if (tile_count == 0) return TIDE_OK;
    float* stage = nullptr;
    tide_status st = scratch_for_stream(stream, &stage);
    if (st != TIDE_OK) return st;
    st = check_pipeline(h_plan, d_plan, tile_begin, tile_count, stage, cap, max_workgroups, &h);
    if (st != TIDE_OK) return st;
    st = issue_tiles_to_stage(h, d_plan, tile_begin, tile_count, stage, max_workgroups, stream);
    if (st != TIDE_OK) return st;
    return issue_stage_to_shards(h, d_plan, tile_begin, tile_count, stage, max_workgroups, stream);
}
