// plan_format.h -- in-memory layout of a libtide plan blob (host and device).
//
// The plan is the descriptor table through which the parameter layout
// becomes part of the kernels' addressing, the central idea of the Abstract
// of "The Endgame of FSDP Communication" (weekinpapers.com).  It is
// built on the host once per layer (plan.cpp), uploaded by the caller, and
// read by the kernels: every workgroup looks up one tile and from it the
// per-rank source pointers and the destination pointer of its run.
//
// Sections start at 256-byte boundaries; all integers are little-endian.
#pragma once

#include <stdint.h>

namespace tide {

constexpr uint32_t kMagic = 0x45444954u;  // "TIDE"
constexpr uint32_t kVersion = 2;
constexpr int kBlock = 256;        // threads per workgroup (4 wave64)
constexpr int kVec = 8;            // bf16 elements per 16-byte vector
constexpr int kTileQuantum = kBlock * kVec;  // tile sizes are multiples of this
constexpr int kMaxRanks = 4096;
constexpr int kRsStaticLds = kBlock * kVec * 4;  // the reduce-scatter kernels' store exchange

// Plan-wide access hints; same values as TIDE_FLAG_* in tide.h.
enum PlanFlags : uint32_t {
    kFlagNtLoads = 1u,   // non-temporal (streaming) gradient / slot loads
    kFlagNtStores = 2u,  // non-temporal shard / parameter stores
};

struct PlanHeader {
    uint32_t magic;
    uint32_t version;
    int32_t R;
    int32_t P;
    int64_t align;
    int64_t S;           // slot numel
    int64_t N;           // sum of d0*c
    int64_t Npad;        // sum of R*m
    int32_t rs_tile;     // elements per reduce-scatter tile
    int32_t ag_tile;     // elements per placement tile
    int64_t n_rs_tiles;
    int64_t n_ag_tiles;
    uint64_t off_params;  // ParamDesc[P]
    uint64_t off_gptr;    // uint64_t[P*R], param-major: [p*R + q]
    uint64_t off_obase;   // uint64_t[R] fp32 arenas
    uint64_t off_full;    // uint64_t[P] bf16 full tensors
    uint64_t off_rs;      // RsTile[n_rs_tiles]
    uint64_t off_ag;      // AgTile[n_ag_tiles]
    uint64_t gathered;    // device address of the gathered buffer
    uint64_t bytes;       // blob bytes in use
    int32_t has_rs;
    int32_t has_ag;
    uint32_t flags;
    uint32_t rs_lds_bytes;    // LDS per reduce-scatter workgroup (0: the kernels' own)
    int64_t rs_launch_tiles;  // tiles per reduce-scatter kernel launch
    int64_t ag_launch_tiles;  // tiles per placement kernel launch
    int64_t rs_launch_tiles_tree;  // the same for the tree-order kernels
};

struct ParamDesc {
    int64_t d0;   // rows
    int64_t c;    // elements per row
    int64_t s;    // chunk rows = ceil(d0 / R)
    int64_t m;    // shard numel = s*c
    int64_t n;    // d0*c
    int64_t off;  // element offset of the shard in each arena / slot
};

// A reduce-scatter tile: `len` consecutive flat indices j0.. of param p, all
// inside rank r's shard.  Output element for j is obase[r] + o0 + (j - j0).
enum RsKind : int32_t {
    kRsVec = 0,     // every rank's source 16-byte aligned at j0, len % 8 == 0
    kRsScalar = 1,  // element-wise (unaligned heads, tails, odd layouts)
    kRsPad = 2,     // padding rows: write +0.0f, read nothing
};

struct RsTile {
    int64_t j0;
    int64_t o0;
    int32_t p;
    int32_t r;
    int32_t len;
    int32_t kind;
};

// A placement tile: copy `len` bf16 elements from gathered + src to
// full[p] + dst.  kind says the widest access both ends allow.
enum AgKind : int32_t {
    kAgVec16 = 0,   // both ends 16-byte aligned, len % 8 == 0
    kAgVec4 = 1,    // both ends 4-byte aligned, len % 2 == 0
    kAgScalar = 2,  // 2-byte elements
    kAgShift = 3,   // destination 16-byte aligned, source not (16-byte loads
                    // from a 2-byte-aligned address); len % 8 == 0
};

struct AgTile {
    int64_t src;
    int64_t dst;
    int32_t p;
    int32_t len;
    int32_t kind;
    int32_t reserved;
};

static_assert(sizeof(PlanHeader) <= 256, "header must fit its section");
static_assert(sizeof(ParamDesc) == 48, "ParamDesc layout");
static_assert(sizeof(RsTile) == 32, "RsTile layout");
static_assert(sizeof(AgTile) == 32, "AgTile layout");

}  // namespace tide
