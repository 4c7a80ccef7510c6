// plan.cpp -- host side of libtide: plan (descriptor table) builder,
// validation and status strings.  Pure host C++; no HIP call is made here.
//
// The plan makes the FSDP2 layout part of the kernels' addressing (Abstract
// of "The Endgame of FSDP Communication", weekinpapers.com): per parameter
// it records the
// shard geometry, per (rank, parameter) the gradient pointer, and it cuts
// every rank's shard into tiles that a workgroup can process without any
// further layout arithmetic.  Shard geometry follows the library contract
// in tide.h (rows split in R chunks of ceil(d0/R), +0.0 padding rows,
// arena offsets rounded up to align_elems).
#include <algorithm>
#include <cstddef>
#include <cstring>
#include <vector>

#include "plan_format.h"
#include "tide.h"

using namespace tide;

namespace {

constexpr int64_t kSection = 256;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Default reduce-scatter tile: at most about 64 KB of HBM traffic per tile
// (R*2 + 4 bytes per element), a power of two in [2048, 32768] elements, so
// 2048 elements (one pass of a 256-lane workgroup) from R = 8 up.  Short
// tiles measured fastest on MI355X (R = 8: 2048 -> 5.90, 4096 -> 5.75,
// 8192 -> 5.48 TB/s with 256 MiB launches).
int32_t default_rs_tile(int32_t R) {
    int64_t want = (int64_t)65536 / (2 * (int64_t)R + 4);
    int64_t t = kTileQuantum;
    while (t * 2 <= want && t < 32768) t *= 2;
    return (int32_t)t;
}

// Placement: 2048-element tiles, streaming loads and stores (measured best).
constexpr int32_t kDefaultAgTile = 2048;
constexpr int32_t kDefaultFlags = TIDE_FLAG_NT_LOADS | TIDE_FLAG_NT_STORES;

// Launch granularity.  Measured on MI355X next to a single-wave bf16 GEMM
// on another hardware queue: one launch for a whole layer starves the GEMM
// (it waits for free compute units that the stream of short workgroups
// never leaves); with launch boundaries the GEMM waits about half a launch.
// Reduce-scatter: about 160 MiB of algorithmic traffic per launch (against
// 256 MiB it halves the slowdown, +3..6% vs +9..13%, for 1-3% less
// bandwidth; 128 MiB costs another 3%).  A launch of fewer than 4
// workgroups per CU is rounded down to whole workgroups per CU (256 tiles,
// one per compute unit of the MI355X), and holds at least 2 per CU: at
// R = 64 a 160 MiB launch would hold 620 tiles, 2.4 per CU, which leaves
// the waves unbalanced (5.6 TB/s), while 512 tiles (132 MiB) read 6.01
// TB/s against 6.12 at 1024 and cut the GEMM's slowdown from +11..15% to
// +3..10%.  Placement: 256 MiB, the same trade: beside the single-wave
// GEMM (Llama-3.1-70B layer, three runs each) 256 MiB launches cost the
// GEMM +7..10%, 512 MiB +22..27%, 1 GiB +59..69% and one launch per call
// +100..144%, while the placement gains 3% from 512 MiB on and loses 4%
// below 256.  An explicit launch size applies to both, unrounded.
//
// A launch of 2 workgroups per CU leaves room beside them (VGPRs, waves,
// LDS) for a workgroup of a concurrent kernel, e.g. the single-wave GEMM's
// (256 VGPRs per wave, 65 KB of LDS), which then shares the CU with
// streaming reduce-scatter waves and finishes late.  (Launches of many
// tiles per CU, as at R = 8, keep up to 7 workgroups of 38 VGPRs (40
// allocated) resident on every CU for their whole length, per the per-tile
// trace: 280 of a SIMD's 512 registers, too few left for the GEMM's
// 256-VGPR waves; it waits about half a launch.)  Such
// launches therefore hold 64 KB of LDS per
// workgroup (the kernel uses 8 KB): two fill 128 of the CU's 160 KB, and a
// workgroup needing more than 32 KB cannot start beside them.  Measured at
// R = 64 (512 tiles per launch, two boxes, 4 processes each): GEMM slowdown
// +2.3..6.5% (mean 5.0 and 4.8%) against +2.9..9.4% (mean 6.0 and 7.3%)
// without the reservation and +11..15% at 1024 tiles; reduce-scatter
// bandwidth unchanged (6.0 TB/s).
constexpr int32_t kDefaultRsLaunchMiB = 160;
constexpr int64_t kCuTiles = 256;
constexpr int64_t kRsRoundBelowTiles = 4 * kCuTiles;
constexpr int64_t kMinRsLaunchTiles = 2 * kCuTiles;
// One round: a CU holds up to 8 workgroups of the kernel that loads 2 ranks
// per batch (R a multiple of 8), 7 of its skewed form (per-tile trace at
// R = 8, 16 and 32), so a launch of up to 7 per CU starts all of its tiles
// together and ends with its most loaded CU, and a longer one of 8.x ends
// with a thin second round.  For such R, launches of 4 to 8.x workgroups
// per CU are rounded to the nearest whole number per CU, at most 7 (one
// round for either form; 8 per CU with the plain form read 0.5% less than
// 7 on the MoE layer) (same buffers, two processes each): at R = 32, 1280 tiles per launch (5 per CU) read
// 6.24-6.26 TB/s against 6.04-6.07 for the byte target's 1204 (4.7 per CU;
// 1024: 6.20, 1536: 6.31, 1792: 6.32); at R = 16, 1792 tiles (7 per CU)
// read 5.80-5.91 against 5.70-5.85 for 2275 (8.9 per CU) on the MoE layer
// (0..+1.7%, four processes) and 5.96-5.98 against 5.87-5.89 on the Llama
// layer's shapes (2048, 8 per CU: 5.70), with the GEMM beside the MoE layer
// at +2.9..5.7% against +4.1..8.1%.  Longer launches keep the byte target (at R = 8, 3584 tiles, 14
// per CU, read 4.5% less than 4096), and so does the kernel that loads 8
// ranks per batch (other R), which was not traced (at R = 18, 1792 tiles
// read 2.5% less than the byte target's 2048).
constexpr int64_t kRsOneRoundTiles = 9 * kCuTiles;
constexpr int64_t kRsMaxPerCuOneRound = 7;
constexpr uint32_t kRsLdsReserve = 64 * 1024;
constexpr int32_t kDefaultAgLaunchMiB = 256;

struct Resolved {
    int64_t align;
    int32_t rs_tile, ag_tile;
    uint32_t flags;
    int64_t rs_launch_bytes;  // <= 0: unlimited
    int64_t ag_launch_bytes;
    int64_t rs_min_tiles;     // lower bound on tiles per reduce-scatter launch
    bool rs_round;            // round short launches to whole workgroups per CU
};

tide_status resolve_opts(const tide_opts* o, int32_t R, Resolved* out) {
    out->align = 1;
    out->rs_tile = default_rs_tile(R);
    out->ag_tile = kDefaultAgTile;
    out->flags = kDefaultFlags;
    out->rs_launch_bytes = (int64_t)kDefaultRsLaunchMiB << 20;
    out->ag_launch_bytes = (int64_t)kDefaultAgLaunchMiB << 20;
    out->rs_min_tiles = kMinRsLaunchTiles;
    out->rs_round = true;
    if (!o) return TIDE_OK;
    if (o->launch_mib < -1 || o->launch_mib > (1 << 20)) return TIDE_EINVAL;
    if (o->launch_mib != 0) {
        out->rs_launch_bytes = out->ag_launch_bytes =
            o->launch_mib == -1 ? 0 : (int64_t)o->launch_mib << 20;
        out->rs_min_tiles = 1;
        out->rs_round = false;
    }
    if (o->align_elems < 1 || o->align_elems > (int64_t)1 << 20) return TIDE_EINVAL;
    out->align = o->align_elems;
    if (o->rs_tile_elems != 0) {
        if (o->rs_tile_elems < 0 || o->rs_tile_elems % kTileQuantum || o->rs_tile_elems > (1 << 24))
            return TIDE_EINVAL;
        out->rs_tile = o->rs_tile_elems;
    }
    if (o->ag_tile_elems != 0) {
        if (o->ag_tile_elems < 0 || o->ag_tile_elems % kTileQuantum || o->ag_tile_elems > (1 << 24))
            return TIDE_EINVAL;
        out->ag_tile = o->ag_tile_elems;
    }
    if (o->flags != -1) {
        if (o->flags & ~(TIDE_FLAG_NT_LOADS | TIDE_FLAG_NT_STORES)) return TIDE_EINVAL;
        out->flags = (uint32_t)o->flags;
    }
    return TIDE_OK;
}

tide_status geometry(const tide_shape* shapes, int32_t P, int32_t R, int64_t align,
                     std::vector<ParamDesc>* params, int64_t* S, int64_t* N, int64_t* Npad) {
    if (P < 0 || R < 1 || R > kMaxRanks) return TIDE_EINVAL;
    if (P > 0 && !shapes) return TIDE_EINVAL;
    params->resize(P);
    int64_t off = 0, n_tot = 0, pad_tot = 0;
    const int64_t kLimit = (int64_t)1 << 46;  // keeps every product below 2^63
    for (int32_t p = 0; p < P; ++p) {
        int64_t d0 = shapes[p].dim0, c = shapes[p].row_numel;
        if (d0 < 0 || c < 0 || d0 > kLimit || c > kLimit) return TIDE_EINVAL;
        if (d0 > 0 && c > kLimit / d0) return TIDE_EINVAL;
        ParamDesc& d = (*params)[p];
        d.d0 = d0;
        d.c = c;
        d.s = ceil_div(d0, R);
        d.m = d.s * c;
        d.n = d0 * c;
        d.off = off;
        off += round_up(d.m, align);
        n_tot += d.n;
        pad_tot += (int64_t)R * d.m;
        if (off > kLimit || pad_tot > kLimit * 16) return TIDE_EINVAL;
    }
    *S = off;
    *N = n_tot;
    *Npad = pad_tot;
    return TIDE_OK;
}

// Upper bounds of the tile counts, valid for any pointer alignment: a run
// of L elements becomes at most ceil(L/T) + 2 tiles (scalar head, vector
// body, scalar tail); each (rank, param) has one valid run and one padding
// run.
int64_t rs_tiles_bound(const std::vector<ParamDesc>& ps, int32_t R, int32_t T) {
    int64_t t = 0;
    for (const ParamDesc& d : ps)
        if (d.m > 0) t += (int64_t)R * (2 * ceil_div(d.m, T) + 3);
    return t;
}

int64_t ag_tiles_bound(const std::vector<ParamDesc>& ps, int32_t R, int32_t T) {
    int64_t t = 0;
    for (const ParamDesc& d : ps)
        if (d.m > 0) t += (int64_t)R * (ceil_div(d.m, T) + 2);
    return t;
}

struct Layout {
    uint64_t off_params, off_gptr, off_obase, off_full, off_rs, off_ag, bytes;
};

Layout section_layout(int32_t P, int32_t R, int64_t n_rs, int64_t n_ag) {
    Layout L;
    uint64_t pos = kSection;  // header
    L.off_params = pos;
    pos += round_up((int64_t)sizeof(ParamDesc) * P, kSection);
    L.off_gptr = pos;
    pos += round_up((int64_t)8 * P * R, kSection);
    L.off_obase = pos;
    pos += round_up((int64_t)8 * R, kSection);
    L.off_full = pos;
    pos += round_up((int64_t)8 * P, kSection);
    L.off_rs = pos;
    pos += round_up((int64_t)sizeof(RsTile) * n_rs, kSection);
    L.off_ag = pos;
    pos += round_up((int64_t)sizeof(AgTile) * n_ag, kSection);
    L.bytes = pos;
    return L;
}

// Overlap check over address ranges of four classes.
enum RangeClass { kRsIn = 0, kRsOut = 1, kAgIn = 2, kAgOut = 3 };
struct Range {
    uint64_t lo, hi;
    int cls;
};

bool ranges_conflict(std::vector<Range>& rs) {
    std::sort(rs.begin(), rs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
    uint64_t max_end[4] = {0, 0, 0, 0};
    bool seen[4] = {false, false, false, false};
    for (const Range& x : rs) {
        auto hits = [&](int c) { return seen[c] && max_end[c] > x.lo; };
        bool bad = false;
        switch (x.cls) {
            case kRsOut: bad = hits(kRsIn) || hits(kRsOut); break;
            case kRsIn: bad = hits(kRsOut); break;
            case kAgOut: bad = hits(kAgIn) || hits(kAgOut); break;
            case kAgIn: bad = hits(kAgOut); break;
        }
        if (bad) return true;
        if (!seen[x.cls] || x.hi > max_end[x.cls]) max_end[x.cls] = x.hi;
        seen[x.cls] = true;
    }
    return false;
}

// Cut the run [jb, je) of param p, rank r into reduce-scatter tiles.
void cut_rs_run(std::vector<RsTile>& out, int32_t p, int32_t r, int64_t jb, int64_t je,
                int64_t o_of_jb, bool vec_ok, int64_t phase_elems, int32_t T) {
    auto emit = [&](int64_t a, int64_t b, int32_t kind) {
        for (int64_t x = a; x < b; x += T) {
            RsTile t;
            t.j0 = x;
            t.o0 = o_of_jb + (x - jb);
            t.p = p;
            t.r = r;
            t.len = (int32_t)std::min<int64_t>(T, b - x);
            t.kind = kind;
            out.push_back(t);
        }
    };
    if (jb >= je) return;
    if (!vec_ok) {
        emit(jb, je, kRsScalar);
        return;
    }
    // first j >= jb whose source address is 16-byte aligned in every rank
    int64_t jv = jb + (((phase_elems - jb) % kVec) + kVec) % kVec;
    int64_t jend = jv + ((je - jv) / kVec) * kVec;
    if (jv >= je || jend <= jv) {
        emit(jb, je, kRsScalar);
        return;
    }
    emit(jb, jv, kRsScalar);
    emit(jv, jend, kRsVec);
    emit(jend, je, kRsScalar);
}

void cut_ag_run(std::vector<AgTile>& out, int32_t p, int64_t src, int64_t dst, int64_t len,
                uint64_t gaddr, uint64_t faddr, int32_t T) {
    auto emit = [&](int64_t s0, int64_t d0, int64_t l, int32_t kind) {
        for (int64_t x = 0; x < l; x += T) {
            AgTile t;
            t.src = s0 + x;
            t.dst = d0 + x;
            t.p = p;
            t.len = (int32_t)std::min<int64_t>(T, l - x);
            t.kind = kind;
            t.reserved = 0;
            out.push_back(t);
        }
    };
    if (len <= 0) return;
    uint64_t sa = gaddr + 2 * (uint64_t)src, da = faddr + 2 * (uint64_t)dst;
    if (sa % 16 != da % 16) {
        // Realigning copy: destination 16-byte aligned from `head` on; the
        // kernel reads the (2-byte-aligned) source 16 bytes at a time from
        // exactly the tile's own elements.
        const int64_t head = std::min<int64_t>(len, (int64_t)(((16 - da % 16) % 16) / 2));
        const int64_t body = ((len - head) / kVec) * kVec;
        if (body > 0) {
            emit(src, dst, head, kAgScalar);
            emit(src + head, dst + head, body, kAgShift);
            emit(src + head + body, dst + head + body, len - head - body, kAgScalar);
            return;
        }
    }
    int32_t kinds[2] = {kAgVec16, kAgVec4};
    uint64_t widths[2] = {16, 4};
    for (int k = 0; k < 2; ++k) {
        uint64_t W = widths[k];
        if (sa % W != da % W) continue;
        int64_t head = (int64_t)(((W - sa % W) % W) / 2);
        int64_t per = (int64_t)W / 2;
        if (head >= len) break;
        int64_t body = ((len - head) / per) * per;
        if (body == 0) break;
        emit(src, dst, head, kAgScalar);
        emit(src + head, dst + head, body, kinds[k]);
        emit(src + head + body, dst + head + body, len - head - body, kAgScalar);
        return;
    }
    emit(src, dst, len, kAgScalar);
}

}  // namespace

extern "C" {

int32_t tide_abi_version(void) { return TIDE_ABI_VERSION; }

const char* tide_status_str(int32_t status) {
    switch (status) {
        case TIDE_OK: return "ok";
        case TIDE_EINVAL: return "invalid argument";
        case TIDE_EALIGN: return "pointer not aligned to its element size";
        case TIDE_EOVERLAP: return "an output range overlaps an input or another output";
        case TIDE_ENOSPACE: return "plan blob too small";
        case TIDE_EHIP: return "HIP runtime error";
        case TIDE_EUNSUPPORTED: return "request not supported by this plan";
        case TIDE_EPLAN: return "not a tide plan or wrong version";
        default: return "unknown status";
    }
}

tide_status tide_desc_size(const tide_shape* shapes, int32_t P, int32_t R, const tide_opts* opts,
                           size_t* blob_bytes) {
    if (!blob_bytes) return TIDE_EINVAL;
    Resolved o;
    tide_status st = resolve_opts(opts, R, &o);
    if (st != TIDE_OK) return st;
    std::vector<ParamDesc> ps;
    int64_t S, N, Npad;
    st = geometry(shapes, P, R, o.align, &ps, &S, &N, &Npad);
    if (st != TIDE_OK) return st;
    Layout L = section_layout(P, R, rs_tiles_bound(ps, R, o.rs_tile), ag_tiles_bound(ps, R, o.ag_tile));
    *blob_bytes = (size_t)L.bytes;
    return TIDE_OK;
}

tide_status tide_desc_geometry(const tide_shape* shapes, int32_t P, int32_t R, const tide_opts* opts,
                               int64_t* chunk_rows, int64_t* shard_numel, int64_t* offsets,
                               int64_t* slot_numel) {
    if (!slot_numel) return TIDE_EINVAL;
    Resolved o;
    tide_status st = resolve_opts(opts, R, &o);
    if (st != TIDE_OK) return st;
    std::vector<ParamDesc> ps;
    int64_t S, N, Npad;
    st = geometry(shapes, P, R, o.align, &ps, &S, &N, &Npad);
    if (st != TIDE_OK) return st;
    for (int32_t p = 0; p < P; ++p) {
        if (chunk_rows) chunk_rows[p] = ps[p].s;
        if (shard_numel) shard_numel[p] = ps[p].m;
        if (offsets) offsets[p] = ps[p].off;
    }
    *slot_numel = S;
    return TIDE_OK;
}

tide_status tide_desc_build(const tide_shape* shapes, int32_t P, int32_t R, const tide_opts* opts,
                            const void* const* grads, void* const* out_base, const void* gathered,
                            void* const* full, void* blob, size_t blob_bytes, tide_plan_info* info) {
    Resolved o;
    tide_status st = resolve_opts(opts, R, &o);
    if (st != TIDE_OK) return st;
    std::vector<ParamDesc> ps;
    int64_t S, N, Npad;
    st = geometry(shapes, P, R, o.align, &ps, &S, &N, &Npad);
    if (st != TIDE_OK) return st;
    const bool has_rs = grads != nullptr;
    const bool has_ag = gathered != nullptr;
    if (has_rs != (out_base != nullptr)) return TIDE_EINVAL;
    if (has_ag != (full != nullptr)) return TIDE_EINVAL;
    if (!blob) return TIDE_EINVAL;

    std::vector<Range> ranges;
    // ---- pointer validation
    if (has_rs) {
        for (int32_t r = 0; r < R; ++r) {
            uint64_t a = (uint64_t)(uintptr_t)out_base[r];
            if (S > 0 && a == 0) return TIDE_EINVAL;
            if (a % 4) return TIDE_EALIGN;
            for (int32_t p = 0; p < P; ++p)
                if (ps[p].m > 0)
                    ranges.push_back({a + 4 * (uint64_t)ps[p].off, a + 4 * (uint64_t)(ps[p].off + ps[p].m), kRsOut});
        }
        for (int32_t q = 0; q < R; ++q)
            for (int32_t p = 0; p < P; ++p) {
                uint64_t a = (uint64_t)(uintptr_t)grads[(int64_t)q * P + p];
                if (ps[p].n == 0) continue;
                if (a == 0) return TIDE_EINVAL;
                if (a % 2) return TIDE_EALIGN;
                ranges.push_back({a, a + 2 * (uint64_t)ps[p].n, kRsIn});
            }
    }
    if (has_ag) {
        uint64_t g = (uint64_t)(uintptr_t)gathered;
        if (g % 2) return TIDE_EALIGN;
        if (S > 0) ranges.push_back({g, g + 2 * (uint64_t)R * (uint64_t)S, kAgIn});
        for (int32_t p = 0; p < P; ++p) {
            uint64_t a = (uint64_t)(uintptr_t)full[p];
            if (ps[p].n == 0) continue;
            if (a == 0) return TIDE_EINVAL;
            if (a % 2) return TIDE_EALIGN;
            ranges.push_back({a, a + 2 * (uint64_t)ps[p].n, kAgOut});
        }
    }
    if (ranges_conflict(ranges)) return TIDE_EOVERLAP;

    // ---- tiles
    std::vector<RsTile> rs;
    std::vector<AgTile> ag;
    if (has_rs) {
        rs.reserve((size_t)std::min<int64_t>(rs_tiles_bound(ps, R, o.rs_tile), (int64_t)1 << 24));
        // per param: whether every rank's source shares one 16-byte phase
        // (the vector path), and the first 16-byte aligned flat index
        std::vector<char> vec_ok(P, 0);
        std::vector<int64_t> phase(P, 0);
        for (int32_t p = 0; p < P; ++p) {
            bool ok = ps[p].n > 0;
            const uint64_t a0 = (uint64_t)(uintptr_t)grads[p];
            for (int32_t q = 1; q < R && ok; ++q)
                if (((uint64_t)(uintptr_t)grads[(int64_t)q * P + p]) % 16 != a0 % 16) ok = false;
            vec_ok[p] = ok;
            phase[p] = (int64_t)(((16 - a0 % 16) % 16) / 2);  // (a0 + 2j) % 16 == 0
        }
        // Output-stationary order: rank outer, then param, then index, so
        // that each rank's fp32 arena is written front to back, one output
        // stream at a time.  Measured against param-outer order (every
        // rank's shard of a param in turn), same bits: +8% on a layer of
        // 389 params at R = 16 (whose shards of ~100 K elements otherwise
        // keep all 16 arenas open for writing at once), +1% at R = 32,
        // neutral at R = 8 and 64.
        for (int32_t r = 0; r < R; ++r) {
            for (int32_t p = 0; p < P; ++p) {
                const ParamDesc& d = ps[p];
                if (d.m == 0) continue;
                int64_t jb = (int64_t)r * d.m, je = std::min<int64_t>(d.n, jb + d.m);
                if (jb < je) cut_rs_run(rs, p, r, jb, je, d.off, vec_ok[p] != 0, phase[p], o.rs_tile);
                int64_t pb = std::max<int64_t>(d.n, jb), pe = jb + d.m;
                for (int64_t x = pb; x < pe; x += o.rs_tile) {
                    RsTile t;
                    t.j0 = x;
                    t.o0 = d.off + (x - jb);
                    t.p = p;
                    t.r = r;
                    t.len = (int32_t)std::min<int64_t>(o.rs_tile, pe - x);
                    t.kind = kRsPad;
                    rs.push_back(t);
                }
            }
        }
    }
    if (has_ag) {
        uint64_t g = (uint64_t)(uintptr_t)gathered;
        for (int32_t p = 0; p < P; ++p) {
            const ParamDesc& d = ps[p];
            if (d.n == 0) continue;
            for (int32_t r = 0; r < R; ++r) {
                int64_t v = std::min<int64_t>(std::max<int64_t>(d.d0 - (int64_t)r * d.s, 0), d.s);
                cut_ag_run(ag, p, (int64_t)r * S + d.off, (int64_t)r * d.m, v * d.c, g,
                           (uint64_t)(uintptr_t)full[p], o.ag_tile);
            }
        }
    }

    Layout L = section_layout(P, R, (int64_t)rs.size(), (int64_t)ag.size());
    // tiles per launch from the launch size and each tile's traffic
    const int64_t rs_tile_bytes = (int64_t)o.rs_tile * (2 * (int64_t)R + 4);
    const int64_t ag_tile_bytes = (int64_t)o.ag_tile * 4;
    int64_t rs_launch = std::max<int64_t>(1, (int64_t)rs.size());
    int64_t ag_launch = std::max<int64_t>(1, (int64_t)ag.size());
    // The tree-order kernels hold 109 VGPRs, so at most 4 of their
    // workgroups fit on a CU: with the fixed order's one-round sizes they
    // read 0.8-1.8% less on the R = 16 and R = 32 layers.  Their launches of
    // 4 to 8.x workgroups per CU (R a multiple of 8) are rounded down to
    // whole rounds of 4 per CU instead: the DiT block (R = 32) 1024 tiles
    // against the byte target's 1204, 5.85-5.86 TB/s against 5.75-5.76; the
    // MoE layer (R = 16) 2048 against 2275, 5.70-5.71 against 5.69-5.70 (same
    // buffers, two processes).
    int64_t rs_launch_tree = rs_launch;
    if (o.rs_launch_bytes > 0) {
        int64_t t = o.rs_launch_bytes / rs_tile_bytes;
        if (o.rs_round && t < kRsRoundBelowTiles) t = t / kCuTiles * kCuTiles;
        int64_t tt = t;
        if (o.rs_round && R % 8 == 0 && t >= kRsRoundBelowTiles && t < kRsOneRoundTiles)
            tt = t / kRsRoundBelowTiles * kRsRoundBelowTiles;
        rs_launch_tree = std::min(rs_launch, std::max<int64_t>(o.rs_min_tiles, tt));
        if (o.rs_round && R % 8 == 0 && t >= kRsRoundBelowTiles && t < kRsOneRoundTiles)
            t = std::min<int64_t>((t + kCuTiles / 2) / kCuTiles, kRsMaxPerCuOneRound) * kCuTiles;
        rs_launch = std::min(rs_launch, std::max<int64_t>(o.rs_min_tiles, t));
    }
    if (o.ag_launch_bytes > 0)
        ag_launch = std::min(ag_launch, std::max<int64_t>(1, o.ag_launch_bytes / ag_tile_bytes));
    const uint32_t rs_lds = (o.rs_round && rs_launch <= kMinRsLaunchTiles) ? kRsLdsReserve : 0u;
    if (info) {
        std::memset(info, 0, sizeof(*info));
        info->R = R;
        info->P = P;
        info->slot_numel = S;
        info->numel = N;
        info->padded_numel = Npad;
        info->rs_tiles = (int64_t)rs.size();
        info->ag_tiles = (int64_t)ag.size();
        info->rs_tile_elems = o.rs_tile;
        info->ag_tile_elems = o.ag_tile;
        info->blob_bytes = (int64_t)L.bytes;
        info->rs_launch_tiles = rs_launch;
        info->ag_launch_tiles = ag_launch;
        info->rs_lds_bytes = rs_lds ? rs_lds : kRsStaticLds;
    }
    if (blob_bytes < L.bytes) return TIDE_ENOSPACE;

    uint8_t* b = static_cast<uint8_t*>(blob);
    std::memset(b, 0, (size_t)L.bytes);
    PlanHeader h;
    std::memset(&h, 0, sizeof h);
    h.magic = kMagic;
    h.version = kVersion;
    h.R = R;
    h.P = P;
    h.align = o.align;
    h.S = S;
    h.N = N;
    h.Npad = Npad;
    h.rs_tile = o.rs_tile;
    h.ag_tile = o.ag_tile;
    h.n_rs_tiles = (int64_t)rs.size();
    h.n_ag_tiles = (int64_t)ag.size();
    h.off_params = L.off_params;
    h.off_gptr = L.off_gptr;
    h.off_obase = L.off_obase;
    h.off_full = L.off_full;
    h.off_rs = L.off_rs;
    h.off_ag = L.off_ag;
    h.gathered = (uint64_t)(uintptr_t)gathered;
    h.bytes = L.bytes;
    h.has_rs = has_rs ? 1 : 0;
    h.has_ag = has_ag ? 1 : 0;
    h.flags = o.flags;
    h.rs_launch_tiles = rs_launch;
    h.ag_launch_tiles = ag_launch;
    h.rs_launch_tiles_tree = rs_launch_tree;
    h.rs_lds_bytes = rs_lds;
    std::memcpy(b, &h, sizeof h);
    if (P) std::memcpy(b + L.off_params, ps.data(), sizeof(ParamDesc) * (size_t)P);
    uint64_t* gp = reinterpret_cast<uint64_t*>(b + L.off_gptr);
    uint64_t* ob = reinterpret_cast<uint64_t*>(b + L.off_obase);
    uint64_t* fp = reinterpret_cast<uint64_t*>(b + L.off_full);
    if (has_rs) {
        for (int32_t p = 0; p < P; ++p)
            for (int32_t q = 0; q < R; ++q)
                gp[(int64_t)p * R + q] = (uint64_t)(uintptr_t)grads[(int64_t)q * P + p];
        for (int32_t r = 0; r < R; ++r) ob[r] = (uint64_t)(uintptr_t)out_base[r];
    }
    if (has_ag)
        for (int32_t p = 0; p < P; ++p) fp[p] = (uint64_t)(uintptr_t)full[p];
    if (!rs.empty()) std::memcpy(b + L.off_rs, rs.data(), sizeof(RsTile) * rs.size());
    if (!ag.empty()) std::memcpy(b + L.off_ag, ag.data(), sizeof(AgTile) * ag.size());
    return TIDE_OK;
}

tide_status tide_plan_query(const void* h_plan, tide_plan_info* info) {
    if (!h_plan || !info) return TIDE_EINVAL;
    PlanHeader h;
    std::memcpy(&h, h_plan, sizeof h);
    if (h.magic != kMagic || h.version != kVersion) return TIDE_EPLAN;
    std::memset(info, 0, sizeof(*info));
    info->R = h.R;
    info->P = h.P;
    info->slot_numel = h.S;
    info->numel = h.N;
    info->padded_numel = h.Npad;
    info->rs_tiles = h.n_rs_tiles;
    info->ag_tiles = h.n_ag_tiles;
    info->rs_tile_elems = h.rs_tile;
    info->ag_tile_elems = h.ag_tile;
    info->blob_bytes = (int64_t)h.bytes;
    info->rs_launch_tiles = h.rs_launch_tiles;
    info->ag_launch_tiles = h.ag_launch_tiles;
    info->rs_lds_bytes = h.rs_lds_bytes ? h.rs_lds_bytes : kRsStaticLds;
    return TIDE_OK;
}

tide_status tide_plan_rank_tiles(const void* h_plan, int32_t r, int64_t* tile_begin,
                                 int64_t* tile_count) {
    if (!h_plan || !tile_begin || !tile_count) return TIDE_EINVAL;
    PlanHeader h;
    std::memcpy(&h, h_plan, sizeof h);
    if (h.magic != kMagic || h.version != kVersion) return TIDE_EPLAN;
    if (!h.has_rs) return TIDE_EUNSUPPORTED;
    if (r < 0 || r >= h.R) return TIDE_EINVAL;
    // tiles are ordered rank-outer: the first tile of a rank >= x by bisection
    const RsTile* t = reinterpret_cast<const RsTile*>(static_cast<const uint8_t*>(h_plan) + h.off_rs);
    auto first_at_least = [&](int32_t x) {
        int64_t lo = 0, hi = h.n_rs_tiles;
        while (lo < hi) {
            const int64_t mid = lo + (hi - lo) / 2;
            int32_t mr;
            std::memcpy(&mr, reinterpret_cast<const uint8_t*>(t + mid) + offsetof(RsTile, r), sizeof mr);
            if (mr < x) lo = mid + 1; else hi = mid;
        }
        return lo;
    };
    *tile_begin = first_at_least(r);
    *tile_count = first_at_least(r + 1) - *tile_begin;
    return TIDE_OK;
}

}  // extern "C"
