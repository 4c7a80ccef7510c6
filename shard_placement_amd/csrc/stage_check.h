// stage_check.h -- validation of staging buffers for the copy-engine-staged
// reduce-scatter (shared by the copy-engine staging in dma.cpp and the fold
// launch in rs.hip).  Host code only.
#pragma once

#include <stdint.h>

#include "tide.h"

namespace tide {

// h_stage[r] (r < R) is the device address of rank r's staging buffer of R
// slots, slot q at h_stage[r] + 2 * q * slot_stride bytes, each slot laid out
// like rank r's fp32 arena (param p at element offset off[p]), in bf16.
// Checks: the plan has reduce-scatter pointers; slot_stride >= S; every
// buffer non-NULL and 2-byte aligned; the R buffers overlap neither each
// other, nor any gradient tensor, nor any output arena.  *vec_ok says whether
// every buffer and the slot stride are 16-byte aligned (vector loads).
tide_status check_stage(const void* h_plan, const uint64_t* h_stage, int64_t slot_stride,
                        bool* vec_ok);

// Whether the byte range [lo, hi) overlaps any gradient tensor or any
// output arena of the plan (a reduce-scatter plan).
bool overlaps_rs_buffers(const void* h_plan, uint64_t lo, uint64_t hi);

// Checks shared by the two-phase pipeline calls: a reduce-scatter plan, a
// valid tile range, a 16-byte aligned staging chunk of at least
// tile_count * rs_tile floats that overlaps no gradient or output arena, a
// 16-byte aligned device plan (when d_plan is not NULL).  On success *h
// holds the plan header.
struct PlanHeader;
tide_status check_pipeline(const void* h_plan, const void* d_plan, int64_t tile_begin,
                           int64_t tile_count, const float* stage, int64_t stage_elems,
                           int32_t max_workgroups, PlanHeader* h);

// The two phases' launches and copies, without the checks: for callers that
// have validated the plan, the tile range and the staging memory already
// (the pipeline driver checks its whole ring once, then issues chunk by
// chunk).  h is the plan's header.
tide_status issue_tiles_to_stage(const PlanHeader& h, const void* d_plan, int64_t tile_begin,
                                 int64_t tile_count, float* stage, int32_t max_workgroups,
                                 tide_stream_t stream);
tide_status issue_stage_to_shards(const PlanHeader& h, const void* d_plan, int64_t tile_begin,
                                  int64_t tile_count, const float* stage, int32_t max_workgroups,
                                  tide_stream_t stream);
tide_status issue_stage_to_shards_sdma(const PlanHeader& h, const void* h_plan,
                                       int64_t tile_begin, int64_t tile_count, const float* stage,
                                       tide_stream_t stream);

}  // namespace tide
