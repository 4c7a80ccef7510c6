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

}  // namespace tide
