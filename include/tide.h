/*
 * tide.h -- C ABI of libtide: the node-local data path of TIDE's
 * layout-aware FSDP2 collectives on one MI355X (gfx950).
 *
 * Sources, cited by page and section:
 *   [Abstract]  "The Endgame of FSDP Communication: Layout-Aware Collectives
 *               on Copy Engines, RDMA, and NVSwitch" (weekinpapers.com),
 *               section Abstract.
 *   [Root]      kongchang.com article "The Endgame of FSDP Communication:
 *               TIDE Zero-Copy Collective Communication Optimization",
 *               section "The Root of FSDP2 Communication Overhead".
 *   [Design]    same article, section "TIDE's Design Approach".
 *
 * FSDP2 keeps gradients and parameters as per-parameter tensors while its
 * collectives use flat rank-major buffers; TIDE folds the placement into
 * the collectives' addressing [Abstract; Root].  This library does that for
 * R simulated ranks whose buffers all sit in one GPU's HBM:
 *
 *   reduce-scatter  R ranks' per-parameter bf16 gradients, read in place,
 *                   are reduced into each rank's fp32 dim-0 shards
 *                   [Abstract: TIDE-RS takes the bf16 gradient tensors
 *                   as they are and produces fp32 shards];
 *   AG placement    a rank-major bf16 gathered buffer [Root] is written
 *                   straight into the per-parameter full tensors, the
 *                   padding rows trimmed [Abstract: TIDE-AG puts shards
 *                   into the parameters' own storage].
 *
 * Layout conventions (the pages leave them open; these readings are the
 * library's contract):
 *   - A parameter of shape [d0, rest...] is d0 rows of c = prod(rest)
 *     elements (c = 1 for 1-D; a 0-d parameter is passed as {1, 1}).
 *   - Rank r owns rows [r*s, r*s + s), s = ceil(d0 / R) ("chunk rows");
 *     rows >= d0 are padding.  Shard numel m = s*c.
 *   - Rank r's fp32 arena holds param p's shard at element offset off[p] =
 *     sum over p' < p of round_up(m[p'], align_elems); slot numel S is the
 *     offset after the last param.  A bf16 gathered slot uses the same
 *     offsets; the gathered buffer is R slots, slot r at element r*S.
 *   - Shard element i of rank r for param p is the sum over ranks of flat
 *     gradient element j = r*m + i when j < d0*c, else +0.0f (padding).
 *     The sum is fp32, in rank order 0..R-1 starting from rank 0's value
 *     (order 0), or pairwise over adjacent ranks level by level with an odd
 *     last element carried up (order 1); each add is one IEEE binary32
 *     round-to-nearest-even add, subnormals kept.
 *
 * Memory and ownership: the caller owns every buffer, including the plan
 * blob (host) and its device copy.  The library allocates no device memory
 * (its one device array, the staging array of tide_rs_two_phase_noalloc, is
 * part of its code object).
 * Kernel launches are asynchronous on the caller's stream and synchronise
 * nothing; the copy-engine calls issued through ROCr (tide_ag_place_dma,
 * tide_rs_stage_dma) are host-synchronous instead (they wait for the
 * caller's stream, then for their copies).  The only state kept between
 * calls is, per device, the ROCr agent and copy-engine list those calls look
 * up once and the staging array's device address (each guarded by a
 * mutex).  Streams and pipeline objects the library
 * creates on request are the caller's to release.  A plan holds raw device addresses: it is
 * invalid once any of them is freed.
 *
 * Errors: every entry point returns a tide_status; nothing is thrown
 * across the ABI and no launch is made when validation fails.  Faults
 * during execution surface at the caller's next synchronisation.
 */
#ifndef TIDE_H
#define TIDE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TIDE_ABI_VERSION 2

/* A hipStream_t (struct ihipStream_t*); NULL is the null stream. */
struct ihipStream_t;
typedef struct ihipStream_t *tide_stream_t;

typedef enum tide_status {
    TIDE_OK = 0,
    TIDE_EINVAL = -1,       /* bad argument: NULL, R < 1, negative size, ... */
    TIDE_EALIGN = -2,       /* a pointer is not aligned to its element size */
    TIDE_EOVERLAP = -3,     /* an output range overlaps an input or output */
    TIDE_ENOSPACE = -4,     /* plan blob too small (needed size reported) */
    TIDE_EHIP = -5,         /* the HIP runtime refused a launch or copy */
    TIDE_EUNSUPPORTED = -6, /* valid request this plan cannot serve */
    TIDE_EPLAN = -7         /* not a plan blob, or wrong version */
} tide_status;

/* One parameter: d0 rows of row_numel elements (0-d => {1, 1}). */
typedef struct tide_shape {
    int64_t dim0;
    int64_t row_numel;
} tide_shape;

/* Plan options; pass NULL for the defaults. */
typedef struct tide_opts {
    int64_t align_elems;   /* arena/slot offset alignment, elements (>= 1; default 1) */
    int32_t rs_tile_elems; /* elements per reduce-scatter tile, multiple of 2048
                              (0: chosen from R, about 64 KB of traffic) */
    int32_t ag_tile_elems; /* elements per placement tile, multiple of 2048 (0: 2048) */
    int32_t flags;         /* -1: library default (both hints); else an OR of TIDE_FLAG_* */
    int32_t launch_mib;    /* algorithmic MiB moved per kernel launch: a call is cut
                              into launches of about this size, so that concurrent
                              kernels on other streams get whole compute units at
                              the launch boundaries (0: defaults, 160 MiB for the
                              reduce-scatter, rounded down to a multiple of 256
                              tiles (one per CU) when it holds fewer than 1024,
                              and at least 512 tiles; for R a multiple of 8 and
                              1024 to 2303 tiles, the fixed order's launches take
                              the nearest whole number of tiles per CU, at most 7
                              (one round of workgroups), and the tree order's
                              whole rounds of 4 per CU (4 or 8); 256 MiB for
                              the placement;
                              -1: one launch; an explicit size is not rounded) */
} tide_opts;

/* Access hints (results are identical with any combination). */
#define TIDE_FLAG_NT_LOADS  1  /* streaming (non-temporal) source loads */
#define TIDE_FLAG_NT_STORES 2  /* streaming (non-temporal) destination stores */

/* What a built plan holds (filled by tide_desc_build / tide_plan_query). */
typedef struct tide_plan_info {
    int32_t R, P;
    int64_t slot_numel;     /* S */
    int64_t numel;          /* N = sum of d0*c */
    int64_t padded_numel;   /* R*S minus alignment gaps = sum of R*m */
    int64_t rs_tiles;       /* 0 when the plan has no reduce-scatter pointers */
    int64_t ag_tiles;       /* 0 when the plan has no placement pointers */
    int32_t rs_tile_elems, ag_tile_elems;
    int64_t blob_bytes;     /* bytes of the blob in use: upload this many */
    int64_t rs_launch_tiles; /* tiles per reduce-scatter launch (fixed order) */
    int64_t ag_launch_tiles; /* tiles per placement launch */
    int64_t rs_lds_bytes;    /* LDS each reduce-scatter workgroup holds: 8 KB (what
                                the kernels use), or 64 KB when a default launch
                                holds at most 512 tiles (2 workgroups per CU), so
                                that two fill 128 of the CU's 160 KB and a concurrent
                                kernel's workgroup needing more than 32 KB cannot
                                start beside them */
} tide_plan_info;

/* Size of the plan blob for these shapes (an upper bound that holds for
 * any pointers).  shapes: P entries, host memory.  [Abstract: the
 * parameter layout becomes part of the collectives' addressing] */
tide_status tide_desc_size(const tide_shape *shapes, int32_t P, int32_t R,
                           const tide_opts *opts, size_t *blob_bytes);

/* Shard geometry without pointers (host only): per param the chunk rows
 * s = ceil(d0/R), shard numel m = s*c and arena/slot offset off; and the
 * slot numel S, so that a caller can size the fp32 arenas (S floats per
 * rank) and the gathered buffer (R*S bf16) before building a plan.  Each
 * output array has P entries (host memory) and may be NULL; slot_numel
 * must not be NULL. */
tide_status tide_desc_geometry(const tide_shape *shapes, int32_t P, int32_t R,
                               const tide_opts *opts, int64_t *chunk_rows,
                               int64_t *shard_numel, int64_t *offsets,
                               int64_t *slot_numel);

/* Build a plan (descriptor table) into caller host memory `blob`.
 *   grads     [R*P] device addresses, rank-major: grads[q*P + p] is rank q's
 *             bf16 gradient of param p (d0*c contiguous elements), or NULL
 *             for a plan without reduce-scatter;
 *   out_base  [R] device addresses of each rank's fp32 arena (>= S floats),
 *             NULL together with grads;
 *   gathered  device address of the bf16 gathered buffer (R*S elements), or
 *             NULL for a plan without placement;
 *   full      [P] device addresses of the bf16 full tensors (d0*c each),
 *             NULL together with gathered.
 * Pointer arrays are host memory and are read, not kept.  Validates
 * element alignment (2 B for bf16, 4 B for fp32) and that no reduce-scatter
 * output overlaps a gradient or another output, and no placement output
 * overlaps the gathered buffer or another output.  Reduce-scatter outputs
 * MAY overlap the gathered buffer (Slot-Reuse: shards staged in vacated
 * all-gather memory [Abstract; Design]).  Zero-sized params need no
 * pointer.  On TIDE_ENOSPACE, info->blob_bytes (if info) holds the size
 * needed.  info may be NULL.  [Abstract; Root] */
tide_status tide_desc_build(const tide_shape *shapes, int32_t P, int32_t R,
                            const tide_opts *opts, const void *const *grads,
                            void *const *out_base, const void *gathered,
                            void *const *full, void *blob, size_t blob_bytes,
                            tide_plan_info *info);

/* Read back what a host plan blob holds. */
tide_status tide_plan_query(const void *h_plan, tide_plan_info *info);

/* The reduce-scatter tiles of output rank r: the plan lists tiles rank by
 * rank (then param, then index), so they are one range [*tile_begin,
 * *tile_begin + *tile_count) for tide_rs_bf16_to_fp32_tiles -- what one GPU
 * of a real job would run for its own shard.  r in [0, R). */
tide_status tide_plan_rank_tiles(const void *h_plan, int32_t r, int64_t *tile_begin,
                                 int64_t *tile_count);

/* Fused reduce-scatter [Abstract: TIDE-RS; Root: each rank ends with the
 * reduction of its own shard].  h_plan: the host blob; d_plan: its device
 * copy (first info.blob_bytes bytes, 16-byte aligned), both unchanged
 * since the build.  order: 0 fixed rank order, 1 pairwise tree.
 * max_workgroups: 0 launches one short-lived workgroup per tile (fixed
 * order, R a multiple of 8, launches of 2048 tiles or more: about 3% more
 * workgroups, the even-numbered XCDs taking 33 of every 64 tiles, the odd
 * ones' spare workgroups exiting at once, because the odd XCDs run each
 * workgroup 5-9% longer); n > 0 caps the grid at n workgroups that stride
 * over the tiles.  Asynchronous on `stream`; allocates nothing. */
tide_status tide_rs_bf16_to_fp32(const void *h_plan, const void *d_plan,
                                 int32_t order, int32_t max_workgroups,
                                 tide_stream_t stream);

/* The same reduce-scatter restricted to tiles [tile_begin, tile_begin +
 * tile_count) of the plan (tide_plan_info.rs_tiles in all; tiles are listed
 * by output rank, then parameter, then flat index, so rank r's tiles are the
 * one range tide_plan_rank_tiles returns).  Lets a caller cut one
 * layer's reduce-scatter into several short launches, e.g. to leave the
 * compute units to concurrent work between them, or to pipeline the
 * gradient reads with a consumer of finished tiles [Abstract: the
 * reduce-scatter runs as two pipelined phases, reading gradients apart from
 * moving results over the network].  A range past
 * the end is TIDE_EINVAL; tile_count == 0 launches nothing. */
tide_status tide_rs_bf16_to_fp32_tiles(const void *h_plan, const void *d_plan,
                                       int32_t order, int64_t tile_begin,
                                       int64_t tile_count, int32_t max_workgroups,
                                       tide_stream_t stream);

/* The same launches dealt over n_streams streams in turn (launch i on
 * streams[i % n_streams]), so that with streams on different hardware queues
 * (e.g. from tide_stream_create_cu_limited) a launch can start on the CUs the
 * previous one is vacating instead of waiting for it to drain.  Same results.
 * Measured on MI355X with two queues: 6.46-6.57 TB/s against 5.99 on the
 * R = 64 layer, 5.92-6.08 against 5.58 on the R = 16 MoE layer, none on the
 * R = 8 layer; but a concurrent single-wave GEMM then loses the launch
 * boundaries that let it in (+12..92% against +1..7%): a mode for when no
 * compute runs beside the reduce-scatter.  The caller orders the streams
 * against its other work (e.g. the others wait for an event of the first,
 * the first waits for events of the others).  n_streams in [1, 64]; with
 * more than one stream none may be the null stream (TIDE_EINVAL: it
 * synchronises with every blocking stream, which would serialise the
 * launches; measured 72 ms against 19 ms for one stream).  The streams'
 * creation order matters too: two masked streams created one right after
 * the other kept 6.42-6.54 TB/s whatever the process created before or
 * after them (five ordinary streams, used), while a pair created one before
 * and one after five ordinary streams ran at 5.90 TB/s, the one-queue rate
 * (the runtime then no longer ran the two side by side; the mechanism was
 * not pinned down).  So create the streams to deal over one right after
 * the other. */
tide_status tide_rs_bf16_to_fp32_streams(const void *h_plan, const void *d_plan,
                                         int32_t order, int32_t max_workgroups,
                                         const tide_stream_t *streams, int32_t n_streams);

/* The reduce-scatter of tide_rs_bf16_to_fp32 (same launches, same
 * results) that also records, for every tile t of the plan, the compute
 * unit that processed it: census[t] = xcc_id << 8 | se_id << 5 | sh_id << 4
 * | cu_id (the GPU's hardware-ID registers).  census: device memory of at
 * least census_len >= rs_tiles uint32 words.  Counting the distinct values
 * gives the number of compute units the reduce-scatter occupied (the one-GPU
 * analog of the pages' reduce-scatter "SM time" [Abstract]). */
tide_status tide_rs_bf16_to_fp32_census(const void *h_plan, const void *d_plan,
                                        int32_t order, int32_t max_workgroups,
                                        uint32_t *census, int64_t census_len,
                                        tide_stream_t stream);

/* The census call that also times every tile: census[t] as above, and
 * stamps[2t], stamps[2t + 1] the GPU's constant-rate real-time counter
 * (100 MHz on MI355X: 10 ns ticks) read when the tile's workgroup starts it
 * and after all of the workgroup's waves have finished it.  From them the
 * caller gets the compute-unit time the reduce-scatter actually held (per
 * CU, the union of the intervals of its tiles), the occupancy-weighted
 * analog of the pages' reduce-scatter "SM time" [Abstract; Performance].
 * census: >= len uint32 words, stamps: >= 2 * len uint64 words (device
 * memory, 4- and 8-byte aligned), len >= rs_tiles.  The timing adds one
 * workgroup barrier per tile; results are those of tide_rs_bf16_to_fp32. */
tide_status tide_rs_bf16_to_fp32_trace(const void *h_plan, const void *d_plan,
                                       int32_t order, int32_t max_workgroups,
                                       uint32_t *census, uint64_t *stamps, int64_t len,
                                       tide_stream_t stream);

/* All-gather placement on the compute units [Abstract: TIDE-AG]: for
 * every param p and rank r, the clamp(d0 - r*s, 0, s) valid rows of slot r
 * are copied to rows [r*s, ...) of full[p]; slot padding is never read.
 * Arguments as for tide_rs_bf16_to_fp32. */
tide_status tide_ag_place(const void *h_plan, const void *d_plan,
                          int32_t max_workgroups, tide_stream_t stream);

/* The same placement issued as host-side copies from the host plan,
 * asynchronous on `stream` [Abstract: placement without compute units].
 * engine_only = 1: one 1-D copy per (param, rank) run with the runtime's
 * no-compute-unit copy kind (hipMemcpyDeviceToDeviceNoCU); the runtime
 * picks the engine: usually the DMA engines, but it has also been seen to
 * run such copies as small blit kernels, so only tide_ag_place_dma is
 * guaranteed to use no compute unit.  engine_only = 0: at most two copies per
 * param (a 2-D copy over the ranks with full shards, a 1-D copy for the
 * partial rank) of the ordinary device-to-device kind, which the runtime
 * executes with a blit kernel. */
tide_status tide_ag_place_sdma(const void *h_plan, int32_t engine_only,
                               tide_stream_t stream);

/* The engine-only placement with its copies spread over n_streams streams
 * (largest first, each to the stream with the fewest bytes so far), so
 * that several DMA engines can work at once.  The caller orders the
 * streams against its other work (e.g. with events).  Same copy kind, and
 * the same caveat, as engine_only = 1 above. */
tide_status tide_ag_place_sdma_streams(const void *h_plan, const tide_stream_t *streams,
                                       int32_t n_streams);

/* The same placement on the DMA copy engines, issued through ROCr: one 1-D
 * copy per (param, rank) run, each pinned to one engine, spread over all
 * the device's engines (largest first, each to the engine with the fewest
 * bytes so far) [Abstract: transport and placement kept off the compute
 * units].
 * Host-synchronous: waits for `stream` to finish its earlier work, then
 * returns when every copy has completed (no kernel runs).  Both waits are
 * bounded: at most 60 s for the stream, and 10 s plus 1 s per GB of copies
 * for the engines; past either deadline the call returns TIDE_EHIP.  After a
 * timeout on the copies they may still be running and writing their
 * destinations, so the caller must not free or reuse those buffers before
 * the device has been synchronised.  Do not overlap
 * it with the runtime's own copy-engine copies (tide_ag_place_sdma, D2H
 * copies) on the same device.  TIDE_EUNSUPPORTED: the device has no copy
 * engine the runtime reports. */
tide_status tide_ag_place_dma(const void *h_plan, tide_stream_t stream);

/* Number of DMA copy engines tide_ag_place_dma / tide_rs_stage_dma use on
 * the current device (*count = 0 and TIDE_EUNSUPPORTED if none). */
tide_status tide_dma_engine_count(int32_t *count);

/* Copy-engine-staged reduce-scatter [Abstract: data movement on the copy
 * engines, the sums in brief thread blocks; Design], in two calls.
 *
 * Staging buffers: h_stage[r] (host array of R device addresses) is rank
 * r's staging buffer of R slots of bf16; slot q starts slot_stride elements
 * after slot q-1 (slot_stride >= S) and is laid out like rank r's fp32
 * arena (param p at element off[p], m_p elements).  A rank's vacated
 * gathered buffer (R*S elements) is such a buffer with slot_stride = S.  The
 * buffers must not overlap each other, any gradient tensor or any output
 * arena (TIDE_EOVERLAP); they are 2-byte aligned (TIDE_EALIGN), and 16-byte
 * aligned buffers with slot_stride % 8 == 0 let the fold use 16-byte loads.
 *
 * Phase 1, tide_rs_stage_dma: for every param p, output rank r and source
 * rank q, the valid part of rank q's slice of p (flat indices [r*m_p,
 * r*m_p + v*c), v = clamp(d0 - r*s, 0, s)) is copied by the DMA engines to
 * slot q of h_stage[r] at element off[p]; padding rows are not copied.
 * Host-synchronous, with the same bounded waits, as tide_ag_place_dma.
 *
 * Phase 2, tide_rs_fold_staged: a kernel folds each rank's R slots into its
 * fp32 arena with the reduce-scatter's tiles, rank order and bits (padding
 * rows +0.0, read from nowhere).  d_stage: a device copy of the R
 * addresses (8-byte aligned).  Asynchronous on `stream`, cut into launches
 * like tide_rs_bf16_to_fp32; order 0 fixed, 1 tree. */
tide_status tide_rs_stage_dma(const void *h_plan, const uint64_t *h_stage,
                              int64_t slot_stride, tide_stream_t stream);
tide_status tide_rs_fold_staged(const void *h_plan, const void *d_plan, int32_t order,
                                const uint64_t *h_stage, const uint64_t *d_stage,
                                int64_t slot_stride, int32_t max_workgroups,
                                tide_stream_t stream);

/* Two-phase pipeline, one GPU's emulation [Abstract: two-phase pipeline;
 * Performance: reduce-scatter buffer nearly constant].  The reduce-scatter
 * of a tile range [tile_begin, tile_begin + tile_count) is split into
 *   phase 1, tide_rs_tiles_to_stage: the fixed-order reduction of those
 *     tiles into a dense staging chunk: tile t's results (len fp32 values;
 *     +0.0 for padding tiles) at stage + (t - tile_begin) * rs_tile_elems;
 *   phase 2, tide_rs_stage_to_shards: a copy of those results to their
 *     places in the fp32 arenas (the stand-in for the network phase that
 *     delivers partial results to their owners).
 * Phase 1 then phase 2 over every tile gives tide_rs_bf16_to_fp32's bits.
 * stage: device memory of stage_elems >= tile_count * rs_tile_elems floats,
 * 16-byte aligned, overlapping no gradient tensor or output arena (checked:
 * TIDE_EOVERLAP).  A caller runs the phases on two streams with an event
 * per chunk and a ring of staging chunks, so the staging memory is bounded
 * by the ring, not the layer.  Asynchronous on `stream`; cut into launches
 * of about the plan's launch size. */
tide_status tide_rs_tiles_to_stage(const void *h_plan, const void *d_plan, int64_t tile_begin,
                                   int64_t tile_count, float *stage, int64_t stage_elems,
                                   int32_t max_workgroups, tide_stream_t stream);
tide_status tide_rs_stage_to_shards(const void *h_plan, const void *d_plan, int64_t tile_begin,
                                    int64_t tile_count, const float *stage, int64_t stage_elems,
                                    int32_t max_workgroups, tide_stream_t stream);

/* Phase 2 with the runtime's no-compute-unit copy kind instead of a kernel
 * (a network stand-in that leaves the compute units alone when the runtime
 * gives the copies to the DMA engines; it may also run them as small blit
 * kernels, the caveat of tide_ag_place_sdma): one stream-ordered copy per
 * run of tiles contiguous in both the chunk and a rank's arena (measured
 * 5.2-5.3 ms for the 3.5 GB of shards of the R = 64 layer).  Asynchronous
 * on `stream`; same arguments and checks as tide_rs_stage_to_shards. */
tide_status tide_rs_stage_to_shards_sdma(const void *h_plan, int64_t tile_begin,
                                         int64_t tile_count, const float *stage,
                                         int64_t stage_elems, tide_stream_t stream);

/* A stream whose kernels may run only on the first n_cu compute units of
 * the device's CU mask (hipExtStreamCreateWithCUMask; default priority), for
 * confining the reduce-scatter's workgroups to part of the chip next to
 * concurrent compute [Abstract: interference with a concurrent GEMM].
 * n_cu in [1, number of CUs]; *out receives the stream; release it with
 * tide_stream_destroy.  Creating a stream synchronises nothing. */
tide_status tide_stream_create_cu_limited(int32_t n_cu, tide_stream_t *out);
/* The same for the mask bits [first_cu, first_cu + n_cu): two streams with
 * disjoint ranges never share a compute unit.  first_cu >= 0, n_cu >= 1,
 * first_cu + n_cu <= number of CUs.  On MI355X consecutive mask bits go to
 * the 8 XCDs in turn (bits [0, 8) are one CU on each XCD), and the runtime
 * refused masks of a single CU (TIDE_EHIP) while masks of 8, 16, 32, 64 and
 * 248 CUs worked. */
tide_status tide_stream_create_cu_range(int32_t first_cu, int32_t n_cu, tide_stream_t *out);
tide_status tide_stream_destroy(tide_stream_t stream);

/* The two-phase reduce-scatter pipeline, with its chunk loop issued by the
 * library [Abstract: the reduce-scatter runs as a two-phase pipeline whose
 * staging stays nearly constant; kongchang.com "Performance"].  Chunk i of
 * chunk_tiles plan tiles is reduced (tide_rs_tiles_to_stage) into slot
 * i % depth of a caller-owned ring of depth slots of chunk_tiles * rs_tile
 * floats, then moved to the shard arenas by phase 2 (phase2 = 0: the
 * tide_rs_stage_to_shards kernel; 1: the copy-kind copies of
 * tide_rs_stage_to_shards_sdma).  The phases run on two streams of the
 * pipeline object, created one right after the other (see
 * tide_rs_bf16_to_fp32_streams), each with a hardware queue of its own,
 * ordered per slot
 * by events: phase 2 of chunk i after its phase 1, phase 1 of chunk i after
 * phase 2 of chunk i - depth.  The result is bit-identical to
 * tide_rs_bf16_to_fp32 with order 0.
 *
 * tide_pipeline_create: depth in [1, 64]; phase2_cus = 0 lets both phases
 * use every CU, phase2_cus = k in [1, CUs) confines phase 2 to the mask
 * bits [0, k) (a consumer with a link's bandwidth) and phase 1 to the rest.
 * Creates two streams and 2 * depth + 3 events on the current device;
 * allocates no device memory.  tide_pipeline_destroy waits for the two
 * streams and releases them (the device is made current for the call).
 *
 * tide_pipeline_run: on the object's device; ring 16-byte aligned, at least
 * min(depth, chunks) * chunk_tiles * rs_tile floats (chunk_tiles is clamped
 * to the plan's tile count), overlapping no gradient or arena; phase2 = 1
 * only with phase2_cus = 0.  Ordered after the earlier work of `stream` and
 * before its later work; asynchronous.  All checks are made before anything
 * is issued.  Calls on one object must not overlap in time from several
 * host threads; calls issued one after another may share the ring, on the
 * same stream or not (a slot is refilled only after the phase 2 that last
 * drained it, also one of an earlier call).  The object's streams are CU-masked, which HIP creates as
 * blocking streams: calls issued back to back on the null stream, whose
 * pending work every blocking stream then waits on implicitly, measured up
 * to 20% slower than on another stream (or with the host waiting between
 * calls), so issue them from a stream other than the null stream. */
typedef struct tide_pipeline *tide_pipeline_t;
tide_status tide_pipeline_create(int32_t depth, int32_t phase2_cus, tide_pipeline_t *out);
tide_status tide_pipeline_run(tide_pipeline_t pipeline, const void *h_plan, const void *d_plan,
                              int64_t chunk_tiles, float *ring, int64_t ring_elems,
                              int32_t phase2, tide_stream_t stream);
tide_status tide_pipeline_destroy(tide_pipeline_t pipeline);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the two
 * phases above over tiles [tile_begin, tile_begin + tile_count) --
 * tide_rs_tiles_to_stage into a staging chunk, then tide_rs_stage_to_shards
 * from it into the shard arenas, both on `stream` -- with the staging chunk
 * in the library's own device array of TIDE_SCRATCH_BYTES instead of caller
 * memory.  The array is part of the library's code object: each device the
 * library runs on holds one until the process ends.  The results are those
 * of the two calls (and of tide_rs_bf16_to_fp32 with order 0 for the same
 * tiles).  tile_count * rs_tile_elems * 4 must not exceed
 * TIDE_SCRATCH_BYTES (TIDE_ENOSPACE otherwise; 4096 tiles of the default
 * 2048 elements fit); other checks as for tide_rs_tiles_to_stage.  Nothing
 * in the array needs clearing between calls (phase 1 writes every word that
 * phase 2 reads).  `stream` must belong to the calling thread's current
 * device (the null stream does), whose copy of the array the kernels use:
 * TIDE_EINVAL for a stream of another device.  Calls and the library
 * allocate nothing.  All calls on one
 * device share its array: calls issued one after another on one stream are
 * ordered, calls that overlap in time on one device (other streams or host
 * threads) race and give undefined results. */
#define TIDE_SCRATCH_BYTES (32u << 20)
tide_status tide_rs_two_phase_noalloc(const void *h_plan, const void *d_plan,
                                      int64_t tile_begin, int64_t tile_count,
                                      int32_t max_workgroups, tide_stream_t stream);

/* Static text for a status code. */
const char *tide_status_str(int32_t status);

/* TIDE_ABI_VERSION of the loaded library. */
int32_t tide_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TIDE_H */
