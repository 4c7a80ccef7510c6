/*
 * tide_oracle.c -- plain CPU oracle for the node-local data path of TIDE's
 * layout-aware FSDP2 collectives.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or table with the HIP
 * library; it is written from the method's definition, not from that code.
 *
 * Sources (cited by page and section, never by line):
 *   [Abstract]   "The Endgame of FSDP Communication: Layout-Aware Collectives
 *                on Copy Engines, RDMA, and NVSwitch" (weekinpapers.com),
 *                section Abstract.  FSDP2 keeps one gradient tensor per
 *                parameter; TIDE-RS reads those bf16 tensors where they lie
 *                and sums them into fp32 shards; TIDE-AG writes shards into
 *                the parameters' own storage without a copy-out pass.
 *   [Root]       kongchang.com article "The Endgame of FSDP Communication:
 *                TIDE Zero-Copy Collective Communication Optimization",
 *                section "The Root of FSDP2 Communication Overhead": the
 *                rank-major buffer (each rank's block contiguous, blocks in
 *                rank order) and what a reduce-scatter does (each rank
 *                starts from a whole buffer and keeps only the sum of its
 *                own shard).
 *
 * Readings taken where the pages are silent (each is also listed with its
 * reason in the design notes):
 *   R1 shard rule: rank r owns dim-0 rows [r*s, r*s+s) with s = ceil(d0/R);
 *      rows >= d0 are padding.  A param of shape [d0, rest...] is flattened
 *      to d0 rows of c = prod(rest) elements (c = 1 for 1-D; a 0-d param is
 *      one row of one element).
 *   R2 padding value: +0.0f (all bits clear), written, never read.
 *   R3 reduction: fp32, fixed rank order 0..R-1, starting from rank 0's
 *      widened value (acc = g0; acc = acc + g1; ...), one IEEE binary32
 *      round-to-nearest-even add per step, subnormals kept.  Optional tree
 *      order: adjacent pairs level by level, an odd last element carried up
 *      unchanged.
 *   R4 arena layout: rank r's fp32 shards of all params sit in one arena in
 *      parameter order, param p at element offset off[p] = sum over p' < p of
 *      round_up(m[p'], align), with m = s*c.  A bf16 gathered slot uses the
 *      same offsets; the gathered buffer holds R slots of S elements each
 *      (S = total after the last param), slot r at element r*S.
 *   R5 all-gather placement copies, for each param p and rank r, the
 *      v = clamp(d0 - r*s, 0, s) valid rows of slot r to rows [r*s, r*s+v) of
 *      the full tensor; padding rows in the slot are never read.
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fopenmp
 *        -shared -fPIC (no flag that reassociates or flushes subnormals).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

/* MXCSR bits: flush-to-zero (bit 15), denormals-are-zero (bit 6), rounding
 * control (bits 13-14, 00 = nearest-even).  The host process may have set
 * any of them; the oracle clears them for its own arithmetic and restores
 * them afterwards, in every thread that does arithmetic. */
#define MXCSR_FTZ 0x8000u
#define MXCSR_DAZ 0x0040u
#define MXCSR_RC  0x6000u

static unsigned ieee_enter(void)
{
    unsigned saved = _mm_getcsr();
    _mm_setcsr(saved & ~(MXCSR_FTZ | MXCSR_DAZ | MXCSR_RC));
    return saved;
}

static void ieee_leave(unsigned saved) { _mm_setcsr(saved); }

/* bf16 is the upper half of a binary32: widening is exact. */
static float widen_bf16(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

int oracle_version(void) { return 1; }

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Shapes and offsets (readings R1, R4).  Outputs per param: chunk rows s,
 * shard numel m, offset off; and the slot numel S. */
int oracle_layout(int32_t P, const int64_t *dim0, const int64_t *rownumel,
                  int32_t R, int64_t align, int64_t *s_out, int64_t *m_out,
                  int64_t *off_out, int64_t *S_out)
{
    if (P < 0 || R < 1 || align < 1 || !S_out) return ORACLE_EINVAL;
    if (P > 0 && (!dim0 || !rownumel || !s_out || !m_out || !off_out))
        return ORACLE_EINVAL;
    int64_t off = 0;
    for (int32_t p = 0; p < P; ++p) {
        if (dim0[p] < 0 || rownumel[p] < 0) return ORACLE_EINVAL;
        int64_t s = ceil_div(dim0[p], R);
        int64_t m = s * rownumel[p];
        s_out[p] = s;
        m_out[p] = m;
        off_out[p] = off;
        off += round_up(m, align);
    }
    *S_out = off;
    return ORACLE_OK;
}

/* Reading R3, fixed order: start from rank 0, add ranks 1..R-1 in order. */
static float fold_fixed(const uint16_t *const *g, int32_t R, int64_t j)
{
    float acc = widen_bf16(g[0][j]);
    for (int32_t q = 1; q < R; ++q) acc = acc + widen_bf16(g[q][j]);
    return acc;
}

/* Reading R3, tree order: sum adjacent pairs level by level; an odd last
 * element moves up unchanged.  work has room for R floats. */
static float fold_tree(const uint16_t *const *g, int32_t R, int64_t j,
                       float *work)
{
    int32_t n = R;
    for (int32_t q = 0; q < R; ++q) work[q] = widen_bf16(g[q][j]);
    while (n > 1) {
        int32_t k = 0;
        int32_t i = 0;
        for (; i + 1 < n; i += 2) work[k++] = work[i] + work[i + 1];
        if (i < n) work[k++] = work[i];
        n = k;
    }
    return work[0];
}

/*
 * Reduce-scatter [Abstract; Root]: grads[q*P + p] points at rank q's bf16
 * gradient of param p (d0*c contiguous elements); out[r] points at rank r's
 * fp32 arena of at least S elements.  For every param p and every flat index
 * j of the padded tensor, 0 <= j < R*m, the element goes to rank j / m at
 * position j % m of that rank's shard: the fold over ranks if j < d0*c,
 * else +0.0f.  Alignment gaps between shards are left untouched.
 * order: 0 = fixed, 1 = tree.
 */
int oracle_rs(int32_t P, const int64_t *dim0, const int64_t *rownumel,
              int32_t R, int64_t align, int32_t order,
              const uint16_t *const *grads, float *const *out)
{
    if (P < 0 || R < 1 || align < 1 || (order != 0 && order != 1))
        return ORACLE_EINVAL;
    if (P == 0) return ORACLE_OK;
    if (!dim0 || !rownumel || !grads || !out) return ORACLE_EINVAL;
    int64_t *s = malloc(sizeof(int64_t) * (size_t)P * 3);
    if (!s) return ORACLE_ENOMEM;
    int64_t *m = s + P, *off = s + 2 * (size_t)P, S = 0;
    int rc = oracle_layout(P, dim0, rownumel, R, align, s, m, off, &S);
    if (rc != ORACLE_OK) { free(s); return rc; }
    for (int32_t r = 0; r < R; ++r)
        if (!out[r]) { free(s); return ORACLE_EINVAL; }

    const uint16_t **g = malloc(sizeof(*g) * (size_t)R);
    if (!g) { free(s); return ORACLE_ENOMEM; }
    int failed = 0;
    for (int32_t p = 0; p < P && !failed; ++p) {
        int64_t n = dim0[p] * rownumel[p];
        int64_t padded = (int64_t)R * m[p];
        for (int32_t q = 0; q < R; ++q) {
            g[q] = grads[(int64_t)q * P + p];
            if (!g[q] && n > 0) failed = 1;
        }
        if (failed) break;
#pragma omp parallel
        {
            unsigned saved = ieee_enter();
            float *work = order == 1 ? malloc(sizeof(float) * (size_t)R) : NULL;
            if (order == 1 && !work) {
#pragma omp atomic write
                failed = 2;
            }
#pragma omp for schedule(static)
            for (int64_t j = 0; j < padded; ++j) {
                int64_t r = j / m[p];
                int64_t i = j % m[p];
                float v = 0.0f;
                if (j < n) {
                    if (order == 0) v = fold_fixed(g, R, j);
                    else if (work) v = fold_tree(g, R, j, work);
                }
                out[r][off[p] + i] = v;
            }
            free(work);
            ieee_leave(saved);
        }
    }
    free(g);
    free(s);
    if (failed == 2) return ORACLE_ENOMEM;
    return failed ? ORACLE_EINVAL : ORACLE_OK;
}

/*
 * One element at a time, for sampled checks at full size: vals holds K
 * groups of R bf16 values (group k = the R ranks' values of one element, in
 * rank order); out[k] is their fold in the given order (0 fixed, 1 tree).
 */
int oracle_fold_points(int32_t R, int32_t order, int64_t K,
                       const uint16_t *vals, float *out)
{
    if (R < 1 || K < 0 || (order != 0 && order != 1)) return ORACLE_EINVAL;
    if (K == 0) return ORACLE_OK;
    if (!vals || !out) return ORACLE_EINVAL;
    const uint16_t **g = malloc(sizeof(*g) * (size_t)R);
    float *work = malloc(sizeof(float) * (size_t)R);
    if (!g || !work) { free(g); free(work); return ORACLE_ENOMEM; }
    unsigned saved = ieee_enter();
    for (int64_t k = 0; k < K; ++k) {
        for (int32_t q = 0; q < R; ++q) g[q] = vals + k * R + q;
        out[k] = order == 0 ? fold_fixed(g, R, 0) : fold_tree(g, R, 0, work);
    }
    ieee_leave(saved);
    free(g);
    free(work);
    return ORACLE_OK;
}

/*
 * All-gather placement [Abstract; Root], reading R5: gathered holds R slots
 * of S bf16 elements; full[p] is param p's bf16 tensor of d0*c elements.
 * Pure bit move; slot padding is never read; nothing outside the valid rows
 * of each full tensor is written.
 */
int oracle_ag(int32_t P, const int64_t *dim0, const int64_t *rownumel,
              int32_t R, int64_t align, const uint16_t *gathered,
              uint16_t *const *full)
{
    if (P < 0 || R < 1 || align < 1) return ORACLE_EINVAL;
    if (P == 0) return ORACLE_OK;
    if (!dim0 || !rownumel || !full) return ORACLE_EINVAL;
    int64_t *s = malloc(sizeof(int64_t) * (size_t)P * 3);
    if (!s) return ORACLE_ENOMEM;
    int64_t *m = s + P, *off = s + 2 * (size_t)P, S = 0;
    int rc = oracle_layout(P, dim0, rownumel, R, align, s, m, off, &S);
    if (rc != ORACLE_OK) { free(s); return rc; }
    if (S > 0 && !gathered) { free(s); return ORACLE_EINVAL; }
    for (int32_t p = 0; p < P; ++p) {
        if (dim0[p] * rownumel[p] > 0 && !full[p]) { free(s); return ORACLE_EINVAL; }
        for (int32_t r = 0; r < R; ++r) {
            int64_t v = dim0[p] - (int64_t)r * s[p];
            if (v < 0) v = 0;
            if (v > s[p]) v = s[p];
            const uint16_t *src = gathered + (int64_t)r * S + off[p];
            uint16_t *dst = full[p] + (int64_t)r * m[p];
            int64_t count = v * rownumel[p];
            for (int64_t k = 0; k < count; ++k) dst[k] = src[k];
        }
    }
    free(s);
    return ORACLE_OK;
}
