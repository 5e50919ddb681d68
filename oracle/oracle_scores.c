/*
 * Oracle (test infrastructure only): pooled block scores of block-sparse
 * video attention, computed the slow, plain way on the CPU.
 *
 * Nothing on the product path links or calls this file; only the tests,
 * the package's smoke check and the benchmark's CPU-baseline leg do.
 *
 * What it computes.  The score of a query block i against a key block j is
 * the scaled dot product of the two block centroids (the block "mean" of
 * the DFSAttn page, "2. Sub-block scoring"; the centroid of the SVG-EAR
 * page, "2. Metodologia, A"), i.e. the block-level attention score the
 * SVG-EAR page, "1. O Problema" says existing routers select on.
 *
 * Numeric definition (the one every implementation must reproduce bit for
 * bit, because the selection mask is decided on these fp32 values):
 *     acc = +0.0f;  for c = 0..d-1:  acc = fmaf(q[c], k[c], acc);
 *     score = sigma * acc            (one fp32 multiply)
 * i.e. a sequential fused-multiply-add dot product in channel order.
 *
 * Built with -ffp-contract=off so that the compiler adds no contraction of
 * its own; fmaf() is the correctly rounded C99 fused multiply-add.
 */
#include <math.h>
#include <stdint.h>

/* out[i*nk + j] = sigma * seqfma_dot(qm[i,:], km[j,:]) ; row-major inputs */
void oracle_block_scores(const float* qm, const float* km, int64_t nq,
                         int64_t nk, int64_t d, float sigma, float* out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < nq; ++i) {
        const float* q = qm + i * d;
        for (int64_t j = 0; j < nk; ++j) {
            const float* k = km + j * d;
            float acc = 0.0f;
            for (int64_t c = 0; c < d; ++c)
                acc = fmaf(q[c], k[c], acc);
            out[i * nk + j] = sigma * acc;
        }
    }
}

/* The same fused-multiply-add chain for one pair of vectors (used by the
 * oracle's own pins to compare against an exact-rational emulation). */
float oracle_seqfma_dot(const float* a, const float* b, int64_t d)
{
    float acc = 0.0f;
    for (int64_t c = 0; c < d; ++c)
        acc = fmaf(a[c], b[c], acc);
    return acc;
}
