/*
 * msa_oracle.c -- plain CPU oracle of the MiniMax Sparse Attention (MSA)
 * forward path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the HIP implementation and is never on the product
 * path.
 *
 * Everything is computed straight from the definitions, row by row, in fp64:
 *
 *   stage 1  s[t,g,j] = (q^I[t,g] . k^I[j]) / sqrt(d_I)        for j <= p
 *   stage 2  S[t,g,b] = max over j in block b with j <= p of s[t,g,j]
 *            (-inf for a block with no visible key)
 *   stage 3  selection = the forced local block local(t) = floor(p / Bk),
 *            plus the best min(k-1, local(t)) blocks among 0..local(t)-1,
 *            ranked by S descending, ties to the lower block index;
 *            written ascending into k slots, -1 padded
 *   stage 4  O[t,h] = softmax(q[t,h] K_g^T / sqrt(d_h)) V_g over exactly the
 *            keys j <= p of the selected blocks of h's group g = h / (Hq/G);
 *            lse = natural log of the softmax denominator (with the max added
 *            back)
 *   stage 4 backward  dq, dK, dV of sum(dO . O) over the same support, the
 *            selection held fixed (msa_oracle_attend_backward)
 *   index KL  the index branch's alignment loss KL(teacher || proxy) over
 *            each row's support and its gradients dq^I, dk^I
 *            (msa_oracle_index_kl_backward)
 *
 * Sources (the MSA study-notes page, dimensionstp.github.io/study-concept/msa):
 *   stages 1-3: section 2-3 "Fixed attention budget", the three displayed
 *     equations for s, S and the block set B; section 3-2 (max pooling of
 *     causally visible token scores); section 3-4 (the local block is always
 *     selected, no sink, no window).
 *   budget: section 2-3 text (block size 128, top-k 16, at most 2048 tokens
 *     per query and group counting the local block); the chipsbuilder news
 *     page ("Che cos'e MSA": k*Bk = 2,048) agrees.
 *   stage 4: section 1-1 (the causal GQA attention formula) restricted to the
 *     support, section 2-3 (Main Branch equation), section 3-3 (exact softmax
 *     on the support, per-head weights, selection shared by the group).
 *
 * Readings where the pages are silent (all stated in the design notes):
 *   - k counts the local block (budget k*Bk tokens including it);
 *   - ties go to the lower block index;
 *   - query row t of a sequence sits at position p = N - T + t (prefill
 *     T == N, decode T == 1 with the new token last in the cache);
 *   - heads map to groups contiguously, g = h / (Hq / G);
 *   - a block that is not yet visible scores -inf and is never a candidate;
 *     the local block's S is its true causal max (selection ignores it).
 *
 * Inputs are the raw bf16 bit patterns (uint16), or for the index branch's
 * 8-bit variant the OCP E4M3 codes (one byte; the Italian news page on MSA,
 * "Co-Design Del Kernel", lists FP8 among the authors' kernel precisions);
 * either is widened to fp64 exactly.  Row-subset mode: every function works on a caller-chosen list of
 * (b, t) query rows so that very long workloads can be checked on a sample.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t B, T, N;
    int32_t Hq, G, d_h, d_I, Bk, k;
} msa_oracle_dims;

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int64_t position_of(const msa_oracle_dims *d, int64_t t)
{
    return d->N - d->T + t;
}

static int64_t block_count(const msa_oracle_dims *d)
{
    return (d->N + d->Bk - 1) / d->Bk;
}

int msa_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One OCP 8-bit E4M3 value (the "fp8" of the index branch variant): sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
 * subnormals M * 2^-9; exponent 15 with mantissa 7 is NaN and there is no
 * infinity. */
static double widen_e4m3(uint8_t code)
{
    const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Widens values [i0, i0 + n) of a bf16 (fp8 == 0) or E4M3 (fp8 != 0) array. */
static void widen_run(const void *base, int64_t i0, int64_t n, int fp8, double *out)
{
    if (fp8) {
        const uint8_t *v = (const uint8_t *)base + i0;
        for (int64_t c = 0; c < n; ++c)
            out[c] = widen_e4m3(v[c]);
    } else {
        const uint16_t *v = (const uint16_t *)base + i0;
        for (int64_t c = 0; c < n; ++c)
            out[c] = widen_bf16(v[c]);
    }
}

/* Stages 1 and 2.  S[r, g, blk] for every listed row r = (row_b[r], row_t[r]).
 * qI_rows: [nrows, G, d_I] (the q^I vectors of the listed rows only),
 * kI: [B, N, d_I]; bf16 bit patterns, or E4M3 codes when fp8 != 0. */
static void block_scores(const msa_oracle_dims *d, int64_t nrows, const int64_t *row_b,
                         const int64_t *row_t, const void *qI_rows, const void *kI,
                         int fp8, double *S)
{
    const int64_t NB = block_count(d);
    const double root = sqrt((double)d->d_I);
    const int64_t G = d->G, dI = d->d_I;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t rg = 0; rg < nrows * G; ++rg) {
        const int64_t r = rg / G, g = rg % G;
        const int64_t b = row_b[r];
        const int64_t p = position_of(d, row_t[r]);
        double *out = S + (r * G + g) * NB;
        double *qd = (double *)malloc(sizeof(double) * dI);
        double *kd = (double *)malloc(sizeof(double) * dI);
        widen_run(qI_rows, (r * G + g) * dI, dI, fp8, qd);
        for (int64_t blk = 0; blk < NB; ++blk)
            out[blk] = -INFINITY;
        for (int64_t j = 0; j <= p; ++j) {
            widen_run(kI, (b * d->N + j) * dI, dI, fp8, kd);
            double dot = 0.0;
            for (int64_t c = 0; c < dI; ++c)
                dot += qd[c] * kd[c];
            const double s = dot / root;
            const int64_t blk = j / d->Bk;
            if (s > out[blk])
                out[blk] = s;
        }
        free(kd);
        free(qd);
    }
}

/* Stages 1 and 2 on bf16 inputs (uint16 bit patterns). */
void msa_oracle_block_scores(const msa_oracle_dims *d, int64_t nrows,
                             const int64_t *row_b, const int64_t *row_t,
                             const uint16_t *qI_rows, const uint16_t *kI,
                             double *S)
{
    block_scores(d, nrows, row_b, row_t, qI_rows, kI, 0, S);
}

/* Stages 1 and 2 on fp8 E4M3 inputs (one byte per value). */
void msa_oracle_block_scores_fp8(const msa_oracle_dims *d, int64_t nrows,
                                 const int64_t *row_b, const int64_t *row_t,
                                 const uint8_t *qI_rows, const uint8_t *kI, double *S)
{
    block_scores(d, nrows, row_b, row_t, qI_rows, kI, 1, S);
}

/* The value of each of the 256 E4M3 codes (for the oracle's own checks). */
void msa_oracle_e4m3_values(double *out)
{
    for (int c = 0; c < 256; ++c)
        out[c] = widen_e4m3((uint8_t)c);
}

/* Stage 3.  idx[r, g, 0..k-1] from S[r, g, 0..NB-1]. */
void msa_oracle_select(const msa_oracle_dims *d, int64_t nrows,
                       const int64_t *row_t, const double *S, int32_t *idx)
{
    const int64_t NB = block_count(d);
    const int64_t G = d->G, k = d->k;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t rg = 0; rg < nrows * G; ++rg) {
        const int64_t r = rg / G;
        const int64_t p = position_of(d, row_t[r]);
        const int64_t local = p / d->Bk;
        const double *sc = S + rg * NB;
        int32_t *out = idx + rg * k;
        const int64_t want = (k - 1 < local) ? k - 1 : local;
        char *taken = (char *)calloc((size_t)(local > 0 ? local : 1), 1);
        int64_t *chosen = (int64_t *)malloc(sizeof(int64_t) * (size_t)(want + 1));
        /* Repeatedly take the best remaining candidate.  The strict ">" keeps
         * the earliest (lowest) block among equal scores. */
        for (int64_t n = 0; n < want; ++n) {
            int64_t best = -1;
            for (int64_t c = 0; c < local; ++c) {
                if (taken[c])
                    continue;
                if (best < 0 || sc[c] > sc[best])
                    best = c;
            }
            taken[best] = 1;
            chosen[n] = best;
        }
        free(taken);
        /* ascending block order */
        for (int64_t a = 1; a < want; ++a) {
            int64_t v = chosen[a], z = a - 1;
            while (z >= 0 && chosen[z] > v) {
                chosen[z + 1] = chosen[z];
                --z;
            }
            chosen[z + 1] = v;
        }
        for (int64_t s = 0; s < k; ++s)
            out[s] = -1;
        for (int64_t s = 0; s < want; ++s)
            out[s] = (int32_t)chosen[s];
        out[want] = (int32_t)local;
        free(chosen);
    }
}

/* Stage 4.  O[r, h, :] and lse[r, h] for every listed row and every head.
 * q_rows: [nrows, Hq, d_h]; K, V: [B, G, N, d_h]; idx: [nrows, G, k]. */
void msa_oracle_attend(const msa_oracle_dims *d, int64_t nrows,
                       const int64_t *row_b, const int64_t *row_t,
                       const uint16_t *q_rows, const uint16_t *K,
                       const uint16_t *V, const int32_t *idx, double *O,
                       double *lse)
{
    const int64_t Hq = d->Hq, G = d->G, dh = d->d_h, k = d->k;
    const int64_t hg = Hq / G;
    const double root = sqrt((double)dh);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t rh = 0; rh < nrows * Hq; ++rh) {
        const int64_t r = rh / Hq, h = rh % Hq;
        const int64_t g = h / hg;
        const int64_t b = row_b[r];
        const int64_t p = position_of(d, row_t[r]);
        const int32_t *sel = idx + (r * G + g) * k;
        const uint16_t *qv = q_rows + (r * Hq + h) * dh;
        double *qd = (double *)malloc(sizeof(double) * dh);
        double *z = (double *)malloc(sizeof(double) * (size_t)(k * d->Bk));
        int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)(k * d->Bk));
        for (int64_t c = 0; c < dh; ++c)
            qd[c] = widen_bf16(qv[c]);
        /* the support: visible keys of the distinct selected blocks */
        int64_t n = 0;
        for (int64_t s = 0; s < k; ++s) {
            const int64_t blk = sel[s];
            if (blk < 0)
                continue;
            int dup = 0;
            for (int64_t u = 0; u < s; ++u)
                if (sel[u] == blk)
                    dup = 1;
            if (dup)
                continue;
            for (int64_t j = blk * d->Bk; j < (blk + 1) * d->Bk && j <= p; ++j)
                key[n++] = j;
        }
        const uint16_t *Kg = K + (b * G + g) * d->N * dh;
        const uint16_t *Vg = V + (b * G + g) * d->N * dh;
        double m = -INFINITY;
        for (int64_t i = 0; i < n; ++i) {
            const uint16_t *kv = Kg + key[i] * dh;
            double dot = 0.0;
            for (int64_t c = 0; c < dh; ++c)
                dot += qd[c] * widen_bf16(kv[c]);
            z[i] = dot / root;
            if (z[i] > m)
                m = z[i];
        }
        double l = 0.0;
        double *o = O + (r * Hq + h) * dh;
        for (int64_t c = 0; c < dh; ++c)
            o[c] = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            const double w = exp(z[i] - m);
            l += w;
            const uint16_t *vv = Vg + key[i] * dh;
            for (int64_t c = 0; c < dh; ++c)
                o[c] += w * widen_bf16(vv[c]);
        }
        for (int64_t c = 0; c < dh; ++c)
            o[c] /= l;
        lse[r * Hq + h] = m + log(l);
        free(qd);
        free(z);
        free(key);
    }
}

/* Stage 4 backward.  The selection is a constant of the step (the discrete
 * top-k has no gradient; the Flash-MSA training blog, "Backward pass", keeps
 * the forward's block indices for it), so the gradients are those of exact
 * softmax attention over each row's support.  With L = sum over rows and heads
 * of dO . O, per (row, head), over the support keys j:
 *   z_j  = q . K_j / sqrt(d_h)          P_j = softmax(z)_j
 *   dP_j = dO . V_j                     dz_j = P_j (dP_j - sum_i P_i dP_i)
 *   dq   = sum_j dz_j K_j / sqrt(d_h)
 *   dK_j += dz_j q / sqrt(d_h)          dV_j += P_j dO
 * (the softmax Jacobian dP_i/dz_j = P_i (delta_ij - P_j) applied to dL/dP).
 * dq: [nrows, Hq, d_h] for the listed rows.  dK, dV: [B, G, nblk*Bk, d_h],
 * the keys of blocks blk_lo .. blk_lo+nblk-1; they receive the contributions
 * of the listed rows only (contributions to other keys are dropped), so a
 * window of blocks is exact when every row that selects one of its blocks is
 * listed.  Row-parallel over (sequence, head); a head's contributions are
 * summed into the group in head order. */
void msa_oracle_attend_backward(const msa_oracle_dims *d, int64_t nrows,
                                const int64_t *row_b, const int64_t *row_t,
                                const uint16_t *q_rows, const uint16_t *dO_rows,
                                const uint16_t *K, const uint16_t *V,
                                const int32_t *idx, int64_t blk_lo, int64_t nblk,
                                double *dq, double *dK, double *dV)
{
    const int64_t Hq = d->Hq, G = d->G, dh = d->d_h, k = d->k, Bk = d->Bk;
    const int64_t hg = Hq / G;
    const int64_t wkeys = nblk * Bk, key_lo = blk_lo * Bk;
    const double root = sqrt((double)dh);
    const size_t per_head = (size_t)(wkeys * dh);
    double *hk = (double *)calloc((size_t)(d->B * Hq) * per_head, sizeof(double));
    double *hv = (double *)calloc((size_t)(d->B * Hq) * per_head, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < d->B * Hq; ++bh) {
        const int64_t b = bh / Hq, h = bh % Hq, g = h / hg;
        double *myk = hk + (size_t)bh * per_head;
        double *myv = hv + (size_t)bh * per_head;
        double *qd = (double *)malloc(sizeof(double) * dh);
        double *go = (double *)malloc(sizeof(double) * dh);
        double *z = (double *)malloc(sizeof(double) * (size_t)(k * Bk));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(k * Bk));
        int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)(k * Bk));
        const uint16_t *Kg = K + (b * G + g) * d->N * dh;
        const uint16_t *Vg = V + (b * G + g) * d->N * dh;
        for (int64_t r = 0; r < nrows; ++r) {
            if (row_b[r] != b)
                continue;
            const int64_t p = position_of(d, row_t[r]);
            const int32_t *sel = idx + (r * G + g) * k;
            for (int64_t c = 0; c < dh; ++c) {
                qd[c] = widen_bf16(q_rows[(r * Hq + h) * dh + c]);
                go[c] = widen_bf16(dO_rows[(r * Hq + h) * dh + c]);
            }
            /* the support: visible keys of the distinct selected blocks */
            int64_t n = 0;
            for (int64_t s = 0; s < k; ++s) {
                const int64_t blk = sel[s];
                if (blk < 0)
                    continue;
                int dup = 0;
                for (int64_t u = 0; u < s; ++u)
                    if (sel[u] == blk)
                        dup = 1;
                if (dup)
                    continue;
                for (int64_t j = blk * Bk; j < (blk + 1) * Bk && j <= p; ++j)
                    key[n++] = j;
            }
            double m = -INFINITY;
            for (int64_t i = 0; i < n; ++i) {
                double dot = 0.0, dv = 0.0;
                for (int64_t c = 0; c < dh; ++c) {
                    dot += qd[c] * widen_bf16(Kg[key[i] * dh + c]);
                    dv += go[c] * widen_bf16(Vg[key[i] * dh + c]);
                }
                z[i] = dot / root;
                dp[i] = dv;
                if (z[i] > m)
                    m = z[i];
            }
            double l = 0.0;
            for (int64_t i = 0; i < n; ++i) {
                z[i] = exp(z[i] - m); /* z now holds the unnormalised P */
                l += z[i];
            }
            double pdp = 0.0;
            for (int64_t i = 0; i < n; ++i) {
                z[i] /= l;
                pdp += z[i] * dp[i];
            }
            double *dqr = dq + (r * Hq + h) * dh;
            for (int64_t c = 0; c < dh; ++c)
                dqr[c] = 0.0;
            for (int64_t i = 0; i < n; ++i) {
                const double dz = z[i] * (dp[i] - pdp);
                const uint16_t *kv = Kg + key[i] * dh;
                for (int64_t c = 0; c < dh; ++c)
                    dqr[c] += dz * widen_bf16(kv[c]) / root;
                const int64_t kw = key[i] - key_lo;
                if (kw < 0 || kw >= wkeys)
                    continue;
                for (int64_t c = 0; c < dh; ++c) {
                    myk[kw * dh + c] += dz * qd[c] / root;
                    myv[kw * dh + c] += z[i] * go[c];
                }
            }
        }
        free(qd);
        free(go);
        free(z);
        free(dp);
        free(key);
    }
    /* group sums, heads in order */
    for (int64_t b = 0; b < d->B; ++b)
        for (int64_t g = 0; g < G; ++g) {
            double *ok = dK + (size_t)(b * G + g) * per_head;
            double *ov = dV + (size_t)(b * G + g) * per_head;
            for (size_t e = 0; e < per_head; ++e) {
                ok[e] = 0.0;
                ov[e] = 0.0;
            }
            for (int64_t h = g * hg; h < (g + 1) * hg; ++h) {
                const double *sk = hk + (size_t)(b * Hq + h) * per_head;
                const double *sv = hv + (size_t)(b * Hq + h) * per_head;
                for (size_t e = 0; e < per_head; ++e) {
                    ok[e] += sk[e];
                    ov[e] += sv[e];
                }
            }
        }
    free(hk);
    free(hv);
}

/* Index-branch KL alignment, backward.  Per row and group, over the row's
 * support J (the visible keys of its selected blocks):
 *   teacher  p_t(j)  = mean over the group's heads h of the main attention
 *            weights softmax_J(q_h . K_j / sqrt(d_h)) (detached: no gradient
 *            flows into q, K; study notes section 4-2 and 4-3);
 *   proxy    p_x(j)  = softmax_J(s_j), s_j = q^I . k^I_j / sqrt(d_I) (the index
 *            scores of stage 1, renormalised over the support, as the
 *            Flash-MSA blog recomputes the proxy lse on the sparse support);
 *   loss     KL(p_t || p_x) = sum_j p_t(j) (log p_t(j) - log p_x(j));
 *   dL/ds_j  = p_x(j) - p_t(j)  (the blog's "KL divergence loss" section);
 *   dq^I     = sum_j (p_x(j) - p_t(j)) k^I_j / sqrt(d_I);
 *   dk^I_j  += (p_x(j) - p_t(j)) q^I / sqrt(d_I), summed over rows and groups.
 * qI_rows [nrows, G, d_I], q_rows [nrows, Hq, d_h], kI [B, N, d_I],
 * K [B, G, N, d_h], idx [nrows, G, k].  Out: dqI [nrows, G, d_I];
 * dkI [B, nblk*Bk, d_I] for the keys of blocks blk_lo .. blk_lo+nblk-1
 * (contributions of the listed rows only); kl [nrows, G]. */
void msa_oracle_index_kl_backward(const msa_oracle_dims *d, int64_t nrows,
                                  const int64_t *row_b, const int64_t *row_t,
                                  const uint16_t *qI_rows, const uint16_t *kI,
                                  const uint16_t *q_rows, const uint16_t *K,
                                  const int32_t *idx, int64_t blk_lo, int64_t nblk,
                                  double *dqI, double *dkI, double *kl)
{
    const int64_t Hq = d->Hq, G = d->G, dh = d->d_h, dI = d->d_I, k = d->k, Bk = d->Bk;
    const int64_t hg = Hq / G;
    const int64_t wkeys = nblk * Bk, key_lo = blk_lo * Bk;
    const double root_h = sqrt((double)dh), root_i = sqrt((double)dI);
    const size_t per_bg = (size_t)(wkeys * dI);
    double *gk = (double *)calloc((size_t)(d->B * G) * per_bg, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bgi = 0; bgi < d->B * G; ++bgi) {
        const int64_t b = bgi / G, g = bgi % G;
        double *myk = gk + (size_t)bgi * per_bg;
        double *qi = (double *)malloc(sizeof(double) * dI);
        double *qh = (double *)malloc(sizeof(double) * dh);
        double *pt = (double *)malloc(sizeof(double) * (size_t)(k * Bk));
        double *z = (double *)malloc(sizeof(double) * (size_t)(k * Bk));
        double *px = (double *)malloc(sizeof(double) * (size_t)(k * Bk));
        int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)(k * Bk));
        const uint16_t *Kg = K + (b * G + g) * d->N * dh;
        const uint16_t *kIb = kI + b * d->N * dI;
        for (int64_t r = 0; r < nrows; ++r) {
            if (row_b[r] != b)
                continue;
            const int64_t p = position_of(d, row_t[r]);
            const int32_t *sel = idx + (r * G + g) * k;
            int64_t n = 0;
            for (int64_t s = 0; s < k; ++s) {
                const int64_t blk = sel[s];
                if (blk < 0)
                    continue;
                int dup = 0;
                for (int64_t u = 0; u < s; ++u)
                    if (sel[u] == blk)
                        dup = 1;
                if (dup)
                    continue;
                for (int64_t j = blk * Bk; j < (blk + 1) * Bk && j <= p; ++j)
                    key[n++] = j;
            }
            /* teacher: mean over the group's heads of the main weights */
            for (int64_t i = 0; i < n; ++i)
                pt[i] = 0.0;
            for (int64_t h = g * hg; h < (g + 1) * hg; ++h) {
                for (int64_t c = 0; c < dh; ++c)
                    qh[c] = widen_bf16(q_rows[(r * Hq + h) * dh + c]);
                double m = -INFINITY;
                for (int64_t i = 0; i < n; ++i) {
                    double dot = 0.0;
                    for (int64_t c = 0; c < dh; ++c)
                        dot += qh[c] * widen_bf16(Kg[key[i] * dh + c]);
                    z[i] = dot / root_h;
                    if (z[i] > m)
                        m = z[i];
                }
                double l = 0.0;
                for (int64_t i = 0; i < n; ++i) {
                    z[i] = exp(z[i] - m);
                    l += z[i];
                }
                for (int64_t i = 0; i < n; ++i)
                    pt[i] += z[i] / l / (double)hg;
            }
            /* proxy: softmax of the index scores over the same support */
            for (int64_t c = 0; c < dI; ++c)
                qi[c] = widen_bf16(qI_rows[(r * G + g) * dI + c]);
            double m = -INFINITY;
            for (int64_t i = 0; i < n; ++i) {
                double dot = 0.0;
                for (int64_t c = 0; c < dI; ++c)
                    dot += qi[c] * widen_bf16(kIb[key[i] * dI + c]);
                px[i] = dot / root_i;
                if (px[i] > m)
                    m = px[i];
            }
            double l = 0.0;
            for (int64_t i = 0; i < n; ++i)
                l += exp(px[i] - m);
            const double lse = m + log(l);
            double loss = 0.0;
            double *dq = dqI + (r * G + g) * dI;
            for (int64_t c = 0; c < dI; ++c)
                dq[c] = 0.0;
            for (int64_t i = 0; i < n; ++i) {
                const double logx = px[i] - lse;
                if (pt[i] > 0.0)
                    loss += pt[i] * (log(pt[i]) - logx);
                const double dz = exp(logx) - pt[i];
                const uint16_t *kv = kIb + key[i] * dI;
                for (int64_t c = 0; c < dI; ++c)
                    dq[c] += dz * widen_bf16(kv[c]) / root_i;
                const int64_t kw = key[i] - key_lo;
                if (kw < 0 || kw >= wkeys)
                    continue;
                for (int64_t c = 0; c < dI; ++c)
                    myk[kw * dI + c] += dz * qi[c] / root_i;
            }
            kl[r * G + g] = loss;
        }
        free(qi);
        free(qh);
        free(pt);
        free(z);
        free(px);
        free(key);
    }
    /* the shared index keys: sum over groups, in group order */
    for (int64_t b = 0; b < d->B; ++b) {
        double *o = dkI + (size_t)b * per_bg;
        for (size_t e = 0; e < per_bg; ++e)
            o[e] = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            const double *sg = gk + (size_t)(b * G + g) * per_bg;
            for (size_t e = 0; e < per_bg; ++e)
                o[e] += sg[e];
        }
    }
    free(gk);
}
