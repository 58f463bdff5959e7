/*
 * oracle.c -- plain, slow, float64 CPU reference of normalized kernelized linear attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's CPU-baseline leg
 * load this file's library. It shares no code, header, table or helper with the HIP library
 * and must never be used as a fallback for it.
 *
 * What it computes, and where the pages define it:
 *   feature map   phi(x) = ELU(x) + 1 with alpha = 1, i.e. x + 1 for x > 0 and exp(x) otherwise
 *                 ("Linear Attention: Accumulating KV in a Fixed-Size State", section
 *                 "Why replace softmax?"; "Linear Attention Math", section "Feature maps:
 *                 elu+1 and positive random features"). mode bit 0 selects phi(x) = x, the
 *                 feature-space convention of the pages' worked examples ("Store Values
 *                 according to Key components": q and k already denote mapped vectors).
 *   causal form   S_t = S_{t-1} + phi(k_t) v_t^T,  z_t = z_{t-1} + phi(k_t),
 *                 o_t = phi(q_t)^T S_t / phi(q_t)^T z_t  -- update first, then read, so token
 *                 t sees itself ("Linear Attention Math", section "The recurrent form: a
 *                 running KV state"; page one, section "Summarize state updates and reads
 *                 with equations").
 *   global form   S = sum_t phi(k_t) v_t^T, z = sum_t phi(k_t), o_t = phi(q_t)^T S / phi(q_t)^T z
 *                 ("Linear Attention Math", section "The associativity trick, written out").
 *   decode step   one step of the recurrence applied to a caller-held state: update, then read
 *                 ("Linear Attention Math", section "The recurrent form"; its last paragraph
 *                 states the O(1) per-token inference form).
 *   unnormalised  mode bit 1 returns the numerator phi(q_t)^T S_t itself (the weighted sum
 *                 before the division; "Linear Attention: Accumulating KV in a Fixed-Size
 *                 State", section "Read the state with a Query", prints such sums).
 *   decay         optional per-head gamma (NULL: none): S_t = gamma S_{t-1} + phi(k_t) v_t^T
 *                 and z_t = gamma z_{t-1} + phi(k_t) in the causal form and the decode step,
 *                 the retention recurrence ("Linear Attention Math", section "The kernel
 *                 cousins: SSMs and RetNet": linear attention with an explicit decay of the carried state;
 *                 with mode bit 1 and the identity map it is that recurrence as stated).
 *   random        oracle_rf_map: positive random features phi(x)_r = exp(w_r . x - |x|^2 / 2)
 *   features      / sqrt(m) for given projections w_r ("Linear Attention Math", section
 *                 "Feature maps: elu+1 and positive random features"); attention over them
 *                 is the identity-phi form applied to the mapped rows.
 * There is no epsilon in the denominator (the denominator is a sum of strictly positive terms
 * under ELU+1; "Linear Attention: From Pairwise Reads to a Recurrent State", section "The
 * reassociation that works", notes that a clamp changes the operation).
 *
 * Layout (row-major, contiguous): q, k [BH, N, d]; v, o [BH, N, dv]; S [BH, d, dv]
 * (rows = key features, columns = value components); z [BH, d]. BH = batch * heads.
 * Every head is independent; heads are split across OpenMP threads, each head is token-serial.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double phi(double x, int mode)
{
    if (mode & 1)
        return x;
    return x > 0.0 ? x + 1.0 : exp(x);
}

/* Causal recurrence over N tokens. S, z hold the initial state on entry (zeros for a fresh
 * sequence) and the state after the last token on return. num and den (may be NULL) receive
 * the numerator phi(q_t)^T S_t [BH, N, dv] and the denominator phi(q_t)^T z_t [BH, N]. */
void oracle_causal(const double *q, const double *k, const double *v, double *o, double *num,
                   double *den, double *S, double *z, long BH, long N, long d, long dv, int mode,
                   const double *gamma)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (long h = 0; h < BH; ++h) {
        double *kf = malloc(sizeof(double) * d);
        double *qf = malloc(sizeof(double) * d);
        double *nm = malloc(sizeof(double) * dv);
        double *Sh = S + h * d * dv;
        double *zh = z + h * d;
        for (long t = 0; t < N; ++t) {
            const double *kt = k + (h * N + t) * d;
            const double *qt = q + (h * N + t) * d;
            const double *vt = v + (h * N + t) * dv;
            /* decay: the state carried from the earlier tokens is scaled by gamma first */
            if (gamma) {
                for (long i = 0; i < d * dv; ++i)
                    Sh[i] *= gamma[h];
                for (long i = 0; i < d; ++i)
                    zh[i] *= gamma[h];
            }
            /* write: add the outer product phi(k_t) v_t^T and phi(k_t) to the key sum */
            for (long i = 0; i < d; ++i) {
                kf[i] = phi(kt[i], mode);
                for (long j = 0; j < dv; ++j)
                    Sh[i * dv + j] += kf[i] * vt[j];
                zh[i] += kf[i];
            }
            /* read: weight the state's rows by phi(q_t); divide by phi(q_t)^T z_t */
            for (long i = 0; i < d; ++i)
                qf[i] = phi(qt[i], mode);
            double dn = 0.0;
            for (long i = 0; i < d; ++i)
                dn += qf[i] * zh[i];
            /* nm[j] = sum_i qf[i] S[i][j], summed in increasing i (row-wise traversal) */
            for (long j = 0; j < dv; ++j)
                nm[j] = 0.0;
            for (long i = 0; i < d; ++i)
                for (long j = 0; j < dv; ++j)
                    nm[j] += qf[i] * Sh[i * dv + j];
            if (den)
                den[h * N + t] = dn;
            if (mode & 2) /* unnormalised form: the numerator is the output */
                dn = 1.0;
            for (long j = 0; j < dv; ++j) {
                o[(h * N + t) * dv + j] = nm[j] / dn;
                if (num)
                    num[(h * N + t) * dv + j] = nm[j];
            }
        }
        free(kf);
        free(qf);
        free(nm);
    }
}

/* Global (non-causal) form: first accumulate S and z over all N key/value tokens (S, z are
 * overwritten), then read each of the Nq queries q [BH, Nq, d] against that one state
 * (Nq = N for the full layer; a smaller Nq reads a chosen subset of query rows). q == NULL
 * computes the state only. */
void oracle_global(const double *q, const double *k, const double *v, double *o, double *num,
                   double *den, double *S, double *z, long BH, long N, long Nq, long d, long dv,
                   int mode)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (long h = 0; h < BH; ++h) {
        double *kf = malloc(sizeof(double) * d);
        double *qf = malloc(sizeof(double) * d);
        double *nm = malloc(sizeof(double) * dv);
        double *Sh = S + h * d * dv;
        double *zh = z + h * d;
        memset(Sh, 0, sizeof(double) * d * dv);
        memset(zh, 0, sizeof(double) * d);
        for (long t = 0; t < N; ++t) {
            const double *kt = k + (h * N + t) * d;
            const double *vt = v + (h * N + t) * dv;
            for (long i = 0; i < d; ++i) {
                kf[i] = phi(kt[i], mode);
                for (long j = 0; j < dv; ++j)
                    Sh[i * dv + j] += kf[i] * vt[j];
                zh[i] += kf[i];
            }
        }
        for (long t = 0; q && t < Nq; ++t) {
            const double *qt = q + (h * Nq + t) * d;
            for (long i = 0; i < d; ++i)
                qf[i] = phi(qt[i], mode);
            double dn = 0.0;
            for (long i = 0; i < d; ++i)
                dn += qf[i] * zh[i];
            for (long j = 0; j < dv; ++j)
                nm[j] = 0.0;
            for (long i = 0; i < d; ++i)
                for (long j = 0; j < dv; ++j)
                    nm[j] += qf[i] * Sh[i * dv + j];
            if (den)
                den[h * Nq + t] = dn;
            if (mode & 2)
                dn = 1.0;
            for (long j = 0; j < dv; ++j) {
                o[(h * Nq + t) * dv + j] = nm[j] / dn;
                if (num)
                    num[(h * Nq + t) * dv + j] = nm[j];
            }
        }
        free(kf);
        free(qf);
        free(nm);
    }
}

/* One decode step for every head: q, k [BH, d]; v, o [BH, dv]; S, z updated in place
 * (S <- S + phi(k) v^T, z <- z + phi(k)), then o = phi(q)^T S / phi(q)^T z. */
void oracle_decode(const double *q, const double *k, const double *v, double *o, double *S,
                   double *z, long BH, long d, long dv, int mode, const double *gamma)
{
#pragma omp parallel for schedule(static)
    for (long h = 0; h < BH; ++h) {
        double *Sh = S + h * d * dv;
        double *zh = z + h * d;
        const double *kh = k + h * d;
        const double *qh = q + h * d;
        const double *vh = v + h * dv;
        if (gamma) {
            for (long i = 0; i < d * dv; ++i)
                Sh[i] *= gamma[h];
            for (long i = 0; i < d; ++i)
                zh[i] *= gamma[h];
        }
        for (long i = 0; i < d; ++i) {
            double kfi = phi(kh[i], mode);
            for (long j = 0; j < dv; ++j)
                Sh[i * dv + j] += kfi * vh[j];
            zh[i] += kfi;
        }
        double dn = 0.0;
        for (long i = 0; i < d; ++i)
            dn += phi(qh[i], mode) * zh[i];
        for (long j = 0; j < dv; ++j)
            o[h * dv + j] = 0.0;
        for (long i = 0; i < d; ++i) {
            const double qfi = phi(qh[i], mode);
            for (long j = 0; j < dv; ++j)
                o[h * dv + j] += qfi * Sh[i * dv + j];
        }
        if (mode & 2)
            dn = 1.0;
        for (long j = 0; j < dv; ++j)
            o[h * dv + j] /= dn;
    }
}

/* Positive random features of `rows` vectors x [rows, d] for the projections W [m, d]:
 * f[i][r] = exp(sum_j W[r][j] x[i][j] - (1/2) sum_j x[i][j]^2) / sqrt(m), so that
 * f(q) . f(k) is an unbiased estimate of exp(q . k) when the rows of W are standard normal
 * ("Linear Attention Math", section "Feature maps: elu+1 and positive random features"). */
void oracle_rf_map(const double *x, const double *W, double *f, long rows, long d, long m)
{
    const double scale = 1.0 / sqrt((double)m);
#pragma omp parallel for schedule(static)
    for (long i = 0; i < rows; ++i) {
        const double *xi = x + i * d;
        double sq = 0.0;
        for (long j = 0; j < d; ++j)
            sq += xi[j] * xi[j];
        for (long r = 0; r < m; ++r) {
            double dot = 0.0;
            for (long j = 0; j < d; ++j)
                dot += W[r * d + j] * xi[j];
            f[i * m + r] = exp(dot - 0.5 * sq) * scale;
        }
    }
}

/* Number of OpenMP threads the functions above use (1 when built without OpenMP). */
int oracle_threads(void)
{
    int n = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
#endif
    return n;
}
