/*
 * oracle.c -- plain fp64 CPU reference for causal retention and causal
 * linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker for the HIP path, not
 * part of it.  Only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark may load it.  It shares no code, header, table or helper
 * with the GPU library.
 *
 * Every function is written from the definitions on the source pages, in the
 * order those pages state them, with no blocking, fusion or reordering beyond
 * what the definition itself says.  All arithmetic is IEEE double.
 *
 * Layouts (row-major, last index fastest):
 *   q, k : [B][H][T][dk]      v, out : [B][H][T][dv]
 *   state: [B][H][dk][dv]     (rows index key features, columns value dims)
 *   gamma: [H]
 *
 * Sources cited below (page title, then the passage):
 *   [RetNet]  "RetNet" (bembew.net)
 *   [ESF]     "Efficient and Sparse Transformers" (temporalbook section 12.5)
 *   [LA]      "Linear attention" (zerotofrontier section 21.2)
 *   [LRR]     "Linear Attention, RWKV, and RetNet" (temporalbook section 13.3)
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_NOMEM (-2)

static int oracle_threads(int nthreads)
{
    return nthreads > 0 ? nthreads : 1;
}

/*
 * Retention, recurrent form.
 *   [RetNet] "Recurrent Representation":  S_n = gamma * S_{n-1} + K_n^T V_n,
 *            O_n = Q_n S_n, with S a d_k x d_v matrix started at zero.
 *   [ESF] section 6, "Recurrent form", and the minimal RetNet recurrent step:
 *            the state is decayed and the outer product k v^T added first,
 *            then the output is read from the updated state.
 *   [LA] "Where linear attention implementations go wrong": reading before
 *            writing would drop the token from its own output.
 * init_state may be NULL (zero initial state).  final_state may be NULL.
 */
int oracle_retention_recurrent(const double *q, const double *k, const double *v,
                               const double *gamma, long B, long H, long T,
                               long dk, long dv, const double *init_state,
                               double *out, double *final_state, int nthreads)
{
    if (!q || !k || !v || !gamma || !out || B < 0 || H <= 0 || T < 0 ||
        dk <= 0 || dv <= 0)
        return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
#pragma omp parallel for num_threads(oracle_threads(nthreads)) schedule(dynamic, 1)
    for (long bh = 0; bh < B * H; ++bh) {
        const long h = bh % H;
        const double g = gamma[h];
        double *S = (double *)malloc((size_t)(dk * dv) * sizeof(double));
        if (!S) {
            err = ORACLE_ERR_NOMEM;
            continue;
        }
        if (init_state)
            memcpy(S, init_state + bh * dk * dv, (size_t)(dk * dv) * sizeof(double));
        else
            memset(S, 0, (size_t)(dk * dv) * sizeof(double));
        for (long t = 0; t < T; ++t) {
            const double *qt = q + (bh * T + t) * dk;
            const double *kt = k + (bh * T + t) * dk;
            const double *vt = v + (bh * T + t) * dv;
            double *ot = out + (bh * T + t) * dv;
            /* S <- gamma * S + k_t v_t^T */
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j)
                    S[i * dv + j] = g * S[i * dv + j] + kt[i] * vt[j];
            /* o_t = q_t S  (row vector times matrix) */
            for (long j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (long i = 0; i < dk; ++i)
                    acc += qt[i] * S[i * dv + j];
                ot[j] = acc;
            }
        }
        if (final_state)
            memcpy(final_state + bh * dk * dv, S, (size_t)(dk * dv) * sizeof(double));
        free(S);
    }
    return err;
}

/*
 * Retention, parallel form, by brute force over the full T x T matrix.
 *   [RetNet] "Parallel Representation" and the single-head definition:
 *            O = (Q K^T (.) D) V,  D_nm = gamma^(n-m) for n >= m, else 0.
 *   [ESF] section 6, "Parallel form": D is lower-triangular with entries
 *            gamma^(i-j).
 * The decay power is formed only for n >= m (a non-negative exponent).
 * Cost O(T^2 (dk + dv)) per head: tiny inputs only.
 */
int oracle_retention_parallel(const double *q, const double *k, const double *v,
                              const double *gamma, long B, long H, long T,
                              long dk, long dv, double *out)
{
    if (!q || !k || !v || !gamma || !out || B < 0 || H <= 0 || T < 0 ||
        dk <= 0 || dv <= 0)
        return ORACLE_ERR_ARG;
    for (long bh = 0; bh < B * H; ++bh) {
        const double g = gamma[bh % H];
        for (long n = 0; n < T; ++n) {
            double *on = out + (bh * T + n) * dv;
            for (long j = 0; j < dv; ++j)
                on[j] = 0.0;
            for (long m = 0; m <= n; ++m) {
                double score = 0.0; /* (Q K^T)_{nm} */
                for (long i = 0; i < dk; ++i)
                    score += q[(bh * T + n) * dk + i] * k[(bh * T + m) * dk + i];
                const double d_nm = pow(g, (double)(n - m));
                for (long j = 0; j < dv; ++j)
                    on[j] += score * d_nm * v[(bh * T + m) * dv + j];
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Selected rows of the retention output, each computed straight from the
 * parallel-form definition (see oracle_retention_parallel):
 *   o_t = sum_{s <= t} gamma^(t-s) (q_t . k_s) v_s.
 * rows holds n triples (b, h, t); row r of the result is rows_out[r][0..dv).
 * Cost O(t (dk + dv)) per row, so single rows can be checked at any T.
 */
int oracle_retention_rows(const double *q, const double *k, const double *v,
                          const double *gamma, long B, long H, long T, long dk,
                          long dv, const long *rows, long n, double *rows_out,
                          int nthreads)
{
    if (!q || !k || !v || !gamma || !rows || !rows_out || H <= 0 || dk <= 0 ||
        dv <= 0)
        return ORACLE_ERR_ARG;
    for (long r = 0; r < n; ++r) {
        const long b = rows[3 * r], h = rows[3 * r + 1], t = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || t < 0 || t >= T)
            return ORACLE_ERR_ARG;
    }
#pragma omp parallel for num_threads(oracle_threads(nthreads)) schedule(dynamic, 1)
    for (long r = 0; r < n; ++r) {
        const long b = rows[3 * r], h = rows[3 * r + 1], t = rows[3 * r + 2];
        const long bh = b * H + h;
        const double g = gamma[h];
        const double *qt = q + (bh * T + t) * dk;
        double *o = rows_out + r * dv;
        for (long j = 0; j < dv; ++j)
            o[j] = 0.0;
        for (long s = 0; s <= t; ++s) {
            double score = 0.0;
            for (long i = 0; i < dk; ++i)
                score += qt[i] * k[(bh * T + s) * dk + i];
            const double w = score * pow(g, (double)(t - s));
            for (long j = 0; j < dv; ++j)
                o[j] += w * v[(bh * T + s) * dv + j];
        }
    }
    return ORACLE_OK;
}

/*
 * Retention, chunkwise form, in fp64.
 *   [ESF] section 6, "Chunkwise form": split the sequence into chunks, use
 *         the parallel form inside a chunk and carry the state across chunks
 *         with the recurrent form.  [RetNet] "Chunked Recurrent
 *         Representation" and [LRR] section 3 describe the same split.
 * None of the pages prints the chunk equations; they follow from unrolling
 * the recurrence S_t = gamma S_{t-1} + k_t v_t^T inside one chunk.  With
 * S_prev the state before the chunk, local index i, j in [0, c), c the chunk
 * length (the last chunk may be shorter):
 *   o_i   = sum_{j <= i} gamma^(i-j) (q_i . k_j) v_j + gamma^(i+1) q_i S_prev
 *   S_new = gamma^c S_prev + sum_j gamma^(c-1-j) k_j v_j^T
 * This function checks that derivation against the recurrence on the CPU.
 */
int oracle_retention_chunkwise(const double *q, const double *k, const double *v,
                               const double *gamma, long B, long H, long T,
                               long dk, long dv, long chunk, double *out,
                               double *final_state)
{
    if (!q || !k || !v || !gamma || !out || B < 0 || H <= 0 || T < 0 ||
        dk <= 0 || dv <= 0 || chunk <= 0)
        return ORACLE_ERR_ARG;
    double *S = (double *)malloc((size_t)(dk * dv) * sizeof(double));
    double *Snew = (double *)malloc((size_t)(dk * dv) * sizeof(double));
    if (!S || !Snew) {
        free(S);
        free(Snew);
        return ORACLE_ERR_NOMEM;
    }
    for (long bh = 0; bh < B * H; ++bh) {
        const double g = gamma[bh % H];
        memset(S, 0, (size_t)(dk * dv) * sizeof(double));
        for (long t0 = 0; t0 < T; t0 += chunk) {
            const long c = (T - t0 < chunk) ? (T - t0) : chunk;
            /* outputs of this chunk, from S_prev = S */
            for (long i = 0; i < c; ++i) {
                const double *qi = q + (bh * T + t0 + i) * dk;
                double *oi = out + (bh * T + t0 + i) * dv;
                /* inter-chunk part: gamma^(i+1) q_i S_prev */
                const double xi = pow(g, (double)(i + 1));
                for (long jv = 0; jv < dv; ++jv) {
                    double acc = 0.0;
                    for (long a = 0; a < dk; ++a)
                        acc += qi[a] * S[a * dv + jv];
                    oi[jv] = xi * acc;
                }
                /* intra-chunk part: masked, decayed scores times values */
                for (long j = 0; j <= i; ++j) {
                    const double *kj = k + (bh * T + t0 + j) * dk;
                    const double *vj = v + (bh * T + t0 + j) * dv;
                    double score = 0.0;
                    for (long a = 0; a < dk; ++a)
                        score += qi[a] * kj[a];
                    const double w = score * pow(g, (double)(i - j));
                    for (long jv = 0; jv < dv; ++jv)
                        oi[jv] += w * vj[jv];
                }
            }
            /* state carried to the next chunk */
            const double gc = pow(g, (double)c);
            for (long a = 0; a < dk * dv; ++a)
                Snew[a] = gc * S[a];
            for (long j = 0; j < c; ++j) {
                const double zeta = pow(g, (double)(c - 1 - j));
                const double *kj = k + (bh * T + t0 + j) * dk;
                const double *vj = v + (bh * T + t0 + j) * dv;
                for (long a = 0; a < dk; ++a)
                    for (long jv = 0; jv < dv; ++jv)
                        Snew[a * dv + jv] += zeta * kj[a] * vj[jv];
            }
            memcpy(S, Snew, (size_t)(dk * dv) * sizeof(double));
        }
        if (final_state)
            memcpy(final_state + bh * dk * dv, S, (size_t)(dk * dv) * sizeof(double));
    }
    free(S);
    free(Snew);
    return ORACLE_OK;
}

/*
 * One recurrent decode step for N sequences x H heads, in place on state.
 *   [ESF] "A Minimal RetNet Recurrent Step in PyTorch": new_state =
 *         gamma * state + outer(k, v); y = q @ new_state.
 *   [RetNet] "Recurrent Representation" (same update and read-out).
 * q, k: [N][H][dk], v, out: [N][H][dv], state: [N][H][dk][dv].
 * The step is applied nsteps times with the same q, k, v (nsteps >= 1); out
 * holds the read-out of the last step.
 */
int oracle_decode_steps(const double *q, const double *k, const double *v,
                        const double *gamma, double *state, double *out, long N,
                        long H, long dk, long dv, long nsteps, int nthreads)
{
    if (!q || !k || !v || !gamma || !state || !out || N < 0 || H <= 0 ||
        dk <= 0 || dv <= 0 || nsteps < 1)
        return ORACLE_ERR_ARG;
#pragma omp parallel for num_threads(oracle_threads(nthreads)) schedule(dynamic, 1)
    for (long nh = 0; nh < N * H; ++nh) {
        const double g = gamma[nh % H];
        const double *qn = q + nh * dk, *kn = k + nh * dk, *vn = v + nh * dv;
        double *S = state + nh * dk * dv;
        double *o = out + nh * dv;
        for (long s = 0; s < nsteps; ++s) {
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j)
                    S[i * dv + j] = g * S[i * dv + j] + kn[i] * vn[j];
            for (long j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (long i = 0; i < dk; ++i)
                    acc += qn[i] * S[i * dv + j];
                o[j] = acc;
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Gradient of retention (zero initial state) with respect to q, k and v, given
 * dout = dL/dout for a scalar loss L.
 *   [LA] section "Decoding, training, and what each costs": the gradients of
 *        the causal recurrence are cumulative sums as well, running forward in
 *        time for the queries and backward in time for the keys and values,
 *        so no per-token state is stored.
 * For the retention recurrence S_t = gamma S_{t-1} + k_t v_t^T, o_t = q_t S_t
 * ([RetNet] "Recurrent Representation") these sums are
 *   dq_t = S_t do_t                          (S_t: the forward state after token t)
 *   U_t  = gamma U_{t+1} + q_t do_t^T,  U_T = 0   (dk x dv, backward in time)
 *   dk_t = U_t v_t,   dv_t = U_t^T k_t
 * dq, dk: [B][H][T][dk], dv: [B][H][T][dv].
 */
int oracle_retention_bwd(const double *q, const double *k, const double *v,
                         const double *gamma, const double *dout, long B, long H,
                         long T, long dk, long dv, double *dq, double *dkk,
                         double *dvv, int nthreads)
{
    if (!q || !k || !v || !gamma || !dout || !dq || !dkk || !dvv || B < 0 || H <= 0 ||
        T < 0 || dk <= 0 || dv <= 0)
        return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
#pragma omp parallel for num_threads(oracle_threads(nthreads)) schedule(dynamic, 1)
    for (long bh = 0; bh < B * H; ++bh) {
        const double g = gamma[bh % H];
        double *Sf = (double *)calloc((size_t)(dk * dv), sizeof(double));
        double *U = (double *)calloc((size_t)(dk * dv), sizeof(double));
        if (!Sf || !U) {
            err = ORACLE_ERR_NOMEM;
            free(Sf); free(U);
            continue;
        }
        /* forward in time: the query gradients */
        for (long t = 0; t < T; ++t) {
            const double *kt = k + (bh * T + t) * dk, *vt = v + (bh * T + t) * dv;
            const double *dot = dout + (bh * T + t) * dv;
            double *dqt = dq + (bh * T + t) * dk;
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j)
                    Sf[i * dv + j] = g * Sf[i * dv + j] + kt[i] * vt[j];
            for (long i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (long j = 0; j < dv; ++j)
                    acc += Sf[i * dv + j] * dot[j];
                dqt[i] = acc;
            }
        }
        /* backward in time: the key and value gradients */
        for (long t = T - 1; t >= 0; --t) {
            const double *qt = q + (bh * T + t) * dk, *kt = k + (bh * T + t) * dk;
            const double *vt = v + (bh * T + t) * dv, *dot = dout + (bh * T + t) * dv;
            double *dkt = dkk + (bh * T + t) * dk, *dvt = dvv + (bh * T + t) * dv;
            for (long i = 0; i < dk; ++i)
                for (long j = 0; j < dv; ++j)
                    U[i * dv + j] = g * U[i * dv + j] + qt[i] * dot[j];
            for (long i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (long j = 0; j < dv; ++j)
                    acc += U[i * dv + j] * vt[j];
                dkt[i] = acc;
            }
            for (long j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (long i = 0; i < dk; ++i)
                    acc += U[i * dv + j] * kt[i];
                dvt[j] = acc;
            }
        }
        free(Sf); free(U);
    }
    return err;
}

/*
 * Retention with the row-sum floor and, optionally, GroupNorm.
 *   [LA] box "An LSTM whose cell is linear attention": the matrix cell and
 *        normaliser evolve as C_t = f C_{t-1} + i v_t k_t^T and
 *        n_t = f n_{t-1} + i k_t, and the read-out divides C_t q_t by
 *        max(|n_t^T q_t|, 1), a floor of 1 the page attributes to RetNet.
 *        With f = gamma and i = 1 (C_t = S_t^T) this is the retention read-out
 *        o_t = q_t S_t divided by its decayed row sum of scores
 *        n_t^T q_t = sum_{s<=t} gamma^(t-s) q_t . k_s, floored at 1 in size;
 *        the same page describes RetNet dividing each row of its scores by the
 *        absolute value of their sum, clamped below at 1, with a normalisation
 *        after it.
 *   [RetNet] "Multi-Scale Retention and Network Architecture": the layer's
 *        optional GroupNorm.  group != 0 replaces each output row (one head's
 *        dv features) by (o - mean(o)) / sqrt(var(o) + eps), with the
 *        population variance and no learned gain or bias.
 */
int oracle_retention_normalized(const double *q, const double *k, const double *v,
                                const double *gamma, long B, long H, long T, long dk,
                                long dv, int group, double eps, double *out, int nthreads)
{
    if (!q || !k || !v || !gamma || !out || B < 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0)
        return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
#pragma omp parallel for num_threads(oracle_threads(nthreads)) schedule(dynamic, 1)
    for (long bh = 0; bh < B * H; ++bh) {
        const double g = gamma[bh % H];
        double *Sn = (double *)calloc((size_t)(dk * dv), sizeof(double));
        double *n = (double *)calloc((size_t)dk, sizeof(double));
        if (!Sn || !n) {
            err = ORACLE_ERR_NOMEM;
            free(Sn); free(n);
            continue;
        }
        for (long t = 0; t < T; ++t) {
            const double *qt = q + (bh * T + t) * dk, *kt = k + (bh * T + t) * dk;
            const double *vt = v + (bh * T + t) * dv;
            double *ot = out + (bh * T + t) * dv;
            for (long i = 0; i < dk; ++i) {
                for (long j = 0; j < dv; ++j)
                    Sn[i * dv + j] = g * Sn[i * dv + j] + kt[i] * vt[j];
                n[i] = g * n[i] + kt[i];
            }
            double r = 0.0;
            for (long i = 0; i < dk; ++i)
                r += n[i] * qt[i];
            const double den = fabs(r) > 1.0 ? fabs(r) : 1.0;
            for (long j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (long i = 0; i < dk; ++i)
                    acc += qt[i] * Sn[i * dv + j];
                ot[j] = acc / den;
            }
            if (group) {
                double mean = 0.0, var = 0.0;
                for (long j = 0; j < dv; ++j)
                    mean += ot[j];
                mean /= (double)dv;
                for (long j = 0; j < dv; ++j)
                    var += (ot[j] - mean) * (ot[j] - mean);
                var /= (double)dv;
                const double rstd = 1.0 / sqrt(var + eps);
                for (long j = 0; j < dv; ++j)
                    ot[j] = (ot[j] - mean) * rstd;
            }
        }
        free(Sn); free(n);
    }
    return err;
}

/*
 * Gated linear attention with a per-token, per-key-channel gate, recurrent form.
 *   [ESF] section "Gated Linear Attention: Toward Input-Dependent Forgetting":
 *        the fixed decay of RetNet becomes a data-dependent gate G_t applied
 *        element-wise to the state, S_t = G_t (.) S_{t-1} + k_t^T v_t, with
 *        RetNet the case G_t = gamma 1 and plain linear attention G_t = 1; the
 *        gate lets the model forget some channels and keep others.
 * Here G_t[i][j] = alpha_t[i] (one gate per key channel, shared by the value
 * columns), given as log-gates lg = log alpha in (-inf, 0]:
 *   S_t[i][j] = exp(lg_t[i]) S_{t-1}[i][j] + k_t[i] v_t[j],   o_t = q_t S_t.
 * lg: [B][H][T][dk].  final_state may be NULL.
 */
int oracle_gla_recurrent(const double *q, const double *k, const double *v,
                         const double *lg, long B, long H, long T, long dk, long dv,
                         double *out, double *final_state, int nthreads)
{
    if (!q || !k || !v || !lg || !out || B < 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0)
        return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
#pragma omp parallel for num_threads(oracle_threads(nthreads)) schedule(dynamic, 1)
    for (long bh = 0; bh < B * H; ++bh) {
        double *Sg = (double *)calloc((size_t)(dk * dv), sizeof(double));
        if (!Sg) {
            err = ORACLE_ERR_NOMEM;
            continue;
        }
        for (long t = 0; t < T; ++t) {
            const double *qt = q + (bh * T + t) * dk, *kt = k + (bh * T + t) * dk;
            const double *vt = v + (bh * T + t) * dv, *gt = lg + (bh * T + t) * dk;
            double *ot = out + (bh * T + t) * dv;
            for (long i = 0; i < dk; ++i) {
                const double a = exp(gt[i]);
                for (long j = 0; j < dv; ++j)
                    Sg[i * dv + j] = a * Sg[i * dv + j] + kt[i] * vt[j];
            }
            for (long j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (long i = 0; i < dk; ++i)
                    acc += qt[i] * Sg[i * dv + j];
                ot[j] = acc;
            }
        }
        if (final_state)
            memcpy(final_state + bh * dk * dv, Sg, (size_t)(dk * dv) * sizeof(double));
        free(Sg);
    }
    return err;
}

/*
 * Feature map phi(x) = elu(x) + 1, entrywise.
 *   [LA] "Linear attention by hand on three tokens": elu(x) = x for x > 0 and
 *        e^x - 1 otherwise, so phi(x) = x + 1 for x >= 0 and e^x for x < 0.
 *   [LRR] section 5 uses the same map (u > 0 -> u + 1, else e^u).
 * Both readings give phi(0) = 1.
 */
static double phi_elu1(double x)
{
    return x > 0.0 ? x + 1.0 : exp(x);
}

/*
 * Causal linear attention with the elu+1 feature map and its normaliser,
 * recurrent form.
 *   [LA] box "Causal linear attention, recurrent form":
 *        S_t = S_{t-1} + phi(k_t) v_t^T,  z_t = z_{t-1} + phi(k_t),
 *        o_t = S_t^T phi(q_t) / (z_t^T phi(q_t)),
 *        with a small eps added to the denominator (the interview task adds
 *        it "as written"; each token is included in its own sum).
 *   [ESF] Code 12.5.1 and [LRR] Code 13.3.2 run the same loop.
 * The loop starts from (S, z) = (init_S, init_z), the state and normaliser
 * after earlier tokens ([LA] "Interview: causal linear attention, recurrent
 * and parallel, plus the decode step" hands exactly that pair from one call
 * to the next); NULL means zero.  final_S [B][H][dk][dv] and final_z
 * [B][H][dk] may be NULL.
 */
int oracle_linattn_recurrent(const double *q, const double *k, const double *v,
                             double eps, long B, long H, long T, long dk, long dv,
                             const double *init_S, const double *init_z,
                             double *out, double *final_S, double *final_z,
                             int nthreads)
{
    if (!q || !k || !v || !out || B < 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0)
        return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
#pragma omp parallel for num_threads(oracle_threads(nthreads)) schedule(dynamic, 1)
    for (long bh = 0; bh < B * H; ++bh) {
        double *S = (double *)calloc((size_t)(dk * dv), sizeof(double));
        double *z = (double *)calloc((size_t)dk, sizeof(double));
        double *pq = (double *)malloc((size_t)dk * sizeof(double));
        double *pk = (double *)malloc((size_t)dk * sizeof(double));
        if (!S || !z || !pq || !pk) {
            err = ORACLE_ERR_NOMEM;
            free(S); free(z); free(pq); free(pk);
            continue;
        }
        if (init_S)
            memcpy(S, init_S + bh * dk * dv, (size_t)(dk * dv) * sizeof(double));
        if (init_z)
            memcpy(z, init_z + bh * dk, (size_t)dk * sizeof(double));
        for (long t = 0; t < T; ++t) {
            const double *qt = q + (bh * T + t) * dk;
            const double *kt = k + (bh * T + t) * dk;
            const double *vt = v + (bh * T + t) * dv;
            double *ot = out + (bh * T + t) * dv;
            for (long i = 0; i < dk; ++i) {
                pq[i] = phi_elu1(qt[i]);
                pk[i] = phi_elu1(kt[i]);
            }
            for (long i = 0; i < dk; ++i) {
                for (long j = 0; j < dv; ++j)
                    S[i * dv + j] += pk[i] * vt[j];
                z[i] += pk[i];
            }
            double den = 0.0;
            for (long i = 0; i < dk; ++i)
                den += z[i] * pq[i];
            den += eps;
            for (long j = 0; j < dv; ++j) {
                double num = 0.0;
                for (long i = 0; i < dk; ++i)
                    num += S[i * dv + j] * pq[i];
                ot[j] = num / den;
            }
        }
        if (final_S)
            memcpy(final_S + bh * dk * dv, S, (size_t)(dk * dv) * sizeof(double));
        if (final_z)
            memcpy(final_z + bh * dk, z, (size_t)dk * sizeof(double));
        free(S); free(z); free(pq); free(pk);
    }
    return err;
}

/*
 * One decode step of causal linear attention for N sequences x H heads, in
 * place on (S, z).
 *   [LA] "Interview: causal linear attention, recurrent and parallel, plus
 *        the decode step": the step takes the state S (d_phi x d_v) and the
 *        normaliser z (d_phi) after t-1 tokens and one token's q, k, v; it
 *        adds phi(k) v^T to S and phi(k) to z, then reads
 *        o = S^T phi(q) / (z^T phi(q) + eps) from the updated pair.
 * q, k: [N][H][dk], v, out: [N][H][dv], S: [N][H][dk][dv], z: [N][H][dk].
 * The step is applied nsteps times with the same token; out holds the last
 * read-out.  (The page's function returns new arrays; the Python wrapper
 * copies S and z first, so its inputs are left unchanged.)
 */
int oracle_linattn_decode_steps(const double *q, const double *k, const double *v,
                                double eps, double *S, double *z, double *out,
                                long N, long H, long dk, long dv, long nsteps,
                                int nthreads)
{
    if (!q || !k || !v || !S || !z || !out || N < 0 || H <= 0 || dk <= 0 ||
        dv <= 0 || nsteps < 1)
        return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
#pragma omp parallel for num_threads(oracle_threads(nthreads)) schedule(dynamic, 1)
    for (long nh = 0; nh < N * H; ++nh) {
        const double *qn = q + nh * dk, *kn = k + nh * dk, *vn = v + nh * dv;
        double *Sn = S + nh * dk * dv, *zn = z + nh * dk, *o = out + nh * dv;
        double *fq = (double *)malloc((size_t)dk * sizeof(double));
        double *fk = (double *)malloc((size_t)dk * sizeof(double));
        if (!fq || !fk) {
            err = ORACLE_ERR_NOMEM;
            free(fq); free(fk);
            continue;
        }
        for (long i = 0; i < dk; ++i) {
            fq[i] = phi_elu1(qn[i]);
            fk[i] = phi_elu1(kn[i]);
        }
        for (long s = 0; s < nsteps; ++s) {
            for (long i = 0; i < dk; ++i) {
                for (long j = 0; j < dv; ++j)
                    Sn[i * dv + j] += fk[i] * vn[j];
                zn[i] += fk[i];
            }
            double den = eps;
            for (long i = 0; i < dk; ++i)
                den += zn[i] * fq[i];
            for (long j = 0; j < dv; ++j) {
                double num = 0.0;
                for (long i = 0; i < dk; ++i)
                    num += Sn[i * dv + j] * fq[i];
                o[j] = num / den;
            }
        }
        free(fq); free(fk);
    }
    return err;
}

/*
 * Causal linear attention, masked parallel form, by brute force.
 *   [LA] theorem "Recurrent and parallel forms agree":
 *        W = (phi(Q) phi(K)^T) (.) L with L the lower-triangular ones,
 *        O = diag(W 1)^{-1} W V  (eps added to each row sum, as the
 *        recurrent form adds it to its denominator).
 * Cost O(T^2 (dk + dv)) per head: tiny inputs only.
 */
int oracle_linattn_parallel(const double *q, const double *k, const double *v,
                            double eps, long B, long H, long T, long dk, long dv,
                            double *out)
{
    if (!q || !k || !v || !out || B < 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0)
        return ORACLE_ERR_ARG;
    for (long bh = 0; bh < B * H; ++bh) {
        for (long t = 0; t < T; ++t) {
            double *ot = out + (bh * T + t) * dv;
            double rowsum = 0.0;
            for (long j = 0; j < dv; ++j)
                ot[j] = 0.0;
            for (long s = 0; s <= t; ++s) {
                double w = 0.0; /* W_ts = phi(q_t) . phi(k_s) */
                for (long i = 0; i < dk; ++i)
                    w += phi_elu1(q[(bh * T + t) * dk + i]) *
                         phi_elu1(k[(bh * T + s) * dk + i]);
                rowsum += w;
                for (long j = 0; j < dv; ++j)
                    ot[j] += w * v[(bh * T + s) * dv + j];
            }
            for (long j = 0; j < dv; ++j)
                ot[j] /= (rowsum + eps);
        }
    }
    return ORACLE_OK;
}

/*
 * Selected rows of the linear-attention output from the masked parallel
 * definition (see oracle_linattn_parallel), one row at a time:
 *   o_t = sum_{s<=t} (phi(q_t).phi(k_s)) v_s / (sum_{s<=t} phi(q_t).phi(k_s) + eps).
 * rows holds n triples (b, h, t).
 */
int oracle_linattn_rows(const double *q, const double *k, const double *v,
                        double eps, long B, long H, long T, long dk, long dv,
                        const long *rows, long n, double *rows_out, int nthreads)
{
    if (!q || !k || !v || !rows || !rows_out || H <= 0 || dk <= 0 || dv <= 0)
        return ORACLE_ERR_ARG;
    for (long r = 0; r < n; ++r) {
        const long b = rows[3 * r], h = rows[3 * r + 1], t = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || t < 0 || t >= T)
            return ORACLE_ERR_ARG;
    }
#pragma omp parallel for num_threads(oracle_threads(nthreads)) schedule(dynamic, 1)
    for (long r = 0; r < n; ++r) {
        const long b = rows[3 * r], h = rows[3 * r + 1], t = rows[3 * r + 2];
        const long bh = b * H + h;
        double *o = rows_out + r * dv;
        double rowsum = 0.0;
        for (long j = 0; j < dv; ++j)
            o[j] = 0.0;
        for (long s = 0; s <= t; ++s) {
            double w = 0.0;
            for (long i = 0; i < dk; ++i)
                w += phi_elu1(q[(bh * T + t) * dk + i]) *
                     phi_elu1(k[(bh * T + s) * dk + i]);
            rowsum += w;
            for (long j = 0; j < dv; ++j)
                o[j] += w * v[(bh * T + s) * dv + j];
        }
        for (long j = 0; j < dv; ++j)
            o[j] /= (rowsum + eps);
    }
    return ORACLE_OK;
}

/* Number of OpenMP threads the oracle would use for a request of nthreads. */
int oracle_threads_used(int nthreads)
{
#ifdef _OPENMP
    int used = 0;
#pragma omp parallel num_threads(oracle_threads(nthreads))
    {
#pragma omp single
        used = omp_get_num_threads();
    }
    return used;
#else
    (void)nthreads;
    return 1;
#endif
}
