/*
 * fa_oracle.c - plain CPU reference for the flash-attention training forward.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline of the bench may call this code. It shares no code, header,
 * constant or helper with the GPU path.
 *
 * What it computes follows the CPU oracle on the method's page
 * ("mlx-native 0.9.0", tests/test_flash_attn_train.rs, section "CPU oracle -
 * forward O + logsumexp L", function sdpa_reference_with_logsumexp), restated
 * here in single precision:
 *
 *   for every batch b, query head h, query row i (kv head = h / (H / Hkv)):
 *     s_j = (sum_d q[i,d] * k[j,d]) * (scale * log2 e)       dot left to right
 *     s_j += log2 e * mask[i,j]                               if a mask is given
 *     s_j = -inf   for j > max(kl - ql, 0) + i                if causal
 *     s_j = -inf   for j < max(kl - ql, 0) + i - window       sliding window
 *     m   = max(-FLT_MAX / 2, max_j s_j)                      finite sentinel
 *     p_j = exp2(s_j - m),  S = sum_j p_j                     left to right
 *     L_i = m * ln 2 + ln S                                   (S = 0 -> -inf)
 *     O_i = sum_j (p_j / S') v_j,  S' = (S == 0 ? 1 : S)       left to right
 *
 * The mask is additive in natural-log units (hence the log2 e factor in the
 * base-2 score space). The causal alignment is bottom-right with the offset
 * clamped at zero, as on the page (kl.saturating_sub(ql) + q_pos). O is
 * returned in f32; fa_oracle_round_bf16 rounds it to bf16 the way the page's
 * oracle_for_bf16 helper does before comparing against a bf16 output.
 *
 * Sliding window (the same page, section 7, "SLIDING-WINDOW MASK (SWA)
 * PARITY"): the page builds it as an additive mask that keeps key j for row i
 * iff j <= i and j + window >= i. fa_oracle_fwd_swa applies that predicate
 * directly, with the causal rule's bottom-right alignment (i replaced by
 * q_abs = max(kl - ql, 0) + i, the same position the causal rule uses; the
 * two agree when ql = kl, the page's case): window + 1 keys at most.
 *
 * Arithmetic is IEEE f32 with no contraction (built with -ffp-contract=off),
 * exp2f/logf from the C library.
 *
 * The backward (fa_oracle_bwd) follows the same page's CPU oracle for the
 * FA-2 backward pass (section "Phase 2 - backward kernel helpers", function
 * sdpa_backward_reference_f32), in natural-log units as written there:
 *
 *   S_ij  = scale * (q_i . k_j)  (+ mask_ij; a -inf mask entry gives -inf),
 *           -inf for a causally hidden key (same alignment as the forward)
 *   P_ij  = exp(S_ij - L_i)      (0 where S_ij = -inf)
 *   dP_ij = dO_i . v_j
 *   D_i   = sum_j P_ij * dP_ij
 *   dS_ij = P_ij * (dP_ij - D_i)
 *   dV_j += P_ij * dO_i,  dQ_i += scale * dS_ij * k_j,  dK_j += scale * dS_ij * q_i
 *
 * dK and dV of a kv head accumulate over every query head of its group; the
 * sums run in the page's loop order (query head, query row, key).
 */
#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static const float ORACLE_LOG2E = 1.44269504088896340736f;
static const float ORACLE_LN2 = 0.693147180559945309417f;

typedef struct {
    const float *q, *k, *v, *mask;
    int64_t H, Hkv, ql, kl, D;
    float scale;
    int causal;
    int64_t window; /* < 0: no sliding window */
} oracle_problem;

/* One query row, flat index row = (b*H + h)*ql + i. o_row gets D floats. */
static void oracle_row(const oracle_problem *p, int64_t row, float *o_row, float *l_out,
                       float *s)
{
    const int64_t D = p->D, kl = p->kl, ql = p->ql;
    const int64_t i = row % ql;
    const int64_t bh = row / ql;
    const int64_t h = bh % p->H;
    const int64_t b = bh / p->H;
    const int64_t kvh = h / (p->H / p->Hkv);
    const float q_scale = p->scale * ORACLE_LOG2E;
    const float *qr = p->q + row * D;
    const float *kh = p->k + (b * p->Hkv + kvh) * kl * D;
    const float *vh = p->v + (b * p->Hkv + kvh) * kl * D;

    /* scaled dot products in base-2 units */
    for (int64_t j = 0; j < kl; ++j) {
        float dot = 0.0f;
        for (int64_t d = 0; d < D; ++d)
            dot += qr[d] * kh[j * D + d];
        s[j] = dot * q_scale;
    }
    /* additive mask, natural-log units converted to base 2 */
    if (p->mask) {
        const float *mr = p->mask + row * kl;
        for (int64_t j = 0; j < kl; ++j)
            s[j] += ORACLE_LOG2E * mr[j];
    }
    /* causal: key j is visible to row i iff j <= q_abs = max(kl - ql, 0) + i */
    const int64_t q_abs = (kl > ql ? kl - ql : 0) + i;
    if (p->causal) {
        for (int64_t j = q_abs + 1; j < kl; ++j)
            s[j] = -INFINITY;
    }
    /* sliding window: keys more than `window` positions before q_abs are hidden */
    if (p->window >= 0) {
        for (int64_t j = 0; j < q_abs - p->window && j < kl; ++j)
            s[j] = -INFINITY;
    }
    /* row max with the finite sentinel -FLT_MAX/2 */
    float m = -FLT_MAX / 2.0f;
    for (int64_t j = 0; j < kl; ++j)
        if (s[j] > m)
            m = s[j];
    /* exponentials (base 2) and their sum */
    float sum = 0.0f;
    for (int64_t j = 0; j < kl; ++j) {
        s[j] = exp2f(s[j] - m);
        sum += s[j];
    }
    *l_out = m * ORACLE_LN2 + logf(sum);
    /* normalised weighted sum of V rows; per output element the terms are
       added in key order, exactly as a d-outer / j-inner loop would */
    const float safe = (sum == 0.0f) ? 1.0f : sum;
    for (int64_t d = 0; d < D; ++d)
        o_row[d] = 0.0f;
    for (int64_t j = 0; j < kl; ++j) {
        const float w = s[j] / safe;
        const float *vr = vh + j * D;
        for (int64_t d = 0; d < D; ++d)
            o_row[d] += w * vr[d];
    }
}

typedef struct {
    const oracle_problem *p;
    const int64_t *rows; /* NULL: rows are 0..n-1 */
    int64_t begin, end;
    float *O, *L;
    int failed;
} oracle_job;

static void *oracle_worker(void *arg)
{
    oracle_job *j = (oracle_job *)arg;
    float *s = (float *)malloc(sizeof(float) * (size_t)(j->p->kl > 0 ? j->p->kl : 1));
    if (!s) {
        j->failed = 1;
        return NULL;
    }
    for (int64_t t = j->begin; t < j->end; ++t) {
        int64_t row = j->rows ? j->rows[t] : t;
        oracle_row(j->p, row, j->O + t * j->p->D, j->L + t, s);
    }
    free(s);
    return NULL;
}

static int oracle_validate(const float *q, const float *k, const float *v, int64_t B,
                           int64_t H, int64_t Hkv, int64_t ql, int64_t kl, int64_t D)
{
    if (B < 0 || ql < 0 || kl < 0 || H < 1 || Hkv < 1 || D < 1)
        return 2;
    if (H % Hkv != 0)
        return 3;
    if (B * H * ql > 0 && !q)
        return 1;
    if (B * Hkv * kl > 0 && (!k || !v))
        return 1;
    return 0;
}

static int oracle_run(const oracle_problem *p, const int64_t *rows, int64_t n_rows, float *O,
                      float *L, int n_threads)
{
    if (n_rows <= 0)
        return 0;
    if (!O || !L)
        return 1;
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > 256)
        n_threads = 256;
    if (n_threads > n_rows)
        n_threads = (int)n_rows;
    oracle_job jobs[256];
    pthread_t tid[256];
    for (int t = 0; t < n_threads; ++t) {
        jobs[t].p = p;
        jobs[t].rows = rows;
        jobs[t].begin = n_rows * t / n_threads;
        jobs[t].end = n_rows * (t + 1) / n_threads;
        jobs[t].O = O;
        jobs[t].L = L;
        jobs[t].failed = 0;
    }
    int started = 0;
    for (int t = 1; t < n_threads; ++t) {
        if (pthread_create(&tid[t], NULL, oracle_worker, &jobs[t]) != 0)
            break;
        started = t;
    }
    /* rows of threads that could not be started are done on this thread */
    for (int t = started + 1; t < n_threads; ++t)
        oracle_worker(&jobs[t]);
    oracle_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t)
        pthread_join(tid[t], NULL);
    for (int t = 0; t < n_threads; ++t)
        if (jobs[t].failed)
            return 4;
    return 0;
}

/*
 * Full forward. Inputs are f32 host arrays (bf16 values widened exactly):
 * q [B,H,ql,D], k/v [B,Hkv,kl,D], mask [B,H,ql,kl] or NULL.
 * Outputs: O [B,H,ql,D] f32, L [B,H,ql] f32.
 * Returns 0 on success, 1 null pointer, 2 bad size, 3 H % Hkv != 0,
 * 4 out of host memory.
 */
int fa_oracle_fwd(const float *q, const float *k, const float *v, const float *mask, int64_t B,
                  int64_t H, int64_t Hkv, int64_t ql, int64_t kl, int64_t D, float scale,
                  int causal, float *O, float *L, int n_threads)
{
    int rc = oracle_validate(q, k, v, B, H, Hkv, ql, kl, D);
    if (rc)
        return rc;
    oracle_problem p = {q, k, v, mask, H, Hkv, ql, kl, D, scale, causal, -1};
    return oracle_run(&p, NULL, B * H * ql, O, L, n_threads);
}

/*
 * Selected rows only: rows[t] is a flat row index (b*H + h)*ql + i; O gets
 * [n_rows, D] and L [n_rows]. Same inputs and return codes as fa_oracle_fwd,
 * plus 2 when a row index is out of range.
 */
int fa_oracle_fwd_rows(const float *q, const float *k, const float *v, const float *mask,
                       int64_t B, int64_t H, int64_t Hkv, int64_t ql, int64_t kl, int64_t D,
                       float scale, int causal, const int64_t *rows, int64_t n_rows, float *O,
                       float *L, int n_threads)
{
    int rc = oracle_validate(q, k, v, B, H, Hkv, ql, kl, D);
    if (rc)
        return rc;
    if (n_rows > 0 && !rows)
        return 1;
    for (int64_t t = 0; t < n_rows; ++t)
        if (rows[t] < 0 || rows[t] >= B * H * ql)
            return 2;
    oracle_problem p = {q, k, v, mask, H, Hkv, ql, kl, D, scale, causal, -1};
    return oracle_run(&p, rows, n_rows, O, L, n_threads);
}

/*
 * Sliding-window causal forward: key j is visible to row i iff
 * q_abs - window <= j <= q_abs, q_abs = max(kl - ql, 0) + i, window >= 0
 * (plus the additive mask when one is given). rows == NULL computes every
 * row (O [B,H,ql,D], L [B,H,ql]); otherwise the n_rows flat rows listed
 * (O [n_rows,D], L [n_rows]). Return codes as fa_oracle_fwd_rows, plus 2 for
 * a negative window.
 */
int fa_oracle_fwd_swa(const float *q, const float *k, const float *v, const float *mask,
                      int64_t B, int64_t H, int64_t Hkv, int64_t ql, int64_t kl, int64_t D,
                      float scale, int64_t window, const int64_t *rows, int64_t n_rows,
                      float *O, float *L, int n_threads)
{
    int rc = oracle_validate(q, k, v, B, H, Hkv, ql, kl, D);
    if (rc)
        return rc;
    if (window < 0)
        return 2;
    oracle_problem p = {q, k, v, mask, H, Hkv, ql, kl, D, scale, 1, window};
    if (!rows)
        return oracle_run(&p, NULL, B * H * ql, O, L, n_threads);
    for (int64_t t = 0; t < n_rows; ++t)
        if (rows[t] < 0 || rows[t] >= B * H * ql)
            return 2;
    return oracle_run(&p, rows, n_rows, O, L, n_threads);
}

/* f32 -> bf16 bits, round to nearest, ties to even (NaN stays a quiet NaN). */
void fa_oracle_round_bf16(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t t = 0; t < n; ++t) {
        uint32_t u;
        memcpy(&u, &x[t], 4);
        if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) {
            out[t] = (uint16_t)((u >> 16) | 0x0040u);
            continue;
        }
        uint32_t lsb = (u >> 16) & 1u;
        out[t] = (uint16_t)((u + 0x7FFFu + lsb) >> 16);
    }
}

/* ---- backward ---- */

typedef struct {
    const float *q, *k, *v, *mask, *L, *dO;
    float *dQ, *dK, *dV;
    int64_t H, Hkv, ql, kl, D;
    float scale;
    int causal;
    int64_t window; /* < 0: no sliding window */
} oracle_bwd_problem;

/* Every query head of kv head (b, kvh), rows in order; dK/dV of that kv head
   and dQ of its query heads are written only here. */
static void oracle_bwd_group(const oracle_bwd_problem *p, int64_t b, int64_t kvh, float *s,
                             float *pr)
{
    const int64_t D = p->D, kl = p->kl, ql = p->ql, G = p->H / p->Hkv;
    const float *kh = p->k + (b * p->Hkv + kvh) * kl * D;
    const float *vh = p->v + (b * p->Hkv + kvh) * kl * D;
    float *dkh = p->dK + (b * p->Hkv + kvh) * kl * D;
    float *dvh = p->dV + (b * p->Hkv + kvh) * kl * D;
    for (int64_t t = 0; t < kl * D; ++t) {
        dkh[t] = 0.0f;
        dvh[t] = 0.0f;
    }
    for (int64_t h = kvh * G; h < (kvh + 1) * G; ++h) {
        for (int64_t i = 0; i < ql; ++i) {
            const int64_t row = (b * p->H + h) * ql + i;
            const float *qr = p->q + row * D;
            const float *dor = p->dO + row * D;
            float *dqr = p->dQ + row * D;
            const float l_i = p->L[row];
            for (int64_t d = 0; d < D; ++d)
                dqr[d] = 0.0f;
            /* scores in natural-log units, masks */
            for (int64_t j = 0; j < kl; ++j) {
                float dot = 0.0f;
                for (int64_t d = 0; d < D; ++d)
                    dot += qr[d] * kh[j * D + d];
                s[j] = p->scale * dot;
                if (p->mask) {
                    const float m = p->mask[row * kl + j];
                    if (m == -INFINITY)
                        s[j] = -INFINITY;
                    else
                        s[j] += m;
                }
            }
            const int64_t q_abs = (kl > ql ? kl - ql : 0) + i;
            if (p->causal) {
                for (int64_t j = q_abs + 1; j < kl; ++j)
                    s[j] = -INFINITY;
            }
            /* sliding window, as in the forward */
            if (p->window >= 0) {
                for (int64_t j = 0; j < q_abs - p->window && j < kl; ++j)
                    s[j] = -INFINITY;
            }
            /* P from the forward's L */
            for (int64_t j = 0; j < kl; ++j)
                pr[j] = (s[j] == -INFINITY) ? 0.0f : expf(s[j] - l_i);
            /* D_i = sum_j P_ij dP_ij; s[] now holds dP */
            float d_i = 0.0f;
            for (int64_t j = 0; j < kl; ++j) {
                float dp = 0.0f;
                for (int64_t d = 0; d < D; ++d)
                    dp += dor[d] * vh[j * D + d];
                s[j] = dp;
                d_i += pr[j] * dp;
            }
            for (int64_t j = 0; j < kl; ++j) {
                const float ds = pr[j] * (s[j] - d_i);
                for (int64_t d = 0; d < D; ++d)
                    dvh[j * D + d] += pr[j] * dor[d];
                for (int64_t d = 0; d < D; ++d) {
                    dqr[d] += p->scale * ds * kh[j * D + d];
                    dkh[j * D + d] += p->scale * ds * qr[d];
                }
            }
        }
    }
}

typedef struct {
    const oracle_bwd_problem *p;
    int64_t begin, end; /* kv-head groups (b * Hkv + kvh) */
    int failed;
} oracle_bwd_job;

static void *oracle_bwd_worker(void *arg)
{
    oracle_bwd_job *j = (oracle_bwd_job *)arg;
    const size_t n = (size_t)(j->p->kl > 0 ? j->p->kl : 1);
    float *s = (float *)malloc(sizeof(float) * n);
    float *pr = (float *)malloc(sizeof(float) * n);
    if (!s || !pr) {
        free(s);
        free(pr);
        j->failed = 1;
        return NULL;
    }
    for (int64_t g = j->begin; g < j->end; ++g)
        oracle_bwd_group(j->p, g / j->p->Hkv, g % j->p->Hkv, s, pr);
    free(s);
    free(pr);
    return NULL;
}

/*
 * Backward. Inputs are f32 host arrays: q, dO [B,H,ql,D]; k, v [B,Hkv,kl,D];
 * mask [B,H,ql,kl] or NULL; L [B,H,ql] (natural-log logsumexp of the forward).
 * Outputs dQ [B,H,ql,D], dK and dV [B,Hkv,kl,D], f32. Same return codes as
 * fa_oracle_fwd.
 */
static int oracle_bwd_run(const oracle_bwd_problem *pp, int64_t B, int n_threads);
int fa_oracle_bwd_swa(const float *q, const float *k, const float *v, const float *mask,
                      const float *L, const float *dO, int64_t B, int64_t H, int64_t Hkv,
                      int64_t ql, int64_t kl, int64_t D, float scale, int causal, int64_t window,
                      float *dQ, float *dK, float *dV, int n_threads);

int fa_oracle_bwd(const float *q, const float *k, const float *v, const float *mask,
                  const float *L, const float *dO, int64_t B, int64_t H, int64_t Hkv, int64_t ql,
                  int64_t kl, int64_t D, float scale, int causal, float *dQ, float *dK, float *dV,
                  int n_threads)
{
    return fa_oracle_bwd_swa(q, k, v, mask, L, dO, B, H, Hkv, ql, kl, D, scale, causal, -1, dQ,
                             dK, dV, n_threads);
}

/*
 * Backward with an optional sliding window (window >= 0; it comes with the
 * causal rule, as in fa_oracle_fwd_swa, so causal must then be 1).
 */
int fa_oracle_bwd_swa(const float *q, const float *k, const float *v, const float *mask,
                      const float *L, const float *dO, int64_t B, int64_t H, int64_t Hkv,
                      int64_t ql, int64_t kl, int64_t D, float scale, int causal, int64_t window,
                      float *dQ, float *dK, float *dV, int n_threads)
{
    if (window >= 0 && !causal)
        return 2;
    int rc = oracle_validate(q, k, v, B, H, Hkv, ql, kl, D);
    if (rc)
        return rc;
    if (B * H * ql > 0 && (!L || !dO || !dQ))
        return 1;
    if (B * Hkv * kl > 0 && (!dK || !dV))
        return 1;
    oracle_bwd_problem p = {q, k, v, mask, L, dO, dQ, dK, dV, H, Hkv, ql, kl, D, scale, causal,
                            window < 0 ? -1 : window};
    return oracle_bwd_run(&p, B, n_threads);
}

static int oracle_bwd_run(const oracle_bwd_problem *pp, int64_t B, int n_threads)
{
    const oracle_bwd_problem p = *pp;
    const int64_t Hkv = p.Hkv;
    const int64_t groups = B * Hkv;
    if (groups <= 0)
        return 0;
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > 256)
        n_threads = 256;
    if (n_threads > groups)
        n_threads = (int)groups;
    oracle_bwd_job jobs[256];
    pthread_t tid[256];
    for (int t = 0; t < n_threads; ++t) {
        jobs[t].p = &p;
        jobs[t].begin = groups * t / n_threads;
        jobs[t].end = groups * (t + 1) / n_threads;
        jobs[t].failed = 0;
    }
    int started = 0;
    for (int t = 1; t < n_threads; ++t) {
        if (pthread_create(&tid[t], NULL, oracle_bwd_worker, &jobs[t]) != 0)
            break;
        started = t;
    }
    for (int t = started + 1; t < n_threads; ++t)
        oracle_bwd_worker(&jobs[t]);
    oracle_bwd_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t)
        pthread_join(tid[t], NULL);
    for (int t = 0; t < n_threads; ++t)
        if (jobs[t].failed)
            return 4;
    /* a query head with ql > 0 but kv heads with kl == 0: dQ is zero */
    return 0;
}
