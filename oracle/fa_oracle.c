/*
 * fa_oracle.c - plain CPU reference for the flash-attention training forward
 * and its backward.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline of the bench may call this code. It shares no code, header,
 * constant or helper with the GPU path.
 *
 * What is computed is softmax attention with its logsumexp, the operation the
 * method's page defines ("mlx-native 0.9.0", tests/test_flash_attn_train.rs,
 * doc comment and section "CPU oracle - forward O + logsumexp L"; the causal
 * alignment is that oracle's, the offset max(kl - ql, 0) clamped at zero).
 * It is written here from the definition, in natural-log units, in single
 * precision, one query row at a time:
 *
 *   query row i of batch b and query head h reads kv head g = h / (H / Hkv)
 *   and sits at key position pos_i = max(kl - ql, 0) + i;
 *   key j is allowed for it unless causal and j > pos_i, or a sliding window
 *   w >= 0 is given and j < pos_i - w;
 *   s_ij = scale * <q_i, k_j> + mask_ij     for an allowed key (-inf else);
 *   a key is visible when s_ij > -inf (a -inf mask entry hides it);
 *   no visible key:  O_i = +0,  L_i = -inf;
 *   otherwise, with m_i = max_j s_ij (any shift gives the same values; the
 *   maximum keeps every exponential at most 1):
 *     L_i = m_i + log(sum_j exp(s_ij - m_i))               (logsumexp)
 *     O_i = sum_j (exp(s_ij - m_i) / sum_k exp(s_ik - m_i)) * v_j   (softmax . V)
 *
 * Every sum runs in index order (dot products over d, the others over j).
 * The sliding window is the page's section 7 band (key j kept for row i iff
 * j <= i and j + w >= i), placed at the causal rule's position pos_i.
 * Keys and values may have different widths (D for q and k, Dv for v and O).
 * An optional sink logit per query head (fa_oracle_fwd_sinks) joins every
 * row's softmax as one more term with a zero value: it enters the maximum and
 * the sum, so L_i = log(exp(sink_h) + sum_j exp(s_ij)) and O_i's weights are
 * exp(s_ij - L_i). (The adjacent SDPA page passes sinks [Hq] without defining
 * them; this is the reading its name and shape fix: a per-head logit with no
 * value.) A row with no visible key then has O_i = +0, L_i = sink_h.
 *
 * The backward (fa_oracle_bwd*) is the FA-2 backward the same page defines
 * (section "Phase 2 - backward kernel helpers", its doc comment), written from
 * those equations with P taken from the forward's L:
 *
 *   P_ij  = exp(s_ij - L_i)  for a visible key, 0 otherwise
 *   dP_ij = <dO_i, v_j>,   D_i = sum_j P_ij dP_ij,   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i,   dV_j = sum_i P_ij dO_i
 *
 * where the sums of dK_j and dV_j run over the query rows of every query head
 * of the kv head's group (head by head, rows in order). D_i is written as the
 * page computes it, sum_j P_ij dP_ij (equal to rowsum(O_i * dO_i) for the
 * exact O); fa_oracle_bwd_given_o instead reads D_i = rowsum(O_i * dO_i) from
 * an O the caller hands in, the doc comment's own form for bf16-rounded
 * inputs, so that both sides of a comparison see the same rounded O. Pairs
 * (i, j) whose key is not allowed for the row contribute
 * exactly zero and are not visited. dQ is computed per query row, dK and dV
 * per key, so both parallelise without shared sums. With sinks the same
 * equations hold given the forward's L (the sink has no value, so it adds
 * nothing to dP or D_i); fa_oracle_bwd_sinks adds the sink logits' own
 * gradient, dsink_h = -sum_{b,i} exp(sink_h - L_i) D_i.
 *
 * Arithmetic is IEEE f32 with no contraction (built with -ffp-contract=off);
 * expf and logf come from the C library.
 */
#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const float *q, *k, *v, *mask;
    int64_t B, H, Hkv, ql, kl, D, Dv;
    float scale;
    int causal;
    int64_t window; /* < 0: no sliding window */
    const float *sinks; /* [H] natural-log logits, or NULL */
} oracle_problem;

/* ---- the definition, per (query row, key) ---- */

/* Key position of query row i (bottom-right alignment, offset clamped at 0). */
static int64_t query_position(const oracle_problem *p, int64_t i)
{
    return (p->kl > p->ql ? p->kl - p->ql : 0) + i;
}

/* Whether the causal rule and the window allow key j for a query at pos (the
   window comes with the causal rule). */
static int key_allowed(const oracle_problem *p, int64_t pos, int64_t j)
{
    if ((p->causal || p->window >= 0) && j > pos)
        return 0;
    if (p->window >= 0 && j < pos - p->window)
        return 0;
    return 1;
}

/* Score of key j for flat query row `row` (natural-log units), -inf when the
   key is not visible. qr: the row of q; kh: the kv head's keys. */
static float score(const oracle_problem *p, int64_t row, int64_t pos, int64_t j,
                   const float *qr, const float *kh)
{
    if (!key_allowed(p, pos, j))
        return -INFINITY;
    float dot = 0.0f;
    for (int64_t d = 0; d < p->D; ++d)
        dot += qr[d] * kh[j * p->D + d];
    float s = p->scale * dot;
    if (p->mask)
        s += p->mask[row * p->kl + j];
    return s;
}

/* The sink logit of a flat query row's head (-inf without sinks). */
static float row_sink(const oracle_problem *p, int64_t row)
{
    return p->sinks ? p->sinks[(row / p->ql) % p->H] : -INFINITY;
}

/* The kv head (b * Hkv + g) a flat query row reads, and its position. */
static void row_coords(const oracle_problem *p, int64_t row, int64_t *kvhead, int64_t *pos)
{
    const int64_t i = row % p->ql, bh = row / p->ql;
    const int64_t b = bh / p->H, h = bh % p->H;
    *kvhead = b * p->Hkv + h / (p->H / p->Hkv);
    *pos = query_position(p, i);
}

/* Forward of one query row: o gets Dv floats, *l the logsumexp; e: kl floats
   of scratch. */
static void forward_row(const oracle_problem *p, int64_t row, float *o, float *l, float *e)
{
    int64_t kvh, pos;
    row_coords(p, row, &kvh, &pos);
    const float *qr = p->q + row * p->D;
    const float *kh = p->k + kvh * p->kl * p->D;
    const float *vh = p->v + kvh * p->kl * p->Dv;
    float m = -INFINITY;
    for (int64_t j = 0; j < p->kl; ++j) {
        e[j] = score(p, row, pos, j, qr, kh);
        if (e[j] > m)
            m = e[j];
    }
    const float sink = row_sink(p, row);
    if (sink > m)
        m = sink;
    for (int64_t d = 0; d < p->Dv; ++d)
        o[d] = 0.0f;
    if (m == -INFINITY) { /* no visible key */
        *l = -INFINITY;
        return;
    }
    float z = 0.0f;
    for (int64_t j = 0; j < p->kl; ++j) {
        e[j] = expf(e[j] - m); /* hidden keys: exp(-inf) = 0 */
        z += e[j];
    }
    z += expf(sink - m); /* the sink's term (exactly 0 without one) */
    *l = m + logf(z);
    for (int64_t j = 0; j < p->kl; ++j) {
        if (e[j] == 0.0f) /* a hidden key adds exactly zero */
            continue;
        const float w = e[j] / z;
        for (int64_t d = 0; d < p->Dv; ++d)
            o[d] += w * vh[j * p->Dv + d];
    }
}

/* ---- a parallel loop over [0, n) ---- */

typedef void (*range_fn)(const void *ctx, int64_t begin, int64_t end, float *scratch);

typedef struct {
    range_fn fn;
    const void *ctx;
    int64_t begin, end;
    size_t scratch;
    int failed;
} range_job;

static void *range_worker(void *arg)
{
    range_job *j = (range_job *)arg;
    float *scratch = (float *)malloc(sizeof(float) * (j->scratch > 0 ? j->scratch : 1));
    if (!scratch) {
        j->failed = 1;
        return NULL;
    }
    j->fn(j->ctx, j->begin, j->end, scratch);
    free(scratch);
    return NULL;
}

/* Runs fn over [0, n) split into n_threads contiguous ranges, each with its
   own scratch of `scratch` floats. Returns 4 when memory ran out. */
static int run_parallel(int64_t n, int n_threads, size_t scratch, range_fn fn, const void *ctx)
{
    if (n <= 0)
        return 0;
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > 256)
        n_threads = 256;
    if (n_threads > n)
        n_threads = (int)n;
    range_job jobs[256];
    pthread_t tid[256];
    for (int t = 0; t < n_threads; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].begin = n * t / n_threads;
        jobs[t].end = n * (t + 1) / n_threads;
        jobs[t].scratch = scratch;
        jobs[t].failed = 0;
    }
    int started = 0;
    for (int t = 1; t < n_threads; ++t) {
        if (pthread_create(&tid[t], NULL, range_worker, &jobs[t]) != 0)
            break;
        started = t;
    }
    /* ranges of threads that could not be started run on this thread */
    for (int t = started + 1; t < n_threads; ++t)
        range_worker(&jobs[t]);
    range_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t)
        pthread_join(tid[t], NULL);
    for (int t = 0; t < n_threads; ++t)
        if (jobs[t].failed)
            return 4;
    return 0;
}

/* ---- forward entry points ---- */

typedef struct {
    const oracle_problem *p;
    const int64_t *rows; /* NULL: row t is flat row t */
    float *O, *L;
} forward_ctx;

static void forward_range(const void *ctx, int64_t begin, int64_t end, float *scratch)
{
    const forward_ctx *c = (const forward_ctx *)ctx;
    for (int64_t t = begin; t < end; ++t)
        forward_row(c->p, c->rows ? c->rows[t] : t, c->O + t * c->p->Dv, c->L + t, scratch);
}

static int validate(const float *q, const float *k, const float *v, int64_t B, int64_t H,
                    int64_t Hkv, int64_t ql, int64_t kl, int64_t D, int64_t Dv)
{
    if (B < 0 || ql < 0 || kl < 0 || H < 1 || Hkv < 1 || D < 1 || Dv < 1)
        return 2;
    if (H % Hkv != 0)
        return 3;
    if (B * H * ql > 0 && !q)
        return 1;
    if (B * Hkv * kl > 0 && (!k || !v))
        return 1;
    return 0;
}

/*
 * The general forward. Inputs are f32 host arrays (bf16 values widened
 * exactly): q [B,H,ql,D], k [B,Hkv,kl,D], v [B,Hkv,kl,Dv], mask [B,H,ql,kl]
 * (natural-log units, -inf hides a key) or NULL; sinks [H] (natural-log
 * logits) or NULL. causal: 0/1; window < 0:
 * none, >= 0: the sliding window, which includes the causal rule (whatever
 * `causal` says). rows == NULL: every row, O [B,H,ql,Dv] and
 * L [B,H,ql]; otherwise the n_rows flat rows listed ((b*H + h)*ql + i),
 * O [n_rows,Dv] and L [n_rows]. Returns 0 on success, 1 null pointer, 2 bad
 * size or row index, 3 H % Hkv != 0, 4 out of host memory.
 */
int fa_oracle_fwd_sinks(const float *q, const float *k, const float *v, const float *mask,
                        int64_t B, int64_t H, int64_t Hkv, int64_t ql, int64_t kl, int64_t D,
                        int64_t Dv, float scale, int causal, int64_t window, const float *sinks,
                        const int64_t *rows, int64_t n_rows, float *O, float *L, int n_threads)
{
    int rc = validate(q, k, v, B, H, Hkv, ql, kl, D, Dv);
    if (rc)
        return rc;
    const int64_t n = rows ? n_rows : B * H * ql;
    if (rows) {
        for (int64_t t = 0; t < n_rows; ++t)
            if (rows[t] < 0 || rows[t] >= B * H * ql)
                return 2;
    }
    if (n <= 0)
        return 0;
    if (!O || !L)
        return 1;
    oracle_problem p = {q, k, v, mask, B, H, Hkv, ql, kl, D, Dv, scale, causal != 0,
                        window < 0 ? -1 : window, sinks};
    forward_ctx c = {&p, rows, O, L};
    return run_parallel(n, n_threads, (size_t)(kl > 0 ? kl : 1), forward_range, &c);
}

/* The general forward without sinks. */
int fa_oracle_fwd_general(const float *q, const float *k, const float *v, const float *mask,
                          int64_t B, int64_t H, int64_t Hkv, int64_t ql, int64_t kl, int64_t D,
                          int64_t Dv, float scale, int causal, int64_t window,
                          const int64_t *rows, int64_t n_rows, float *O, float *L, int n_threads)
{
    return fa_oracle_fwd_sinks(q, k, v, mask, B, H, Hkv, ql, kl, D, Dv, scale, causal, window,
                               NULL, rows, n_rows, O, L, n_threads);
}

/* Full forward with Dv = D, no window (the layout of fa_oracle_fwd_general). */
int fa_oracle_fwd(const float *q, const float *k, const float *v, const float *mask, int64_t B,
                  int64_t H, int64_t Hkv, int64_t ql, int64_t kl, int64_t D, float scale,
                  int causal, float *O, float *L, int n_threads)
{
    return fa_oracle_fwd_general(q, k, v, mask, B, H, Hkv, ql, kl, D, D, scale, causal, -1, NULL,
                                 0, O, L, n_threads);
}

/* Selected flat rows, Dv = D, no window. */
int fa_oracle_fwd_rows(const float *q, const float *k, const float *v, const float *mask,
                       int64_t B, int64_t H, int64_t Hkv, int64_t ql, int64_t kl, int64_t D,
                       float scale, int causal, const int64_t *rows, int64_t n_rows, float *O,
                       float *L, int n_threads)
{
    if (n_rows > 0 && !rows)
        return 1;
    return fa_oracle_fwd_general(q, k, v, mask, B, H, Hkv, ql, kl, D, D, scale, causal, -1,
                                 rows ? rows : (const int64_t *)&n_rows, rows ? n_rows : 0, O, L,
                                 n_threads);
}

/* Sliding-window causal forward (window >= 0, else code 2), all rows
   (rows == NULL) or the listed ones; Dv = D. */
int fa_oracle_fwd_swa(const float *q, const float *k, const float *v, const float *mask,
                      int64_t B, int64_t H, int64_t Hkv, int64_t ql, int64_t kl, int64_t D,
                      float scale, int64_t window, const int64_t *rows, int64_t n_rows,
                      float *O, float *L, int n_threads)
{
    if (window < 0)
        return 2;
    return fa_oracle_fwd_general(q, k, v, mask, B, H, Hkv, ql, kl, D, D, scale, 1, window, rows,
                                 n_rows, O, L, n_threads);
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
    oracle_problem p;
    const float *L, *dO;
    const float *O;        /* NULL, or the given O [B,H,ql,Dv] that D_i is read from */
    const int64_t *groups; /* kv heads b * Hkv + g computed, in output order */
    int64_t n_groups, G;
    float *Di;             /* D_i of every computed query row (output order) */
    float *dQ, *dK, *dV;   /* [n_groups, G, ql, D], [n_groups, kl, D], [n_groups, kl, Dv] */
} backward_ctx;

/* Flat input row of output query row t (group-major: group, head, row). */
static int64_t bwd_query_row(const backward_ctx *c, int64_t t, int64_t *pos)
{
    const oracle_problem *p = &c->p;
    const int64_t per_group = c->G * p->ql;
    const int64_t kvh = c->groups[t / per_group], r = t % per_group;
    const int64_t b = kvh / p->Hkv, g = kvh % p->Hkv;
    const int64_t h = g * c->G + r / p->ql, i = r % p->ql;
    *pos = query_position(p, i);
    return (b * p->H + h) * p->ql + i;
}

/* dQ_i and D_i, per query row. */
static void backward_rows(const void *ctx, int64_t begin, int64_t end, float *scratch)
{
    const backward_ctx *c = (const backward_ctx *)ctx;
    const oracle_problem *p = &c->p;
    float *P = scratch, *dP = scratch + (p->kl > 0 ? p->kl : 1);
    for (int64_t t = begin; t < end; ++t) {
        int64_t pos, kvh, unused;
        const int64_t row = bwd_query_row(c, t, &pos);
        row_coords(p, row, &kvh, &unused);
        const float *qr = p->q + row * p->D, *gr = c->dO + row * p->Dv;
        const float *kh = p->k + kvh * p->kl * p->D, *vh = p->v + kvh * p->kl * p->Dv;
        const float l_i = c->L[row];
        float d_i = 0.0f;
        for (int64_t j = 0; j < p->kl; ++j) {
            const float s = score(p, row, pos, j, qr, kh);
            P[j] = (s == -INFINITY) ? 0.0f : expf(s - l_i);
            float dp = 0.0f;
            for (int64_t d = 0; d < p->Dv; ++d)
                dp += gr[d] * vh[j * p->Dv + d];
            dP[j] = dp;
            d_i += P[j] * dp;
        }
        if (c->O) { /* D_i = rowsum(O_i * dO_i) of the O the caller hands in */
            const float *orow = c->O + row * p->Dv;
            d_i = 0.0f;
            for (int64_t d = 0; d < p->Dv; ++d)
                d_i += orow[d] * gr[d];
        }
        c->Di[t] = d_i;
        float *dq = c->dQ + t * p->D;
        for (int64_t d = 0; d < p->D; ++d)
            dq[d] = 0.0f;
        for (int64_t j = 0; j < p->kl; ++j) {
            if (!key_allowed(p, pos, j))
                continue;
            const float coef = p->scale * (P[j] * (dP[j] - d_i));
            for (int64_t d = 0; d < p->D; ++d)
                dq[d] += coef * kh[j * p->D + d];
        }
    }
}

/* dK_j and dV_j, per key (after every D_i is known). */
static void backward_keys(const void *ctx, int64_t begin, int64_t end, float *scratch)
{
    (void)scratch;
    const backward_ctx *c = (const backward_ctx *)ctx;
    const oracle_problem *p = &c->p;
    for (int64_t u = begin; u < end; ++u) {
        const int64_t gi = u / p->kl, j = u % p->kl;
        const int64_t kvh = c->groups[gi];
        const float *kh = p->k + kvh * p->kl * p->D, *vh = p->v + kvh * p->kl * p->Dv;
        float *dk = c->dK + u * p->D, *dv = c->dV + u * p->Dv;
        for (int64_t d = 0; d < p->D; ++d)
            dk[d] = 0.0f;
        for (int64_t d = 0; d < p->Dv; ++d)
            dv[d] = 0.0f;
        for (int64_t r = 0; r < c->G * p->ql; ++r) {
            const int64_t t = gi * c->G * p->ql + r;
            int64_t pos;
            const int64_t row = bwd_query_row(c, t, &pos);
            if (!key_allowed(p, pos, j))
                continue;
            const float *qr = p->q + row * p->D, *gr = c->dO + row * p->Dv;
            const float s = score(p, row, pos, j, qr, kh);
            const float P = (s == -INFINITY) ? 0.0f : expf(s - c->L[row]);
            float dp = 0.0f;
            for (int64_t d = 0; d < p->Dv; ++d)
                dp += gr[d] * vh[j * p->Dv + d];
            const float coef = p->scale * (P * (dp - c->Di[t]));
            for (int64_t d = 0; d < p->Dv; ++d)
                dv[d] += P * gr[d];
            for (int64_t d = 0; d < p->D; ++d)
                dk[d] += coef * qr[d];
        }
    }
}

/*
 * The general backward. Inputs as fa_oracle_fwd_general, plus L [B,H,ql] (the
 * forward's natural-log logsumexp), dO [B,H,ql,Dv] and O (NULL: D_i is
 * sum_j P_ij dP_ij; else the O [B,H,ql,Dv] that D_i = rowsum(O_i * dO_i)
 * reads). groups: the kv heads
 * (b * Hkv + g) to compute, or NULL for all of them in order; the outputs
 * hold the computed kv heads in that order: dQ [n_groups, H/Hkv, ql, D] (the
 * group's query heads), dK [n_groups, kl, D], dV [n_groups, kl, Dv]. With
 * groups NULL that is dQ [B,H,ql,D], dK [B,Hkv,kl,D], dV [B,Hkv,kl,Dv].
 * Return codes as fa_oracle_fwd_general.
 */
static int backward(const float *q, const float *k, const float *v, const float *mask,
                    const float *L, const float *dO, const float *O, int64_t B, int64_t H,
                    int64_t Hkv, int64_t ql, int64_t kl, int64_t D, int64_t Dv, float scale,
                    int causal, int64_t window, const int64_t *groups, int64_t n_groups,
                    float *dQ, float *dK, float *dV, int n_threads)
{
    int rc = validate(q, k, v, B, H, Hkv, ql, kl, D, Dv);
    if (rc)
        return rc;
    int64_t *all = NULL;
    if (!groups) {
        n_groups = B * Hkv;
        all = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_groups > 0 ? n_groups : 1));
        if (!all)
            return 4;
        for (int64_t t = 0; t < n_groups; ++t)
            all[t] = t;
        groups = all;
    } else {
        for (int64_t t = 0; t < n_groups; ++t)
            if (groups[t] < 0 || groups[t] >= B * Hkv) {
                free(all);
                return 2;
            }
    }
    const int64_t G = H / Hkv;
    const int64_t n_q = n_groups * G * ql, n_k = n_groups * kl;
    if ((n_q > 0 && (!L || !dO || !dQ)) || (n_k > 0 && (!dK || !dV))) {
        free(all);
        return 1;
    }
    float *Di = (float *)malloc(sizeof(float) * (size_t)(n_q > 0 ? n_q : 1));
    if (!Di) {
        free(all);
        return 4;
    }
    backward_ctx c = {{q, k, v, mask, B, H, Hkv, ql, kl, D, Dv, scale, causal != 0,
                       window < 0 ? -1 : window, NULL},
                      L, dO, O, groups, n_groups, G, Di, dQ, dK, dV};
    rc = run_parallel(n_q, n_threads, (size_t)(2 * (kl > 0 ? kl : 1)), backward_rows, &c);
    if (!rc)
        rc = run_parallel(n_k, n_threads, 1, backward_keys, &c);
    free(Di);
    free(all);
    return rc;
}

int fa_oracle_bwd_general(const float *q, const float *k, const float *v, const float *mask,
                          const float *L, const float *dO, int64_t B, int64_t H, int64_t Hkv,
                          int64_t ql, int64_t kl, int64_t D, int64_t Dv, float scale, int causal,
                          int64_t window, const int64_t *groups, int64_t n_groups, float *dQ,
                          float *dK, float *dV, int n_threads)
{
    return backward(q, k, v, mask, L, dO, NULL, B, H, Hkv, ql, kl, D, Dv, scale, causal, window,
                    groups, n_groups, dQ, dK, dV, n_threads);
}

/*
 * The backward with D_i read from a given O [B,H,ql,Dv] (f32 values, e.g. the
 * forward's bf16 output widened): D_i = rowsum(O_i * dO_i), the form the
 * page's backward-helper doc comment states for bf16-rounded inputs. Every
 * other step as fa_oracle_bwd_general, for every kv head (window < 0: none,
 * else causal = 1 is needed, as fa_oracle_bwd_swa). O NULL: code 1.
 */
int fa_oracle_bwd_given_o(const float *q, const float *k, const float *v, const float *mask,
                          const float *L, const float *dO, const float *O, int64_t B, int64_t H,
                          int64_t Hkv, int64_t ql, int64_t kl, int64_t D, int64_t Dv, float scale,
                          int causal, int64_t window, float *dQ, float *dK, float *dV,
                          int n_threads)
{
    if (!O && B * H * ql * Dv > 0)
        return 1;
    if (window >= 0 && !causal)
        return 2;
    return backward(q, k, v, mask, L, dO, O, B, H, Hkv, ql, kl, D, Dv, scale, causal, window,
                    NULL, 0, dQ, dK, dV, n_threads);
}

/* Backward of every kv head, Dv = D, no window. */
int fa_oracle_bwd(const float *q, const float *k, const float *v, const float *mask,
                  const float *L, const float *dO, int64_t B, int64_t H, int64_t Hkv, int64_t ql,
                  int64_t kl, int64_t D, float scale, int causal, float *dQ, float *dK, float *dV,
                  int n_threads)
{
    return fa_oracle_bwd_general(q, k, v, mask, L, dO, B, H, Hkv, ql, kl, D, D, scale, causal, -1,
                                 NULL, 0, dQ, dK, dV, n_threads);
}

/* Backward with a sliding window (window >= 0 needs causal = 1, else code 2). */
int fa_oracle_bwd_swa(const float *q, const float *k, const float *v, const float *mask,
                      const float *L, const float *dO, int64_t B, int64_t H, int64_t Hkv,
                      int64_t ql, int64_t kl, int64_t D, float scale, int causal, int64_t window,
                      float *dQ, float *dK, float *dV, int n_threads)
{
    if (window >= 0 && !causal)
        return 2;
    return fa_oracle_bwd_general(q, k, v, mask, L, dO, B, H, Hkv, ql, kl, D, D, scale, causal,
                                 window, NULL, 0, dQ, dK, dV, n_threads);
}

/* ---- the gradient of the sink logits ---- */

typedef struct {
    oracle_problem p;
    const float *L, *dO;
    float *Di; /* D_i of every query row, [B,H,ql] */
} sink_ctx;

/* D_i = sum_j P_ij dP_ij of each flat query row, as the backward computes it. */
static void sink_rows(const void *ctx, int64_t begin, int64_t end, float *scratch)
{
    (void)scratch;
    const sink_ctx *c = (const sink_ctx *)ctx;
    const oracle_problem *p = &c->p;
    for (int64_t row = begin; row < end; ++row) {
        int64_t kvh, pos;
        row_coords(p, row, &kvh, &pos);
        const float *qr = p->q + row * p->D, *gr = c->dO + row * p->Dv;
        const float *kh = p->k + kvh * p->kl * p->D, *vh = p->v + kvh * p->kl * p->Dv;
        float d_i = 0.0f;
        for (int64_t j = 0; j < p->kl; ++j) {
            const float s = score(p, row, pos, j, qr, kh);
            if (s == -INFINITY)
                continue;
            const float P = expf(s - c->L[row]);
            float dp = 0.0f;
            for (int64_t d = 0; d < p->Dv; ++d)
                dp += gr[d] * vh[j * p->Dv + d];
            d_i += P * dp;
        }
        c->Di[row] = d_i;
    }
}

/*
 * The gradient of the loss with respect to each query head's sink logit, for
 * the forward with sinks (the reading above: one more softmax term, with a
 * zero value). O_i depends on sink_h only through L_i, whose derivative is
 * the sink's own weight p_i = exp(sink_h - L_i); so dO_i/dsink_h = -p_i O_i,
 * and with D_i = <dO_i, O_i> = sum_j P_ij dP_ij (as the backward computes it)
 *
 *     dsink_h = -sum_{b,i} p_i D_i     (over every batch and row of head h).
 *
 * A sink of -inf has p_i = 0 and a zero gradient. Inputs as
 * fa_oracle_bwd_general (L from the forward with the same sinks), sinks [H]
 * (read), dsinks [H] (written). p_i and each product in f32, the sum over
 * (b, i) in f64, in index order. Return codes as fa_oracle_fwd_general.
 */
int fa_oracle_bwd_sinks(const float *q, const float *k, const float *v, const float *mask,
                        const float *L, const float *dO, int64_t B, int64_t H, int64_t Hkv,
                        int64_t ql, int64_t kl, int64_t D, int64_t Dv, float scale, int causal,
                        int64_t window, const float *sinks, float *dsinks, int n_threads)
{
    int rc = validate(q, k, v, B, H, Hkv, ql, kl, D, Dv);
    if (rc)
        return rc;
    if (window >= 0 && !causal)
        return 2;
    const int64_t n = B * H * ql;
    if (!sinks || !dsinks || (n > 0 && (!L || !dO)))
        return 1;
    float *Di = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    if (!Di)
        return 4;
    sink_ctx c = {{q, k, v, mask, B, H, Hkv, ql, kl, D, Dv, scale, causal != 0,
                   window < 0 ? -1 : window, sinks},
                  L, dO, Di};
    rc = run_parallel(n, n_threads, 1, sink_rows, &c);
    if (!rc) {
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            if (sinks[h] != -INFINITY) {
                for (int64_t b = 0; b < B; ++b)
                    for (int64_t i = 0; i < ql; ++i) {
                        const int64_t row = (b * H + h) * ql + i;
                        const float p_i = expf(sinks[h] - L[row]);
                        acc += (double)(p_i * Di[row]);
                    }
            }
            dsinks[h] = (float)(-acc);
        }
    }
    free(Di);
    return rc;
}
