/*
 * h3_oracle.c -- plain fp64 CPU reference for the arithmetic steps of the
 * Ulysses H3 hot path.  TEST INFRASTRUCTURE ONLY: it is loaded by tests/,
 * by the smoke check and by the CPU-baseline leg of bench.py, never by the
 * product library.  It shares no code, header or constant with the HIP path.
 *
 * Everything is written for clarity, not speed: no blocking, no fusion, no
 * reordering beyond the definitions below.  The only concession to size is
 * that callers pick which rows to evaluate, so a huge problem can be checked
 * on a sample of rows, and that independent rows run on several threads.
 *
 * Inputs are raw bfloat16 bit patterns (uint16_t); each is widened exactly
 * to double (bits << 16 is the IEEE float with the same value).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_bits_to_double(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Segment-masked attention over a packed multi-segment sequence.           */
/*                                                                          */
/* Source: "Distributed H3 Execution", introduction -- attention runs on    */
/* the head side over the whole native packed sequence, with no semantic    */
/* padding.  The pages do not write the score function out; the reading    */
/* taken is plain softmax attention restricted to the query's own segment   */
/* (block-diagonal, non-causal), logits scaled by 1/sqrt(head_dim) given    */
/* by the caller.  For the gated QKVG form ("[perf] Harden Ulysses          */
/* agreement ...", Problem and behavior: packed QKVG operands) the fourth   */
/* plane G gates the output elementwise: o <- o * 1/(1+exp(-g)).            */
/*                                                                          */
/* Layout of q, k, v, g: [n_tokens][n_heads][head_dim], token-major.        */
/* out: [n_rows][n_heads][head_dim] doubles, row r is token rows[r].        */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint16_t *q, *k, *v, *g;
    int64_t n_tokens;
    int32_t n_heads, head_dim;
    const int64_t *cu;
    int32_t n_seg;
    double scale;
    const int64_t *rows;
    int64_t n_rows;
    double *out;
    int64_t next_task;      /* shared work counter, guarded by lock */
    pthread_mutex_t lock;
    int status;
} attn_job;

/* Which segment holds token t: the s with cu[s] <= t < cu[s+1]. */
static int32_t segment_of(const int64_t *cu, int32_t n_seg, int64_t t) {
    for (int32_t s = 0; s < n_seg; ++s)
        if (cu[s] <= t && t < cu[s + 1]) return s;
    return -1;
}

static void attn_one(const attn_job *J, int64_t r, int32_t h, double *z, double *qrow, double *acc) {
    const int32_t D = J->head_dim, H = J->n_heads;
    const int64_t t = J->rows[r];
    const int32_t s = segment_of(J->cu, J->n_seg, t);
    const int64_t lo = J->cu[s], hi = J->cu[s + 1];
    for (int32_t d = 0; d < D; ++d) qrow[d] = bf16_bits_to_double(J->q[(t * H + h) * D + d]);
    /* logits z_u = scale * <q_t, k_u> for every key u of the same segment */
    double zmax = -INFINITY;
    for (int64_t u = lo; u < hi; ++u) {
        double dot = 0.0;
        const uint16_t *krow = J->k + (u * H + h) * D;
        for (int32_t d = 0; d < D; ++d) dot += qrow[d] * bf16_bits_to_double(krow[d]);
        z[u - lo] = J->scale * dot;
        if (z[u - lo] > zmax) zmax = z[u - lo];
    }
    /* softmax weights and the weighted sum of value rows */
    double denom = 0.0;
    for (int32_t d = 0; d < D; ++d) acc[d] = 0.0;
    for (int64_t u = lo; u < hi; ++u) {
        double p = exp(z[u - lo] - zmax);
        denom += p;
        const uint16_t *vrow = J->v + (u * H + h) * D;
        for (int32_t d = 0; d < D; ++d) acc[d] += p * bf16_bits_to_double(vrow[d]);
    }
    double *o = J->out + (r * H + h) * D;
    for (int32_t d = 0; d < D; ++d) {
        double val = acc[d] / denom;
        if (J->g) {
            double gv = bf16_bits_to_double(J->g[(t * H + h) * D + d]);
            val *= 1.0 / (1.0 + exp(-gv));
        }
        o[d] = val;
    }
}

static void *attn_worker(void *arg) {
    attn_job *J = (attn_job *)arg;
    int64_t longest = 0;
    for (int32_t s = 0; s < J->n_seg; ++s)
        if (J->cu[s + 1] - J->cu[s] > longest) longest = J->cu[s + 1] - J->cu[s];
    double *z = (double *)malloc(sizeof(double) * (size_t)(longest > 0 ? longest : 1));
    double *qrow = (double *)malloc(sizeof(double) * (size_t)J->head_dim);
    double *acc = (double *)malloc(sizeof(double) * (size_t)J->head_dim);
    if (!z || !qrow || !acc) {
        pthread_mutex_lock(&J->lock);
        J->status = -2;
        pthread_mutex_unlock(&J->lock);
        free(z); free(qrow); free(acc);
        return NULL;
    }
    const int64_t total = J->n_rows * J->n_heads;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t task = J->next_task++;
        pthread_mutex_unlock(&J->lock);
        if (task >= total) break;
        attn_one(J, task / J->n_heads, (int32_t)(task % J->n_heads), z, qrow, acc);
    }
    free(z); free(qrow); free(acc);
    return NULL;
}

static int run_threads(void *(*fn)(void *), void *job, int32_t n_threads) {
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    pthread_t tid[256];
    int started = 0;
    for (int32_t i = 0; i < n_threads; ++i) {
        if (pthread_create(&tid[i], NULL, fn, job) != 0) break;
        ++started;
    }
    if (started == 0) fn(job);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward of the segment-masked, optionally gated attention above.        */
/*                                                                          */
/* With z_tu = scale*<q_t,k_u> over the keys u of t's segment,              */
/* p_tu = exp(z_tu - lse_t), lse_t = ln sum_u exp(z_tu), the ungated row    */
/* a_t = sum_u p_tu v_u and the output o_t = a_t * sig(g_t) (sig = 1 when   */
/* there is no gate), the chain rule for an incoming gradient do_t gives:   */
/*   e_t   = do_t * sig(g_t)               (gradient reaching a_t)         */
/*   dg_t  = do_t * a_t * sig(g_t) * (1 - sig(g_t))                          */
/*   D_t   = <e_t, a_t>                                                     */
/*   ds_tu = p_tu * (<e_t, v_u> - D_t)     (softmax Jacobian)               */
/*   dq_t  = scale * sum_u ds_tu k_u                                        */
/*   dk_u  = scale * sum_t ds_tu q_t,   dv_u = sum_t p_tu e_t               */
/* The query-side terms of one row need only that row; the key-side terms  */
/* of one key need lse_t and D_t of every query t of its segment.          */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint16_t *q, *k, *v, *g, *dout;
    int64_t n_tokens;
    int32_t n_heads, head_dim;
    const int64_t *cu;
    int32_t n_seg;
    double scale;
    const int64_t *rows;        /* query rows (row pass) or key rows (key pass) */
    int64_t n_rows;
    double *lse, *delta;        /* row pass: outputs [n_rows][H]; key pass: inputs [n_tokens][H] */
    double *dq, *dg;            /* row pass: [n_rows][H][D] (dg may be NULL) */
    double *dk, *dv;            /* key pass: [n_rows][H][D] */
    int64_t next_task;
    pthread_mutex_t lock;
    int status;
} bwd_job;

static double sig(double x) { return 1.0 / (1.0 + exp(-x)); }

/* query-side terms of row r (token t), head h */
static void bwd_row_one(const bwd_job *J, int64_t r, int32_t h, double *z, double *qrow, double *a, double *e) {
    const int32_t D = J->head_dim, H = J->n_heads;
    const int64_t t = J->rows[r];
    const int32_t s = segment_of(J->cu, J->n_seg, t);
    const int64_t lo = J->cu[s], hi = J->cu[s + 1];
    for (int32_t d = 0; d < D; ++d) qrow[d] = bf16_bits_to_double(J->q[(t * H + h) * D + d]);
    double zmax = -INFINITY;
    for (int64_t u = lo; u < hi; ++u) {
        double dot = 0.0;
        const uint16_t *krow = J->k + (u * H + h) * D;
        for (int32_t d = 0; d < D; ++d) dot += qrow[d] * bf16_bits_to_double(krow[d]);
        z[u - lo] = J->scale * dot;
        if (z[u - lo] > zmax) zmax = z[u - lo];
    }
    double denom = 0.0;
    for (int64_t u = lo; u < hi; ++u) denom += exp(z[u - lo] - zmax);
    const double lse = zmax + log(denom);
    /* a_t and e_t */
    for (int32_t d = 0; d < D; ++d) a[d] = 0.0;
    for (int64_t u = lo; u < hi; ++u) {
        const double p = exp(z[u - lo] - lse);
        const uint16_t *vrow = J->v + (u * H + h) * D;
        for (int32_t d = 0; d < D; ++d) a[d] += p * bf16_bits_to_double(vrow[d]);
    }
    double delta = 0.0;
    for (int32_t d = 0; d < D; ++d) {
        const double dov = bf16_bits_to_double(J->dout[(t * H + h) * D + d]);
        const double sg = J->g ? sig(bf16_bits_to_double(J->g[(t * H + h) * D + d])) : 1.0;
        e[d] = dov * sg;
        if (J->dg) J->dg[(r * H + h) * D + d] = J->g ? dov * a[d] * sg * (1.0 - sg) : 0.0;
        delta += e[d] * a[d];
    }
    J->lse[r * H + h] = lse;
    J->delta[r * H + h] = delta;
    if (!J->dq) return;     /* only lse and delta asked for */
    /* dq_t = scale * sum_u p_tu (<e_t, v_u> - D_t) k_u */
    double *dq = J->dq + (r * H + h) * D;
    for (int32_t d = 0; d < D; ++d) dq[d] = 0.0;
    for (int64_t u = lo; u < hi; ++u) {
        const double p = exp(z[u - lo] - lse);
        const uint16_t *vrow = J->v + (u * H + h) * D;
        double dp = 0.0;
        for (int32_t d = 0; d < D; ++d) dp += e[d] * bf16_bits_to_double(vrow[d]);
        const double ds = p * (dp - delta);
        const uint16_t *krow = J->k + (u * H + h) * D;
        for (int32_t d = 0; d < D; ++d) dq[d] += J->scale * ds * bf16_bits_to_double(krow[d]);
    }
}

/* key-side terms of key row r (token u), head h; lse and delta hold every token's values */
static void bwd_key_one(const bwd_job *J, int64_t r, int32_t h, double *krow, double *vrow) {
    const int32_t D = J->head_dim, H = J->n_heads;
    const int64_t u = J->rows[r];
    const int32_t s = segment_of(J->cu, J->n_seg, u);
    const int64_t lo = J->cu[s], hi = J->cu[s + 1];
    for (int32_t d = 0; d < D; ++d) {
        krow[d] = bf16_bits_to_double(J->k[(u * H + h) * D + d]);
        vrow[d] = bf16_bits_to_double(J->v[(u * H + h) * D + d]);
    }
    double *dk = J->dk + (r * H + h) * D, *dv = J->dv + (r * H + h) * D;
    for (int32_t d = 0; d < D; ++d) dk[d] = dv[d] = 0.0;
    for (int64_t t = lo; t < hi; ++t) {
        double dot = 0.0;
        for (int32_t d = 0; d < D; ++d) dot += bf16_bits_to_double(J->q[(t * H + h) * D + d]) * krow[d];
        const double p = exp(J->scale * dot - J->lse[t * H + h]);
        double dp = 0.0;
        for (int32_t d = 0; d < D; ++d) {
            const double dov = bf16_bits_to_double(J->dout[(t * H + h) * D + d]);
            const double sg = J->g ? sig(bf16_bits_to_double(J->g[(t * H + h) * D + d])) : 1.0;
            const double ed = dov * sg;
            dv[d] += p * ed;
            dp += ed * vrow[d];
        }
        const double ds = p * (dp - J->delta[t * H + h]);
        for (int32_t d = 0; d < D; ++d) dk[d] += J->scale * ds * bf16_bits_to_double(J->q[(t * H + h) * D + d]);
    }
}

static void *bwd_row_worker(void *arg) {
    bwd_job *J = (bwd_job *)arg;
    int64_t longest = 0;
    for (int32_t s = 0; s < J->n_seg; ++s)
        if (J->cu[s + 1] - J->cu[s] > longest) longest = J->cu[s + 1] - J->cu[s];
    double *z = (double *)malloc(sizeof(double) * (size_t)(longest > 0 ? longest : 1));
    double *buf = (double *)malloc(sizeof(double) * 3 * (size_t)J->head_dim);
    if (!z || !buf) {
        pthread_mutex_lock(&J->lock);
        J->status = -2;
        pthread_mutex_unlock(&J->lock);
        free(z); free(buf);
        return NULL;
    }
    const int64_t total = J->n_rows * J->n_heads;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t task = J->next_task++;
        pthread_mutex_unlock(&J->lock);
        if (task >= total) break;
        bwd_row_one(J, task / J->n_heads, (int32_t)(task % J->n_heads), z, buf, buf + J->head_dim,
                    buf + 2 * J->head_dim);
    }
    free(z); free(buf);
    return NULL;
}

static void *bwd_key_worker(void *arg) {
    bwd_job *J = (bwd_job *)arg;
    double *buf = (double *)malloc(sizeof(double) * 2 * (size_t)J->head_dim);
    if (!buf) {
        pthread_mutex_lock(&J->lock);
        J->status = -2;
        pthread_mutex_unlock(&J->lock);
        return NULL;
    }
    const int64_t total = J->n_rows * J->n_heads;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t task = J->next_task++;
        pthread_mutex_unlock(&J->lock);
        if (task >= total) break;
        bwd_key_one(J, task / J->n_heads, (int32_t)(task % J->n_heads), buf, buf + J->head_dim);
    }
    free(buf);
    return NULL;
}

static int bwd_check(const int64_t *cu, int32_t n_seg, int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                     const int64_t *rows, int64_t n_rows) {
    if (n_seg < 1 || n_heads < 1 || head_dim < 1 || !cu || cu[0] != 0 || cu[n_seg] != n_tokens) return -1;
    for (int32_t s = 0; s < n_seg; ++s)
        if (cu[s + 1] <= cu[s]) return -1;
    if (n_rows > 0 && !rows) return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= n_tokens) return -1;
    return 0;
}

/* Query-side pass: lse, delta [n_rows][H]; dq, dg [n_rows][H][D] (dg NULL when g is NULL; dq NULL
 * when only lse and delta are wanted). */
int h3o_attn_bwd_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                      const uint16_t *dout, int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                      const int64_t *cu, int32_t n_seg, double scale, const int64_t *rows, int64_t n_rows,
                      double *lse, double *delta, double *dq, double *dg, int32_t n_threads) {
    if (!q || !k || !v || !dout || !lse || !delta) return -1;
    if (bwd_check(cu, n_seg, n_tokens, n_heads, head_dim, rows, n_rows)) return -1;
    bwd_job J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.g = g; J.dout = dout;
    J.n_tokens = n_tokens; J.n_heads = n_heads; J.head_dim = head_dim;
    J.cu = cu; J.n_seg = n_seg; J.scale = scale;
    J.rows = rows; J.n_rows = n_rows;
    J.lse = lse; J.delta = delta; J.dq = dq; J.dg = g ? dg : NULL;
    pthread_mutex_init(&J.lock, NULL);
    run_threads(bwd_row_worker, &J, n_threads);
    pthread_mutex_destroy(&J.lock);
    return J.status;
}

/* Key-side pass: dk, dv [n_rows][H][D] for key rows; lse_all, delta_all [n_tokens][H] from the
 * query-side pass over every token of the segments involved. */
int h3o_attn_bwd_keys(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                      const uint16_t *dout, int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                      const int64_t *cu, int32_t n_seg, double scale, const int64_t *rows, int64_t n_rows,
                      const double *lse_all, const double *delta_all, double *dk, double *dv, int32_t n_threads) {
    if (!q || !k || !v || !dout || !lse_all || !delta_all || !dk || !dv) return -1;
    if (bwd_check(cu, n_seg, n_tokens, n_heads, head_dim, rows, n_rows)) return -1;
    bwd_job J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.g = g; J.dout = dout;
    J.n_tokens = n_tokens; J.n_heads = n_heads; J.head_dim = head_dim;
    J.cu = cu; J.n_seg = n_seg; J.scale = scale;
    J.rows = rows; J.n_rows = n_rows;
    J.lse = (double *)lse_all; J.delta = (double *)delta_all; J.dk = dk; J.dv = dv;
    pthread_mutex_init(&J.lock, NULL);
    run_threads(bwd_key_worker, &J, n_threads);
    pthread_mutex_destroy(&J.lock);
    return J.status;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int h3o_attn_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v, const uint16_t *g,
                  int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                  const int64_t *cu, int32_t n_seg, double scale,
                  const int64_t *rows, int64_t n_rows, double *out, int32_t n_threads) {
    if (!q || !k || !v || !cu || !out || (n_rows > 0 && !rows)) return -1;
    if (n_seg < 1 || n_heads < 1 || head_dim < 1 || cu[0] != 0 || cu[n_seg] != n_tokens) return -1;
    for (int32_t s = 0; s < n_seg; ++s)
        if (cu[s + 1] <= cu[s]) return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= n_tokens) return -1;
    attn_job J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.g = g;
    J.n_tokens = n_tokens; J.n_heads = n_heads; J.head_dim = head_dim;
    J.cu = cu; J.n_seg = n_seg; J.scale = scale;
    J.rows = rows; J.n_rows = n_rows; J.out = out;
    pthread_mutex_init(&J.lock, NULL);
    run_threads(attn_worker, &J, n_threads);
    pthread_mutex_destroy(&J.lock);
    return J.status;
}

/* ------------------------------------------------------------------------ */
/* Per-segment AdaLN modulation and residual gating on one token interval.  */
/*                                                                          */
/* Source: "Distributed H3 Execution", Partition Contract -- a token-       */
/* sharded rank's local row i is global token a + i, and each segment is    */
/* intersected with [a, b) and shifted by -a for these ops.  That table is  */
/* computed by the caller (oracle.clip_segments) and passed in as           */
/* (seg_id[e], local_begin[e], local_end[e]).  The pages name the two ops   */
/* but do not write them out; the reading taken is the usual DiT form:      */
/*   MODULATE (mode 0): y = (x - mean) / sqrt(var + eps) * (1 + scale_s)    */
/*                      + shift_s, mean and biased var over the channels;   */
/*   GATE     (mode 1): y = x + gate_s * b.                                 */
/*   GATE then MODULATE (mode 2): the residual x + gate_s * b of one         */
/*                      sub-block, modulated by the next sub-block's        */
/*                      shift_s / scale_s (the chain the pages' clipped     */
/*                      table serves; the residual itself is mode 1).       */
/* Parameters are rows of [n_segments][channels], picked by GLOBAL id s.    */
/*                                                                          */
/* x, b: [n_local][channels].  rows: local row indices to evaluate.         */
/* out: [n_rows][channels] doubles.                                         */
/* ------------------------------------------------------------------------ */

typedef struct {
    int32_t mode;
    const uint16_t *x, *b, *shift, *scale, *gate;
    int64_t n_local;
    int32_t channels;
    const int32_t *seg_id;
    const int64_t *local_begin, *local_end;
    int32_t n_entries;
    double eps;
    const int64_t *rows;
    int64_t n_rows;
    double *out;
    int64_t next_task;
    pthread_mutex_t lock;
    int status;
} adaln_job;

/* LayerNorm of the fp64 row v (mean and biased variance over its C values),
 * then * (1 + scale[s]) + shift[s], in place. */
static void modulate_row(const adaln_job *J, int32_t s, double *v) {
    const int32_t C = J->channels;
    double mean = 0.0;
    for (int32_t c = 0; c < C; ++c) mean += v[c];
    mean /= C;
    double var = 0.0;
    for (int32_t c = 0; c < C; ++c) {
        double dev = v[c] - mean;
        var += dev * dev;
    }
    var /= C;
    double inv = 1.0 / sqrt(var + J->eps);
    for (int32_t c = 0; c < C; ++c) {
        double xhat = (v[c] - mean) * inv;
        double sc = bf16_bits_to_double(J->scale[(int64_t)s * C + c]);
        double sh = bf16_bits_to_double(J->shift[(int64_t)s * C + c]);
        v[c] = xhat * (1.0 + sc) + sh;
    }
}

static void adaln_one(const adaln_job *J, int64_t r) {
    const int64_t i = J->rows[r];
    const int32_t C = J->channels;
    int32_t s = -1;
    for (int32_t e = 0; e < J->n_entries; ++e)
        if (J->local_begin[e] <= i && i < J->local_end[e]) { s = J->seg_id[e]; break; }
    double *y = J->out + r * C;
    if (s < 0) {                     /* row not covered by any segment: caller error */
        for (int32_t c = 0; c < C; ++c) y[c] = NAN;
        return;
    }
    const uint16_t *xr = J->x + i * C;
    if (J->mode == 0) {              /* modulation of x */
        for (int32_t c = 0; c < C; ++c) y[c] = bf16_bits_to_double(xr[c]);
        modulate_row(J, s, y);
    } else {                         /* residual gating x + gate[s] * b ... */
        const uint16_t *br = J->b + i * C;
        for (int32_t c = 0; c < C; ++c) {
            double gt = bf16_bits_to_double(J->gate[(int64_t)s * C + c]);
            y[c] = bf16_bits_to_double(xr[c]) + gt * bf16_bits_to_double(br[c]);
        }
        if (J->mode == 2) modulate_row(J, s, y);   /* ... then the next sub-block's modulation of it */
    }
}

static void *adaln_worker(void *arg) {
    adaln_job *J = (adaln_job *)arg;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t task = J->next_task;
        J->next_task += 64;
        pthread_mutex_unlock(&J->lock);
        if (task >= J->n_rows) break;
        int64_t end = task + 64 < J->n_rows ? task + 64 : J->n_rows;
        for (int64_t r = task; r < end; ++r) adaln_one(J, r);
    }
    return NULL;
}

int h3o_adaln_rows(int32_t mode, const uint16_t *x, const uint16_t *b,
                   const uint16_t *shift, const uint16_t *scale, const uint16_t *gate,
                   int64_t n_local, int32_t channels,
                   const int32_t *seg_id, const int64_t *local_begin, const int64_t *local_end,
                   int32_t n_entries, double eps,
                   const int64_t *rows, int64_t n_rows, double *out, int32_t n_threads) {
    if (!x || !out || channels < 1 || n_entries < 0 || (n_rows > 0 && !rows)) return -1;
    if (mode != 0 && mode != 1 && mode != 2) return -1;
    if (mode != 1 && (!shift || !scale)) return -1;
    if (mode != 0 && (!b || !gate)) return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= n_local) return -1;
    adaln_job J;
    memset(&J, 0, sizeof J);
    J.mode = mode; J.x = x; J.b = b; J.shift = shift; J.scale = scale; J.gate = gate;
    J.n_local = n_local; J.channels = channels;
    J.seg_id = seg_id; J.local_begin = local_begin; J.local_end = local_end;
    J.n_entries = n_entries; J.eps = eps;
    J.rows = rows; J.n_rows = n_rows; J.out = out;
    pthread_mutex_init(&J.lock, NULL);
    run_threads(adaln_worker, &J, n_threads);
    pthread_mutex_destroy(&J.lock);
    return J.status;
}
