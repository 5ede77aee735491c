/*
 * oracle.c -- plain fp64 CPU reference for Parallax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no source, header or helper with the
 * HIP implementation.
 *
 * What it computes (page "Parallax: Parameterized Local Linear Attention
 * Gives Transformers a 'Second Eye'", section 1.3 and the formula in the
 * opening quote): for one query row with query q, probe rho, keys k_1..k_L
 * and values v_1..v_L,
 *
 *     s_j   = scale * (q . k_j)                        (softmax logits, sec 1.1)
 *     p_j   = exp(s_j) / sum_i exp(s_i)                (softmax weights)
 *     o_SA  = vbar = sum_j p_j v_j,   kbar = sum_j p_j k_j
 *     S_KV  = sum_j p_j (v_j - vbar)(k_j - kbar)^T     (dv x dk, weighted covariance
 *                                                       of K and V, sec 1.3)
 *     o     = o_SA - S_KV . rho                        (sec 1.3)
 *
 * Readings where the page is silent (each is listed with its reason in the
 * design notes): the covariance uses the same softmax weights p as o_SA, is
 * centred on both sides and divided by sum p = 1; rho contracts with the key
 * side so the output lives in value space; the logit scale applies to q.k
 * only; query head h reads KV head h / (Hq/Hkv); an empty row (L = 0) gives
 * o = 0; prefill row i sees keys 0..i.
 *
 * Local window (the "local window" the same page leaves open, section 3.1):
 * with window W >= 1 a row keeps only its W most recent keys -- a decode row
 * over L cached tokens uses keys max(0, L-W) .. L-1, prefill row i uses keys
 * max(0, i-W+1) .. i; W = 0 means every key (full attention).
 *
 * Two independent forms are provided:
 *   ORC_FORM_EXPLICIT  -- the definition above written out: logits, max,
 *                         normalised weights, weighted means, the explicit
 *                         dv x dk covariance matrix, then the matrix-vector
 *                         product with rho.  O(L dk dv) per row.
 *   ORC_FORM_STREAMING -- the one-pass form over the same sums: running max m,
 *                         Z = sum e^s, R = sum e^s t (t = rho . k), A = sum e^s v,
 *                         B = sum e^s t v, each rescaled by exp(m_old - m_new)
 *                         when the max grows, then o = a - (b - a r) with
 *                         a = A/Z, r = R/Z, b = B/Z.  O(L (dk + dv)) per row.
 *   The second follows from the first because sum_j p_j (v_j - vbar) = 0, so
 *   S_KV rho = sum_j p_j t_j v_j - vbar (sum_j p_j t_j).
 *
 * Training side (causal prefill): orc_prefill_stats gives the per-row
 * quantities a forward pass keeps for its backward pass (log of the softmax
 * denominator, r, o_SA) and orc_prefill_backward the gradients of
 * sum(dout * out) with respect to q, rho, k and v, by the chain rule through
 * the forward steps (written out above the two functions).
 *
 * Arithmetic: fp64, libm exp, sequential sums in index order.  Build with
 * -ffp-contract=off so results do not depend on FMA contraction.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2 };
enum { ORC_FORM_EXPLICIT = 0, ORC_FORM_STREAMING = 1 };

/* Read element i of an array of the given type as fp64.  bf16 is the upper
 * half of an IEEE binary32, so widening is exact. */
static double orc_get(const void *p, int dtype, int64_t i) {
    if (dtype == ORC_F64) return ((const double *)p)[i];
    if (dtype == ORC_F32) return (double)((const float *)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Where token j of (batch b, kv head hk) lives.  Strided mode (block_table
 * == NULL): offset = b*s0 + hk*sh + j*st.  Paged mode: the token sits in
 * physical page block_table[b][j / page_size] at slot j % page_size, and
 * offset = page*s0 + hk*sh + slot*st. */
typedef struct {
    const void *k, *v;
    int dtype;
    int64_t k_s0, k_sh, k_st;
    int64_t v_s0, v_sh, v_st;
    const int32_t *block_table;
    int page_size, max_blocks;
} orc_kv;

static int64_t kv_off(const orc_kv *kv, int is_v, int b, int hk, int j) {
    int64_t s0 = is_v ? kv->v_s0 : kv->k_s0;
    int64_t sh = is_v ? kv->v_sh : kv->k_sh;
    int64_t st = is_v ? kv->v_st : kv->k_st;
    if (kv->block_table == NULL) return (int64_t)b * s0 + (int64_t)hk * sh + (int64_t)j * st;
    int32_t page = kv->block_table[(int64_t)b * kv->max_blocks + j / kv->page_size];
    int slot = j % kv->page_size;
    return (int64_t)page * s0 + (int64_t)hk * sh + (int64_t)slot * st;
}

/* Scratch for one thread: logits (L), weighted means, a centred key,
 * covariance (dv x dk), moment sums, the row's q and rho in fp64. */
typedef struct {
    double *s, *kbar, *kc, *vbar, *cov, *A, *Bm, *qd, *rd;
} orc_scratch;

/* The definition written out (explicit covariance matrix), over the keys
 * j0 .. j1-1; logits of key j are kept in s[j - j0]. */
static void row_explicit(const double *q, const double *rho, int dk, int dv, double scale,
                         int j0, int j1, const orc_kv *kv, int b, int hk, double *o,
                         orc_scratch *w) {
    if (j1 <= j0) {
        for (int c = 0; c < dv; ++c) o[c] = 0.0;
        return;
    }
    double *p = w->s - j0;
    /* logits and their maximum */
    double smax = -INFINITY;
    for (int j = j0; j < j1; ++j) {
        int64_t ko = kv_off(kv, 0, b, hk, j);
        double dot = 0.0;
        for (int e = 0; e < dk; ++e) dot += q[e] * orc_get(kv->k, kv->dtype, ko + e);
        p[j] = scale * dot;
        if (p[j] > smax) smax = p[j];
    }
    /* softmax weights p_j (stored over the logits) */
    double den = 0.0;
    for (int j = j0; j < j1; ++j) {
        p[j] = exp(p[j] - smax);
        den += p[j];
    }
    for (int j = j0; j < j1; ++j) p[j] /= den;
    /* weighted means kbar, vbar (vbar is the softmax output o_SA) */
    for (int e = 0; e < dk; ++e) w->kbar[e] = 0.0;
    for (int c = 0; c < dv; ++c) w->vbar[c] = 0.0;
    for (int j = j0; j < j1; ++j) {
        int64_t ko = kv_off(kv, 0, b, hk, j), vo = kv_off(kv, 1, b, hk, j);
        for (int e = 0; e < dk; ++e) w->kbar[e] += p[j] * orc_get(kv->k, kv->dtype, ko + e);
        for (int c = 0; c < dv; ++c) w->vbar[c] += p[j] * orc_get(kv->v, kv->dtype, vo + c);
    }
    /* S_KV[c][e] = sum_j p_j (v_jc - vbar_c)(k_je - kbar_e) */
    memset(w->cov, 0, sizeof(double) * (size_t)dv * (size_t)dk);
    for (int j = j0; j < j1; ++j) {
        int64_t ko = kv_off(kv, 0, b, hk, j), vo = kv_off(kv, 1, b, hk, j);
        for (int e = 0; e < dk; ++e) w->kc[e] = orc_get(kv->k, kv->dtype, ko + e) - w->kbar[e];
        for (int c = 0; c < dv; ++c) {
            double dvc = p[j] * (orc_get(kv->v, kv->dtype, vo + c) - w->vbar[c]);
            double *row = w->cov + (size_t)c * (size_t)dk;
            for (int e = 0; e < dk; ++e) row[e] += dvc * w->kc[e];
        }
    }
    /* o = o_SA - S_KV rho */
    for (int c = 0; c < dv; ++c) {
        const double *row = w->cov + (size_t)c * (size_t)dk;
        double corr = 0.0;
        for (int e = 0; e < dk; ++e) corr += row[e] * rho[e];
        o[c] = w->vbar[c] - corr;
    }
}

/* The one-pass moment form (running max, Z, R, A, B) over keys j0 .. j1-1. */
static void row_streaming(const double *q, const double *rho, int dk, int dv, double scale,
                          int j0, int j1, const orc_kv *kv, int b, int hk, double *o,
                          orc_scratch *w) {
    if (j1 <= j0) {
        for (int c = 0; c < dv; ++c) o[c] = 0.0;
        return;
    }
    double m = -INFINITY, Z = 0.0, R = 0.0;
    for (int c = 0; c < dv; ++c) w->A[c] = w->Bm[c] = 0.0;
    for (int j = j0; j < j1; ++j) {
        int64_t ko = kv_off(kv, 0, b, hk, j), vo = kv_off(kv, 1, b, hk, j);
        double qk = 0.0, t = 0.0;
        for (int e = 0; e < dk; ++e) {
            double kje = orc_get(kv->k, kv->dtype, ko + e);
            qk += q[e] * kje;
            t += rho[e] * kje;
        }
        double s = scale * qk;
        double mn = s > m ? s : m;
        double alpha = (m == -INFINITY) ? 0.0 : exp(m - mn);
        double wj = exp(s - mn);
        double wt = wj * t;
        Z = alpha * Z + wj;
        R = alpha * R + wt;
        for (int c = 0; c < dv; ++c) {
            double vjc = orc_get(kv->v, kv->dtype, vo + c);
            w->A[c] = alpha * w->A[c] + wj * vjc;
            w->Bm[c] = alpha * w->Bm[c] + wt * vjc;
        }
        m = mn;
    }
    double r = R / Z;
    for (int c = 0; c < dv; ++c) {
        double a = w->A[c] / Z, bb = w->Bm[c] / Z;
        o[c] = a - (bb - a * r);
    }
}

/* ---------------------------------------------------------------- jobs --- */

typedef struct {
    /* problem */
    int form, dk, dv, Hq, Hkv;
    double scale;
    const void *q, *rho;
    int q_dtype, rho_dtype;
    orc_kv kv;
    double *out;
    /* decode: rows are (b, h); lengths from seq_lens or L_all */
    const int32_t *seq_lens;
    int L_all;
    /* prefill: rows are (b, row_sel[r], h) over S tokens; n_rows == 0 => decode */
    int S, n_rows;
    int window; /* 0: every key; W >= 1: the W most recent keys of each row */
    const int32_t *row_sel;
    int64_t n_units;
    int maxL;
    /* work split */
    int nthreads;
} orc_job;

typedef struct {
    const orc_job *job;
    int tid;
} orc_thread_arg;

static void *orc_worker(void *argp) {
    orc_thread_arg *ta = (orc_thread_arg *)argp;
    const orc_job *J = ta->job;
    orc_scratch w;
    size_t Ls = (size_t)(J->maxL > 0 ? J->maxL : 1);
    w.s = (double *)malloc(sizeof(double) * Ls);
    w.kbar = (double *)malloc(sizeof(double) * (size_t)J->dk);
    w.kc = (double *)malloc(sizeof(double) * (size_t)J->dk);
    w.vbar = (double *)malloc(sizeof(double) * (size_t)J->dv);
    w.A = (double *)malloc(sizeof(double) * (size_t)J->dv);
    w.Bm = (double *)malloc(sizeof(double) * (size_t)J->dv);
    w.qd = (double *)malloc(sizeof(double) * (size_t)J->dk);
    w.rd = (double *)malloc(sizeof(double) * (size_t)J->dk);
    w.cov = (J->form == ORC_FORM_EXPLICIT)
                ? (double *)malloc(sizeof(double) * (size_t)J->dk * (size_t)J->dv)
                : NULL;
    int G = J->Hq / J->Hkv;
    for (int64_t u = ta->tid; u < J->n_units; u += J->nthreads) {
        int b, h, L;
        int64_t qoff, ooff;
        if (J->n_rows == 0) { /* decode: q [B,Hq,dk], out [B,Hq,dv] */
            b = (int)(u / J->Hq);
            h = (int)(u % J->Hq);
            L = J->seq_lens ? J->seq_lens[b] : J->L_all;
            qoff = u * J->dk;
            ooff = u * J->dv;
        } else { /* prefill: q [B,S,Hq,dk], out [B,n_rows,Hq,dv] */
            int64_t per_b = (int64_t)J->n_rows * J->Hq;
            b = (int)(u / per_b);
            int r = (int)((u % per_b) / J->Hq);
            h = (int)(u % J->Hq);
            int i = J->row_sel[r];
            L = i + 1; /* causal: keys 0..i */
            qoff = (((int64_t)b * J->S + i) * J->Hq + h) * J->dk;
            ooff = u * J->dv;
        }
        /* keys j0 .. L-1: all of them, or the window's most recent ones */
        int j0 = (J->window > 0 && L > J->window) ? L - J->window : 0;
        for (int e = 0; e < J->dk; ++e) {
            w.qd[e] = orc_get(J->q, J->q_dtype, qoff + e);
            w.rd[e] = orc_get(J->rho, J->rho_dtype, qoff + e);
        }
        int hk = h / G;
        if (J->form == ORC_FORM_EXPLICIT)
            row_explicit(w.qd, w.rd, J->dk, J->dv, J->scale, j0, L, &J->kv, b, hk, J->out + ooff,
                         &w);
        else
            row_streaming(w.qd, w.rd, J->dk, J->dv, J->scale, j0, L, &J->kv, b, hk, J->out + ooff,
                          &w);
    }
    free(w.s); free(w.kbar); free(w.kc); free(w.vbar); free(w.A); free(w.Bm); free(w.qd); free(w.rd);
    free(w.cov);
    return NULL;
}

static int orc_run(orc_job *J, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if ((int64_t)nthreads > J->n_units) nthreads = (int)(J->n_units > 0 ? J->n_units : 1);
    J->nthreads = nthreads;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    orc_thread_arg *ta = (orc_thread_arg *)malloc(sizeof(orc_thread_arg) * (size_t)nthreads);
    int started = 0, rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        ta[i].job = J;
        ta[i].tid = i;
        if (i == 0) continue; /* thread 0 runs on the caller */
        if (pthread_create(&th[i], NULL, orc_worker, &ta[i]) != 0) { rc = -1; break; }
        started = i;
    }
    if (rc == 0) orc_worker(&ta[0]);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    free(th);
    free(ta);
    return rc;
}

/*
 * Decode: one query row per (batch b, query head h).
 *   q, rho : [B, Hq, dk] of q_dtype / rho_dtype
 *   k, v   : strided  -> element offset b*s0 + hk*sh + j*st (+ e)
 *            paged    -> page*s0 + hk*sh + slot*st (+ e), page from block_table
 *   seq_lens : [B] or NULL (then every row sees L_all tokens)
 *   window : 0 (every cached token) or W >= 1 (the last W of each row)
 *   out    : [B, Hq, dv] fp64
 * Returns 0 on success, -1 on bad arguments or thread failure.
 */
int orc_decode(int form, int B, int Hq, int Hkv, int dk, int dv, double scale,
               const void *q, int q_dtype, const void *rho, int rho_dtype,
               const void *k, const void *v, int kv_dtype,
               int64_t k_s0, int64_t k_sh, int64_t k_st,
               int64_t v_s0, int64_t v_sh, int64_t v_st,
               const int32_t *seq_lens, int L_all,
               const int32_t *block_table, int page_size, int max_blocks,
               int window, double *out, int nthreads) {
    if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || dk < 1 || dv < 1 || window < 0) return -1;
    if (block_table != NULL && page_size < 1) return -1;
    orc_job J;
    memset(&J, 0, sizeof J);
    J.form = form; J.dk = dk; J.dv = dv; J.Hq = Hq; J.Hkv = Hkv; J.scale = scale;
    J.q = q; J.rho = rho; J.q_dtype = q_dtype; J.rho_dtype = rho_dtype;
    J.kv.k = k; J.kv.v = v; J.kv.dtype = kv_dtype;
    J.kv.k_s0 = k_s0; J.kv.k_sh = k_sh; J.kv.k_st = k_st;
    J.kv.v_s0 = v_s0; J.kv.v_sh = v_sh; J.kv.v_st = v_st;
    J.kv.block_table = block_table; J.kv.page_size = page_size; J.kv.max_blocks = max_blocks;
    J.out = out; J.seq_lens = seq_lens; J.L_all = L_all;
    J.window = window;
    J.n_rows = 0;
    J.n_units = (int64_t)B * Hq;
    J.maxL = L_all;
    if (seq_lens)
        for (int b = 0; b < B; ++b) if (seq_lens[b] > J.maxL) J.maxL = seq_lens[b];
    return orc_run(&J, nthreads);
}

/*
 * Causal prefill: row i of (b, h) attends to keys 0..i of KV head h/(Hq/Hkv)
 * (with window W >= 1: keys max(0, i-W+1)..i).
 *   q, rho : [B, S, Hq, dk];  k: [B, S, Hkv, dk];  v: [B, S, Hkv, dv]
 *   rows   : n_rows query positions evaluated for every (b, h)
 *   out    : [B, n_rows, Hq, dv] fp64
 */
int orc_prefill(int form, int B, int S, int Hq, int Hkv, int dk, int dv, double scale,
                const void *q, int q_dtype, const void *rho, int rho_dtype,
                const void *k, const void *v, int kv_dtype,
                const int32_t *rows, int n_rows, int window, double *out, int nthreads) {
    if (B < 0 || S < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || dk < 1 || dv < 1 || n_rows < 1 ||
        window < 0)
        return -1;
    int maxL = 0;
    for (int r = 0; r < n_rows; ++r) {
        if (rows[r] < 0 || rows[r] >= S) return -1;
        if (rows[r] + 1 > maxL) maxL = rows[r] + 1;
    }
    orc_job J;
    memset(&J, 0, sizeof J);
    J.form = form; J.dk = dk; J.dv = dv; J.Hq = Hq; J.Hkv = Hkv; J.scale = scale;
    J.q = q; J.rho = rho; J.q_dtype = q_dtype; J.rho_dtype = rho_dtype;
    J.kv.k = k; J.kv.v = v; J.kv.dtype = kv_dtype;
    /* k [B,S,Hkv,dk]: batch stride S*Hkv*dk, head stride dk, token stride Hkv*dk */
    J.kv.k_s0 = (int64_t)S * Hkv * dk; J.kv.k_sh = dk; J.kv.k_st = (int64_t)Hkv * dk;
    J.kv.v_s0 = (int64_t)S * Hkv * dv; J.kv.v_sh = dv; J.kv.v_st = (int64_t)Hkv * dv;
    J.kv.block_table = NULL;
    J.out = out;
    J.S = S; J.n_rows = n_rows; J.row_sel = rows;
    J.window = window;
    J.n_units = (int64_t)B * n_rows * Hq;
    J.maxL = maxL;
    return orc_run(&J, nthreads);
}

/* ------------------------------------------------------------ training --- */
/*
 * Causal prefill, training side: the statistics a forward pass keeps for the
 * backward pass, and the gradients.  Both are written from the definition:
 * each query row recomputes its logits, weights and moments over its keys
 * (row i sees keys j0 .. i, j0 = max(0, i-W+1) with a window W >= 1, else 0).
 *
 * The gradient follows the chain rule through the steps of the forward pass
 * (page "Parallax: Parameterized Local Linear Attention Gives Transformers a
 * 'Second Eye'", section 1.3 for the forward; section 2.2 for training the
 * layer), for the scalar loss sum(dout * out):
 *
 *   o = a - b + a r        a = sum_j p_j v_j,  r = sum_j p_j t_j,
 *                          b = sum_j p_j t_j v_j
 *   gA = (1 + r) g,  gB = -g,  gR = a . g                    (g = dout row)
 *   dp_j = gA . v_j + gR t_j + t_j (gB . v_j)
 *   dt_j = p_j (gR + gB . v_j)
 *   dv_j += p_j (gA + t_j gB)
 *   ds_j = p_j (dp_j - sum_l p_l dp_l)                        (softmax)
 *   dq   = scale sum_j ds_j k_j,  dk_j += scale ds_j q        (s = scale q.k)
 *   drho = sum_j dt_j k_j,        dk_j += dt_j rho            (t = rho.k)
 */

typedef void (*orc_unit_fn)(const void *ctx, int64_t u, double *scratch);

typedef struct {
    const void *ctx;
    orc_unit_fn fn;
    int64_t n_units;
    size_t scratch_doubles;
    int nthreads, tid;
    int failed;
} orc_par_arg;

static void *orc_par_worker(void *argp) {
    orc_par_arg *a = (orc_par_arg *)argp;
    double *scratch = (double *)malloc(sizeof(double) * (a->scratch_doubles ? a->scratch_doubles : 1));
    if (scratch == NULL) {
        a->failed = 1;
        return NULL;
    }
    for (int64_t u = a->tid; u < a->n_units; u += a->nthreads) a->fn(a->ctx, u, scratch);
    free(scratch);
    return NULL;
}

/* Runs fn(ctx, u, scratch) for u = 0 .. n_units-1 on nthreads threads. */
static int orc_parallel(const void *ctx, orc_unit_fn fn, int64_t n_units, size_t scratch_doubles,
                        int nthreads) {
    if (n_units <= 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if ((int64_t)nthreads > n_units) nthreads = (int)n_units;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    orc_par_arg *ta = (orc_par_arg *)calloc((size_t)nthreads, sizeof(orc_par_arg));
    if (th == NULL || ta == NULL) {
        free(th);
        free(ta);
        return -1;
    }
    int started = 0, rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        ta[i].ctx = ctx; ta[i].fn = fn; ta[i].n_units = n_units;
        ta[i].scratch_doubles = scratch_doubles; ta[i].nthreads = nthreads; ta[i].tid = i;
        if (i == 0) continue;
        if (pthread_create(&th[i], NULL, orc_par_worker, &ta[i]) != 0) { rc = -1; break; }
        started = i;
    }
    if (rc == 0) orc_par_worker(&ta[0]);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; ++i) rc |= ta[i].failed ? -1 : 0;
    free(th);
    free(ta);
    return rc;
}

typedef struct {
    int B, S, Hq, Hkv, dk, dv, window;
    double scale;
    const void *q, *rho, *k, *v, *dout;
    int q_dtype, rho_dtype, kv_dtype, dout_dtype;
    const int32_t *rows;
    int n_rows;
    /* stats outputs, [B, n_rows, Hq] (+ dv) */
    double *lse, *rmean, *osa;
    /* gradient outputs */
    double *dq, *drho; /* [B, n_rows, Hq, dk] */
    double *dkk, *dvv; /* [B, S, Hkv, dk] / [B, S, Hkv, dv] */
} orc_train;

static double orc_k(const orc_train *T, int b, int j, int hk, int e) {
    return orc_get(T->k, T->kv_dtype, (((int64_t)b * T->S + j) * T->Hkv + hk) * T->dk + e);
}

static double orc_v(const orc_train *T, int b, int j, int hk, int c) {
    return orc_get(T->v, T->kv_dtype, (((int64_t)b * T->S + j) * T->Hkv + hk) * T->dv + c);
}

/* One row's forward quantities over keys j0..i: weights p (normalised), probe
 * projections t, the log of the softmax denominator (natural log, of the
 * unshifted logits), r = sum p t and a = sum p v (o_SA).  Returns j0. */
static int orc_row_forward(const orc_train *T, int b, int h, int i, const double *qd,
                           const double *rd, double *p, double *t, double *lse, double *r,
                           double *a) {
    int hk = h / (T->Hq / T->Hkv);
    int j0 = (T->window > 0 && i + 1 > T->window) ? i + 1 - T->window : 0;
    double smax = -INFINITY;
    for (int j = j0; j <= i; ++j) {
        double qk = 0.0, tj = 0.0;
        for (int e = 0; e < T->dk; ++e) {
            double kje = orc_k(T, b, j, hk, e);
            qk += qd[e] * kje;
            tj += rd[e] * kje;
        }
        p[j - j0] = T->scale * qk;
        t[j - j0] = tj;
        if (p[j - j0] > smax) smax = p[j - j0];
    }
    double den = 0.0;
    for (int j = j0; j <= i; ++j) {
        p[j - j0] = exp(p[j - j0] - smax);
        den += p[j - j0];
    }
    for (int j = j0; j <= i; ++j) p[j - j0] /= den;
    *lse = smax + log(den);
    double rr = 0.0;
    for (int j = j0; j <= i; ++j) rr += p[j - j0] * t[j - j0];
    *r = rr;
    for (int c = 0; c < T->dv; ++c) a[c] = 0.0;
    for (int j = j0; j <= i; ++j)
        for (int c = 0; c < T->dv; ++c) a[c] += p[j - j0] * orc_v(T, b, j, hk, c);
    return j0;
}

static void orc_load_row(const orc_train *T, int b, int h, int i, double *qd, double *rd) {
    int64_t off = (((int64_t)b * T->S + i) * T->Hq + h) * T->dk;
    for (int e = 0; e < T->dk; ++e) {
        qd[e] = orc_get(T->q, T->q_dtype, off + e);
        rd[e] = orc_get(T->rho, T->rho_dtype, off + e);
    }
}

/* unit = (b, selected row, h) */
static void orc_stats_unit(const void *ctx, int64_t u, double *w) {
    const orc_train *T = (const orc_train *)ctx;
    int64_t per_b = (int64_t)T->n_rows * T->Hq;
    int b = (int)(u / per_b), ri = (int)((u % per_b) / T->Hq), h = (int)(u % T->Hq);
    int i = T->rows[ri];
    double *qd = w, *rd = qd + T->dk, *p = rd + T->dk, *t = p + T->S;
    orc_load_row(T, b, h, i, qd, rd);
    orc_row_forward(T, b, h, i, qd, rd, p, t, &T->lse[u], &T->rmean[u], T->osa + u * T->dv);
}

/* unit = (b, kv head): every selected row of the G query heads that read it,
 * so the key/value gradients of this unit are summed by one thread in a
 * fixed order. */
static void orc_backward_unit(const void *ctx, int64_t u, double *w) {
    const orc_train *T = (const orc_train *)ctx;
    int b = (int)(u / T->Hkv), hk = (int)(u % T->Hkv);
    int G = T->Hq / T->Hkv, dk = T->dk, dv = T->dv;
    double *qd = w, *rd = qd + dk, *p = rd + dk, *t = p + T->S, *dp = t + T->S, *dt = dp + T->S;
    double *a = dt + T->S, *bv = a + dv, *g = bv + dv, *gA = g + dv, *gB = gA + dv;
    for (int h = hk * G; h < (hk + 1) * G; ++h) {
        for (int ri = 0; ri < T->n_rows; ++ri) {
            int i = T->rows[ri];
            orc_load_row(T, b, h, i, qd, rd);
            double lse, r;
            int j0 = orc_row_forward(T, b, h, i, qd, rd, p, t, &lse, &r, a);
            int n = i + 1 - j0;
            /* b = sum_j p_j t_j v_j */
            for (int c = 0; c < dv; ++c) bv[c] = 0.0;
            for (int jj = 0; jj < n; ++jj)
                for (int c = 0; c < dv; ++c) bv[c] += p[jj] * t[jj] * orc_v(T, b, j0 + jj, hk, c);
            /* o = a - b + a r  ->  gA = (1 + r) g, gB = -g, gR = a . g */
            int64_t go = (((int64_t)b * T->S + i) * T->Hq + h) * dv;
            double gR = 0.0;
            for (int c = 0; c < dv; ++c) {
                g[c] = orc_get(T->dout, T->dout_dtype, go + c);
                gA[c] = (1.0 + r) * g[c];
                gB[c] = -g[c];
                gR += a[c] * g[c];
            }
            /* a, r, b as sums over the keys -> gradients of p_j, t_j, v_j */
            for (int jj = 0; jj < n; ++jj) {
                int j = j0 + jj;
                double gAv = 0.0, gBv = 0.0;
                for (int c = 0; c < dv; ++c) {
                    double vjc = orc_v(T, b, j, hk, c);
                    gAv += gA[c] * vjc;
                    gBv += gB[c] * vjc;
                }
                dp[jj] = gAv + gR * t[jj] + t[jj] * gBv;
                dt[jj] = p[jj] * (gR + gBv);
                double *dvo = T->dvv + (((int64_t)b * T->S + j) * T->Hkv + hk) * dv;
                for (int c = 0; c < dv; ++c) dvo[c] += p[jj] * (gA[c] + t[jj] * gB[c]);
            }
            /* softmax: ds_j = p_j (dp_j - sum_l p_l dp_l); ds is kept in dp */
            double pdp = 0.0;
            for (int jj = 0; jj < n; ++jj) pdp += p[jj] * dp[jj];
            for (int jj = 0; jj < n; ++jj) dp[jj] = p[jj] * (dp[jj] - pdp);
            /* s_j = scale q . k_j and t_j = rho . k_j */
            int64_t qo = (((int64_t)b * T->n_rows + ri) * T->Hq + h) * dk;
            for (int e = 0; e < dk; ++e) T->dq[qo + e] = T->drho[qo + e] = 0.0;
            for (int jj = 0; jj < n; ++jj) {
                int j = j0 + jj;
                double *dko = T->dkk + (((int64_t)b * T->S + j) * T->Hkv + hk) * dk;
                for (int e = 0; e < dk; ++e) {
                    double kje = orc_k(T, b, j, hk, e);
                    T->dq[qo + e] += T->scale * dp[jj] * kje;
                    T->drho[qo + e] += dt[jj] * kje;
                    dko[e] += T->scale * dp[jj] * qd[e] + dt[jj] * rd[e];
                }
            }
        }
    }
}

static int orc_train_check(int B, int S, int Hq, int Hkv, int dk, int dv, int window,
                           const int32_t *rows, int n_rows) {
    if (B < 1 || S < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || dk < 1 || dv < 1 || window < 0 ||
        n_rows < 1 || rows == NULL)
        return -1;
    for (int r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= S) return -1;
    return 0;
}

/*
 * Forward statistics of causal prefill rows (what a forward pass keeps for
 * the backward pass):
 *   lse   [B, n_rows, Hq]      natural log of sum_j exp(scale q.k_j)
 *   rmean [B, n_rows, Hq]      r = sum_j p_j (rho . k_j)
 *   osa   [B, n_rows, Hq, dv]  a = o_SA = sum_j p_j v_j
 * Shapes as orc_prefill.
 */
int orc_prefill_stats(int B, int S, int Hq, int Hkv, int dk, int dv, double scale,
                      const void *q, int q_dtype, const void *rho, int rho_dtype,
                      const void *k, const void *v, int kv_dtype,
                      const int32_t *rows, int n_rows, int window,
                      double *lse, double *rmean, double *osa, int nthreads) {
    if (orc_train_check(B, S, Hq, Hkv, dk, dv, window, rows, n_rows) != 0) return -1;
    orc_train T;
    memset(&T, 0, sizeof T);
    T.B = B; T.S = S; T.Hq = Hq; T.Hkv = Hkv; T.dk = dk; T.dv = dv; T.window = window;
    T.scale = scale;
    T.q = q; T.rho = rho; T.k = k; T.v = v;
    T.q_dtype = q_dtype; T.rho_dtype = rho_dtype; T.kv_dtype = kv_dtype;
    T.rows = rows; T.n_rows = n_rows;
    T.lse = lse; T.rmean = rmean; T.osa = osa;
    return orc_parallel(&T, orc_stats_unit, (int64_t)B * n_rows * Hq,
                        (size_t)2 * dk + (size_t)2 * S, nthreads);
}

/*
 * Gradients of sum(dout * out) for causal prefill, out as orc_prefill.
 *   dout       [B, S, Hq, dv]
 *   rows       the query rows whose terms are included; dq, drho are given
 *              for them, and dk, dv sum the contributions of these rows only
 *              (so they are exact for key j when every row that sees key j
 *              is in rows; all rows 0..S-1 give the full gradients)
 *   dq, drho   [B, n_rows, Hq, dk]
 *   dk         [B, S, Hkv, dk];  dv [B, S, Hkv, dv]  (zeroed here)
 */
int orc_prefill_backward(int B, int S, int Hq, int Hkv, int dk, int dv, double scale,
                         const void *q, int q_dtype, const void *rho, int rho_dtype,
                         const void *k, const void *v, int kv_dtype,
                         const void *dout, int dout_dtype,
                         const int32_t *rows, int n_rows, int window,
                         double *dq, double *drho, double *dkk, double *dvv, int nthreads) {
    if (orc_train_check(B, S, Hq, Hkv, dk, dv, window, rows, n_rows) != 0) return -1;
    orc_train T;
    memset(&T, 0, sizeof T);
    T.B = B; T.S = S; T.Hq = Hq; T.Hkv = Hkv; T.dk = dk; T.dv = dv; T.window = window;
    T.scale = scale;
    T.q = q; T.rho = rho; T.k = k; T.v = v; T.dout = dout;
    T.q_dtype = q_dtype; T.rho_dtype = rho_dtype; T.kv_dtype = kv_dtype; T.dout_dtype = dout_dtype;
    T.rows = rows; T.n_rows = n_rows;
    T.dq = dq; T.drho = drho; T.dkk = dkk; T.dvv = dvv;
    memset(dkk, 0, sizeof(double) * (size_t)B * S * Hkv * dk);
    memset(dvv, 0, sizeof(double) * (size_t)B * S * Hkv * dv);
    return orc_parallel(&T, orc_backward_unit, (int64_t)B * Hkv,
                        (size_t)2 * dk + (size_t)4 * S + (size_t)5 * dv, nthreads);
}
