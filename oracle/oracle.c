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
