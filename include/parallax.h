/*
 * parallax.h -- C ABI of libparallax: Parallax attention on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (page "Parallax: Parameterized Local Linear Attention Gives
 * Transformers a 'Second Eye'", section 1.3, and the formula quoted at its
 * top): for each query row with query q, probe rho and the keys k_j / values
 * v_j it attends to,
 *
 *     s_j  = scale * (q . k_j),   p_j = softmax(s)_j,   t_j = rho . k_j
 *     o_SA = sum_j p_j v_j
 *     S_KV = sum_j p_j (v_j - vbar)(k_j - kbar)^T      (weighted covariance of K and V)
 *     o    = o_SA - S_KV rho
 *
 * which one pass over the cache evaluates through Z = sum e^{s_j},
 * R = sum e^{s_j} t_j, A = sum e^{s_j} v_j, B = sum e^{s_j} t_j v_j as
 * o = A/Z - B/Z + A R / Z^2.  The keys and values are read once and serve both
 * the softmax branch and the covariance branch (page "Parallax keeps softmax,
 * adds covariance correction branch", second paragraph).  rho is an input:
 * in the model it is a learned projection W_R x of the layer input (page
 * "Parallax: Parameterized Local Linear Attention...", section 1.3); W_R = 0
 * gives plain softmax attention.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or synchronises.
 *   - Strides are in ELEMENTS of the tensor's own type; the last (head-dim)
 *     axis is always contiguous.
 *   - Calls are asynchronous on `hip_stream` (a hipStream_t; NULL = the null
 *     stream).  A status of PARALLAX_OK means the work was enqueued.
 *   - All argument checks run on the host before any HIP call; on error
 *     nothing is launched and no memory is touched.  parallax_last_error()
 *     then describes the failure (thread-local).
 *   - Grouped-query attention: query head h reads KV head h / (Hq / Hkv).
 *   - Supported head dims: 64 and 128 (d_k = d_v = head_dim).
 *   - Every key/value/query/probe/output row, and every pointer, must be
 *     16-byte aligned (strides times element size multiples of 16 bytes);
 *     otherwise PARALLAX_ERR_UNSUPPORTED.
 */
#ifndef PARALLAX_H
#define PARALLAX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PARALLAX_ABI_VERSION 5 /* 4 added parallax_decode_no_alloc, 5 the prefill's
                                  workgroups field */

typedef enum {
    PARALLAX_OK = 0,
    PARALLAX_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent shapes */
    PARALLAX_ERR_UNSUPPORTED = 2, /* valid but not implemented (head dim, dtype, alignment) */
    PARALLAX_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    PARALLAX_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} parallax_status_t;

typedef enum { PARALLAX_F32 = 0, PARALLAX_BF16 = 1 } parallax_dtype_t;

/* ------------------------------------------------------------- decode --- */
/*
 * Decode: one query row per (batch b, query head h), attending to every
 * cached token 0 .. L_b-1 of its KV head (the cache already holds the
 * current token).  L_b = seq_lens[b] if seq_lens is given, else max_seq_len.
 * A row with L_b = 0 yields o = 0.
 *
 * Local window (window >= 1): the row attends to its last `window` cached
 * tokens only, max(0, L_b - window) .. L_b-1 -- the local window that the
 * same page leaves open (section 3.1); window = 0 is full attention.  Tokens
 * before the window are never read, nor is any address formed from the page
 * id of a page that holds only such tokens (its block-table entry may be
 * read), so they may hold anything.
 *
 * Cache layouts (`kv_dtype` elements; k and v each have their own strides):
 *   contiguous (block_table == NULL): token j of (b, hk) at
 *       k + b*k_stride_0 + hk*k_stride_h + j*k_stride_t
 *     with L_b <= max_seq_len <= the cache capacity (not checked on device).
 *   paged (block_table != NULL): token j lives in physical page
 *       pg = block_table[b*max_blocks_per_seq + j/block_size], slot j%block_size:
 *       k + pg*k_stride_0 + hk*k_stride_h + slot*k_stride_t
 *     block_size must be 16.  seq_lens is required; the caller guarantees
 *     0 <= seq_lens[b] <= max_blocks_per_seq*16 and valid page ids.  Entries
 *     of block_table past a sequence's last block are never read, nor are
 *     slots past its last token.
 *
 * Inputs: q, rho fp32 [B, Hq, d] (strides q_stride_b, q_stride_h ...);
 * output out fp32 [B, Hq, d].  Arithmetic: fp32 accumulation.  With a bf16
 * cache the products run on bf16 matrix cores: q, rho and the softmax
 * weights enter as two-term (hi + lo) bf16 splits (about 16 significant
 * bits).  With an fp32 cache everything runs in fp32 on the vector ALUs.
 */
typedef struct {
    uint32_t struct_size; /* = sizeof(parallax_decode_args_t) */
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    float scale; /* logit scale, any finite value (usually 1/sqrt(head_dim)) */

    const float *q;
    int64_t q_stride_b, q_stride_h;
    const float *rho;
    int64_t rho_stride_b, rho_stride_h;
    float *out;
    int64_t out_stride_b, out_stride_h;

    int32_t kv_dtype; /* parallax_dtype_t */
    const void *k;
    int64_t k_stride_0, k_stride_h, k_stride_t;
    const void *v;
    int64_t v_stride_0, v_stride_h, v_stride_t;

    const int32_t *seq_lens; /* [B] device, or NULL */
    int32_t max_seq_len;     /* >= every seq_lens[b]; >= 1 */

    const int32_t *block_table; /* [B, max_blocks_per_seq] device, or NULL */
    int32_t block_size;
    int32_t max_blocks_per_seq;

    int32_t split_tokens; /* tokens per context split; 0 = chosen by the library,
                             else a positive multiple of 256 */
    int32_t window;       /* 0 = every cached token; W >= 1 = each row's last W tokens;
                             < 0 is PARALLAX_ERR_INVALID_ARG (added in ABI version 2) */
} parallax_decode_args_t;

/*
 * Bytes of device workspace parallax_decode needs for these arguments
 * (written to *bytes; 0 when one split covers every sequence).  The
 * workspace holds one partial record (running max, Z, R, A, B) per split
 * and query head, then one 8-byte arrival flag per split: the split that
 * finds every flag of its sequence set merges the records, in the same
 * launch.  A flag is set to a 64-bit tag drawn fresh for every call, and
 * the merging split clears them to 0; any other content counts as not
 * arrived unless it equals this call's tag (a 2^-64 chance per flag), so the
 * workspace's contents before the call do not matter.  Two calls that can
 * run concurrently need separate workspaces.  16-byte alignment is required.
 */
parallax_status_t parallax_decode_workspace_size(const parallax_decode_args_t *args,
                                                 size_t *bytes);

/* Enqueue a decode.  workspace may be NULL only if the required size is 0. */
parallax_status_t parallax_decode(const parallax_decode_args_t *args, void *workspace,
                                  size_t workspace_bytes, void *hip_stream);

/*
 * parallax_decode without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation): the split partials go to a scratch array that the
 * library owns on each device, PARALLAX_NO_ALLOC_SCRATCH_BYTES bytes, held
 * from the library's first use on that device until the process ends.  The
 * caller still provides every input and the output.  No call here allocates
 * or frees memory; the first call on a device looks up the array's address
 * there (a device's code is loaded by its first launch, as for any entry
 * point).
 *   - Same arguments, kernels and results as parallax_decode while the
 *     partials of the library's split choice fit the scratch (bit for bit).
 *     Beyond that, with split_tokens = 0 the call takes fewer, longer splits
 *     (down to one, which needs no partials), so results then differ from
 *     parallax_decode's by fp32 rounding only; with an explicit split_tokens
 *     whose partials exceed the scratch it returns PARALLAX_ERR_WORKSPACE.
 *   - Every call on a device shares that device's scratch, and nothing in it
 *     has to be cleared between calls: two calls that can overlap on one
 *     device (different streams, concurrently replayed graphs) race and may
 *     return wrong results.  Serialise them, or use parallax_decode with
 *     separate workspaces.
 */
#define PARALLAX_NO_ALLOC_SCRATCH_BYTES (64u << 20)
parallax_status_t parallax_decode_no_alloc(const parallax_decode_args_t *args, void *hip_stream);

/* --------------------------------------------- LLA solved-probe decode --- */
/*
 * Decode with local linear attention's solved probe instead of a given rho
 * (page "Parallax: Parameterized Local Linear Attention Gives Transformers a
 * 'Second Eye'": section 1.2 -- each token solves a regularised system
 * S x = mu by conjugate gradients, every iteration one sweep over the KV
 * cache; section 1.3 -- rho* = S^{-1} mu is the optimal probe, and Parallax
 * with that probe is LLA).  For each decode row, with p the softmax weights
 * over its keys (window included):
 *     rho* = (S_KK + lambda I)^{-1} (kbar - q),
 *     S_KK = sum_j p_j (k_j - kbar)(k_j - kbar)^T,  kbar = sum_j p_j k_j,
 * approximated by `iterations` conjugate-gradient steps from x = 0; then
 * out = o_SA - S_KV rho* exactly as parallax_decode computes it.  (mu =
 * kbar - q makes out the intercept of the softmax-weighted local linear fit
 * v ~ b + W (k - q) with penalty lambda |W|^2.)
 * The CG matrix-vector product is the decode pass with the keys as values:
 * S_KK y = kbar - o(V = K, rho = y); one call runs iterations + 2 decode
 * passes and no host synchronisation.  A row without keys gets rho* = 0.
 * `decode` is used as for parallax_decode except that decode->rho is ignored
 * (may be NULL).  rho_out fp32 [B, Hq, d] contiguous, may be NULL; resid fp32
 * [B, Hq], may be NULL: |mu - (S_KK + lambda I) x| / |mu| after the last step,
 * as the recurrence carries it.  lambda must be finite and > 0; iterations in
 * [1, 4096] (else PARALLAX_ERR_INVALID_ARG).  Workspace:
 * parallax_decode_lla_workspace_size bytes, 16-byte aligned.
 */
typedef struct {
    uint32_t struct_size; /* = sizeof(parallax_lla_args_t) */
    float lambda;
    int32_t iterations;
    float *rho_out;
    float *resid;
} parallax_lla_args_t;

parallax_status_t parallax_decode_lla_workspace_size(const parallax_decode_args_t *decode,
                                                     const parallax_lla_args_t *lla,
                                                     size_t *bytes);
parallax_status_t parallax_decode_lla(const parallax_decode_args_t *decode,
                                      const parallax_lla_args_t *lla, void *workspace,
                                      size_t workspace_bytes, void *hip_stream);

/* ------------------------------------------------- probe projection --- */
/*
 * The query and probe projections of T token rows in one launch:
 *     q[t] = W_Q x[t],   rho[t] = W_R x[t]
 * (page "Parallax: Parameterized Local Linear Attention Gives Transformers a
 * 'Second Eye'", section 1.3: the probe is a learned linear projection of the
 * layer input; W_R = 0 gives plain softmax attention).  x bf16 [T, D];
 * w_q, w_r bf16 [Hq * head_dim, D] (row n = head n / head_dim, element
 * n % head_dim) with row stride w_stride_n; q and rho [T, Hq, head_dim] of
 * out_dtype (PARALLAX_F32 for parallax_decode, PARALLAX_BF16 for
 * parallax_prefill; a [B, S] token grid is T = B * S rows when its token
 * stride is uniform).  bf16 matrix cores, fp32 accumulation, one rounding
 * to out_dtype.  D must be a multiple of 256, head_dim 64 or 128, T in
 * [1, 4194304]; pointers 16-byte aligned, strides multiples of 16 bytes
 * (else PARALLAX_ERR_UNSUPPORTED / INVALID_ARG).
 */
typedef struct {
    uint32_t struct_size; /* = sizeof(parallax_qr_projection_args_t) */
    int32_t tokens;
    int32_t model_dim;
    int32_t num_q_heads;
    int32_t head_dim;
    parallax_dtype_t out_dtype;
    const void *x;
    int64_t x_stride_t;
    const void *w_q;
    const void *w_r;
    int64_t w_stride_n;
    void *q;
    int64_t q_stride_t, q_stride_h;
    void *rho;
    int64_t rho_stride_t, rho_stride_h;
} parallax_qr_projection_args_t;

parallax_status_t parallax_qr_projection(const parallax_qr_projection_args_t *args,
                                         void *hip_stream);

/* ------------------------------------------------------------ prefill --- */
/*
 * Causal prefill: row i of (b, h) attends to keys 0..i of KV head
 * h / (Hq/Hkv) -- with a local window W >= 1 (see decode) to keys
 * max(0, i-W+1) .. i only.  q, rho bf16 [B, S, Hq, d]; k, v bf16 [B, S, Hkv, d];
 * out fp32 [B, S, Hq, d].  causal must be 1; head_dim must be 64 or 128; the GQA
 * group Hq/Hkv must be 1, 2, 4, 8 or 16 (else PARALLAX_ERR_UNSUPPORTED).  Products
 * run on the bf16 matrix cores with fp32 accumulation; the softmax
 * numerators e^{s} and e^{s} t are rounded to bf16 before they multiply V.
 */
typedef struct {
    uint32_t struct_size; /* = sizeof(parallax_prefill_args_t) */
    int32_t batch;
    int32_t seq_len;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    float scale; /* logit scale, any finite value (usually 1/sqrt(head_dim); 0 gives
                    uniform weights over a row's keys); else PARALLAX_ERR_INVALID_ARG */
    int32_t causal;

    const void *q;
    int64_t q_stride_b, q_stride_s, q_stride_h;
    const void *rho;
    int64_t rho_stride_b, rho_stride_s, rho_stride_h;
    const void *k;
    int64_t k_stride_b, k_stride_s, k_stride_h;
    const void *v;
    int64_t v_stride_b, v_stride_s, v_stride_h;
    float *out;
    int64_t out_stride_b, out_stride_s, out_stride_h;
    int32_t window; /* 0 = keys 0..i; W >= 1 = keys max(0, i-W+1)..i; < 0 is
                       PARALLAX_ERR_INVALID_ARG (added in ABI version 2) */

    /* Optional outputs for a backward pass (added in ABI version 3); each may
     * be NULL, and is written when not.  With p_ij the softmax weights of
     * row i:
     *   lse   fp32 [B, Hq, S], contiguous: log of sum_j exp(scale q_i.k_j)
     *         over the row's keys (natural log);
     *   rmean fp32 [B, Hq, S], contiguous: r_i = sum_j p_ij (rho_i . k_j);
     *   o_sa  fp32, the shape and strides of out: the softmax output
     *         a_i = sum_j p_ij v_j.
     * 16-byte aligned. */
    float *lse;
    float *rmean;
    float *o_sa;
    /* Head dim 128 runs a fixed set of persistent workgroups, each taking its
     * share of the (query block, head block) items in turn, and the shortest
     * items (about one round of them) as one workgroup each: 0 = one
     * persistent workgroup per compute unit (the default), n >= 1 = at most
     * n (for tests and tuning; results do not depend on it).  Head dim 64
     * runs one workgroup per item and ignores it.  < 0 is
     * PARALLAX_ERR_INVALID_ARG (added in ABI version 5). */
    int32_t workgroups;
} parallax_prefill_args_t;

parallax_status_t parallax_prefill(const parallax_prefill_args_t *args, void *hip_stream);

/* ---------------------------------------------------- prefill backward --- */
/*
 * Gradients of a causal prefill (same keys per row as parallax_prefill,
 * window included) for the loss sum(dout * out): dq, drho [B, S, Hq, d] and
 * dk, dv [B, S, Hkv, d], fp32, OVERWRITTEN (not accumulated).  Training the
 * layer end to end is how the page "Parallax: Parameterized Local Linear
 * Attention Gives Transformers a 'Second Eye'" (section 2.2) uses it; the
 * derivation follows the forward formula above by the chain rule:
 * with g = dout_i, c = a_i . g, u_j = g . v_j and D = g . o_i + r_i c,
 *     dv_j += p_ij (1 + r_i - t_ij) g
 *     ds_ij = p_ij (u_j (1 + r_i - t_ij) + c t_ij - D),  dt_ij = p_ij (c - u_j)
 *     dq_i  = scale sum_j ds_ij k_j,   drho_i = sum_j dt_ij k_j,
 *     dk_j += scale ds_ij q_i + dt_ij rho_i   (summed over rows and the GQA group)
 * Inputs: q, rho, k, v as the forward (bf16); dout bf16 [B, S, Hq, d]; out,
 * o_sa fp32 (the forward's output and its o_sa, sharing out's strides); lse
 * and rmean fp32 [B, Hq, S] contiguous (the forward's optional outputs).  The
 * products run on the bf16 matrix cores with fp32 accumulation; the weights
 * (1 + r - t) p, ds and dt are rounded to bf16 before they meet dout, q, rho
 * and k.  Deterministic: no atomics, fixed summation order.
 * Supported: causal = 1, head_dim 64 or 128, GQA group 1, 2, 4, 8 or 16 (else
 * PARALLAX_ERR_UNSUPPORTED).  Workspace: parallax_prefill_backward_workspace_size
 * bytes (16 per query row), 16-byte aligned, owned by the caller; its
 * contents on entry do not matter.
 */
typedef struct {
    uint32_t struct_size; /* = sizeof(parallax_prefill_backward_args_t) */
    int32_t batch;
    int32_t seq_len;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    float scale; /* as the forward's: any finite value */
    int32_t causal;
    int32_t window; /* as parallax_prefill_args_t */

    const void *q;
    int64_t q_stride_b, q_stride_s, q_stride_h;
    const void *rho;
    int64_t rho_stride_b, rho_stride_s, rho_stride_h;
    const void *k;
    int64_t k_stride_b, k_stride_s, k_stride_h;
    const void *v;
    int64_t v_stride_b, v_stride_s, v_stride_h;
    const void *dout;
    int64_t dout_stride_b, dout_stride_s, dout_stride_h;
    const float *out;  /* forward output */
    const float *o_sa; /* forward o_sa, out's strides */
    int64_t out_stride_b, out_stride_s, out_stride_h;
    const float *lse;   /* [B, Hq, S] */
    const float *rmean; /* [B, Hq, S] */
    float *dq;
    float *drho; /* dq's strides */
    int64_t dq_stride_b, dq_stride_s, dq_stride_h;
    float *dk;
    float *dv; /* dk's strides */
    int64_t dk_stride_b, dk_stride_s, dk_stride_h;
} parallax_prefill_backward_args_t;

parallax_status_t parallax_prefill_backward_workspace_size(
    const parallax_prefill_backward_args_t *args, size_t *bytes);
parallax_status_t parallax_prefill_backward(const parallax_prefill_backward_args_t *args,
                                            void *workspace, size_t workspace_bytes,
                                            void *hip_stream);

/* ------------------------------------------------------------- misc --- */
const char *parallax_status_string(parallax_status_t status);
const char *parallax_last_error(void); /* detail of this thread's last non-OK status */
int parallax_abi_version(void);        /* PARALLAX_ABI_VERSION */

#ifdef __cplusplus
}
#endif

#endif /* PARALLAX_H */
