// Internal launch parameters shared by the host dispatcher (api.hip) and the
// gfx950 kernels (decode.hip, prefill.hip, prefill_bwd.hip, lla.hip, proj.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace plx {

// Number of floats in one split's partial record for one query head:
// A[d], B[d], m, Z, R and one pad word (keeps records 16-byte aligned).
__host__ __device__ constexpr int partial_floats(int d) { return 2 * d + 4; }

// Page size of the paged cache (tokens per block-table entry); also the
// step of the fp32 decode loop, so one of its steps reads exactly one page.
constexpr int kDecodeStepTokens = 16;

struct DecodeParams {
    const float *q;
    const float *rho;
    float *out;
    int64_t q_sb, q_sh, rho_sb, rho_sh, out_sb, out_sh;
    const void *k;
    const void *v;
    int64_t k_s0, k_sh, k_st;
    int64_t v_s0, v_sh, v_st;
    const int32_t *seq_lens;  // may be null: every row has max_seq_len tokens
    const int32_t *block_table;
    int32_t max_seq_len;
    int32_t max_blocks;
    int32_t num_kv_heads;
    int32_t split;      // tokens per split (a multiple of 256)
    int32_t nsplit;     // splits per (batch, kv head) in the grid
    float scale_log2;   // logit scale times log2(e): logits are kept in base 2
    float *partials;    // [B*Hkv*nsplit][G][partial_floats(d)] or null when nsplit == 1
    int32_t window;     // 0: every cached token; W >= 1: each row's last W tokens
    // Split merge inside the split kernel: when non-null, one 64-bit arrival
    // flag per split of every (batch, KV head) unit, [units][nsplit], right
    // after the partials.  A split sets its flag to `epoch` once its records
    // are complete; a split that then finds every flag of its row set merges
    // the row and clears the flags.  Null: the partials are left for
    // decode_merge_kernel.
    unsigned long long *arrivals;
    unsigned long long epoch;  // this call's tag, never 0
};

// Arrival flags after the partials, 8-byte aligned (records are 16).
__host__ __device__ constexpr int64_t arrival_bytes(int64_t units, int nsplit) {
    return units * nsplit * 8;
}

struct PrefillParams {
    const uint16_t *q;
    const uint16_t *rho;
    const uint16_t *k;
    const uint16_t *v;
    float *out;
    int64_t q_sb, q_ss, q_sh;
    int64_t r_sb, r_ss, r_sh;
    int64_t k_sb, k_ss, k_sh;
    int64_t v_sb, v_ss, v_sh;
    int64_t o_sb, o_ss, o_sh;
    int32_t batch, seq_len, num_q_heads, num_kv_heads;
    // workgroup head blocks per KV head, set by the launcher: a workgroup
    // serves the kernel's G query heads hb*G .. hb*G + G - 1 of KV head
    // hb / head_blocks (1 unless a GQA group is split over workgroups)
    int32_t head_blocks;
    // |scale| * log2(e) (1 for scale 0): positive, so the row max of the raw
    // scores is the row max of the logits
    float scale_log2;
    // how the query operand enters the score products so that the logits
    // stay scale * q.k with the positive factor above: 0 as it is (scale > 0),
    // 1 negated (scale < 0), 2 zeroed (scale = 0: every logit 0)
    int32_t q_sign;
    int32_t window;  // 0: keys 0..i; W >= 1: keys max(0, i-W+1)..i
    // head dim 128: at most this many persistent workgroups, each running
    // its share of the query blocks in turn (0: one per compute unit)
    int32_t workgroups;
    // set by the launcher: workgroups 0 .. persist - 1 each run
    // static_rounds items; the items after those rounds run one per
    // workgroup (0, 0: every workgroup runs one item)
    int32_t persist;
    int32_t static_rounds;
    // optional outputs for a backward pass (each may be null): natural-log
    // softmax denominator and r per row, [B, Hq, S]; o_SA with out's strides
    float *lse;
    float *rmean;
    float *o_sa;
};

// Causal prefill backward.  rowstat is the workspace: one float4 per row
// (b, h, i) at ((b * Hq + h) * S + i), holding (lse * log2 e, 1 + r, c, D)
// with c = o_SA . dout and D = dout . out + r c.
struct PrefillBwdParams {
    const uint16_t *q;
    const uint16_t *rho;
    const uint16_t *k;
    const uint16_t *v;
    const uint16_t *dout;
    const float *out;
    const float *o_sa;
    const float *lse;
    const float *rmean;
    float *dq;
    float *drho;
    float *dk;
    float *dv;
    float4 *rowstat;
    int64_t q_sb, q_ss, q_sh;
    int64_t r_sb, r_ss, r_sh;
    int64_t k_sb, k_ss, k_sh;
    int64_t v_sb, v_ss, v_sh;
    int64_t g_sb, g_ss, g_sh;    // dout
    int64_t o_sb, o_ss, o_sh;    // out and o_sa
    int64_t dq_sb, dq_ss, dq_sh; // dq and drho
    int64_t dk_sb, dk_ss, dk_sh; // dk and dv
    int32_t batch, seq_len, num_q_heads, num_kv_heads;
    int32_t head_blocks;  // as in PrefillParams (query-side dq kernel only)
    float scale;       // natural logit scale
    float scale_log2;  // scale * log2(e)
    int32_t window;
};

// Conjugate-gradient state of local linear attention's solved probe, one
// row per (batch, query head), vectors contiguous [B * Hq][d].
struct LlaParams {
    const float *q;
    int64_t q_sb, q_sh;
    const float *kbar;  // o(V = K, rho = 0)
    const float *ok;    // o(V = K, rho = dir) of the current sweep
    float *x, *r, *dir;
    float *rs;          // [B * Hq][2]: |r|^2 and |mu|^2
    const int32_t *seq_lens;  // may be null: every row has max_seq_len tokens
    int32_t max_seq_len;
    float *rho_out;     // may be null
    float *resid;       // may be null
    int32_t batch, num_q_heads, d;
    float lambda;
};

// q = W_Q x and rho = W_R x for T token rows (x [T, D], weights [N, D],
// outputs [T, Hq, d] with N = Hq * d).
struct ProjParams {
    const uint16_t *x;
    int64_t x_st;
    const uint16_t *w_q;
    const uint16_t *w_r;
    int64_t w_sn;
    void *q;
    void *rho;
    int64_t q_st, q_sh, r_st, r_sh;
    int32_t tokens, model_dim, n, head_dim;
    int32_t out_bf16;
};

// Launchers (defined next to their kernels).  They return the HIP status of
// the launch.
// lla: the decode is a sweep of the solved probe's conjugate gradients
// (keys as values, rho = the search direction); the merge kernel then also
// runs one step on every row (and runs even when no row has two splits).
hipError_t launch_decode(const DecodeParams &p, int kv_dtype, int d, int group, bool paged,
                         int batch, hipStream_t stream, const LlaParams *lla = nullptr);
hipError_t launch_prefill(const PrefillParams &p, int d, hipStream_t stream);
hipError_t launch_prefill_backward(const PrefillBwdParams &p, int d, hipStream_t stream);
hipError_t launch_lla_zero(float *a, int64_t n, hipStream_t stream);
hipError_t launch_lla_init(const LlaParams &p, hipStream_t stream);
hipError_t launch_lla_finish(const LlaParams &p, hipStream_t stream);
hipError_t launch_qr_projection(const ProjParams &p, hipStream_t stream);

}  // namespace plx
