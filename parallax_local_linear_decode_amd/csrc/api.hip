// api.hip -- the C ABI of libparallax (declared in include/parallax.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, so argument errors are reported (and testable) on machines
// without a GPU.  Nothing runs at load time.
#include "parallax.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <time.h>
#include <unistd.h>

#include <atomic>
#include <mutex>

#include "kernels.hpp"

#define PLX_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";

parallax_status_t fail(parallax_status_t s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool bytes16(int64_t stride_elems, int64_t elem_size) {
    return ((stride_elems * elem_size) & 15) == 0;
}

// Splits are whole numbers of 256 tokens: 8 waves x 32-token steps of the
// bf16 kernel (and 4 x 16-token steps x 4 of the fp32 kernel).
constexpr int kSplitQuantum = 256;
// About one 8-wave workgroup per CU of a 256-CU MI355X: more, shorter splits
// lose more to per-workgroup setup and to the merge than they gain.
constexpr int64_t kTargetWorkgroups = 256;
// Longest split: bounds the tail left by the longest rows of a ragged batch.
constexpr int kMaxSplit = 4096;

struct DecodePlan {
    int group;
    bool paged;
    int split;
    int nsplit;
    size_t workspace_bytes;
};

int64_t round_up(int64_t x, int64_t q) { return ((x + q - 1) / q) * q; }

// Workspace of a decode plan: the split records, then one arrival word per
// (batch, KV head) unit for the in-kernel merge; nothing for a single split.
size_t decode_ws_bytes(int64_t units, int group, int d, int nsplit) {
    if (nsplit <= 1) return 0;
    return (size_t)(units * nsplit * group * plx::partial_floats(d) * 4) +
           (size_t)plx::arrival_bytes(units, nsplit);
}

// A fresh tag per decode launch, telling this call's arrival flags from
// whatever a workspace held before: a process-wide count, mixed with the
// process id and start time so that the tags of different processes (and
// bytes a workspace happened to hold) match only by chance, 1 in 2^64.
std::atomic<unsigned long long> g_epoch{0};
unsigned long long next_epoch() {
    static const unsigned long long salt = [] {
        unsigned long long x = (unsigned long long)getpid() * 0x9E3779B97F4A7C15ull;
        x ^= (unsigned long long)time(nullptr) * 0xC2B2AE3D27D4EB4Full;
        return x;
    }();
    for (;;) {
        // splitmix64 of (salt + count): distinct counts give distinct tags
        unsigned long long z = salt + 0x9E3779B97F4A7C15ull * (g_epoch.fetch_add(1) + 1);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        z ^= z >> 31;
        if (z != 0) return z;
    }
}

int choose_split(int64_t units, int max_len) {
    int64_t split = round_up((max_len * units + kTargetWorkgroups - 1) / kTargetWorkgroups,
                             kSplitQuantum);
    if (split > kMaxSplit) split = kMaxSplit;
    if (split > round_up(max_len, kSplitQuantum)) split = round_up(max_len, kSplitQuantum);
    if (split < kSplitQuantum) split = kSplitQuantum;
    return (int)split;
}

parallax_status_t plan_decode(const parallax_decode_args_t *a, DecodePlan *pl) {
    if (a == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "decode: args is NULL");
    if (a->struct_size != sizeof(parallax_decode_args_t))
        return fail(PARALLAX_ERR_INVALID_ARG, "decode: struct_size %u, expected %zu",
                    a->struct_size, sizeof(parallax_decode_args_t));
    if (a->batch < 1 || a->num_q_heads < 1 || a->num_kv_heads < 1)
        return fail(PARALLAX_ERR_INVALID_ARG, "decode: batch and head counts must be >= 1");
    if (a->num_q_heads % a->num_kv_heads != 0)
        return fail(PARALLAX_ERR_INVALID_ARG, "decode: num_q_heads %% num_kv_heads != 0");
    const int group = a->num_q_heads / a->num_kv_heads;
    if (a->head_dim < 1) return fail(PARALLAX_ERR_INVALID_ARG, "decode: head_dim must be >= 1");
    if (a->kv_dtype != PARALLAX_F32 && a->kv_dtype != PARALLAX_BF16)
        return fail(PARALLAX_ERR_INVALID_ARG, "decode: unknown kv_dtype %d", a->kv_dtype);
    if (!isfinite(a->scale)) return fail(PARALLAX_ERR_INVALID_ARG, "decode: scale is not finite");
    if (!a->q || !a->rho || !a->out || !a->k || !a->v)
        return fail(PARALLAX_ERR_INVALID_ARG, "decode: q, rho, out, k and v must be non-NULL");
    if (a->max_seq_len < 1) return fail(PARALLAX_ERR_INVALID_ARG, "decode: max_seq_len must be >= 1");
    if (a->q_stride_b < 0 || a->q_stride_h < 0 || a->rho_stride_b < 0 || a->rho_stride_h < 0 ||
        a->out_stride_b < 0 || a->out_stride_h < 0 || a->k_stride_0 < 0 || a->k_stride_h < 0 ||
        a->k_stride_t < 0 || a->v_stride_0 < 0 || a->v_stride_h < 0 || a->v_stride_t < 0)
        return fail(PARALLAX_ERR_INVALID_ARG, "decode: strides must be non-negative");
    if (a->split_tokens < 0 || (a->split_tokens > 0 && a->split_tokens % kSplitQuantum != 0))
        return fail(PARALLAX_ERR_INVALID_ARG, "decode: split_tokens must be 0 or a multiple of %d",
                    kSplitQuantum);
    if (a->window < 0) return fail(PARALLAX_ERR_INVALID_ARG, "decode: window must be >= 0");
    const bool paged = a->block_table != nullptr;
    if (paged) {
        if (a->seq_lens == nullptr)
            return fail(PARALLAX_ERR_INVALID_ARG, "decode: a paged cache needs seq_lens");
        if (a->max_blocks_per_seq < 1)
            return fail(PARALLAX_ERR_INVALID_ARG, "decode: max_blocks_per_seq must be >= 1");
        if (a->block_size != plx::kDecodeStepTokens)
            return fail(PARALLAX_ERR_UNSUPPORTED, "decode: block_size %d (only 16 is supported)",
                        a->block_size);
        if ((int64_t)a->max_seq_len > (int64_t)a->max_blocks_per_seq * a->block_size)
            return fail(PARALLAX_ERR_INVALID_ARG,
                        "decode: max_seq_len exceeds max_blocks_per_seq * block_size");
    }
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(PARALLAX_ERR_UNSUPPORTED, "decode: head_dim %d (supported: 64, 128)",
                    a->head_dim);
    if (group != 1 && group != 2 && group != 4 && group != 8)
        return fail(PARALLAX_ERR_UNSUPPORTED, "decode: GQA group %d (supported: 1, 2, 4, 8)",
                    group);
    const int64_t kv_es = a->kv_dtype == PARALLAX_BF16 ? 2 : 4;
    if (!aligned16(a->q) || !aligned16(a->rho) || !aligned16(a->out) || !aligned16(a->k) ||
        !aligned16(a->v))
        return fail(PARALLAX_ERR_UNSUPPORTED, "decode: every pointer must be 16-byte aligned");
    if (!bytes16(a->q_stride_b, 4) || !bytes16(a->q_stride_h, 4) || !bytes16(a->rho_stride_b, 4) ||
        !bytes16(a->rho_stride_h, 4) || !bytes16(a->out_stride_b, 4) ||
        !bytes16(a->out_stride_h, 4) || !bytes16(a->k_stride_0, kv_es) ||
        !bytes16(a->k_stride_h, kv_es) || !bytes16(a->k_stride_t, kv_es) ||
        !bytes16(a->v_stride_0, kv_es) || !bytes16(a->v_stride_h, kv_es) ||
        !bytes16(a->v_stride_t, kv_es))
        return fail(PARALLAX_ERR_UNSUPPORTED, "decode: every stride must span a multiple of 16 bytes");

    const int64_t units = (int64_t)a->batch * a->num_kv_heads;
    // tokens a row's splits cover at most: every cached token, or the window
    // plus its start rounded down to a 32-token step
    const int span = a->window > 0 && a->window < a->max_seq_len - 31
                         ? a->window + 31
                         : a->max_seq_len;
    int split = a->split_tokens > 0 ? a->split_tokens : choose_split(units, span);
    int nsplit = (span + split - 1) / split;
    if (units * nsplit > 0x7fffffffLL)
        return fail(PARALLAX_ERR_UNSUPPORTED, "decode: grid too large (%lld workgroups)",
                    (long long)(units * nsplit));
    pl->group = group;
    pl->paged = paged;
    pl->split = split;
    pl->nsplit = nsplit;
    pl->workspace_bytes = decode_ws_bytes(units, group, a->head_dim, nsplit);
    return PARALLAX_OK;
}

parallax_status_t check_prefill(const parallax_prefill_args_t *a) {
    if (a == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "prefill: args is NULL");
    if (a->struct_size != sizeof(parallax_prefill_args_t))
        return fail(PARALLAX_ERR_INVALID_ARG, "prefill: struct_size %u, expected %zu",
                    a->struct_size, sizeof(parallax_prefill_args_t));
    if (a->batch < 1 || a->seq_len < 1 || a->num_q_heads < 1 || a->num_kv_heads < 1)
        return fail(PARALLAX_ERR_INVALID_ARG, "prefill: batch, seq_len and head counts must be >= 1");
    if (a->num_q_heads % a->num_kv_heads != 0)
        return fail(PARALLAX_ERR_INVALID_ARG, "prefill: num_q_heads %% num_kv_heads != 0");
    if (!isfinite(a->scale)) return fail(PARALLAX_ERR_INVALID_ARG, "prefill: scale is not finite");
    if (!a->q || !a->rho || !a->k || !a->v || !a->out)
        return fail(PARALLAX_ERR_INVALID_ARG, "prefill: q, rho, k, v and out must be non-NULL");
    const int64_t strides[] = {a->q_stride_b, a->q_stride_s, a->q_stride_h, a->rho_stride_b,
                               a->rho_stride_s, a->rho_stride_h, a->k_stride_b, a->k_stride_s,
                               a->k_stride_h, a->v_stride_b, a->v_stride_s, a->v_stride_h,
                               a->out_stride_b, a->out_stride_s, a->out_stride_h};
    for (int64_t s : strides)
        if (s < 0) return fail(PARALLAX_ERR_INVALID_ARG, "prefill: strides must be non-negative");
    if (a->causal != 1)
        return fail(PARALLAX_ERR_UNSUPPORTED, "prefill: only causal = 1 is supported");
    if (a->window < 0) return fail(PARALLAX_ERR_INVALID_ARG, "prefill: window must be >= 0");
    if (a->workgroups < 0)
        return fail(PARALLAX_ERR_INVALID_ARG, "prefill: workgroups must be >= 0");
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(PARALLAX_ERR_UNSUPPORTED, "prefill: head_dim %d (supported: 64, 128)",
                    a->head_dim);
    const int group = a->num_q_heads / a->num_kv_heads;
    if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16)
        return fail(PARALLAX_ERR_UNSUPPORTED, "prefill: GQA group %d (supported: 1, 2, 4, 8, 16)",
                    group);
    if ((int64_t)a->batch * a->num_q_heads * ((a->seq_len + 31) / 32) > 0x7fffffffLL)
        return fail(PARALLAX_ERR_UNSUPPORTED, "prefill: grid too large");
    if (!aligned16(a->q) || !aligned16(a->rho) || !aligned16(a->k) || !aligned16(a->v) ||
        !aligned16(a->out))
        return fail(PARALLAX_ERR_UNSUPPORTED, "prefill: every pointer must be 16-byte aligned");
    for (int i = 0; i < 12; ++i)
        if (!bytes16(strides[i], 2))
            return fail(PARALLAX_ERR_UNSUPPORTED, "prefill: strides must span multiples of 16 bytes");
    for (int i = 12; i < 15; ++i)
        if (!bytes16(strides[i], 4))
            return fail(PARALLAX_ERR_UNSUPPORTED, "prefill: strides must span multiples of 16 bytes");
    if (!aligned16(a->lse) || !aligned16(a->rmean) || !aligned16(a->o_sa))
        return fail(PARALLAX_ERR_UNSUPPORTED, "prefill: lse, rmean and o_sa must be 16-byte aligned");
    return PARALLAX_OK;
}

parallax_status_t check_prefill_backward(const parallax_prefill_backward_args_t *a) {
    if (a == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "prefill backward: args is NULL");
    if (a->struct_size != sizeof(parallax_prefill_backward_args_t))
        return fail(PARALLAX_ERR_INVALID_ARG, "prefill backward: struct_size %u, expected %zu",
                    a->struct_size, sizeof(parallax_prefill_backward_args_t));
    if (a->batch < 1 || a->seq_len < 1 || a->num_q_heads < 1 || a->num_kv_heads < 1)
        return fail(PARALLAX_ERR_INVALID_ARG,
                    "prefill backward: batch, seq_len and head counts must be >= 1");
    if (a->num_q_heads % a->num_kv_heads != 0)
        return fail(PARALLAX_ERR_INVALID_ARG, "prefill backward: num_q_heads %% num_kv_heads != 0");
    if (!isfinite(a->scale))
        return fail(PARALLAX_ERR_INVALID_ARG, "prefill backward: scale is not finite");
    if (!a->q || !a->rho || !a->k || !a->v || !a->dout || !a->out || !a->o_sa || !a->lse ||
        !a->rmean || !a->dq || !a->drho || !a->dk || !a->dv)
        return fail(PARALLAX_ERR_INVALID_ARG,
                    "prefill backward: every tensor pointer must be non-NULL");
    const int64_t strides[] = {a->q_stride_b,    a->q_stride_s,    a->q_stride_h,
                               a->rho_stride_b,  a->rho_stride_s,  a->rho_stride_h,
                               a->k_stride_b,    a->k_stride_s,    a->k_stride_h,
                               a->v_stride_b,    a->v_stride_s,    a->v_stride_h,
                               a->dout_stride_b, a->dout_stride_s, a->dout_stride_h,
                               a->out_stride_b,  a->out_stride_s,  a->out_stride_h,
                               a->dq_stride_b,   a->dq_stride_s,   a->dq_stride_h,
                               a->dk_stride_b,   a->dk_stride_s,   a->dk_stride_h};
    for (int64_t s : strides)
        if (s < 0)
            return fail(PARALLAX_ERR_INVALID_ARG, "prefill backward: strides must be non-negative");
    if (a->causal != 1)
        return fail(PARALLAX_ERR_UNSUPPORTED, "prefill backward: only causal = 1 is supported");
    if (a->window < 0)
        return fail(PARALLAX_ERR_INVALID_ARG, "prefill backward: window must be >= 0");
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(PARALLAX_ERR_UNSUPPORTED, "prefill backward: head_dim %d (supported: 64, 128)",
                    a->head_dim);
    const int group = a->num_q_heads / a->num_kv_heads;
    if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16)
        return fail(PARALLAX_ERR_UNSUPPORTED,
                    "prefill backward: GQA group %d (supported: 1, 2, 4, 8, 16)", group);
    if ((int64_t)a->batch * a->num_q_heads * ((a->seq_len + 31) / 32) > 0x7fffffffLL ||
        (int64_t)a->batch * a->num_q_heads * a->seq_len > 0x7fffffffLL * 16LL)
        return fail(PARALLAX_ERR_UNSUPPORTED, "prefill backward: grid too large");
    const void *ptrs[] = {a->q,   a->rho, a->k,     a->v,  a->dout, a->out, a->o_sa,
                          a->lse, a->rmean, a->dq, a->drho, a->dk, a->dv};
    for (const void *ptr : ptrs)
        if (!aligned16(ptr))
            return fail(PARALLAX_ERR_UNSUPPORTED,
                        "prefill backward: every pointer must be 16-byte aligned");
    for (int i = 0; i < 15; ++i)
        if (!bytes16(strides[i], 2))
            return fail(PARALLAX_ERR_UNSUPPORTED,
                        "prefill backward: strides must span multiples of 16 bytes");
    for (int i = 15; i < 24; ++i)
        if (!bytes16(strides[i], 4))
            return fail(PARALLAX_ERR_UNSUPPORTED,
                        "prefill backward: strides must span multiples of 16 bytes");
    return PARALLAX_OK;
}

size_t prefill_backward_workspace(const parallax_prefill_backward_args_t *a) {
    return (size_t)a->batch * a->num_q_heads * a->seq_len * 16;  // one float4 per query row
}

plx::DecodeParams decode_params(const parallax_decode_args_t *a, const DecodePlan &pl,
                                void *workspace) {
    plx::DecodeParams p;
    p.q = a->q;
    p.rho = a->rho;
    p.out = a->out;
    p.q_sb = a->q_stride_b;
    p.q_sh = a->q_stride_h;
    p.rho_sb = a->rho_stride_b;
    p.rho_sh = a->rho_stride_h;
    p.out_sb = a->out_stride_b;
    p.out_sh = a->out_stride_h;
    p.k = a->k;
    p.v = a->v;
    p.k_s0 = a->k_stride_0;
    p.k_sh = a->k_stride_h;
    p.k_st = a->k_stride_t;
    p.v_s0 = a->v_stride_0;
    p.v_sh = a->v_stride_h;
    p.v_st = a->v_stride_t;
    p.seq_lens = a->seq_lens;
    p.block_table = a->block_table;
    p.max_seq_len = a->max_seq_len;
    p.max_blocks = pl.paged ? a->max_blocks_per_seq : 0;
    p.num_kv_heads = a->num_kv_heads;
    p.split = pl.split;
    p.nsplit = pl.nsplit;
    p.scale_log2 = (float)((double)a->scale * 1.4426950408889634);
    p.partials = pl.workspace_bytes > 0 ? static_cast<float *>(workspace) : nullptr;
    p.window = a->window;
    // the split records are merged by the last arriving split of each row
    const int64_t units = (int64_t)a->batch * a->num_kv_heads;
    p.arrivals = pl.workspace_bytes > 0
                     ? reinterpret_cast<unsigned long long *>(
                           static_cast<unsigned char *>(workspace) + pl.workspace_bytes -
                           plx::arrival_bytes(units, pl.nsplit))
                     : nullptr;
    p.epoch = next_epoch();
    return p;
}

// Solved-probe decode: the decode plan of the user's arguments (rho is not
// read), then the conjugate-gradient vectors kbar, o_k, x, r, dir ([B*Hq][d]
// each) and [B*Hq][2] squared norms after the decode partials.
struct LlaPlan {
    DecodePlan dplan;
    size_t decode_bytes;
    size_t total_bytes;
};

constexpr int kLlaMaxIterations = 4096;

parallax_status_t plan_lla(const parallax_decode_args_t *dec, const parallax_lla_args_t *lla,
                           LlaPlan *lp) {
    if (dec == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "lla: decode args is NULL");
    if (lla == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "lla: lla args is NULL");
    if (lla->struct_size != sizeof(parallax_lla_args_t))
        return fail(PARALLAX_ERR_INVALID_ARG, "lla: struct_size %u, expected %zu", lla->struct_size,
                    sizeof(parallax_lla_args_t));
    if (!isfinite(lla->lambda) || !(lla->lambda > 0.0f))
        return fail(PARALLAX_ERR_INVALID_ARG, "lla: lambda must be finite and > 0");
    if (lla->iterations < 1 || lla->iterations > kLlaMaxIterations)
        return fail(PARALLAX_ERR_INVALID_ARG, "lla: iterations must be in [1, %d]",
                    kLlaMaxIterations);
    if (!aligned16(lla->rho_out))
        return fail(PARALLAX_ERR_UNSUPPORTED, "lla: rho_out must be 16-byte aligned");
    if (dec->struct_size != sizeof(parallax_decode_args_t))  // before reading the rest
        return fail(PARALLAX_ERR_INVALID_ARG, "decode: struct_size %u, expected %zu",
                    dec->struct_size, sizeof(parallax_decode_args_t));
    // rho is not read: validate the rest with q standing in for it
    parallax_decode_args_t probe = *dec;
    probe.rho = dec->q;
    probe.rho_stride_b = dec->q_stride_b;
    probe.rho_stride_h = dec->q_stride_h;
    parallax_status_t s = plan_decode(&probe, &lp->dplan);
    if (s != PARALLAX_OK) return s;
    const size_t n = (size_t)dec->batch * dec->num_q_heads * dec->head_dim;
    lp->decode_bytes = (size_t)round_up((int64_t)lp->dplan.workspace_bytes, 256);
    lp->total_bytes = lp->decode_bytes + (5 * n + 2 * (size_t)dec->batch * dec->num_q_heads) * 4;
    return PARALLAX_OK;
}

constexpr int64_t kProjMaxTokens = 4194304;  // grid.y limit at 64 tokens per workgroup

parallax_status_t check_projection(const parallax_qr_projection_args_t *a) {
    if (a == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "projection: args is NULL");
    if (a->struct_size != sizeof(parallax_qr_projection_args_t))
        return fail(PARALLAX_ERR_INVALID_ARG, "projection: struct_size %u, expected %zu",
                    a->struct_size, sizeof(parallax_qr_projection_args_t));
    if (a->tokens < 1 || a->model_dim < 1 || a->num_q_heads < 1 || a->head_dim < 1)
        return fail(PARALLAX_ERR_INVALID_ARG,
                    "projection: tokens, model_dim, num_q_heads and head_dim must be >= 1");
    if (a->out_dtype != PARALLAX_F32 && a->out_dtype != PARALLAX_BF16)
        return fail(PARALLAX_ERR_INVALID_ARG, "projection: unknown out_dtype %d", a->out_dtype);
    if (!a->x || !a->w_q || !a->w_r || !a->q || !a->rho)
        return fail(PARALLAX_ERR_INVALID_ARG, "projection: x, w_q, w_r, q and rho must be non-NULL");
    if (a->x_stride_t < 0 || a->w_stride_n < 0 || a->q_stride_t < 0 || a->q_stride_h < 0 ||
        a->rho_stride_t < 0 || a->rho_stride_h < 0)
        return fail(PARALLAX_ERR_INVALID_ARG, "projection: strides must be non-negative");
    if (a->tokens > kProjMaxTokens)
        return fail(PARALLAX_ERR_UNSUPPORTED, "projection: tokens %d above %lld", a->tokens,
                    (long long)kProjMaxTokens);
    if (a->model_dim % 256 != 0)
        return fail(PARALLAX_ERR_UNSUPPORTED, "projection: model_dim %d is not a multiple of 256",
                    a->model_dim);
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(PARALLAX_ERR_UNSUPPORTED, "projection: head_dim %d (supported: 64, 128)",
                    a->head_dim);
    if ((int64_t)a->num_q_heads * a->head_dim * 2 / 16 > 0x7fffffffLL)
        return fail(PARALLAX_ERR_UNSUPPORTED, "projection: too many output features");
    const int64_t oes = a->out_dtype == PARALLAX_F32 ? 4 : 2;
    if (!aligned16(a->x) || !aligned16(a->w_q) || !aligned16(a->w_r) || !aligned16(a->q) ||
        !aligned16(a->rho))
        return fail(PARALLAX_ERR_UNSUPPORTED, "projection: every pointer must be 16-byte aligned");
    if (!bytes16(a->x_stride_t, 2) || !bytes16(a->w_stride_n, 2) || !bytes16(a->q_stride_t, oes) ||
        !bytes16(a->q_stride_h, oes) || !bytes16(a->rho_stride_t, oes) ||
        !bytes16(a->rho_stride_h, oes))
        return fail(PARALLAX_ERR_UNSUPPORTED,
                    "projection: every stride must span a multiple of 16 bytes");
    return PARALLAX_OK;
}

parallax_status_t hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return PARALLAX_OK;
    return fail(PARALLAX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- the no-allocation decode's scratch ----------------------------------
// Its split partials live in a library-owned device array instead of a
// caller workspace.  In host code `scratch` names a host-side shadow, not the
// device memory: the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is used.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

}  // namespace

static __device__ __align__(256) unsigned char scratch[PARALLAX_NO_ALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the device `stream` belongs to (the current
// device for the null stream).
parallax_status_t scratch_address(hipStream_t stream, void **out) {
    int dev = -1;
    hipError_t e = stream == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_status(e, "decode (no alloc): device of the stream");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PARALLAX_ERR_UNSUPPORTED, "decode (no alloc): device %d beyond %d", dev,
                    kMaxDevices);
    void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr != nullptr) {
        *out = ptr;
        return PARALLAX_OK;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur >= 0 && cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return hip_status(e, "decode (no alloc): scratch address");
        if (ptr == nullptr)
            return fail(PARALLAX_ERR_HIP, "decode (no alloc): scratch address is NULL");
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    *out = ptr;
    return PARALLAX_OK;
}

// The decode plan, with the split raised (fewer splits, smaller partials)
// when the library's choice needs more than the scratch holds.
parallax_status_t plan_decode_no_alloc(const parallax_decode_args_t *a, DecodePlan *pl) {
    parallax_status_t s = plan_decode(a, pl);
    if (s != PARALLAX_OK || pl->workspace_bytes <= PARALLAX_NO_ALLOC_SCRATCH_BYTES) return s;
    if (a->split_tokens > 0)
        return fail(PARALLAX_ERR_WORKSPACE,
                    "decode (no alloc): split_tokens %d needs %zu bytes of partials, above the "
                    "%zu-byte scratch",
                    a->split_tokens, pl->workspace_bytes, (size_t)PARALLAX_NO_ALLOC_SCRATCH_BYTES);
    const int64_t units = (int64_t)a->batch * a->num_kv_heads;
    const int64_t per_split = units * pl->group * plx::partial_floats(a->head_dim) * 4;
    const int64_t fit = (int64_t)PARALLAX_NO_ALLOC_SCRATCH_BYTES /
                        (per_split + plx::arrival_bytes(units, 1));  // splits that fit
    const int span = a->window > 0 && a->window < a->max_seq_len - 31 ? a->window + 31
                                                                      : a->max_seq_len;
    int split = (int)round_up(span, kSplitQuantum);  // one split: no partials at all
    if (fit >= 2) split = (int)round_up((span + fit - 1) / fit, kSplitQuantum);
    pl->split = split;
    pl->nsplit = (span + split - 1) / split;
    pl->workspace_bytes = decode_ws_bytes(units, pl->group, a->head_dim, pl->nsplit);
    return PARALLAX_OK;
}

}  // namespace

PLX_EXPORT int parallax_abi_version(void) { return PARALLAX_ABI_VERSION; }

PLX_EXPORT const char *parallax_status_string(parallax_status_t s) {
    switch (s) {
        case PARALLAX_OK: return "PARALLAX_OK";
        case PARALLAX_ERR_INVALID_ARG: return "PARALLAX_ERR_INVALID_ARG";
        case PARALLAX_ERR_UNSUPPORTED: return "PARALLAX_ERR_UNSUPPORTED";
        case PARALLAX_ERR_WORKSPACE: return "PARALLAX_ERR_WORKSPACE";
        case PARALLAX_ERR_HIP: return "PARALLAX_ERR_HIP";
    }
    return "PARALLAX_ERR_UNKNOWN";
}

PLX_EXPORT const char *parallax_last_error(void) { return g_last_error; }

PLX_EXPORT parallax_status_t parallax_decode_workspace_size(const parallax_decode_args_t *args,
                                                            size_t *bytes) {
    if (bytes == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "decode: bytes is NULL");
    DecodePlan pl;
    parallax_status_t s = plan_decode(args, &pl);
    if (s != PARALLAX_OK) return s;
    *bytes = pl.workspace_bytes;
    return PARALLAX_OK;
}

PLX_EXPORT parallax_status_t parallax_decode(const parallax_decode_args_t *a, void *workspace,
                                             size_t workspace_bytes, void *hip_stream) {
    DecodePlan pl;
    parallax_status_t s = plan_decode(a, &pl);
    if (s != PARALLAX_OK) return s;
    if (pl.workspace_bytes > 0) {
        if (workspace == nullptr || workspace_bytes < pl.workspace_bytes)
            return fail(PARALLAX_ERR_WORKSPACE, "decode: workspace of %zu bytes needed, %zu given",
                        pl.workspace_bytes, workspace == nullptr ? (size_t)0 : workspace_bytes);
        if (!aligned16(workspace))
            return fail(PARALLAX_ERR_WORKSPACE, "decode: workspace must be 16-byte aligned");
    }
    plx::DecodeParams p = decode_params(a, pl, workspace);
    return hip_status(plx::launch_decode(p, a->kv_dtype, a->head_dim, pl.group, pl.paged, a->batch,
                                         static_cast<hipStream_t>(hip_stream)),
                      "decode launch");
}

PLX_EXPORT parallax_status_t parallax_decode_no_alloc(const parallax_decode_args_t *a,
                                                      void *hip_stream) {
    DecodePlan pl;
    parallax_status_t s = plan_decode_no_alloc(a, &pl);
    if (s != PARALLAX_OK) return s;
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    void *ws = nullptr;
    if (pl.workspace_bytes > 0) {
        s = scratch_address(stream, &ws);
        if (s != PARALLAX_OK) return s;
    }
    plx::DecodeParams p = decode_params(a, pl, ws);
    return hip_status(plx::launch_decode(p, a->kv_dtype, a->head_dim, pl.group, pl.paged, a->batch,
                                         stream),
                      "decode launch");
}

PLX_EXPORT parallax_status_t parallax_decode_lla_workspace_size(const parallax_decode_args_t *dec,
                                                                const parallax_lla_args_t *lla,
                                                                size_t *bytes) {
    if (bytes == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "lla: bytes is NULL");
    LlaPlan lp;
    parallax_status_t s = plan_lla(dec, lla, &lp);
    if (s != PARALLAX_OK) return s;
    *bytes = lp.total_bytes;
    return PARALLAX_OK;
}

PLX_EXPORT parallax_status_t parallax_decode_lla(const parallax_decode_args_t *dec,
                                                 const parallax_lla_args_t *lla, void *workspace,
                                                 size_t workspace_bytes, void *hip_stream) {
    LlaPlan lp;
    parallax_status_t s = plan_lla(dec, lla, &lp);
    if (s != PARALLAX_OK) return s;
    if (workspace == nullptr || workspace_bytes < lp.total_bytes)
        return fail(PARALLAX_ERR_WORKSPACE, "lla: workspace of %zu bytes needed, %zu given",
                    lp.total_bytes, workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (!aligned16(workspace))
        return fail(PARALLAX_ERR_WORKSPACE, "lla: workspace must be 16-byte aligned");
    hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    const int64_t n = (int64_t)dec->batch * dec->num_q_heads * dec->head_dim;
    float *vec = reinterpret_cast<float *>(ws + lp.decode_bytes);
    float *kbar = vec, *ok = vec + n, *x = vec + 2 * n, *r = vec + 3 * n, *dir = vec + 4 * n;
    float *rs = vec + 5 * n;

    // the user's decode with rho = x, and the CG sweep: keys as values, rho = dir
    plx::DecodeParams fin = decode_params(dec, lp.dplan, workspace);
    fin.rho = x;
    fin.rho_sb = (int64_t)dec->num_q_heads * dec->head_dim;
    fin.rho_sh = dec->head_dim;
    plx::DecodeParams sweep = fin;
    sweep.arrivals = nullptr;  // the sweeps' records go to the merge kernel (the CG step)
    sweep.v = sweep.k;
    sweep.v_s0 = sweep.k_s0;
    sweep.v_sh = sweep.k_sh;
    sweep.v_st = sweep.k_st;
    sweep.rho = dir;
    sweep.out = kbar;
    sweep.out_sb = fin.rho_sb;
    sweep.out_sh = fin.rho_sh;

    plx::LlaParams lpar;
    lpar.q = dec->q;
    lpar.q_sb = dec->q_stride_b;
    lpar.q_sh = dec->q_stride_h;
    lpar.kbar = kbar;
    lpar.ok = ok;
    lpar.x = x;
    lpar.r = r;
    lpar.dir = dir;
    lpar.rs = rs;
    lpar.seq_lens = dec->seq_lens;
    lpar.max_seq_len = dec->max_seq_len;
    lpar.rho_out = lla->rho_out;
    lpar.resid = lla->resid;
    lpar.batch = dec->batch;
    lpar.num_q_heads = dec->num_q_heads;
    lpar.d = dec->head_dim;
    lpar.lambda = lla->lambda;

    auto run_decode = [&](const plx::DecodeParams &dp, const plx::LlaParams *step) {
        return plx::launch_decode(dp, dec->kv_dtype, dec->head_dim, lp.dplan.group, lp.dplan.paged,
                                  dec->batch, stream, step);
    };
    hipError_t e = plx::launch_lla_zero(dir, n, stream);  // rho = 0: the sweep gives kbar
    if (e == hipSuccess) e = run_decode(sweep, nullptr);
    if (e == hipSuccess) e = plx::launch_lla_init(lpar, stream);
    sweep.out = ok;
    // each iteration: the sweep, then the step inside its merge kernel
    for (int it = 0; it < lla->iterations && e == hipSuccess; ++it) e = run_decode(sweep, &lpar);
    if (e == hipSuccess) e = run_decode(fin, nullptr);
    if (e == hipSuccess) e = plx::launch_lla_finish(lpar, stream);
    return hip_status(e, "lla launch");
}

PLX_EXPORT parallax_status_t parallax_qr_projection(const parallax_qr_projection_args_t *a,
                                                    void *hip_stream) {
    parallax_status_t s = check_projection(a);
    if (s != PARALLAX_OK) return s;
    plx::ProjParams p;
    p.x = static_cast<const uint16_t *>(a->x);
    p.x_st = a->x_stride_t;
    p.w_q = static_cast<const uint16_t *>(a->w_q);
    p.w_r = static_cast<const uint16_t *>(a->w_r);
    p.w_sn = a->w_stride_n;
    p.q = a->q;
    p.rho = a->rho;
    p.q_st = a->q_stride_t;
    p.q_sh = a->q_stride_h;
    p.r_st = a->rho_stride_t;
    p.r_sh = a->rho_stride_h;
    p.tokens = a->tokens;
    p.model_dim = a->model_dim;
    p.n = a->num_q_heads * a->head_dim;
    p.head_dim = a->head_dim;
    p.out_bf16 = a->out_dtype == PARALLAX_BF16 ? 1 : 0;
    return hip_status(plx::launch_qr_projection(p, static_cast<hipStream_t>(hip_stream)),
                      "projection launch");
}

PLX_EXPORT parallax_status_t parallax_prefill(const parallax_prefill_args_t *a, void *hip_stream) {
    parallax_status_t s = check_prefill(a);
    if (s != PARALLAX_OK) return s;
    plx::PrefillParams p;
    p.q = static_cast<const uint16_t *>(a->q);
    p.rho = static_cast<const uint16_t *>(a->rho);
    p.k = static_cast<const uint16_t *>(a->k);
    p.v = static_cast<const uint16_t *>(a->v);
    p.out = a->out;
    p.q_sb = a->q_stride_b;
    p.q_ss = a->q_stride_s;
    p.q_sh = a->q_stride_h;
    p.r_sb = a->rho_stride_b;
    p.r_ss = a->rho_stride_s;
    p.r_sh = a->rho_stride_h;
    p.k_sb = a->k_stride_b;
    p.k_ss = a->k_stride_s;
    p.k_sh = a->k_stride_h;
    p.v_sb = a->v_stride_b;
    p.v_ss = a->v_stride_s;
    p.v_sh = a->v_stride_h;
    p.o_sb = a->out_stride_b;
    p.o_ss = a->out_stride_s;
    p.o_sh = a->out_stride_h;
    p.batch = a->batch;
    p.seq_len = a->seq_len;
    p.num_q_heads = a->num_q_heads;
    p.num_kv_heads = a->num_kv_heads;
    // the kernel multiplies raw scores by a positive factor (masking and the
    // row max rely on it); the sign of the scale moves into the query operand
    p.q_sign = a->scale > 0.0f ? 0 : (a->scale < 0.0f ? 1 : 2);
    p.scale_log2 = (float)(a->scale != 0.0f ? fabs((double)a->scale) * 1.4426950408889634 : 1.0);
    p.window = a->window;
    p.workgroups = a->workgroups;
    p.lse = a->lse;
    p.rmean = a->rmean;
    p.o_sa = a->o_sa;
    return hip_status(plx::launch_prefill(p, a->head_dim, static_cast<hipStream_t>(hip_stream)),
                      "prefill launch");
}

PLX_EXPORT parallax_status_t parallax_prefill_backward_workspace_size(
    const parallax_prefill_backward_args_t *args, size_t *bytes) {
    if (bytes == nullptr) return fail(PARALLAX_ERR_INVALID_ARG, "prefill backward: bytes is NULL");
    parallax_status_t s = check_prefill_backward(args);
    if (s != PARALLAX_OK) return s;
    *bytes = prefill_backward_workspace(args);
    return PARALLAX_OK;
}

PLX_EXPORT parallax_status_t parallax_prefill_backward(const parallax_prefill_backward_args_t *a,
                                                       void *workspace, size_t workspace_bytes,
                                                       void *hip_stream) {
    parallax_status_t s = check_prefill_backward(a);
    if (s != PARALLAX_OK) return s;
    const size_t need = prefill_backward_workspace(a);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(PARALLAX_ERR_WORKSPACE,
                    "prefill backward: workspace of %zu bytes needed, %zu given", need,
                    workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (!aligned16(workspace))
        return fail(PARALLAX_ERR_WORKSPACE, "prefill backward: workspace must be 16-byte aligned");
    plx::PrefillBwdParams p;
    p.q = static_cast<const uint16_t *>(a->q);
    p.rho = static_cast<const uint16_t *>(a->rho);
    p.k = static_cast<const uint16_t *>(a->k);
    p.v = static_cast<const uint16_t *>(a->v);
    p.dout = static_cast<const uint16_t *>(a->dout);
    p.out = a->out;
    p.o_sa = a->o_sa;
    p.lse = a->lse;
    p.rmean = a->rmean;
    p.dq = a->dq;
    p.drho = a->drho;
    p.dk = a->dk;
    p.dv = a->dv;
    p.rowstat = static_cast<float4 *>(workspace);
    p.q_sb = a->q_stride_b;
    p.q_ss = a->q_stride_s;
    p.q_sh = a->q_stride_h;
    p.r_sb = a->rho_stride_b;
    p.r_ss = a->rho_stride_s;
    p.r_sh = a->rho_stride_h;
    p.k_sb = a->k_stride_b;
    p.k_ss = a->k_stride_s;
    p.k_sh = a->k_stride_h;
    p.v_sb = a->v_stride_b;
    p.v_ss = a->v_stride_s;
    p.v_sh = a->v_stride_h;
    p.g_sb = a->dout_stride_b;
    p.g_ss = a->dout_stride_s;
    p.g_sh = a->dout_stride_h;
    p.o_sb = a->out_stride_b;
    p.o_ss = a->out_stride_s;
    p.o_sh = a->out_stride_h;
    p.dq_sb = a->dq_stride_b;
    p.dq_ss = a->dq_stride_s;
    p.dq_sh = a->dq_stride_h;
    p.dk_sb = a->dk_stride_b;
    p.dk_ss = a->dk_stride_s;
    p.dk_sh = a->dk_stride_h;
    p.batch = a->batch;
    p.seq_len = a->seq_len;
    p.num_q_heads = a->num_q_heads;
    p.num_kv_heads = a->num_kv_heads;
    p.scale = a->scale;
    p.scale_log2 = (float)((double)a->scale * 1.4426950408889634);
    p.window = a->window;
    return hip_status(
        plx::launch_prefill_backward(p, a->head_dim, static_cast<hipStream_t>(hip_stream)),
        "prefill backward launch");
}
