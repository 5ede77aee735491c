// decode.hip -- Parallax decode attention for gfx950 (CDNA4).
//
// One pass over the KV cache computes, for every query head of a KV head,
// the softmax sums and the covariance-correction sums at once (page "Parallax:
// Parameterized Local Linear Attention Gives Transformers a 'Second Eye'",
// sections 1.3 and 2.2; the zubnet.ai news item on Parallax, second
// paragraph: one KV stream feeds both branches):
//
//   s_j = scale (q . k_j)   t_j = rho . k_j
//   Z = sum e^{s_j}   R = sum e^{s_j} t_j   A = sum e^{s_j} v_j   B = sum e^{s_j} t_j v_j
//   o = a - (b - a r)   with a = A/Z, r = R/Z, b = B/Z
//
// which equals o_SA - S_KV rho for the softmax-weighted covariance S_KV.
//
// Design (decode is bound by HBM reads of K and V: 4 flop per KV byte at
// GQA group 2, far under the chip's VALU balance, so no matrix cores):
//   * grid: (batch, KV head, context split); one workgroup of 4 waves reads
//     each key/value row once and serves all G query heads of its KV head.
//   * lanes: a token row is split into 16-byte pieces, one per lane
//     (16 lanes per row for bf16 d=128), so one wave-wide load covers whole
//     rows and is fully coalesced; each wave step covers 16 tokens (= one
//     page of the paged cache).
//   * bf16 keys meet q and rho through v_dot2_f32_bf16 with q and rho split
//     into bf16 hi + lo parts (about 16 mantissa bits); values are widened to
//     fp32 exactly and accumulated with fp32 FMA.
//   * per-token dot products are summed across the lanes of a row with DPP
//     butterflies, which leave every lane of the row with bitwise the same sum.
//   * logits are kept in base 2 (scale * log2 e folded into q); the running
//     reference max is only raised when a logit exceeds it by more than 8, so
//     the rescale of A and B is rare; every weight stays below 2^8.
//   * splits of one (batch, KV head) write partial (m, Z, R, A, B) records;
//     the last split to arrive (atomic ticket) merges them and writes o, then
//     re-arms the ticket, so a single launch does the whole decode.
#include "kernels.hpp"

#include <math.h>

namespace plx {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kRescaleSlack = 8.0f;  // base-2 headroom before the reference max moves

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of N lanes (N in 2..32).  Each step adds a value
// and its partner's, so partners compute the same sum in swapped order and
// every lane of the group ends with bitwise the same result.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp_mov<0xB1>(x);                          // quad_perm [1,0,3,2]
    if constexpr (N >= 4) x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
    if constexpr (N >= 8) x += dpp_mov<0x141>(x);   // row_half_mirror
    if constexpr (N >= 16) x += dpp_mov<0x140>(x);  // row_mirror
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    return x;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x2_t pack_bf16(float a, float b) {
    bf16x2_t r = {(__bf16)a, (__bf16)b};
    return r;
}

// Lane geometry for a cache element type and head dim.
template <typename KV, int D>
struct Geo {
    static constexpr int VEC = 16 / (int)sizeof(KV);     // elements per 16-byte lane load
    static constexpr int LPT = D / VEC;                  // lanes per token row
    static constexpr int TPL = 64 / LPT;                 // token rows per wave-wide load
    static constexpr int U = kDecodeStepTokens / TPL;    // loads per 16-token step
    static_assert(LPT >= 2 && LPT <= 32 && (LPT & (LPT - 1)) == 0, "unsupported geometry");
    static_assert(U * TPL == kDecodeStepTokens, "step must be a whole number of loads");
};

// Query-side operands of one lane: its VEC-wide slice of q (pre-scaled to
// base-2 logits) and of rho for each of the G heads.
template <typename KV, int D, int G>
struct QueryRegs;

template <int D, int G>
struct QueryRegs<uint16_t, D, G> {  // bf16 cache: two-term bf16 splits
    static constexpr int P = Geo<uint16_t, D>::VEC / 2;
    bf16x2_t qh[G][P], ql[G][P], rh[G][P], rl[G][P];

    __device__ void set(int g, const float *q, const float *r) {
        for (int i = 0; i < P; ++i) {
            float q0 = q[2 * i], q1 = q[2 * i + 1], r0 = r[2 * i], r1 = r[2 * i + 1];
            qh[g][i] = pack_bf16(q0, q1);
            rh[g][i] = pack_bf16(r0, r1);
            ql[g][i] = pack_bf16(q0 - (float)qh[g][i][0], q1 - (float)qh[g][i][1]);
            rl[g][i] = pack_bf16(r0 - (float)rh[g][i][0], r1 - (float)rh[g][i][1]);
        }
    }
    // Partial (this lane's slice) of q.k and rho.k for head g.
    __device__ __forceinline__ void dots(int g, const uint4 &kw, float &s, float &t) const {
        const uint32_t w[4] = {kw.x, kw.y, kw.z, kw.w};
        float sh = 0.f, sl = 0.f, th = 0.f, tl = 0.f;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            bf16x2_t kk = __builtin_bit_cast(bf16x2_t, w[i]);
            sh = __builtin_amdgcn_fdot2_f32_bf16(qh[g][i], kk, sh, false);
            sl = __builtin_amdgcn_fdot2_f32_bf16(ql[g][i], kk, sl, false);
            th = __builtin_amdgcn_fdot2_f32_bf16(rh[g][i], kk, th, false);
            tl = __builtin_amdgcn_fdot2_f32_bf16(rl[g][i], kk, tl, false);
        }
        s = sh + sl;
        t = th + tl;
    }
    __device__ __forceinline__ static void widen(const uint4 &vw, float *vf) {
        const uint32_t w[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            vf[2 * i] = bf16_lo(w[i]);
            vf[2 * i + 1] = bf16_hi(w[i]);
        }
    }
};

template <int D, int G>
struct QueryRegs<float, D, G> {  // fp32 cache: plain fp32 FMA
    static constexpr int VEC = 4;
    float qf[G][VEC], rf[G][VEC];

    __device__ void set(int g, const float *q, const float *r) {
        for (int i = 0; i < VEC; ++i) {
            qf[g][i] = q[i];
            rf[g][i] = r[i];
        }
    }
    __device__ __forceinline__ void dots(int g, const uint4 &kw, float &s, float &t) const {
        const float k[4] = {__uint_as_float(kw.x), __uint_as_float(kw.y), __uint_as_float(kw.z),
                            __uint_as_float(kw.w)};
        float s0 = qf[g][0] * k[0], t0 = rf[g][0] * k[0];
#pragma unroll
        for (int i = 1; i < VEC; ++i) {
            s0 = fmaf(qf[g][i], k[i], s0);
            t0 = fmaf(rf[g][i], k[i], t0);
        }
        s = s0;
        t = t0;
    }
    __device__ __forceinline__ static void widen(const uint4 &vw, float *vf) {
        vf[0] = __uint_as_float(vw.x);
        vf[1] = __uint_as_float(vw.y);
        vf[2] = __uint_as_float(vw.z);
        vf[3] = __uint_as_float(vw.w);
    }
};

// Running sums of one lane for one head: reference max m (base 2), Z, R and
// this lane's VEC-wide slices of A and B.
template <int VEC>
struct Acc {
    float m, Z, R, A[VEC], B[VEC];
    __device__ void init() {
        m = -INFINITY;
        Z = R = 0.f;
        for (int e = 0; e < VEC; ++e) A[e] = B[e] = 0.f;
    }
    __device__ __forceinline__ void scale_by(float alpha) {
        Z *= alpha;
        R *= alpha;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            A[e] *= alpha;
            B[e] *= alpha;
        }
    }
    // Fold another lane's state (same slice) into this one.
    __device__ __forceinline__ void merge(float m2, float Z2, float R2, const float *A2,
                                          const float *B2) {
        float mn = fmaxf(m, m2);
        float a1 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        float a2 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
        Z = a1 * Z + a2 * Z2;
        R = a1 * R + a2 * R2;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            A[e] = a1 * A[e] + a2 * A2[e];
            B[e] = a1 * B[e] + a2 * B2[e];
        }
        m = mn;
    }
};

__device__ __forceinline__ uint4 load16(const void *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

template <typename KV, int D, int G, bool PAGED>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_kernel(DecodeParams p) {
    using Gm = Geo<KV, D>;
    constexpr int VEC = Gm::VEC, LPT = Gm::LPT, TPL = Gm::TPL, U = Gm::U;
    constexpr int REC = partial_floats(D);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = lane / LPT;  // token row of this lane within a wave-wide load
    const int sub = lane % LPT;  // 16-byte piece of the row

    const int split_idx = blockIdx.x % p.nsplit;
    const int unit = blockIdx.x / p.nsplit;  // b * Hkv + hk
    const int b = unit / p.num_kv_heads;
    const int hk = unit % p.num_kv_heads;

    int L = p.seq_lens ? p.seq_lens[b] : p.max_seq_len;
    L = max(0, min(L, PAGED ? p.max_blocks * kDecodeStepTokens : p.max_seq_len));
    const int nsp = max(1, min(p.nsplit, (L + p.split - 1) / p.split));
    if (split_idx >= nsp) return;
    const int t0 = split_idx * p.split;
    const int t1 = min(L, t0 + p.split);
    const int nsteps = max(0, (t1 - t0 + kDecodeStepTokens - 1) / kDecodeStepTokens);

    // ---- query operands
    QueryRegs<KV, D, G> qr;
    {
        const int h0 = hk * G;
        for (int g = 0; g < G; ++g) {
            const float *qp = p.q + b * p.q_sb + (int64_t)(h0 + g) * p.q_sh + sub * VEC;
            const float *rp = p.rho + b * p.rho_sb + (int64_t)(h0 + g) * p.rho_sh + sub * VEC;
            float qv[VEC], rv[VEC];
            for (int i = 0; i < VEC; i += 4) {
                float4 a = *reinterpret_cast<const float4 *>(qp + i);
                float4 c = *reinterpret_cast<const float4 *>(rp + i);
                qv[i] = a.x * p.scale_log2;
                qv[i + 1] = a.y * p.scale_log2;
                qv[i + 2] = a.z * p.scale_log2;
                qv[i + 3] = a.w * p.scale_log2;
                rv[i] = c.x;
                rv[i + 1] = c.y;
                rv[i + 2] = c.z;
                rv[i + 3] = c.w;
            }
            qr.set(g, qv, rv);
        }
    }

    Acc<VEC> acc[G];
    for (int g = 0; g < G; ++g) acc[g].init();

    const KV *kc = static_cast<const KV *>(p.k);
    const KV *vc = static_cast<const KV *>(p.v);
    const int64_t row_off_k = (int64_t)sub * VEC;

    // Base pointers of the 16-token step starting at token `base`.
    auto step_bases = [&](int base, const KV *&kb, const KV *&vb) {
        if constexpr (PAGED) {
            const int pg = p.block_table[(int64_t)b * p.max_blocks + base / kDecodeStepTokens];
            kb = kc + (int64_t)pg * p.k_s0 + (int64_t)hk * p.k_sh;
            vb = vc + (int64_t)pg * p.v_s0 + (int64_t)hk * p.v_sh;
        } else {
            kb = kc + (int64_t)b * p.k_s0 + (int64_t)hk * p.k_sh + (int64_t)base * p.k_st;
            vb = vc + (int64_t)b * p.v_s0 + (int64_t)hk * p.v_sh + (int64_t)base * p.v_st;
        }
    };
    // Issue the loads of one step.  Rows past t1 re-read the step's last
    // valid token (always in bounds); their weight is forced to zero.
    auto issue = [&](int st, uint4 *kw, uint4 *vw) {
        const int base = t0 + st * kDecodeStepTokens;
        const KV *kb, *vb;
        step_bases(base, kb, vb);
        const int last = t1 - 1 - base;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int j = u * TPL + row;
            j = j <= last ? j : last;
            kw[u] = load16(kb + (int64_t)j * p.k_st + row_off_k);
            vw[u] = load16(vb + (int64_t)j * p.v_st + row_off_k);
        }
    };

    uint4 kw[U], vw[U];
    int st = wave;
    if (st < nsteps) issue(st, kw, vw);
    while (st < nsteps) {
        uint4 kcur[U], vcur[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            kcur[u] = kw[u];
            vcur[u] = vw[u];
        }
        const int base = t0 + st * kDecodeStepTokens;
        const int nst = st + kDecodeWaves;
        if (nst < nsteps) issue(nst, kw, vw);  // prefetch the next step

#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool valid = base + u * TPL + row < t1;
            float vf[VEC];
            QueryRegs<KV, D, G>::widen(vcur[u], vf);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float s, t;
                qr.dots(g, kcur[u], s, t);
                s = group_sum<LPT>(s);
                t = group_sum<LPT>(t);
                s = valid ? s : -INFINITY;
                Acc<VEC> &a = acc[g];
                if (s > a.m + kRescaleSlack) {  // also taken by the first token
                    a.scale_by(__builtin_amdgcn_exp2f(a.m - s));
                    a.m = s;
                }
                const float w = valid ? __builtin_amdgcn_exp2f(s - a.m) : 0.f;
                const float wt = w * t;
                a.Z += w;
                a.R += wt;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    a.A[e] = fmaf(w, vf[e], a.A[e]);
                    a.B[e] = fmaf(wt, vf[e], a.B[e]);
                }
            }
        }
        st = nst;
    }

    // ---- merge the token rows of this wave (lanes LPT, 2*LPT, ... apart)
#pragma unroll
    for (int off = LPT; off < 64; off *= 2) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            Acc<VEC> &a = acc[g];
            float m2 = __shfl_xor(a.m, off), Z2 = __shfl_xor(a.Z, off),
                  R2 = __shfl_xor(a.R, off);
            float A2[VEC], B2[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                A2[e] = __shfl_xor(a.A[e], off);
                B2[e] = __shfl_xor(a.B[e], off);
            }
            a.merge(m2, Z2, R2, A2, B2);
        }
    }

    // ---- merge the waves through LDS
    __shared__ float red[kDecodeWaves][G][REC];
    if (row == 0) {
        for (int g = 0; g < G; ++g) {
            for (int e = 0; e < VEC; ++e) {
                red[wave][g][sub * VEC + e] = acc[g].A[e];
                red[wave][g][D + sub * VEC + e] = acc[g].B[e];
            }
            if (sub == 0) {
                red[wave][g][2 * D] = acc[g].m;
                red[wave][g][2 * D + 1] = acc[g].Z;
                red[wave][g][2 * D + 2] = acc[g].R;
            }
        }
    }
    __syncthreads();

    const bool single = nsp == 1;
    float *my_rec = single ? nullptr
                           : p.partials + ((int64_t)unit * p.nsplit + split_idx) * G * REC;
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * kDecodeWaves) {
        const int g = idx / D, e = idx % D;
        float M = -INFINITY;
        for (int w = 0; w < kDecodeWaves; ++w) M = fmaxf(M, red[w][g][2 * D]);
        float Z = 0.f, R = 0.f, A = 0.f, B = 0.f;
        if (M != -INFINITY) {
            for (int w = 0; w < kDecodeWaves; ++w) {
                const float al = __builtin_amdgcn_exp2f(red[w][g][2 * D] - M);
                Z += al * red[w][g][2 * D + 1];
                R += al * red[w][g][2 * D + 2];
                A += al * red[w][g][e];
                B += al * red[w][g][D + e];
            }
        }
        if (single) {
            float o = 0.f;
            if (Z > 0.f) {
                const float inv = 1.0f / Z;
                const float av = A * inv, bv = B * inv, r = R * inv;
                o = av - (bv - av * r);
            }
            p.out[b * p.out_sb + (int64_t)(hk * G + g) * p.out_sh + e] = o;
        } else {
            float *rec = my_rec + g * REC;
            rec[e] = A;
            rec[D + e] = B;
            if (e == 0) {
                rec[2 * D] = M;
                rec[2 * D + 1] = Z;
                rec[2 * D + 2] = R;
            }
        }
    }
    if (single) return;

    // ---- the last split of this (batch, KV head) to finish merges all splits
    __shared__ int is_last;
    __threadfence();  // release this split's record to the whole device
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = atomicAdd(&p.counters[unit], 1u);
        is_last = prev == (unsigned)(nsp - 1);
    }
    __syncthreads();
    if (!is_last) return;
    __threadfence();  // acquire the other splits' records
    if (threadIdx.x == 0)
        __hip_atomic_store(&p.counters[unit], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    const float *recs = p.partials + (int64_t)unit * p.nsplit * G * REC;
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * kDecodeWaves) {
        const int g = idx / D, e = idx % D;
        float M = -INFINITY;
        for (int c = 0; c < nsp; ++c) M = fmaxf(M, recs[(c * G + g) * REC + 2 * D]);
        float Z = 0.f, R = 0.f, A = 0.f, B = 0.f;
        for (int c = 0; c < nsp; ++c) {
            const float *rec = recs + (c * G + g) * REC;
            const float al = __builtin_amdgcn_exp2f(rec[2 * D] - M);
            Z += al * rec[2 * D + 1];
            R += al * rec[2 * D + 2];
            A += al * rec[e];
            B += al * rec[D + e];
        }
        const float inv = 1.0f / Z;
        const float av = A * inv, bv = B * inv, r = R * inv;
        p.out[b * p.out_sb + (int64_t)(hk * G + g) * p.out_sh + e] = av - (bv - av * r);
    }
}

template <typename KV, int D, int G>
hipError_t launch_g(const DecodeParams &p, bool paged, int batch, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)batch * p.num_kv_heads * p.nsplit));
    const dim3 block(64 * kDecodeWaves);
    if (paged)
        hipLaunchKernelGGL((decode_kernel<KV, D, G, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((decode_kernel<KV, D, G, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <typename KV, int D>
hipError_t launch_d(const DecodeParams &p, int group, bool paged, int batch, hipStream_t s) {
    switch (group) {
        case 1: return launch_g<KV, D, 1>(p, paged, batch, s);
        case 2: return launch_g<KV, D, 2>(p, paged, batch, s);
        case 4: return launch_g<KV, D, 4>(p, paged, batch, s);
        case 8: return launch_g<KV, D, 8>(p, paged, batch, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int kv_dtype, int d, int group, bool paged,
                         int batch, hipStream_t stream) {
    if (kv_dtype == 1) {  // bf16
        if (d == 128) return launch_d<uint16_t, 128>(p, group, paged, batch, stream);
        if (d == 64) return launch_d<uint16_t, 64>(p, group, paged, batch, stream);
    } else {
        if (d == 128) return launch_d<float, 128>(p, group, paged, batch, stream);
        if (d == 64) return launch_d<float, 64>(p, group, paged, batch, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace plx
