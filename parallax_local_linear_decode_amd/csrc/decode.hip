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
// Common structure: grid = context splits x (batch x KV head) units, split
// major, so consecutive workgroups (dealt round-robin to the XCDs) belong to
// different units and every XCD gets a like share of work.  A workgroup
// reads each key/value row of its split once and serves all G query heads of
// its KV head.  Logits are kept in base 2 (scale * log2 e folded into q).
// The running reference max only moves when a logit exceeds it by more than
// 8, so rescaling is rare and every weight stays below 2^8.
// Each split leaves a partial record (m, Z, R, A, B) per query head; with
// more than one split a small merge kernel combines them.  Every launch is
// self-contained: no cross-workgroup fences, atomics or counters.
//
// bf16 cache -- matrix-core kernel.  Scores and both value sums are dense
// contractions over the shared KV stream, so they run on bf16 MFMA
// (16x16x32, fp32 accumulate):
//   scores  D1[token][col] = K[token][:] . C[col][:]   with columns
//           q_h hi, rho_h hi, q_h lo, rho_h lo   (two-term bf16 splits of
//           fp32 q and rho, about 16 significant bits);
//   sums    D2[d][col] = sum_token V[token][d] . P[token][col]   with columns
//           w_h hi, w_h t_h hi, w_h lo, w_h t_h lo  (w = e^{s - m}),
//   so A_h, B_h come out of the same MFMAs as hi + lo column pairs.  The
//   softmax step works directly in the MFMA accumulator layout, using DPP
//   row shifts to move values between columns.  V reaches the MFMA through a
//   wave-private LDS tile read back with ds_read_b64_tr_b16, which returns
//   the token-major tile transposed into operand layout.  Eight waves per
//   workgroup, 32 tokens per wave step, next step's loads in flight while the
//   current step computes.
//
// fp32 cache -- VALU kernel (the fp32 path exists for fp32-accurate checks;
// matrix cores have no fp32-exact mode at this precision):
//   a token row is split into 16-byte pieces, one per lane, so one wave-wide
//   load covers whole rows; per-token dot products are summed across the row
//   with DPP butterflies; values accumulate with fp32 FMA.
#include "kernels.hpp"
#include "lla_row.hpp"

#include <math.h>

namespace plx {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kRescaleSlack = 8.0f;  // base-2 headroom before the reference max moves

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, true);
}
// Within each row of 16 lanes: lane i receives lane i+N (shl) / i-N (shr);
// lanes whose source falls outside the row receive 0.
template <int N> __device__ __forceinline__ float row_shl(float x) { return dpp_f<0x100 + N>(x); }
template <int N> __device__ __forceinline__ float row_shr(float x) { return dpp_f<0x110 + N>(x); }
template <int N> __device__ __forceinline__ uint32_t row_shr_u(uint32_t x) { return dpp_u<0x110 + N>(x); }

__device__ __forceinline__ float read_lane(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint4 load16(const void *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

// Window starts are rounded down to whole 32-token steps, so a step never
// straddles more than two 16-token pages.
constexpr int kWindowAlign = 32;

// Sequence length L of batch row b, clamped to what the cache can hold; the
// first token tb the row attends to (0, or L - window for the local-window
// variant); tbase, tb rounded down to a step boundary, where split 0 starts
// (tokens tbase .. tb-1 are masked); and the number of splits the row uses
// (at least one, so an empty row still gets its zero output written).
template <bool PAGED>
__device__ __forceinline__ void row_extent(const DecodeParams &p, int b, int &L, int &tb,
                                           int &tbase, int &nsp) {
    L = p.seq_lens ? p.seq_lens[b] : p.max_seq_len;
    L = max(0, min(L, PAGED ? p.max_blocks * kDecodeStepTokens : p.max_seq_len));
    tb = p.window > 0 ? max(0, L - p.window) : 0;
    tbase = tb & ~(kWindowAlign - 1);
    nsp = max(1, min(p.nsplit, (L - tbase + p.split - 1) / p.split));
}

__device__ __forceinline__ float finish(float A, float B, float Z, float R) {
    if (!(Z > 0.f)) return 0.f;  // empty row
    const float inv = 1.0f / Z;
    const float a = A * inv, bb = B * inv, r = R * inv;
    return a - (bb - a * r);
}

// Reads and writes of split records that other compute units -- possibly on
// another XCD, whose L2 is not coherent with this one -- exchange within one
// launch: device-scope atomics, which go through to the device-coherent level.
__device__ __forceinline__ float load_shared(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_shared(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sums of element e of head g over split records [lo, hi) at `recs` (one
// unit): the running max M over the records, and Z, R, A, B with every
// record's sums scaled to it.  Sixteen records' loads are in flight at a time
// (one round trip for up to sixteen records).
constexpr int kMergeChunk = 16;
template <int D, int G, bool SHARED>
__device__ __forceinline__ void merge_range(const float *recs, int lo, int hi, int g, int e,
                                            float &M, float &Z, float &R, float &A, float &B) {
    constexpr int REC = partial_floats(D);
    auto ld = [](const float *q) { return SHARED ? load_shared(q) : *q; };
    M = -INFINITY;
    Z = R = A = B = 0.f;
    for (int c0 = lo; c0 < hi; c0 += kMergeChunk) {
        float mm[kMergeChunk], zz[kMergeChunk], rr[kMergeChunk], aa[kMergeChunk], bb[kMergeChunk];
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i) {
            const float *rec = recs + (min(c0 + i, hi - 1) * G + g) * REC;
            const bool live = c0 + i < hi;
            mm[i] = live ? ld(rec + 2 * D) : -INFINITY;
            zz[i] = ld(rec + 2 * D + 1);
            rr[i] = ld(rec + 2 * D + 2);
            aa[i] = ld(rec + e);
            bb[i] = ld(rec + D + e);
        }
        float Mn = M;
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i) Mn = fmaxf(Mn, mm[i]);
        const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
        Z *= sc;
        R *= sc;
        A *= sc;
        B *= sc;
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i) {
            const float al = mm[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mm[i] - Mn);
            Z += al * zz[i];
            R += al * rr[i];
            A += al * aa[i];
            B += al * bb[i];
        }
        M = Mn;
    }
}

// o of element e of head g from the nsp split records at `recs` (one unit).
template <int D, int G, bool SHARED>
__device__ __forceinline__ float merge_records(const float *recs, int nsp, int g, int e) {
    float M, Z, R, A, B;
    merge_range<D, G, SHARED>(recs, 0, nsp, g, e, M, Z, R, A, B);
    return finish(A, B, Z, R);
}

// Arrival of split `split_idx` of `unit`, by one wave of the workgroup once
// every wave's record stores are complete at device scope: set this split's
// flag, then read the row's flags.  True if all nsp carry this call's tag --
// then every record of the row is complete.  The split whose flag lands last
// sees them all; one that lands at nearly the same time may too, and both
// merge (the same records give the same bits).
__device__ __forceinline__ bool arrive_all(const DecodeParams &p, int unit, int split_idx, int nsp,
                                           int lane) {
    unsigned long long *f = p.arrivals + (int64_t)unit * p.nsplit;
    if (lane == 0)
        __hip_atomic_store(f + split_idx, p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    bool mine = true;
    for (int i = lane; i < nsp; i += 64)
        mine &= __hip_atomic_load(f + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == p.epoch;
    return __all(mine);
}

// Merge NW per-wave records (red[w][head][...]) of this workgroup; write
// the output if the row has a single split, else this split's record -- and,
// with the in-kernel merge, let the row's last arriving split merge them.
template <int D, int G, int NW>
__device__ void finish_block(const DecodeParams &p, float (*red)[G][partial_floats(D)], int b,
                             int hk, int unit, int split_idx, int nsp) {
    constexpr int REC = partial_floats(D);
    const bool fused = p.arrivals != nullptr && nsp > 1;
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * NW) {
        const int g = idx / D, e = idx % D;
        float M = -INFINITY;
        for (int w = 0; w < NW; ++w) M = fmaxf(M, red[w][g][2 * D]);
        float Z = 0.f, R = 0.f, A = 0.f, B = 0.f;
        if (M != -INFINITY) {
            for (int w = 0; w < NW; ++w) {
                const float al = __builtin_amdgcn_exp2f(red[w][g][2 * D] - M);
                Z += al * red[w][g][2 * D + 1];
                R += al * red[w][g][2 * D + 2];
                A += al * red[w][g][e];
                B += al * red[w][g][D + e];
            }
        }
        if (nsp == 1) {
            p.out[b * p.out_sb + (int64_t)(hk * G + g) * p.out_sh + e] = finish(A, B, Z, R);
        } else {
            float *rec = p.partials + (((int64_t)unit * p.nsplit + split_idx) * G + g) * REC;
            if (fused) {
                store_shared(rec + e, A);
                store_shared(rec + D + e, B);
                if (e == 0) {
                    store_shared(rec + 2 * D, M);
                    store_shared(rec + 2 * D + 1, Z);
                    store_shared(rec + 2 * D + 2, R);
                }
            } else {
                rec[e] = A;
                rec[D + e] = B;
                if (e == 0) {
                    rec[2 * D] = M;
                    rec[2 * D + 1] = Z;
                    rec[2 * D + 2] = R;
                }
            }
        }
    }
    if (!fused) return;
    // Every thread waits until its record stores are complete at device
    // scope (vmcnt counts stores on this architecture); then one thread
    // counts the workgroup in.  No release fence: the records themselves
    // were written through to the device-coherent level.
    __shared__ int last;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (threadIdx.x < 64) {
        const bool all = arrive_all(p, unit, split_idx, nsp, threadIdx.x);
        if (threadIdx.x == 0) last = all ? 1 : 0;
    }
    __syncthreads();
    if (!last) return;
    const float *recs = p.partials + (int64_t)unit * p.nsplit * G * REC;
    // With more threads than elements, a row of more than sixteen splits is
    // merged in PARTS record ranges side by side (one round trip of loads
    // instead of one per sixteen records); ranges 1.. hand their sums to
    // range 0 through `red`, which is free again after the barriers above.
    constexpr int PARTS = 64 * NW > G * D ? 64 * NW / (G * D) : 1;
    if (PARTS > 1 && nsp > kMergeChunk) {
        const int part = threadIdx.x / (G * D), idx = threadIdx.x % (G * D);
        const int g = idx / D, e = idx % D;
        const int per = (nsp + PARTS - 1) / PARTS;
        const int lo = min(part * per, nsp), hi = min(lo + per, nsp);
        float M, Z, R, A, B;
        merge_range<D, G, true>(recs, lo, hi, g, e, M, Z, R, A, B);
        if (part > 0) {
            red[part][g][e] = A;
            red[part][g][D + e] = B;
            if (e == 0) {
                red[part][g][2 * D] = M;
                red[part][g][2 * D + 1] = Z;
                red[part][g][2 * D + 2] = R;
            }
        }
        __syncthreads();
        if (part == 0) {
            for (int q = 1; q < PARTS; ++q) {
                const float Mq = red[q][g][2 * D];
                const float Mn = fmaxf(M, Mq);
                const float s0 = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
                const float s1 = Mq == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mq - Mn);
                Z = Z * s0 + s1 * red[q][g][2 * D + 1];
                R = R * s0 + s1 * red[q][g][2 * D + 2];
                A = A * s0 + s1 * red[q][g][e];
                B = B * s0 + s1 * red[q][g][D + e];
                M = Mn;
            }
            p.out[b * p.out_sb + (int64_t)(hk * G + g) * p.out_sh + e] = finish(A, B, Z, R);
        }
    } else {
        for (int idx = threadIdx.x; idx < G * D; idx += 64 * NW) {
            const int g = idx / D, e = idx % D;
            p.out[b * p.out_sb + (int64_t)(hk * G + g) * p.out_sh + e] =
                merge_records<D, G, true>(recs, nsp, g, e);
        }
    }
    // Every split of the row has arrived: clear its flags, so that the next
    // launch with this tag (a replayed graph) starts from none.  A split
    // still reading them then sees fewer than all and does not merge.
    for (int i = threadIdx.x; i < nsp; i += 64 * NW)
        __hip_atomic_store(p.arrivals + (int64_t)unit * p.nsplit + i, 0ull, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// ===================================================== bf16: matrix cores ===

constexpr int kMfmaStep = 32;  // tokens per wave step (two 16-token MFMA row blocks)

// Waves per workgroup: 8 (two per SIMD) or 4 (one per SIMD; at most 168
// registers, so three such workgroups share a CU).  4 when eight query heads
// per KV head at d = 128 need more than the 256 registers two waves can each
// hold; else 4 when a workgroup's split has at most four 32-token steps (no
// wave idles) or when the grid has more workgroups than the 256 CUs (three
// workgroups per CU keep more loads in flight than one); 8 otherwise, where
// one workgroup per CU is all there is.
template <int D, int G>
constexpr int mfma_waves_max() { return (D == 128 && G == 8) ? 4 : 8; }
constexpr int kShortSteps = 4;    // steps per workgroup up to which 4 waves are used
constexpr int kDeviceCUs = 256;   // compute units of an MI355X

template <int D, int G, bool PAGED, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 && !(D == 128 && G == 8) ? 3 : 2) void
decode_mfma_kernel(DecodeParams p) {
    constexpr int kMfmaWaves = NW;
    constexpr int HS = G < 4 ? G : 4;     // query heads per 16-column set
    constexpr int NCS = G / HS;           // column sets (2 when G = 8)
    constexpr int KS = D / 32;            // score MFMAs per row block (K = 32 each)
    constexpr int DB = D / 16;            // 16-row blocks of the value sums
    constexpr int DQ = D / 4;             // head-dim values per lane group in the scores
    constexpr int LPR = D / 8;            // lanes per V row in a coalesced 16-byte load
    constexpr int RPL = 64 / LPR;         // V rows per wave-wide load
    constexpr int VLD = kMfmaStep / RPL;  // V loads per lane per step
    constexpr int VROW = 2 * D + 16;      // bytes per LDS row of the V tile (padded)
    constexpr int REC = partial_floats(D);

    __shared__ __attribute__((aligned(16))) unsigned char vtile[kMfmaWaves][kMfmaStep * VROW];
    __shared__ float red[kMfmaWaves][G][REC];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15;  // MFMA column (scores/sums) or row (V^T) index
    const int g = lane >> 4;  // lane group: which 8 k-slots of an MFMA operand

    const int units = gridDim.x / p.nsplit;
    const int split_idx = blockIdx.x / units;  // split-major order
    const int unit = blockIdx.x % units;
    const int b = unit / p.num_kv_heads;
    const int hk = unit % p.num_kv_heads;
    int L, tb, tbase, nsp;
    row_extent<PAGED>(p, b, L, tb, tbase, nsp);
    if (split_idx >= nsp) return;
    const int t0 = tbase + split_idx * p.split;
    const int t1 = min(L, t0 + p.split);
    const int nsteps = (t1 - t0 + kMfmaStep - 1) / kMfmaStep;

    // ---- running state: reference max per head (wave-uniform), value sums
    // in the MFMA accumulator layout, per-lane partial column totals
    float mref[NCS][HS];
    f32x4_t acc[NCS][DB];
    float ztot[NCS];
#pragma unroll
    for (int s = 0; s < NCS; ++s) {
        for (int h = 0; h < HS; ++h) mref[s][h] = -INFINITY;
        for (int db = 0; db < DB; ++db) acc[s][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        ztot[s] = 0.f;
    }

    const uint16_t *kc = static_cast<const uint16_t *>(p.k);
    const uint16_t *vc = static_cast<const uint16_t *>(p.v);
    // A step's 32 tokens start on a page boundary, so a paged step spans two
    // pages; their ids are wave-uniform and are fetched a step ahead.
    struct Pages {
        int p0, p1;
    };
    auto step_pages = [&](int st) -> Pages {
        Pages pg = {0, 0};
        if constexpr (PAGED) {
            const int base = t0 + st * kMfmaStep;
            const int32_t *row = p.block_table + (int64_t)b * p.max_blocks;
            pg.p0 = __builtin_amdgcn_readfirstlane(row[base / kDecodeStepTokens]);
            pg.p1 = __builtin_amdgcn_readfirstlane(
                row[min(base + kDecodeStepTokens, t1 - 1) / kDecodeStepTokens]);
        }
        return pg;
    };
    // Element offset of token j (clamped to [base, t1)) of this (b, hk).
    auto tok_off = [&](int j, int base, const Pages &pg, int64_t s0, int64_t sh,
                       int64_t stt) -> int64_t {
        if constexpr (PAGED) {
            const int pgid = j - base < kDecodeStepTokens ? pg.p0 : pg.p1;
            return (int64_t)pgid * s0 + (int64_t)hk * sh + (int64_t)(j % kDecodeStepTokens) * stt;
        } else {
            return (int64_t)b * s0 + (int64_t)hk * sh + (int64_t)j * stt;
        }
    };

    // Loads of one step: K straight into score-operand layout (lane c, g of
    // row block rb holds token 16*rb + c, head-dim values DQ*g + 8*ks ..),
    // V as coalesced 16-byte row pieces.  Tokens past t1 re-read token t1-1
    // and tokens before the window start tb re-read token tb, so nothing
    // outside the row's window is read (a page that lies wholly before the
    // window supplies no address).
    auto issue_k = [&](int st, const Pages &pg, uint4 (&kr)[2][KS]) {
        const int base = t0 + st * kMfmaStep;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const int j = max(tb, min(base + 16 * rb + c, t1 - 1));
            const int64_t off = tok_off(j, base, pg, p.k_s0, p.k_sh, p.k_st) + DQ * g;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kr[rb][ks] = load16(kc + off + 8 * ks);
        }
    };
    auto issue_v = [&](int st, const Pages &pg, uint4 (&vr)[VLD]) {
        const int base = t0 + st * kMfmaStep;
#pragma unroll
        for (int u = 0; u < VLD; ++u) {
            const int j = max(tb, min(base + RPL * u + lane / LPR, t1 - 1));
            vr[u] = load16(vc + tok_off(j, base, pg, p.v_s0, p.v_sh, p.v_st) + 8 * (lane % LPR));
        }
    };

    // the first step's loads go out before the query-side setup below
    uint4 kr[2][KS], vr[VLD];
    Pages pg_next = {0, 0};
    if (wave < nsteps) {
        const Pages pg = step_pages(wave);
        issue_k(wave, pg, kr);
        issue_v(wave, pg, vr);
        if (wave + kMfmaWaves < nsteps) pg_next = step_pages(wave + kMfmaWaves);
    }

    // ---- score-side operands: column c of set s is q or rho of head
    // hk*G + s*HS + c%HS, its bf16 hi part (c < 2*HS) or lo part; head-dim
    // value d = DQ*g + 8*ks + i sits in k-slot 8*g + i of score MFMA ks.
    const int which = c / HS;  // 0 q hi, 1 rho hi, 2 q lo, 3 rho lo, >= 4 unused
    bf16x8_t bq[NCS][KS];
#pragma unroll
    for (int s = 0; s < NCS; ++s) {
        const int head = hk * G + s * HS + (c % HS);
        const bool is_rho = which & 1;
        const float *src = is_rho ? p.rho + b * p.rho_sb + (int64_t)head * p.rho_sh
                                  : p.q + b * p.q_sb + (int64_t)head * p.q_sh;
        const float mul = is_rho ? 1.0f : p.scale_log2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float x[8];
            if (which < 4) {
                const float4 a = *reinterpret_cast<const float4 *>(src + DQ * g + 8 * ks);
                const float4 e = *reinterpret_cast<const float4 *>(src + DQ * g + 8 * ks + 4);
                x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
                x[4] = e.x; x[5] = e.y; x[6] = e.z; x[7] = e.w;
            } else {
                for (int i = 0; i < 8; ++i) x[i] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float v = x[i] * mul;
                const __bf16 hi = (__bf16)v;
                bq[s][ks][i] = which < 2 ? hi : (__bf16)(v - (float)hi);
            }
        }
    }

    unsigned char *vt = vtile[wave];

    auto process = [&](int st, int nst, uint4 (&kr)[2][KS], uint4 (&vr)[VLD]) {
        const int base = t0 + st * kMfmaStep;
        const Pages pg = pg_next;  // pages of step nst
        if (nst >= 0 && nst + kMfmaWaves < nsteps) pg_next = step_pages(nst + kMfmaWaves);
        // V rows into the wave's LDS tile (row-major, padded rows)
#pragma unroll
        for (int u = 0; u < VLD; ++u)
            *reinterpret_cast<uint4 *>(vt + (RPL * u + lane / LPR) * VROW + 16 * (lane % LPR)) =
                vr[u];
        if (nst >= 0) issue_v(nst, pg, vr);

        // scores: d1[s][rb] lane (c, g) = column c, tokens 16*rb + 4*g + j
        f32x4_t d1[NCS][2];
#pragma unroll
        for (int s = 0; s < NCS; ++s)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, kr[rb][ks]), bq[s][ks], a, 0, 0, 0);
                d1[s][rb] = a;
            }
        if (nst >= 0) issue_k(nst, pg, kr);

        // k-slot r (0..7) of this lane's group <-> token of the step
        bool valid[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int tok = base + (r < 4 ? 4 * g + r : 16 + 4 * g + r - 4);
            valid[r] = tok < t1 && tok >= tb;
        }

        bf16x8_t pw[NCS];
#pragma unroll
        for (int s = 0; s < NCS; ++s) {
            float y[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float x = r < 4 ? d1[s][0][r] : d1[s][1][r - 4];
                y[r] = x + row_shl<2 * HS>(x);  // hi + lo columns: lanes c < HS hold s, next HS hold t
            }
            // step max of each head's logits (lanes c < HS), over all 4 groups
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 8; ++r) mx = fmaxf(mx, valid[r] ? y[r] : -INFINITY);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            bool moved = false;
            float alpha[HS];
#pragma unroll
            for (int h = 0; h < HS; ++h) {
                const float tm = read_lane(mx, h);
                alpha[h] = 1.0f;
                if (tm > mref[s][h] + kRescaleSlack) {  // wave-uniform
                    alpha[h] = __builtin_amdgcn_exp2f(mref[s][h] - tm);
                    mref[s][h] = tm;
                    moved = true;
                }
            }
            float m_lane = mref[s][0];
#pragma unroll
            for (int h = 1; h < HS; ++h) m_lane = (c % HS) == h ? mref[s][h] : m_lane;
            if (moved) {  // rescale the sums of every column of a moved head
                float al = alpha[0];
#pragma unroll
                for (int h = 1; h < HS; ++h) al = (c % HS) == h ? alpha[h] : al;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[s][db] *= al;
                ztot[s] *= al;
            }
            // weights and probe-weighted weights, split into bf16 hi + lo
            uint32_t opw[4];
            float colsum = 0.f;
#pragma unroll
            for (int r = 0; r < 8; r += 2) {
                float full[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float w = valid[r + q] ? __builtin_amdgcn_exp2f(y[r + q] - m_lane) : 0.f;
                    const float wt = w * row_shl<HS>(y[r + q]);  // t of head c sits HS lanes up
                    const float wt_here = row_shr<HS>(wt);        // lanes HS..2HS-1 take it
                    full[q] = c < HS ? w : (c < 2 * HS ? wt_here : 0.f);
                }
                const uint32_t hi = pack_bf16x2(full[0], full[1]);
                const uint32_t lo =
                    pack_bf16x2(full[0] - bf16_lo(hi), full[1] - bf16_hi(hi));
                const uint32_t lo_here = row_shr_u<2 * HS>(lo);  // lo parts move 2*HS lanes up
                const uint32_t o = c < 2 * HS ? hi : (c < 4 * HS ? lo_here : 0u);
                opw[r / 2] = o;
                colsum += bf16_lo(o) + bf16_hi(o);
            }
            ztot[s] += colsum;
            pw[s] = __builtin_bit_cast(bf16x8_t, uint4{opw[0], opw[1], opw[2], opw[3]});
        }

        // value sums: V^T operand rows d = 16*db + c, k-slots as above, read
        // transposed out of the LDS tile (4 tokens x 16 head-dim values per read)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
            const int col = 16 * db + 4 * (c % 4);
            const unsigned char *a0 = vt + (4 * g + c / 4) * VROW + 2 * col;
            const unsigned char *a1 = vt + (16 + 4 * g + c / 4) * VROW + 2 * col;
            const i16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(__attribute__((address_space(3))) unsigned char *)a0);
            const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(__attribute__((address_space(3))) unsigned char *)a1);
            const bf16x8_t vop = __builtin_bit_cast(
                bf16x8_t, (short __attribute__((ext_vector_type(8)))){lo4[0], lo4[1], lo4[2], lo4[3],
                                                                      hi4[0], hi4[1], hi4[2], hi4[3]});
#pragma unroll
            for (int s = 0; s < NCS; ++s)
                acc[s][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pw[s], acc[s][db], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // One register buffer per operand: the next step's V loads start as soon
    // as this step's V rows are in LDS, its K loads as soon as the score
    // MFMAs have consumed K; the other waves of the CU cover the latency.
    {
        int st = wave;
        while (st < nsteps) {
            const int nst = st + kMfmaWaves;
            process(st, nst < nsteps ? nst : -1, kr, vr);
            st = nst;
        }
    }

    // ---- this wave's record per head: hi + lo columns summed
#pragma unroll
    for (int s = 0; s < NCS; ++s) {
        float zr = ztot[s] + row_shl<2 * HS>(ztot[s]);
        zr += __shfl_xor(zr, 16);
        zr += __shfl_xor(zr, 32);
        const int head = s * HS + (c % HS);
        float *rec = red[wave][head];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = acc[s][db][j] + row_shl<2 * HS>(acc[s][db][j]);
                const int d = 16 * db + 4 * g + j;
                if (c < HS) rec[d] = v;               // A
                else if (c < 2 * HS) rec[D + d] = v;  // B
            }
        if (g == 0 && c < HS) {
            float m_lane = mref[s][0];
            for (int h = 1; h < HS; ++h) m_lane = c == h ? mref[s][h] : m_lane;
            rec[2 * D] = m_lane;
            rec[2 * D + 1] = zr;
        } else if (g == 0 && c < 2 * HS) {
            rec[2 * D + 2] = zr;
        }
    }
    __syncthreads();
    finish_block<D, G, kMfmaWaves>(p, red, b, hk, unit, split_idx, nsp);
}

// ============================================================ fp32: VALU ===

constexpr int kValuWaves = 4;

template <int D, int G, bool PAGED>
__global__ __launch_bounds__(64 * kValuWaves) void decode_valu_kernel(DecodeParams p) {
    constexpr int VEC = 4;                          // fp32 values per 16-byte load
    constexpr int LPT = D / VEC;                    // lanes per token row
    constexpr int TPL = 64 / LPT;                   // token rows per wave-wide load
    constexpr int U = kDecodeStepTokens / TPL;      // loads per 16-token step
    constexpr int REC = partial_floats(D);
    static_assert(LPT == 16 || LPT == 32, "fp32 rows of 64 or 128 values");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = lane / LPT;
    const int sub = lane % LPT;

    const int units = gridDim.x / p.nsplit;
    const int split_idx = blockIdx.x / units;  // split-major order
    const int unit = blockIdx.x % units;
    const int b = unit / p.num_kv_heads;
    const int hk = unit % p.num_kv_heads;
    int L, tb, tbase, nsp;
    row_extent<PAGED>(p, b, L, tb, tbase, nsp);
    if (split_idx >= nsp) return;
    const int t0 = tbase + split_idx * p.split;
    const int t1 = min(L, t0 + p.split);
    const int nsteps = (t1 - t0 + kDecodeStepTokens - 1) / kDecodeStepTokens;

    float qv[G][VEC], rv[G][VEC];
    for (int h = 0; h < G; ++h) {
        const float4 a = *reinterpret_cast<const float4 *>(
            p.q + b * p.q_sb + (int64_t)(hk * G + h) * p.q_sh + sub * VEC);
        const float4 e = *reinterpret_cast<const float4 *>(
            p.rho + b * p.rho_sb + (int64_t)(hk * G + h) * p.rho_sh + sub * VEC);
        qv[h][0] = a.x * p.scale_log2; qv[h][1] = a.y * p.scale_log2;
        qv[h][2] = a.z * p.scale_log2; qv[h][3] = a.w * p.scale_log2;
        rv[h][0] = e.x; rv[h][1] = e.y; rv[h][2] = e.z; rv[h][3] = e.w;
    }
    float m[G], Z[G], R[G], A[G][VEC], B[G][VEC];
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        Z[h] = R[h] = 0.f;
        for (int e = 0; e < VEC; ++e) A[h][e] = B[h][e] = 0.f;
    }

    const float *kc = static_cast<const float *>(p.k);
    const float *vc = static_cast<const float *>(p.v);
    for (int st = wave; st < nsteps; st += kValuWaves) {
        const int base = t0 + st * kDecodeStepTokens;
        if (base + kDecodeStepTokens <= tb) continue;  // step wholly before the window
        int64_t kb, vb;
        if constexpr (PAGED) {
            const int pg = p.block_table[(int64_t)b * p.max_blocks + base / kDecodeStepTokens];
            kb = (int64_t)pg * p.k_s0 + (int64_t)hk * p.k_sh - (int64_t)base * p.k_st;
            vb = (int64_t)pg * p.v_s0 + (int64_t)hk * p.v_sh - (int64_t)base * p.v_st;
        } else {
            kb = (int64_t)b * p.k_s0 + (int64_t)hk * p.k_sh;
            vb = (int64_t)b * p.v_s0 + (int64_t)hk * p.v_sh;
        }
        uint4 kw[U], vw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // rows past t1 re-read t1-1, rows before the window re-read tb
            const int j = max(tb, min(base + u * TPL + row, t1 - 1));
            kw[u] = load16(kc + kb + (int64_t)j * p.k_st + sub * VEC);
            vw[u] = load16(vc + vb + (int64_t)j * p.v_st + sub * VEC);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tok = base + u * TPL + row;
            const bool valid = tok < t1 && tok >= tb;
            const float kf[4] = {__uint_as_float(kw[u].x), __uint_as_float(kw[u].y),
                                 __uint_as_float(kw[u].z), __uint_as_float(kw[u].w)};
            const float vf[4] = {__uint_as_float(vw[u].x), __uint_as_float(vw[u].y),
                                 __uint_as_float(vw[u].z), __uint_as_float(vw[u].w)};
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float s = qv[h][0] * kf[0], t = rv[h][0] * kf[0];
#pragma unroll
                for (int e = 1; e < VEC; ++e) {
                    s = fmaf(qv[h][e], kf[e], s);
                    t = fmaf(rv[h][e], kf[e], t);
                }
                // butterfly sums over the row's lanes: partners add in swapped
                // order, so every lane of a row ends with the same bits
                s += dpp_f<0xB1>(s); t += dpp_f<0xB1>(t);    // quad_perm [1,0,3,2]
                s += dpp_f<0x4E>(s); t += dpp_f<0x4E>(t);    // quad_perm [2,3,0,1]
                s += dpp_f<0x141>(s); t += dpp_f<0x141>(t);  // row_half_mirror
                s += dpp_f<0x140>(s); t += dpp_f<0x140>(t);  // row_mirror
                if constexpr (LPT == 32) {
                    s += __shfl_xor(s, 16);
                    t += __shfl_xor(t, 16);
                }
                s = valid ? s : -INFINITY;
                if (s > m[h] + kRescaleSlack) {
                    const float al = __builtin_amdgcn_exp2f(m[h] - s);
                    Z[h] *= al; R[h] *= al;
                    for (int e = 0; e < VEC; ++e) { A[h][e] *= al; B[h][e] *= al; }
                    m[h] = s;
                }
                const float w = valid ? __builtin_amdgcn_exp2f(s - m[h]) : 0.f;
                const float wt = w * t;
                Z[h] += w;
                R[h] += wt;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    A[h][e] = fmaf(w, vf[e], A[h][e]);
                    B[h][e] = fmaf(wt, vf[e], B[h][e]);
                }
            }
        }
    }

    // merge the token rows of this wave, then the waves through LDS
    for (int off = LPT; off < 64; off *= 2)
        for (int h = 0; h < G; ++h) {
            const float m2 = __shfl_xor(m[h], off), Z2 = __shfl_xor(Z[h], off),
                        R2 = __shfl_xor(R[h], off);
            const float mn = fmaxf(m[h], m2);
            const float a1 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[h] - mn);
            const float a2 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
            Z[h] = a1 * Z[h] + a2 * Z2;
            R[h] = a1 * R[h] + a2 * R2;
            for (int e = 0; e < VEC; ++e) {
                const float A2 = __shfl_xor(A[h][e], off), B2 = __shfl_xor(B[h][e], off);
                A[h][e] = a1 * A[h][e] + a2 * A2;
                B[h][e] = a1 * B[h][e] + a2 * B2;
            }
            m[h] = mn;
        }
    __shared__ float red[kValuWaves][G][REC];
    if (row == 0)
        for (int h = 0; h < G; ++h) {
            for (int e = 0; e < VEC; ++e) {
                red[wave][h][sub * VEC + e] = A[h][e];
                red[wave][h][D + sub * VEC + e] = B[h][e];
            }
            if (sub == 0) {
                red[wave][h][2 * D] = m[h];
                red[wave][h][2 * D + 1] = Z[h];
                red[wave][h][2 * D + 2] = R[h];
            }
        }
    __syncthreads();
    finish_block<D, G, kValuWaves>(p, red, b, hk, unit, split_idx, nsp);
}

// ================================================================ merge ===

// One workgroup per (batch, KV head): combine the split records of rows
// that used more than one split and write o.  LLA: the decode is a sweep of
// the solved probe's conjugate gradients (keys as values, rho = the search
// direction); the rows' outputs stay in LDS (a single-split unit's are read
// back from where the split kernel wrote them) and one wave per row runs the
// step right away, for every unit, saving a launch per iteration.
template <int D, int G, bool PAGED, bool LLA>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p, LlaParams lq) {
    constexpr int REC = partial_floats(D);
    // LLA: the rows' sweep outputs stay here for the conjugate-gradient step
    __shared__ float osh[LLA ? G : 1][D];
    const int unit = blockIdx.x;
    const int b = unit / p.num_kv_heads;
    const int hk = unit % p.num_kv_heads;
    int L, tb, tbase, nsp;
    row_extent<PAGED>(p, b, L, tb, tbase, nsp);
    if (nsp <= 1) {  // written by the split kernel
        if constexpr (!LLA) return;
        for (int idx = threadIdx.x; idx < G * D; idx += 256)
            osh[idx / D][idx % D] =
                p.out[b * p.out_sb + (int64_t)(hk * G + idx / D) * p.out_sh + idx % D];
    } else {
        const float *recs = p.partials + (int64_t)unit * p.nsplit * G * REC;
        for (int idx = threadIdx.x; idx < G * D; idx += 256) {
            const int g = idx / D, e = idx % D;
            const float o = merge_records<D, G, false>(recs, nsp, g, e);
            if constexpr (LLA) osh[g][e] = o;
            else p.out[b * p.out_sb + (int64_t)(hk * G + g) * p.out_sh + e] = o;
        }
    }
    if constexpr (LLA) {
        __syncthreads();
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        for (int g = wave; g < G; g += 4)
            lla_step_row(lq, (int64_t)b * lq.num_q_heads + hk * G + g, true, lane, osh[g]);
    }
}

template <int D, int G, bool PAGED>
hipError_t launch_all(const DecodeParams &p, bool bf16, int batch, hipStream_t stream,
                      const LlaParams *lla) {
    // Workgroup w takes split w / units of unit w % units.  Consecutive
    // workgroups are dealt round-robin to the eight XCDs, so in this order
    // every XCD gets every eighth unit with all of its splits; in unit-major
    // order each XCD would get fixed split indices, and with ragged rows the
    // high ones are mostly empty, leaving XCDs idle.
    const unsigned units = (unsigned)((int64_t)batch * p.num_kv_heads);
    const dim3 grid((unsigned)((int64_t)units * p.nsplit));
    if (bf16) {
        constexpr int NWMAX = mfma_waves_max<D, G>();
        // tokens a row's splits cover at most (as the host sized the split)
        const int span = p.window > 0 && p.window < p.max_seq_len - (kWindowAlign - 1)
                             ? p.window + kWindowAlign - 1
                             : p.max_seq_len;
        const int steps = (min(p.split, span) + kMfmaStep - 1) / kMfmaStep;
        if (NWMAX == 8 && steps > kShortSteps && grid.x <= (unsigned)kDeviceCUs)
            hipLaunchKernelGGL((decode_mfma_kernel<D, G, PAGED, NWMAX>), grid, dim3(64 * NWMAX), 0,
                               stream, p);
        else
            hipLaunchKernelGGL((decode_mfma_kernel<D, G, PAGED, 4>), grid, dim3(64 * 4), 0, stream,
                               p);
    } else
        hipLaunchKernelGGL((decode_valu_kernel<D, G, PAGED>), grid, dim3(64 * kValuWaves), 0,
                           stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (lla != nullptr)
        hipLaunchKernelGGL((decode_merge_kernel<D, G, PAGED, true>), dim3(units), dim3(256), 0,
                           stream, p, *lla);
    else if (p.nsplit > 1 && p.arrivals == nullptr)
        hipLaunchKernelGGL((decode_merge_kernel<D, G, PAGED, false>), dim3(units), dim3(256), 0,
                           stream, p, LlaParams{});
    return hipGetLastError();
}

template <int D, int G>
hipError_t launch_g(const DecodeParams &p, bool bf16, bool paged, int batch, hipStream_t s,
                    const LlaParams *lla) {
    return paged ? launch_all<D, G, true>(p, bf16, batch, s, lla)
                 : launch_all<D, G, false>(p, bf16, batch, s, lla);
}

template <int D>
hipError_t launch_d(const DecodeParams &p, bool bf16, int group, bool paged, int batch,
                    hipStream_t s, const LlaParams *lla) {
    switch (group) {
        case 1: return launch_g<D, 1>(p, bf16, paged, batch, s, lla);
        case 2: return launch_g<D, 2>(p, bf16, paged, batch, s, lla);
        case 4: return launch_g<D, 4>(p, bf16, paged, batch, s, lla);
        case 8: return launch_g<D, 8>(p, bf16, paged, batch, s, lla);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int kv_dtype, int d, int group, bool paged,
                         int batch, hipStream_t stream, const LlaParams *lla) {
    const bool bf16 = kv_dtype == 1;
    if (d == 128) return launch_d<128>(p, bf16, group, paged, batch, stream, lla);
    if (d == 64) return launch_d<64>(p, bf16, group, paged, batch, stream, lla);
    return hipErrorInvalidValue;
}

}  // namespace plx
