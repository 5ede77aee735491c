// prefill_bwd.hip -- backward pass of causal Parallax prefill for gfx950
// (CDNA4), bf16 matrix cores.
//
// Forward, per query row i (page "Parallax: Parameterized Local Linear
// Attention Gives Transformers a 'Second Eye'", section 1.3):
//   s_j = scale q.k_j, p = softmax(s), t_j = rho.k_j,
//   a = sum p_j v_j, r = sum p_j t_j, b = sum p_j t_j v_j, o = a - b + a r.
// With g = dL/do, c = a.g and u_j = g.v_j the chain rule gives
//   dL/dv_j += p_j (1 + r - t_j) g
//   dL/dp_j  = u_j (1 + r - t_j) + c t_j,   sum_j p_j dL/dp_j = g.o + r c =: D
//   dL/ds_j  = p_j (dL/dp_j - D)            (softmax)
//   dL/dt_j  = p_j (c - u_j)
//   dq = scale sum_j ds_j k_j,  drho = sum_j dt_j k_j,
//   dk_j += scale ds_j q + dt_j rho          (summed over rows and GQA heads)
// The forward pass keeps, per row, lse = log sum_j e^{s_j}, r and a; then
// p_j = e^{s_j - lse} is recomputed exactly, with no running max.
//
// Three kernels, all deterministic (fixed summation order, no atomics):
//   prep  one 16-lane group per row: c = a.g and D = g.o + r c, stored with
//         lse * log2(e) and 1 + r as one float4 per row (the workspace);
//   dq    query-major, the forward's structure: a workgroup holds 128 query
//         rows of the G heads of one KV head, 32-key K/V tiles stream through
//         LDS.  Score wave p recomputes S^T = K Q^T, T^T = K rho^T and
//         U^T = V dout^T (keys x queries) and forms dS^T, dT^T in bf16; value
//         wave p + 4 accumulates dq^T += K^T dS^T and drho^T += K^T dT^T (K^T
//         through ds_read_b64_tr_b16), one tile behind.
//   dkv   key-major, the same pair structure with roles swapped: a workgroup
//         holds 128 keys of one KV head (32 per pair, K and V resident in the
//         score wave), and 32-row tiles of q, rho and dout of every query head
//         of the group stream through LDS.  Score wave: S = Q K^T, T = rho K^T,
//         U = dout V^T (queries x keys), then W = p (1 + r - t), scale dS and
//         dT in bf16; value wave: dv^T += dout^T W, dk^T += q^T dS + rho^T dT.
// Tiles read by both roles live two epochs (score wave in epoch t, value
// wave in epoch t + 1), so they are triple-buffered in LDS; each epoch ends
// with one barrier.  The value waves, whose MFMAs end early in the epoch, do
// all the staging (global loads into registers, then LDS stores), so the
// score waves' MFMA and VALU work is the epoch's critical path: dq runs the
// loads two tiles ahead through two register stages, dkv (more registers
// live in its value waves) one tile ahead through one stage, stored at the
// start of the next epoch.  Loads are issued unconditionally so the
// compiler's wait counts stay exact.
#include "kernels.hpp"

#include <math.h>

#include <type_traits>

namespace plx {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBwPairs = 4;                 // score/value wave pairs per workgroup
constexpr int kBwRows = 32;                 // query rows (dq) or keys (dkv) per pair
constexpr int kBwTile = 32;                 // rows of a streamed tile
// LDS bytes per tile row (head dim D = 64 or 128).  Tiles here are read both
// row-wise (16 bytes per lane) and transposed (ds_read_b64_tr_b16, 8 bytes
// per lane); a 32-byte pad keeps the transposed reads conflict free (the
// row-wise reads then pair up on banks).  Measured alternatives at D = 128: a
// 16-byte pad, and an XOR swizzle that is conflict free for both patterns,
// ran within 1% (the swizzle's address arithmetic cost what its
// conflict-free reads saved).
template <int D>
constexpr int bw_row_bytes() { return 2 * D + 32; }
template <int D>
constexpr int bw_tile_bytes() { return kBwTile * bw_row_bytes<D>(); }
// One thread's piece of a tile row (16 per row): 16 bytes at D = 128, 8 at 64.
template <int D>
using BwPiece = std::conditional_t<D == 128, uint4, uint2>;
template <int D>
__device__ __forceinline__ BwPiece<D> ldp(const uint16_t *p) {
    return *reinterpret_cast<const BwPiece<D> *>(p);
}

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xffff0000u);
}

// Byte offset of triple-buffer slot t % 3.  Passed through readfirstlane so
// the loop optimizer treats it as an opaque value: otherwise it turns every
// LDS address derived from it into an induction variable of its own, which
// costs dozens of registers.
template <int D>
__device__ __forceinline__ int slot3(int t) {
    return __builtin_amdgcn_readfirstlane((t % 3) * bw_tile_bytes<D>());
}

__device__ __forceinline__ f32x4_t mfma(const bf16x8_t &a, const bf16x8_t &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A operand of a 16x16x32 MFMA holding the transpose of a 32-row LDS tile:
// row 16db + (lane % 16) of the result is head-dim column 16db + lane % 16
// of the tile, k-slot r is tile row 4g + r (r < 4) or 16 + 4g + r - 4.
template <int D>
__device__ __forceinline__ bf16x8_t tr_operand(const unsigned char *tile, int db, int c, int g) {
    typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
    constexpr int RB = bw_row_bytes<D>();
    const int col = 16 * db + 4 * (c % 4);
    const unsigned char *a0 = tile + (4 * g + c / 4) * RB + 2 * col;
    const unsigned char *a1 = tile + (16 + 4 * g + c / 4) * RB + 2 * col;
    const i16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)(__attribute__((address_space(3))) unsigned char *)a0);
    const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)(__attribute__((address_space(3))) unsigned char *)a1);
    return __builtin_bit_cast(
        bf16x8_t, i16x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]});
}

// ------------------------------------------------------------------ prep ---
// 16 lanes per row, EL = D / 16 head-dim values each.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(PrefillBwdParams p) {
    constexpr int EL = D / 16;
    const int64_t rows = (int64_t)p.batch * p.num_q_heads * p.seq_len;
    const int64_t u = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;
    const int part = threadIdx.x % 16;
    const int64_t uu = u < rows ? u : rows - 1;
    const int i = (int)(uu % p.seq_len);
    const int h = (int)((uu / p.seq_len) % p.num_q_heads);
    const int b = (int)(uu / ((int64_t)p.seq_len * p.num_q_heads));
    const BwPiece<D> gw = ldp<D>(p.dout + (int64_t)b * p.g_sb + (int64_t)i * p.g_ss +
                                 (int64_t)h * p.g_sh + EL * part);
    const uint32_t *gwords = reinterpret_cast<const uint32_t *>(&gw);
    const int64_t ooff = (int64_t)b * p.o_sb + (int64_t)i * p.o_ss + (int64_t)h * p.o_sh + EL * part;
    float ca = 0.f, go = 0.f;
#pragma unroll
    for (int e4 = 0; e4 < EL / 4; ++e4) {
        const float4 o = *reinterpret_cast<const float4 *>(p.out + ooff + 4 * e4);
        const float4 a = *reinterpret_cast<const float4 *>(p.o_sa + ooff + 4 * e4);
        const float gv[4] = {bf16_lo(gwords[2 * e4]), bf16_hi(gwords[2 * e4]),
                             bf16_lo(gwords[2 * e4 + 1]), bf16_hi(gwords[2 * e4 + 1])};
        const float ov[4] = {o.x, o.y, o.z, o.w};
        const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ca = fmaf(av[e], gv[e], ca);
            go = fmaf(ov[e], gv[e], go);
        }
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) {
        ca += __shfl_xor(ca, m, 16);
        go += __shfl_xor(go, m, 16);
    }
    if (u < rows && part == 0) {
        const float r = p.rmean[uu];
        p.rowstat[uu] = float4{p.lse[uu] * 1.4426950408889634f, 1.0f + r, ca, fmaf(r, ca, go)};
    }
}

// -------------------------------------------------------------------- dq ---
template <int D, int G, bool WIN>
__global__ __launch_bounds__(128 * kBwPairs) void bwd_dq_kernel(PrefillBwdParams p) {
    constexpr int KS = D / 32;             // score MFMAs per 16-key block
    constexpr int DB = D / 16;             // 16-row blocks of the gradient sums
    constexpr int DQ = D / 4;              // head-dim values per lane group (scores)
    constexpr int RB = bw_row_bytes<D>(), TB = bw_tile_bytes<D>();
    constexpr int PE = D / 16;             // elements per tile piece
    constexpr int PPH = kBwPairs / G;      // pairs per query head
    constexpr int QB = kBwRows * PPH;      // query rows per head per workgroup

    __shared__ __attribute__((aligned(16))) unsigned char ktile[3 * TB];
    __shared__ __attribute__((aligned(16))) unsigned char vtile[2][TB];
    __shared__ uint4 pbuf[2][kBwPairs][4][64];  // dS^T (qc 0, 1), dT^T (qc 0, 1), B-operand layout

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int S = p.seq_len;
    const float c2 = p.scale_log2;
    const bool score_wave = wave < kBwPairs;
    const int pair = wave % kBwPairs;

    const int nhb = p.num_kv_heads * p.head_blocks;  // blocks of G query heads
    const int units = p.batch * nhb;
    const int nqb = (S + QB - 1) / QB;
    const int qb = nqb - 1 - (int)(blockIdx.x / units);  // longest causal rows first
    const int unit = blockIdx.x % units;
    const int b = unit / nhb;
    const int hb = unit % nhb;
    const int hk = hb / p.head_blocks;  // the KV head of query heads hb*G .. hb*G + G - 1
    const int head = hb * G + pair / PPH;
    const int r0 = qb * QB + (pair % PPH) * kBwRows;  // first query row of this pair
    const int key_end = min(S, (qb + 1) * QB);
    const int ntiles = (key_end + kBwTile - 1) / kBwTile;
    const int pair_tiles = min(ntiles, (min(S, r0 + kBwRows) + kBwTile - 1) / kBwTile);
    const int W = WIN ? p.window : 0;
    const int t_first = (W > 0 ? max(0, qb * QB - W + 1) / kBwTile : 0) & ~1;
    const int pair_lo = W > 0 ? max(0, r0 - W + 1) / kBwTile : 0;

    const uint16_t *kg = p.k + (int64_t)b * p.k_sb + (int64_t)hk * p.k_sh;
    const uint16_t *vg = p.v + (int64_t)b * p.v_sb + (int64_t)hk * p.v_sh;
    // Staging, value waves only: thread tv takes keys rv and rv + 16 of a
    // tile, 16-byte piece cv of each row.
    const int tv = tid - 64 * kBwPairs;
    const int rv = (tv >> 4) & 15, cv = tv & 15;
    const int64_t ko = (int64_t)rv * p.k_ss + PE * cv, vo = (int64_t)rv * p.v_ss + PE * cv;
    struct Stage {
        BwPiece<D> k[2], v[2];
    } kst[2];  // tile j in stage j & 1
    auto issue = [&](int t, Stage &st) {
        const int key0 = min(t * kBwTile, S - 1);
        const uint16_t *ks_ = kg + (int64_t)key0 * p.k_ss;
        const uint16_t *vs_ = vg + (int64_t)key0 * p.v_ss;
        if (key0 + kBwTile <= S) {
            st.k[0] = ldp<D>(ks_ + ko);
            st.v[0] = ldp<D>(vs_ + vo);
            st.k[1] = ldp<D>(ks_ + 16 * p.k_ss + ko);
            st.v[1] = ldp<D>(vs_ + 16 * p.v_ss + vo);
        } else {  // a ragged last tile: keys past the end read key S - 1
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int kk = min(rv + 16 * i, S - 1 - key0);
                st.k[i] = ldp<D>(ks_ + (int64_t)kk * p.k_ss + PE * cv);
                st.v[i] = ldp<D>(vs_ + (int64_t)kk * p.v_ss + PE * cv);
            }
        }
    };
    auto store = [&](unsigned char *kt, unsigned char *vt, const Stage &st) {
        using P = BwPiece<D>;
        const int off = rv * RB + 2 * PE * cv;
        *reinterpret_cast<P *>(kt + off) = st.k[0];
        *reinterpret_cast<P *>(kt + off + 16 * RB) = st.k[1];
        *reinterpret_cast<P *>(vt + off) = st.v[0];
        *reinterpret_cast<P *>(vt + off + 16 * RB) = st.v[1];
    };
    // End of epoch t: K and V tile t + 1 go to LDS (K buffer (t+1) % 3 last
    // held tile t - 2, read by the value waves in epoch t - 1; V buffer
    // (t+1) & 1 held tile t - 1, read by the score waves in epoch t - 1), and
    // their register stage takes the loads of tile t + 3.
    auto advance = [&](int t, auto par) {
        constexpr int P = decltype(par)::value;
        store(ktile + slot3<D>(t + 1), vtile[1 - P], kst[1 - P]);
        issue(t + 3, kst[1 - P]);
        __syncthreads();
    };
    auto prologue = [&] {
        issue(t_first, kst[0]);
        store(ktile + slot3<D>(t_first), vtile[0], kst[0]);
        issue(t_first + 1, kst[1]);
        issue(t_first + 2, kst[0]);
        __syncthreads();
    };

    if (score_wave) {
        // Query-side B operands: column c of block cb is q row r0 + 16cb + c
        // (cb < 2) or the rho row of the same query (cb >= 2); gop[qc] holds
        // the dout rows.  Head-dim value 32g + 8ks + i sits in k-slot 8g + i of
        // MFMA ks, the slots the K and V A-operands use.
        bf16x8_t xop[4][KS], gop[2][KS];
        float4 st[2];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int row = min(r0 + 16 * (cb & 1) + c, S - 1);
            const uint16_t *src = cb < 2 ? p.q + (int64_t)b * p.q_sb + (int64_t)row * p.q_ss +
                                               (int64_t)head * p.q_sh
                                         : p.rho + (int64_t)b * p.r_sb + (int64_t)row * p.r_ss +
                                               (int64_t)head * p.r_sh;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                xop[cb][ks] = __builtin_bit_cast(bf16x8_t, ld16(src + DQ * g + 8 * ks));
        }
#pragma unroll
        for (int qc = 0; qc < 2; ++qc) {
            const int row = min(r0 + 16 * qc + c, S - 1);
            const uint16_t *src =
                p.dout + (int64_t)b * p.g_sb + (int64_t)row * p.g_ss + (int64_t)head * p.g_sh;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                gop[qc][ks] = __builtin_bit_cast(bf16x8_t, ld16(src + DQ * g + 8 * ks));
            st[qc] = p.rowstat[((int64_t)b * p.num_q_heads + head) * S + row];
        }

        // d1[rb][cb]: lane (c, g) = query column c of block cb, keys
        // 32t + 16rb + 4g + j; du[rb][qc] the same for U^T.
        auto scores = [&](int t, f32x4_t (&d1)[2][4], f32x4_t (&du)[2][2]) {
            const unsigned char *kt = ktile + slot3<D>(t);
            const unsigned char *vt = vtile[t & 1];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) d1[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                du[rb][0] = du[rb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                // the half's K and V operands are all read before its MFMAs
                // (one LDS latency per half, not one per pair of reads)
                bf16x8_t kop[KS], vop[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    kop[ks] = __builtin_bit_cast(
                        bf16x8_t, ld16(kt + (16 * rb + c) * RB + 2 * DQ * g + 16 * ks));
                    vop[ks] = __builtin_bit_cast(
                        bf16x8_t, ld16(vt + (16 * rb + c) * RB + 2 * DQ * g + 16 * ks));
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb)
                        d1[rb][cb] = mfma(kop[ks], xop[cb][ks], d1[rb][cb]);
#pragma unroll
                    for (int qc = 0; qc < 2; ++qc)
                        du[rb][qc] = mfma(vop[ks], gop[qc][ks], du[rb][qc]);
                }
            }
        };
        // dS^T and dT^T of tile t in bf16, as B operands of the value MFMAs
        // (k-slot r holds key 4g + r for r < 4, else 16 + 4g + r - 4).
        auto grads = [&](int t, const f32x4_t (&d1)[2][4], const f32x4_t (&du)[2][2],
                         auto mask_tag) {
            constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
            for (int qc = 0; qc < 2; ++qc) {
                const int qi = r0 + 16 * qc + c;
                const float lse2 = st[qc].x, r1 = st[qc].y, cc = st[qc].z, dd = st[qc].w;
                uint32_t sw[4], tw[4];
#pragma unroll
                for (int r = 0; r < 8; r += 2) {
                    float ds2[2], dt2[2];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int rr = r + h2;
                        const float s = rr < 4 ? d1[0][qc][rr] : d1[1][qc][rr - 4];
                        const float tt = rr < 4 ? d1[0][qc + 2][rr] : d1[1][qc + 2][rr - 4];
                        const float uu = rr < 4 ? du[0][qc][rr] : du[1][qc][rr - 4];
                        float pw = __builtin_amdgcn_exp2f(fmaf(s, c2, -lse2));
                        if constexpr (MASK) {
                            const int key = t * kBwTile + (rr < 4 ? 4 * g + rr : 16 + 4 * g + rr - 4);
                            pw = key <= qi && key < S && (W == 0 || key > qi - W) ? pw : 0.0f;
                        }
                        // dL/dp - D = u (1 + r - t) + (c t - D), formed as
                        // (u (1 + r) - D) + t (c - u): c - u is dT's factor too
                        const float cu = cc - uu;
                        ds2[h2] = pw * fmaf(tt, cu, fmaf(uu, r1, -dd));
                        dt2[h2] = pw * cu;
                    }
                    sw[r / 2] = pack_bf16x2(ds2[0], ds2[1]);
                    tw[r / 2] = pack_bf16x2(dt2[0], dt2[1]);
                }
                pbuf[t & 1][pair][qc][lane] = uint4{sw[0], sw[1], sw[2], sw[3]};
                pbuf[t & 1][pair][qc + 2][lane] = uint4{tw[0], tw[1], tw[2], tw[3]};
            }
        };
        auto score_step = [&](int t) {
            if (t >= pair_lo && t < pair_tiles) {
                f32x4_t d1[2][4], du[2][2];
                scores(t, d1, du);
                if (t * kBwTile + kBwTile - 1 <= r0 && t * kBwTile + kBwTile <= S &&
                    (W == 0 || t * kBwTile > r0 + kBwRows - 1 - W))
                    grads(t, d1, du, std::false_type{});
                else
                    grads(t, d1, du, std::true_type{});
            }
        };
        __syncthreads();  // the value waves' prologue
        for (int t = t_first; t <= ntiles; t += 2) {
            score_step(t);
            __syncthreads();
            score_step(t + 1);
            __syncthreads();
        }
    } else {
        // acc[db][cb]: rows d = 16db + 4g + j, column c of block cb (dS^T rows
        // 0-15, 16-31, dT^T rows 0-15, 16-31) -> dq^T (cb < 2), drho^T (cb >= 2)
        f32x4_t acc[DB][4];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) acc[db][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        auto value_tile = [&](int u) {
            bf16x8_t pop[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                pop[cb] = __builtin_bit_cast(bf16x8_t, pbuf[u & 1][pair][cb][lane]);
            const unsigned char *kt = ktile + slot3<D>(u);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8_t kop = tr_operand<D>(kt, db, c, g);
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) acc[db][cb] = mfma(kop, pop[cb], acc[db][cb]);
            }
        };

        prologue();
        for (int t = t_first; t <= ntiles; t += 2) {
            if (t - 1 >= pair_lo && t - 1 < pair_tiles) value_tile(t - 1);
            advance(t, std::integral_constant<int, 0>{});
            if (t >= pair_lo && t < pair_tiles) value_tile(t);
            advance(t + 1, std::integral_constant<int, 1>{});
        }

#pragma unroll
        for (int qc = 0; qc < 2; ++qc) {
            const int qi = r0 + 16 * qc + c;
            if (qi >= S) continue;
            const int64_t off = (int64_t)b * p.dq_sb + (int64_t)qi * p.dq_ss + (int64_t)head * p.dq_sh;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                *reinterpret_cast<float4 *>(p.dq + off + 16 * db + 4 * g) =
                    float4{p.scale * acc[db][qc][0], p.scale * acc[db][qc][1],
                           p.scale * acc[db][qc][2], p.scale * acc[db][qc][3]};
                *reinterpret_cast<float4 *>(p.drho + off + 16 * db + 4 * g) =
                    float4{acc[db][qc + 2][0], acc[db][qc + 2][1], acc[db][qc + 2][2],
                           acc[db][qc + 2][3]};
            }
        }
    }
}

// ------------------------------------------------------------------- dkv ---
template <int D, int G, bool WIN>
__global__ __launch_bounds__(128 * kBwPairs) void bwd_dkv_kernel(PrefillBwdParams p) {
    constexpr int KS = D / 32;
    constexpr int DB = D / 16;
    constexpr int DQ = D / 4;
    constexpr int RB = bw_row_bytes<D>(), TB = bw_tile_bytes<D>();
    constexpr int PE = D / 16;
    constexpr int KB = kBwRows * kBwPairs;  // keys per workgroup

    __shared__ __attribute__((aligned(16))) unsigned char qtile[3 * TB];
    __shared__ __attribute__((aligned(16))) unsigned char rtile[3 * TB];
    __shared__ __attribute__((aligned(16))) unsigned char gtile[3 * TB];
    __shared__ float4 stile[3][kBwTile];          // row statistics of the tile's rows
    __shared__ uint4 pbuf[2][kBwPairs][6][64];    // W, scale dS, dT (key blocks 0, 1)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int S = p.seq_len;
    const float c2 = p.scale_log2;
    const bool score_wave = wave < kBwPairs;
    const int pair = wave % kBwPairs;

    const int units = p.batch * p.num_kv_heads;
    const int kb = (int)(blockIdx.x / units);  // most query rows first
    const int unit = blockIdx.x % units;
    const int b = unit / p.num_kv_heads;
    const int hk = unit % p.num_kv_heads;
    const int k0 = kb * KB;
    const int kp = k0 + pair * kBwRows;  // first key of this pair
    const int W = WIN ? p.window : 0;
    // Query tiles qt_lo .. qt_hi of every head of the group see some key of
    // the workgroup; the stream visits them head by head.
    const int ntq = (S + kBwTile - 1) / kBwTile;
    const int qt_lo = k0 / kBwTile;
    const int qt_hi = W > 0 ? min(ntq - 1, (k0 + KB - 1 + W - 1) / kBwTile) : ntq - 1;
    const int nq = qt_hi - qt_lo + 1;
    const int ntiles = G * nq;
    // this pair's tiles within each head's run (none when its keys are past S)
    const int pq_lo = kp < S ? kp / kBwTile : ntq;
    const int pq_hi = W > 0 ? min(qt_hi, (kp + kBwRows - 1 + W - 1) / kBwTile) : qt_hi;

    auto tile_head = [&](int t) { return hk * G + t / nq; };
    auto tile_qt = [&](int t) { return qt_lo + t % nq; };

    // Staging, value waves only: thread tv takes rows rv and rv + 16 of a
    // tile, piece cv (of 16) of each row, and float se of the tile's 128
    // statistics floats (its 32 rows' float4s are contiguous).  One register
    // stage: tile t + 1, loaded during epoch t - 1, goes to LDS at the start
    // of epoch t (its slot and statistics row last held tile t - 2, read in
    // epoch t - 1); then the stage takes the loads of tile t + 2 (after the
    // value MFMAs of epoch t; at head dim 64 before them).
    const int tv = tid - 64 * kBwPairs;
    const int rv = (tv >> 4) & 15, cv = tv & 15, se = tv & 127;
    const int64_t qo = (int64_t)rv * p.q_ss + PE * cv;
    const int64_t ro = (int64_t)rv * p.r_ss + PE * cv;
    const int64_t go = (int64_t)rv * p.g_ss + PE * cv;
    struct {
        BwPiece<D> q[2], r[2], g[2];
        float s;
    } st;
    auto issue = [&](int t) {
        const int tt = min(t, ntiles - 1);
        const int h = tile_head(tt);
        const int row0 = tile_qt(tt) * kBwTile;
        const uint16_t *qs = p.q + (int64_t)b * p.q_sb + (int64_t)row0 * p.q_ss + (int64_t)h * p.q_sh;
        const uint16_t *rs = p.rho + (int64_t)b * p.r_sb + (int64_t)row0 * p.r_ss + (int64_t)h * p.r_sh;
        const uint16_t *gs = p.dout + (int64_t)b * p.g_sb + (int64_t)row0 * p.g_ss + (int64_t)h * p.g_sh;
        const float *ss = reinterpret_cast<const float *>(p.rowstat + ((int64_t)b * p.num_q_heads + h) * S);
        if (row0 + kBwTile <= S) {
            st.q[0] = ldp<D>(qs + qo);
            st.r[0] = ldp<D>(rs + ro);
            st.g[0] = ldp<D>(gs + go);
            st.q[1] = ldp<D>(qs + 16 * p.q_ss + qo);
            st.r[1] = ldp<D>(rs + 16 * p.r_ss + ro);
            st.g[1] = ldp<D>(gs + 16 * p.g_ss + go);
        } else {  // a ragged last tile: rows past the end read row S - 1
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int64_t rr = min(rv + 16 * i, S - 1 - row0);
                st.q[i] = ldp<D>(qs + rr * p.q_ss + PE * cv);
                st.r[i] = ldp<D>(rs + rr * p.r_ss + PE * cv);
                st.g[i] = ldp<D>(gs + rr * p.g_ss + PE * cv);
            }
        }
        st.s = ss[4 * min(row0 + (se >> 2), S - 1) + (se & 3)];
    };
    auto store = [&](int t) {
        using P = BwPiece<D>;
        const int off = slot3<D>(t) + rv * RB + 2 * PE * cv;
        constexpr int O16 = 16 * RB;
        *reinterpret_cast<P *>(qtile + off) = st.q[0];
        *reinterpret_cast<P *>(rtile + off) = st.r[0];
        *reinterpret_cast<P *>(gtile + off) = st.g[0];
        *reinterpret_cast<P *>(qtile + off + O16) = st.q[1];
        *reinterpret_cast<P *>(rtile + off + O16) = st.r[1];
        *reinterpret_cast<P *>(gtile + off + O16) = st.g[1];
        // threads tv and tv + 128 store the same statistics float: no lane
        // condition, so no branch around a store that waits on a load
        reinterpret_cast<float *>(stile[t % 3])[se] = st.s;
    };
    auto active = [&](int t) {
        if (t < 0 || t >= ntiles) return false;
        const int qt = tile_qt(t);
        return qt >= pq_lo && qt <= pq_hi;
    };

    if (score_wave) {
        // Key-side B operands: column c of block kc is key kp + 16kc + c;
        // head-dim value DQ g + 8ks + i in k-slot 8g + i of MFMA ks.
        bf16x8_t kop[2][KS], vop[2][KS];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const int key = min(kp + 16 * kc + c, S - 1);
            const uint16_t *ks_ = p.k + (int64_t)b * p.k_sb + (int64_t)key * p.k_ss + (int64_t)hk * p.k_sh;
            const uint16_t *vs_ = p.v + (int64_t)b * p.v_sb + (int64_t)key * p.v_ss + (int64_t)hk * p.v_sh;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                kop[kc][ks] = __builtin_bit_cast(bf16x8_t, ld16(ks_ + DQ * g + 8 * ks));
                vop[kc][ks] = __builtin_bit_cast(bf16x8_t, ld16(vs_ + DQ * g + 8 * ks));
            }
        }

        // sd/td/ud[rb][kc]: lane (c, g) = key column c of block kc, tile rows
        // 16rb + 4g + j.
        auto scores = [&](int t, f32x4_t (&sd)[2][2], f32x4_t (&td)[2][2], f32x4_t (&ud)[2][2]) {
            const int buf = slot3<D>(t);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
                for (int kc = 0; kc < 2; ++kc)
                    sd[rb][kc] = td[rb][kc] = ud[rb][kc] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                // the half's q, rho and dout operands are all read before its
                // MFMAs (one LDS latency per half, not one per three reads)
                bf16x8_t qa[KS], ra[KS], ga[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int off = (16 * rb + c) * RB + 2 * DQ * g + 16 * ks;
                    qa[ks] = __builtin_bit_cast(bf16x8_t, ld16(qtile + buf + off));
                    ra[ks] = __builtin_bit_cast(bf16x8_t, ld16(rtile + buf + off));
                    ga[ks] = __builtin_bit_cast(bf16x8_t, ld16(gtile + buf + off));
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc) {
                        sd[rb][kc] = mfma(qa[ks], kop[kc][ks], sd[rb][kc]);
                        td[rb][kc] = mfma(ra[ks], kop[kc][ks], td[rb][kc]);
                        ud[rb][kc] = mfma(ga[ks], vop[kc][ks], ud[rb][kc]);
                    }
                }
            }
        };
        // W = p (1 + r - t), scale dS and dT of tile t in bf16, as B operands
        // of the value MFMAs (column = key, k-slot r = tile row 4g + r for
        // r < 4, else 16 + 4g + r - 4).
        auto grads = [&](int t, const f32x4_t (&sd)[2][2], const f32x4_t (&td)[2][2],
                         const f32x4_t (&ud)[2][2], auto mask_tag) {
            constexpr bool MASK = decltype(mask_tag)::value;
            const int buf = t % 3;
            const int row0 = tile_qt(t) * kBwTile;
            uint32_t ww[8], sw[8], tw[8];  // [4 kc + k-slot pair]
            // one 16-row half at a time: its four rows' statistics are live
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                float4 rs[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) rs[j] = stile[buf][16 * rb + 4 * g + j];
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    const int key = kp + 16 * kc + c;
#pragma unroll
                    for (int j = 0; j < 4; j += 2) {
                        float w2[2], ds2[2], dt2[2];
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2) {
                            const float s = sd[rb][kc][j + h2];
                            const float tt = td[rb][kc][j + h2];
                            const float uu = ud[rb][kc][j + h2];
                            const float4 st = rs[j + h2];
                            float pw = __builtin_amdgcn_exp2f(fmaf(s, c2, -st.x));
                            if constexpr (MASK) {
                                const int qi = row0 + 16 * rb + 4 * g + j + h2;
                                pw = key <= qi && qi < S && key < S && (W == 0 || key > qi - W)
                                         ? pw
                                         : 0.0f;
                            }
                            const float m1 = st.y - tt;  // 1 + r - t
                            w2[h2] = pw * m1;
                            ds2[h2] = (p.scale * pw) * fmaf(uu, m1, fmaf(tt, st.z, -st.w));
                            dt2[h2] = pw * (st.z - uu);
                        }
                        // k-slot 4rb + j of the value MFMAs' B operand
                        ww[4 * kc + 2 * rb + j / 2] = pack_bf16x2(w2[0], w2[1]);
                        sw[4 * kc + 2 * rb + j / 2] = pack_bf16x2(ds2[0], ds2[1]);
                        tw[4 * kc + 2 * rb + j / 2] = pack_bf16x2(dt2[0], dt2[1]);
                    }
                }
            }
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                pbuf[t & 1][pair][kc][lane] =
                    uint4{ww[4 * kc], ww[4 * kc + 1], ww[4 * kc + 2], ww[4 * kc + 3]};
                pbuf[t & 1][pair][2 + kc][lane] =
                    uint4{sw[4 * kc], sw[4 * kc + 1], sw[4 * kc + 2], sw[4 * kc + 3]};
                pbuf[t & 1][pair][4 + kc][lane] =
                    uint4{tw[4 * kc], tw[4 * kc + 1], tw[4 * kc + 2], tw[4 * kc + 3]};
            }
        };
        auto score_step = [&](int t) {
            if (active(t)) {
                f32x4_t sd[2][2], td[2][2], ud[2][2];
                scores(t, sd, td, ud);
                const int row0 = tile_qt(t) * kBwTile;
                // unmasked when every row of the tile sees every key of the pair
                if (row0 >= kp + kBwRows - 1 && row0 + kBwTile <= S && kp + kBwRows <= S &&
                    (W == 0 || row0 + kBwTile - 1 - W < kp))
                    grads(t, sd, td, ud, std::false_type{});
                else
                    grads(t, sd, td, ud, std::true_type{});
            }
        };
        __syncthreads();  // the value waves' prologue
        for (int t = 0; t < ntiles; ++t) {
            score_step(t);
            __syncthreads();
        }
    } else {
        // dvt[db][kc], dkt[db][kc]: rows d = 16db + 4g + j, key column c of
        // block kc.
        f32x4_t dvt[DB][2], dkt[DB][2];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) dvt[db][kc] = dkt[db][kc] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        auto value_tile = [&](int u) {
            bf16x8_t pw[2], ps[2], pt[2];
#pragma unroll
            for (int kc = 0; kc < 2; ++kc) {
                pw[kc] = __builtin_bit_cast(bf16x8_t, pbuf[u & 1][pair][kc][lane]);
                ps[kc] = __builtin_bit_cast(bf16x8_t, pbuf[u & 1][pair][2 + kc][lane]);
                pt[kc] = __builtin_bit_cast(bf16x8_t, pbuf[u & 1][pair][4 + kc][lane]);
            }
            const int buf = slot3<D>(u);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8_t ga = tr_operand<D>(gtile + buf, db, c, g);
                const bf16x8_t qa = tr_operand<D>(qtile + buf, db, c, g);
                const bf16x8_t ra = tr_operand<D>(rtile + buf, db, c, g);
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    dvt[db][kc] = mfma(ga, pw[kc], dvt[db][kc]);
                    dkt[db][kc] = mfma(qa, ps[kc], dkt[db][kc]);
                    dkt[db][kc] = mfma(ra, pt[kc], dkt[db][kc]);
                }
                // keep the transposed reads of later blocks from being hoisted
                // all at once (48 reads would need 96 registers)
                if (db % 2 == 1) __builtin_amdgcn_sched_barrier(0);
            }
        };

        issue(0);
        store(0);
        issue(1);
        __syncthreads();
        for (int t = 0; t < ntiles; ++t) {
            store(t + 1);
            // head dim 64: the next loads go out before the value MFMAs
            // (-3% time; at 128 +1%, so there they follow them)
            if constexpr (D == 64) issue(t + 2);
            if (active(t - 1)) value_tile(t - 1);
            if constexpr (D != 64) issue(t + 2);
            __syncthreads();
        }
        if (active(ntiles - 1)) value_tile(ntiles - 1);

#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            const int key = kp + 16 * kc + c;
            if (key >= S) continue;
            const int64_t off = (int64_t)b * p.dk_sb + (int64_t)key * p.dk_ss + (int64_t)hk * p.dk_sh;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                *reinterpret_cast<float4 *>(p.dk + off + 16 * db + 4 * g) =
                    float4{dkt[db][kc][0], dkt[db][kc][1], dkt[db][kc][2], dkt[db][kc][3]};
                *reinterpret_cast<float4 *>(p.dv + off + 16 * db + 4 * g) =
                    float4{dvt[db][kc][0], dvt[db][kc][1], dvt[db][kc][2], dvt[db][kc][3]};
            }
        }
    }
}

// GQA groups 8 and 16: the dq kernel runs G / 4 workgroups of four query
// heads per KV head; the dk/dv kernel streams all G heads' rows past each
// key block.
template <int D, int G, bool WIN>
hipError_t launch_bwd(const PrefillBwdParams &pin, hipStream_t stream) {
    constexpr int GQ = G > 4 ? 4 : G;  // query heads per dq workgroup
    PrefillBwdParams p = pin;
    p.head_blocks = G / GQ;
    const int units = p.batch * p.num_kv_heads;
    const int qb_rows = kBwRows * kBwPairs / GQ;
    const int nqb = (p.seq_len + qb_rows - 1) / qb_rows;
    const int nkb = (p.seq_len + kBwRows * kBwPairs - 1) / (kBwRows * kBwPairs);
    hipLaunchKernelGGL((bwd_dq_kernel<D, GQ, WIN>), dim3((unsigned)(units * p.head_blocks * nqb)),
                       dim3(128 * kBwPairs), 0, stream, p);
    hipLaunchKernelGGL((bwd_dkv_kernel<D, G, WIN>), dim3((unsigned)(units * nkb)),
                       dim3(128 * kBwPairs), 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_backward_d(const PrefillBwdParams &p, hipStream_t stream) {
    const int64_t rows = (int64_t)p.batch * p.num_q_heads * p.seq_len;
    hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int G = p.num_q_heads / p.num_kv_heads;
    const bool win = p.window > 0 && p.window < p.seq_len;
    switch (G * 2 + (win ? 1 : 0)) {
        case 2: return launch_bwd<D, 1, false>(p, stream);
        case 3: return launch_bwd<D, 1, true>(p, stream);
        case 4: return launch_bwd<D, 2, false>(p, stream);
        case 5: return launch_bwd<D, 2, true>(p, stream);
        case 8: return launch_bwd<D, 4, false>(p, stream);
        case 9: return launch_bwd<D, 4, true>(p, stream);
        case 16: return launch_bwd<D, 8, false>(p, stream);
        case 17: return launch_bwd<D, 8, true>(p, stream);
        case 32: return launch_bwd<D, 16, false>(p, stream);
        case 33: return launch_bwd<D, 16, true>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill_backward(const PrefillBwdParams &p, int d, hipStream_t stream) {
    if (d == 128) return launch_prefill_backward_d<128>(p, stream);
    if (d == 64) return launch_prefill_backward_d<64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace plx
