// prefill.hip -- causal Parallax prefill for gfx950 (CDNA4), bf16 matrix cores.
//
// Row i of (batch b, query head h) attends to keys 0..i of KV head h/G and
// computes o_i = o_SA,i - S_KV^(i) rho_i (page "Parallax: Parameterized Local
// Linear Attention Gives Transformers a 'Second Eye'", section 1.3), through
// the same sums as decode: with s_ij = scale q_i.k_j and t_ij = rho_i.k_j,
//   Z_i = sum_j e^{s_ij}, R_i = sum_j e^{s_ij} t_ij,
//   A_i = sum_j e^{s_ij} v_j, B_i = sum_j e^{s_ij} t_ij v_j,
//   o_i = a - (b - a r),  a = A/Z, r = R/Z, b = B/Z.
// Both products are dense matrix products over a shared K/V tile (section
// 2.2 of that page: the covariance work is arranged for the matrix cores):
//   scores  D1[key][col] = K[key][:] . X[col][:]   X = 32 q rows and the 32
//           rho rows of the same queries (64 columns, 4 blocks of 16);
//   sums    D2[d][col]   = sum_key V[key][d] . P[key][col]   P = E (32 cols)
//           and E*T (32 cols), E = e^{s - m} rounded to bf16; one more block
//           against a tile of ones gives Z and R;
// all as 16x16x32 bf16 MFMAs with fp32 accumulation.  s and t of the same
// query row land in the same lane, so the softmax needs no data movement
// except the row max across the four lane groups.
//
// Workgroup: 8 waves in 4 pairs; a pair owns 32 query rows.  Wave p (score
// wave) computes the scores and softmax numerators of tile t and hands
// P = [E | E*T] (in value-MFMA operand layout) and the rows' rescale factors
// to wave p + 4 (value wave) through LDS; the value wave, which holds the 144
// accumulators, runs the value MFMAs of tile t - 1.  The two roles' registers
// are disjoint, so two waves fit on every SIMD, and the pair shares a SIMD, so
// one wave's MFMAs overlap the other's VALU work (a single wave per SIMD keeps
// the matrix core about a third busy).  The pairs cover 128/G rows of each of
// the G query heads of one KV head, so every 32-key K/V tile in LDS serves the
// whole GQA group (G <= 4; larger groups run as blocks of four heads).  K and V tiles of 32 keys are double-buffered in LDS with
// one barrier per tile: in the epoch where the score waves work on tile t and
// the value waves on tile t - 1, K tile t + 1 and V tile t are written to LDS;
// global loads run two tiles ahead of those stores.  V reaches the MFMA
// through ds_read_b64_tr_b16.  Query blocks are scheduled longest (highest
// causal row) first; tiles past a pair's last row are skipped.
#include "kernels.hpp"

#include <math.h>

#include <type_traits>

namespace plx {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPfPairs = 4;               // score/value wave pairs per workgroup
constexpr int kPfRows = 32;               // query rows per pair
constexpr int kPfKeys = 32;               // keys per tile
// LDS bytes per tile row (head dim D = 64 or 128).  K rows are read 16
// bytes per lane, one row per lane of a 16-lane group: a 16-byte pad puts the
// 16 rows on distinct banks (strides of 68 and 36 banks).  V is read through
// ds_read_b64_tr_b16 (8 bytes per lane, 8 rows per 32 lanes): a 32-byte pad
// puts those rows on distinct bank pairs (strides of 72 and 40 banks; with
// 16 bytes they overlapped in pairs; +2% at batch 4 x 8192, D = 128).
template <int D>
constexpr int pf_row_bytes() { return 2 * D + 16; }
template <int D>
constexpr int pf_vrow_bytes() { return 2 * D + 32; }
constexpr float kSlack = 8.0f;            // base-2 headroom before a row's reference max moves

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

// Max over the four 16-lane groups (lanes c, c+16, c+32, c+48).  A compare
// and select per step: fmaxf on the swapped values first quiets both inputs
// (two more instructions), and the scores are never NaN.
__device__ __forceinline__ float group_max(float x) {
    const int xi = __builtin_bit_cast(int, x);
    auto a = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);  // rows 0<->1, 2<->3
    const float a0 = __builtin_bit_cast(float, (int)a[0]), a1 = __builtin_bit_cast(float, (int)a[1]);
    x = a0 > a1 ? a0 : a1;
    const int yi = __builtin_bit_cast(int, x);
    auto b2 = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);  // halves 0<->1
    const float b0 = __builtin_bit_cast(float, (int)b2[0]), b1 = __builtin_bit_cast(float, (int)b2[1]);
    return b0 > b1 ? b0 : b1;
}

// WIN: the local-window form (instantiated separately, so full causal
// attention carries none of its index arithmetic).  STATS: also write lse, r
// and o_SA for a backward pass (separately too: the plain forward keeps the
// code it had without them).
// D = 64: at most 128 registers (a few spill), so two workgroups share a CU
// (four waves per SIMD; LDS 54 KB each): 703 -> 846 TFLOP/s at batch 4 x 8192.
template <int D, int G, bool WIN, bool STATS>
__global__ __launch_bounds__(128 * kPfPairs, D == 64 ? 4 : 1) void prefill_kernel(PrefillParams p) {
    constexpr int KS = D / 32;                      // score MFMAs per 16-key block
    constexpr int DB = D / 16;                      // 16-row blocks of the value sums
    constexpr int DQ = D / 4;                       // head-dim values per lane group (scores)
    constexpr int RB = pf_row_bytes<D>(), VRB = pf_vrow_bytes<D>();
    constexpr int PB = 2 * D * kPfKeys / (128 * kPfPairs);  // tile bytes per thread (16 or 8)
    constexpr int PPH = kPfPairs / G;               // pairs per query head
    constexpr int QB = kPfRows * PPH;               // query rows per head per workgroup
    constexpr int TILE = kPfKeys * RB;
    using Piece = std::conditional_t<PB == 16, uint4, uint2>;

    __shared__ __attribute__((aligned(16))) unsigned char ktile[2][TILE];
    __shared__ __attribute__((aligned(16))) unsigned char vtile[2][kPfKeys * VRB];
    __shared__ uint4 pbuf[2][kPfPairs][4][64];     // P operands, in value-MFMA lane layout
    __shared__ float abuf[2][kPfPairs][2][16];      // per-row rescale factors
    __shared__ float mfin[kPfPairs][2][16];         // final reference max per row

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int S = p.seq_len;
    const float c2 = p.scale_log2;
    const bool score_wave = wave < kPfPairs;
    const int pair = wave % kPfPairs;

    const int nhb = p.num_kv_heads * p.head_blocks;  // blocks of G query heads
    const int units = p.batch * nhb;
    const int nqb = (S + QB - 1) / QB;
    const int qb = nqb - 1 - (int)(blockIdx.x / units);  // longest causal rows first
    const int unit = blockIdx.x % units;
    const int b = unit / nhb;
    const int hb = unit % nhb;
    const int hk = hb / p.head_blocks;  // the KV head of query heads hb*G .. hb*G + G - 1
    const int head = hb * G + pair / PPH;
    const int r0 = qb * QB + (pair % PPH) * kPfRows;  // first query row of this pair
    const int key_end = min(S, (qb + 1) * QB);        // keys this workgroup needs
    const int ntiles = (key_end + kPfKeys - 1) / kPfKeys;
    const int pair_tiles = min(ntiles, (min(S, r0 + kPfRows) + kPfKeys - 1) / kPfKeys);
    // Local window W >= 1: row i keeps keys i-W+1 .. i.  Tiles below the
    // workgroup's first needed key are skipped; the loop starts on an even
    // tile (the LDS buffer of tile t is t & 1, fixed at compile time).
    const int W = WIN ? p.window : 0;
    const int t_first = (W > 0 ? max(0, qb * QB - W + 1) / kPfKeys : 0) & ~1;
    const int pair_lo = W > 0 ? max(0, r0 - W + 1) / kPfKeys : 0;  // first tile of this pair

    // ---- cooperative tile loads: thread t moves PB bytes (piece t%16) of key
    // t/16.  Tiles travel through two register stages per operand, so a K or V
    // tile load is issued two iterations before its LDS store.
    const uint16_t *kg = p.k + (int64_t)b * p.k_sb + (int64_t)hk * p.k_sh;
    const uint16_t *vg = p.v + (int64_t)b * p.v_sb + (int64_t)hk * p.v_sh;
    // K tile j in register stage kst<j & 1>, V tile j in vst<j & 1>: named
    // registers picked at compile time (an array of stages was kept in
    // scratch memory when the compiler indexed it at run time)
    Piece k0, k1, v0, v1;
    auto kst = [&](auto par) -> Piece & {
        if constexpr (decltype(par)::value == 0) return k0;
        else return k1;
    };
    auto vst = [&](auto par) -> Piece & {
        if constexpr (decltype(par)::value == 0) return v0;
        else return v1;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    auto issue_k = [&](int t, Piece &dst) {
        const int key = min(t * kPfKeys + tid / 16, S - 1);
        dst = *reinterpret_cast<const Piece *>(kg + (int64_t)key * p.k_ss + PB / 2 * (tid % 16));
    };
    auto issue_v = [&](int t, Piece &dst) {
        const int key = min(t * kPfKeys + tid / 16, S - 1);
        dst = *reinterpret_cast<const Piece *>(vg + (int64_t)key * p.v_ss + PB / 2 * (tid % 16));
    };
    auto store = [&](unsigned char *tile, const Piece &st) {
        *reinterpret_cast<Piece *>(tile + (tid / 16) * RB + PB * (tid % 16)) = st;
    };
    auto vstore = [&](unsigned char *tile, const Piece &st) {
        *reinterpret_cast<Piece *>(tile + (tid / 16) * VRB + PB * (tid % 16)) = st;
    };
    // End of iteration t (P = t & 1): K tile t+1 replaces tile t-1 (read by
    // the score waves in iteration t-1), V tile t replaces tile t-2 (read by
    // the value waves in iteration t-1); the freed register stages take the
    // loads of K tile t+3 and V tile t+2.  Loads and stores run on every
    // iteration, also past the last tile: their keys are clamped to S - 1 and
    // a buffer written there is never read.  Every path through the loop then
    // has the same four loads in flight, which keeps the compiler's memory
    // wait counts exact (a data-dependent load count makes it wait for all of
    // them, the newest included).
    auto advance = [&](int t, auto par) {
        constexpr int P = decltype(par)::value;
        using Q = std::integral_constant<int, 1 - P>;
        store(ktile[1 - P], kst(Q{}));
        vstore(vtile[P], vst(par));
        issue_k(t + 3, kst(Q{}));
        issue_v(t + 2, vst(par));
        __syncthreads();
    };
    // Prologue, common to both roles (after the score waves' q / rho loads):
    // K tile 0 into LDS; K tiles 1, 2 and V tiles 0, 1 in flight, in the
    // order the loop keeps them.
    auto prologue = [&] {
        issue_k(t_first, kst(I0{}));
        store(ktile[0], kst(I0{}));
        issue_k(t_first + 1, kst(I1{}));
        issue_v(t_first, vst(I0{}));
        issue_k(t_first + 2, kst(I0{}));
        issue_v(t_first + 1, vst(I1{}));
        __syncthreads();
    };

    if (score_wave) {
        // ---- query-side operands: column block cb < 2 holds q rows r0 + 16cb + c,
        // cb >= 2 the rho rows of the same queries; head-dim value DQ g + 8ks + i
        // sits in k-slot 8g + i of score MFMA ks (the slots the K operand uses)
        bf16x8_t xop[4][KS];
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
        float mref[2] = {-INFINITY, -INFINITY};  // base-2 reference max per query row

        // Scores of tile t: d1[rb][cb] lane (c, g) = column c of block cb, keys
        // 32t + 16rb + 4g + j.
        auto scores = [&](int t, f32x4_t (&d1)[2][4]) {
            const unsigned char *kt = ktile[t & 1];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) d1[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8_t kop = __builtin_bit_cast(
                        bf16x8_t, ld16(kt + (16 * rb + c) * RB + 2 * DQ * g + 16 * ks));
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb)
                        d1[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, xop[cb][ks],
                                                                             d1[rb][cb], 0, 0, 0);
                }
            }
        };
        // Softmax numerators of tile t: E = 2^(c2 s - m) and E*T in bf16, laid
        // out as the B operands of the value MFMAs (k-slot r holds key 4g + r
        // for r < 4, else 16 + 4g + r - 4 of the tile), handed to the value
        // wave through LDS.  A row's reference max moves (by select) only when
        // the tile's max exceeds it by more than kSlack; alpha < 1 then tells
        // the value wave to rescale that row's sums first.  MASK: the tile
        // crosses the diagonal, S or (local window) a row's window start.
        auto numerators = [&](int t, const f32x4_t (&d1)[2][4], auto mask_tag) {
            constexpr bool MASK = decltype(mask_tag)::value;
            // The two 16-row halves (qc) run side by side, phase by phase, so
            // their dependency chains (max, cross-group max, exp) overlap.
            float sv[2][8], gm[2];
#pragma unroll
            for (int qc = 0; qc < 2; ++qc) {
                const int qi = r0 + 16 * qc + c;
                float tmax = -INFINITY;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    sv[qc][r] = r < 4 ? d1[0][qc][r] : d1[1][qc][r - 4];
                    if constexpr (MASK) {
                        const int key = t * kPfKeys + (r < 4 ? 4 * g + r : 16 + 4 * g + r - 4);
                        sv[qc][r] = key <= qi && key < S && (W == 0 || key > qi - W)
                                        ? sv[qc][r]
                                        : -INFINITY;
                    }
                    tmax = __builtin_fmaxf(tmax, sv[qc][r]);
                }
                gm[qc] = tmax;
            }
#pragma unroll
            for (int qc = 0; qc < 2; ++qc) gm[qc] = group_max(gm[qc]);
            float mnew[2], alpha[2];
#pragma unroll
            for (int qc = 0; qc < 2; ++qc) {
                const float tm2 = gm[qc] * c2;
                mnew[qc] = tm2 > mref[qc] + kSlack ? tm2 : mref[qc];
                alpha[qc] = __builtin_amdgcn_exp2f(mref[qc] - mnew[qc]);  // 1 unless moved
                if constexpr (MASK && WIN) {
                    // a row that has met no key yet (its window starts past
                    // this tile) keeps m = -inf: weights 0, factor 1
                    if (mnew[qc] == -INFINITY) alpha[qc] = 1.0f;
                }
                mref[qc] = mnew[qc];
                if constexpr (MASK && WIN) {
                    if (mnew[qc] == -INFINITY) mnew[qc] = 0.0f;  // exp2(-inf - 0) = 0 below
                }
            }
#pragma unroll
            for (int qc = 0; qc < 2; ++qc) {
                uint32_t ew[4], etw[4];
#pragma unroll
                for (int r = 0; r < 8; r += 2) {
                    const float e0 = __builtin_amdgcn_exp2f(fmaf(sv[qc][r], c2, -mnew[qc]));
                    const float e1 = __builtin_amdgcn_exp2f(fmaf(sv[qc][r + 1], c2, -mnew[qc]));
                    const float t0 = r < 4 ? d1[0][qc + 2][r] : d1[1][qc + 2][r - 4];
                    const float t1 = r < 4 ? d1[0][qc + 2][r + 1] : d1[1][qc + 2][r - 3];
                    ew[r / 2] = pack_bf16x2(e0, e1);
                    etw[r / 2] = pack_bf16x2(e0 * t0, e1 * t1);
                }
                pbuf[t & 1][pair][qc][lane] = uint4{ew[0], ew[1], ew[2], ew[3]};
                pbuf[t & 1][pair][qc + 2][lane] = uint4{etw[0], etw[1], etw[2], etw[3]};
                // every lane group holds the row's factor; all four write the
                // same value (no lane condition, so no branch splits the code)
                abuf[t & 1][pair][qc][c] = alpha[qc];
            }
        };
        auto score_step = [&](int t) {
            if (t >= pair_lo && t < pair_tiles) {
                f32x4_t d1[2][4];
                scores(t, d1);
                // no masking when every key of the tile is in every row's range
                if (t * kPfKeys + kPfKeys - 1 <= r0 && t * kPfKeys + kPfKeys <= S &&
                    (W == 0 || t * kPfKeys > r0 + kPfRows - 1 - W))
                    numerators(t, d1, std::false_type{});
                else
                    numerators(t, d1, std::true_type{});
            }
        };
        // Two iterations per trip fix each iteration's register stage at compile
        // time.  Both halves always run (iterations past the last tile do no
        // math), so the two roles pass the same number of barriers.
        prologue();
        for (int t = t_first; t <= ntiles; t += 2) {
            score_step(t);
            advance(t, std::integral_constant<int, 0>{});
            score_step(t + 1);
            advance(t + 1, std::integral_constant<int, 1>{});
        }
        if constexpr (STATS) {  // the value wave turns its Z into log(sum e^s)
            mfin[pair][0][c] = mref[0];
            mfin[pair][1][c] = mref[1];
            __syncthreads();
        }
    } else {
        // Value sums: acc[db][cb] = D2 rows d = 16db + 4g + j, column c of block
        // cb (E rows 0-15, 16-31, E*T rows 0-15, 16-31).  Block db = DB
        // multiplies a tile of ones, so its rows carry Z (cb < 2) and R (cb >= 2).
        f32x4_t acc[DB + 1][4];
#pragma unroll
        for (int db = 0; db <= DB; ++db)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) acc[db][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        auto value_tile = [&](int u) {
            const float al0 = abuf[u & 1][pair][0][c], al1 = abuf[u & 1][pair][1][c];
            if (__builtin_amdgcn_ballot_w64(al0 != 1.0f || al1 != 1.0f)) {  // rare after tile 0
#pragma unroll
                for (int db = 0; db <= DB; ++db) {
                    acc[db][0] *= al0;
                    acc[db][2] *= al0;
                    acc[db][1] *= al1;
                    acc[db][3] *= al1;
                }
            }
            bf16x8_t pop[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                pop[cb] = __builtin_bit_cast(bf16x8_t, pbuf[u & 1][pair][cb][lane]);
            const unsigned char *vt = vtile[u & 1];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
                const int col = 16 * db + 4 * (c % 4);
                const unsigned char *a0 = vt + (4 * g + c / 4) * VRB + 2 * col;
                const unsigned char *a1 = vt + (16 + 4 * g + c / 4) * VRB + 2 * col;
                const i16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(__attribute__((address_space(3))) unsigned char *)a0);
                const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(__attribute__((address_space(3))) unsigned char *)a1);
                const bf16x8_t vop = __builtin_bit_cast(
                    bf16x8_t, i16x8_t{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]});
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
                    acc[db][cb] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[cb], acc[db][cb], 0, 0, 0);
            }
            const bf16x8_t ones = __builtin_bit_cast(
                bf16x8_t, uint4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                acc[DB][cb] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pop[cb], acc[DB][cb], 0, 0, 0);
        };

        prologue();
        for (int t = t_first; t <= ntiles; t += 2) {
            if (t - 1 >= pair_lo && t - 1 < pair_tiles) value_tile(t - 1);
            advance(t, std::integral_constant<int, 0>{});
            if (t >= pair_lo && t < pair_tiles) value_tile(t);
            advance(t + 1, std::integral_constant<int, 1>{});
        }

        if constexpr (STATS) __syncthreads();  // mfin written by the score waves

        // ---- o = a - (b - a r) per query row; lane (c, g) holds d = 16db + 4g + j
#pragma unroll
        for (int qc = 0; qc < 2; ++qc) {
            const int qi = r0 + 16 * qc + c;
            if (qi >= S) continue;
            const float inv = 1.0f / acc[DB][qc][0];
            const float r = acc[DB][qc + 2][0] * inv;
            const int64_t ooff = (int64_t)b * p.o_sb + (int64_t)qi * p.o_ss + (int64_t)head * p.o_sh;
            float *orow = p.out + ooff;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                float o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float a = acc[db][qc][j] * inv, bb = acc[db][qc + 2][j] * inv;
                    o[j] = a - (bb - a * r);
                }
                *reinterpret_cast<float4 *>(orow + 16 * db + 4 * g) =
                    float4{o[0], o[1], o[2], o[3]};
            }
            // what a backward pass needs: log of the softmax denominator
            // (natural log; Z is kept relative to 2^m), r and o_SA
            if constexpr (STATS) {
                const int64_t ri = ((int64_t)b * p.num_q_heads + head) * S + qi;
                if (p.lse != nullptr && g == 0)
                    p.lse[ri] = (mfin[pair][qc][c] + __builtin_log2f(acc[DB][qc][0])) *
                                0.6931471805599453f;
                if (p.rmean != nullptr && g == 0) p.rmean[ri] = r;
            }
            if (STATS && p.o_sa != nullptr) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    *reinterpret_cast<float4 *>(p.o_sa + ooff + 16 * db + 4 * g) =
                        float4{acc[db][qc][0] * inv, acc[db][qc][1] * inv, acc[db][qc][2] * inv,
                               acc[db][qc][3] * inv};
            }
        }
    }
}

// GQA groups 8 and 16: G / 4 workgroups of four query heads each per KV head
// (each loads the KV tiles once for its four heads).
template <int D>
hipError_t launch_prefill_d(const PrefillParams &pin, hipStream_t stream) {
    PrefillParams p = pin;
    const int group = p.num_q_heads / p.num_kv_heads;
    const int G = group > 4 ? 4 : group;  // query heads per workgroup
    p.head_blocks = group / G;
    const int units = p.batch * p.num_kv_heads * p.head_blocks;
    const int qb_rows = kPfRows * kPfPairs / G;
    const dim3 grid((unsigned)(units * ((p.seq_len + qb_rows - 1) / qb_rows)));
    const dim3 block(128 * kPfPairs);
    const bool win = p.window > 0 && p.window < p.seq_len;  // else every key 0..i is in range
    const bool stats = p.lse != nullptr || p.rmean != nullptr || p.o_sa != nullptr;
#define PLX_PREFILL_CASE(G_, W_, S_)                                                         \
    case G_ * 4 + W_ * 2 + S_:                                                               \
        hipLaunchKernelGGL((prefill_kernel<D, G_, W_, S_>), grid, block, 0, stream, p);      \
        break;
    switch (G * 4 + (win ? 2 : 0) + (stats ? 1 : 0)) {
        PLX_PREFILL_CASE(1, 0, 0) PLX_PREFILL_CASE(1, 0, 1)
        PLX_PREFILL_CASE(1, 1, 0) PLX_PREFILL_CASE(1, 1, 1)
        PLX_PREFILL_CASE(2, 0, 0) PLX_PREFILL_CASE(2, 0, 1)
        PLX_PREFILL_CASE(2, 1, 0) PLX_PREFILL_CASE(2, 1, 1)
        PLX_PREFILL_CASE(4, 0, 0) PLX_PREFILL_CASE(4, 0, 1)
        PLX_PREFILL_CASE(4, 1, 0) PLX_PREFILL_CASE(4, 1, 1)
        default: return hipErrorInvalidValue;
    }
#undef PLX_PREFILL_CASE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams &p, int d, hipStream_t stream) {
    if (d == 128) return launch_prefill_d<128>(p, stream);
    if (d == 64) return launch_prefill_d<64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace plx
