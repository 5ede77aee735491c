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
//
// Work items: one item is one query block of one (batch, head block).  At
// head dim 128 the launch is persistent: one workgroup per CU runs a list of
// items back to back as one stream of tile positions, so the next item's K/V
// tiles are already in flight while the last ones of the current item are
// consumed, and the score waves' wait for the next item's q/rho rows
// overlaps the value waves' last tile and outputs of the current one (a new
// workgroup instead starts with a full memory round trip, ~3.5 us, against
// ~1 us per tile, and ends with its outputs while nothing else runs on the
// CU).  At head dim 64 two workgroups share a CU (that overlap hides the
// same latency) and each runs one item.
#include "kernels.hpp"

#include <math.h>

#include <algorithm>
#include <atomic>
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
constexpr float kSlackWeight = 256.0f;    // 2^kSlack: the largest weight a kept reference allows

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
template <int D>
constexpr bool pf_persistent() { return D == 128; }

template <int D, int G, bool WIN, bool STATS>
__global__ __launch_bounds__(128 * kPfPairs, D == 64 ? 4 : 1) void prefill_kernel(PrefillParams p) {
    constexpr int KS = D / 32;                      // score MFMAs per 16-key block
    constexpr int DB = D / 16;                      // 16-row blocks of the value sums
    constexpr int DQ = D / 4;                       // head-dim values per lane group (scores)
    constexpr int RB = pf_row_bytes<D>(), VRB = pf_vrow_bytes<D>();
    constexpr int PB = 2 * D * kPfKeys / (128 * kPfPairs);  // tile bytes per thread (16 or 8)
    constexpr int PPH = kPfPairs / G;               // pairs per query head
    constexpr int QB = kPfRows * PPH;               // query rows per head per item
    constexpr int TILE = kPfKeys * RB;
    using Piece = std::conditional_t<PB == 16, uint4, uint2>;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    __shared__ __attribute__((aligned(16))) unsigned char ktile[2][TILE];
    __shared__ __attribute__((aligned(16))) unsigned char vtile[2][kPfKeys * VRB];
    __shared__ uint4 pbuf[2][kPfPairs][4][64];     // P operands, in value-MFMA lane layout
    __shared__ float abuf[2][kPfPairs][2][16];      // per-row rescale factors
    __shared__ float mfin[2][kPfPairs][2][16];      // final reference max per row, by item parity

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int S = p.seq_len;
    const float c2 = p.scale_log2;
    const bool score_wave = wave < kPfPairs;
    const int pair = wave % kPfPairs;
    const int W = WIN ? p.window : 0;

    // ---- work list.  Item k: query block nqb - 1 - k / units (longest causal
    // rows first) of unit k % units = (batch, head block).  The P persistent
    // workgroups (the first P) take one item per round of P for R rounds:
    // workgroup w item rP + w in even rounds; in odd rounds the groups of
    // eight workgroups take their items in reverse order (the long items of
    // one round pair with short ones of the next), keeping item % 8 == w % 8,
    // so a unit's items stay on one XCD when P and the unit count are
    // multiples of 8 (workgroups go to the XCDs in turn).  The items after
    // the R rounds -- the shortest ones -- run one per workgroup: the hardware
    // starts those as persistent workgroups finish, which evens out the
    // workgroups' differing speeds.
    const int nhb = p.num_kv_heads * p.head_blocks;  // blocks of G query heads
    const int units = p.batch * nhb;
    const int nqb = (S + QB - 1) / QB;
    const int P = p.persist;
    const int wg = blockIdx.x;
    const bool persistent = pf_persistent<D>() && wg < P;
    auto item_id = [&](int i) __attribute__((always_inline)) -> int {
        if (!persistent) return p.static_rounds * P + (wg - P);
        int off = wg;
        if (i & 1) off = P % 8 == 0 ? P - 8 - (wg & ~7) + (wg & 7) : P - 1 - wg;
        return i * P + off;
    };
    // (head dim 64 launches one workgroup per item: the constant lets the
    // compiler drop the item changes)
    const int n_mine = persistent ? p.static_rounds : 1;

    // Item i of this workgroup: tiles [t0, t1) hold its keys (local window
    // W >= 1: row r keeps keys r-W+1 .. r, so tiles below the item's first
    // needed key are skipped).  The items' tiles form one stream of
    // positions, t0 .. tend - 1 for this item: an even number (a position's
    // LDS buffers and register stages are fixed at compile time by its
    // parity) and at least four, the last four being the item's tail (the
    // loads that run three positions ahead leave the item only there, and
    // reach at most the next item); positions from t1 on do no math.
    struct Item {
        int i, t0, t1, tend, qb, b, hb;
        const uint16_t *kb, *vb;  // K and V rows of the item's (batch, KV head)
    };
    auto item_get = [&](int i, Item &u) __attribute__((always_inline)) {
        const int k = item_id(i);
        u.i = i;
        u.qb = nqb - 1 - k / units;
        u.t1 = (min(S, (u.qb + 1) * QB) + kPfKeys - 1) / kPfKeys;
        u.t0 = W > 0 ? max(0, u.qb * QB - W + 1) / kPfKeys : 0;
        const int len = max(u.t1 - u.t0, 4);
        u.tend = u.t0 + len + (len & 1);
        const int unit = k % units;
        u.b = unit / nhb;
        u.hb = unit % nhb;
        const int hk = u.hb / p.head_blocks;  // the KV head of query heads hb*G .. hb*G + G - 1
        u.kb = p.k + (int64_t)u.b * p.k_sb + (int64_t)hk * p.k_sh;
        u.vb = p.v + (int64_t)u.b * p.v_sb + (int64_t)hk * p.v_sh;
    };
    // This wave's pair within an item: query head, first row, and the tiles
    // [lo, hi) holding keys its rows see (hi stops at the pair's last row).
    struct PairRange {
        int head, r0, lo, hi;
    };
    auto pair_range = [&](const Item &u) __attribute__((always_inline)) {
        PairRange x;
        x.head = u.hb * G + pair / PPH;
        x.r0 = u.qb * QB + (pair % PPH) * kPfRows;
        x.hi = min(u.t1, (min(S, x.r0 + kPfRows) + kPfKeys - 1) / kPfKeys);
        x.lo = W > 0 ? max(0, x.r0 - W + 1) / kPfKeys : 0;
        return x;
    };
    Item cur, nxt;  // the current item and the one after it (the same when none)
    item_get(0, cur);
    nxt = cur;
    if (n_mine > 1) item_get(1, nxt);
    // the next item takes over: both roles move on in step
    auto next_item = [&]() __attribute__((always_inline)) {
        cur = nxt;
        if (cur.i + 1 < n_mine) item_get(cur.i + 1, nxt);
    };

    // ---- cooperative tile loads: thread t moves PB bytes (piece t%16) of key
    // t/16.  Tiles travel through two register stages per operand, so a K or V
    // tile load is issued two positions before its LDS store.
    // K tile of position j in register stage kst<j & 1>, V tile in vst<j & 1>:
    // named registers picked at compile time (an array of stages was kept in
    // scratch memory when the compiler indexed it at run time)
    Piece k0, k1, v0, v1;
    auto kst = [&](auto par) __attribute__((always_inline)) -> Piece & {
        if constexpr (decltype(par)::value == 0) return k0;
        else return k1;
    };
    auto vst = [&](auto par) __attribute__((always_inline)) -> Piece & {
        if constexpr (decltype(par)::value == 0) return v0;
        else return v1;
    };
    // The tile of position tt of the current item.  TAIL: tt may run past the
    // item's end; then it is a tile of the next item, or, after the last
    // item, the last tile again (loaded, never read).
    auto tile_load = [&](int tt, bool is_v, Piece &dst, auto tail) __attribute__((always_inline)) {
        const uint16_t *base = is_v ? cur.vb : cur.kb;  // (by value: pointers to the
        if (decltype(tail)::value && tt >= cur.tend) {  // items would keep them in memory)
            if (cur.i + 1 < n_mine) {
                tt = nxt.t0 + (tt - cur.tend);
                base = is_v ? nxt.vb : nxt.kb;
            } else {
                tt = cur.tend - 1;
            }
        }
        const int key = min(tt * kPfKeys + tid / 16, S - 1);
        const int64_t ss = is_v ? p.v_ss : p.k_ss;
        dst = *reinterpret_cast<const Piece *>(base + (int64_t)key * ss + PB / 2 * (tid % 16));
    };
    auto store = [&](unsigned char *tile, const Piece &st) __attribute__((always_inline)) {
        *reinterpret_cast<Piece *>(tile + (tid / 16) * RB + PB * (tid % 16)) = st;
    };
    auto vstore = [&](unsigned char *tile, const Piece &st) __attribute__((always_inline)) {
        *reinterpret_cast<Piece *>(tile + (tid / 16) * VRB + PB * (tid % 16)) = st;
    };
    // End of position t (parity P): K tile t+1 replaces tile t-1 (read by the
    // score waves at position t-1), V tile t replaces tile t-2 (read by the
    // value waves at position t-1); the freed register stages take the loads
    // of K tile t+3 and V tile t+2.  Loads and stores run at every position,
    // also past the last one: a buffer written there is never read.  Every
    // path through the loop then has the same loads in flight, which keeps
    // the compiler's memory wait counts exact (a data-dependent load count
    // makes it wait for all of them, the newest included).
    using Main = std::false_type;
    using Tail = std::true_type;
    auto advance = [&](int t, auto par, auto tail) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        using Q = std::integral_constant<int, 1 - P>;
        store(ktile[1 - P], kst(Q{}));
        vstore(vtile[P], vst(par));
        tile_load(t + 3, false, kst(Q{}), tail);
        tile_load(t + 2, true, vst(par), tail);
        __syncthreads();
    };
    // Prologue, common to both roles (after the score waves' q / rho loads):
    // K tile of position 0 into LDS; K tiles 1, 2 and V tiles 0, 1 in flight,
    // in the order the loop keeps them.
    auto prologue = [&]() __attribute__((always_inline)) {
        tile_load(cur.t0, false, kst(I0{}), Main{});
        store(ktile[0], kst(I0{}));
        tile_load(cur.t0 + 1, false, kst(I1{}), Main{});
        tile_load(cur.t0, true, vst(I0{}), Main{});
        tile_load(cur.t0 + 2, false, kst(I0{}), Main{});
        tile_load(cur.t0 + 1, true, vst(I1{}), Main{});
        __syncthreads();
    };

    if (score_wave) {
        PairRange pr = pair_range(cur);
        // ---- query-side operands: column block cb < 2 holds q rows r0 + 16cb + c,
        // cb >= 2 the rho rows of the same queries; head-dim value DQ g + 8ks + i
        // sits in k-slot 8g + i of score MFMA ks (the slots the K operand uses).
        // An item after the first loads them at its first position, while the
        // value waves finish the previous item.
        bf16x8_t xop[4][KS], xnext[4][KS];
        auto load_x = [&](bf16x8_t (&x)[4][KS], const Item &u, const PairRange &r)
                          __attribute__((always_inline)) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int row = min(r.r0 + 16 * (cb & 1) + c, S - 1);
                const uint16_t *src =
                    cb < 2 ? p.q + (int64_t)u.b * p.q_sb + (int64_t)row * p.q_ss + (int64_t)r.head * p.q_sh
                           : p.rho + (int64_t)u.b * p.r_sb + (int64_t)row * p.r_ss + (int64_t)r.head * p.r_sh;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    x[cb][ks] = __builtin_bit_cast(bf16x8_t, ld16(src + DQ * g + 8 * ks));
            }
        };
        // Loaded operands into use.  The masked scores below are set to -inf
        // and the row max is taken on raw scores, so the factor applied to
        // them must be positive: a negative scale negates q, a zero scale
        // zeroes it (here, not at the load, which would wait for the data).
        auto take_x = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    uint4 w = __builtin_bit_cast(uint4, xnext[cb][ks]);
                    if (cb < 2 && p.q_sign != 0) {
                        const uint32_t x = p.q_sign == 1 ? 0x80008000u : 0u;
                        const uint32_t keep = p.q_sign == 1 ? 0xffffffffu : 0u;
                        w = uint4{(w.x & keep) ^ x, (w.y & keep) ^ x, (w.z & keep) ^ x,
                                  (w.w & keep) ^ x};
                    }
                    xop[cb][ks] = __builtin_bit_cast(bf16x8_t, w);
                }
        };
        load_x(xnext, cur, pr);
        take_x();
        float mref[2];  // base-2 reference max per query row

        // Scores of the tile at parity P: d1[rb][cb] lane (c, g) = column c of
        // block cb, keys 32t + 16rb + 4g + j.
        auto scores = [&](auto par, f32x4_t (&d1)[2][4]) __attribute__((always_inline)) {
            const unsigned char *kt = ktile[decltype(par)::value];
            // every K operand of the tile is read before the first MFMA, so
            // the LDS latency is paid once per tile rather than once per
            // pair of reads (the compiler otherwise reuses the operand
            // registers and waits on each pair in turn)
            bf16x8_t kop[2][KS];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kop[rb][ks] = __builtin_bit_cast(
                        bf16x8_t, ld16(kt + (16 * rb + c) * RB + 2 * DQ * g + 16 * ks));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) d1[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb)
                        d1[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            kop[rb][ks], xop[cb][ks], d1[rb][cb], 0, 0, 0);
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
        auto numerators = [&](int t, auto par, const f32x4_t (&d1)[2][4],
                              auto mask_tag) __attribute__((always_inline)) {
            constexpr bool MASK = decltype(mask_tag)::value;
            constexpr int P = decltype(par)::value;
            float sv[2][8];
#pragma unroll
            for (int qc = 0; qc < 2; ++qc) {
                const int qi = pr.r0 + 16 * qc + c;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    sv[qc][r] = r < 4 ? d1[0][qc][r] : d1[1][qc][r - 4];
                    if constexpr (MASK) {
                        const int key = t * kPfKeys + (r < 4 ? 4 * g + r : 16 + 4 * g + r - 4);
                        sv[qc][r] = key <= qi && key < S && (W == 0 || key > qi - W)
                                        ? sv[qc][r]
                                        : -INFINITY;
                    }
                }
            }
            // The weights against the rows' current reference.  It stays
            // unless a weight exceeds 2^kSlack or a row has no reference yet;
            // only then (a wave-uniform branch, rare after an item's first
            // tile) are the rows' tile maxima taken across the lane groups
            // and the weights formed again against the moved reference.
            float ev[2][8];
            float emax = 0.0f;
#pragma unroll
            for (int qc = 0; qc < 2; ++qc)
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    ev[qc][r] = __builtin_amdgcn_exp2f(fmaf(sv[qc][r], c2, -mref[qc]));
                    emax = __builtin_fmaxf(emax, ev[qc][r]);
                }
            float alpha[2] = {1.0f, 1.0f};
            const bool move = !(emax <= kSlackWeight) || mref[0] == -INFINITY || mref[1] == -INFINITY;
            if (__builtin_amdgcn_ballot_w64(move)) {
                // The two 16-row halves (qc) run side by side, phase by phase,
                // so their dependency chains (max, cross-group max, exp) overlap.
                float gm[2];
#pragma unroll
                for (int qc = 0; qc < 2; ++qc) {
                    float tmax = -INFINITY;
#pragma unroll
                    for (int r = 0; r < 8; ++r) tmax = __builtin_fmaxf(tmax, sv[qc][r]);
                    gm[qc] = tmax;
                }
#pragma unroll
                for (int qc = 0; qc < 2; ++qc) gm[qc] = group_max(gm[qc]);
                float mnew[2];
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
                for (int qc = 0; qc < 2; ++qc)
#pragma unroll
                    for (int r = 0; r < 8; ++r)
                        ev[qc][r] = __builtin_amdgcn_exp2f(fmaf(sv[qc][r], c2, -mnew[qc]));
            }
#pragma unroll
            for (int qc = 0; qc < 2; ++qc) {
                uint32_t ew[4], etw[4];
#pragma unroll
                for (int r = 0; r < 8; r += 2) {
                    const float e0 = ev[qc][r], e1 = ev[qc][r + 1];
                    const float t0 = r < 4 ? d1[0][qc + 2][r] : d1[1][qc + 2][r - 4];
                    const float t1 = r < 4 ? d1[0][qc + 2][r + 1] : d1[1][qc + 2][r - 3];
                    ew[r / 2] = pack_bf16x2(e0, e1);
                    etw[r / 2] = pack_bf16x2(e0 * t0, e1 * t1);
                }
                pbuf[P][pair][qc][lane] = uint4{ew[0], ew[1], ew[2], ew[3]};
                pbuf[P][pair][qc + 2][lane] = uint4{etw[0], etw[1], etw[2], etw[3]};
                // every lane group holds the row's factor; all four write the
                // same value (no lane condition, so no branch splits the code)
                abuf[P][pair][qc][c] = alpha[qc];
            }
        };
        auto score_half = [&](int t, auto par, auto tail) __attribute__((always_inline)) {
            if (t >= pr.lo && t < pr.hi) {
                f32x4_t d1[2][4];
                scores(par, d1);
                // no masking when every key of the tile is in every row's range
                if (t * kPfKeys + kPfKeys - 1 <= pr.r0 && t * kPfKeys + kPfKeys <= S &&
                    (W == 0 || t * kPfKeys > pr.r0 + kPfRows - 1 - W))
                    numerators(t, par, d1, std::false_type{});
                else
                    numerators(t, par, d1, std::true_type{});
            }
            // an item's last position has parity 1; the value wave turns its
            // Z into log(sum e^s) at the next one
            if constexpr (STATS && decltype(par)::value == 1) {
                if (t == cur.tend - 1) {
                    mfin[cur.i & 1][pair][0][c] = mref[0];
                    mfin[cur.i & 1][pair][1][c] = mref[1];
                }
            }
            advance(t, par, tail);
        };
        // Two positions per trip fix each position's buffers and register
        // stages at compile time; both roles pass one barrier per position,
        // and one more after the last, where the value waves finish.
        prologue();
        if constexpr (!pf_persistent<D>()) {  // one item: a plain loop
            mref[0] = mref[1] = -INFINITY;
            for (int t = cur.t0; t < cur.tend; t += 2) {
                score_half(t, I0{}, Tail{});
                score_half(t + 1, I1{}, Tail{});
            }
        } else for (;;) {
            mref[0] = mref[1] = -INFINITY;
            int t = cur.t0;
            for (; t < cur.tend - 4; t += 2) {
                score_half(t, I0{}, Main{});
                score_half(t + 1, I1{}, Main{});
            }
            // the next item's q / rho, in flight during the tail (straight
            // code, so the compiler's wait counts stay exact and it waits for
            // them only two positions on); after the last item the current
            // rows again
            const PairRange nr = pair_range(nxt);
            load_x(xnext, nxt, nr);
            score_half(t, I0{}, Tail{});
            score_half(t + 1, I1{}, Tail{});
            score_half(t + 2, I0{}, Tail{});
            score_half(t + 3, I1{}, Tail{});
            if (cur.i + 1 >= n_mine) break;
            next_item();
            pr = nr;
            take_x();
        }
        advance(cur.tend, I0{}, Tail{});
    } else {
        // Value sums: acc[db][cb] = D2 rows d = 16db + 4g + j, column c of block
        // cb (E rows 0-15, 16-31, E*T rows 0-15, 16-31).  Block db = DB
        // multiplies a tile of ones, so its rows carry Z (cb < 2) and R (cb >= 2).
        f32x4_t acc[DB + 1][4];
        auto clear = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int db = 0; db <= DB; ++db)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) acc[db][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        };
        clear();

        auto value_tile = [&](auto par) __attribute__((always_inline)) {
            constexpr int P = decltype(par)::value;
            const float al0 = abuf[P][pair][0][c], al1 = abuf[P][pair][1][c];
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
                pop[cb] = __builtin_bit_cast(bf16x8_t, pbuf[P][pair][cb][lane]);
            const unsigned char *vt = vtile[P];
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

        // ---- o = a - (b - a r) per query row of item u (range x); lane (c, g)
        // holds d = 16db + 4g + j.  Output rows are written with non-temporal
        // stores (nothing here reads them again).  DEFER: o replaces the E
        // sums in the accumulators and store_outputs writes it later.
        auto store_outputs = [&](const Item &u, const PairRange &x) __attribute__((always_inline)) {
#pragma unroll
            for (int qc = 0; qc < 2; ++qc) {
                const int qi = x.r0 + 16 * qc + c;
                if (qi >= S) continue;
                float *orow = p.out + (int64_t)u.b * p.o_sb + (int64_t)qi * p.o_ss + (int64_t)x.head * p.o_sh;
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    __builtin_nontemporal_store(acc[db][qc], reinterpret_cast<f32x4_t *>(orow + 16 * db + 4 * g));
            }
        };
        auto epilogue = [&](const Item &u, const PairRange &x, auto defer) __attribute__((always_inline)) {
#pragma unroll
            for (int qc = 0; qc < 2; ++qc) {
                const int qi = x.r0 + 16 * qc + c;
                if (qi >= S) continue;
                const float inv = 1.0f / acc[DB][qc][0];
                const float r = acc[DB][qc + 2][0] * inv;
                const int64_t ooff =
                    (int64_t)u.b * p.o_sb + (int64_t)qi * p.o_ss + (int64_t)x.head * p.o_sh;
                float *orow = p.out + ooff;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    // fused steps written out: left to the compiler, the
                    // contraction would depend on whether a is also stored
                    // (o_SA), and the two builds would differ in the last bit
                    float o[4], a[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        a[j] = acc[db][qc][j] * inv;
                        const float bmar = __builtin_fmaf(inv, acc[db][qc + 2][j], -(a[j] * r));  // b - a r
                        o[j] = __builtin_fmaf(inv, acc[db][qc][j], -bmar);
                    }
                    // o_SA for a backward pass
                    if (STATS && p.o_sa != nullptr)
                        *reinterpret_cast<float4 *>(p.o_sa + ooff + 16 * db + 4 * g) =
                            float4{a[0], a[1], a[2], a[3]};
                    if constexpr (decltype(defer)::value)
                        acc[db][qc] = f32x4_t{o[0], o[1], o[2], o[3]};
                    else
                        __builtin_nontemporal_store(f32x4_t{o[0], o[1], o[2], o[3]},
                                                    reinterpret_cast<f32x4_t *>(orow + 16 * db + 4 * g));
                }
                // and the log of its softmax denominator (natural log; Z is
                // kept relative to 2^m) and r
                if constexpr (STATS) {
                    const int64_t ri = ((int64_t)u.b * p.num_q_heads + x.head) * S + qi;
                    if (p.lse != nullptr && g == 0)
                        p.lse[ri] = (mfin[u.i & 1][pair][qc][c] + __builtin_log2f(acc[DB][qc][0])) *
                                    0.6931471805599453f;
                    if (p.rmean != nullptr && g == 0) p.rmean[ri] = r;
                }
            }
        };
        // Position t sums the tile of position t - 1 (parity 1 - P).  At an
        // item's first position that is the previous item's last position,
        // whose outputs are then written: stored after the position's
        // barrier, since the staging wait before it counts the stores too
        // (the memory counter holds loads and stores, and the wait is sized
        // for the positions without stores) and would hold the wave until
        // they were written.
        PairRange pr = pair_range(cur), pv = pr;
        Item prv = cur;
        auto value_half = [&](int t, auto par, auto tail) __attribute__((always_inline)) {
            using Q = std::integral_constant<int, 1 - decltype(par)::value>;
            // (one copy of the tile code: the item boundary only picks the
            // position and range)
            const bool first = decltype(par)::value == 0 && t == cur.t0;
            const int u = first ? prv.tend - 1 : t - 1;
            const int lo = first ? pv.lo : pr.lo, hi = first ? pv.hi : pr.hi;
            if (u >= lo && u < hi && (!first || cur.i > 0)) value_tile(Q{});
            if (first && cur.i > 0) epilogue(prv, pv, std::true_type{});
            advance(t, par, tail);
            if (first && cur.i > 0) {
                store_outputs(prv, pv);
                clear();
            }
        };

        prologue();
        if constexpr (!pf_persistent<D>()) {  // one item: a plain loop
            for (int t = cur.t0; t < cur.tend; t += 2) {
                value_half(t, I0{}, Tail{});
                value_half(t + 1, I1{}, Tail{});
            }
        } else for (;;) {
            int t = cur.t0;
            for (; t < cur.tend - 4; t += 2) {
                value_half(t, I0{}, Main{});
                value_half(t + 1, I1{}, Main{});
            }
            value_half(t, I0{}, Tail{});
            value_half(t + 1, I1{}, Tail{});
            value_half(t + 2, I0{}, Tail{});
            value_half(t + 3, I1{}, Tail{});
            if (cur.i + 1 >= n_mine) break;
            prv = cur;
            pv = pr;
            next_item();
            pr = pair_range(cur);
        }
        // the position after the last: its last tile and outputs
        if (cur.tend - 1 >= pr.lo && cur.tend - 1 < pr.hi) value_tile(I1{});
        epilogue(cur, pr, std::false_type{});
        advance(cur.tend, I0{}, Tail{});
    }
}

// GQA groups 8 and 16: G / 4 workgroups of four query heads each per KV head
// (each loads the KV tiles once for its four heads).
// Compute units of the stream's device (cached per device).
int device_cus(hipStream_t stream) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = -1;
    if ((stream == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(stream, &dev)) != hipSuccess ||
        dev < 0)
        return 0;
    if (dev < kMaxDevices) {
        const int n = cache[dev].load(std::memory_order_relaxed);
        if (n > 0) return n;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

template <int D>
hipError_t launch_prefill_d(const PrefillParams &pin, hipStream_t stream) {
    PrefillParams p = pin;
    const int group = p.num_q_heads / p.num_kv_heads;
    const int G = group > 4 ? 4 : group;  // query heads per workgroup
    p.head_blocks = group / G;
    const int units = p.batch * p.num_kv_heads * p.head_blocks;
    const int qb_rows = kPfRows * kPfPairs / G;
    const int64_t nitems = (int64_t)units * ((p.seq_len + qb_rows - 1) / qb_rows);
    int64_t wgs = nitems;  // one item per workgroup
    p.persist = 0;
    p.static_rounds = 0;
    if (pf_persistent<D>()) {
        // one persistent workgroup per CU (a multiple of 8, see the work
        // list), or the caller's count; all rounds but the last full one
        // and the remainder run on them
        int64_t cap = p.workgroups;
        if (cap <= 0) {
            const int cus = device_cus(stream);
            if (cus <= 0) return hipErrorInvalidDevice;
            cap = cus >= 8 ? cus / 8 * 8 : cus;
        }
        cap = std::min(nitems, cap);
        const int64_t rounds = nitems / cap - 1;
        if (rounds >= 1) {
            p.persist = (int32_t)cap;
            p.static_rounds = (int32_t)rounds;
            wgs = cap + (nitems - rounds * cap);
        }
    }
    const dim3 grid((unsigned)wgs);
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
