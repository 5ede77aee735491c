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
//   scores  D1[key][col] = K[key][:] . X[col][:]   X = the wave's 32 q rows
//           and its 32 rho rows (64 columns, 4 blocks of 16);
//   sums    D2[d][col]   = sum_key V[key][d] . P[key][col]   P = E (32 cols)
//           and E*T (32 cols), E = e^{s - m} rounded to bf16;
// all as 16x16x32 bf16 MFMAs with fp32 accumulation.  s and t of the same
// query row land in the same lane, so the softmax needs no data movement
// except the row max across the four lane groups; the rescale of a row's
// sums is a per-lane multiply.
//
// Workgroup: 4 waves (one per SIMD; each holds 32 query rows, its Q / rho
// operands and 128 accumulators) covering 128/G rows of each of the G query
// heads of one KV head, so every K/V tile in LDS serves the whole GQA group.
// K/V tiles of 32 keys are double-buffered in LDS (one barrier per tile; K
// is two tiles and V one tile ahead of the math, their global loads in
// flight during the current tile's math).  The next tile's score MFMAs are
// interleaved with the current tile's softmax VALU work (one wave per SIMD
// has nothing else to overlap them with).  V reaches the MFMA through
// ds_read_b64_tr_b16.  Query blocks are scheduled longest (highest causal
// row) first; tiles past a wave's last row are skipped.
#include "kernels.hpp"

#include <math.h>

#include <type_traits>

namespace plx {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPfWaves = 4;               // waves per workgroup
constexpr int kPfRows = 32;               // query rows per wave
constexpr int kPfKeys = 32;               // keys per tile
constexpr int kPfD = 128;                 // head dim
constexpr int kPfRowBytes = 2 * kPfD + 16;  // LDS bytes per tile row (16-byte pad)
constexpr float kSlack = 8.0f;            // base-2 headroom before a row's reference max moves

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

// Max over the four 16-lane groups (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float group_max(float x) {
    const int xi = __builtin_bit_cast(int, x);
    auto a = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);  // rows 0<->1, 2<->3
    x = fmaxf(__builtin_bit_cast(float, (int)a[0]), __builtin_bit_cast(float, (int)a[1]));
    const int yi = __builtin_bit_cast(int, x);
    auto b2 = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);  // halves 0<->1
    return fmaxf(__builtin_bit_cast(float, (int)b2[0]), __builtin_bit_cast(float, (int)b2[1]));
}

template <int G>
__global__ __launch_bounds__(64 * kPfWaves) void prefill_kernel(PrefillParams p) {
    constexpr int D = kPfD;
    constexpr int KS = D / 32;                      // score MFMAs per 16-key block
    constexpr int DB = D / 16;                      // 16-row blocks of the value sums
    constexpr int WPH = kPfWaves / G;               // waves per query head
    constexpr int QB = kPfRows * WPH;               // query rows per head per workgroup
    constexpr int TILE = kPfKeys * kPfRowBytes;

    __shared__ __attribute__((aligned(16))) unsigned char ktile[2][TILE];
    __shared__ __attribute__((aligned(16))) unsigned char vtile[2][TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int S = p.seq_len;
    const float c2 = p.scale_log2;

    const int units = p.batch * p.num_kv_heads;
    const int nqb = (S + QB - 1) / QB;
    const int qb = nqb - 1 - (int)(blockIdx.x / units);  // longest causal rows first
    const int unit = blockIdx.x % units;
    const int b = unit / p.num_kv_heads;
    const int hk = unit % p.num_kv_heads;
    const int head = hk * G + wave / WPH;
    const int r0 = qb * QB + (wave % WPH) * kPfRows;  // first query row of this wave
    const int key_end = min(S, (qb + 1) * QB);        // keys this workgroup needs
    const int ntiles = (key_end + kPfKeys - 1) / kPfKeys;
    const int wave_tiles = min(ntiles, (min(S, r0 + kPfRows) + kPfKeys - 1) / kPfKeys);

    // ---- cooperative tile loads: thread t moves 16 bytes of key 16u + t/16.
    // K runs two tiles ahead of the math and V one tile ahead, so the scores
    // of tile t+1 can be computed while tile t's softmax runs.
    const uint16_t *kg = p.k + (int64_t)b * p.k_sb + (int64_t)hk * p.k_sh;
    const uint16_t *vg = p.v + (int64_t)b * p.v_sb + (int64_t)hk * p.v_sh;
    uint4 kst[2], vst[2];
    auto issue_k = [&](int t) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int key = min(t * kPfKeys + 16 * u + tid / 16, S - 1);
            kst[u] = ld16(kg + (int64_t)key * p.k_ss + 8 * (tid % 16));
        }
    };
    auto issue_v = [&](int t) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int key = min(t * kPfKeys + 16 * u + tid / 16, S - 1);
            vst[u] = ld16(vg + (int64_t)key * p.v_ss + 8 * (tid % 16));
        }
    };
    auto store = [&](unsigned char *tile, const uint4 (&st)[2]) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
            *reinterpret_cast<uint4 *>(tile + (16 * u + tid / 16) * kPfRowBytes + 16 * (tid % 16)) =
                st[u];
    };

    issue_k(0);
    issue_v(0);

    // ---- query-side operands: column block cb < 2 holds q rows r0 + 16cb + c,
    // cb >= 2 the rho rows of the same queries; head-dim value 32g + 8ks + i
    // sits in k-slot 8g + i of score MFMA ks (the same slots the K operand uses)
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
            xop[cb][ks] = __builtin_bit_cast(bf16x8_t, ld16(src + 32 * g + 8 * ks));
    }

    // Value sums: acc[db][cb] = D2 rows d = 16db + 4g + j, column c of block
    // cb (E rows 0-15, 16-31, E*T rows 0-15, 16-31).  Block db = DB multiplies
    // a tile of ones, so its rows carry Z (cb < 2) and R (cb >= 2).
    f32x4_t acc[DB + 1][4];
#pragma unroll
    for (int db = 0; db <= DB; ++db)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[db][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float mref[2] = {-INFINITY, -INFINITY};  // base-2 reference max per query row

    auto scores = [&](int t, f32x4_t (&d1)[2][4]) {
        const unsigned char *kt = ktile[t & 1];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) d1[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8_t kop = __builtin_bit_cast(
                    bf16x8_t, ld16(kt + (16 * rb + c) * kPfRowBytes + 64 * g + 16 * ks));
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
                    d1[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, xop[cb][ks],
                                                                         d1[rb][cb], 0, 0, 0);
            }
        }
    };

    // Softmax numerators of tile t: E = 2^(c2 s - m) and E*T in bf16, as the
    // B operands of the value MFMAs; k-slot r holds key 4g + r (r < 4) or
    // 16 + 4g + r - 4 of the tile.  MASK: the tile crosses the diagonal or S.
    // Branch-free: a row's reference max moves (by select) only when the
    // tile's max exceeds it by more than kSlack; alpha[qc] < 1 then tells the
    // caller to rescale that row's sums before this tile's value MFMAs.
    auto numerators = [&](int t, const f32x4_t (&d1)[2][4], bf16x8_t (&pop)[4],
                          float (&alpha)[2], auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
        for (int qc = 0; qc < 2; ++qc) {
            const int qi = r0 + 16 * qc + c;
            float sv[8];
            float tmax = -INFINITY;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                sv[r] = r < 4 ? d1[0][qc][r] : d1[1][qc][r - 4];
                if constexpr (MASK) {
                    const int key = t * kPfKeys + (r < 4 ? 4 * g + r : 16 + 4 * g + r - 4);
                    sv[r] = key <= qi && key < S ? sv[r] : -INFINITY;
                }
                tmax = __builtin_fmaxf(tmax, sv[r]);
            }
            const float tm2 = group_max(tmax) * c2;
            const float mnew = tm2 > mref[qc] + kSlack ? tm2 : mref[qc];
            alpha[qc] = __builtin_amdgcn_exp2f(mref[qc] - mnew);  // 1 unless moved; 0 at start
            mref[qc] = mnew;
            uint32_t ew[4], etw[4];
#pragma unroll
            for (int r = 0; r < 8; r += 2) {
                const float e0 = __builtin_amdgcn_exp2f(fmaf(sv[r], c2, -mnew));
                const float e1 = __builtin_amdgcn_exp2f(fmaf(sv[r + 1], c2, -mnew));
                const float t0 = r < 4 ? d1[0][qc + 2][r] : d1[1][qc + 2][r - 4];
                const float t1 = r < 4 ? d1[0][qc + 2][r + 1] : d1[1][qc + 2][r - 3];
                ew[r / 2] = pack_bf16x2(e0, e1);
                etw[r / 2] = pack_bf16x2(e0 * t0, e1 * t1);
            }
            pop[qc] = __builtin_bit_cast(bf16x8_t, uint4{ew[0], ew[1], ew[2], ew[3]});
            pop[qc + 2] = __builtin_bit_cast(bf16x8_t, uint4{etw[0], etw[1], etw[2], etw[3]});
        }
    };

    // Rows whose reference max moved: scale their sums (rare after tile 0).
    auto rescale = [&](const float (&alpha)[2]) {
        if (__builtin_amdgcn_ballot_w64(alpha[0] != 1.0f || alpha[1] != 1.0f)) {
#pragma unroll
            for (int db = 0; db <= DB; ++db)
#pragma unroll
                for (int qc = 0; qc < 2; ++qc) {
                    acc[db][qc] *= alpha[qc];
                    acc[db][qc + 2] *= alpha[qc];
                }
        }
    };

    auto value_sums = [&](int t, const bf16x8_t (&pop)[4]) {
        const unsigned char *vt = vtile[t & 1];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
            const int col = 16 * db + 4 * (c % 4);
            const unsigned char *a0 = vt + (4 * g + c / 4) * kPfRowBytes + 2 * col;
            const unsigned char *a1 = vt + (16 + 4 * g + c / 4) * kPfRowBytes + 2 * col;
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
            acc[DB][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pop[cb], acc[DB][cb], 0, 0, 0);
    };

    // prologue: K tiles 0 and 1 and V tile 0 in LDS, K tile 2 and V tile 1 in flight
    store(ktile[0], kst);
    store(vtile[0], vst);
    if (ntiles > 1) {
        issue_k(1);
        store(ktile[1], kst);
    }
    if (ntiles > 2) issue_k(2);
    if (ntiles > 1) issue_v(1);
    __syncthreads();

    // One tile of math.  The next tile's score MFMAs (independent of this
    // tile's softmax) are interleaved with the softmax VALU work; the tile's
    // value MFMAs follow.  The scores of the tile after the wave's last one
    // read a stale (in-bounds) LDS tile and are never used.
    auto tile = [&](int t, const f32x4_t (&d1)[2][4], f32x4_t (&d1n)[2][4], auto mask_tag) {
        bf16x8_t pop[4];
        float alpha[2];
        scores(t + 1, d1n);
        numerators(t, d1, pop, alpha, mask_tag);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one score MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // then softmax VALU
        }
        rescale(alpha);
        value_sums(t, pop);
    };
    auto step = [&](int t, const f32x4_t (&d1)[2][4], f32x4_t (&d1n)[2][4]) {
        if (t < wave_tiles) {
            const bool full = t * kPfKeys + kPfKeys - 1 <= r0 && t * kPfKeys + kPfKeys <= S;
            if (full)
                tile(t, d1, d1n, std::false_type{});
            else
                tile(t, d1, d1n, std::true_type{});
        }
        // K tile t+2 replaces tile t (last read by scores(t) one iteration ago);
        // V tile t+1 replaces tile t-1 (last read by value_sums(t-1))
        if (t + 2 < ntiles) store(ktile[t & 1], kst);
        if (t + 1 < ntiles) store(vtile[(t + 1) & 1], vst);
        if (t + 3 < ntiles) issue_k(t + 3);
        if (t + 2 < ntiles) issue_v(t + 2);
        __syncthreads();
    };

    f32x4_t d1a[2][4], d1b[2][4];
    scores(0, d1a);
    for (int t = 0; t < ntiles; t += 2) {  // two tiles per trip: score buffers swap roles
        step(t, d1a, d1b);
        if (t + 1 < ntiles) step(t + 1, d1b, d1a);
    }

    // ---- o = a - (b - a r) per query row; lane (c, g) holds d = 16db + 4g + j
#pragma unroll
    for (int qc = 0; qc < 2; ++qc) {
        const int qi = r0 + 16 * qc + c;
        if (qi >= S) continue;
        const float inv = 1.0f / acc[DB][qc][0];
        const float r = acc[DB][qc + 2][0] * inv;
        float *orow = p.out + (int64_t)b * p.o_sb + (int64_t)qi * p.o_ss + (int64_t)head * p.o_sh;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            float o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a = acc[db][qc][j] * inv, bb = acc[db][qc + 2][j] * inv;
                o[j] = a - (bb - a * r);
            }
            *reinterpret_cast<float4 *>(orow + 16 * db + 4 * g) = float4{o[0], o[1], o[2], o[3]};
        }
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams &p, int d, hipStream_t stream) {
    if (d != kPfD) return hipErrorInvalidValue;
    const int G = p.num_q_heads / p.num_kv_heads;
    const int units = p.batch * p.num_kv_heads;
    const int qb_rows = kPfRows * kPfWaves / G;
    const dim3 grid((unsigned)(units * ((p.seq_len + qb_rows - 1) / qb_rows)));
    const dim3 block(64 * kPfWaves);
    switch (G) {
        case 1: hipLaunchKernelGGL(prefill_kernel<1>, grid, block, 0, stream, p); break;
        case 2: hipLaunchKernelGGL(prefill_kernel<2>, grid, block, 0, stream, p); break;
        case 4: hipLaunchKernelGGL(prefill_kernel<4>, grid, block, 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace plx
