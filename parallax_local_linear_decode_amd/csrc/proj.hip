// proj.hip -- the query and probe projections q = W_Q x and rho = W_R x in
// one launch (page "Parallax: Parameterized Local Linear Attention Gives
// Transformers a 'Second Eye'", section 1.3: the probe is a learned linear
// map of the layer input, costing about one extra projection matrix).
//
// The two weight matrices are treated as one stacked [2N, D] matrix
// (N = heads * head_dim), so every token row of x is read once for both
// outputs, and the results land directly in the strided [T, Hq, d] layouts
// the attention kernels read (fp32 for decode, bf16 for prefill).
//
// Three kernels, by token count, all on bf16 MFMAs with fp32 accumulation
// (the two LDS-tiled ones add the k terms of an output element in the same
// order, so their results agree bit for bit):
//  * up to 128 tokens (decode), proj_kernel: bound by streaming the weights
//    from HBM.  Workgroup: 16 RT stacked weight rows x 16 NT tokens; its
//    eight waves split the model dimension D into eighths, each accumulating
//    partial 16 x 16 tiles; the partials are summed in LDS in wave order.
//    One row tile per workgroup (2N / 16 workgroups, 256 for 2N = 4096, so
//    every CU streams), and a wave issues all loads of its eighth of D before
//    the MFMAs, so the whole weight set is requested at once.  From 65 to 128
//    tokens two row tiles per workgroup let one token load serve two weight
//    loads.
//  * prefill sizes, proj_tiled_kernel: an LDS-tiled GEMM, 256 x 256 tiles on
//    eight waves (or 128 x 128 on four), loads one chunk ahead in registers.
//  * prefill sizes with N a multiple of 256, proj_big_kernel: 256 x 256 tiles
//    on four waves of 128 x 128, fed by global->LDS loads through two LDS
//    stages of 64-wide K chunks.
#include "kernels.hpp"

#include <atomic>
#include <type_traits>

namespace plx {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t ld_bf16x8(const uint16_t *p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(p));
}

constexpr int kWaves = 8;  // waves per workgroup, each one eighth of D

template <int RT, int NT, bool BF16OUT>
__global__ __launch_bounds__(64 * kWaves) void proj_kernel(ProjParams p) {
    constexpr int kRows = 16 * RT;  // stacked weight rows per workgroup
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar loop
    const int c = lane & 15;
    const int g = lane >> 4;
    const int row0 = blockIdx.x * kRows;  // first stacked row: [0, N) W_Q, [N, 2N) W_R
    const bool is_r = row0 >= p.n;        // N is a multiple of 32: a block never straddles
    const int f0 = row0 - (is_r ? p.n : 0);
    const int t0 = blockIdx.y * 16 * NT;
    const int T = p.tokens;

    // A operands: weight rows f0 + 16 rt + c, model dims k + 8g .. k + 8g + 7;
    // B operands: token rows t0 + 16 nt + c, the same model dims.
    const uint16_t *w[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        w[rt] = (is_r ? p.w_r : p.w_q) + (int64_t)(f0 + 16 * rt + c) * p.w_sn + 8 * g;
    const uint16_t *xr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        xr[nt] = p.x + (int64_t)min(t0 + 16 * nt + c, T - 1) * p.x_st + 8 * g;

    const int kq = p.model_dim / kWaves;
    const int k_begin = wave * kq;
    const int steps = kq / 32;
    f32x4_t acc[RT][NT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // CH steps' loads are issued together, then their MFMAs: with one row
    // tile a wave's whole eighth of D = 2048 is in flight per lane
    constexpr int CH = RT == 1 ? 8 : 2;
    int st = 0;
    for (; st + CH <= steps; st += CH) {
        bf16x8_t a[CH][RT], b[CH][NT];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int k = k_begin + 32 * (st + i);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) a[i][rt] = ld_bf16x8(w[rt] + k);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) b[i][nt] = ld_bf16x8(xr[nt] + k);
        }
        // keep the scheduler from interleaving the MFMAs into the loads (it
        // would trade loads in flight for registers)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < CH; ++i)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][rt], b[i][nt],
                                                                          acc[rt][nt], 0, 0, 0);
    }
    for (; st < steps; ++st) {
        const int k = k_begin + 32 * st;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const bf16x8_t a = ld_bf16x8(w[rt] + k);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ld_bf16x8(xr[nt] + k),
                                                                      acc[rt][nt], 0, 0, 0);
        }
    }

    __shared__ f32x4_t red[kWaves][RT][NT][64];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) red[wave][rt][nt][lane] = acc[rt][nt];
    __syncthreads();

    // wave w finishes tiles u = w, w + 8, ... of the 2 NT (row tile, token
    // block) pairs; lane (c, g) holds features f0 + 16 rt + 4g + j (j = 0..3)
    // of token t0 + 16 nt + c
    for (int u = wave; u < RT * NT; u += kWaves) {
        const int rt = u % RT, nt = u / RT;
        const int t = t0 + 16 * nt + c;
        if (t >= T) continue;
        f32x4_t s = red[0][rt][nt][lane];
#pragma unroll
        for (int w2 = 1; w2 < kWaves; ++w2) s += red[w2][rt][nt][lane];
        const int f = f0 + 16 * rt + 4 * g;
        const int h = f / p.head_dim, e = f % p.head_dim;
        const int64_t off = (int64_t)t * (is_r ? p.r_st : p.q_st) +
                            (int64_t)h * (is_r ? p.r_sh : p.q_sh) + e;
        if constexpr (BF16OUT) {
            typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
            const bf16x4_t v = {(__bf16)s[0], (__bf16)s[1], (__bf16)s[2], (__bf16)s[3]};
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(is_r ? p.rho : p.q) + off) =
                __builtin_bit_cast(uint2, v);
        } else {
            *reinterpret_cast<float4 *>(static_cast<float *>(is_r ? p.rho : p.q) + off) =
                float4{s[0], s[1], s[2], s[3]};
        }
    }
}

template <int RT, int NT>
hipError_t launch_nt(const ProjParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)(2 * p.n / (16 * RT)), (unsigned)((p.tokens + 16 * NT - 1) / (16 * NT)));
    if (p.out_bf16)
        hipLaunchKernelGGL((proj_kernel<RT, NT, true>), grid, dim3(64 * kWaves), 0, stream, p);
    else
        hipLaunchKernelGGL((proj_kernel<RT, NT, false>), grid, dim3(64 * kWaves), 0, stream, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------- tiled ---
// Prefill sizes (many tokens): a plain GEMM C[t][n] = sum_k x[t][k] W[n][k]
// with both operands contiguous in k.  Workgroup tile: MT stacked weight rows
// x NT tokens, WM x WN waves of 16 TI x 16 TJ (TI x TJ MFMA tiles each).  K
// advances in chunks of 64 through a double-buffered LDS tile pair; each
// chunk's global loads run one chunk ahead through registers (every thread
// moves four 16-byte pieces of each operand), and both the loads and the
// LDS stores are spread one or two at a time between the MFMAs, so the
// matrix cores do not idle while a workgroup stages.  Per k the workgroup
// loads (MT + NT) * 2 bytes for 2 MT NT flops: the 256 x 256 tile halves the
// L2 traffic per flop of the 128 x 128 one.
constexpr int kChunk = 64;                       // k per LDS chunk
constexpr int kCUs = 256;                        // compute units of an MI355X
constexpr int kLdsRow = kChunk * 2 + 16;         // 144-byte rows: 16 rows on distinct banks

template <int WM_, int WN_, int TI_, int TJ_>
struct TileCfg {
    static constexpr int WM = WM_, WN = WN_, TI = TI_, TJ = TJ_;
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int kMT = 16 * TI * WM;  // stacked weight rows
    static constexpr int kNT = 16 * TJ * WN;  // tokens
    static constexpr int kLdsW = kMT * kLdsRow;
    static constexpr int kLdsX = kNT * kLdsRow;
    static constexpr int kStride = kThreads / 8;  // loader row stride
    static_assert(kMT == 4 * kStride && kNT == 4 * kStride, "four pieces per thread and operand");
};
using Tile128 = TileCfg<2, 2, 4, 4>;
using Tile256 = TileCfg<2, 4, 8, 4>;

template <class C, bool BF16OUT>
__global__ __launch_bounds__(C::kThreads) void proj_tiled_kernel(ProjParams p) {
    constexpr int TI = C::TI, TJ = C::TJ, WM = C::WM;
    __shared__ __attribute__((aligned(16))) unsigned char wt[2][C::kLdsW];
    __shared__ __attribute__((aligned(16))) unsigned char xt[2][C::kLdsX];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int wr = wave % WM, wc = wave / WM;  // wave's row block (weights), column block (tokens)
    const int row0 = blockIdx.x * C::kMT;      // first stacked weight row
    const int t0 = blockIdx.y * C::kNT;
    const int T = p.tokens;

    // loader: thread tid moves row tid / 8 + kStride i, 16-byte piece tid % 8
    // of both operands; offsets from the operand bases (no pointer arrays:
    // the compiler kept those in scratch memory)
    const int lrow = tid / 8, lpc = tid % 8;
    int64_t woff[4], xoff[4];
    bool wr_is_r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = row0 + lrow + C::kStride * i;  // stacked row (< 2N: 2N is a multiple of kMT)
        wr_is_r[i] = r >= p.n;
        woff[i] = (int64_t)(wr_is_r[i] ? r - p.n : r) * p.w_sn + 8 * lpc;
        xoff[i] = (int64_t)min(t0 + lrow + C::kStride * i, T - 1) * p.x_st + 8 * lpc;
    }
    uint4 ws0, ws1, ws2, ws3, xs0, xs1, xs2, xs3;  // staging registers, one chunk
    // piece j (0-7) of the staging: j < 4 the weight rows, else the tokens
    auto store_piece = [&](int j, int buf) __attribute__((always_inline)) {
        constexpr int RS = C::kStride * kLdsRow;
        unsigned char *d = (j < 4 ? wt[buf] : xt[buf]) + lrow * kLdsRow + 16 * lpc + (j & 3) * RS;
        const uint4 v = j == 0 ? ws0 : j == 1 ? ws1 : j == 2 ? ws2 : j == 3 ? ws3
                      : j == 4 ? xs0 : j == 5 ? xs1 : j == 6 ? xs2 : xs3;
        *reinterpret_cast<uint4 *>(d) = v;
    };
    auto issue_piece = [&](int j, int k0) __attribute__((always_inline)) {
        if (j < 4) {
            const uint4 v = *reinterpret_cast<const uint4 *>((wr_is_r[j] ? p.w_r : p.w_q) + woff[j] + k0);
            if (j == 0) ws0 = v;
            else if (j == 1) ws1 = v;
            else if (j == 2) ws2 = v;
            else ws3 = v;
        } else {
            const uint4 v = *reinterpret_cast<const uint4 *>(p.x + xoff[j - 4] + k0);
            if (j == 4) xs0 = v;
            else if (j == 5) xs1 = v;
            else if (j == 6) xs2 = v;
            else xs3 = v;
        }
    };

    f32x4_t acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nchunks = p.model_dim / kChunk;
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_piece(j, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) store_piece(j, 0);
    if (nchunks > 1)
#pragma unroll
        for (int j = 0; j < 8; ++j) issue_piece(j, kChunk);
    __syncthreads();
    for (int ch = 0; ch < nchunks; ++ch) {
        const int buf = ch & 1;
        // Chunk ch + 1 (loaded during chunk ch - 1) goes to the other buffer,
        // free since the barrier that ended chunk ch - 1, in the first k half;
        // the registers take chunk ch + 2 in the second.  Both are spread
        // over the MFMAs.  On the last chunks the loads repeat the last chunk
        // and the stores hit a buffer nobody reads again.
        const int k2 = min(ch + 2, nchunks - 1) * kChunk;
#pragma unroll
        for (int kk = 0; kk < kChunk / 32; ++kk) {
            bf16x8_t b[TJ];
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                b[j] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const uint4 *>(
                                  xt[buf] + (16 * TJ * wc + 16 * j + c) * kLdsRow + 64 * kk + 16 * g));
            auto aread = [&](int i) __attribute__((always_inline)) {
                return __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const uint4 *>(
                                  wt[buf] + (16 * TI * wr + 16 * i + c) * kLdsRow + 64 * kk + 16 * g));
            };
            bf16x8_t a = aread(0);
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const bf16x8_t an = aread(i + 1 < TI ? i + 1 : i);
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[i][j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = 0; q < 8 / TI; ++q) {
                    if (kk == 0) store_piece(i * (8 / TI) + q, 1 - buf);
                    else issue_piece(i * (8 / TI) + q, k2);
                }
                __builtin_amdgcn_sched_barrier(0);
                a = an;
            }
        }
        __syncthreads();
    }

    // acc[i][j]: lane (c, g) holds stacked rows row0 + 16 TI wr + 16 i + 4g +
    // (0..3) of token t0 + 16 TJ wc + 16 j + c
#pragma unroll
    for (int i = 0; i < TI; ++i) {
        const int r = row0 + 16 * TI * wr + 16 * i + 4 * g;  // the 16-row tile never straddles N
        const bool is_r = r >= p.n;
        const int f = r - (is_r ? p.n : 0);
        const int h = f / p.head_dim, e = f % p.head_dim;
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int t = t0 + 16 * TJ * wc + 16 * j + c;
            if (t >= T) continue;
            const int64_t off = (int64_t)t * (is_r ? p.r_st : p.q_st) +
                                (int64_t)h * (is_r ? p.r_sh : p.q_sh) + e;
            const f32x4_t s = acc[i][j];
            if constexpr (BF16OUT) {
                typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
                const bf16x4_t v = {(__bf16)s[0], (__bf16)s[1], (__bf16)s[2], (__bf16)s[3]};
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(is_r ? p.rho : p.q) + off) =
                    __builtin_bit_cast(uint2, v);
            } else {
                *reinterpret_cast<float4 *>(static_cast<float *>(is_r ? p.rho : p.q) + off) =
                    float4{s[0], s[1], s[2], s[3]};
            }
        }
    }
}

template <class C>
hipError_t launch_tiled(const ProjParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)(2 * p.n / C::kMT), (unsigned)((p.tokens + C::kNT - 1) / C::kNT));
    if (p.out_bf16)
        hipLaunchKernelGGL((proj_tiled_kernel<C, true>), grid, dim3(C::kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((proj_tiled_kernel<C, false>), grid, dim3(C::kThreads), 0, stream, p);
    return hipGetLastError();
}

// ------------------------------------------------------------ big tiles ---
// The largest prefill sizes (N a multiple of 256 and enough 256 x 256 tiles
// to fill the CUs): 256 x 256 output tiles on four waves of 128 x 128 each
// (8 x 8 16x16x32 MFMA tiles, 256 fp32 accumulators per lane, which only fit
// in the accumulation registers).  Per k a wave reads (128 + 128) * 2 bytes
// from LDS for 2 * 128 * 128 flops, half the LDS traffic per flop of the
// eight-wave tile.
//
// K runs in chunks of 64 through two LDS stages of 64 KB (the weight tile,
// then the token tile, 128-byte rows), filled by global->LDS buffer loads
// (16 bytes per lane, no staging registers, no LDS store instructions).  A
// load instruction writes 1 KB = eight 128-byte rows in lane order (so every
// request is a whole 128-byte line), and rows cannot be padded: the eight
// 16-byte pieces of row R are stored in the order piece ^ (R % 8) instead,
// which puts the eight rows one operand read touches on distinct banks.  A
// chunk is two k-steps of 32, each 64 MFMAs per wave on operands read one
// k-step ahead into a second register set: the second k-step's reads run
// under the first one's MFMAs; then one barrier publishes chunk c + 1's stage
// (every wave has waited for its own loads of it) and frees chunk c's (every
// wave has its operands in registers), which takes chunk c + 2's loads while
// chunk c + 1's first k-step is read, both under the second k-step's MFMAs.
constexpr int kBigT = 256;                    // tile rows and tokens
constexpr int kBigK = 64;                     // k per stage
constexpr int kBigRow = kBigK * 2;            // 128-byte rows
constexpr int kBigOp = kBigT * kBigRow;       // one operand of one stage
constexpr int kBigStage = 2 * kBigOp;         // weights then tokens
static_assert(2 * kBigStage <= 160 * 1024, "two stages fit the 160 KB of LDS of a gfx950 CU");

// s_waitcnt immediates: vector memory count (bits 3:0 and 15:14) 0 pending,
// LDS count (bits 11:8) 0, export count (6:4) free;
// kWaitLds: the LDS count only (vector memory count 63);
// kWait16: as kWait0 but 16 vector memory operations may still be pending
constexpr int kWait0 = 0x0070, kWaitLds = 0xC07F, kWait16 = 0x4070;

// The workgroup barrier of the big-tile kernel, after the caller's explicit
// wait.  __syncthreads() would add a release fence, for which the compiler
// may wait for every pending vector memory operation (at the output's
// barriers: the next tile's loads and this tile's stores, which need no
// wait); the empty asm statements keep the compiler from moving memory
// accesses across the barrier instead.
__device__ __forceinline__ void big_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <bool BF16OUT>
__global__ __launch_bounds__(256) void proj_big_kernel(ProjParams p, int n_rb, int n_tb) {
    __shared__ __attribute__((aligned(1024))) unsigned char st0[kBigStage];
    __shared__ __attribute__((aligned(1024))) unsigned char st1[kBigStage];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15;
    const int g = lane >> 4;
    const int T = p.tokens;
    const int nt = n_rb * n_tb;

    // One workgroup per CU runs tiles blockIdx.x, + gridDim.x, ... (the
    // grid is a multiple of 8, so a workgroup's tiles stay on its XCD); the
    // next tile's first loads are issued before this tile's outputs are
    // stored.  Tile order: workgroups are dealt to the eight XCDs in turn,
    // so when the tile count divides by 8, XCD x gets the x-th eighth of the
    // order; the order walks groups of four token blocks, row block by row
    // block, so the 32 tiles an XCD runs at a time cover 4 token blocks x 8
    // row blocks and share those tiles in its L2.
    struct Tile {
        int row0, t0;
        bool is_r;
    };
    auto tile_of = [&](int bid) __attribute__((always_inline)) {
        Tile ti;
        const int lid = nt % 8 == 0 ? (bid % 8) * (nt / 8) + bid / 8 : bid;
        const int grp = lid / (4 * n_rb);
        const int gsz = min(4, n_tb - 4 * grp);
        const int in = lid - grp * 4 * n_rb;
        const int tb = 4 * grp + in % gsz, rb = in / gsz;
        ti.row0 = rb * kBigT;
        ti.t0 = tb * kBigT;
        ti.is_r = ti.row0 >= p.n;  // N is a multiple of 256: a tile never straddles
        return ti;
    };
    // Buffer resources over a tile's weight rows and token rows: a load past
    // the last token row returns zeros (those outputs are not stored); byte
    // offsets fit 32 bits (the launcher checks 256 * stride * 2 < 2^31).
    auto wres_of = [&](const Tile &ti) __attribute__((always_inline)) {
        const uint16_t *wbase =
            (ti.is_r ? p.w_r : p.w_q) + (int64_t)(ti.row0 - (ti.is_r ? p.n : 0)) * p.w_sn;
        return __builtin_amdgcn_make_buffer_rsrc((void *)wbase, (short)0,
                                                 (int)(((kBigT - 1) * p.w_sn + p.model_dim) * 2), 0x00020000);
    };
    auto xres_of = [&](const Tile &ti) __attribute__((always_inline)) {
        const uint16_t *xbase = p.x + (int64_t)ti.t0 * p.x_st;
        return __builtin_amdgcn_make_buffer_rsrc(
            (void *)xbase, (short)0,
            (int)(((min(T - ti.t0, kBigT) - 1) * (int64_t)p.x_st + p.model_dim) * 2), 0x00020000);
    };

    // Loads: wave w fills rows 64 w + 8 j + lane / 8 (j = 0..7) of both
    // operands; lane i lands at byte 16 i of its instruction's 1 KB, i.e.
    // physical piece i % 8 of its row, which holds logical piece
    // (i % 8) ^ (row % 8) (row % 8 == lane / 8 for every j).
    const int wsn = (int)p.w_sn, xst = (int)p.x_st;
    const int lr = lane >> 3, lp = (lane & 7) ^ lr;
    const int wv = (lr * wsn + 8 * lp) * 2, xv = (lr * xst + 8 * lp) * 2;
    auto dma = [&](const Tile &ti, unsigned char *stage, int k0) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t wres = wres_of(ti), xres = xres_of(ti);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 64 * wave + 8 * j;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wres, (__attribute__((address_space(3))) void *)(stage + r * kBigRow), 16, wv,
                (r * wsn + k0) * 2, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xres, (__attribute__((address_space(3))) void *)(stage + kBigOp + r * kBigRow), 16, xv,
                (r * xst + k0) * 2, 0, 0);
        }
    };

    // Operand reads: wave (wr, wc) = (wave % 2, wave / 2) owns weight rows
    // 128 wr .. + 127 and tokens 128 wc .. + 127 of the tile; MFMA tile i
    // (j) is rows (tokens) 16 i + c, k-slots 8 g .. 8 g + 7 of k-step kk =
    // logical piece 4 kk + g.  Every such row has row % 8 == c % 8.
    const int wr = wave & 1, wc = wave >> 1;
    const int aoff = (128 * wr + c) * kBigRow, boff = kBigOp + (128 * wc + c) * kBigRow;
    struct Ops {
        bf16x8_t a[8], b[8];
    };
    auto read_ops = [&](const unsigned char *stage, int kk, Ops &o) __attribute__((always_inline)) {
        const int po = 16 * ((4 * kk + g) ^ (c & 7));
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            o.a[n] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(
                                                      stage + aoff + po + 16 * n * kBigRow));
            o.b[n] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(
                                                      stage + boff + po + 16 * n * kBigRow));
        }
    };

    f32x4_t acc[8][8];
    auto mfmas = [&](const Ops &o) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.a[i], o.b[j], acc[i][j], 0, 0, 0);
    };

    // Chunk ch in stage `cur` (the other stage is `nxt`): oa holds its first
    // k-step on entry and the next chunk's first k-step on exit.  The last
    // two chunks load nothing more (and the last reads nothing more): those
    // are separate instances, so the loop body has no branches.  Scheduling
    // barriers pin the order (the compiler otherwise moves each read next to
    // its first use and waits for it there, and sinks MFMAs below the
    // barrier); scheduling-group barriers spread the loads and reads over
    // the MFMAs, so the matrix core is not idle while the wave (one per SIMD)
    // issues them.
    const int nch = p.model_dim / kBigK;  // a multiple of 4 (model_dim % 256 == 0)
    Ops oa, ob;
    auto chunk = [&](const Tile &ti, int ch, unsigned char *cur, unsigned char *nxt, auto more_loads,
                     auto more_reads) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        read_ops(cur, 1, ob);
        mfmas(oa);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);  // eight MFMAs
        }
        __builtin_amdgcn_sched_barrier(0);
        // this wave's reads of `cur` back and its loads of chunk ch + 1
        // landed (no later loads are in flight)
        __builtin_amdgcn_s_waitcnt(kWait0);
        big_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(more_loads)::value) dma(ti, cur, (ch + 2) * kBigK);
        if constexpr (decltype(more_reads)::value) read_ops(nxt, 0, oa);
        mfmas(ob);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (decltype(more_loads)::value) __builtin_amdgcn_sched_group_barrier(0x010, 2, 0);
            if constexpr (decltype(more_reads)::value) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

    // (tiles are rebuilt from their index where needed: a tile kept across
    // loop iterations went to scratch memory)
    int bid = blockIdx.x;
    bool stores_after = false;  // the previous tile's last 16 stores follow its last loads
    {
        const Tile first = tile_of(bid);
        dma(first, st0, 0);
        dma(first, st1, kBigK);
    }
    for (;;) {
        const Tile cur = tile_of(bid);
        // chunks 0 and 1 landed.  The vector memory counter counts loads
        // and stores and they complete in issue order (the compiler's own
        // waits rely on it), so after a whole bf16 tile, whose last 16
        // stores were issued after the last of these loads, those stores
        // need not be waited for (+0.7%)
        if (stores_after) __builtin_amdgcn_s_waitcnt(kWait16);
        else __builtin_amdgcn_s_waitcnt(kWait0);
        big_barrier();
        read_ops(st0, 0, oa);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int ch = 0; ch < nch - 2; ch += 2) {
            chunk(cur, ch, st0, st1, T_{}, T_{});
            chunk(cur, ch + 1, st1, st0, T_{}, T_{});
        }
        chunk(cur, nch - 2, st0, st1, F_{}, T_{});
        chunk(cur, nch - 1, st1, st0, F_{}, F_{});

        // acc[i][j]: lane (c, g) holds stacked rows row0 + 128 wr + 16 i +
        // 4 g + (0..3) of token t0 + 128 wc + 16 j + c
        const int fbase = cur.row0 - (cur.is_r ? p.n : 0);
        const int nbid = bid + (int)gridDim.x;
        const bool more = nbid < nt;
        if constexpr (BF16OUT) {
            // bf16 outputs go through LDS, so every token's 256 features
            // leave as 16-byte pieces of whole lines (the lane layout above
            // writes 8 bytes per token and row group, 16 tokens apart).  The
            // tile is [256 tokens][256 features] bf16, 512-byte rows (tokens
            // 0..127 in st0, 128..255 in st1); 16-byte piece k of row r sits
            // at k ^ (r % 16), so the 16 rows one write touches land on
            // distinct banks.
            __builtin_amdgcn_s_waitcnt(kWaitLds);
            big_barrier();  // every wave's last operand reads are back
            unsigned char *ot = wc ? st1 : st0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int col = 128 * wr + 16 * i + 4 * g;  // feature, a multiple of 4
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int r = 16 * j + c;  // row within the half (r % 16 == c)
                    const f32x4_t v = acc[i][j];
                    const bf16x4_t b = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
                    const int piece = (col >> 3) ^ c;
                    *reinterpret_cast<uint2 *>(ot + r * 512 + 16 * piece + 2 * (col & 7)) =
                        __builtin_bit_cast(uint2, b);
                }
            }
            __builtin_amdgcn_s_waitcnt(kWaitLds);
            big_barrier();
            // Two halves: tokens 0..127 (st0), then 128..255 (st1).  In each,
            // wave w takes tokens 32 w .. 32 w + 31 of the half, two per
            // instruction (lane half hl = lane / 32, piece lane % 32); once
            // every wave has read a half, its stage takes the next tile's
            // first (second) chunk while the half's pieces are stored.
            const int hl = lane >> 5, k = lane & 31;
            const int f = fbase + 8 * k;
            const int h = f / p.head_dim, e = f % p.head_dim;
            uint16_t *out = static_cast<uint16_t *>(cur.is_r ? p.rho : p.q) +
                            (int64_t)h * (cur.is_r ? p.r_sh : p.q_sh) + e;
            const int64_t ost = cur.is_r ? p.r_st : p.q_st;
            auto half_out = [&](const unsigned char *it, unsigned char *stage, int half, int k0)
                __attribute__((always_inline)) {
                uint4 vals[16];
#pragma unroll
                for (int s2 = 0; s2 < 16; ++s2) {
                    const int r = 32 * wave + 2 * s2 + hl;
                    vals[s2] = *reinterpret_cast<const uint4 *>(it + r * 512 + 16 * (k ^ (r & 15)));
                }
                __builtin_amdgcn_s_waitcnt(kWaitLds);
                big_barrier();  // every wave has read this half: its stage is free
                if (more) dma(tile_of(nbid), stage, k0);
                // tokens t0 + 128 half + 32 w + hl + 2 s2; a whole tile stores
                // unconditionally (per-store conditions sent vals to scratch)
                const int tb0 = cur.t0 + 128 * half + 32 * wave + hl;
                uint16_t *o = out + (int64_t)tb0 * ost;
                // non-temporal stores: the outputs are not read again here,
                // and streaming them past the caches let them complete sooner
                // (the next tile's loads complete after them: one counter,
                // in issue order); +3-5% at 32768 tokens
                typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
                auto put = [&](int s2) __attribute__((always_inline)) {
                    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, vals[s2]),
                                                reinterpret_cast<u32x4_t *>(o + 2 * s2 * ost));
                };
                if (cur.t0 + kBigT <= T) {
#pragma unroll
                    for (int s2 = 0; s2 < 16; ++s2) put(s2);
                } else {
                    const int nv = T - tb0;  // this lane's stores with t < T: 2 s2 < nv
#pragma unroll
                    for (int s2 = 0; s2 < 16; ++s2)
                        if (2 * s2 < nv) put(s2);
                }
            };
            half_out(st0, st0, 0, 0);
            half_out(st1, st1, 1, kBigK);
            stores_after = cur.t0 + kBigT <= T;
        } else {
            __builtin_amdgcn_s_waitcnt(kWaitLds);
            big_barrier();  // every wave's last operand reads are back
            if (more) {
                const Tile nx = tile_of(nbid);
                dma(nx, st0, 0);
                dma(nx, st1, kBigK);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int f = fbase + 128 * wr + 16 * i + 4 * g;
                const int h = f / p.head_dim, e = f % p.head_dim;
                const int64_t hoff = (int64_t)h * (cur.is_r ? p.r_sh : p.q_sh) + e;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int t = cur.t0 + 128 * wc + 16 * j + c;
                    if (t >= T) continue;
                    const int64_t off = (int64_t)t * (cur.is_r ? p.r_st : p.q_st) + hoff;
                    const f32x4_t v = acc[i][j];
                    *reinterpret_cast<float4 *>(static_cast<float *>(cur.is_r ? p.rho : p.q) + off) =
                        float4{v[0], v[1], v[2], v[3]};
                }
            }
        }
        if (!more) break;
        bid = nbid;
    }
}

// Compute units of the stream's device (cached per device; 0 if unknown).  The
// prefill's launcher keeps its own copy of this helper in its file.
int stream_cus(hipStream_t stream) {
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

hipError_t launch_big(const ProjParams &p, hipStream_t stream) {
    const int n_rb = 2 * p.n / kBigT, n_tb = (p.tokens + kBigT - 1) / kBigT;
    // one workgroup per CU (128 KB of LDS each), a multiple of 8 workgroups
    const int cus = stream_cus(stream);
    const int cap = max(8, (cus > 0 ? cus : kCUs) / 8 * 8);
    const int grid = min(n_rb * n_tb, cap);
    if (p.out_bf16)
        hipLaunchKernelGGL((proj_big_kernel<true>), dim3((unsigned)grid), dim3(256), 0, stream, p, n_rb, n_tb);
    else
        hipLaunchKernelGGL((proj_big_kernel<false>), dim3((unsigned)grid), dim3(256), 0, stream, p, n_rb, n_tb);
    return hipGetLastError();
}

}  // namespace

// Up to 16 tokens (decode): token blocks of 16 and the weight-streaming
// kernel; up to 64: blocks of 64; up to 128: blocks of 64 with two row tiles
// per workgroup (one row tile doubled the weight re-reads there); beyond: an
// LDS-tiled GEMM.  256 x 256 tiles when that grid fills the CUs: the
// four-wave kernel when N is a multiple of 256 (and its 32-bit offsets
// reach), else the eight-wave one when 2N is a multiple of 256; otherwise
// 128 x 128 tiles (2N is always a multiple of 128: head_dim is 64 or 128).
hipError_t launch_qr_projection(const ProjParams &p, hipStream_t stream) {
    if (p.tokens <= 16) return launch_nt<1, 1>(p, stream);
    if (p.tokens <= 64) return launch_nt<1, 4>(p, stream);
    if (p.tokens <= 128) return launch_nt<2, 4>(p, stream);
    const int64_t big = (int64_t)(2 * p.n / Tile256::kMT) * ((p.tokens + Tile256::kNT - 1) / Tile256::kNT);
    // the large-tile kernel's 32-bit buffer offsets span 256 rows of either operand
    const bool offsets32 = (int64_t)kBigT * p.w_sn * 2 + 2 * p.model_dim < (1LL << 31) &&
                           (int64_t)kBigT * p.x_st * 2 + 2 * p.model_dim < (1LL << 31);
    if (p.n % kBigT == 0 && big >= kCUs && offsets32) return launch_big(p, stream);
    if ((2 * p.n) % Tile256::kMT == 0 && big >= kCUs) return launch_tiled<Tile256>(p, stream);
    return launch_tiled<Tile128>(p, stream);
}

}  // namespace plx
