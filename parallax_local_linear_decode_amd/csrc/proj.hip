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
// Workgroup: 16 RT stacked weight rows x 16 NT tokens; its eight waves split
// the model dimension D into eighths, each accumulating partial 16 x 16
// tiles with 16x16x32 bf16 MFMAs and fp32 accumulation; the partials are
// summed in LDS in wave order.  At decode sizes (up to 64 tokens) the product
// is bound by streaming the weights from HBM: one row tile per workgroup
// (2N / 16 workgroups, 256 for 2N = 4096, so every CU streams), and a wave
// issues all loads of its eighth of D before the MFMAs, so the whole weight
// set is requested at once.  From 65 to 128 tokens two row tiles per
// workgroup let one token load serve two weight loads.
#include "kernels.hpp"

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

}  // namespace

// Up to 16 tokens (decode): token blocks of 16 and the weight-streaming
// kernel; up to 64: blocks of 64; up to 128: blocks of 64 with two row tiles
// per workgroup (one row tile doubled the weight re-reads there); beyond: the LDS-tiled GEMM, with 256 x 256
// tiles when 2N is a multiple of 256 and that grid fills the CUs, else with
// 128 x 128 tiles (2N is always a multiple of 128: head_dim is 64 or 128).
hipError_t launch_qr_projection(const ProjParams &p, hipStream_t stream) {
    if (p.tokens <= 16) return launch_nt<1, 1>(p, stream);
    if (p.tokens <= 64) return launch_nt<1, 4>(p, stream);
    if (p.tokens <= 128) return launch_nt<2, 4>(p, stream);
    const int64_t big = (int64_t)(2 * p.n / Tile256::kMT) * ((p.tokens + Tile256::kNT - 1) / Tile256::kNT);
    if ((2 * p.n) % Tile256::kMT == 0 && big >= kCUs) return launch_tiled<Tile256>(p, stream);
    return launch_tiled<Tile128>(p, stream);
}

}  // namespace plx
