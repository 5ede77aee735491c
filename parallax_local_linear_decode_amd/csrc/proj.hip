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
// Workgroup: 32 stacked weight rows x 16 * NT tokens; its eight waves split
// the model dimension D into eighths, each accumulating partial 16 x 16
// tiles (two row tiles per token block, so one token load serves two weight
// loads) with 16x16x32 bf16 MFMAs and fp32 accumulation; the partials are
// summed in LDS in wave order.  At decode sizes (a few tokens) the product is
// bound by streaming the weights from HBM: a wave issues all loads of its
// eighth before the MFMAs, and the grid has 2N / 32 workgroups of eight
// waves, so the whole weight set is requested at once.
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
constexpr int kRows = 32;  // stacked weight rows per workgroup (two 16-row tiles)

template <int NT, bool BF16OUT>
__global__ __launch_bounds__(64 * kWaves) void proj_kernel(ProjParams p) {
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
    const uint16_t *w[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
        w[rt] = (is_r ? p.w_r : p.w_q) + (int64_t)(f0 + 16 * rt + c) * p.w_sn + 8 * g;
    const uint16_t *xr[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        xr[nt] = p.x + (int64_t)min(t0 + 16 * nt + c, T - 1) * p.x_st + 8 * g;

    const int kq = p.model_dim / kWaves;
    const int k_begin = wave * kq;
    const int steps = kq / 32;
    f32x4_t acc[2][NT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // CH steps' loads are issued together, then their MFMAs: at decode sizes
    // (NT = 1) a wave's whole eighth of D = 2048 is in flight per lane
    constexpr int CH = NT == 1 ? 8 : 2;
    int st = 0;
    for (; st + CH <= steps; st += CH) {
        bf16x8_t a[CH][2], b[CH][NT];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int k = k_begin + 32 * (st + i);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) a[i][rt] = ld_bf16x8(w[rt] + k);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) b[i][nt] = ld_bf16x8(xr[nt] + k);
        }
        // keep the scheduler from interleaving the MFMAs into the loads (it
        // would trade loads in flight for registers)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < CH; ++i)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i][rt], b[i][nt],
                                                                          acc[rt][nt], 0, 0, 0);
    }
    for (; st < steps; ++st) {
        const int k = k_begin + 32 * st;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const bf16x8_t a = ld_bf16x8(w[rt] + k);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ld_bf16x8(xr[nt] + k),
                                                                      acc[rt][nt], 0, 0, 0);
        }
    }

    __shared__ f32x4_t red[kWaves][2][NT][64];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) red[wave][rt][nt][lane] = acc[rt][nt];
    __syncthreads();

    // wave w finishes tiles u = w, w + 8, ... of the 2 NT (row tile, token
    // block) pairs; lane (c, g) holds features f0 + 16 rt + 4g + j (j = 0..3)
    // of token t0 + 16 nt + c
    for (int u = wave; u < 2 * NT; u += kWaves) {
        const int rt = u % 2, nt = u / 2;
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

template <int NT>
hipError_t launch_nt(const ProjParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)(2 * p.n / kRows), (unsigned)((p.tokens + 16 * NT - 1) / (16 * NT)));
    if (p.out_bf16)
        hipLaunchKernelGGL((proj_kernel<NT, true>), grid, dim3(64 * kWaves), 0, stream, p);
    else
        hipLaunchKernelGGL((proj_kernel<NT, false>), grid, dim3(64 * kWaves), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

// Token blocks of 16 up to 16 tokens (decode), else of 64 (each weight
// element then serves 64 tokens per load).
hipError_t launch_qr_projection(const ProjParams &p, hipStream_t stream) {
    return p.tokens <= 16 ? launch_nt<1>(p, stream) : launch_nt<4>(p, stream);
}

}  // namespace plx
