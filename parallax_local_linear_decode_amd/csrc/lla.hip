// lla.hip -- per-row vector kernels of local linear attention's solved probe
// (page "Parallax: Parameterized Local Linear Attention Gives Transformers a
// 'Second Eye'", section 1.2: each token solves S x = mu by conjugate
// gradients, every iteration one sweep over the KV cache).  The step itself
// (lla_row.hpp) runs inside the decode merge kernel after each sweep.
//
// For decode row (b, h) with softmax weights p over its keys the system is
// (S_KK + lam I) x = mu, mu = kbar - q, S_KK = sum p_j (k_j - kbar)(k_j - kbar)^T.
// The sweep is the decode kernel itself with the keys passed as values: its
// output with probe y is kbar - S_KK y, so S_KK y = kbar - o(V = K, rho = y),
// and kbar = o(V = K, rho = 0).  These kernels set up and read out the
// conjugate-gradient state: one 64-lane wave per row, head-dim element e in
// lane e % 64 (two per lane at d = 128).
#include "kernels.hpp"
#include "lla_row.hpp"

#include <algorithm>

namespace plx {
namespace {

constexpr int kRowsPerBlock = 4;  // one wave per row

struct RowView {
    int64_t u;  // row index b * Hq + h
    int b, h;
    bool live;
};

__device__ __forceinline__ RowView row_of(const LlaParams &p) {
    RowView r;
    const int64_t rows = (int64_t)p.batch * p.num_q_heads;
    r.u = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / 64;
    r.live = r.u < rows;
    if (!r.live) r.u = rows - 1;
    r.b = (int)(r.u / p.num_q_heads);
    r.h = (int)(r.u % p.num_q_heads);
    return r;
}

__global__ __launch_bounds__(256) void lla_zero_kernel(float *a, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        a[i] = 0.0f;
}

// mu = kbar - q (0 for a row without keys); x = 0, r = p = mu, rs = rs0 = |mu|^2.
__global__ __launch_bounds__(256) void lla_init_kernel(LlaParams p) {
    const RowView rv = row_of(p);
    const int lane = threadIdx.x % 64;
    const int L = p.seq_lens ? p.seq_lens[rv.b] : p.max_seq_len;
    const float *q = p.q + (int64_t)rv.b * p.q_sb + (int64_t)rv.h * p.q_sh;
    const int64_t off = rv.u * p.d;
    float s = 0.0f;
    for (int e = lane; e < p.d; e += 64) {
        const float mu = L > 0 ? p.kbar[off + e] - q[e] : 0.0f;
        if (rv.live) {
            p.x[off + e] = 0.0f;
            p.r[off + e] = mu;
            p.dir[off + e] = mu;
        }
        s += mu * mu;
    }
    s = lla_wave_sum(s);
    if (rv.live && lane == 0) {
        p.rs[2 * rv.u] = s;
        p.rs[2 * rv.u + 1] = s;
    }
}

// rho_out = x; resid = |r| / |mu| (0 for a row with mu = 0).
__global__ __launch_bounds__(256) void lla_finish_kernel(LlaParams p) {
    const RowView rv = row_of(p);
    if (!rv.live) return;
    const int lane = threadIdx.x % 64;
    const int64_t off = rv.u * p.d;
    if (p.rho_out != nullptr)
        for (int e = lane; e < p.d; e += 64) p.rho_out[off + e] = p.x[off + e];
    if (p.resid != nullptr && lane == 0) {
        const float rs = p.rs[2 * rv.u], rs0 = p.rs[2 * rv.u + 1];
        p.resid[rv.u] = rs0 > 0.0f ? sqrtf(rs / rs0) : 0.0f;
    }
}

unsigned row_blocks(const LlaParams &p) {
    const int64_t rows = (int64_t)p.batch * p.num_q_heads;
    return (unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
}

}  // namespace

hipError_t launch_lla_zero(float *a, int64_t n, hipStream_t stream) {
    const unsigned blocks = (unsigned)std::min<int64_t>(1024, (n + 255) / 256);
    hipLaunchKernelGGL(lla_zero_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream, a, n);
    return hipGetLastError();
}

hipError_t launch_lla_init(const LlaParams &p, hipStream_t stream) {
    hipLaunchKernelGGL(lla_init_kernel, dim3(row_blocks(p)), dim3(64 * kRowsPerBlock), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_lla_finish(const LlaParams &p, hipStream_t stream) {
    hipLaunchKernelGGL(lla_finish_kernel, dim3(row_blocks(p)), dim3(64 * kRowsPerBlock), 0, stream,
                       p);
    return hipGetLastError();
}

}  // namespace plx
