// lla_row.hpp -- one conjugate-gradient step of local linear attention's
// solved probe for one decode row (page "Parallax: Parameterized Local Linear
// Attention Gives Transformers a 'Second Eye'", section 1.2: each token solves
// S x = mu by conjugate gradients, every iteration one sweep over the KV
// cache).  Shared by the decode merge kernel, which runs it right after a
// sweep's outputs are merged, and the vector kernels of lla.hip.
//
// One 64-lane wave per row, head-dim element e in lane e % 64 (two per lane
// at d = 128); dot products reduce across the wave and every lane takes lane
// 0's sum, so the update is the same on every lane.
#pragma once

#include "kernels.hpp"

namespace plx {

__device__ __forceinline__ float lla_wave_sum(float s) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    return __shfl(s, 0);
}

// Row u = b * Hq + h after the sweep o_k = o(V = K, rho = dir), whose values
// ok[e] the caller passes (global memory or LDS):
// A dir = (kbar - o_k) + lam dir; alpha = rs / dir.A dir; x += alpha dir;
// r -= alpha A dir; beta = |r|^2 / rs; dir = r + beta dir.  All 64 lanes of
// the wave call it; a row that is not live (a clamped tail row) joins the
// reductions and stores nothing.
__device__ __forceinline__ void lla_step_row(const LlaParams &p, int64_t u, bool live, int lane,
                                             const float *ok) {
    const int64_t off = u * p.d;
    constexpr int kMaxPer = 2;  // d <= 128
    float ap[kMaxPer], dv[kMaxPer];
    float pap = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
        const int e = lane + 64 * i;
        ap[i] = dv[i] = 0.0f;
        if (e < p.d) {
            dv[i] = p.dir[off + e];
            ap[i] = (p.kbar[off + e] - ok[e]) + p.lambda * dv[i];
            pap += dv[i] * ap[i];
        }
    }
    pap = lla_wave_sum(pap);
    const float rs = p.rs[2 * u];
    const float alpha = pap > 0.0f && rs > 0.0f ? rs / pap : 0.0f;
    float rr[kMaxPer];
    float rsn = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
        const int e = lane + 64 * i;
        rr[i] = 0.0f;
        if (e < p.d) {
            rr[i] = p.r[off + e] - alpha * ap[i];
            rsn += rr[i] * rr[i];
        }
    }
    rsn = lla_wave_sum(rsn);
    const float beta = rs > 0.0f ? rsn / rs : 0.0f;
    if (!live) return;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
        const int e = lane + 64 * i;
        if (e < p.d) {
            p.x[off + e] += alpha * dv[i];
            p.r[off + e] = rr[i];
            p.dir[off + e] = rr[i] + beta * dv[i];
        }
    }
    if (lane == 0) p.rs[2 * u] = rsn;
}

}  // namespace plx
