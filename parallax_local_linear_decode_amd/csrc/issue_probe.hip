// issue_probe.hip -- how matrix-core and vector work share one SIMD: the
// measurement behind the compute ceilings of the prefill kernels, where a
// wave of matrix products and a wave of softmax or gradient arithmetic share
// each SIMD.  Built into libparallax_probe.so; not part of libparallax or its
// C ABI.
//
// One workgroup of eight waves per CU (the static LDS below keeps a second
// one off the CU), so waves w and w + 4 share SIMD w.  Waves 0-3 run chains of
// independent 16x16x32 bf16 MFMAs, waves 4-7 chains of independent fp32 FMAs
// or base-2 exponentials; either group can be switched off, and waves 0-3
// can run the vector work instead (two vector waves per SIMD).  Comparing the
// time of both groups together with each group alone shows how far the two
// kinds of work overlap on a SIMD, and one vector wave against two shows how
// much of the SIMD's vector rate one wave can issue.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;          // independent accumulators / values per lane
constexpr int kPadBytes = 96 * 1024;  // more than half of a CU's 160 KB of LDS

__global__ __launch_bounds__(512) void issue_probe(int mode, int mfma_iters, int valu_iters,
                                                   float *sink) {
    __shared__ float pad[kPadBytes / 4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (threadIdx.x == 0) pad[blockIdx.x % (kPadBytes / 4)] = 0.f;
    float result = 0.f;
    if (wave < 4 && (mode & 1) && !(mode & 8)) {
        bf16x8_t a, b;
        for (int i = 0; i < 8; ++i) {
            a[i] = (__bf16)(0.001f * (lane + i));
            b[i] = (__bf16)(0.002f * (lane - i));
        }
        f32x4_t acc[kChains];
        for (int j = 0; j < kChains; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < mfma_iters; ++it) {
#pragma unroll
            for (int j = 0; j < kChains; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
        }
        for (int j = 0; j < kChains; ++j) result += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    } else if ((wave >= 4 && (mode & 2)) || (wave < 4 && (mode & 8))) {
        float x[kChains];
        for (int j = 0; j < kChains; ++j) x[j] = 0.25f + 0.01f * (lane + j);
        const float y = 0.999f + 1e-6f * lane, z = 1e-3f;
        if (mode & 4) {
            for (int it = 0; it < valu_iters; ++it) {
#pragma unroll
                for (int j = 0; j < kChains; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
            }
        } else {
            for (int it = 0; it < valu_iters; ++it) {
#pragma unroll
                for (int j = 0; j < kChains; ++j) x[j] = fmaf(x[j], y, z);
            }
        }
        for (int j = 0; j < kChains; ++j) result += x[j];
    }
    // keeps the work and the LDS allocation; practically never taken
    if (result == 1234.5f + pad[lane]) sink[threadIdx.x] = result;
}

}  // namespace

// mode: bit 0 runs the MFMA waves, bit 1 the vector waves, bit 2 makes the
// vector waves' work exponentials instead of FMAs, bit 3 gives waves 0-3 the
// vector work instead of MFMAs.  `workgroups` should be the
// CU count.  `sink` is a device buffer of at least 512 floats.  Returns 0, 1 for
// bad arguments, 4 for a launch error.
extern "C" __attribute__((visibility("default"))) int parallax_probe_issue(
    int mode, int mfma_iters, int valu_iters, int workgroups, float *sink, void *stream) {
    if (sink == nullptr || workgroups < 1 || mfma_iters < 0 || valu_iters < 0 || mode < 0 ||
        mode > 15)
        return 1;
    hipLaunchKernelGGL(issue_probe, dim3(workgroups), dim3(512), 0,
                       static_cast<hipStream_t>(stream), mode, mfma_iters, valu_iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}
