// read_probe.hip -- a plain read-only streaming kernel: the HBM reference the
// benchmark reports beside the decode rates.  Built into its own library
// (libparallax_probe.so); not part of libparallax or its C ABI.
//
// Grid-stride loop, one 16-byte load per thread per iteration, 2048 x 256
// threads: on MI355X this shape reads a cold buffer fastest (more loads in
// flight per thread or more workgroups read slower).
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void read_stream(const uint4 *__restrict__ p, size_t n16,
                                                   unsigned *sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    unsigned acc = 0;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;  // keeps the loads; practically never taken
}

// The decode kernel's read shape without its arithmetic: workgroup w of
// eight waves reads rows [w * span, (w + 1) * span) of a K half and a V half
// (256-byte rows), each wave 32 rows of each per step, steps dealt to the
// waves in turn, one step of loads in flight (the next step's loads are
// issued once the current ones have been consumed).
__global__ __launch_bounds__(512) void read_decode_shape(const unsigned char *__restrict__ K,
                                                         const unsigned char *__restrict__ V,
                                                         int span, unsigned *sink) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const size_t base = (size_t)blockIdx.x * span * 256;
    const int nsteps = span / 32;
    uint4 kr[8], vr[8];
    auto issue = [&](int st) {
        const size_t rb = base + (size_t)st * 32 * 256 + (lane / 16) * 256 + 16 * (lane % 16);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            kr[u] = *reinterpret_cast<const uint4 *>(K + rb + u * 1024);
            vr[u] = *reinterpret_cast<const uint4 *>(V + rb + u * 1024);
        }
    };
    unsigned acc = 0;
    if (wave < nsteps) issue(wave);
    for (int st = wave; st < nsteps; st += 8) {
        unsigned a = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) a ^= kr[u].x ^ kr[u].w ^ vr[u].y ^ vr[u].z;
        acc += a;
        if (st + 8 < nsteps) issue(st + 8);
    }
    if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;  // keeps the loads; practically never taken
}

}  // namespace

// Reads `bytes` (a multiple of 16) at `buf` once on `stream`.  `sink` is a
// device buffer of at least 256 unsigned ints.  Returns 0, 1 for bad
// arguments, 4 for a launch error.
extern "C" __attribute__((visibility("default"))) int parallax_probe_read(const void *buf,
                                                                          size_t bytes,
                                                                          unsigned *sink,
                                                                          void *stream) {
    if (buf == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0) return 1;
    hipLaunchKernelGGL(read_stream, dim3(2048), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// Reads `bytes` at `buf` once in the decode kernel's shape: the first half as
// K rows, the second as V rows, `workgroups` workgroups of eight waves.  Each
// half must split into `workgroups` spans of whole 32-row steps.  Returns 0,
// 1 for bad arguments, 4 for a launch error.
extern "C" __attribute__((visibility("default"))) int parallax_probe_read_decode_shape(
    const void *buf, size_t bytes, int workgroups, unsigned *sink, void *stream) {
    if (buf == nullptr || sink == nullptr || workgroups < 1) return 1;
    const size_t half = bytes / 2;
    if (bytes % 2 != 0 || half % ((size_t)workgroups * 32 * 256) != 0) return 1;
    const size_t span = half / 256 / workgroups;
    if (span > 0x7fffffff) return 1;
    const unsigned char *K = static_cast<const unsigned char *>(buf);
    hipLaunchKernelGGL(read_decode_shape, dim3(workgroups), dim3(512), 0,
                       static_cast<hipStream_t>(stream), K, K + half, (int)span, sink);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}
