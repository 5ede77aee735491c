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
