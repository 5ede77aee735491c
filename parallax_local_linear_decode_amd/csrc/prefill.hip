// prefill.hip -- causal Parallax prefill for gfx950 (matrix-core kernel: in progress).
#include "kernels.hpp"

namespace plx {

hipError_t launch_prefill(const PrefillParams &, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace plx
