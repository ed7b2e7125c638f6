// decode_bf16.hip - BF16-weight variants of the one-kernel decode; compiled
// apart from the MXFP4 ones so the two build in parallel.
#include "decode_launch.hpp"

namespace moe {
namespace dec {
hipError_t launch_bf16(DecArgs& a, hipStream_t st) { return launch_w<1>(a, st); }
}  // namespace dec
}  // namespace moe
