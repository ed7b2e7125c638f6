// decode_nvfp4.hip - NVFP4-weight variants of the one-kernel decode (e2m1
// codes with an E4M3 scale per 16 elements and an fp32 scale per matrix).
#include "decode_launch.hpp"

namespace moe {
namespace dec {
hipError_t launch_nvfp4(DecArgs& a, hipStream_t st) { return launch_w<3>(a, st); }
}  // namespace dec
}  // namespace moe
