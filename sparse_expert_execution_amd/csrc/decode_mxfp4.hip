// decode_mxfp4.hip - MXFP4-weight variants of the one-kernel decode.
#include "decode_launch.hpp"

namespace moe {
namespace dec {
hipError_t launch_mxfp4(DecArgs& a, hipStream_t st) { return launch_w<2>(a, st); }
}  // namespace dec
}  // namespace moe
