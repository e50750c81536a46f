// rq_decode_anchor4.hip -- decode launches for an INT4 quantized anchor
// (the kernel template is in rq_decode_kernel.hpp).

#include "rq_decode_kernel.hpp"

namespace rq {

template hipError_t launch_decode_aq<4, 0>(const DecodeArgs &, int, int, bool, hipStream_t);

}  // namespace rq
