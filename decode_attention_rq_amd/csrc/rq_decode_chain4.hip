// rq_decode_chain4.hip -- decode launches with chained references (the
// Previous-/Next-loop policies), INT4 quantized anchor at the chain's root.
// The kernel template is in rq_decode_kernel.hpp.

#include "rq_decode_kernel.hpp"

namespace rq {

template hipError_t launch_decode_aq<4, 1>(const DecodeArgs &, int, int, bool, hipStream_t);

}  // namespace rq
