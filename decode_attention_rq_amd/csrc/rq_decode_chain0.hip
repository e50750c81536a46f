// rq_decode_chain0.hip -- decode launches with chained references (the
// Previous-/Next-loop policies), BF16 reference at the chain's root.
// The kernel template is in rq_decode_kernel.hpp.

#include "rq_decode_kernel.hpp"

namespace rq {

template hipError_t launch_decode_aq<0, 1>(const DecodeArgs &, int, int, bool, hipStream_t);

}  // namespace rq
