// rq_decode_chain4_one.hip -- decode launches along a chain of references
// (INT4 anchor at the root) that compute one loop slot: a call for a single
// loop reads every link between it and the root, but wants only its own
// output.  The kernel template is in rq_decode_kernel.hpp.

#include "rq_decode_kernel.hpp"

namespace rq {

template hipError_t launch_decode_aq<4, 2>(const DecodeArgs &, int, int, bool, hipStream_t);

}  // namespace rq
