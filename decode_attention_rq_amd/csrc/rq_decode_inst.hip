// rq_decode_inst.hip -- one instantiation of the decode kernel's launcher:
// head_dim RQ_INST_D, reference kind RQ_INST_AQ (0: BF16 reference rows; 2,
// 4: quantized anchor bits) and chain mode RQ_INST_CHAIN (0: independent
// references; 1: chained, every slot computed; 2: chained, slot 0 alone).
// The build compiles this file once per combination (defines on the
// command line), so the variants compile in parallel.  The kernel template
// is in rq_decode_kernel.hpp.

#include "rq_decode_kernel.hpp"

#if !defined(RQ_INST_D) || !defined(RQ_INST_AQ) || !defined(RQ_INST_CHAIN)
#error "rq_decode_inst.hip needs RQ_INST_D, RQ_INST_AQ and RQ_INST_CHAIN"
#endif

namespace rq {

template hipError_t launch_decode_d<RQ_INST_D, RQ_INST_AQ, RQ_INST_CHAIN>(const DecodeArgs &, int, bool,
                                                                          hipStream_t);
#if RQ_INST_AQ == 0 && RQ_INST_CHAIN == 0
template int decode_blocks_per_cu_d<RQ_INST_D>();
#endif

}  // namespace rq
