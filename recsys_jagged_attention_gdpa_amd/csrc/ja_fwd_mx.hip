// Forward launches for MXFP8 inputs (the kernels are in ja_fwd_kernels.h),
// compiled with the compiler's default instruction scheduling.
#include "ja_fwd_kernels.h"

namespace ja {

hipError_t launch_fwd_mx(const AttnParams &p, int D, int mode, int act, int cus, bool few_q, bool long_units,
                         hipStream_t stream) {
    return launch_fwd_fmt<true>(p, D, mode, act, cus, few_q, long_units, stream);
}

}  // namespace ja
