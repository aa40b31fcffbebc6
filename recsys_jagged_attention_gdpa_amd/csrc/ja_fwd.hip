// Forward launches for bf16 inputs (the kernels are in
// ja_fwd_kernels.h); MXFP8 inputs go to ja_fwd_mx.hip and the GDPA
// long-sequence kernel is launched from ja_fwd_gdpa.hip.  The translation
// units are compiled apart so that each can take the instruction scheduling
// that suits its kernels (the build gives this one the compiler's
// latency-hiding "max-ilp" scheduler: the JFA forward measured 3.5 % faster
// with it, the MXFP8 forward 2 % slower).
#include "ja_fwd_kernels.h"

namespace ja {

hipError_t launch_fwd_bf16(const AttnParams &p, int D, int mode, int act, int cus, bool few_q, bool long_units,
                           hipStream_t stream) {
    if (p.mx) return launch_fwd_mx(p, D, mode, act, cus, few_q, long_units, stream);
    return launch_fwd_fmt<false>(p, D, mode, act, cus, few_q, long_units, stream);
}

}  // namespace ja
