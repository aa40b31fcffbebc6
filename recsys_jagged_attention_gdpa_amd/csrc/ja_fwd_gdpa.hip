// Launch of the long-sequence forward kernel for bf16 GDPA inputs (the kernels
// are in ja_fwd_kernels.h), a translation unit of its own so that the build can
// give this kernel the compiler's iterative latency-hiding scheduler: the
// GELU-erf long-tail forward measured 2 % faster with it, while the short-K/V
// forward (3 % slower with it) and the JFA forward (2-3 % slower) stay in
// ja_fwd.hip.
#include "ja_fwd_kernels.h"

namespace ja {

template <int D, int ACT>
hipError_t launch_fwd_gdpa_long(const AttnParams &p, int cus, hipStream_t stream) {
    hipLaunchKernelGGL((fwd_kernel<D, GDPA, ACT, 4, KV_TILE, false, false>), dim3(2 * cus), dim3(4 * WAVE), 0, stream,
                       kernel_timer().with_busy(p, K_FWD));
    return hipGetLastError();
}

template hipError_t launch_fwd_gdpa_long<32, SILU>(const AttnParams &, int, hipStream_t);
template hipError_t launch_fwd_gdpa_long<32, GELU_TANH>(const AttnParams &, int, hipStream_t);
template hipError_t launch_fwd_gdpa_long<32, GELU_ERF>(const AttnParams &, int, hipStream_t);
template hipError_t launch_fwd_gdpa_long<64, SILU>(const AttnParams &, int, hipStream_t);
template hipError_t launch_fwd_gdpa_long<64, GELU_TANH>(const AttnParams &, int, hipStream_t);
template hipError_t launch_fwd_gdpa_long<64, GELU_ERF>(const AttnParams &, int, hipStream_t);
template hipError_t launch_fwd_gdpa_long<128, SILU>(const AttnParams &, int, hipStream_t);
template hipError_t launch_fwd_gdpa_long<128, GELU_TANH>(const AttnParams &, int, hipStream_t);
template hipError_t launch_fwd_gdpa_long<128, GELU_ERF>(const AttnParams &, int, hipStream_t);

}  // namespace ja
