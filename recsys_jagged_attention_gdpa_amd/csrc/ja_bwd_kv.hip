// dK/dV launches (the kernels are in ja_bwd_kernels.h), a translation unit of
// their own so that the build can give them the compiler's iterative
// latency-hiding scheduler, which slows the dQ kernel down.
#include "ja_bwd_kernels.h"

namespace ja {

template <int D, int MODE, int ACT>
static hipError_t launch_kv_t(const AttnParams &p, int grid, hipStream_t st) {
    const KernelTimer &t = kernel_timer();
    t.begin(K_BWD_KV, st);
    hipLaunchKernelGGL((dkdv_kernel<D, MODE, ACT>), dim3(grid / 2), dim3(BWD_THREADS), 0, st, t.with_busy(p, K_BWD_KV));
    t.end(K_BWD_KV, st);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_kv_d(const AttnParams &p, int mode, int act, int grid, hipStream_t st) {
    if (mode == JFA) return launch_kv_t<D, JFA, SILU>(p, grid, st);
    switch (act) {
    case SILU: return launch_kv_t<D, GDPA, SILU>(p, grid, st);
    case GELU_TANH: return launch_kv_t<D, GDPA, GELU_TANH>(p, grid, st);
    default: return launch_kv_t<D, GDPA, GELU_ERF>(p, grid, st);
    }
}

hipError_t launch_bwd_kv(const AttnParams &p, int D, int mode, int act, int grid, hipStream_t st) {
    switch (D) {
    case 32: return launch_kv_d<32>(p, mode, act, grid, st);
    case 64: return launch_kv_d<64>(p, mode, act, grid, st);
    default: return launch_kv_d<128>(p, mode, act, grid, st);
    }
}

}  // namespace ja
