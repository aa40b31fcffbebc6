// Backward launches (the kernels are in ja_bwd_kernels.h): the delta pass, the
// fused short-K/V units and the dQ units here, the dK/dV units in
// ja_bwd_kv.hip.  The two translation units are compiled apart so that each
// can take the instruction scheduling that suits its kernels: the build gives
// the dK/dV unit the compiler's iterative latency-hiding scheduler and this
// one the iterative occupancy-first scheduler (measured against the default in
// the same runs: dK/dV -6 % on the GELU-erf long-tail workload and -0.5 % on
// the JFA one; dQ -1 to -2 %, where the latency-hiding scheduler made dQ 2.8x
// slower).
#include "ja_bwd_kernels.h"

namespace ja {

template <int D, int MODE, int ACT, bool ROPE>
static hipError_t launch_bwd_t(const AttnParams &p, int grid, bool long_units, hipStream_t st) {
    const bool db = p.dbias_slots != nullptr;
    const KernelTimer &t = kernel_timer();
    if (MODE == JFA && p.total_q > 0) {
        const int64_t threads = p.total_q * p.H * (D / 8);
        t.begin(K_BWD_DELTA, st);
        hipLaunchKernelGGL((delta_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, p);
        t.end(K_BWD_DELTA, st);
    }
    t.begin(K_BWD_FUSED, st);
    hipLaunchKernelGGL((fused_kernel<D, MODE, ACT, ROPE>), dim3(2 * grid), dim3(WAVE), 0, st, t.with_busy(p, K_BWD_FUSED));
    t.end(K_BWD_FUSED, st);
    if (!long_units) return hipGetLastError();
    const hipError_t e = launch_bwd_kv(p, D, MODE, ACT, grid, st);
    if (e != hipSuccess) return e;
    t.begin(K_BWD_Q, st);
    if (db)
        hipLaunchKernelGGL((dq_kernel<D, MODE, ACT, ROPE, true>), dim3(grid), dim3(BWD_THREADS), 0, st,
                           t.with_busy(p, K_BWD_Q));
    else
        hipLaunchKernelGGL((dq_kernel<D, MODE, ACT, ROPE, false>), dim3(grid), dim3(BWD_THREADS), 0, st,
                           t.with_busy(p, K_BWD_Q));
    t.end(K_BWD_Q, st);
    return hipGetLastError();
}

template <int D, bool ROPE>
static hipError_t launch_bwd_r(const AttnParams &p, int mode, int act, int grid, bool lu, hipStream_t st) {
    if (mode == JFA) return launch_bwd_t<D, JFA, SILU, ROPE>(p, grid, lu, st);
    switch (act) {
    case SILU: return launch_bwd_t<D, GDPA, SILU, ROPE>(p, grid, lu, st);
    case GELU_TANH: return launch_bwd_t<D, GDPA, GELU_TANH, ROPE>(p, grid, lu, st);
    default: return launch_bwd_t<D, GDPA, GELU_ERF, ROPE>(p, grid, lu, st);
    }
}

// Kernels without the rotary turn-back are their own instantiations, so its
// registers never weigh on the plain kernels.
template <int D>
static hipError_t launch_bwd_d(const AttnParams &p, int mode, int act, int grid, bool lu, hipStream_t st) {
    return p.rope_back ? launch_bwd_r<D, true>(p, mode, act, grid, lu, st)
                       : launch_bwd_r<D, false>(p, mode, act, grid, lu, st);
}

hipError_t launch_bwd_bf16(const AttnParams &p, int D, int mode, int act, int grid, bool long_units,
                           hipStream_t st) {
    switch (D) {
    case 32: return launch_bwd_d<32>(p, mode, act, grid, long_units, st);
    case 64: return launch_bwd_d<64>(p, mode, act, grid, long_units, st);
    default: return launch_bwd_d<128>(p, mode, act, grid, long_units, st);
    }
}

}  // namespace ja
