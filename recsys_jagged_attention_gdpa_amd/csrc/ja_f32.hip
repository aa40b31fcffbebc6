// fp32 kernels: the same GDPA / JFA forward and backward for fp32 tensors.
//
// gfx950's matrix cores take fp32 only at a fraction of the bf16 rate and the
// fp32 form exists for small, accuracy-sensitive problems, so these kernels
// are plain one-thread-per-row loops in fp32 on the vector ALUs: one thread
// owns a (query row, head) in the forward and dQ passes, or a (key row, head)
// in the dK / dV pass.  Masking and bias follow the same sample-local rules as
// the bf16 kernels.
#include "ja_device.h"
#include "ja_kernels.h"

namespace ja {

constexpr int F32_THREADS = 128;

// Sample that owns global row r of a jagged tensor with offsets off[0..B].
__device__ __forceinline__ int find_sample(const int32_t *off, int B, int64_t r) {
    int lo = 0, hi = B - 1;  // last b with off[b] <= r
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <int ACT>
__device__ __forceinline__ float act_f32(float x) {
    if constexpr (ACT == SILU) return x / (1.0f + expf(-x));
    else if constexpr (ACT == GELU_TANH) return 0.5f * x * (1.0f + tanhf(GELU_C * (x + GELU_A * x * x * x)));
    else return 0.5f * x * (1.0f + erff(x * INV_SQRT2));
}

template <int ACT>
__device__ __forceinline__ float act_grad_f32(float x) {
    if constexpr (ACT == SILU) {
        const float s = 1.0f / (1.0f + expf(-x));
        return s * (1.0f + x * (1.0f - s));
    } else if constexpr (ACT == GELU_TANH) {
        const float t = tanhf(GELU_C * (x + GELU_A * x * x * x));
        return 0.5f * (1.0f + t) + 0.5f * x * (1.0f - t * t) * GELU_C * (1.0f + 3.0f * GELU_A * x * x);
    } else {
        return 0.5f * (1.0f + erff(x * INV_SQRT2)) + x * INV_SQRT_2PI * expf(-0.5f * x * x);
    }
}

__device__ __forceinline__ float dot_f32(const float *a, const float *b, int D) {
    float s = 0.0f;
    for (int d = 0; d < D; ++d) s = __builtin_fmaf(a[d], b[d], s);
    return s;
}

// Map an output row to (sample, local row).
__device__ __forceinline__ void out_row_owner(const AttnParams &p, int64_t r, int &b, int &i) {
    if (p.q_off) {
        b = find_sample(p.q_off, p.B, r);
        i = (int)(r - p.q_off[b]);
    } else {
        b = (int)(r / p.lq_fixed);
        i = (int)(r % p.lq_fixed);
    }
}

template <int D, int MODE, int ACT>
__global__ __launch_bounds__(F32_THREADS) void fwd_f32_kernel(const AttnParams p) {
    const int64_t gid = (int64_t)blockIdx.x * F32_THREADS + threadIdx.x;
    if (gid >= p.total_q_out * p.H) return;
    const int h = (int)(gid % p.H);
    const int64_t r = gid / p.H;
    int b, i;
    out_row_owner(p, r, b, i);
    const Sample s = load_sample(p.q_off, p.lq_fixed, p.kv_off, b);
    const float *Q = static_cast<const float *>(p.q);
    const float *K = static_cast<const float *>(p.k);
    const float *V = static_cast<const float *>(p.v);
    BiasArgs bz{p.bias, p.bias_kind, p.bias_lo, p.bias_hi, p.bias_hi - p.bias_lo + 1};
    const float *brow = bz.kind ? bz.table + (int64_t)h * bz.width : nullptr;
    const float *qi = Q + ((s.qs + i) * p.H + h) * (int64_t)D;
    float acc[D];
    for (int d = 0; d < D; ++d) acc[d] = 0.0f;
    float m = -INFINITY, l = 0.0f;
    const int kend = key_end(i, s.lq, s.lk, p.causal, p.window);
    for (int j = key_begin(i, s.lq, s.lk, p.window); j < kend; ++j) {
        const float *kj = K + ((s.ks + j) * p.H + h) * (int64_t)D;
        const float *vj = V + ((s.ks + j) * p.H + h) * (int64_t)D;
        float x = p.scale * dot_f32(qi, kj, D);
        if (brow) x += bias_at(bz, brow, i, j);
        if constexpr (MODE == GDPA) {
            const float a = act_f32<ACT>(x);
            for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(a, vj[d], acc[d]);
        } else {
            const float mn = fmaxf(m, x);
            const float alpha = expf(m - mn);
            const float pj = expf(x - mn);
            l = l * alpha + pj;
            for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(pj, vj[d], acc[d] * alpha);
            m = mn;
        }
    }
    float norm = 1.0f;
    if constexpr (MODE == JFA) {
        norm = l > 0.0f ? 1.0f / l : 0.0f;
        p.lse[(int64_t)h * p.total_q_out + r] = l > 0.0f ? m + logf(l) : -INFINITY;
    }
    float *oi = static_cast<float *>(p.out) + (r * p.H + h) * (int64_t)D;
    for (int d = 0; d < D; ++d) oi[d] = acc[d] * norm;
}

// JFA backward preprocess: delta_i = <dO_i, O_i>, stored [H, Tq].
template <int D>
__global__ __launch_bounds__(F32_THREADS) void delta_f32_kernel(const AttnParams p) {
    const int64_t gid = (int64_t)blockIdx.x * F32_THREADS + threadIdx.x;
    if (gid >= p.total_q * p.H) return;
    const int h = (int)(gid % p.H);
    const int64_t r = gid / p.H;
    const float *o = static_cast<const float *>(p.o) + (r * p.H + h) * (int64_t)D;
    const float *g = static_cast<const float *>(p.dout) + (r * p.H + h) * (int64_t)D;
    p.delta[(int64_t)h * p.total_q + r] = dot_f32(o, g, D);
}

template <int D, int MODE, int ACT>
__global__ __launch_bounds__(F32_THREADS) void dq_f32_kernel(const AttnParams p) {
    const int64_t gid = (int64_t)blockIdx.x * F32_THREADS + threadIdx.x;
    if (gid >= p.total_q * p.H) return;
    const int h = (int)(gid % p.H);
    const int64_t r = gid / p.H;
    int b, i;
    out_row_owner(p, r, b, i);
    const Sample s = load_sample(p.q_off, p.lq_fixed, p.kv_off, b);
    const float *Q = static_cast<const float *>(p.q);
    const float *K = static_cast<const float *>(p.k);
    const float *V = static_cast<const float *>(p.v);
    BiasArgs bz{p.bias, p.bias_kind, p.bias_lo, p.bias_hi, p.bias_hi - p.bias_lo + 1};
    const float *brow = bz.kind ? bz.table + (int64_t)h * bz.width : nullptr;
    const float *qi = Q + (r * p.H + h) * (int64_t)D;
    const float *gi = static_cast<const float *>(p.dout) + (r * p.H + h) * (int64_t)D;
    float lse = 0.0f, dlt = 0.0f;
    if constexpr (MODE == JFA) {
        lse = p.lse[(int64_t)h * p.total_q + r];
        dlt = p.delta[(int64_t)h * p.total_q + r];
    }
    float acc[D];
    for (int d = 0; d < D; ++d) acc[d] = 0.0f;
    const int kend = key_end(i, s.lq, s.lk, p.causal, p.window);
    for (int j = key_begin(i, s.lq, s.lk, p.window); j < kend; ++j) {
        const float *kj = K + ((s.ks + j) * p.H + h) * (int64_t)D;
        const float *vj = V + ((s.ks + j) * p.H + h) * (int64_t)D;
        float x = p.scale * dot_f32(qi, kj, D);
        if (brow) x += bias_at(bz, brow, i, j);
        const float dp = dot_f32(gi, vj, D);
        float ds;
        if constexpr (MODE == GDPA) ds = dp * act_grad_f32<ACT>(x);
        else ds = expf(x - lse) * (dp - dlt);
        for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(ds, kj[d], acc[d]);
    }
    float *dq = static_cast<float *>(p.dq) + (r * p.H + h) * (int64_t)D;
    for (int d = 0; d < D; ++d) dq[d] = acc[d] * p.scale;
}

template <int D, int MODE, int ACT>
__global__ __launch_bounds__(F32_THREADS) void dkdv_f32_kernel(const AttnParams p) {
    const int64_t gid = (int64_t)blockIdx.x * F32_THREADS + threadIdx.x;
    if (gid >= p.total_k * p.H) return;
    const int h = (int)(gid % p.H);
    const int64_t r = gid / p.H;
    const int b = find_sample(p.kv_off, p.B, r);
    const Sample s = load_sample(p.q_off, p.lq_fixed, p.kv_off, b);
    const int j = (int)(r - s.ks);
    const float *Q = static_cast<const float *>(p.q);
    const float *G = static_cast<const float *>(p.dout);
    BiasArgs bz{p.bias, p.bias_kind, p.bias_lo, p.bias_hi, p.bias_hi - p.bias_lo + 1};
    const float *brow = bz.kind ? bz.table + (int64_t)h * bz.width : nullptr;
    const float *kj = static_cast<const float *>(p.k) + (r * p.H + h) * (int64_t)D;
    const float *vj = static_cast<const float *>(p.v) + (r * p.H + h) * (int64_t)D;
    float dk[D], dv[D];
    for (int d = 0; d < D; ++d) dk[d] = dv[d] = 0.0f;
    // query rows that see key j: j < key_end(i)  <=>  i >= j - (lk - lq) under causal masking
    int i_first = p.causal ? j - (s.lk - s.lq) : 0;
    i_first = i_first < 0 ? 0 : i_first;
    for (int i = i_first; i < s.lq; ++i) {
        if (j < key_begin(i, s.lq, s.lk, p.window) || j >= key_end(i, s.lq, s.lk, p.causal, p.window)) continue;
        const float *qi = Q + ((s.qs + i) * p.H + h) * (int64_t)D;
        const float *gi = G + ((s.qs + i) * p.H + h) * (int64_t)D;
        float x = p.scale * dot_f32(qi, kj, D);
        if (brow) x += bias_at(bz, brow, i, j);
        const float dp = dot_f32(gi, vj, D);
        float w, ds;
        if constexpr (MODE == GDPA) {
            w = act_f32<ACT>(x);
            ds = dp * act_grad_f32<ACT>(x);
        } else {
            const int64_t row = s.qs + i;
            w = expf(x - p.lse[(int64_t)h * p.total_q + row]);
            ds = w * (dp - p.delta[(int64_t)h * p.total_q + row]);
        }
        for (int d = 0; d < D; ++d) {
            dk[d] = __builtin_fmaf(ds, qi[d], dk[d]);
            dv[d] = __builtin_fmaf(w, gi[d], dv[d]);
        }
    }
    float *dkp = static_cast<float *>(p.dk) + (r * p.H + h) * (int64_t)D;
    float *dvp = static_cast<float *>(p.dv) + (r * p.H + h) * (int64_t)D;
    for (int d = 0; d < D; ++d) {
        dkp[d] = dk[d] * p.scale;
        dvp[d] = dv[d];
    }
}

// Gradient of the bias table: one thread per (head, table entry c) adds dX of
// every valid pair that reads entry c, sample by sample in order.  An interior
// entry is one relative position (REL: i - j = lo + c) or one key (KEYPOS:
// j = lo + c), so only those pairs are visited; the two end entries also take
// every clamped position and scan the pairs beyond them.
template <int D, int MODE, int ACT>
__global__ __launch_bounds__(F32_THREADS) void dbias_f32_kernel(const AttnParams p) {
    const BiasArgs bz{p.bias, p.bias_kind, p.bias_lo, p.bias_hi, p.bias_hi - p.bias_lo + 1};
    const int64_t gid = (int64_t)blockIdx.x * F32_THREADS + threadIdx.x;
    if (gid >= (int64_t)p.H * bz.width) return;
    const int h = (int)(gid / bz.width), c = (int)(gid % bz.width);
    const float *brow = bz.table + (int64_t)h * bz.width;
    const float *Q = static_cast<const float *>(p.q);
    const float *K = static_cast<const float *>(p.k);
    const float *V = static_cast<const float *>(p.v);
    const float *G = static_cast<const float *>(p.dout);
    const bool first = c == 0, last = c == bz.width - 1;
    const int target = bz.lo + c;  // position read by entry c when not clamped
    float acc = 0.0f;
    for (int b = 0; b < p.B; ++b) {
        const Sample s = load_sample(p.q_off, p.lq_fixed, p.kv_off, b);
        for (int i = 0; i < s.lq; ++i) {
            const int64_t r = s.qs + i;
            const float *qi = Q + (r * p.H + h) * (int64_t)D;
            const float *gi = G + (r * p.H + h) * (int64_t)D;
            const int kend = key_end(i, s.lq, s.lk, p.causal, p.window);
            const int kbeg = key_begin(i, s.lq, s.lk, p.window);
            // keys of row i whose position maps to entry c: [ja, jb)
            int ja = kbeg, jb = kend;
            if (bz.kind == BIAS_REL) {  // position i - j
                if (!last) ja = max(ja, i - target);       // i - j <= target
                if (!first) jb = min(jb, i - target + 1);  // i - j >= target
            } else {                    // position j
                if (!first) ja = max(ja, target);
                if (!last) jb = min(jb, target + 1);
            }
            ja = ja < 0 ? 0 : ja;
            for (int j = ja; j < jb; ++j) {
                const float *kj = K + ((s.ks + j) * p.H + h) * (int64_t)D;
                const float *vj = V + ((s.ks + j) * p.H + h) * (int64_t)D;
                const float x = p.scale * dot_f32(qi, kj, D) + bias_at(bz, brow, i, j);
                const float dp = dot_f32(gi, vj, D);
                if constexpr (MODE == GDPA) {
                    acc += dp * act_grad_f32<ACT>(x);
                } else {
                    acc += expf(x - p.lse[(int64_t)h * p.total_q + r]) * (dp - p.delta[(int64_t)h * p.total_q + r]);
                }
            }
        }
    }
    p.dbias[gid] = acc;
}

static inline unsigned grid_for(int64_t n) { return (unsigned)((n + F32_THREADS - 1) / F32_THREADS); }

template <int D, int MODE, int ACT>
static hipError_t fwd_f32_t(const AttnParams &p, hipStream_t st) {
    const int64_t n = p.total_q_out * p.H;
    const KernelTimer &t = kernel_timer();
    t.begin(K_FWD, st);
    if (n > 0) hipLaunchKernelGGL((fwd_f32_kernel<D, MODE, ACT>), dim3(grid_for(n)), dim3(F32_THREADS), 0, st, p);
    t.end(K_FWD, st);
    return hipGetLastError();
}

template <int D, int MODE, int ACT>
static hipError_t bwd_f32_t(const AttnParams &p, hipStream_t st) {
    const int64_t nq = p.total_q * p.H, nk = p.total_k * p.H;
    const KernelTimer &t = kernel_timer();
    if (MODE == JFA) {
        t.begin(K_BWD_DELTA, st);
        if (nq > 0) hipLaunchKernelGGL((delta_f32_kernel<D>), dim3(grid_for(nq)), dim3(F32_THREADS), 0, st, p);
        t.end(K_BWD_DELTA, st);
    }
    t.begin(K_BWD_Q, st);
    if (nq > 0) hipLaunchKernelGGL((dq_f32_kernel<D, MODE, ACT>), dim3(grid_for(nq)), dim3(F32_THREADS), 0, st, p);
    t.end(K_BWD_Q, st);
    t.begin(K_BWD_KV, st);
    if (nk > 0) hipLaunchKernelGGL((dkdv_f32_kernel<D, MODE, ACT>), dim3(grid_for(nk)), dim3(F32_THREADS), 0, st, p);
    t.end(K_BWD_KV, st);
    if (p.dbias) {
        const int64_t nb = (int64_t)p.H * (p.bias_hi - p.bias_lo + 1);
        t.begin(K_BWD_DBIAS, st);
        hipLaunchKernelGGL((dbias_f32_kernel<D, MODE, ACT>), dim3(grid_for(nb)), dim3(F32_THREADS), 0, st, p);
        t.end(K_BWD_DBIAS, st);
    }
    return hipGetLastError();
}

template <int D, bool BWD>
static hipError_t dispatch_act(const AttnParams &p, int mode, int act, hipStream_t st) {
    if (mode == JFA) return BWD ? bwd_f32_t<D, JFA, SILU>(p, st) : fwd_f32_t<D, JFA, SILU>(p, st);
    switch (act) {
    case SILU: return BWD ? bwd_f32_t<D, GDPA, SILU>(p, st) : fwd_f32_t<D, GDPA, SILU>(p, st);
    case GELU_TANH: return BWD ? bwd_f32_t<D, GDPA, GELU_TANH>(p, st) : fwd_f32_t<D, GDPA, GELU_TANH>(p, st);
    default: return BWD ? bwd_f32_t<D, GDPA, GELU_ERF>(p, st) : fwd_f32_t<D, GDPA, GELU_ERF>(p, st);
    }
}

template <bool BWD>
static hipError_t dispatch_d(const AttnParams &p, int D, int mode, int act, hipStream_t st) {
    switch (D) {
    case 32: return dispatch_act<32, BWD>(p, mode, act, st);
    case 64: return dispatch_act<64, BWD>(p, mode, act, st);
    default: return dispatch_act<128, BWD>(p, mode, act, st);
    }
}

hipError_t launch_fwd_f32(const AttnParams &p, int D, int mode, int act, hipStream_t st) {
    return dispatch_d<false>(p, D, mode, act, st);
}

hipError_t launch_bwd_f32(const AttnParams &p, int D, int mode, int act, hipStream_t st) {
    return dispatch_d<true>(p, D, mode, act, st);
}

}  // namespace ja
