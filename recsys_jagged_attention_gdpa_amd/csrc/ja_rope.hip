// Rotary position embedding for the attention kernels (gfx950).
//
// The pages name a rotary embedding fused into their block-attention kernel
// ("Meta redesigns AI training infrastructure...", section "Custom Kernels and
// 5D Parallelism for Trillion-Parameter Scale") without defining it.  Here it
// is RoFormer's rotation in split-half form: element d < D/2 and element
// d + D/2 of a query or key row at sample-local position t turn by the angle
// t * base^(-2d/D); values are not turned.
//
// Where it runs.  The attention kernels bring key and query tiles from HBM
// into LDS with buffer->LDS copies, which move bytes without passing through
// registers, and the long kernels are bound by LDS bandwidth and VALU issue.
// Turning K inside them would cost an LDS read-modify-write and the
// trigonometry on every visit of a key tile (each query tile of a sample
// visits all its key tiles).  So every row is turned once, by this streaming
// pass, into a turned copy in the caller's workspace; backward turns the dQ
// and dK it produced (gradients of the turned rows) back in place, which is
// the rotation's transpose.
//
// Thread layout: one thread per (row, 4 consecutive pairs); it works out the
// row's position (binary search in the offsets), the 4 angles in fp64 and
// their sine / cosine once, then turns those pairs in every head.
//
// Precision.  The turned rows are operands of bf16 products, so they are bf16
// values: each is the bf16 value nearest to the turn (ties to even), with the
// turn computed in fp64 (cosine and sine of the fp64 angle t * inv_freq[d],
// inv_freq = base^(-2d/D) computed on the host in fp64) and rounded once,
// straight from fp64 to bf16.  Rounding through float32 first would round twice
// and differ from the nearest bf16 value wherever the turn lies within half a
// float32 step of a bf16 midpoint; a float32 turn would be off by a few float32
// steps and differ more often still.  fp32 tensors get the fp64 turn rounded
// once to float32.
#include "ja_device.h"
#include "ja_kernels.h"

namespace ja {

constexpr int ROPE_THREADS = 256;
constexpr int ROPE_PAIRS = 4;  // consecutive pairs per thread

// Position of row `row` within its sample: the last sample b < B whose first
// row is at or before it (empty samples share their start with the next one,
// so the sample found always holds the row).
__device__ __forceinline__ int64_t rope_position(const int32_t *off, int B, int64_t row) {
    if (off == nullptr) return row;  // one shared block: row r sits at position r
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)off[mid] <= row) lo = mid;
        else hi = mid - 1;
    }
    return row - off[lo];
}

// Nearest bf16 value (ties to even) of a double, as bf16 bits.  Normal range:
// round the significand to 8 bits in place (add half a step minus one plus the
// kept part's last bit, clear the 45 dropped bits; a carry moves the exponent),
// after which the double is exactly a bf16 value and converts to float32 exactly
// (past the largest bf16 value it becomes infinite).  Below 2^-126 bf16 steps
// are a fixed 2^-133: round x * 2^133 to an integer instead.
__device__ __forceinline__ uint32_t bf16_bits_nearest(double x) {
    float f;
    if (__builtin_fabs(x) >= 0x1p-126) {
        uint64_t u = __builtin_bit_cast(uint64_t, x);
        u += ((1ull << 44) - 1) + ((u >> 45) & 1ull);
        u &= ~((1ull << 45) - 1);
        f = (float)__builtin_bit_cast(double, u);
    } else {
        f = (float)(__builtin_rint(x * 0x1p133) * 0x1p-133);
    }
    return __builtin_bit_cast(uint32_t, f) >> 16;
}

template <typename T> struct RopeIO;
template <> struct RopeIO<bf16> {
    static __device__ __forceinline__ void load(const bf16 *p, double x[ROPE_PAIRS]) {
        const u32x2 w = *reinterpret_cast<const u32x2 *>(p);
        x[0] = (double)__uint_as_float(w[0] << 16);
        x[1] = (double)__uint_as_float(w[0] & 0xffff0000u);
        x[2] = (double)__uint_as_float(w[1] << 16);
        x[3] = (double)__uint_as_float(w[1] & 0xffff0000u);
    }
    static __device__ __forceinline__ void store(bf16 *p, const double x[ROPE_PAIRS]) {
        u32x2 w;
        w[0] = bf16_bits_nearest(x[0]) | (bf16_bits_nearest(x[1]) << 16);
        w[1] = bf16_bits_nearest(x[2]) | (bf16_bits_nearest(x[3]) << 16);
        *reinterpret_cast<u32x2 *>(p) = w;
    }
};
template <> struct RopeIO<float> {
    static __device__ __forceinline__ void load(const float *p, double x[ROPE_PAIRS]) {
        const f32x4 w = *reinterpret_cast<const f32x4 *>(p);
        for (int e = 0; e < ROPE_PAIRS; ++e) x[e] = (double)w[e];
    }
    static __device__ __forceinline__ void store(float *p, const double x[ROPE_PAIRS]) {
        f32x4 w;
        for (int e = 0; e < ROPE_PAIRS; ++e) w[e] = (float)x[e];
        *reinterpret_cast<f32x4 *>(p) = w;
    }
};

template <typename T, int D>
__global__ __launch_bounds__(ROPE_THREADS) void rope_kernel(const RopeParams p) {
    constexpr int HALF = D / 2;
    constexpr int CPR = HALF / ROPE_PAIRS;  // threads per row
    const int64_t item = (int64_t)blockIdx.x * ROPE_THREADS + threadIdx.x;
    const int64_t n0 = p.seg[0].rows * CPR;
    const int si = item < n0 ? 0 : 1;
    const RopeSeg s = p.seg[si];
    const int64_t it = si ? item - n0 : item;
    if (it >= s.rows * CPR) return;
    const int64_t row = it / CPR;
    const int d0 = (int)(it % CPR) * ROPE_PAIRS;
    const double t = (double)rope_position(s.off, s.B, row);

    double c[ROPE_PAIRS], sn[ROPE_PAIRS];
#pragma unroll
    for (int e = 0; e < ROPE_PAIRS; ++e) {
        // angle t * base^(-2d/D) in fp64: positions reach the tens of thousands,
        // where an fp32 angle would be off by ~1e-3 rad
        const double a = t * p.inv_freq[d0 + e];
        double sd, cd;
        sincos(a, &sd, &cd);
        c[e] = cd;
        sn[e] = p.sign * sd;  // sign -1: the inverse turn
    }
    const T *src = static_cast<const T *>(s.src) + row * p.H * D;
    T *dst = static_cast<T *>(s.dst) + row * p.H * D;
    for (int h = 0; h < p.H; ++h) {
        double x0[ROPE_PAIRS], x1[ROPE_PAIRS], y0[ROPE_PAIRS], y1[ROPE_PAIRS];
        RopeIO<T>::load(src + h * D + d0, x0);
        RopeIO<T>::load(src + h * D + HALF + d0, x1);
#pragma unroll
        for (int e = 0; e < ROPE_PAIRS; ++e) {
            y0[e] = x0[e] * c[e] - x1[e] * sn[e];
            y1[e] = x0[e] * sn[e] + x1[e] * c[e];
        }
        RopeIO<T>::store(dst + h * D + d0, y0);
        RopeIO<T>::store(dst + h * D + HALF + d0, y1);
    }
}

template <typename T>
static hipError_t launch_rope_t(const RopeParams &p, int D, hipStream_t stream) {
    const int cpr = D / 2 / ROPE_PAIRS;
    const int64_t items = (p.seg[0].rows + p.seg[1].rows) * cpr;
    if (items == 0) return hipSuccess;
    const dim3 grid((unsigned)((items + ROPE_THREADS - 1) / ROPE_THREADS));
    switch (D) {
    case 32: rope_kernel<T, 32><<<grid, ROPE_THREADS, 0, stream>>>(p); break;
    case 64: rope_kernel<T, 64><<<grid, ROPE_THREADS, 0, stream>>>(p); break;
    default: rope_kernel<T, 128><<<grid, ROPE_THREADS, 0, stream>>>(p); break;
    }
    return hipGetLastError();
}

hipError_t launch_rope(const RopeParams &p, int D, bool f32, int timer_id, hipStream_t stream) {
    kernel_timer().begin(timer_id, stream);
    const hipError_t e = f32 ? launch_rope_t<float>(p, D, stream) : launch_rope_t<bf16>(p, D, stream);
    kernel_timer().end(timer_id, stream);
    return e;
}

}  // namespace ja
