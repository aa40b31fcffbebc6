// Global -> register -> LDS staging of row tiles (bf16 [rows, D] slices of a
// token-major [T, H, D] tensor), into the swizzled LDS layout of ja_device.h.
#pragma once

#include "ja_device.h"

namespace ja {

// ROWS rows of two tensors (e.g. K and V, or Q and dO) of one head, staged by
// NT threads.  Rows at or past `limit` (sample-local) are written as zeros.
template <int ROWS, int D, int NT>
struct PairLoader {
    static constexpr int CHUNKS = ROWS * D / 8;
    static constexpr int PER_THREAD = (CHUNKS + NT - 1) / NT;
    static_assert(CHUNKS % NT == 0 || CHUNKS < NT, "tile / thread count mismatch");
    u32x4 a[PER_THREAD], b[PER_THREAD];

    __device__ __forceinline__ void load(const bf16 *A, const bf16 *B, int64_t row0, int H, int h, int r0,
                                         int limit, int tid) {
#pragma unroll
        for (int it = 0; it < PER_THREAD; ++it) {
            const int cid = tid + it * NT;
            const int r = cid / (D / 8), c = cid % (D / 8);
            const int rr = r0 + r;
            if (cid >= CHUNKS) continue;
            if (rr < limit) {
                const int64_t off = ((row0 + rr) * H + h) * (int64_t)D + c * 8;
                a[it] = *reinterpret_cast<const u32x4 *>(A + off);
                b[it] = *reinterpret_cast<const u32x4 *>(B + off);
            } else {
                a[it] = u32x4{0, 0, 0, 0};
                b[it] = u32x4{0, 0, 0, 0};
            }
        }
    }
    __device__ __forceinline__ void store(lchar *ta, lchar *tb, int tid) {
#pragma unroll
        for (int it = 0; it < PER_THREAD; ++it) {
            const int cid = tid + it * NT;
            const int r = cid / (D / 8), c = cid % (D / 8);
            if (cid >= CHUNKS) continue;
            lds_write16(ta, lds_off<D>(r, c), a[it]);
            lds_write16(tb, lds_off<D>(r, c), b[it]);
        }
    }
};

// One lane's row of a tile in MFMA operand layout (chunk 2kk+g for k-step kk),
// read straight from global memory; zeros when the row is out of range.
template <int D>
__device__ __forceinline__ void load_row_operand(bf16x8 (&reg)[D / 16], const bf16 *base, int64_t row, int H, int h,
                                                 bool valid, int g) {
    if (valid) {
        const bf16 *p = base + (row * H + h) * (int64_t)D + g * 8;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) reg[kk] = *reinterpret_cast<const bf16x8 *>(p + kk * 16);
    } else {
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) reg[kk] = bf16x8{};
    }
}

// Store a D^T-layout accumulator block set (lane owns one output row; element e
// of block db is column db*32 + crow(e, g)) as bf16, multiplied by `mul`.
template <int D>
__device__ __forceinline__ void store_row_acc(bf16 *row_ptr, const f32x16 (&acc)[D / 32], float mul, int g) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d = db * 32 + r4 * 8 + g * 4;
            u32x2 v2;
            v2[0] = pack2(acc[db][r4 * 4 + 0] * mul, acc[db][r4 * 4 + 1] * mul);
            v2[1] = pack2(acc[db][r4 * 4 + 2] * mul, acc[db][r4 * 4 + 3] * mul);
            *reinterpret_cast<u32x2 *>(row_ptr + d) = v2;
        }
    }
}

// As store_row_acc, and also store the rounding residual x - bf16(x) as bf16.
template <int D>
__device__ __forceinline__ void store_row_acc_split(bf16 *row_ptr, bf16 *res_ptr, const f32x16 (&acc)[D / 32],
                                                    float mul, int g) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d = db * 32 + r4 * 8 + g * 4;
            float x[4], rsd[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                x[t] = acc[db][r4 * 4 + t] * mul;
                rsd[t] = x[t] - bf2f(f2bf(x[t]));
            }
            *reinterpret_cast<u32x2 *>(row_ptr + d) = u32x2{pack2(x[0], x[1]), pack2(x[2], x[3])};
            *reinterpret_cast<u32x2 *>(res_ptr + d) = u32x2{pack2(rsd[0], rsd[1]), pack2(rsd[2], rsd[3])};
        }
    }
}

// Pack 16 fp32 accumulator values (C layout of one 32x32 block) into the two
// bf16x8 B operands of the 16-wide k-steps they cover.
__device__ __forceinline__ void pack_operands(const float (&v)[16], bf16x8 &lo, bf16x8 &hi) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        lo[e] = f2bf(v[e]);
        hi[e] = f2bf(v[8 + e]);
    }
}

}  // namespace ja
