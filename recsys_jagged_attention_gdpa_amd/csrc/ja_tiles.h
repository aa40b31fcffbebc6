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

// A slice of one head of a [T, H, D] bf16 tensor: rows 0 .. rows-1 starting at
// global row `row0`, read and written through a bounds-checked descriptor.
template <int D>
struct HeadSlice {
    rsrc_t r;
    uint32_t row_bytes;  // H * D * 2
    __device__ __forceinline__ HeadSlice(const void *base, int64_t row0, int rows, int H, int h) {
        const bf16 *p = static_cast<const bf16 *>(base) + (row0 * H + h) * (int64_t)D;
        r = make_rsrc(p, rows_span(rows, H, D, 2));
        row_bytes = (uint32_t)(H * D * 2);
    }
    // 16 bytes (chunk c = 8 bf16) of row `row`; zeros past the slice.
    template <int CP = CP_DEFAULT>
    __device__ __forceinline__ u32x4 load16(int row, int c) const {
        return buf_load16<CP>(r, (uint32_t)row * row_bytes + (uint32_t)c * 16u);
    }
    __device__ __forceinline__ void store8(int row, int d, u32x2 v) const {
        buf_store8(r, (uint32_t)row * row_bytes + (uint32_t)d * 2u, v);
    }
    template <int CP = CP_DEFAULT>
    __device__ __forceinline__ void store16(int row, int c, u32x4 v) const {
        buf_store16<CP>(r, (uint32_t)row * row_bytes + (uint32_t)c * 16u, v);
    }
};

// ROWS rows of two head slices (Q and dO) staged through registers into the
// swizzled LDS layout by NT threads; rows past the slice become zeros.
template <int ROWS, int D, int NT, int CP = CP_DEFAULT>
struct PairSliceLoader {
    static constexpr int CHUNKS = ROWS * D / 8;
    static constexpr int PER_THREAD = CHUNKS / NT;
    static_assert(PER_THREAD >= 1 && CHUNKS % NT == 0, "tile / thread count mismatch");
    u32x4 a[PER_THREAD], b[PER_THREAD];
    __device__ __forceinline__ void load(const HeadSlice<D> &A, const HeadSlice<D> &B, int r0, int tid) {
#pragma unroll
        for (int it = 0; it < PER_THREAD; ++it) {
            const int cid = tid + it * NT;
            const int r = cid / (D / 8), c = cid % (D / 8);
            a[it] = A.template load16<CP>(r0 + r, c);
            b[it] = B.template load16<CP>(r0 + r, c);
        }
    }
    __device__ __forceinline__ void store(lchar *ta, lchar *tb, int tid) const {
#pragma unroll
        for (int it = 0; it < PER_THREAD; ++it) {
            const int cid = tid + it * NT;
            const int r = cid / (D / 8), c = cid % (D / 8);
            lds_write16(ta, lds_off<D>(r, c), a[it]);
            lds_write16(tb, lds_off<D>(r, c), b[it]);
        }
    }
};

// ROWS x D tile of one head slice copied by NT threads straight from global
// memory into the swizzled LDS layout (buffer_load ... lds: lane i of an
// instruction writes LDS bytes base + 16 i .. +15, so each lane fetches the
// logical chunk that the swizzle puts in its slot).  Rows past the slice land
// as zeros.  The copy is complete once this wave's vector-memory counter has
// drained; other waves' parts need a barrier after that.
template <int ROWS, int D, int NT>
__device__ __forceinline__ void dma_tile(lchar *tile, const HeadSlice<D> &S, int r0, int tid) {
    constexpr int CH = D / 8, SLOTS = ROWS * CH, PER_INSTR = NT / WAVE * WAVE;
    static_assert(SLOTS % NT == 0 || (SLOTS < NT && SLOTS % WAVE == 0), "tile / thread count mismatch");
    const int wv = tid / WAVE, lane = tid % WAVE;
#pragma unroll
    for (int it = 0; it < (SLOTS >= NT ? SLOTS / NT : 1); ++it) {
        const int first = it * PER_INSTR + wv * WAVE;  // first slot of this wave's instruction
        if (SLOTS < NT && first >= SLOTS) break;       // a small tile: only the first waves copy
        const int q = first + lane;
        const int r = q / CH, c = (q % CH) ^ swz<D>(r);
        buf_load16_lds(S.r, tile + first * 16, (uint32_t)(r0 + r) * S.row_bytes + (uint32_t)c * 16u);
    }
}

// A 32-row tile of one head slice, loaded by one wave with 16 bytes per lane
// (whole rows per instruction) into registers, then written to a swizzled LDS
// tile; rows past the slice become zeros.
template <int D, int CP = CP_DEFAULT>
struct WaveTile {
    static constexpr int PER_LANE = 32 * D / 8 / WAVE;
    u32x4 a[PER_LANE];
    __device__ __forceinline__ void load(const HeadSlice<D> &S, int r0, int lane) {
#pragma unroll
        for (int it = 0; it < PER_LANE; ++it) {
            const int cid = lane + it * WAVE;
            a[it] = S.template load16<CP>(r0 + cid / (D / 8), cid % (D / 8));
        }
    }
    __device__ __forceinline__ void store(lchar *t, int lane) const {
#pragma unroll
        for (int it = 0; it < PER_LANE; ++it) {
            const int cid = lane + it * WAVE;
            lds_write16(t, lds_off<D>(cid / (D / 8), cid % (D / 8)), a[it]);
        }
    }
};

// One lane's row of a head slice in MFMA operand layout (chunk 2kk+g for k-step kk).
template <int D, int CP = CP_DEFAULT>
__device__ __forceinline__ void load_row_operand(bf16x8 (&reg)[D / 16], const HeadSlice<D> &S, int row, int g) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) reg[kk] = __builtin_bit_cast(bf16x8, S.template load16<CP>(row, 2 * kk + g));
}

// The rotary turn's transpose on one lane's D^T-layout accumulator set (the
// gradient of a row at sample-local position t, element e of block db being
// column db*32 + crow(e, g)): column d < D/2 and its partner d + D/2 sit in the
// same lane, in block db + D/64 at the same element (D = 32: element e + 8 of
// the one block).  rev[d] is the pair's frequency in turns per position; the
// angle t * rev[d] is formed and reduced to [-1/2, 1/2] turn in fp64 (positions
// reach the hundreds of thousands), its sine and cosine taken by the hardware's
// fp32 sine and cosine, which take turns (absolute error about 2^-23, far below
// the bf16 rounding of the gradient that follows).
template <int D>
__device__ __forceinline__ void rope_back_acc(f32x16 (&acc)[D / 32], int t, const double *rev, int g) {
    // (cos, sin) of the angle of pair d at position t
    auto angle = [&](int d, float &cs, float &sn) {
        const double r = (double)t * rev[d];
        const float f = (float)(r - __builtin_rint(r));
        sn = __builtin_amdgcn_sinf(f);
        cs = __builtin_amdgcn_cosf(f);
    };
    if constexpr (D == 32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float cs, sn;
            angle(crow(e, g), cs, sn);
            const float x = acc[0][e], y = acc[0][e + 8];
            acc[0][e] = cs * x + sn * y;
            acc[0][e + 8] = cs * y - sn * x;
        }
    } else {
        constexpr int HB = D / 64;
#pragma unroll
        for (int db = 0; db < HB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float cs, sn;
                angle(db * 32 + crow(e, g), cs, sn);
                const float x = acc[db][e], y = acc[db + HB][e];
                acc[db][e] = cs * x + sn * y;
                acc[db + HB][e] = cs * y - sn * x;
            }
    }
}

// Store a D^T-layout accumulator block set (lane owns row `row` of the slice;
// element e of block db is column db*32 + crow(e, g)) as bf16 times `mul`.
// Rows past the slice are dropped by the descriptor.
template <int D>
__device__ __forceinline__ void store_row_acc(const HeadSlice<D> &S, int row, const f32x16 (&acc)[D / 32], float mul,
                                              int g) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            S.store8(row, db * 32 + r4 * 8 + g * 4,
                     u32x2{pack2(acc[db][r4 * 4 + 0] * mul, acc[db][r4 * 4 + 1] * mul),
                           pack2(acc[db][r4 * 4 + 2] * mul, acc[db][r4 * 4 + 3] * mul)});
}

// Output tiles leave a wave as whole rows: the D^T-layout accumulators (lane
// owns row l32; element e of block db is column db*32 + crow(e, g)) are first
// written, as bf16 times `mul`, into a 32 x D swizzled LDS tile owned by the
// wave, then read back row-major and stored with 16 bytes per lane (4 rows of
// 256 bytes per instruction for D = 128).  Writing 8-byte pieces of 32
// different rows straight to memory costs about a fifth of the achievable
// HBM bandwidth.  RESID stages the rounding residual x - bf16(x) instead.
template <int D, bool RESID = false>
__device__ __forceinline__ void stage_acc_block(lchar *st, const f32x16 &acc, int db, float mul, int l32, int g) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        float x[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            x[t] = acc[r4 * 4 + t] * mul;
            if (RESID) x[t] = x[t] - bf2f(f2bf(x[t]));
        }
        const u32x2 v{pack2(x[0], x[1]), pack2(x[2], x[3])};
        *reinterpret_cast<__attribute__((address_space(3))) u32x2 *>(st + lds_off<D>(l32, db * 4 + r4) + g * 8) = v;
    }
}

// The rounding residual x - bf16(x) of one accumulator block (x = acc * mul),
// stored straight from the D^T layout (lane owns row `row`).
template <int D>
__device__ __forceinline__ void store_resid_block(const HeadSlice<D> &R, int row, const f32x16 &acc, int db, float mul,
                                                  int g) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        float rs[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float x = acc[r4 * 4 + t] * mul;
            rs[t] = x - bf2f(f2bf(x));
        }
        R.store8(row, db * 32 + r4 * 8 + g * 4, u32x2{pack2(rs[0], rs[1]), pack2(rs[2], rs[3])});
    }
}

template <int D, bool RESID = false>
__device__ __forceinline__ void stage_row_acc(lchar *st, const f32x16 (&acc)[D / 32], float mul, int l32, int g) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) stage_acc_block<D, RESID>(st, acc[db], db, mul, l32, g);
}

// Store a staged 32 x D tile as rows row0 .. row0+31 of S (one wave; rows past
// the slice are dropped by the descriptor).
template <int D>
__device__ __forceinline__ void store_staged(const HeadSlice<D> &S, const lchar *st, int row0, int lane) {
    constexpr int CH = D / 8;
#pragma unroll
    for (int it = 0; it < 32 * CH / WAVE; ++it) {
        const int cid = lane + it * WAVE;
        const int r = cid / CH, c = cid % CH;
        S.template store16<CP_NT>(row0 + r, c, __builtin_bit_cast(u32x4, lds_read16(st, lds_off<D>(r, c))));
    }
}

// Stage and store one accumulator tile (the two steps above, with the LDS
// write -> read ordering in between).
template <int D, bool RESID = false>
__device__ __forceinline__ void store_tile(const HeadSlice<D> &S, lchar *st, int row0, const f32x16 (&acc)[D / 32],
                                           float mul, int lane) {
    stage_row_acc<D, RESID>(st, acc, mul, lane & 31, lane >> 5);
    lds_wave_sync();
    store_staged<D>(S, st, row0, lane);
}

// As above, and also store the rounding residual x - bf16(x) into R.
template <int D>
__device__ __forceinline__ void store_row_acc_split(const HeadSlice<D> &S, const HeadSlice<D> &R, int row,
                                                    const f32x16 (&acc)[D / 32], float mul, int g) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            float x[4], rs[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                x[t] = acc[db][r4 * 4 + t] * mul;
                rs[t] = x[t] - bf2f(f2bf(x[t]));
            }
            const int d = db * 32 + r4 * 8 + g * 4;
            S.store8(row, d, u32x2{pack2(x[0], x[1]), pack2(x[2], x[3])});
            R.store8(row, d, u32x2{pack2(rs[0], rs[1]), pack2(rs[2], rs[3])});
        }
}

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
// The bf16 rounding residuals v - bf16(v), packed like pack_operands: with
// both packings as operands, two MFMAs into one accumulator multiply by v to
// about 2^-17 relative instead of 2^-9.
__device__ __forceinline__ void pack_residual_operands(const float (&v)[16], bf16x8 &lo, bf16x8 &hi) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        lo[e] = f2bf(v[e] - bf2f(f2bf(v[e])));
        hi[e] = f2bf(v[8 + e] - bf2f(f2bf(v[8 + e])));
    }
}

__device__ __forceinline__ void pack_operands(const float (&v)[16], bf16x8 &lo, bf16x8 &hi) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        lo[e] = f2bf(v[e]);
        hi[e] = f2bf(v[8 + e]);
    }
}

// ------------------------------------------------------------------ MXFP8
// MXFP8 inputs (OCP Microscaling: FP8 E4M3 elements, one E8M0 scale 2^(E-127)
// per block of 32 consecutive head-dimension elements of a row and head) are
// read as codes and decoded to bf16 after the load, so the attention arithmetic
// is the bf16 path's on exactly the decoded values: each chunk of 8 elements
// lies inside one block, and v_cvt_scalef32_pk_bf16_fp8 turns two codes into
// two bf16 values times a float32 scale (byte pairs 0-1 / 2-3 by its word
// select; checked on the hardware against the format's table).  A scale code
// becomes the float32 with that biased exponent; codes 0 and 255 (2^-127, NaN)
// are outside what the kernels decode (they read as scales 0 and infinity).

// Codes of one 8-element chunk and its block's scale code.
struct MXRaw {
    u32x2 codes;
    uint32_t scale;
};

__device__ __forceinline__ u32x4 mx_decode(const MXRaw &r) {
    const float sc = __builtin_bit_cast(float, r.scale << 23);
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.codes[0], sc, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.codes[0], sc, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.codes[1], sc, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.codes[1], sc, true);
    return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                 __builtin_bit_cast(uint32_t, d)};
}

// Codes of two adjacent chunks (16 elements, inside one block) and the block's
// scale code.
struct MXRaw2 {
    u32x4 codes;
    uint32_t scale;
};

__device__ __forceinline__ void mx_decode2(const MXRaw2 &r, u32x4 &lo, u32x4 &hi) {
    lo = mx_decode(MXRaw{u32x2{r.codes[0], r.codes[1]}, r.scale});
    hi = mx_decode(MXRaw{u32x2{r.codes[2], r.codes[3]}, r.scale});
}

// One head of an MXFP8 [T, H, D] tensor (codes) with its [T, H, D / 32] scale
// codes: rows 0 .. rows-1 from global row `row0`, through bounds-checked
// descriptors (rows past the slice read as zero codes, i.e. zeros).
template <int D>
struct MXSlice {
    rsrc_t c, s;
    uint32_t row_bytes, srow_bytes;  // H * D and H * D / 32
    __device__ __forceinline__ MXSlice(const void *codes, const void *scales, int64_t row0, int rows, int H, int h) {
        c = make_rsrc(static_cast<const uint8_t *>(codes) + (row0 * H + h) * (int64_t)D, rows_span(rows, H, D, 1));
        s = make_rsrc(static_cast<const uint8_t *>(scales) + (row0 * H + h) * (int64_t)(D / 32),
                      rows_span(rows, H, D / 32, 1));
        row_bytes = (uint32_t)(H * D);
        srow_bytes = (uint32_t)(H * D / 32);
    }
    // chunk ch (elements 8 ch .. 8 ch + 7, in block ch / 4) of row `row`;
    // valid = false reads zeros (an always out-of-range offset)
    __device__ __forceinline__ MXRaw raw(int row, int ch, bool valid = true) const {
        const uint32_t oc = valid ? (uint32_t)row * row_bytes + (uint32_t)ch * 8u : OOB;
        const uint32_t os = valid ? (uint32_t)row * srow_bytes + (uint32_t)(ch >> 2) : OOB;
        MXRaw r;
        r.codes = __builtin_amdgcn_raw_buffer_load_b64(c, (int)oc, 0, 0);
        r.scale = __builtin_amdgcn_raw_buffer_load_b8(s, (int)os, 0, 0);
        return r;
    }
    __device__ __forceinline__ u32x4 load16(int row, int ch) const { return mx_decode(raw(row, ch)); }
    // 16 codes (chunks 2 pr and 2 pr + 1) of row `row`, no scale
    __device__ __forceinline__ u32x4 codes16(int row, int pr) const {
        return __builtin_amdgcn_raw_buffer_load_b128(c, (int)((uint32_t)row * row_bytes + (uint32_t)pr * 16u), 0, 0);
    }
    // chunks 2 pr and 2 pr + 1 (16 elements, in block pr / 2) of row `row`: one
    // 16-byte load of codes and one scale byte
    __device__ __forceinline__ MXRaw2 raw2(int row, int pr, bool valid = true) const {
        const uint32_t oc = valid ? (uint32_t)row * row_bytes + (uint32_t)pr * 16u : OOB;
        const uint32_t os = valid ? (uint32_t)row * srow_bytes + (uint32_t)(pr >> 1) : OOB;
        MXRaw2 r;
        r.codes = __builtin_amdgcn_raw_buffer_load_b128(c, (int)oc, 0, 0);
        r.scale = __builtin_amdgcn_raw_buffer_load_b8(s, (int)os, 0, 0);
        return r;
    }
};

// One lane's row of an MXFP8 slice in MFMA operand layout (chunk 2kk+g for k-step kk).
template <int D>
__device__ __forceinline__ void load_row_operand(bf16x8 (&reg)[D / 16], const MXSlice<D> &S, int row, int g) {
    MXRaw r[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) r[kk] = S.raw(row, 2 * kk + g);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) reg[kk] = __builtin_bit_cast(bf16x8, mx_decode(r[kk]));
}

// ROWS rows of two MXFP8 slices (K and V) staged by NT threads into bf16 tiles
// of the swizzled LDS layout: load() issues the reads of the codes, store()
// decodes and writes, so the loads can stay in flight across other work.
template <int ROWS, int D, int NT>
struct MXPairLoader {
    static constexpr int PAIRS = ROWS * D / 16;  // 16-code pieces (two chunks)
    static constexpr int PER_THREAD = (PAIRS + NT - 1) / NT;
    static_assert(PAIRS % NT == 0 || PAIRS < NT, "tile / thread count mismatch");
    MXRaw2 a[PER_THREAD], b[PER_THREAD];
    __device__ __forceinline__ void load(const MXSlice<D> &A, const MXSlice<D> &B, int r0, int tid) {
#pragma unroll
        for (int it = 0; it < PER_THREAD; ++it) {
            const int cid = tid + it * NT;
            const int r = cid / (D / 16), pr = cid % (D / 16);
            // slots past the tile (PAIRS < NT) read zeros
            a[it] = A.raw2(r0 + r, pr, cid < PAIRS);
            b[it] = B.raw2(r0 + r, pr, cid < PAIRS);
        }
    }
    __device__ __forceinline__ void store(lchar *ta, lchar *tb, int tid) const {
#pragma unroll
        for (int it = 0; it < PER_THREAD; ++it) {
            const int cid = tid + it * NT;
            const int r = cid / (D / 16), pr = cid % (D / 16);
            if (PAIRS % NT != 0 && cid >= PAIRS) continue;
            u32x4 lo, hi;
            mx_decode2(a[it], lo, hi);
            lds_write16(ta, lds_off<D>(r, 2 * pr), lo);
            lds_write16(ta, lds_off<D>(r, 2 * pr + 1), hi);
            mx_decode2(b[it], lo, hi);
            lds_write16(tb, lds_off<D>(r, 2 * pr), lo);
            lds_write16(tb, lds_off<D>(r, 2 * pr + 1), hi);
        }
    }
};

// One MXFP8 tensor's ROWS rows staged like MXPairLoader (codes in registers,
// decoded into a bf16 tile by store()).
template <int ROWS, int D, int NT>
struct MXTileLoader {
    static constexpr int PAIRS = ROWS * D / 16;
    static constexpr int PER_THREAD = (PAIRS + NT - 1) / NT;
    static_assert(PAIRS % NT == 0 || PAIRS < NT, "tile / thread count mismatch");
    MXRaw2 a[PER_THREAD];
    __device__ __forceinline__ void load(const MXSlice<D> &A, int r0, int tid) {
#pragma unroll
        for (int it = 0; it < PER_THREAD; ++it) {
            const int cid = tid + it * NT;
            a[it] = A.raw2(r0 + cid / (D / 16), cid % (D / 16), cid < PAIRS);
        }
    }
    __device__ __forceinline__ void store(lchar *ta, int tid) const {
#pragma unroll
        for (int it = 0; it < PER_THREAD; ++it) {
            const int cid = tid + it * NT;
            const int r = cid / (D / 16), pr = cid % (D / 16);
            if (PAIRS % NT != 0 && cid >= PAIRS) continue;
            u32x4 lo, hi;
            mx_decode2(a[it], lo, hi);
            lds_write16(ta, lds_off<D>(r, 2 * pr), lo);
            lds_write16(ta, lds_off<D>(r, 2 * pr + 1), hi);
        }
    }
};

// ---------------------------------------------- fp8 codes for the fp8 MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands (layouts checked on the
// hardware with exact small-integer data): lane l gives row / column l % 32;
// bytes 0-15 of its 32 code bytes belong to the first 32-element block of the
// 64-element k-step and bytes 16-31 to the second, so both lane halves feed
// both blocks (any pairing A and B share gives the same sums; here half g takes
// codes 16 g .. 16 g + 15 of each block); the scale of (row r, block kb) is
// byte 0 of lane r + 32 kb's scale operand; the accumulator layout is the bf16
// 32x32 one.  Code tiles in LDS have D-byte rows whose 16-byte chunks are
// XOR-swizzled so that the operand reads of 8 consecutive rows at one chunk
// hit 8 different bank groups: by the row's low three bits for 128-byte rows,
// by bits 1-2 for 64-byte rows (two rows share a 128-byte bank line).
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int D>
__device__ __forceinline__ int f8_off(int r, int c) {
    static_assert(D == 64 || D == 128, "code tiles for D = 64 or 128");
    if constexpr (D == 128) return r * 128 + ((c ^ (r & 7)) << 4);
    else return r * 64 + ((c ^ ((r >> 1) & 3)) << 4);
}

// ROWS rows of D codes copied by NT threads straight into a swizzled code
// tile (buffer_load ... lds; lane i of an instruction writes 16 bytes at slot
// i, so each lane fetches the chunk the swizzle puts there).  Rows past the
// slice land as zero codes.
template <int ROWS, int D, int NT>
__device__ __forceinline__ void dma_f8_tile(lchar *tile, const MXSlice<D> &S, int r0, int tid) {
    constexpr int CH = D / 16, SLOTS = ROWS * CH, PER_INSTR = NT / WAVE * WAVE;
    static_assert(SLOTS % NT == 0, "tile / thread count mismatch");
    const int wv = tid / WAVE, lane = tid % WAVE;
#pragma unroll
    for (int it = 0; it < SLOTS / NT; ++it) {
        const int first = it * PER_INSTR + wv * WAVE;
        const int q = first + lane;
        const int r = q / CH;
        const int c = (f8_off<D>(r, q % CH) - r * D) >> 4;  // the swizzle is an involution
        buf_load16_lds(S.c, tile + first * 16, (uint32_t)(r0 + r) * S.row_bytes + (uint32_t)c * 16u);
    }
}

// Operand (k-step ks) of row r of a code tile, for lane half g.
template <int D>
__device__ __forceinline__ i32x8 lds_read_f8_operand(const lchar *tile, int r, int ks, int g) {
    const u32x4 lo = __builtin_bit_cast(u32x4, lds_read16(tile, f8_off<D>(r, 4 * ks + g)));
    const u32x4 hi = __builtin_bit_cast(u32x4, lds_read16(tile, f8_off<D>(r, 4 * ks + 2 + g)));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Operand (k-step ks) of row `row` of an MXFP8 slice, for lane half g.
template <int D>
__device__ __forceinline__ i32x8 f8_row_operand(const MXSlice<D> &S, int row, int ks, int g) {
    const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(S.c, (int)((uint32_t)row * S.row_bytes + (uint32_t)(4 * ks + g) * 16u), 0, 0);
    const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(S.c, (int)((uint32_t)row * S.row_bytes + (uint32_t)(4 * ks + 2 + g) * 16u), 0, 0);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
// Scale code of block `blk` of row `row`.
template <int D>
__device__ __forceinline__ int f8_scale(const MXSlice<D> &S, int row, int blk) {
    return (int)__builtin_amdgcn_raw_buffer_load_b8(S.s, (int)((uint32_t)row * S.srow_bytes + (uint32_t)blk), 0, 0);
}

// A 32-row block of MXFP8 codes read by one wave (16 codes per lane and load,
// whole rows per instruction) and written as codes into a swizzled code tile
// for the fp8 MFMA, with the scale codes of the lane's operand row r0 + l % 32
// for blocks 2 ks + l / 32.
template <int D>
struct F8WaveTile {
    static constexpr int PER_LANE = 32 * D / 16 / WAVE;
    static_assert((32 * D / 16) % WAVE == 0, "tile / lane count mismatch");
    u32x4 a[PER_LANE];
    int sc[D / 64];
    __device__ __forceinline__ void load(const MXSlice<D> &S, int r0, int lane) {
#pragma unroll
        for (int it = 0; it < PER_LANE; ++it) {
            const int cid = lane + it * WAVE;
            a[it] = S.codes16(r0 + cid / (D / 16), cid % (D / 16));
        }
#pragma unroll
        for (int ks = 0; ks < D / 64; ++ks) sc[ks] = f8_scale<D>(S, r0 + (lane & 31), 2 * ks + (lane >> 5));
    }
    __device__ __forceinline__ void store(lchar *t, int lane) const {
#pragma unroll
        for (int it = 0; it < PER_LANE; ++it) {
            const int cid = lane + it * WAVE;
            lds_write16(t, f8_off<D>(cid / (D / 16), cid % (D / 16)), a[it]);
        }
    }
};

// ------------------------------------------ fp8 PV product (P in FP8 E4M3)
// O^T += V^T P^T on the block-scaled fp8 MFMA, 64 keys (two 32-key blocks) per
// instruction and 32 head-dimension rows per output block.  The MFMA takes one
// scale per (operand row or column, 32-key block); MXFP8 values carry theirs per
// (key, 32-element block of the head dimension), which varies along the key
// axis the product sums over.  So each value row is first re-encoded to one
// exponent per key: S_j = the largest of the row's block scale codes, every
// code c of block b becoming the E4M3 value nearest to value(c) * 2^(s_jb - S_j)
// (exact unless it lands below the normal range).  The value operand then takes
// unit scales, and P takes the key's scale: P'_ij = P_ij * 2^(S_j - 127), encoded
// as E4M3 (nearest, ties to even) against one power-of-two scale per (query,
// 32-key block) that puts the block's largest |P'| in [128, 256).

// A row's D / 32 scale codes as one word (byte b: block b), read once per row:
// lane j of a wave loads the word of row rows[j] and lanes that need it take
// it from there by a cross-lane read, instead of every lane issuing a one- or
// two-byte load of its own (many small loads per tile were measured to cost
// the pooling forward 16 % of its time).
template <int D>
__device__ __forceinline__ uint32_t f8_scale_word(const MXSlice<D> &S, int row, bool ok) {
    const uint32_t os = ok ? (uint32_t)row * S.srow_bytes : OOB;
    if constexpr (D == 128) return __builtin_amdgcn_raw_buffer_load_b32(S.s, (int)os, 0, 0);
    else return __builtin_amdgcn_raw_buffer_load_b16(S.s, (int)os, 0, 0);
}
__device__ __forceinline__ uint32_t lane_word(uint32_t w, int src_lane) {
    return (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane << 2, (int)w);
}

// 2^(S - 127) for an E8M0 code S as a float (2^-127, code 0, is a subnormal).
__device__ __forceinline__ float v_factor(uint32_t code) {
    return __builtin_bit_cast(float, code ? code << 23 : 0x00400000u);
}

// Value rows of a tile staged as re-encoded codes: load() issues the reads of
// 16 codes per piece and of the rows' scale words, store() re-encodes them into
// a code tile (f8_off layout) and writes each row's factor 2^(S_j - 127) into
// s_row[row].
template <int ROWS, int D, int NT>
struct F8VLoader {
    static constexpr int PIECES = ROWS * D / 16;
    static constexpr int PER_THREAD = (PIECES + NT - 1) / NT;
    static constexpr int CPR = D / 16;        // pieces per row
    static constexpr int RPW = WAVE / CPR;    // rows one wave's pieces of one step cover
    static_assert(PIECES % NT == 0 || PIECES < NT, "tile / thread count mismatch");
    static_assert(PER_THREAD * RPW <= WAVE, "one scale word per lane");
    u32x4 c[PER_THREAD];
    uint32_t wrow;  // lane j < PER_THREAD * RPW: the scale word of step j / RPW's row j % RPW for this wave
    __device__ __forceinline__ void load(const MXSlice<D> &S, int r0, int tid) {
#pragma unroll
        for (int it = 0; it < PER_THREAD; ++it) {
            const int q = tid + it * NT;
            const bool ok = q < PIECES;
            const int r = r0 + q / CPR;
            const uint32_t oc = ok ? (uint32_t)r * S.row_bytes + (uint32_t)(q % CPR) * 16u : OOB;
            c[it] = __builtin_amdgcn_raw_buffer_load_b128(S.c, (int)oc, 0, 0);
        }
        const int wv = tid / WAVE, lane = tid % WAVE;
        const int q0 = wv * WAVE + (lane / RPW) * NT;  // first piece of that step for this wave
        wrow = f8_scale_word<D>(S, r0 + q0 / CPR + lane % RPW, lane < PER_THREAD * RPW && q0 < PIECES);
    }
    __device__ __forceinline__ void store(lchar *tile, lfloat *s_row, int tid) const {
#pragma unroll
        for (int it = 0; it < PER_THREAD; ++it) {
            const int q = tid + it * NT;
            // every lane takes part in the cross-lane read, then idle lanes skip
            const uint32_t w = lane_word(wrow, it * RPW + (tid % WAVE) / CPR);
            if (PIECES % NT != 0 && q >= PIECES) continue;
            const int r = q / CPR, pc = q % CPR;
            uint32_t smax = w & 255u, sb = (w >> (8 * (pc >> 1))) & 255u;
#pragma unroll
            for (int b = 1; b < D / 32; ++b) smax = max(smax, (w >> (8 * b)) & 255u);
            u32x4 v = c[it];
            if (smax - sb >= 20u) {
                v = u32x4{};  // every |value| * 2^(sb - smax) <= 448 * 2^-20 rounds to zero
            } else if (sb != smax) {
                // value(c) * 2^(sb - smax): exact products, then nearest E4M3
                const float f = __builtin_bit_cast(float, (127u - (smax - sb)) << 23);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    typedef float f32x2 __attribute__((ext_vector_type(2)));
                    const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[k], f, false);
                    const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[k], f, true);
                    int o = __builtin_amdgcn_cvt_pk_fp8_f32(lo[0], lo[1], 0, false);
                    o = __builtin_amdgcn_cvt_pk_fp8_f32(hi[0], hi[1], o, true);
                    v[k] = (uint32_t)o;
                }
            }
            lds_write16(tile, f8_off<D>(r, pc), v);
            if (pc == 0) s_row[r] = v_factor(smax);
        }
    }
};

// V^T operand (head-dimension block db: row db*32 + l % 32) of the fp8 PV
// product from a code tile of NKB (1 or 2) 32-key blocks, by transposing reads
// (ds_read_b64_tr_b8: within each group of 16 lanes, lane i receives byte i % 8
// of the 8-byte pieces addressed by lanes 2j + i / 8, j = 0 .. 7; checked on the
// hardware).  Lane half g gets keys crow(e, g), e = 0 .. 15, of each block in
// byte order e: the order of the P^T operand built from the score accumulator.
// A missing second block reads as zero codes.
template <int D, int NKB>
__device__ __forceinline__ i32x8 lds_read_vt_f8(const lchar *tile, int db, int lane) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) i32x2 li32x2;
    const int s = lane & 15, G = lane >> 4, g = G >> 1;
    const int c = 2 * db + (G & 1), half = (s & 1) * 8;
    i32x8 out = i32x8{};
#pragma unroll
    for (int r = 0; r < 2 * NKB; ++r) {
        const int row = (r >> 1) * 32 + crow(8 * (r & 1) + (s >> 1), g);
        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((li32x2 *)(tile + f8_off<D>(row, c) + half));
        out[2 * r] = v[0];
        out[2 * r + 1] = v[1];
    }
    return out;
}

// One 32-key block of the P^T operand of the fp8 PV product: a lane's 16 P
// values (query l % 32, keys crow(e, g) of the block) and the block's per-key
// factors f[0 .. 31] = 2^(S_j - 127) (v_factor) give 16 E4M3 codes in byte
// order e; the return value is the block's E8M0 scale code (the same in both
// lane halves; unit when every P' of the block is zero).  P' = P f_j is the
// exact product (a power-of-two factor; it rounds only where P' falls below
// the fp32 normal range, far below anything the block's scale keeps).
__device__ __forceinline__ int encode_p_block(const float (&pv)[16], const lfloat *f, int g, u32x4 &codes) {
    typedef __attribute__((address_space(3))) const f32x4 lcf32x4;
    float pp[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // factors of keys crow(4q .. 4q + 3, g): 4 consecutive entries
        const f32x4 fq = *(lcf32x4 *)(f + q * 8 + g * 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) pp[4 * q + t] = pv[4 * q + t] * fq[t];
    }
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) m = fmaxf(m, __builtin_fabsf(pp[e]));
    m = pair_max(m);  // the block's other 16 keys sit in lane ^ 32
    // largest |P'| = f * 2^k, f in [0.5, 1): scale 2^(k - 8) puts it in [128, 256)
    const int e8 = __builtin_amdgcn_frexp_expf(m) - 8 + 127;
    const int ex = m > 0.0f ? min(max(e8, 1), 254) : 127;
    // 2^(127 - ex) as a float: ex <= 247 for a finite m, so the power is normal
    const float sc = __builtin_bit_cast(float, (uint32_t)(254 - ex) << 23);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(pp[4 * q] * sc, pp[4 * q + 1] * sc, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(pp[4 * q + 2] * sc, pp[4 * q + 3] * sc, w, true);
        codes[q] = (uint32_t)w;
    }
    return ex;
}

// The P^T operand from its blocks: bytes 0-15 block 0, 16-31 block 1 (zero
// codes when there is one block); this lane's scale operand is the code of
// block g.
__device__ __forceinline__ i32x8 p_f8_operand(const u32x4 &b0, const u32x4 &b1) {
    return i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
}

// WaveTile for an MXFP8 slice: 32 rows read as codes by one wave, decoded when
// written to the LDS tile.
template <int D>
struct MXWaveTile {
    static constexpr int PER_LANE = 32 * D / 16 / WAVE;  // 16-code pieces per lane
    static_assert((32 * D / 16) % WAVE == 0, "tile / lane count mismatch");
    MXRaw2 a[PER_LANE];
    __device__ __forceinline__ void load(const MXSlice<D> &S, int r0, int lane) {
#pragma unroll
        for (int it = 0; it < PER_LANE; ++it) {
            const int cid = lane + it * WAVE;
            a[it] = S.raw2(r0 + cid / (D / 16), cid % (D / 16));
        }
    }
    __device__ __forceinline__ void store(lchar *t, int lane) const {
#pragma unroll
        for (int it = 0; it < PER_LANE; ++it) {
            const int cid = lane + it * WAVE;
            const int r = cid / (D / 16), pr = cid % (D / 16);
            u32x4 lo, hi;
            mx_decode2(a[it], lo, hi);
            lds_write16(t, lds_off<D>(r, 2 * pr), lo);
            lds_write16(t, lds_off<D>(r, 2 * pr + 1), hi);
        }
    }
};

}  // namespace ja
