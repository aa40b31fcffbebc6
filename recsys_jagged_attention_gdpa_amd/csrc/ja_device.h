// Device-side building blocks shared by the gfx950 jagged attention kernels:
// vector types, MFMA wrappers, the swizzled LDS tile layout, activations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ja {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

enum Mode { GDPA = 0, JFA = 1 };
enum Act { SILU = 0, GELU_TANH = 1, GELU_ERF = 2 };
enum BiasKind { BIAS_NONE = 0, BIAS_REL = 1, BIAS_KEYPOS = 2 };

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_32x32x16_bf16.  Lane layouts (checked on gfx950):
//   A (32 x 16): lane l holds row l%32, k = (l/32)*8 + 0..7
//   B (16 x 32): lane l holds col l%32, k = (l/32)*8 + 0..7
//   C (32 x 32): lane l holds col l%32, rows (e/4)*8 + (l/32)*4 + e%4, e = 0..15
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (within a 32-block) of accumulator element e for lane half g = l/32.
__device__ __forceinline__ int crow(int e, int g) { return (e >> 2) * 8 + g * 4 + (e & 3); }

// ------------------------------------------------------ LDS tile layout
// A tile of R rows x D bf16 is stored row-major with its 16-byte chunks
// permuted per row: chunk c of row r lives at chunk c ^ swz(r).  The
// permutation keeps both access patterns the kernels use free of bank
// conflicts: 16-byte row reads by 8+ consecutive rows at one chunk, and the
// transposing 8-byte reads (4 consecutive rows x 64 bytes per 32 lanes).
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    else return (r >> 2) & 3;
}

// Byte offset of chunk c (8 bf16) of row r.
template <int D>
__device__ __forceinline__ int lds_off(int r, int c) {
    return r * (D * 2) + ((c ^ swz<D>(r)) << 4);
}

// LDS pointers carry their address space so every tile access compiles to a
// ds_* instruction.
typedef __attribute__((address_space(3))) char lchar;
typedef __attribute__((address_space(3))) bf16x8 lbf16x8;
typedef __attribute__((address_space(3))) u32x4 lu32x4;
typedef __attribute__((address_space(3))) s16x4 ls16x4;
typedef __attribute__((address_space(3))) float lfloat;
typedef __attribute__((address_space(3))) uint8_t lu8;

__device__ __forceinline__ bf16x8 lds_read16(const lchar *base, int off) {
    return *reinterpret_cast<const lbf16x8 *>(base + off);
}

__device__ __forceinline__ void lds_write16(lchar *base, int off, u32x4 v) {
    *reinterpret_cast<lu32x4 *>(base + off) = v;
}

// Transposing read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane
// m supplies the address of 4 bf16; lane i receives element i%4 of the values
// addressed by lanes 4j + i/4, j = 0..3.  With lane m addressing row
// key0 + m/4, columns d0 + 4(m%4) .. +3 of a row-major tile, lane i receives
// column d0 + i of rows key0 .. key0+3.
__device__ __forceinline__ bf16x4 lds_read_tr(const lchar *base, int off) {
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ls16x4 *)(base + off));
    return __builtin_bit_cast(bf16x4, r);
}

// Transposed MFMA operand (row d = d0 + l%32 of the transposed tile, k = 8
// rows of the original tile): rows r0 + g*4 + 0..3 and r0 + 8 + g*4 + 0..3 of
// the row-major tile, with g = l/32.  This row order matches the accumulator
// layout's row order (crow), so a C-layout block can be reused as the other
// operand without any shuffle.
template <int D>
__device__ __forceinline__ bf16x8 lds_read_tr_operand(const lchar *tile, int r0, int d0, int lane) {
    const int l16 = lane & 15;
    const int G = lane >> 4;
    const int g = G >> 1;
    const int dcol = d0 + ((G & 1) << 4) + ((l16 & 3) << 2);
    const int c = dcol >> 3;
    const int within = (dcol & 7) << 1;
    const int ra = r0 + g * 4 + (l16 >> 2);
    const int rb = ra + 8;
    bf16x4 lo = lds_read_tr(tile, lds_off<D>(ra, c) + within);
    bf16x4 hi = lds_read_tr(tile, lds_off<D>(rb, c) + within);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ----------------------------------------------------------- conversions
__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ bf16 f2bf(float x) { return (bf16)x; }  // round to nearest even

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(bf16)a, (bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------------ activations
// SiLU(x) = x * sigmoid(x); GELU (tanh form) = x * sigmoid(2u),
// u = sqrt(2/pi) (x + 0.044715 x^3); GELU (erf form) = x * Phi(x).
constexpr float GELU_C = 0.7978845608028654f;  // sqrt(2/pi)
constexpr float GELU_A = 0.044715f;
constexpr float INV_SQRT2 = 0.7071067811865476f;
constexpr float INV_SQRT_2PI = 0.3989422804014327f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// sigmoid(z) with z given as -z * log2(e) (so one v_exp and one v_rcp).
__device__ __forceinline__ float sigmoid_from_neg_log2(float nz) { return fast_rcp(1.0f + fast_exp2(nz)); }

// Standard normal CDF for GELU (erf form): Phi(x) ~= sigmoid(a1 x + a3 x^3 +
// a5 x^5) on [-9, 9], the argument clamped there (Phi(-9) < 1e-18; the
// polynomial turns over near |x| = 11.6).  |error| <= 1.9e-5 on the whole real
// line, far below the bf16 resolution of the P and dX operands, for one
// v_med3_f32, one v_exp_f32, one v_rcp_f32 and three multiply-adds.  a1, a3,
// a5 come from fit_normal_cdf.py (a minimax fit of the sigmoid form); they are
// stored times -log2(e), so sigmoid(p) = 1 / (1 + exp2(p')).
constexpr float PHI_CLAMP = 9.0f;
constexpr float PHI_A1 = 1.5954352491099784f * -LOG2E;
constexpr float PHI_A3 = 0.07359716688590114f * -LOG2E;
constexpr float PHI_A5 = -0.0006317657957178257f * -LOG2E;
__device__ __forceinline__ float normal_cdf(float x) {
    const float xc = __builtin_amdgcn_fmed3f(x, -PHI_CLAMP, PHI_CLAMP);
    const float x2 = xc * xc;
    const float z = xc * __builtin_fmaf(__builtin_fmaf(PHI_A5, x2, PHI_A3), x2, PHI_A1);
    return fast_rcp(1.0f + fast_exp2(z));
}
__device__ __forceinline__ float normal_pdf(float x) { return INV_SQRT_2PI * fast_exp2(x * x * (-0.5f * LOG2E)); }

template <int ACT>
__device__ __forceinline__ float act_fwd(float x) {
    if constexpr (ACT == SILU) {
        return x * sigmoid_from_neg_log2(-x * LOG2E);
    } else if constexpr (ACT == GELU_TANH) {
        const float x2 = x * x;
        const float t = __builtin_fmaf(x2, -2.0f * LOG2E * GELU_C * GELU_A, -2.0f * LOG2E * GELU_C);
        return x * sigmoid_from_neg_log2(x * t);
    } else {
        return x * normal_cdf(x);
    }
}

// Activation value and derivative together (backward).
template <int ACT>
__device__ __forceinline__ void act_fwd_grad(float x, float &y, float &dy) {
    if constexpr (ACT == SILU) {
        const float s = sigmoid_from_neg_log2(-x * LOG2E);
        y = x * s;
        dy = __builtin_fmaf(y, 1.0f - s, s);  // s (1 + x (1 - s))
    } else if constexpr (ACT == GELU_TANH) {
        const float x2 = x * x;
        const float t = __builtin_fmaf(x2, -2.0f * LOG2E * GELU_C * GELU_A, -2.0f * LOG2E * GELU_C);
        const float s = sigmoid_from_neg_log2(x * t);  // sigmoid(2u) = (1 + tanh u) / 2
        y = x * s;
        // d/dx [x s(2u)] = s + x * 2 s (1 - s) * u'(x),  u' = c (1 + 3 a x^2)
        const float du = GELU_C * __builtin_fmaf(3.0f * GELU_A, x2, 1.0f);
        dy = __builtin_fmaf(2.0f * x * s * (1.0f - s), du, s);
    } else {
        const float cdf = normal_cdf(x);
        y = x * cdf;
        dy = __builtin_fmaf(x, normal_pdf(x), cdf);  // Phi + x phi
    }
}

// Order this wave's LDS writes before its later LDS reads of other lanes'
// data (waits for the LDS queue; also a compiler memory barrier).
__device__ __forceinline__ void lds_wave_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// --------------------------------------------------------- buffer access
// Bounds-checked loads and stores through a buffer descriptor: offsets at or
// past num_records read as zero and are not stored.  A descriptor per
// (sample, head) slice turns the ragged row tail into a hardware bound, so the
// streaming loops carry no branches around their memory operations (branches
// there force the compiler to wait for every outstanding access).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_FLAGS = 0x00020000;  // raw 32-bit data format (gfx9 family)
constexpr uint32_t OOB = 0xFFFFFFFFu;   // an offset that is always out of range

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, RSRC_FLAGS);
}
// Bytes spanned by `rows` rows of one head in a [T, H, D] slice starting at that head's first row.
__device__ __forceinline__ uint32_t rows_span(int rows, int H, int D, int esize) {
    return rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * H * D + D) * esize) : 0u;
}
// Cache policy of an access: CP_NT marks data touched once (streamed inputs,
// outputs), so it does not displace data that other units re-read from L2.
constexpr int CP_DEFAULT = 0;
constexpr int CP_NT = 2;
template <int CP = CP_DEFAULT>
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CP);
}
// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes dst + 16 i (dst wave-uniform, in M0); out-of-range lanes write zeros.
// Issued as inline assembly on purpose: the compiler does not know which LDS
// bytes a copy of this kind writes, so after the builtin form it waits for the
// copy to land before the next LDS read of any buffer, which serialises the
// prefetch of the next tile with the reads of the current one.  Callers wait
// for completion themselves (vmcnt, then a barrier for other waves' parts)
// before reading the destination; nothing else in these kernels uses M0.
__device__ __forceinline__ void buf_load16_lds(rsrc_t r, __attribute__((address_space(3))) void *dst, uint32_t off) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(off), "s"(r)
                 : "memory");
}
template <int CP = CP_DEFAULT>
__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, CP));
}
template <int CP = CP_DEFAULT>
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, CP);
}
template <int CP = CP_DEFAULT>
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, CP);
}
template <int CP = CP_DEFAULT>
__device__ __forceinline__ void buf_store_f32(rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, CP);
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector memory
// operations are outstanding, leaving the LDS / export counters unconstrained.
__device__ __host__ constexpr int waitcnt_vm(int n) {
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// ---------------------------------------------------------- misc helpers
__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Max / sum of a value over lanes l and l ^ 32 (the two halves of the wave
// hold different keys of the same query rows).  v_permlane32_swap exchanges
// lanes 32..63 of its first register with lanes 0..31 of its second, so with
// both holding v every lane ends up with its own and its partner's value, and
// no LDS round trip is needed.  It is issued as inline assembly because the
// compiler folds the builtin's two results into one when both inputs are the
// same value; the s_nop covers the VALU-write -> permlane-read hazard.
__device__ __forceinline__ void pair_swap(float &a, float &b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float pair_max(float v) {
    float a = v, b = v;
    pair_swap(a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum(float v) {
    float a = v, b = v;
    pair_swap(a, b);
    return a + b;
}

// v_permlane16_swap_b32: rows of 16 lanes 1 and 3 of a trade places with rows
// 0 and 2 of b, so a becomes (a0, b0, a2, b2) and b (a1, b1, a3, b3) (checked
// on the hardware).  The builtin, so that the compiler places the wait states a
// matrix-core result needs before this read (inline assembly is opaque to that).
__device__ __forceinline__ void row_swap16(uint32_t &a, uint32_t &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    a = r[0];
    b = r[1];
}
__device__ __forceinline__ void row_swap16(float &a, float &b) {
    uint32_t x = __builtin_bit_cast(uint32_t, a), y = __builtin_bit_cast(uint32_t, b);
    row_swap16(x, y);
    a = __builtin_bit_cast(float, x);
    b = __builtin_bit_cast(float, y);
}
// The same with both registers holding one vector-ALU result (the builtin's two
// results may be folded into one when its inputs are equal; the s_nop covers
// the VALU-write -> permlane-read hazard).
__device__ __forceinline__ void row_swap16_same(int &a, int &b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// True on every lane when the predicate holds on any lane (a wave-uniform test).
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

__device__ __forceinline__ float shfl_xor32(float v) {
    // exchange with lane ^ 32 (the other half of the wave)
    const int lane = threadIdx.x & 63;
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(((lane ^ 32) << 2), __builtin_bit_cast(int, v)));
}

// Sample geometry shared by every kernel.
struct Sample {
    int64_t qs;  // first query row (global) of the sample
    int64_t o0;  // first output row (global)
    int64_t ks;  // first key row (global)
    int lq, lk;
};

__device__ __forceinline__ Sample load_sample(const int32_t *q_off, int lq_fixed, const int32_t *kv_off, int b) {
    Sample s;
    if (q_off) {
        const int a = q_off[b], e = q_off[b + 1];
        s.qs = a;
        s.o0 = a;
        s.lq = e - a;
    } else {
        s.qs = 0;
        s.o0 = (int64_t)b * lq_fixed;
        s.lq = lq_fixed;
    }
    const int ka = kv_off[b], ke = kv_off[b + 1];
    s.ks = ka;
    s.lk = ke - ka;
    return s;
}

// Keys visible to query row i are [key_begin, key_end) (empty when begin >= end).
// With ia = i + lk - lq the row's position aligned to the keys (bottom-right):
// causal masking ends them at ia; a sliding window w > 0 keeps aligned
// distances ia - j below w, and without causal masking also j - ia below w.
__device__ __forceinline__ int key_end(int i, int lq, int lk, int causal, int window) {
    if (!causal && !window) return lk;
    const int e = i + lk - lq + (causal ? 1 : window);
    return e < 0 ? 0 : (e > lk ? lk : e);
}
__device__ __forceinline__ int key_begin(int i, int lq, int lk, int window) {
    if (!window) return 0;
    const int b = i + lk - lq - window + 1;
    return b < 0 ? 0 : (b > lk ? lk : b);
}

struct BiasArgs {
    const float *table;
    int kind, lo, hi, width;
};

// Raw bias windows.  A tile's window in LDS holds, for every relative
// position (or key) the tile can touch, the already-clamped table value, so a
// lookup is a per-lane base plus a compile-time offset (no per-element index
// arithmetic):
//  * row-major tiles (a lane owns a query row, its elements run over keys:
//    forward and dQ units), rows [i0, i0 + ni), keys [j0, j0 + nj):
//    REL    entry p = table[clamp(i0 + ni - 1 - j0 - p)]; (i, j) reads (i0 + ni - 1 - i) + (j - j0)
//    KEYPOS entry p = table[clamp(j0 + p)];            (i, j) reads j - j0
//  * key-major tiles (a lane owns a key, its elements run over query rows:
//    dK/dV units):
//    REL    entry p = table[clamp(i0 - (j0 + nj - 1) + p)]; (i, j) reads (j0 + nj - 1 - j) + (i - i0)
//    KEYPOS entry p = table[clamp(j0 + p)];                   (i, j) reads j - j0
// The table offset (from bias_lo) thread t stages, or -1 for no entry.
__device__ __forceinline__ int bias_stage_rowmajor(const BiasArgs &bz, int i0, int ni, int j0, int nj, int t) {
    if (bz.kind == BIAS_REL) return t < ni + nj - 1 ? clampi(i0 + ni - 1 - j0 - t, bz.lo, bz.hi) - bz.lo : -1;
    if (bz.kind == BIAS_KEYPOS) return t < nj ? clampi(j0 + t, bz.lo, bz.hi) - bz.lo : -1;
    return -1;
}
__device__ __forceinline__ int bias_stage_keymajor(const BiasArgs &bz, int i0, int ni, int j0, int nj, int t) {
    if (bz.kind == BIAS_REL) return t < ni + nj - 1 ? clampi(i0 - (j0 + nj - 1) + t, bz.lo, bz.hi) - bz.lo : -1;
    if (bz.kind == BIAS_KEYPOS) return t < nj ? clampi(j0 + t, bz.lo, bz.hi) - bz.lo : -1;
    return -1;
}

__device__ __forceinline__ float bias_at(const BiasArgs &bz, const float *row, int i, int j) {
    if (bz.kind == BIAS_REL) return row[clampi(i - j, bz.lo, bz.hi) - bz.lo];
    if (bz.kind == BIAS_KEYPOS) return row[clampi(j, bz.lo, bz.hi) - bz.lo];
    return 0.0f;
}

}  // namespace ja
