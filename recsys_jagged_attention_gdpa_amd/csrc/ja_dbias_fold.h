// Bias-table gradient folded into the dQ units.
//
// The bias enters the scores additively, X = scale QK^T + bias, so a table
// entry's gradient is the sum of dX over the (query, key) pairs that read it:
// REL entries collect the diagonals i - j of dX, KEYPOS entries its columns j,
// positions clamped into [lo, hi].  The dQ units already hold every dX block
// of their rows in registers (fp32, before it is rounded for the dQ product),
// so they add these sums as a by-product instead of a separate pass
// recomputing S and dP.
//
// Layout of a dX block in a dQ unit: the wave's 32 query rows are its lanes'
// columns (row i = iw + lane % 32) and the 16 values of a lane are 16 of the
// block's 32 keys (key jb + crow(e, lane / 32)).  Per block:
//   * a block whose positions all clamp to one end entry (the common case far
//     from the diagonal on long samples) only adds into a per-lane register;
//   * otherwise the block goes through LDS in four chunks of 8 keys, and each
//     lane sums one line of it: REL lane d < 63 the diagonal r - c = d - 31,
//     KEYPOS lane c < 32 (after a reduction over row groups) the column c.
// REL diagonals span two consecutive blocks, so a register window (lane d:
// position iw - jb + d - 31) carries the partial sums: after each block its
// upper 32 lanes are complete and leave, the lower ones move up by 32.
//
// Order and ownership: every (unit, wave) writes its own row of W partial sums
// in the workspace (each entry exactly once, untouched entries as zeros), so
// which workgroup ran a unit does not matter; a reduction adds the rows in unit
// order.  The sums are therefore deterministic with dynamically scheduled units.
#pragma once

#include "ja_device.h"

namespace ja {

// A wave's staging area: one 32-row x 8-key chunk of a dX block, 9 floats per
// row (8 keys, 1 pad: lanes reading down a diagonal hit distinct banks), with
// 7 zero rows above and 7 below, so that a diagonal read that runs off the
// chunk reads zeros instead of needing a per-read bound.
constexpr int DBF_PAD = 7;
constexpr int DBF_STRIDE = 9;
constexpr int DBF_ROWS = 32 + 2 * DBF_PAD;
constexpr int DBF_FLOATS = DBF_ROWS * DBF_STRIDE;

// Sum of v over the 64 lanes, the same butterfly order on every call.
__device__ __forceinline__ float wave_sum_fixed(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ float sum16(const float (&v)[16]) {
    float s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = v[2 * i] + v[2 * i + 1];
    return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

struct DbiasFold {
    float *scr;    // this wave's staging area (LDS, DBF_FLOATS floats)
    rsrc_t slot;   // this (unit, wave)'s row of W partial sums
    int lo, hi, W;
    bool rel;      // REL (diagonals) or KEYPOS (columns)
    float win;     // REL window: lane d holds position iw - jb + d - 31 of the current block jb
    float acc_lo, acc_hi;  // this lane's dX that clamps to the first / last entry

    // Once per workgroup: the pad rows are zero for good (chunks only ever
    // write the 32 middle rows).
    __device__ __forceinline__ void init(float *area, int kind, int lo_, int hi_, int lane) {
        scr = area;
        rel = kind == BIAS_REL;
        lo = lo_;
        hi = hi_;
        W = hi_ - lo_ + 1;
        for (int i = lane; i < DBF_FLOATS; i += 64) scr[i] = 0.0f;
    }
    __device__ __forceinline__ void begin(float *slots, int64_t slot_index) {
        slot = make_rsrc(slots + slot_index * W, (uint32_t)W * 4u);
        win = 0.0f;
        acc_lo = 0.0f;
        acc_hi = 0.0f;
    }
    // Position pos's complete sum v (on lanes where `done`): the end entries
    // collect in registers, interior entries are stored.
    __device__ __forceinline__ void put(bool done, int pos, float v) {
        const bool l = pos <= lo, h = pos >= hi;
        acc_lo += (done & l) ? v : 0.0f;
        acc_hi += (done & !l & h) ? v : 0.0f;
        buf_store_f32(slot, (done & !l & !h) ? (uint32_t)(pos - lo) * 4u : OOB, v);
    }

    // dX block of the wave's rows iw .. iw + 31 and keys jb .. jb + 31
    // (sample-local), layout as above; invalid pairs hold zeros.  `lane` is
    // taken through an empty asm statement so that the lane-dependent staging
    // addresses are formed per block instead of being held in registers across
    // the key loop (the dQ units have none to spare).
    __device__ __forceinline__ void block(const float (&dx)[16], int iw, int jb, int lane_) {
        const int pmin = rel ? iw - jb - 31 : jb, pmax = rel ? iw - jb + 31 : jb + 31;
        if (pmax <= lo) {  // wave-uniform; the window's lanes lie below the block's top
            acc_lo += sum16(dx) + win;
            win = 0.0f;
            return;
        }
        if (pmin >= hi) {
            acc_hi += sum16(dx) + win;
            win = 0.0f;
            return;
        }
        int lane = lane_;
        asm volatile("" : "+v"(lane));
        const int l32 = lane & 31, g = lane >> 5;
        float *wr = scr + (l32 + DBF_PAD) * DBF_STRIDE + 4 * g;
        if (rel) {
            float t = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int i = 0; i < 4; ++i) wr[i] = dx[4 * q + i];
                // lane d reads diagonal d - 31 of chunk q: key 8q + c of row
                // d - 31 + 8q + c, i.e. staging row base + c, column c
                const int base = lane - 24 + 8 * q;
                const float *rd = scr + clampi(base, 0, 38) * DBF_STRIDE;
                float v[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) v[c] = rd[c * (DBF_STRIDE + 1)];
                const float s = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
                t += (base >= 0 && base <= 38) ? s : 0.0f;  // lanes off the chunk's diagonals
            }
            win += t;
            // lanes 31..62 are complete (the next block starts 32 keys on)
            put(lane >= 31 && lane < 63, iw - jb + lane - 31, win);
            // lanes 0..30 move to 32..62 for the next block; lane 31 (done) would land on 63
            float up = 0.0f, rest = lane == 31 ? 0.0f : win;
            pair_swap(up, rest);  // up: lanes 32..63 <- lanes 0..31 of rest, lanes 0..31 zero
            win = up;
        } else {
            float cs[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int i = 0; i < 4; ++i) wr[i] = dx[4 * q + i];
                // lane L: column L % 8 of chunk q over rows 4 (L / 8) .. + 3
                const float *rd = scr + (4 * (lane >> 3) + DBF_PAD) * DBF_STRIDE + (lane & 7);
                cs[q] = (rd[0] + rd[DBF_STRIDE]) + (rd[2 * DBF_STRIDE] + rd[3 * DBF_STRIDE]);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                cs[q] += __shfl_xor(cs[q], 8, 64);
                cs[q] += __shfl_xor(cs[q], 16, 64);
                cs[q] += __shfl_xor(cs[q], 32, 64);
            }
            const int gq = (lane >> 3) & 3;
            const float v = gq == 0 ? cs[0] : gq == 1 ? cs[1] : gq == 2 ? cs[2] : cs[3];
            put(lane < 32, jb + lane, v);  // lane c: key jb + c
        }
    }

    // End of a unit: flush the window, store the two end entries and zeros at
    // the interior entries no block reached.  jb_first / jb_end: the first key
    // block of the loop and the key after its last block.
    __device__ __forceinline__ void finish(int iw, int jb_first, int jb_end, int lane) {
        int bmin, bmax;  // interior positions stored by put() over the unit
        if (rel) {
            put(lane >= 32 && lane < 63, iw - jb_end + lane - 31, win);
            bmin = iw - jb_end + 1;
            bmax = iw - jb_first + 31;
        } else {
            bmin = jb_first;
            bmax = jb_end - 1;
        }
        const float lo_s = wave_sum_fixed(acc_lo), hi_s = wave_sum_fixed(acc_hi);
        for (int c = lane; c < W; c += 64) {
            const int pos = lo + c;
            const bool end = c == 0 || c == W - 1;
            const float v = c == 0 ? (W == 1 ? lo_s + hi_s : lo_s) : (c == W - 1 ? hi_s : 0.0f);
            if (end || pos < bmin || pos > bmax) buf_store_f32(slot, (uint32_t)c * 4u, v);
        }
    }
};

}  // namespace ja
