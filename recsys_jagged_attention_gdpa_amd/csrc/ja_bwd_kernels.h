// Backward kernels (bf16 in, fp32 accumulate) for GDPA and JFA on gfx950.
//
// With dP = dO V^T and X the scores:
//   GDPA  dX = dP * act'(X),        P = act(X)
//   JFA   dX = P * (dP - delta),    P = exp(X - LSE), delta_i = <dO_i, O_i>
//   dV = P^T dO,  dK = scale dX^T Q,  dQ = scale dX K.
//
// The pages' backward avoids both redundant recomputation and atomic writes
// by splitting the dQ computation off in a non-sequence-parallel scheme
// ("Meta redesigns AI training infrastructure...", section "Eliminating
// Compute Waste in Asymmetric Workloads").  Here every output row is written
// exactly once, by one unit, with no atomics:
//   * dK/dV units (sample, 128-key tile, head): each wave owns 32 keys and
//     loops over the query rows that see them; dK, dV accumulate in registers.
//   * dQ units (sample, 128-query tile, head): each wave owns 32 query rows and
//     loops over the key tiles they see; dQ accumulates in registers.
//     These two unit kinds recompute X and dP once each.
//   * Fused units for samples with at most 32 keys, (sample, head): the keys
//     stay resident and the unit loops over all query rows; dQ of each block
//     is complete when the block is done, dK and dV when the sample is done,
//     so nothing is recomputed.  This is the short key/value regime, where
//     the pages pipeline across the outer loop because the inner loop has
//     only one or two iterations ("Meta redesigns...", section "Custom Kernels
//     and 5D Parallelism...").
// With a rotary embedding the units read turned q and k, so dQ and dK come out
// as gradients of the turned rows.  The dQ and fused units turn their dQ rows
// back (the turn's transpose) in registers before the store.  dK is turned back
// by a streaming pass instead: the dK/dV kernel runs one wave per SIMD at the
// edge of its register budget, and any epilogue added to it changes how the
// compiler schedules its main loop (measured: 8 % slower, more than the pass).
#pragma once

#include "ja_dbias_fold.h"
#include "ja_device.h"
#include "ja_kernels.h"
#include "ja_tiles.h"

namespace ja {

constexpr int BWD_THREADS = 256;

// --------------------------------------------------------------- JFA delta
// delta[h][r] = <dO[r, h, :], O[r, h, :]> (fp32 [H, Tq]), O taken as o + o_res when
// the forward's rounding residual is given.  D/8 lanes per row,
// one 16-byte chunk each, reduced by lane shuffles.
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const AttnParams p) {
    constexpr int TPR = D / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t rowh = gid / TPR;  // r * H + h
    const int c = (int)(gid % TPR);
    const int64_t n = p.total_q * p.H;
    float acc = 0.0f;
    if (rowh < n) {
        // O and its residual are read only here: nontemporal
        const bf16x8 o = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(static_cast<const bf16 *>(p.o) + rowh * D + c * 8));
        const bf16x8 d = *reinterpret_cast<const bf16x8 *>(static_cast<const bf16 *>(p.dout) + rowh * D + c * 8);
        if (p.o_res) {
            // O = bf16 output + its rounding residual: delta exact to fp32 rounding
            const bf16x8 r = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(static_cast<const bf16 *>(p.o_res) + rowh * D + c * 8));
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(bf2f(o[e]) + bf2f(r[e]), bf2f(d[e]), acc);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(bf2f(o[e]), bf2f(d[e]), acc);
        }
    }
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (rowh < n && c == 0) {
        const int64_t r = rowh / p.H;
        const int h = (int)(rowh % p.H);
        p.delta[(int64_t)h * p.total_q + r] = acc;
    }
}

// Element-wise backward of one score: returns P (the weight used for dV)
// and writes dX (without the scale factor).
template <int MODE, int ACT>
__device__ __forceinline__ float score_bwd(float s_raw, float scale, float bias, float dp, float lse2, float dlt,
                                           bool valid, float &dx) {
    const float x = __builtin_fmaf(s_raw, scale, bias);
    if constexpr (MODE == GDPA) {
        float y, dy;
        act_fwd_grad<ACT>(x, y, dy);
        dx = valid ? dp * dy : 0.0f;
        return valid ? y : 0.0f;
    } else {
        const float pr = valid ? fast_exp2(__builtin_fmaf(x, LOG2E, -lse2)) : 0.0f;
        dx = pr * (dp - dlt);
        return pr;
    }
}

// ------------------------------------------------------------- dQ units
// DB: also the bias-table gradient's partial sums (p.dbias_slots: one row of
// W entries per (unit, wave)), from the dX blocks the unit forms anyway.
template <int D, int MODE, int ACT, bool ROPE, bool DB>
__global__ __launch_bounds__(BWD_THREADS, 2) void dq_kernel(const AttnParams p) {
    constexpr int BN = KV_TILE;
    constexpr int BM = Q_TILE;
    constexpr int TILE_BYTES = BN * D * 2;
    constexpr int NKK = D / 16, NDB = D / 32, NNB = BN / 32;
    constexpr int WIN = BM + BN - 1;
    static_assert(WIN <= BWD_THREADS, "one bias window entry per thread");
    __shared__ __attribute__((aligned(16))) char smem[4 * TILE_BYTES];
    __shared__ float s_bias[2][WIN];
    __shared__ float s_fold[DB ? BWD_THREADS / WAVE : 1][DB ? DBF_FLOATS : 1];
    __shared__ int s_unit;
    lchar *const lbase = (lchar *)smem;

    const int H = p.H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int n_units = p.counters->units;
    if (n_units == 0) return;
    const BiasArgs bz{p.bias, p.bias_kind, p.bias_lo, p.bias_hi, p.bias_hi - p.bias_lo + 1};
    DbiasFold fold;
    if constexpr (DB) fold.init(s_fold[wv], bz.kind, bz.lo, bz.hi, lane);

    const uint64_t busy_t0 = busy_start(p.busy);
    const int xcd = xcd_id();
    int slices_done = 0;
    for (;;) {
        if (tid == 0) s_unit = next_tile_unit(p.counters, n_units, xcd, slices_done);
        __syncthreads();
        const int w = s_unit;
        __syncthreads();
        if (w < 0) break;
        const UnitRef u = tile_unit(p.tiles, w, n_units, H);
        const int2 tile = u.tile;
        const int h = u.h;
        const Sample s = load_sample(p.q_off, p.lq_fixed, p.kv_off, tile.x);
        const int i0 = tile.y * BM;
        const int iw = i0 + wv * 32;
        const int irow = iw + l32;
        const bool row_ok = irow < s.lq;
        const int i_last = (i0 + BM < s.lq ? i0 + BM : s.lq) - 1;
        const int nkv = (key_end(i_last, s.lq, s.lk, p.causal, p.window) + BN - 1) / BN;
        const int jt_first = key_begin(i0, s.lq, s.lk, p.window) / BN;  // tiles before it see no row of the unit
        const HeadSlice<D> Qs(p.q, s.qs, s.lq, H, h), Gs(p.dout, s.qs, s.lq, H, h), dQs(p.dq, s.qs, s.lq, H, h);
        const HeadSlice<D> Ks(p.k, s.ks, s.lk, H, h), Vs(p.v, s.ks, s.lk, H, h);
        const rsrc_t brs = make_rsrc(bz.kind ? bz.table + (int64_t)h * bz.width : nullptr,
                                     bz.kind ? (uint32_t)bz.width * 4u : 0u);

        bf16x8 qreg[NKK], greg[NKK];
        load_row_operand<D>(qreg, Qs, irow, g);
        load_row_operand<D>(greg, Gs, irow, g);
        float lse2 = 0.0f, dlt = 0.0f;
        if constexpr (MODE == JFA) {
            const uint32_t off = (uint32_t)irow * 4u;  // rows past the sample read zeros
            const rsrc_t lr = make_rsrc(p.lse + (int64_t)h * p.total_q + s.qs, (uint32_t)s.lq * 4u);
            const rsrc_t dr = make_rsrc(p.delta + (int64_t)h * p.total_q + s.qs, (uint32_t)s.lq * 4u);
            lse2 = buf_load_f32(lr, off) * LOG2E;
            dlt = buf_load_f32(dr, off);
        }
        const int my_kend = key_end(irow, s.lq, s.lk, p.causal, p.window);
        const int my_kbeg = key_begin(irow, s.lq, s.lk, p.window);
        // keys every row of the wave sees: [wkb, wke)
        const int wke = key_end(iw, s.lq, s.lk, p.causal, p.window);
        const int wkb = key_begin(iw + 31, s.lq, s.lk, p.window);

        f32x16 dqacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16{};
        if constexpr (DB) fold.begin(p.dbias_slots, (int64_t)w * (BWD_THREADS / WAVE) + wv);

        // Key / value tile jt is copied straight into LDS buffer (jt & 1); the
        // bias window (JFA: in log2 units) goes through a register.
        float bnext = 0.0f;
        auto load_tile = [&](int jt) {
            lchar *kt = lbase + (jt & 1) * 2 * TILE_BYTES;
            dma_tile<BN, D, BWD_THREADS>(kt, Ks, jt * BN, tid);
            dma_tile<BN, D, BWD_THREADS>(kt + TILE_BYTES, Vs, jt * BN, tid);
            const int bi = bias_stage_rowmajor(bz, i0, BM, jt * BN, BN, tid);
            bnext = buf_load_f32(brs, bi >= 0 ? (uint32_t)bi * 4u : OOB);
        };
        auto store_tile = [&](int buf) {
            if (tid < WIN) s_bias[buf][tid] = MODE == JFA ? bnext * LOG2E : bnext;
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's part of the tile has landed
        };
        load_tile(jt_first);
        store_tile(jt_first & 1);
        __syncthreads();
        const float sl = MODE == JFA ? p.scale * LOG2E : p.scale;
        const float nl = -lse2;

        for (int jt = jt_first; jt < nkv; ++jt) {
            const int j0 = jt * BN;
            const lchar *Kt = lbase + (jt & 1) * 2 * TILE_BYTES;
            const lchar *Vt = Kt + TILE_BYTES;
            const float *bwin = s_bias[jt & 1];
            load_tile(jt + 1);  // past the last tile: zeros, no traffic
            __builtin_amdgcn_sched_barrier(0);

            // Wave-uniform: does this tile cross the key end, the diagonal, the
            // window start or the query end?
            const bool masked = (j0 + BN > wke) | (j0 < wkb) | (iw + 32 > s.lq);
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb) {
                f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const int off = lds_off<D>(nb * 32 + l32, 2 * kk + g);
                    sacc = mfma32(lds_read16(Kt, off), qreg[kk], sacc);
                    dpacc = mfma32(lds_read16(Vt, off), greg[kk], dpacc);
                }
                // JFA: the exponent x + bias - LSE (log2 units); without a bias the
                // scale and -LSE fold into one FMA
                if (bz.kind) {
                    // raw window: entry (i0 + BM - 1 - irow) + (j - j0) (REL) or j - j0 (KEYPOS)
                    const int bbase = (bz.kind == BIAS_REL ? BM - 1 - wv * 32 - l32 : 0) + g * 4 + nb * 32;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        sacc[e] = __builtin_fmaf(sacc[e], sl, bwin[bbase + (e >> 2) * 8 + (e & 3)]);
                        if constexpr (MODE == JFA) sacc[e] += nl;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 16; ++e) sacc[e] = MODE == JFA ? __builtin_fmaf(sacc[e], sl, nl) : sacc[e] * sl;
                }
                float dx[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    if constexpr (MODE == JFA) {
                        dx[e] = fast_exp2(sacc[e]) * (dpacc[e] - dlt);
                    } else {
                        float y, dy;
                        act_fwd_grad<ACT>(sacc[e], y, dy);
                        dx[e] = dpacc[e] * dy;
                    }
                }
                if (masked) {
                    // invalid pairs (and rows without a visible key, LSE = -inf) give nothing
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int j = j0 + nb * 32 + crow(e, g);
                        dx[e] = (row_ok & (j < my_kend) & (j >= my_kbeg)) ? dx[e] : 0.0f;
                    }
                }
                if constexpr (DB) fold.block(dx, iw, j0 + nb * 32, lane);
                bf16x8 dsb[2];
                pack_operands(dx, dsb[0], dsb[1]);
                // dQ^T += K^T dX^T over this block's 32 keys
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        dqacc[db] = mfma32(lds_read_tr_operand<D>(Kt, nb * 32 + hf * 16, db * 32, lane), dsb[hf], dqacc[db]);
            }
            store_tile((jt + 1) & 1);
            __syncthreads();
        }
        if constexpr (DB) fold.finish(iw, jt_first * BN, (nkv > jt_first ? nkv : jt_first) * BN, lane);
        if constexpr (ROPE) rope_back_acc<D>(dqacc, irow, p.rope_rev, g);
        store_row_acc<D>(dQs, irow, dqacc, p.scale, g);
    }
    busy_end(p.busy, p.busy_cap, busy_t0);
}

// ----------------------------------------------------------- dK/dV units
template <int D, int MODE, int ACT>
__global__ __launch_bounds__(BWD_THREADS, 1) void dkdv_kernel(const AttnParams p) {
    constexpr int BQ = BWD_Q_STEP;  // query rows per step
    constexpr int BK = BWD_KV_UNIT; // 128 keys per unit
    constexpr int TILE_BYTES = BQ * D * 2;
    constexpr int NKK = D / 16, NDB = D / 32;
    constexpr int WIN = BQ + BK - 1;
    static_assert(WIN <= BWD_THREADS, "one bias window entry per thread");
    __shared__ __attribute__((aligned(16))) char smem[4 * TILE_BYTES];
    __shared__ __attribute__((aligned(16))) float s_lse[2][BQ];
    __shared__ __attribute__((aligned(16))) float s_dlt[2][BQ];
    __shared__ float s_bias[2][WIN];
    __shared__ int s_unit;
    lchar *const lbase = (lchar *)smem;

    const int H = p.H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int n_units = p.counters2->units;
    if (n_units == 0) return;
    const BiasArgs bz{p.bias, p.bias_kind, p.bias_lo, p.bias_hi, p.bias_hi - p.bias_lo + 1};

    const uint64_t busy_t0 = busy_start(p.busy);
    const int xcd = xcd_id();
    int slices_done = 0;
    for (;;) {
        if (tid == 0) s_unit = next_tile_unit(p.counters2, n_units, xcd, slices_done);
        __syncthreads();
        const int w = s_unit;
        __syncthreads();
        if (w < 0) break;
        const UnitRef u = tile_unit(p.tiles2, w, n_units, H);
        const int2 tile = u.tile;
        const int h = u.h;
        const Sample s = load_sample(p.q_off, p.lq_fixed, p.kv_off, tile.x);
        const int jt0 = tile.y * BK;
        const int jw = jt0 + wv * 32;       // first key of this wave
        const int jkey = jw + l32;          // this lane's key (C-layout column)
        const HeadSlice<D> Qs(p.q, s.qs, s.lq, H, h), Gs(p.dout, s.qs, s.lq, H, h);
        const HeadSlice<D> Ks(p.k, s.ks, s.lk, H, h), Vs(p.v, s.ks, s.lk, H, h);
        const rsrc_t brs = make_rsrc(bz.kind ? bz.table + (int64_t)h * bz.width : nullptr,
                                     bz.kind ? (uint32_t)bz.width * 4u : 0u);
        const rsrc_t lr = make_rsrc(MODE == JFA ? p.lse + (int64_t)h * p.total_q + s.qs : nullptr,
                                    MODE == JFA ? (uint32_t)s.lq * 4u : 0u);
        const rsrc_t dr = make_rsrc(MODE == JFA ? p.delta + (int64_t)h * p.total_q + s.qs : nullptr,
                                    MODE == JFA ? (uint32_t)s.lq * 4u : 0u);

        bf16x8 kreg[NKK], vreg[NKK];
        load_row_operand<D>(kreg, Ks, jkey, g);
        load_row_operand<D>(vreg, Vs, jkey, g);
        f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) dkacc[db] = dvacc[db] = f32x16{};

        // Query rows that see any key of the unit, [ia0, ia_end): with ia = i + lk - lq
        // the aligned position, causal masking needs ia >= jt0, a window w needs
        // ia < jt0 + BK - 1 + w and (without causal masking) ia > jt0 - w.
        const int shift = s.lk - s.lq;  // causal: key j visible to row i iff j <= i + shift
        const int win = p.window;
        int ia0 = p.causal ? jt0 - shift : (win ? jt0 - win - shift + 1 : 0);
        ia0 = ia0 < 0 ? 0 : ia0;
        int ia_end = win ? jt0 + BK - 1 + win - shift : s.lq;
        ia_end = ia_end > s.lq ? s.lq : ia_end;
        const int nsteps = ia0 < ia_end ? (ia_end - ia0 + BQ - 1) / BQ : 0;

        // Query / dO rows of step st are copied straight into LDS buffer
        // (st & 1); the step's LSE, delta and bias window go through registers.
        // JFA stores -LSE and the bias in log2 units, so P = exp2(fma(s, sl2, b - lse2)).
        float bnext = 0.0f, lnext = 0.0f, dnext = 0.0f;
        auto load_step = [&](int st) {
            const int ia = ia0 + st * BQ;
            lchar *qt = lbase + (st & 1) * 2 * TILE_BYTES;
            dma_tile<BQ, D, BWD_THREADS>(qt, Qs, ia, tid);
            dma_tile<BQ, D, BWD_THREADS>(qt + TILE_BYTES, Gs, ia, tid);
            const int bi = bias_stage_keymajor(bz, ia, BQ, jt0, BK, tid);
            bnext = buf_load_f32(brs, bi >= 0 ? (uint32_t)bi * 4u : OOB);
            if constexpr (MODE == JFA) {
                const uint32_t off = tid < BQ ? (uint32_t)(ia + tid) * 4u : OOB;
                lnext = buf_load_f32(lr, off);
                dnext = buf_load_f32(dr, off);
            }
        };
        auto store_step = [&](int buf) {
            if (tid < WIN) s_bias[buf][tid] = MODE == JFA ? bnext * LOG2E : bnext;
            if (MODE == JFA && tid < BQ) {
                s_lse[buf][tid] = -lnext * LOG2E;
                s_dlt[buf][tid] = dnext;
            }
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's part of the tiles has landed
        };
        load_step(0);
        store_step(0);
        __syncthreads();
        const float sl = MODE == JFA ? p.scale * LOG2E : p.scale;

        for (int st = 0; st < nsteps; ++st) {
            const int ia = ia0 + st * BQ;
            const lchar *Qt = lbase + (st & 1) * 2 * TILE_BYTES;
            const lchar *Gt = Qt + TILE_BYTES;
            const float *bwin = s_bias[st & 1];
            load_step(st + 1);  // past the last step: zeros, no traffic
            __builtin_amdgcn_sched_barrier(0);

            // Wave-uniform: does this step cross the query end or the diagonal?
            const bool masked = (ia + BQ > s.lq) | (p.causal && (jw + 31 > ia + shift)) |
                                (win && ((jw < key_begin(ia + BQ - 1, s.lq, s.lk, win)) |
                                         (jw + 32 > key_end(ia, s.lq, s.lk, p.causal, win))));
            // Software pipeline over the step's 32-row blocks: the next block's S
            // and dP products are issued inside the current block's element-wise
            // stage (one basic block), so the scheduler can interleave the matrix
            // and vector work of this single wave per SIMD.
            f32x16 sa = f32x16{}, da = f32x16{};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const int off = lds_off<D>(l32, 2 * kk + g);
                sa = mfma32(lds_read16(Qt, off), kreg[kk], sa);
                da = mfma32(lds_read16(Gt, off), vreg[kk], da);
            }
#pragma unroll
            for (int qb = 0; qb < BQ / 32; ++qb) {
                // x = s * sl + bias; invalid pairs are zeroed after the element-wise
                // stage (rows without any visible key have LSE = -inf, so their
                // exponent is not finite and must not be used).
                if (bz.kind == BIAS_REL) {
                    // raw window: entry (jt0 + BK - 1 - jkey) + (i - ia)
                    const int bbase = BK - 1 - wv * 32 - l32 + g * 4 + qb * 32;
#pragma unroll
                    for (int e = 0; e < 16; ++e) sa[e] = __builtin_fmaf(sa[e], sl, bwin[bbase + (e >> 2) * 8 + (e & 3)]);
                } else if (bz.kind == BIAS_KEYPOS) {
                    const float b = bwin[wv * 32 + l32];  // entry jkey - jt0, the same for every row
#pragma unroll
                    for (int e = 0; e < 16; ++e) sa[e] = __builtin_fmaf(sa[e], sl, b);
                } else if constexpr (MODE == GDPA) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) sa[e] *= sl;
                }
                f32x16 sn = f32x16{}, dn = f32x16{};
                if (qb + 1 < BQ / 32) {
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) {
                        const int off = lds_off<D>((qb + 1) * 32 + l32, 2 * kk + g);
                        sn = mfma32(lds_read16(Qt, off), kreg[kk], sn);
                        dn = mfma32(lds_read16(Gt, off), vreg[kk], dn);
                    }
                }
                float pv[16], dx[16];
                if constexpr (MODE == JFA) {
                    // with a bias S already holds x; without one the scale folds into the FMA
                    const float xm = bz.kind ? 1.0f : sl;
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int il = qb * 32 + r4 * 8 + g * 4;  // rows crow(4 r4 .. 4 r4 + 3, g)
                        const f32x4 nl = *reinterpret_cast<const __attribute__((address_space(3))) f32x4 *>(
                            (const lchar *)&s_lse[st & 1][il]);
                        const f32x4 dl = *reinterpret_cast<const __attribute__((address_space(3))) f32x4 *>(
                            (const lchar *)&s_dlt[st & 1][il]);
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const int e = r4 * 4 + t;
                            pv[e] = fast_exp2(__builtin_fmaf(sa[e], xm, nl[t]));
                            dx[e] = pv[e] * (da[e] - dl[t]);
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        float dy;
                        act_fwd_grad<ACT>(sa[e], pv[e], dy);
                        dx[e] = da[e] * dy;
                    }
                }
                if (masked) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int i = ia + qb * 32 + crow(e, g);
                        const int dist = i + shift - jkey;  // aligned distance
                        const bool valid = (i < s.lq) & (!p.causal | (dist >= 0)) &
                                           (!win | ((dist < win) & (p.causal | (-dist < win))));
                        pv[e] = valid ? pv[e] : 0.0f;
                        dx[e] = valid ? dx[e] : 0.0f;
                    }
                }
                bf16x8 pb[2], dsb[2];
                pack_operands(pv, pb[0], pb[1]);
                pack_operands(dx, dsb[0], dsb[1]);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        dvacc[db] = mfma32(lds_read_tr_operand<D>(Gt, qb * 32 + ks * 16, db * 32, lane), pb[ks], dvacc[db]);
                        dkacc[db] = mfma32(lds_read_tr_operand<D>(Qt, qb * 32 + ks * 16, db * 32, lane), dsb[ks], dkacc[db]);
                    }
                }
                sa = sn;
                da = dn;
            }
            store_step((st + 1) & 1);
            __syncthreads();
        }
        const HeadSlice<D> dKs(p.dk, s.ks, s.lk, H, h), dVs(p.dv, s.ks, s.lk, H, h);
        store_row_acc<D>(dKs, jkey, dkacc, p.scale, g);
        store_row_acc<D>(dVs, jkey, dvacc, 1.0f, g);
    }
    busy_end(p.busy, p.busy_cap, busy_t0);
}

// ------------------------------------------------- fused short-K/V units
// One unit per (sample, head) with at most 32 keys, run by ONE wave (the
// workgroup is a single wave): the wave keeps K and V as MFMA operands in
// registers, streams the sample's query rows in 32-row blocks, loading the
// next block's Q and dO rows into registers while the current block is
// computed (outer-loop pipelining: the inner loop over keys has one step),
// and owns dK and dV for the whole sample, so no barrier and no cross-wave
// reduction is needed.  A block computes X and dP once, dV and dK into
// registers, dX^T through a small LDS transpose, and the block's complete dQ.
// Memory accesses go through per-sample buffer descriptors (no branches
// around them), so the next block's loads stay in flight.
template <int D, int MODE, int ACT, bool ROPE>
__global__ __launch_bounds__(WAVE, 1) void fused_kernel(const AttnParams p) {
    constexpr int NKK = D / 16, NDB = D / 32;
    constexpr int TILE = 32 * D * 2;           // one 32-row tile
    constexpr int DS_STRIDE = 80;              // bytes per row of the dX scratch (32 bf16 + pad)
    constexpr int DS_BYTES = 32 * DS_STRIDE;
    __shared__ __attribute__((aligned(16))) char smem[4 * TILE + DS_BYTES];
    lchar *const Qt = (lchar *)smem;   // this block's Q rows
    lchar *const Gt = Qt + TILE;       // this block's dO rows
    lchar *const Kt = Gt + TILE;       // the sample's keys (resident for the unit)
    lchar *const Vt = Kt + TILE;       // the sample's values
    lchar *const Sx = Vt + TILE;       // dX transpose scratch

    const int H = p.H;
    const int lane = threadIdx.x;
    const int g = lane >> 5, l32 = lane & 31;
    const int n_units = p.counters3->units;
    if (n_units == 0) return;
    const BiasArgs bz{p.bias, p.bias_kind, p.bias_lo, p.bias_hi, p.bias_hi - p.bias_lo + 1};

    const uint64_t busy_t0 = busy_start(p.busy);
    for (;;) {
        int w = 0;
        if (lane == 0) w = atomicAdd(&p.counters3->cursor, 1);
        w = __builtin_amdgcn_readfirstlane(w);
        if (w >= n_units) break;
        const int2 tile = p.tiles3[w / H];
        const int h = w % H;
        const Sample s = load_sample(p.q_off, p.lq_fixed, p.kv_off, tile.x);
        const int jkey = l32;
        const bool key_ok = jkey < s.lk;
        const float *brow = bz.kind ? bz.table + (int64_t)h * bz.width : nullptr;
        const int shift = s.lk - s.lq;
        const int nblk = (s.lq + 31) / 32;
        const HeadSlice<D> Qs(p.q, s.qs, s.lq, H, h), Gs(p.dout, s.qs, s.lq, H, h), dQs(p.dq, s.qs, s.lq, H, h);
        const HeadSlice<D> Ks(p.k, s.ks, s.lk, H, h), Vs(p.v, s.ks, s.lk, H, h);
        const rsrc_t lse_r = make_rsrc(p.lse ? p.lse + (int64_t)h * p.total_q + s.qs : nullptr,
                                       MODE == JFA ? (uint32_t)s.lq * 4u : 0u);
        const rsrc_t dlt_r = make_rsrc(p.delta ? p.delta + (int64_t)h * p.total_q + s.qs : nullptr,
                                       MODE == JFA ? (uint32_t)s.lq * 4u : 0u);

        // Keys and values of the sample (rows past lk read as zeros) and the
        // first query block; all waited for before the block loop, so that the
        // waits the compiler derives inside the loop reflect only the loop's
        // own order (next block's loads, then this block's stores).
        PairSliceLoader<32, D, WAVE, CP_NT> nx;
        {
            PairSliceLoader<32, D, WAVE, CP_NT> kv;
            kv.load(Ks, Vs, 0, lane);
            nx.load(Qs, Gs, 0, lane);
            kv.store(Kt, Vt, lane);
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

        f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) dkacc[db] = dvacc[db] = f32x16{};

        for (int blk = 0; blk < nblk; ++blk) {
            const int ia = blk * 32;
            nx.store(Qt, Gt, lane);
            lds_wave_sync();
            float lse2[16], dlt[16], bv[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t off = (uint32_t)(ia + crow(e, g)) * 4u;
                lse2[e] = MODE == JFA ? buf_load_f32<CP_NT>(lse_r, off) * LOG2E : 0.0f;
                dlt[e] = MODE == JFA ? buf_load_f32<CP_NT>(dlt_r, off) : 0.0f;
                bv[e] = 0.0f;
            }
            if (brow) {
#pragma unroll
                for (int e = 0; e < 16; ++e) bv[e] = bias_at(bz, brow, ia + crow(e, g), jkey);
            }
            nx.load(Qs, Gs, ia + 32, lane);  // next block; past the sample: zeros, no traffic
            __builtin_amdgcn_sched_barrier(0);  // keep the next block's loads ahead of this block's work

            // X = Q K^T and dP = dO V^T: lane holds key jkey, query rows crow(e, g).
            f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const int off = lds_off<D>(l32, 2 * kk + g);
                sacc = mfma32(lds_read16(Qt, off), lds_read16(Kt, off), sacc);
                dpacc = mfma32(lds_read16(Gt, off), lds_read16(Vt, off), dpacc);
            }
            const bool masked = (ia + 32 > s.lq) | (s.lk < 32) | (p.causal != 0) | (p.window != 0);
            float pv[16], dx[16];
            if (!masked) {  // wave-uniform: interior blocks carry no per-element tests
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    pv[e] = score_bwd<MODE, ACT>(sacc[e], p.scale, bv[e], dpacc[e], lse2[e], dlt[e], true, dx[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int i = ia + crow(e, g);
                    const int dist = i + shift - jkey;  // aligned distance
                    const bool valid = (i < s.lq) & key_ok & (!p.causal | (dist >= 0)) &
                                       (!p.window | ((dist < p.window) & (p.causal | (-dist < p.window))));
                    pv[e] = score_bwd<MODE, ACT>(sacc[e], p.scale, bv[e], dpacc[e], lse2[e], dlt[e], valid, dx[e]);
                }
            }
            bf16x8 pb[2], dsb[2];
            pack_operands(pv, pb[0], pb[1]);
            pack_operands(dx, dsb[0], dsb[1]);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    dvacc[db] = mfma32(lds_read_tr_operand<D>(Gt, ks * 16, db * 32, lane), pb[ks], dvacc[db]);
                    dkacc[db] = mfma32(lds_read_tr_operand<D>(Qt, ks * 16, db * 32, lane), dsb[ks], dkacc[db]);
                }
            }
            // dX (query i, key j) -> scratch row i, column j; read back as dX^T operands.
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int i = crow(e, g);
                *reinterpret_cast<__attribute__((address_space(3))) bf16 *>(Sx + i * DS_STRIDE + jkey * 2) = f2bf(dx[e]);
            }
            lds_wave_sync();
            bf16x8 dtb[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const lchar *row = Sx + l32 * DS_STRIDE + (ks * 16 + g * 4) * 2;
                const u32x2 lo = *reinterpret_cast<const __attribute__((address_space(3))) u32x2 *>(row);
                const u32x2 hi = *reinterpret_cast<const __attribute__((address_space(3))) u32x2 *>(row + 16);
                dtb[ks] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
            // dQ^T = K^T dX^T, one 32-wide block of the head dimension at a time;
            // the block's Q tile is no longer read, so it stages dQ for the store.
            f32x16 dqacc[NDB];
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                dqacc[db] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    dqacc[db] = mfma32(lds_read_tr_operand<D>(Kt, ks * 16, db * 32, lane), dtb[ks], dqacc[db]);
            }
            if constexpr (ROPE) rope_back_acc<D>(dqacc, ia + l32, p.rope_rev, g);
            store_tile<D>(dQs, Qt, ia, dqacc, p.scale, lane);
            lds_wave_sync();  // every LDS read of this block is done before the next stores
        }
        const HeadSlice<D> dKs(p.dk, s.ks, s.lk, H, h), dVs(p.dv, s.ks, s.lk, H, h);
        store_tile<D>(dKs, Qt, 0, dkacc, p.scale, lane);
        store_tile<D>(dVs, Gt, 0, dvacc, 1.0f, lane);
    }
    busy_end(p.busy, p.busy_cap, busy_t0);
}

}  // namespace ja
