// Gradient of the attention bias table (bf16 in, fp32 accumulate) on gfx950.
//
// The bias enters the scores additively, X = scale QK^T + bias, so the
// gradient of a table entry is the sum of dX over the (query, key) pairs that
// read it: REL entries collect the diagonals i - j of dX, KEYPOS entries its
// columns j, clamped into [lo, hi].  The pages list custom attention biases
// among what the jagged kernels support ("GEM Training: How Meta Doubled the
// Efficiency...", section "What happened"); their gradient is not described
// there, so this is the plain derivative of that additive term.
//
// One pass over (sample, 128-query tile, head) units recomputes S = QK^T and
// dP = dO V^T per 32-key tile on the matrix cores (as the dQ units do) and
// forms dX; each wave then stages its 32 x 32 blocks of dX in LDS and sums
// them along diagonals (REL) or columns (KEYPOS) into its own row of per-entry
// sums in LDS.  Blocks whose positions all clamp to one end of the table (far
// from the diagonal, the common case on long samples) skip the staging: their
// dX only adds into a per-lane register, reduced once per unit.
//
// The result is deterministic: the grid is fixed (DBIAS_GRID workgroups),
// workgroup g takes units g, g + G, g + 2G, ... in order, and units are
// numbered head-major, so each workgroup sees every head in one contiguous
// run; when its head changes it adds its four wave rows in a fixed order and
// writes one partial row per (workgroup, head).  A second kernel adds the G
// partial rows of each head in workgroup order.  No atomics.
//
// When the dQ units fold the sums in (samples with more than FUSED_MAX_LK
// keys, whose dX the dQ units form anyway), this pass only takes the samples
// of the fused short-K/V units, and the reduction also adds the dQ units'
// partial rows: first per chunk of units (unit order within a chunk, the four
// waves of a unit in order), then the chunks in order.
#include "ja_dbias_fold.h"
#include "ja_device.h"
#include "ja_kernels.h"
#include "ja_tiles.h"

namespace ja {

constexpr int DBIAS_THREADS = 256;
constexpr int SCR_STRIDE = 33;  // floats per row of a wave's 32 x 32 staging block (odd: no bank conflicts)

// Key tiles of 32 rows keep a workgroup's LDS (tiles, staging blocks and the
// four per-wave rows of W sums, sized at launch) within half the CU's for
// tables of up to ~1,300 entries, so two workgroups share a CU.
constexpr int DBIAS_BN = 32;

template <int D, int MODE, int ACT>
__global__ __launch_bounds__(DBIAS_THREADS, 2) void dbias_kernel(const AttnParams p) {
    constexpr int BN = DBIAS_BN;
    constexpr int BM = Q_TILE;
    constexpr int TILE_BYTES = BN * D * 2;
    constexpr int NKK = D / 16, NNB = BN / 32;
    constexpr int WIN = BM + BN - 1;
    static_assert(WIN <= DBIAS_THREADS, "one bias window entry per thread");
    __shared__ __attribute__((aligned(16))) char smem[4 * TILE_BYTES];
    __shared__ float s_bias[2][WIN];
    extern __shared__ float s_bins[];  // four rows of W sums, one per wave (dynamic: 16 W bytes)
    __shared__ float s_scr[4][32 * SCR_STRIDE];
    lchar *const lbase = (lchar *)smem;

    const int H = p.H;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const BiasArgs bz{p.bias, p.bias_kind, p.bias_lo, p.bias_hi, p.bias_hi - p.bias_lo + 1};
    const int W = bz.width;
    const int n_units = p.counters4->units;
    float *bins = s_bins + wv * W;
    float *scr = s_scr[wv];
    for (int c = tid; c < 4 * W; c += DBIAS_THREADS) s_bins[c] = 0.0f;

    // Partial row (workgroup, head hh) of the output sums.
    auto part_row = [&](int hh) { return p.dbias_part + ((int64_t)blockIdx.x * H + hh) * W; };
    // Write this workgroup's sums for head hh (the four wave rows added in
    // order) and clear them; heads strictly between hh and h_next get zero rows.
    auto flush = [&](int hh, int h_next) {
        __syncthreads();
        if (hh >= 0) {
            float *row = part_row(hh);
            for (int c = tid; c < W; c += DBIAS_THREADS) {
                row[c] = ((s_bins[c] + s_bins[W + c]) + s_bins[2 * W + c]) + s_bins[3 * W + c];
                s_bins[c] = s_bins[W + c] = s_bins[2 * W + c] = s_bins[3 * W + c] = 0.0f;
            }
        }
        for (int z = hh + 1; z < h_next; ++z) {
            float *row = part_row(z);
            for (int c = tid; c < W; c += DBIAS_THREADS) row[c] = 0.0f;
        }
        __syncthreads();
    };

    const uint64_t busy_t0 = busy_start(p.busy);
    int h_cur = -1;
    for (int w = blockIdx.x; w < n_units; w += gridDim.x) {
        const UnitRef u = tile_unit(p.tiles4, w, n_units, H);
        const int2 tile = u.tile;
        const int h = u.h;
        if (h != h_cur) {
            flush(h_cur, h);
            h_cur = h;
        }
        const Sample s = load_sample(p.q_off, p.lq_fixed, p.kv_off, tile.x);
        const int i0 = tile.y * BM;
        const int iw = i0 + wv * 32;
        const int irow = iw + l32;
        const bool row_ok = irow < s.lq;
        const int i_last = (i0 + BM < s.lq ? i0 + BM : s.lq) - 1;
        const int nkv = (key_end(i_last, s.lq, s.lk, p.causal, p.window) + BN - 1) / BN;
        const int jt_first = key_begin(i0, s.lq, s.lk, p.window) / BN;  // tiles before it see no row of the unit
        const HeadSlice<D> Qs(p.q, s.qs, s.lq, H, h), Gs(p.dout, s.qs, s.lq, H, h);
        const HeadSlice<D> Ks(p.k, s.ks, s.lk, H, h), Vs(p.v, s.ks, s.lk, H, h);
        const rsrc_t brs = make_rsrc(bz.table + (int64_t)h * W, (uint32_t)W * 4u);

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
        float acc_lo = 0.0f, acc_hi = 0.0f;  // this lane's dX of blocks clamped whole to an end entry

        // Key / value tile jt is copied straight into LDS buffer (jt & 1); the
        // bias window (JFA: in log2 units) goes through a register.
        float bnext = 0.0f;
        auto load_tile = [&](int jt) {
            lchar *kt = lbase + (jt & 1) * 2 * TILE_BYTES;
            dma_tile<BN, D, DBIAS_THREADS>(kt, Ks, jt * BN, tid);
            dma_tile<BN, D, DBIAS_THREADS>(kt + TILE_BYTES, Vs, jt * BN, tid);
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
                // raw window: entry (i0 + BM - 1 - irow) + (j - j0) (REL) or j - j0 (KEYPOS)
                const int bbase = (bz.kind == BIAS_REL ? BM - 1 - wv * 32 - l32 : 0) + g * 4 + nb * 32;
                float dx[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float x = __builtin_fmaf(sacc[e], sl, bwin[bbase + (e >> 2) * 8 + (e & 3)]);
                    if constexpr (MODE == JFA) {
                        dx[e] = fast_exp2(x + nl) * (dpacc[e] - dlt);
                    } else {
                        float y, dy;
                        act_fwd_grad<ACT>(x, y, dy);
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

                const int jb = j0 + nb * 32;  // first key of the block
                // Positions the block covers (wave-uniform).  A block whose every
                // position clamps to one end entry only adds into a register.
                const int pmin = bz.kind == BIAS_REL ? iw - jb - 31 : jb;
                const int pmax = bz.kind == BIAS_REL ? iw - jb + 31 : jb + 31;
                if (pmax <= bz.lo) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc_lo += dx[e];
                    continue;
                }
                if (pmin >= bz.hi) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc_hi += dx[e];
                    continue;
                }
                // Stage the 32 x 32 block (row irow - iw = l32, key crow(e, g)) and
                // sum it along one line per lane.
#pragma unroll
                for (int e = 0; e < 16; ++e) scr[l32 * SCR_STRIDE + crow(e, g)] = dx[e];
                lds_wave_sync();
                float v = 0.0f;
                int pos;  // table position of this lane's line
                bool line = true;
                if (bz.kind == BIAS_REL) {
                    // lane d < 63 sums the diagonal r - c = d - 31 of the block
                    const int dl = lane - 31;
#pragma unroll
                    for (int r = 0; r < 32; ++r) {
                        const int c = r - dl;
                        if (c >= 0 && c < 32) v += scr[r * SCR_STRIDE + c];
                    }
                    pos = iw - jb + dl;
                    line = lane < 63;
                } else {
                    // lane c < 32 sums column c (key jb + c) over the block's rows
                    const int c = lane & 31;
#pragma unroll
                    for (int r = 0; r < 32; ++r) v += scr[r * SCR_STRIDE + c];
                    pos = jb + c;
                    line = lane < 32;
                }
                lds_wave_sync();  // the block's reads are done before the next block's writes
                v = line ? v : 0.0f;
                const int bin = clampi(pos, bz.lo, bz.hi) - bz.lo;
                // Lines of distinct positions hit distinct interior entries; the two
                // end entries collect every clamped line, summed across the wave first.
                const float lo_sum = wave_sum_fixed(line && bin == 0 ? v : 0.0f);
                const float hi_sum = wave_sum_fixed(line && bin == W - 1 && bin != 0 ? v : 0.0f);
                if (line && bin > 0 && bin < W - 1) bins[bin] += v;
                if (lane == 0) {
                    bins[0] += lo_sum;
                    if (W > 1) bins[W - 1] += hi_sum;
                }
            }
            store_tile((jt + 1) & 1);
            __syncthreads();
        }
        {
            const float lo_sum = wave_sum_fixed(acc_lo), hi_sum = wave_sum_fixed(acc_hi);
            if (lane == 0) {
                bins[0] += lo_sum;
                bins[W - 1] += hi_sum;
            }
        }
    }
    flush(h_cur, H);
    busy_end(p.busy, p.busy_cap, busy_t0);
}

// Partial rows of the dQ units (DbiasFold): chunks[ch][h][c] = sum over the
// units u of chunk ch of head h (in order) of the rows of u's four waves (in
// order), entry c.  The units of head h are h n .. h n + n - 1 (head-major
// numbering, n = units / H); chunk ch holds n ch / CH .. n (ch + 1) / CH - 1.
// Block (c-group of 64 entries, h, ch); its four waves take one wave index each.
__global__ __launch_bounds__(256) void dbias_slots_kernel(const float *slots, float *chunks,
                                                          const PlanCounters *ctr, int H, int W) {
    constexpr int WV = 4;  // waves per dQ unit
    const int c = blockIdx.x * 64 + (threadIdx.x & 63), wv = threadIdx.x >> 6;
    const int h = blockIdx.y, ch = blockIdx.z;
    const int n = ctr->units / H;
    const int u0 = (int)((int64_t)n * ch / DBIAS_SLOT_CHUNKS), u1 = (int)((int64_t)n * (ch + 1) / DBIAS_SLOT_CHUNKS);
    float s = 0.0f;
    if (c < W)
        for (int u = u0; u < u1; ++u) s += slots[(((int64_t)h * n + u) * WV + wv) * W + c];
    __shared__ float red[WV][64];
    red[wv][threadIdx.x & 63] = s;
    __syncthreads();
    if (wv == 0 && c < W) {
        const int l = threadIdx.x;
        chunks[((int64_t)ch * H + h) * W + c] = ((red[0][l] + red[1][l]) + red[2][l]) + red[3][l];
    }
}

// dbias[h][c] = sum over workgroups g (in order) of partial row (g, h), entry c,
// plus (when the dQ units fold the sums in) the chunk sums in chunk order.
__global__ __launch_bounds__(256) void dbias_reduce_kernel(const float *part, const float *chunks, float *out,
                                                           int H, int W, int G) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)H * W) return;
    const int h = (int)(idx / W), c = (int)(idx % W);
    float s = 0.0f;
    for (int gi = 0; gi < G; ++gi) s += part[((int64_t)gi * H + h) * W + c];
    if (chunks) {
        float f = 0.0f;
        for (int ch = 0; ch < DBIAS_SLOT_CHUNKS; ++ch) f += chunks[((int64_t)ch * H + h) * W + c];
        s += f;
    }
    out[idx] = s;
}

template <int D, int MODE, int ACT>
static hipError_t launch_dbias_t(const AttnParams &p, hipStream_t st) {
    const int W = p.bias_hi - p.bias_lo + 1;
    const int64_t n = (int64_t)p.H * W;
    const KernelTimer &t = kernel_timer();
    t.begin(K_BWD_DBIAS, st);
    hipLaunchKernelGGL((dbias_kernel<D, MODE, ACT>), dim3(DBIAS_GRID), dim3(DBIAS_THREADS),
                       (size_t)4 * W * sizeof(float), st, t.with_busy(p, K_BWD_DBIAS));
    if (p.dbias_slots)
        hipLaunchKernelGGL(dbias_slots_kernel, dim3((unsigned)((W + 63) / 64), (unsigned)p.H, DBIAS_SLOT_CHUNKS),
                           dim3(256), 0, st, (const float *)p.dbias_slots, p.dbias_chunks,
                           (const PlanCounters *)p.counters, p.H, W);
    hipLaunchKernelGGL(dbias_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       (const float *)p.dbias_part, (const float *)(p.dbias_slots ? p.dbias_chunks : nullptr),
                       p.dbias, p.H, W, DBIAS_GRID);
    t.end(K_BWD_DBIAS, st);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_dbias_d(const AttnParams &p, int mode, int act, hipStream_t st) {
    if (mode == JFA) return launch_dbias_t<D, JFA, SILU>(p, st);
    switch (act) {
    case SILU: return launch_dbias_t<D, GDPA, SILU>(p, st);
    case GELU_TANH: return launch_dbias_t<D, GDPA, GELU_TANH>(p, st);
    default: return launch_dbias_t<D, GDPA, GELU_ERF>(p, st);
    }
}

hipError_t launch_dbias_bf16(const AttnParams &p, int D, int mode, int act, hipStream_t st) {
    switch (D) {
    case 32: return launch_dbias_d<32>(p, mode, act, st);
    case 64: return launch_dbias_d<64>(p, mode, act, st);
    default: return launch_dbias_d<128>(p, mode, act, st);
    }
}

}  // namespace ja
