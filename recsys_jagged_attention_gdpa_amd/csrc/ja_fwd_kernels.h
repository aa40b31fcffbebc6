// Forward kernels (bf16 in, fp32 accumulate) for GDPA and JFA on gfx950.
//
// GDPA: O_i = sum_j act(scale <q_i,k_j> + bias_ij) v_j, no normalisation —
// "two matrix multiplications with an element-wise activation in between"
// ("GEM Training: How Meta Doubled the Efficiency...", section "What to
// watch").  Without a softmax there is no running maximum, no rescaling of the
// accumulator and no final normaliser (the pages credit dropping that
// correction stage for freeing resources: "Meta redesigns AI training
// infrastructure...", section "Custom Kernels and 5D Parallelism...").
// JFA: the same contraction with an online softmax (running max m and sum l,
// accumulator rescaled when m grows), epilogue O / l and LSE = m + ln l.
//
// Structure: a persistent grid pulls (sample, 128-row query tile, head) units
// from the planner's longest-first list.  Each of the 4 waves owns 32 query
// rows and keeps them in registers; key / value tiles of 64 rows are staged in
// LDS (double-buffered through registers) and shared by the 4 waves.
//   S^T = K Q^T      (v_mfma_f32_32x32x16_bf16; A = K rows from LDS, B = Q)
//   P^T = act(S^T)   (element-wise in registers)
//   O^T += V^T P^T   (A = V^T by transposing LDS reads, B = P^T straight
//                     from the S^T accumulator: its lane layout already is
//                     the B-operand layout, keys permuted consistently)
// Jagged masking is by offset subtraction: every index is sample-local and a
// tile is masked element-wise only when it crosses the sample's key end or
// the causal diagonal ("Meta redesigns...", section "Eliminating Compute
// Waste in Asymmetric Workloads").  Key rows past the sample's end are loaded
// as zeros.
#pragma once

#include <type_traits>

#include "ja_device.h"
#include "ja_kernels.h"
#include "ja_tiles.h"

namespace ja {

constexpr int FWD_THREADS = 256;
constexpr float RESCALE_SLACK = 8.0f;  // log2 units a running softmax max may lag the true max

// End of a tile step: the tiles that every thread of the unit copied are in
// LDS.  A unit of one wave only orders its own LDS accesses (its DMA has
// landed: store_tile waited for it); a multi-wave unit needs the barrier.
template <bool ONE_WAVE>
__device__ __forceinline__ void unit_sync() {
    if constexpr (ONE_WAVE) {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    } else {
        __syncthreads();
    }
}

// Heads per workgroup of the one-wave units: FEW_Q_HEADS, or fewer where that
// many copies of a unit's LDS tiles would not fit.
template <int D, int BN, bool MX>
constexpr int few_q_heads() {
    constexpr int tiles = 4 * BN * D * ((MX && D >= 64) ? 1 : 2);  // a unit's double-buffered key / value tiles
    return 4 * tiles <= 136 * 1024 ? FEW_Q_HEADS : 2 * tiles <= 136 * 1024 ? 2 : 1;
}

// WAVES waves per workgroup, each owning 32 query rows of the unit's tile
// (BM = 32 WAVES rows), key tiles of BN rows.  The usual shape is 4 waves x
// 64-key tiles.
// SPLIT (JFA with the rounding residual requested): P enters the PV product as
// bf16(P) plus its bf16 residual, two MFMAs into the same accumulator, so O
// (and delta = <dO, O> formed from it in backward) is accurate to ~2^-17
// rather than carrying the 2^-9 rounding of P.
// MX (MXFP8 inputs: E4M3 codes with a scale per 32 head-dimension elements):
// with D = 64 or 128, S^T = K Q^T and O^T = V'^T P'^T run on the block-scaled
// fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) straight from the codes: key
// tiles reach LDS as codes by buffer->LDS copies, query codes stay in
// registers, value rows come through registers and are re-encoded to one
// scale per key on their way into the code tile, and P is encoded as E4M3 per
// 32-key block with that key's scale folded in; the block scales go in as the
// MFMA's scale operands.  With D = 32 the codes are decoded to bf16 after the
// load (key / value tiles through registers) and the bf16 products run.
//
// WAVES = 1 (one block of at most 32 shared query rows, pooling by learned
// seed queries): a unit is one wave over a 32-row query tile, and the waves of
// a workgroup are independent units, one head each of the same sample (head
// groups of few_q_heads()), each with its own LDS tiles and no barrier inside
// its loop.  The heads of a sample share the cache lines of their key and
// value rows (64-byte rows of fp8 codes fill half a line), so running them side
// by side on one CU fetches each line from HBM once.
// HQ (GDPA one-wave units of at most 16 query rows): half the 32 lanes of a
// score block would hold padding rows, so after the S product the real rows of
// the tile's two 32-key blocks are packed into one block's registers
// (v_permlane16_swap), the element-wise stage and the P encoding run once on
// them, and the P operands are unpacked again for the PV product.
template <int D, int MODE, int ACT, int WAVES, int BN, bool SPLIT, bool MX, bool HQ = false>
__global__ __launch_bounds__((WAVES == 1 ? few_q_heads<D, BN, MX>() : WAVES) * WAVE, 2) void fwd_kernel(const AttnParams p) {
    static_assert(!HQ || (WAVES == 1 && MODE == GDPA && BN == 64), "packed rows: GDPA one-wave units, two key blocks");
    constexpr bool F8S = MX && D >= 64;  // S and PV on the fp8 MFMA (key and value tiles hold codes)
    constexpr bool IW = WAVES == 1;      // independent waves, one unit each
    constexpr int WGW = IW ? few_q_heads<D, BN, MX>() : 1;  // waves (units) per workgroup
    constexpr int NT = WAVES * WAVE;
    constexpr int BM = 32 * WAVES;
    constexpr int TILE_BYTES = BN * D * (F8S ? 1 : 2);
    constexpr int NKK = D / 16;  // k-steps over the head dimension
    constexpr int NDB = D / 32;  // 32-wide blocks of the head dimension
    constexpr int NNB = BN / 32; // 32-key blocks per tile
    constexpr int NKS = BN / 16; // 16-key k-steps per tile
    constexpr int WIN = BM + BN - 1;  // largest bias window of a (unit, key tile)
    constexpr int WPT = (WIN + NT - 1) / NT;  // bias window entries per thread
    __shared__ __attribute__((aligned(16))) char smem[WGW][4 * TILE_BYTES];
    __shared__ float s_bias_w[WGW][2][WIN];
    __shared__ __attribute__((aligned(16))) float s_vsc_w[WGW][2][F8S ? BN : 4];  // F8S: each value row's factor 2^(S_j - 127)
    __shared__ int s_unit;

    const int H = p.H;
    const int tid = threadIdx.x;
    // the wave index as a scalar: with independent waves it selects the head,
    // so everything addressed through it (descriptors included) stays uniform
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int ut = IW ? lane : tid;  // thread index within the unit
    const int uw = IW ? 0 : wv;      // wave index within the unit
    lchar *const lbase = (lchar *)smem[IW ? wv : 0];
    float(*const s_bias)[WIN] = s_bias_w[IW ? wv : 0];
    float(*const s_vsc)[F8S ? BN : 4] = s_vsc_w[IW ? wv : 0];
    // IW: units are (list entry, group of WGW heads)
    const int hg = (p.H + WGW - 1) / WGW;
    const int n_units = IW ? p.counters->units / p.H * hg : p.counters->units;
    if (n_units == 0) return;
    const BiasArgs bz{p.bias, p.bias_kind, p.bias_lo, p.bias_hi, p.bias_hi - p.bias_lo + 1};
    const float sl2 = p.scale * LOG2E;

    const uint64_t busy_t0 = busy_start(p.busy);
    const int xcd = xcd_id();
    int slices_done = 0;
    for (;;) {
        if (tid == 0) s_unit = next_tile_unit(p.counters, n_units, xcd, slices_done);
        __syncthreads();
        const int w = s_unit;
        __syncthreads();
        if (w < 0) break;
        const UnitRef u = IW ? UnitRef{p.tiles[w / hg], (w % hg) * WGW + wv} : tile_unit(p.tiles, w, n_units, H);
        const int2 tile = u.tile;
        const int h = u.h;
        if (IW && h >= H) continue;            // a wave past the last head of the group
        const Sample s = load_sample(p.q_off, p.lq_fixed, p.kv_off, tile.x);
        const int i0 = tile.y * BM;            // first query row of the unit (sample-local)
        const int iw = i0 + uw * 32;           // first row of this wave
        const int irow = iw + l32;             // this lane's query row
        const int i_last = (i0 + BM < s.lq ? i0 + BM : s.lq) - 1;
        const int kend = key_end(i_last, s.lq, s.lk, p.causal, p.window);
        const int nkv = (kend + BN - 1) / BN;
        const int jt_first = key_begin(i0, s.lq, s.lk, p.window) / BN;  // tiles before it see no row of the unit
        const HeadSlice<D> Qs(p.q, s.qs, s.lq, H, h), Os(p.out, s.o0, s.lq, H, h);
        const HeadSlice<D> Ks(p.k, s.ks, s.lk, H, h), Vs(p.v, s.ks, s.lk, H, h);
        const bool res = MODE == JFA && p.o_res_out != nullptr;
        const HeadSlice<D> Rs(res ? p.o_res_out : p.out, s.o0, res ? s.lq : 0, H, h);
        const rsrc_t brs = make_rsrc(bz.kind ? bz.table + (int64_t)h * bz.width : nullptr,
                                     bz.kind ? (uint32_t)bz.width * 4u : 0u);

        // Q rows of this lane, in B-operand layout: chunk 2kk+g of row irow.
        constexpr int NKS8 = D / 64;          // 64-code k-steps of the fp8 MFMA
        bf16x8 qreg[F8S ? 1 : NKK];
        i32x8 qf[F8S ? NKS8 : 1];  // F8S: query codes, operand layout
        int qsc[F8S ? NKS8 : 1];   // F8S: their block scale codes
        if constexpr (F8S) {
            const MXSlice<D> Qm(p.q, p.q_sc, s.qs, s.lq, H, h);
#pragma unroll
            for (int ks = 0; ks < NKS8; ++ks) {
                qf[ks] = f8_row_operand<D>(Qm, irow, ks, g);
                qsc[ks] = f8_scale<D>(Qm, irow, 2 * ks + g);
            }
        } else if constexpr (MX) {
            load_row_operand<D>(qreg, MXSlice<D>(p.q, p.q_sc, s.qs, s.lq, H, h), irow, g);
        } else {
            load_row_operand<D>(qreg, Qs, irow, g);
        }
        const MXSlice<D> Km(p.k, p.k_sc, s.ks, MX ? s.lk : 0, H, h), Vm(p.v, p.v_sc, s.ks, MX ? s.lk : 0, H, h);
        MXPairLoader<BN, D, NT> mxl;  // MX: key and value codes, decoded into LDS
        F8VLoader<BN, D, NT> mxv;     // F8S: value codes, re-encoded to one scale per key
        uint32_t kwn = 0;                 // F8S: scale word of key row lane of the next tile
        int ksc[NNB][F8S ? NKS8 : 1];     // F8S: the lane's key-row scale codes, current tile
        static_assert(!F8S || BN <= WAVE, "one key row per lane");

        f32x16 oacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
        float m_run = -INFINITY, l_run = 0.0f;  // JFA running max (log2 units) and partial sum

        // Key / value tile jt goes to LDS buffer (jt & 1): bf16 tiles and the
        // fp8 key codes are copied straight into it, decoded MXFP8 tiles pass
        // through registers (loaded here, written by store_tile); the bias window
        // it needs goes through a register.  Loads past the sample read zeros.
        float bnext[WPT];
        auto load_tile = [&](int jt) {
            lchar *kt = lbase + (jt & 1) * 2 * TILE_BYTES;
            if constexpr (F8S) {
                dma_f8_tile<BN, D, NT>(kt, Km, jt * BN, ut);
                mxv.load(Vm, jt * BN, ut);
                kwn = f8_scale_word<D>(Km, jt * BN + lane, lane < BN);
            } else if constexpr (MX) {
                mxl.load(Km, Vm, jt * BN, ut);
            } else {
                dma_tile<BN, D, NT>(kt, Ks, jt * BN, ut);
                dma_tile<BN, D, NT>(kt + TILE_BYTES, Vs, jt * BN, ut);
            }
#pragma unroll
            for (int r = 0; r < WPT; ++r) {
                const int bi = bias_stage_rowmajor(bz, i0, BM, jt * BN, BN, ut + r * NT);
                bnext[r] = buf_load_f32(brs, bi >= 0 ? (uint32_t)bi * 4u : OOB);
            }
        };
        auto store_tile = [&](int buf) {
            if constexpr (F8S) {
                mxv.store(lbase + buf * 2 * TILE_BYTES + TILE_BYTES, (lfloat *)s_vsc[buf], ut);
#pragma unroll
                for (int nb = 0; nb < NNB; ++nb) {
                    const uint32_t w = lane_word(kwn, nb * 32 + l32);  // key row nb * 32 + l32
#pragma unroll
                    for (int ks = 0; ks < NKS8; ++ks) ksc[nb][ks] = (int)((w >> (8 * (2 * ks + g))) & 255u);
                }
            } else if constexpr (MX) {
                mxl.store(lbase + buf * 2 * TILE_BYTES, lbase + buf * 2 * TILE_BYTES + TILE_BYTES, ut);
            }
#pragma unroll
            for (int r = 0; r < WPT; ++r)  // JFA works in log2 units
                if (ut + r * NT < WIN) s_bias[buf][ut + r * NT] = MODE == JFA ? bnext[r] * LOG2E : bnext[r];
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's part of the tile has landed
        };
        load_tile(jt_first);
        store_tile(jt_first & 1);
        unit_sync<IW>();

        // keys of the wave's rows: every row sees [wkb, wke) at least; masking is
        // needed only where a tile leaves that range
        const int wke = key_end(iw, s.lq, s.lk, p.causal, p.window);
        const int wkb = key_begin(iw + 31, s.lq, s.lk, p.window);
        // HQ: lanes 16 .. 31 of each half hold rows 0 .. 15 of the second key block
        const int qlane = HQ ? (lane & 15) : l32;
        const int nbo = HQ ? ((lane >> 4) & 1) * 32 : 0;  // HQ: key offset of this lane's block
        const int erow = iw + qlane;                     // query row of this lane's values
        const int my_kbeg = key_begin(erow, s.lq, s.lk, p.window);
        for (int jt = jt_first; jt < nkv; ++jt) {
            const int j0 = jt * BN;
            const lchar *Kt = lbase + (jt & 1) * 2 * TILE_BYTES;
            const lchar *Vt = Kt + TILE_BYTES;
            const float *bwin = s_bias[jt & 1];
            load_tile(jt + 1);  // past the last tile: zeros, no traffic
            __builtin_amdgcn_sched_barrier(0);

            // S^T block per 32 keys: lane holds query irow, keys crow(e, g).
            f32x16 sacc[NNB];
#pragma unroll
            for (int nb = 0; nb < NNB; ++nb) {
                sacc[nb] = f32x16{};
                if constexpr (F8S) {
#pragma unroll
                    for (int ks = 0; ks < NKS8; ++ks) {
                        const i32x8 a = lds_read_f8_operand<D>(Kt, nb * 32 + l32, ks, g);
                        sacc[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[ks], sacc[nb], 0, 0, 0,
                                                                                  ksc[nb][ks], 0, qsc[ks]);
                    }
                } else {
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) {
                        const bf16x8 a = lds_read16(Kt, lds_off<D>(nb * 32 + l32, 2 * kk + g));
                        sacc[nb] = mfma32(a, qreg[kk], sacc[nb]);
                    }
                }
            }

            // Element-wise stage.  A tile needs per-element masking only when it
            // crosses the key end, (causal) the diagonal or (window) the window
            // start of this wave's rows; that test and the bias kind are
            // wave-uniform, so each variant is a straight-line loop behind one
            // scalar branch.
            const bool masked = (j0 + BN > wke) || (j0 < wkb);
            const int my_kend = key_end(erow, s.lq, s.lk, p.causal, p.window);
            constexpr int NBE = HQ ? 1 : NNB;  // score blocks the element-wise stage runs on
            if constexpr (HQ) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float x = sacc[0][e], y = sacc[1][e];
                    row_swap16(x, y);
                    sacc[0][e] = x;
                    sacc[1][e] = y;
                }
            }
            bf16x8 pb[F8S ? 1 : NKS], pbl[SPLIT && !F8S ? NKS : 1];
            u32x4 pf8[2] = {u32x4{}, u32x4{}};  // F8S: P^T codes of the tile's 32-key blocks
            int pex[2] = {127, 127};             // F8S: their E8M0 scale codes
            // x = scale * s + bias (JFA: in log2 units); without bias only the
            // scale is applied, folded into later arithmetic where possible.
            if (bz.kind) {
                // raw window: entry (i0 + BM - 1 - irow) + (j - j0) (REL) or j - j0 (KEYPOS)
                const int bbase = (bz.kind == BIAS_REL ? BM - 1 - uw * 32 - qlane : 0) + g * 4 + nbo;
#pragma unroll
                for (int nb = 0; nb < NBE; ++nb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float b = bwin[bbase + nb * 32 + (e >> 2) * 8 + (e & 3)];
                        sacc[nb][e] = __builtin_fmaf(sacc[nb][e], MODE == GDPA ? p.scale : sl2, b);
                    }
            }
            const float xmul = bz.kind ? 1.0f : (MODE == GDPA ? p.scale : sl2);  // remaining scale
            if constexpr (MODE == GDPA) {
                if (!bz.kind) {
#pragma unroll
                    for (int nb = 0; nb < NBE; ++nb)
#pragma unroll
                        for (int e = 0; e < 16; ++e) sacc[nb][e] *= p.scale;
                }
#pragma unroll
                for (int nb = 0; nb < NBE; ++nb) {
                    float pv[16];
#pragma unroll
                    for (int e = 0; e < 16; ++e) pv[e] = act_fwd<ACT>(sacc[nb][e]);
                    if (masked) {
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int j = j0 + nb * 32 + nbo + crow(e, g);
                            pv[e] = ((j >= my_kend) | (j < my_kbeg)) ? 0.0f : pv[e];
                        }
                    }
                    if constexpr (F8S) {
                        pex[nb] = encode_p_block(pv, (const lfloat *)s_vsc[jt & 1] + nb * 32 + nbo, g, pf8[nb]);
                    } else {
                        pack_operands(pv, pb[2 * nb], pb[2 * nb + 1]);
                    }
                }
                if constexpr (HQ) {
                    // back to one operand per key block: rows 0 and 2 (queries 0 .. 15)
                    // of block 1 come from rows 1 and 3 of the packed registers
                    if constexpr (F8S) {
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            uint32_t x = pf8[0][k], y = 0u;
                            row_swap16(x, y);
                            pf8[0][k] = x;
                            pf8[1][k] = y;
                        }
                        // scale codes: ea takes block 0's code into every row, eb block 1's
                        // (the block-1 code of query q sits in row 3 and reaches row 2)
                        int ea = pex[0], eb = pex[0];
                        row_swap16_same(ea, eb);
                        pex[0] = ea;
                        pex[1] = eb;
                    } else {
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2) {
                            const u32x4 a = __builtin_bit_cast(u32x4, pb[h2]);
                            u32x4 lo, hi;
#pragma unroll
                            for (int k = 0; k < 4; ++k) {
                                uint32_t x = a[k], y = 0u;
                                row_swap16(x, y);
                                lo[k] = x;
                                hi[k] = y;
                            }
                            pb[h2] = __builtin_bit_cast(bf16x8, lo);
                            pb[2 + h2] = __builtin_bit_cast(bf16x8, hi);
                        }
                    }
                }
            } else {
                if (masked) {
#pragma unroll
                    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int j = j0 + nb * 32 + crow(e, g);
                            sacc[nb][e] = ((j >= my_kend) | (j < my_kbeg)) ? -INFINITY : sacc[nb][e];
                        }
                }
                float tmax = -INFINITY;
#pragma unroll
                for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, sacc[nb][e]);
                tmax = pair_max(tmax) * xmul;  // xmul > 0, so the max commutes with it
                // The running max is only moved (and O, l rescaled) when the tile's
                // max exceeds it by more than RESCALE_SLACK (log2 units); otherwise
                // P is formed against the stale max and stays below 2^RESCALE_SLACK.
                if (wave_any(tmax > m_run + RESCALE_SLACK)) {
                    // fp8 P: whole-number maxima, so every rescale is by a power of two
                    // and P is encoded against a reference the scales absorb exactly
                    const float m_new = F8S ? ceilf(fmaxf(m_run, tmax)) : fmaxf(m_run, tmax);
                    const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m_run - m_new);
                    m_run = m_new;
                    l_run *= alpha;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
                }
                const float nm = m_run == -INFINITY ? 0.0f : -m_run;
#pragma unroll
                for (int nb = 0; nb < NNB; ++nb) {
                    float pv[16];
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        pv[e] = fast_exp2(__builtin_fmaf(sacc[nb][e], xmul, nm));
                        l_run += pv[e];
                    }
                    if constexpr (F8S) {
                        pex[nb] = encode_p_block(pv, (const lfloat *)s_vsc[jt & 1] + nb * 32, g, pf8[nb]);
                    } else {
                        pack_operands(pv, pb[2 * nb], pb[2 * nb + 1]);
                        if constexpr (SPLIT) pack_residual_operands(pv, pbl[2 * nb], pbl[2 * nb + 1]);
                    }
                }
            }

            // O^T += V^T P^T over the tile's keys.
            if constexpr (F8S) {
                const i32x8 bop = p_f8_operand(pf8[0], pf8[1]);
                const int scb = g ? pex[1] : pex[0];
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const i32x8 a = lds_read_vt_f8<D, NNB>(Vt, db, lane);
                    oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop, oacc[db], 0, 0, 0, 127, 0, scb);
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const bf16x8 a = lds_read_tr_operand<D>(Vt, ks * 16, db * 32, lane);
                        oacc[db] = mfma32(a, pb[ks % (F8S ? 1 : NKS)], oacc[db]);
                        if constexpr (SPLIT && !F8S) oacc[db] = mfma32(a, pbl[ks % (SPLIT && !F8S ? NKS : 1)], oacc[db]);
                    }
                }
            }

            store_tile((jt + 1) & 1);
            unit_sync<IW>();
        }

        // Epilogue: lane owns query row irow; d = db*32 + crow(e, g).
        float norm = 1.0f;
        if constexpr (MODE == JFA) {
            const float l_tot = pair_sum(l_run);
            const bool any = l_tot > 0.0f;
            norm = any ? 1.0f / l_tot : 0.0f;
            const rsrc_t lr = make_rsrc(p.lse + (int64_t)h * p.total_q_out + s.o0, (uint32_t)s.lq * 4u);
            buf_store_f32(lr, g == 0 ? (uint32_t)irow * 4u : OOB, any ? (m_run + log2f(l_tot)) * LN2 : -INFINITY);
            store_row_acc_split<D>(Os, Rs, irow, oacc, norm, g);
        } else {
            store_row_acc<D>(Os, irow, oacc, norm, g);
        }
    }
    busy_end(p.busy, p.busy_cap, busy_t0);
}

// ------------------------------------------------------------------------
// Short key/value samples (at most 32 keys), one unit per (sample, head).
// The inner loop over key tiles would have a single iteration, so the
// pipelining moves to the outer loop ("Meta redesigns...", section "Custom
// Kernels and 5D Parallelism...": outer-loop software pipelining when the
// inner loop runs one or two iterations): K and V stay in LDS for the whole
// sample, each wave claims 32-row query blocks from a per-unit counter, and
// it loads its next block's Q rows into registers while the current block is
// computed.  Loads and stores go through per-sample buffer descriptors, so the
// loop body has no branches around memory operations and the next block's
// loads stay in flight across the current block's stores.
// MX: MXFP8 inputs.  With D = 64 or 128, S^T = K Q^T runs on the block-scaled
// fp8 MFMA: key codes stay codes in LDS, each Q block is staged as codes in the
// wave's tile, the block scales go in as the MFMA's scale operands, and only V
// is decoded to bf16 for the PV product.  With D = 32 all three are decoded.
template <int D, int MODE, int ACT, bool SPLIT, bool MX>
__global__ __launch_bounds__(FWD_THREADS, 2) void fwd_short_kernel(const AttnParams p) {
    constexpr int KV_BYTES = 32 * D * 2;
    constexpr int NKK = D / 16, NDB = D / 32;
    constexpr int NWAVES = FWD_THREADS / WAVE;
    __shared__ __attribute__((aligned(16))) char smem[(2 + NWAVES) * KV_BYTES];
    __shared__ __attribute__((aligned(16))) float s_vsc[32];  // F8: each value row's factor 2^(S_j - 127)
    __shared__ int s_unit, s_blk;
    lchar *const Kt = (lchar *)smem;
    lchar *const Vt = Kt + KV_BYTES;

    const int H = p.H;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    lchar *const Ot = Vt + KV_BYTES * (1 + wv);  // this wave's output staging tile
    const int g = lane >> 5, l32 = lane & 31;
    const int n_units = p.counters2->units;
    if (n_units == 0) return;
    const BiasArgs bz{p.bias, p.bias_kind, p.bias_lo, p.bias_hi, p.bias_hi - p.bias_lo + 1};
    const float sl2 = p.scale * LOG2E;

    const uint64_t busy_t0 = busy_start(p.busy);
    for (;;) {
        if (threadIdx.x == 0) {
            s_unit = atomicAdd(&p.counters2->cursor, 1);
            s_blk = FWD_THREADS / WAVE;  // blocks 0..3 go to waves 0..3
        }
        __syncthreads();
        const int w = s_unit;
        if (w >= n_units) break;
        const int2 tile = p.tiles2[w / H];
        const int h = w % H;
        const Sample s = load_sample(p.q_off, p.lq_fixed, p.kv_off, tile.x);
        const float *brow = bz.kind ? bz.table + (int64_t)h * bz.width : nullptr;
        constexpr bool F8 = MX && D >= 64;  // S and PV on the fp8 MFMA
        constexpr int NKS8 = D / 64;
        int ksc[F8 ? NKS8 : 1];              // F8: scale codes of the lane's key row l % 32
        if constexpr (F8) {
            const MXSlice<D> Km(p.k, p.k_sc, s.ks, s.lk, H, h);
            F8VLoader<32, D, FWD_THREADS> vl;
            vl.load(MXSlice<D>(p.v, p.v_sc, s.ks, s.lk, H, h), 0, threadIdx.x);
            constexpr int KPIECES = 32 * D / 16;  // 16-code pieces of the key tile
            if (threadIdx.x < KPIECES) {
                const int r = threadIdx.x / (D / 16), pr = threadIdx.x % (D / 16);
                lds_write16(Kt, f8_off<D>(r, pr), Km.codes16(r, pr));
            }
#pragma unroll
            for (int ks = 0; ks < NKS8; ++ks) ksc[ks] = f8_scale<D>(Km, l32, 2 * ks + g);
            vl.store(Vt, (lfloat *)s_vsc, threadIdx.x);
        } else if constexpr (MX) {
            MXPairLoader<32, D, FWD_THREADS> kv;
            kv.load(MXSlice<D>(p.k, p.k_sc, s.ks, s.lk, H, h), MXSlice<D>(p.v, p.v_sc, s.ks, s.lk, H, h), 0,
                    threadIdx.x);
            kv.store(Kt, Vt, threadIdx.x);
        } else {
            PairLoader<32, D, FWD_THREADS> kv;
            kv.load(static_cast<const bf16 *>(p.k), static_cast<const bf16 *>(p.v), s.ks, H, h, 0, s.lk, threadIdx.x);
            kv.store(Kt, Vt, threadIdx.x);
        }
        using QSlice = std::conditional_t<MX, MXSlice<D>, HeadSlice<D>>;
        using QTile = std::conditional_t<F8, F8WaveTile<D>, std::conditional_t<MX, MXWaveTile<D>, WaveTile<D>>>;
        const QSlice Qs = [&]() {
            if constexpr (MX) return MXSlice<D>(p.q, p.q_sc, s.qs, s.lq, H, h);
            else return HeadSlice<D>(p.q, s.qs, s.lq, H, h);
        }();
        const HeadSlice<D> Os(p.out, s.o0, s.lq, H, h);
        // the residual (JFA, optional) and LSE slices; zero-sized when not written
        const bool res = MODE == JFA && p.o_res_out != nullptr;
        const HeadSlice<D> Rs(res ? p.o_res_out : p.out, s.o0, res ? s.lq : 0, H, h);
        const rsrc_t lse_r = make_rsrc(MODE == JFA ? p.lse + (int64_t)h * p.total_q_out + s.o0 : p.lse,
                                       MODE == JFA ? (uint32_t)s.lq * 4u : 0u);
        const int nblk = (s.lq + 31) / 32;
        const bool masked = s.lk < 32 || p.causal || p.window;
        // One 32-row query block, with Q rows in `qreg`; the next block's rows
        // are loaded into `qnext` first, so they are in flight meanwhile.  The
        // wave's LDS tile holds the block's Q rows, then its output rows.
        auto block = [&](int blk, const QTile &qreg, QTile &qnext) -> int {
            const int irow = blk * 32 + l32;
            qreg.store(Ot, lane);
            lds_wave_sync();
            float bv[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) bv[e] = 0.0f;
            if (brow) {
#pragma unroll
                for (int e = 0; e < 16; ++e) bv[e] = bias_at(bz, brow, irow, crow(e, g));
            }
            int nxt = 0;
            if (lane == 0) nxt = atomicAdd(&s_blk, 1);
            nxt = __builtin_amdgcn_readfirstlane(nxt);
            qnext.load(Qs, nxt * 32, lane);  // past the sample: zeros, no traffic
            __builtin_amdgcn_sched_barrier(0);  // keep the next block's loads ahead of this block's work

            f32x16 sacc = f32x16{};
            if constexpr (F8) {
#pragma unroll
                for (int ks = 0; ks < NKS8; ++ks)
                    sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        lds_read_f8_operand<D>(Kt, l32, ks, g), lds_read_f8_operand<D>(Ot, l32, ks, g), sacc, 0, 0, 0,
                        ksc[ks], 0, qreg.sc[ks]);
            } else {
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const int off = lds_off<D>(l32, 2 * kk + g);
                    sacc = mfma32(lds_read16(Kt, off), lds_read16(Ot, off), sacc);
                }
            }
            const int my_kend = key_end(irow, s.lq, s.lk, p.causal, p.window);
            const int my_kbeg = key_begin(irow, s.lq, s.lk, p.window);
            float pv[16];
            float norm = 1.0f, lse_row = 0.0f;
            // masked is unit-uniform: interior units carry no per-element tests
            if constexpr (MODE == GDPA) {
#pragma unroll
                for (int e = 0; e < 16; ++e) pv[e] = act_fwd<ACT>(__builtin_fmaf(sacc[e], p.scale, bv[e]));
                if (masked) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int j = crow(e, g);
                        pv[e] = ((j >= my_kend) | (j < my_kbeg)) ? 0.0f : pv[e];
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) pv[e] = __builtin_fmaf(sacc[e], sl2, bv[e] * LOG2E);
                if (masked) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int j = crow(e, g);
                        pv[e] = ((j >= my_kend) | (j < my_kbeg)) ? -INFINITY : pv[e];
                    }
                }
                float m = -INFINITY;
#pragma unroll
                for (int e = 0; e < 16; ++e) m = fmaxf(m, pv[e]);
                m = fmaxf(m, shfl_xor32(m));
                // fp8 P: a whole-number reference, which the block scale absorbs exactly
                const float shift = m == -INFINITY ? 0.0f : (F8 ? ceilf(m) : m);
                float l = 0.0f;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    pv[e] = fast_exp2(pv[e] - shift);
                    l += pv[e];
                }
                l += shfl_xor32(l);
                norm = l > 0.0f ? 1.0f / l : 0.0f;
                lse_row = l > 0.0f ? (shift + log2f(l)) * LN2 : -INFINITY;
            }
            bf16x8 pb[2], pbl[2];
            i32x8 pf8 = i32x8{};  // F8: P^T codes (one 32-key block) and this lane's scale operand
            int scb = 127;
            if constexpr (F8) {
                u32x4 c0;
                const int ex = encode_p_block(pv, (const lfloat *)s_vsc, g, c0);
                pf8 = p_f8_operand(c0, u32x4{});
                scb = g ? 127 : ex;
            } else {
                pack_operands(pv, pb[0], pb[1]);
                if constexpr (SPLIT) pack_residual_operands(pv, pbl[0], pbl[1]);
            }
            if constexpr (MODE == JFA) buf_store_f32(lse_r, g == 0 ? (uint32_t)irow * 4u : OOB, lse_row);
            // One 32-wide block of the head dimension at a time, staged as it
            // completes, so only one accumulator block is live.  The optional
            // rounding residual (JFA) is written straight from the registers.
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                f32x16 acc = f32x16{};
                if constexpr (F8) {
                    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(lds_read_vt_f8<D, 1>(Vt, db, lane), pf8, acc,
                                                                          0, 0, 0, 127, 0, scb);
                } else {
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const bf16x8 a = lds_read_tr_operand<D>(Vt, ks * 16, db * 32, lane);
                        acc = mfma32(a, pb[ks], acc);
                        if constexpr (SPLIT) acc = mfma32(a, pbl[ks], acc);
                    }
                }
                stage_acc_block<D>(Ot, acc, db, norm, l32, g);
                if (MODE == JFA && res) store_resid_block<D>(Rs, irow, acc, db, norm, g);
            }
            lds_wave_sync();
            store_staged<D>(Os, Ot, blk * 32, lane);
            return nxt;
        };

        int blk = wv;
        QTile qa, qb;
        qa.load(Qs, blk * 32, lane);
        // Enter the loop with nothing outstanding, so the loop's waits cover
        // only the previous block's prefetch, not its stores.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __syncthreads();
        // two register sets alternate, so no copy waits on the loads in flight
        for (;;) {
            if (blk >= nblk) break;
            blk = block(blk, qa, qb);
            if (blk >= nblk) break;
            blk = block(blk, qb, qa);
        }
        __syncthreads();  // K / V of this unit are no longer read
    }
    busy_end(p.busy, p.busy_cap, busy_t0);
}

// The bf16 GDPA units of the long-sequence kernel are launched from a
// translation unit of their own (ja_fwd_gdpa.hip), which the build compiles
// with its own instruction scheduler; it instantiates every (D, ACT).
template <int D, int ACT>
hipError_t launch_fwd_gdpa_long(const AttnParams &p, int cus, hipStream_t stream);

template <int D, int MODE, int ACT, bool SPLIT, bool MX>
inline hipError_t launch_fwd_s(const AttnParams &p, int cus, bool few_q, bool long_units, hipStream_t stream) {
    const KernelTimer &t = kernel_timer();
    t.begin(K_FWD_SHORT, stream);
    hipLaunchKernelGGL((fwd_short_kernel<D, MODE, ACT, SPLIT, MX>), dim3(2 * cus), dim3(FWD_THREADS), 0, stream,
                       t.with_busy(p, K_FWD_SHORT));
    t.end(K_FWD_SHORT, stream);
    if (!long_units) return hipGetLastError();
    t.begin(K_FWD, stream);
    constexpr int FQH = few_q_heads<D, FEW_Q_KV_TILE, MX>();
    if (few_q && MODE == GDPA && p.lq_fixed <= 16)  // at most 16 shared query rows: packed rows
        hipLaunchKernelGGL((fwd_kernel<D, GDPA, ACT, 1, FEW_Q_KV_TILE, false, MX, true>), dim3(8 / FQH * cus),
                           dim3(FQH * WAVE), 0, stream, t.with_busy(p, K_FWD));
    else if (few_q)  // every unit is one block of <= 32 shared query rows
        hipLaunchKernelGGL((fwd_kernel<D, MODE, ACT, 1, FEW_Q_KV_TILE, SPLIT, MX>), dim3(8 / FQH * cus),
                           dim3(FQH * WAVE), 0, stream, t.with_busy(p, K_FWD));
    else if constexpr (MODE == GDPA && !MX)
        (void)launch_fwd_gdpa_long<D, ACT>(p, cus, stream);
    else
        hipLaunchKernelGGL((fwd_kernel<D, MODE, ACT, 4, KV_TILE, SPLIT, MX>), dim3(2 * cus), dim3(4 * WAVE), 0, stream,
                           t.with_busy(p, K_FWD));
    t.end(K_FWD, stream);
    return hipGetLastError();
}

// Launch of the forward kernels for one input format (MX: MXFP8 codes).
template <int D, int MODE, int ACT, bool MX>
inline hipError_t launch_fwd_t(const AttnParams &p, int cus, bool few_q, bool long_units, hipStream_t stream) {
    if (MODE == JFA && p.o_res_out) return launch_fwd_s<D, MODE, ACT, true, MX>(p, cus, few_q, long_units, stream);
    return launch_fwd_s<D, MODE, ACT, false, MX>(p, cus, few_q, long_units, stream);
}

template <int D, bool MX>
inline hipError_t launch_fwd_d(const AttnParams &p, int mode, int act, int cus, bool few_q, bool lu,
                               hipStream_t stream) {
    if (mode == JFA) return launch_fwd_t<D, JFA, SILU, MX>(p, cus, few_q, lu, stream);
    switch (act) {
    case SILU: return launch_fwd_t<D, GDPA, SILU, MX>(p, cus, few_q, lu, stream);
    case GELU_TANH: return launch_fwd_t<D, GDPA, GELU_TANH, MX>(p, cus, few_q, lu, stream);
    default: return launch_fwd_t<D, GDPA, GELU_ERF, MX>(p, cus, few_q, lu, stream);
    }
}

template <bool MX>
inline hipError_t launch_fwd_fmt(const AttnParams &p, int D, int mode, int act, int cus, bool few_q, bool lu,
                                 hipStream_t stream) {
    switch (D) {
    case 32: return launch_fwd_d<32, MX>(p, mode, act, cus, few_q, lu, stream);
    case 64: return launch_fwd_d<64, MX>(p, mode, act, cus, few_q, lu, stream);
    default: return launch_fwd_d<128, MX>(p, mode, act, cus, few_q, lu, stream);
    }
}

}  // namespace ja
