// Internal interface between the C-ABI host layer (ja_api.cpp) and the kernel
// translation units: parameter blocks and launch functions.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ja {

// Work-unit tiles: queries are cut into blocks of Q_TILE rows (forward and the
// dQ units of backward), keys into blocks of KV_TILE rows.
constexpr int Q_TILE = 128;
constexpr int KV_TILE = 64;
constexpr int BWD_KV_UNIT = 128;   // keys owned by one dK/dV unit
constexpr int BWD_Q_STEP = 128;    // queries per inner step of a dK/dV unit
constexpr int FUSED_MAX_LK = 32;   // samples with at most this many keys use the fused backward unit
constexpr int DBIAS_GRID = 512;    // workgroups of the bias-gradient pass (fixed: fixes the summation order)
constexpr int DBIAS_MAX_BINS = 4096;  // largest bias table row the gradient pass takes
constexpr int DBIAS_SLOT_CHUNKS = 64;  // chunks of dQ units whose partial rows are added first (fixed order)

// The chip's accelerator dies (XCDs), each with its own L2.
constexpr int XCDS = 8;

constexpr int ROPE_MAX_HALF = 64;  // D / 2 for the largest head dimension

// Plan (scheduler) output lives at the start of the workspace.
struct PlanCounters {
    int units;   // number of work units (tiles x heads)
    int cursor;  // next unit to hand out (whole-sample lists)
    int flag;    // offsets validation verdict (first block only)
    int pad[29];
    // Tile lists: the units are cut into XCDS contiguous slices, slice c
    // handed out by xcursor[c][0] (one 128-byte line per slice).
    int xcursor[XCDS][32];
};

enum PlanKind {
    PLAN_Q_TILES = 0,   // units = (sample, query tile of tile_rows rows); cost from the keys each row sees
    PLAN_KV_TILES = 1,  // units = (sample, key tile of tile_rows rows); cost from the queries that see it
    PLAN_SAMPLES = 2,   // units = whole samples (one tile each); cost from the query rows
};

struct PlanParams {
    const int32_t *q_off;
    const int32_t *kv_off;
    int lq_fixed;
    int B, H;
    int causal;
    int kind;
    int tile_rows;   // rows per unit tile
    int inner_rows;  // rows per inner-loop step (cost unit)
    int only_short;  // PLAN_SAMPLES: keep samples with lk <= FUSED_MAX_LK; PLAN_KV/Q: skip them (1), not (0),
                     // or keep only them (2)
    int window;      // sliding window (0: none)
    int stable;      // tile lists: 1 = ties in cost keep sample order (a function of the offsets alone)
    int2 *tiles;     // out: (sample, tile) pairs, most expensive first
    int max_tiles;
    PlanCounters *counters;
};

struct AttnParams {
    const void *q, *k, *v;
    const void *o;      // JFA backward: forward output
    const void *o_res;  // JFA backward: optional bf16 rounding residual of o
    void *o_res_out;    // JFA forward: optional residual output
    const void *dout;   // backward: upstream gradient
    void *out;          // forward: O
    void *dq, *dk, *dv; // backward outputs
    float *lse;         // JFA forward: written; backward: read
    float *delta;       // JFA backward: rowwise <dO, O>, [H, Tq]
    const int32_t *q_off, *kv_off;
    int lq_fixed;
    int B, H;
    int64_t total_q_out;  // rows of O (= Tq, or B * lq_fixed)
    int64_t total_q, total_k;
    float scale;
    int causal;
    int window;  // sliding window: aligned distances below it are kept (0: none)
    int bias_kind, bias_lo, bias_hi;
    const float *bias;
    const int2 *tiles;
    PlanCounters *counters;
    const int2 *tiles2;       // backward: dK/dV units; forward: short-K/V units
    PlanCounters *counters2;
    const int2 *tiles3;       // backward: fused short-K/V units
    PlanCounters *counters3;
    const int2 *tiles4;       // bias gradient: query tiles of every sample
    PlanCounters *counters4;
    float *dbias;             // bias gradient output [H][hi - lo + 1], or NULL
    float *dbias_part;        // bias gradient partial rows [DBIAS_GRID][H][hi - lo + 1]
    // Bias gradient folded into the dQ units (NULL: not folded): one row of W
    // partial sums per (dQ unit, wave), and their sums per chunk of units
    // [DBIAS_SLOT_CHUNKS][H][W]
    float *dbias_slots;
    float *dbias_chunks;
    // MXFP8 forward: q, k, v hold E4M3 codes and these their E8M0 scale codes
    // [T, H, D / 32] (all NULL for bf16 / fp32 inputs)
    const uint8_t *q_sc, *k_sc, *v_sc;
    int mx;  // 1: q, k, v are MXFP8 (forward only)
    // Measurement aid: when non-NULL, each workgroup of the launch writes the shader
    // clock cycles from its start to its exit into busy[blockIdx.x] (busy_cap entries)
    uint64_t *busy;
    int busy_cap;
    // Backward with a rotary embedding: the dQ rows leave the kernels turned back
    // (the turn's transpose) by the angle of their row's sample-local position;
    // rope_rev[d] = base^(-2d/D) / (2 pi), turns per position of pair (d, d + D/2).
    int rope_back;
    double rope_rev[ROPE_MAX_HALF];
};

// Units of the tile lists (PLAN_Q_TILES, PLAN_KV_TILES) are numbered
// head-major: unit w is entry w % n of the list (n = units / H) for head
// w / n, so consecutive units are consecutive tiles of one (sample, head).
// Whole-sample lists use unit w = entry w / H, head w % H.
struct UnitRef {
    int2 tile;
    int h;
};
__device__ __forceinline__ UnitRef tile_unit(const int2 *tiles, int w, int n_units, int H) {
    const int n = n_units / H;
    return UnitRef{tiles[w % n], w / n};
}

// Busy-time stamps (measurement aid, AttnParams::busy): the shader clock at the
// workgroup's start, and at its exit the elapsed cycles written by one thread.
__device__ __forceinline__ uint64_t busy_start(const uint64_t *busy) {
    return busy ? __builtin_amdgcn_s_memtime() : 0;
}
__device__ __forceinline__ void busy_end(uint64_t *busy, int cap, uint64_t t0) {
    if (busy && threadIdx.x == 0 && (int)blockIdx.x < cap) busy[blockIdx.x] = __builtin_amdgcn_s_memtime() - t0;
}

// The XCD this workgroup runs on (hardware register XCC_ID).
__device__ __forceinline__ int xcd_id() { return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (XCDS - 1); }

// Next unit of a tile list for a workgroup on XCD `xcd`: its own slice first,
// so the tiles of one (sample, head) — adjacent in the list — run on one XCD
// and share their keys and values (or queries) in that XCD's L2; then the
// other slices in turn once its own is exhausted.  `k` counts the slices this
// workgroup has exhausted (start at 0).  Returns -1 when no unit is left.
__device__ __forceinline__ int next_tile_unit(PlanCounters *c, int n_units, int xcd, int &k) {
    while (k < XCDS) {
        const int sl = (xcd + k) & (XCDS - 1);
        const int b = (int)((int64_t)n_units * sl / XCDS), e = (int)((int64_t)n_units * (sl + 1) / XCDS);
        const int w = b + atomicAdd(&c->xcursor[sl][0], 1);
        if (w < e) return w;
        ++k;
    }
    return -1;
}

// Plans up to PLAN_MAX lists in one launch (one workgroup per list).
constexpr int PLAN_MAX = 4;
struct PlanBatch {
    PlanParams list[PLAN_MAX];
};
hipError_t launch_plan(const PlanParams *lists, int n, hipStream_t stream);

// Opt-in validation of the offsets (device side): *flag = 1 when they break the
// layout rules (see launch_check_offsets), else 0.
struct OffsetsCheck {
    const int32_t *q_off;  // NULL: shared query block, nothing to check
    const int32_t *kv_off;
    int B;
    int64_t total_q, total_k;
    int max_kv_len;        // 0: no bound
    int *flag;
};
hipError_t launch_check_offsets(const OffsetsCheck &c, hipStream_t stream);

// Optional per-kernel event recording around launches (measurement aid).
enum KernelId {
    K_PLAN = 0, K_FWD = 1, K_BWD_FUSED = 2, K_BWD_KV = 3, K_BWD_Q = 4, K_BWD_DELTA = 5, K_FWD_SHORT = 6,
    K_BWD_DBIAS = 7, K_ROPE = 8, K_ROPE_BACK = 9, K_CHECK_OFFSETS = 10, K_COUNT = 11
};
// One (start, stop) event pair per kernel id; a null pair records nothing.
// busy[id] (with its capacity) receives per-workgroup busy cycles of that kernel.
struct KernelTimer {
    hipEvent_t start[K_COUNT] = {}, stop[K_COUNT] = {};
    uint64_t *busy[K_COUNT] = {};
    int busy_cap[K_COUNT] = {};
    // the launch parameters of kernel `id`: p with that kernel's busy-time buffer
    AttnParams with_busy(const AttnParams &p, int id) const {
        AttnParams q = p;
        q.busy = busy[id];
        q.busy_cap = busy_cap[id];
        return q;
    }
    void begin(int id, hipStream_t s) const {
        if (start[id]) (void)hipEventRecord(start[id], s);
    }
    void end(int id, hipStream_t s) const {
        if (stop[id]) (void)hipEventRecord(stop[id], s);
    }
};
const KernelTimer &kernel_timer();

// mode: 0 GDPA, 1 JFA.  act: 0 SiLU, 1 GELU tanh, 2 GELU erf.
// cus: compute units; few_q: every sample has one shared block of <= 32 query
// rows (q_offsets NULL, lq_fixed <= FEW_Q_ROWS), planned as 32-row query tiles.
constexpr int FEW_Q_ROWS = 32;
constexpr int FEW_Q_KV_TILE = 64;  // key tile of those units
constexpr int FEW_Q_HEADS = 4;     // heads of one sample per workgroup (a wave each) in those units
// long_units: launch the long-sequence kernels (false when no sample has more
// than FUSED_MAX_LK keys, so only the short-K/V units have work).
hipError_t launch_fwd_bf16(const AttnParams &p, int D, int mode, int act, int cus, bool few_q, bool long_units,
                           hipStream_t stream);
// The same for MXFP8 inputs (p.mx set); launch_fwd_bf16 forwards to it.
hipError_t launch_fwd_mx(const AttnParams &p, int D, int mode, int act, int cus, bool few_q, bool long_units,
                         hipStream_t stream);
hipError_t launch_bwd_bf16(const AttnParams &p, int D, int mode, int act, int grid, bool long_units,
                           hipStream_t stream);
// The dK/dV units alone; launch_bwd_bf16 calls it between the fused and the dQ units.
hipError_t launch_bwd_kv(const AttnParams &p, int D, int mode, int act, int grid, hipStream_t stream);
// Bias-table gradient (p.dbias, p.dbias_part, p.tiles4 / p.counters4 planned).
hipError_t launch_dbias_bf16(const AttnParams &p, int D, int mode, int act, hipStream_t stream);
// Rotary embedding pass: up to two segments (rows of one [rows, H, D] tensor
// each, with the offsets that give each row its sample-local position, or
// NULL for a shared block whose row r sits at position r), turned by
// sign * t * base^(-2d/D) from src into dst (dst may equal src).
struct RopeSeg {
    const void *src;
    void *dst;
    const int32_t *off;
    int64_t rows;
    int B;
};
struct RopeParams {
    RopeSeg seg[2];
    int H;
    float sign;                       // +1 forward turn, -1 inverse
    double inv_freq[ROPE_MAX_HALF];   // base^(-2d/D), d < D/2
};
hipError_t launch_rope(const RopeParams &p, int D, bool f32, int timer_id, hipStream_t stream);
hipError_t launch_fwd_f32(const AttnParams &p, int D, int mode, int act, hipStream_t stream);
hipError_t launch_bwd_f32(const AttnParams &p, int D, int mode, int act, hipStream_t stream);

}  // namespace ja
