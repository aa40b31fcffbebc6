// C-ABI host layer: argument checks, workspace layout, kernel launches.
// The declarations and their contracts are in include/jagged_attn.h.
#include "jagged_attn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "ja_kernels.h"

namespace {

thread_local int g_last_hip_error = 0;
thread_local ja::KernelTimer g_timer;

constexpr size_t ALIGN = 256;
constexpr int MAX_DEVICES = 64;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// Compute units of the current device, cached per device.
int cu_count() {
    static std::atomic<int> cache[MAX_DEVICES];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

int64_t total_q_out(const ja_problem &p) {
    return p.q_offsets ? p.total_q : (int64_t)p.batch * p.lq_fixed;
}

// Capacity of a unit list cutting `rows` jagged rows of B samples into tiles of `tile` rows.
int64_t tile_cap(int64_t rows, int B, int tile) { return rows / tile + B + 1; }

struct Layout {
    size_t counters;  // 4 PlanCounters blocks
    size_t tiles_q, tiles_k, tiles_s, delta, tiles_a, dbias_part, dbias_slots, dbias_chunks, rope_q, rope_k, total;
    int64_t cap_q, cap_k, cap_s;
};

int64_t bias_width(const ja_problem &p) { return (int64_t)p.bias_hi - p.bias_lo + 1; }

// The sliding window as the kernels take it: a window wider than any sample's
// aligned distances (at most Lq + Lk <= total_q + total_k) keeps every pair, so
// larger values are clamped to total_q + total_k + 1, which keeps the kernels'
// 32-bit index sums (row + key count + window) in range.
int eff_window(const ja_problem &p) {
    const int64_t cap = p.total_q + p.total_k + 1;
    return (int)((int64_t)p.window < cap ? p.window : cap);
}

Layout layout_of(const ja_problem &p, int pass) {
    Layout L{};
    const int64_t tq = p.q_offsets ? p.total_q : (int64_t)p.lq_fixed * p.batch;
    L.cap_q = tile_cap(tq, p.batch, ja::Q_TILE);
    L.cap_k = tile_cap(p.total_k, p.batch, ja::BWD_KV_UNIT);
    L.cap_s = (int64_t)p.batch + 1;
    size_t off = 0;
    L.counters = off;
    off += align_up(4 * sizeof(ja::PlanCounters));
    L.tiles_q = off;
    off += align_up((size_t)L.cap_q * sizeof(int2));
    L.tiles_s = off;
    off += align_up((size_t)L.cap_s * sizeof(int2));
    if (pass == JA_PASS_BWD || pass == JA_PASS_BWD_DBIAS) {
        L.tiles_k = off;
        off += align_up((size_t)L.cap_k * sizeof(int2));
        L.delta = off;
        off += align_up((size_t)p.heads * (size_t)(p.total_q > 0 ? p.total_q : 1) * sizeof(float));
    }
    if (pass == JA_PASS_BWD_DBIAS) {
        L.tiles_a = off;  // query tiles of every sample
        off += align_up((size_t)L.cap_q * sizeof(int2));
        L.dbias_part = off;
        off += align_up((size_t)ja::DBIAS_GRID * p.heads * (size_t)bias_width(p) * sizeof(float));
        // the dQ units' partial rows: one per (unit, wave), and their chunk sums
        L.dbias_slots = off;
        off += align_up((size_t)L.cap_q * p.heads * 4 * (size_t)bias_width(p) * sizeof(float));
        L.dbias_chunks = off;
        off += align_up((size_t)ja::DBIAS_SLOT_CHUNKS * p.heads * (size_t)bias_width(p) * sizeof(float));
    }
    if (p.rope_base > 0.0f && !p.rope_inputs_turned) {  // turned copies of q and k
        const size_t row = (size_t)p.heads * p.head_dim * (p.dtype == JA_BF16 ? 2 : 4);
        L.rope_q = off;
        off += align_up((size_t)(p.total_q > 0 ? p.total_q : 1) * row);
        L.rope_k = off;
        off += align_up((size_t)(p.total_k > 0 ? p.total_k : 1) * row);
    }
    L.total = off;
    return L;
}

ja_status check_problem(const ja_problem *p, int pass) {
    if (!p) return JA_ERR_NULL;
    if (p->batch < 1 || p->heads < 1) return JA_ERR_SHAPE;
    if (p->head_dim != 32 && p->head_dim != 64 && p->head_dim != 128) return JA_ERR_UNSUPPORTED;
    if (p->dtype != JA_BF16 && p->dtype != JA_F32) return JA_ERR_UNSUPPORTED;
    if (p->act < JA_ACT_SILU || p->act > JA_ACT_GELU_ERF) return JA_ERR_UNSUPPORTED;
    if (p->bias_kind < JA_BIAS_NONE || p->bias_kind > JA_BIAS_KEYPOS) return JA_ERR_UNSUPPORTED;
    if (p->causal != 0 && p->causal != 1) return JA_ERR_UNSUPPORTED;
    if (!p->kv_offsets) return JA_ERR_NULL;
    if (p->total_q < 0 || p->total_k < 0 || p->total_q > INT_MAX || p->total_k > INT_MAX) return JA_ERR_SHAPE;
    if (!p->q_offsets) {
        if (pass != JA_PASS_FWD) return JA_ERR_UNSUPPORTED;
        if (p->lq_fixed < 0 || p->total_q != p->lq_fixed) return JA_ERR_SHAPE;
        if ((int64_t)p->lq_fixed * p->batch > INT_MAX) return JA_ERR_SHAPE;
    }
    if (p->bias_kind != JA_BIAS_NONE) {
        if (!p->bias_table) return JA_ERR_NULL;
        if (p->bias_lo > p->bias_hi) return JA_ERR_SHAPE;
        if ((int64_t)p->bias_hi - p->bias_lo + 1 > (1 << 24)) return JA_ERR_SHAPE;
    }
    // The bias-gradient pass needs a table and keeps one row of it per wave in LDS.
    if (pass == JA_PASS_BWD_DBIAS && (p->bias_kind == JA_BIAS_NONE || bias_width(*p) > ja::DBIAS_MAX_BINS))
        return JA_ERR_UNSUPPORTED;
    if (!(p->scale == p->scale)) return JA_ERR_SHAPE;  // NaN scale
    if (p->max_kv_len < 0) return JA_ERR_SHAPE;
    if (p->window < 0) return JA_ERR_SHAPE;
    if (!(p->rope_base >= 0.0f) || std::isinf(p->rope_base)) return JA_ERR_SHAPE;  // NaN, negative, inf
    if (p->rope_inputs_turned != 0 && p->rope_inputs_turned != 1) return JA_ERR_SHAPE;
    // Kernels address a (sample, head) slice with 32-bit byte offsets; bounding
    // every [rows, H, D] tensor below 4 GiB bounds every slice (the sample
    // lengths themselves live on the device).
    const int64_t row_bytes = (int64_t)p->heads * p->head_dim * (p->dtype == JA_BF16 ? 2 : 4);
    const int64_t q_rows = total_q_out(*p) > p->total_q ? total_q_out(*p) : p->total_q;
    if (q_rows * row_bytes > (int64_t)UINT32_MAX || p->total_k * row_bytes > (int64_t)UINT32_MAX)
        return JA_ERR_UNSUPPORTED;
    // Work-unit counts (tiles x heads) must fit in int32.
    const Layout L = layout_of(*p, pass);
    const int64_t cap = L.cap_q > L.cap_k ? L.cap_q : L.cap_k;
    if (cap * p->heads > INT_MAX) return JA_ERR_SHAPE;
    if (total_q_out(*p) * p->heads > (int64_t)INT_MAX * 64) return JA_ERR_SHAPE;
    return JA_OK;
}

ja_status check_workspace(const ja_problem *p, int pass, void *ws, size_t bytes) {
    if (!ws || (reinterpret_cast<uintptr_t>(ws) % ALIGN) != 0) return JA_ERR_WORKSPACE;
    if (bytes < layout_of(*p, pass).total) return JA_ERR_WORKSPACE;
    return JA_OK;
}

ja::AttnParams base_params(const ja_problem &p, const Layout &L, void *ws) {
    ja::AttnParams a{};
    char *w = static_cast<char *>(ws);
    a.q_off = p.q_offsets;
    a.kv_off = p.kv_offsets;
    a.lq_fixed = p.lq_fixed;
    a.B = p.batch;
    a.H = p.heads;
    a.total_q_out = total_q_out(p);
    a.total_q = p.total_q;
    a.total_k = p.total_k;
    a.scale = p.scale;
    a.causal = p.causal;
    a.window = eff_window(p);
    a.bias_kind = p.bias_kind;
    a.bias_lo = p.bias_lo;
    a.bias_hi = p.bias_hi;
    a.bias = p.bias_kind != JA_BIAS_NONE ? p.bias_table : nullptr;
    if (a.bias == nullptr) a.bias_kind = JA_BIAS_NONE;
    auto *ctr = reinterpret_cast<ja::PlanCounters *>(w + L.counters);
    a.counters = ctr;
    a.counters2 = ctr + 1;
    a.counters3 = ctr + 2;
    a.counters4 = ctr + 3;
    a.tiles = reinterpret_cast<const int2 *>(w + L.tiles_q);
    a.tiles2 = reinterpret_cast<const int2 *>(w + L.tiles_k);
    a.tiles3 = reinterpret_cast<const int2 *>(w + L.tiles_s);
    a.tiles4 = reinterpret_cast<const int2 *>(w + L.tiles_a);
    a.delta = reinterpret_cast<float *>(w + L.delta);
    a.dbias_part = reinterpret_cast<float *>(w + L.dbias_part);
    return a;
}

ja::PlanParams plan_of(const ja_problem &p, int kind, int tile_rows, int inner_rows, int only_short,
                       const int2 *tiles, int64_t cap, ja::PlanCounters *ctr) {
    ja::PlanParams q{};
    q.q_off = p.q_offsets;
    q.kv_off = p.kv_offsets;
    q.lq_fixed = p.lq_fixed;
    q.B = p.batch;
    q.H = p.heads;
    q.causal = p.causal;
    q.window = eff_window(p);
    q.kind = kind;
    q.tile_rows = tile_rows;
    q.inner_rows = inner_rows;
    q.only_short = only_short;
    q.tiles = const_cast<int2 *>(tiles);
    q.max_tiles = (int)cap;
    q.counters = ctr;
    return q;
}

// Rotary embedding: turn q and k into the workspace copies (sign +1) and point
// the attention parameters at them, or turn dq and dk back in place (sign -1);
// with_q false turns the k segment only.
hipError_t rope_turn(const ja_problem &p, const void *q_src, void *q_dst, const void *k_src, void *k_dst,
                     float sign, int timer_id, hipStream_t s, bool with_q = true) {
    ja::RopeParams r{};
    r.seg[0] = ja::RopeSeg{q_src, q_dst, p.q_offsets, with_q ? p.total_q : 0, p.batch};
    r.seg[1] = ja::RopeSeg{k_src, k_dst, p.kv_offsets, p.total_k, p.batch};
    r.H = p.heads;
    r.sign = sign;
    const double base = (double)p.rope_base;
    for (int d = 0; d < p.head_dim / 2; ++d) r.inv_freq[d] = std::pow(base, -2.0 * d / p.head_dim);
    return ja::launch_rope(r, p.head_dim, p.dtype == JA_F32, timer_id, s);
}

// Frequencies of the turn in turns per position, base^(-2d/D) / (2 pi), for the
// backward units' turn-back.
void rope_frequencies(const ja_problem &p, ja::AttnParams &a) {
    const double base = (double)p.rope_base;
    const double two_pi = 6.283185307179586;  // nearest double to 2 pi
    for (int d = 0; d < p.head_dim / 2; ++d) a.rope_rev[d] = std::pow(base, -2.0 * d / p.head_dim) / two_pi;
}

hipError_t rope_inputs(const ja_problem &p, const Layout &L, void *ws, ja::AttnParams &a, hipStream_t s) {
    if (!(p.rope_base > 0.0f) || p.rope_inputs_turned) return hipSuccess;
    char *w = static_cast<char *>(ws);
    void *qr = w + L.rope_q, *kr = w + L.rope_k;
    const hipError_t e = rope_turn(p, a.q, qr, a.k, kr, 1.0f, ja::K_ROPE, s);
    a.q = qr;
    a.k = kr;
    return e;
}

ja_status hip_status(hipError_t e) {
    if (e == hipSuccess) return JA_OK;
    g_last_hip_error = (int)e;
    return JA_ERR_HIP;
}

// Opt-in offsets validation (environment JA_CHECK_OFFSETS=1): a device kernel
// checks the offsets and the call waits for its verdict before launching
// anything else.  JA_ERR_BAD_OFFSETS when they break the layout rules.
bool check_offsets_asked() {
    const char *e = std::getenv("JA_CHECK_OFFSETS");
    return e && e[0] == '1' && e[1] == '\0';
}

ja_status check_offsets(const ja_problem &p, const Layout &L, void *ws, hipStream_t s) {
    if (!check_offsets_asked()) return JA_OK;
    auto *ctr = reinterpret_cast<ja::PlanCounters *>(static_cast<char *>(ws) + L.counters);
    ja::OffsetsCheck c{p.q_offsets, p.kv_offsets, p.batch, p.q_offsets ? p.total_q : 0, p.total_k,
                       p.max_kv_len, &ctr->flag};
    hipError_t e = ja::launch_check_offsets(c, s);
    int bad = 1;
    if (e == hipSuccess) e = hipMemcpyAsync(&bad, &ctr->flag, sizeof(int), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e);
    return bad ? JA_ERR_BAD_OFFSETS : JA_OK;
}

// MXFP8 scale codes of q, k, v (all NULL: bf16 / fp32 inputs).
struct MXScales {
    const void *q, *k, *v;
};

ja_status run_fwd(const ja_problem *p, int mode, const void *q, const void *k, const void *v, void *o, float *lse,
                  void *o_res, void *ws, size_t ws_bytes, void *stream, const MXScales *mx = nullptr) {
    ja_status st = check_problem(p, JA_PASS_FWD);
    if (st != JA_OK) return st;
    // MXFP8 inputs: bf16 outputs, no rotary embedding (the turn works on bf16 / fp32 rows)
    if (mx && (p->dtype != JA_BF16 || p->rope_base > 0.0f)) return JA_ERR_UNSUPPORTED;
    // A tensor with no rows is never touched, so its pointer may be NULL.
    const bool has_q = p->total_q > 0, has_o = total_q_out(*p) > 0, has_k = p->total_k > 0;
    if ((has_q && !q) || (has_k && (!k || !v)) || (has_o && !o)) return JA_ERR_NULL;
    if (mx && ((has_q && !mx->q) || (has_k && (!mx->k || !mx->v)))) return JA_ERR_NULL;
    if (mode == 1 && has_o && !lse) return JA_ERR_NULL;
    st = check_workspace(p, JA_PASS_FWD, ws, ws_bytes);
    if (st != JA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Layout L = layout_of(*p, JA_PASS_FWD);
    st = check_offsets(*p, L, ws, s);
    if (st != JA_OK) return st;
    ja::AttnParams a = base_params(*p, L, ws);
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = o;
    a.lse = lse;
    a.o_res_out = p->dtype == JA_BF16 ? o_res : nullptr;
    if (mx) {
        a.q_sc = static_cast<const uint8_t *>(mx->q);
        a.k_sc = static_cast<const uint8_t *>(mx->k);
        a.v_sc = static_cast<const uint8_t *>(mx->v);
        a.mx = 1;
    }
    hipError_t e = rope_inputs(*p, L, ws, a, s);
    if (e != hipSuccess) return hip_status(e);
    if (p->dtype == JA_F32) return hip_status(ja::launch_fwd_f32(a, p->head_dim, mode, p->act, s));
    // two unit lists: query tiles of samples with more than 32 keys, and whole
    // (sample, head) units of samples with at most 32 keys
    a.tiles2 = a.tiles3;
    a.counters2 = a.counters3;
    // One shared block of at most 32 query rows (known here, since it is not
    // jagged): one-wave units over 32-row tiles instead of 4-wave 128-row ones.
    const bool few_q = p->q_offsets == nullptr && p->lq_fixed <= ja::FEW_Q_ROWS;
    const int q_tile = few_q ? ja::FEW_Q_ROWS : ja::Q_TILE, kv_tile = few_q ? ja::FEW_Q_KV_TILE : ja::KV_TILE;
    // The caller's bound on key counts may rule out every long-sequence unit.
    const bool long_units = !(p->max_kv_len > 0 && p->max_kv_len <= ja::FUSED_MAX_LK);
    ja::PlanParams pp[2] = {plan_of(*p, ja::PLAN_SAMPLES, 1, 32, 0, a.tiles3, L.cap_s, a.counters3),
                            plan_of(*p, ja::PLAN_Q_TILES, q_tile, kv_tile, 1, a.tiles, L.cap_q, a.counters)};
    e = ja::launch_plan(pp, long_units ? 2 : 1, s);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(ja::launch_fwd_bf16(a, p->head_dim, mode, p->act, cu_count(), few_q, long_units, s));
}

ja_status run_bwd(const ja_problem *p, int mode, const void *q, const void *k, const void *v, const void *o,
                  const void *o_res, const void *dout, const float *lse, void *dq, void *dk, void *dv, float *dbias,
                  void *ws, size_t ws_bytes, void *stream) {
    const int pass = dbias ? JA_PASS_BWD_DBIAS : JA_PASS_BWD;
    ja_status st = check_problem(p, pass);
    if (st != JA_OK) return st;
    // A tensor with no rows is never touched, so its pointer may be NULL.
    const bool has_q = p->total_q > 0, has_k = p->total_k > 0;
    if ((has_q && (!q || !dout || !dq)) || (has_k && (!k || !v || !dk || !dv))) return JA_ERR_NULL;
    if (mode == 1 && has_q && (!o || !lse)) return JA_ERR_NULL;
    st = check_workspace(p, pass, ws, ws_bytes);
    if (st != JA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Layout L = layout_of(*p, pass);
    st = check_offsets(*p, L, ws, s);
    if (st != JA_OK) return st;
    ja::AttnParams a = base_params(*p, L, ws);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dbias = dbias;
    a.o_res = p->dtype == JA_BF16 ? o_res : nullptr;
    a.dout = dout;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.lse = const_cast<float *>(lse);
    const bool rope = p->rope_base > 0.0f;
    hipError_t e = rope_inputs(*p, L, ws, a, s);
    if (e != hipSuccess) return hip_status(e);
    if (p->dtype == JA_F32) {  // the scalar kernels leave the turn-back to a pass
        e = ja::launch_bwd_f32(a, p->head_dim, mode, p->act, s);
        if (e == hipSuccess && rope) e = rope_turn(*p, dq, dq, dk, dk, -1.0f, ja::K_ROPE_BACK, s);
        return hip_status(e);
    }
    const bool long_units = !(p->max_kv_len > 0 && p->max_kv_len <= ja::FUSED_MAX_LK);
    ja::PlanParams pp[ja::PLAN_MAX];
    int n = 0;
    pp[n++] = plan_of(*p, ja::PLAN_SAMPLES, 1, 32, 0, a.tiles3, L.cap_s, a.counters3);
    if (long_units) {
        pp[n++] = plan_of(*p, ja::PLAN_Q_TILES, ja::Q_TILE, ja::KV_TILE, 1, a.tiles, L.cap_q, a.counters);
        pp[n++] = plan_of(*p, ja::PLAN_KV_TILES, ja::BWD_KV_UNIT, ja::BWD_Q_STEP, 1, a.tiles2, L.cap_k, a.counters2);
    }
    if (dbias) {
        // The dQ units fold the sums of their samples in (partial rows in unit
        // order, so their list must be a function of the offsets alone); the
        // separate pass takes the samples of the fused short-K/V units, or every
        // sample when no long unit runs.  Its summation order follows its list.
        if (long_units) {
            pp[1].stable = 1;
            a.dbias_slots = reinterpret_cast<float *>(static_cast<char *>(ws) + L.dbias_slots);
            a.dbias_chunks = reinterpret_cast<float *>(static_cast<char *>(ws) + L.dbias_chunks);
        }
        pp[n] = plan_of(*p, ja::PLAN_Q_TILES, ja::Q_TILE, ja::KV_TILE, long_units ? 2 : 0, a.tiles4, L.cap_q,
                        a.counters4);
        pp[n++].stable = 1;
    }
    e = ja::launch_plan(pp, n, s);
    if (e != hipSuccess) return hip_status(e);
    if (rope) {  // the dQ units turn their rows back before storing them
        a.rope_back = 1;
        rope_frequencies(*p, a);
    }
    e = ja::launch_bwd_bf16(a, p->head_dim, mode, p->act, 2 * cu_count(), long_units, s);
    if (e == hipSuccess && dbias) e = ja::launch_dbias_bf16(a, p->head_dim, mode, p->act, s);
    // dk, the gradient of the turned keys, is turned back by a pass
    if (e == hipSuccess && rope) e = rope_turn(*p, nullptr, nullptr, dk, dk, -1.0f, ja::K_ROPE_BACK, s, false);
    return hip_status(e);
}

// Built-in scratch of the no-allocation forward (jagged_attn_fwd_noalloc): the
// forward's workspace (plan counters and unit lists) lives in this device array,
// one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// its device address is looked up once per device and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[JA_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void *g_scratch[MAX_DEVICES];

// Device address of this device's scratch (looked up on the first call on it).
hipError_t scratch_ptr(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

const ja::KernelTimer &ja::kernel_timer() { return g_timer; }

extern "C" {

ja_status jagged_rope(const ja_problem *p, const void *q, const void *k, void *q_turned, void *k_turned,
                      void *stream) {
    ja_status st = check_problem(p, JA_PASS_FWD);
    if (st != JA_OK) return st;
    if (!(p->rope_base > 0.0f)) return JA_ERR_SHAPE;
    if ((p->total_q > 0 && (!q || !q_turned)) || (p->total_k > 0 && (!k || !k_turned))) return JA_ERR_NULL;
    return hip_status(rope_turn(*p, q, q_turned, k, k_turned, 1.0f, ja::K_ROPE, static_cast<hipStream_t>(stream)));
}

ja_status ja_profile_kernel(int kernel_id, void *start_event, void *stop_event) {
    if (kernel_id < JA_KERNEL_PLAN || kernel_id >= ja::K_COUNT) return JA_ERR_UNSUPPORTED;
    if ((start_event == nullptr) != (stop_event == nullptr)) return JA_ERR_NULL;
    g_timer.start[kernel_id] = static_cast<hipEvent_t>(start_event);
    g_timer.stop[kernel_id] = static_cast<hipEvent_t>(stop_event);
    return JA_OK;
}

ja_status ja_profile_busy(int kernel_id, void *device_buffer, int capacity) {
    if (kernel_id < JA_KERNEL_PLAN || kernel_id >= ja::K_COUNT) return JA_ERR_UNSUPPORTED;
    if ((device_buffer == nullptr) != (capacity == 0) || capacity < 0) return JA_ERR_SHAPE;
    g_timer.busy[kernel_id] = static_cast<uint64_t *>(device_buffer);
    g_timer.busy_cap[kernel_id] = capacity;
    return JA_OK;
}

size_t ja_workspace_size(const ja_problem *p, int pass) {
    if (pass != JA_PASS_FWD && pass != JA_PASS_BWD && pass != JA_PASS_BWD_DBIAS) return 0;
    if (check_problem(p, pass) != JA_OK) return 0;
    return layout_of(*p, pass).total;
}

ja_status jagged_gdpa_fwd(const ja_problem *p, const void *q, const void *k, const void *v, void *o, void *workspace,
                          size_t workspace_bytes, void *stream) {
    return run_fwd(p, 0, q, k, v, o, nullptr, nullptr, workspace, workspace_bytes, stream);
}

ja_status jagged_attn_fwd(const ja_problem *p, const void *q, const void *k, const void *v, void *o, float *lse,
                          void *o_residual, void *workspace, size_t workspace_bytes, void *stream) {
    return run_fwd(p, 1, q, k, v, o, lse, o_residual, workspace, workspace_bytes, stream);
}

ja_status jagged_gdpa_fwd_mx(const ja_problem *p, const void *q, const void *q_scale, const void *k,
                             const void *k_scale, const void *v, const void *v_scale, void *o, void *workspace,
                             size_t workspace_bytes, void *stream) {
    const MXScales mx{q_scale, k_scale, v_scale};
    return run_fwd(p, 0, q, k, v, o, nullptr, nullptr, workspace, workspace_bytes, stream, &mx);
}

ja_status jagged_attn_fwd_noalloc(const ja_problem *p, const void *q, const void *k, const void *v, void *o,
                                  float *lse, void *o_residual, void *stream) {
    ja_status st = check_problem(p, JA_PASS_FWD);
    if (st != JA_OK) return st;
    if (layout_of(*p, JA_PASS_FWD).total > JA_NOALLOC_SCRATCH_BYTES) return JA_ERR_WORKSPACE;
    void *ws = nullptr;
    const hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) return hip_status(e);
    return run_fwd(p, 1, q, k, v, o, lse, o_residual, ws, JA_NOALLOC_SCRATCH_BYTES, stream);
}

ja_status jagged_attn_fwd_mx(const ja_problem *p, const void *q, const void *q_scale, const void *k,
                             const void *k_scale, const void *v, const void *v_scale, void *o, float *lse,
                             void *o_residual, void *workspace, size_t workspace_bytes, void *stream) {
    const MXScales mx{q_scale, k_scale, v_scale};
    return run_fwd(p, 1, q, k, v, o, lse, o_residual, workspace, workspace_bytes, stream, &mx);
}

ja_status jagged_gdpa_bwd(const ja_problem *p, const void *q, const void *k, const void *v, const void *dout, void *dq,
                          void *dk, void *dv, float *dbias, void *workspace, size_t workspace_bytes, void *stream) {
    return run_bwd(p, 0, q, k, v, nullptr, nullptr, dout, nullptr, dq, dk, dv, dbias, workspace, workspace_bytes,
                   stream);
}

ja_status jagged_attn_bwd(const ja_problem *p, const void *q, const void *k, const void *v, const void *o,
                          const void *o_residual, const void *dout, const float *lse, void *dq, void *dk, void *dv,
                          float *dbias, void *workspace, size_t workspace_bytes, void *stream) {
    return run_bwd(p, 1, q, k, v, o, o_residual, dout, lse, dq, dk, dv, dbias, workspace, workspace_bytes, stream);
}

const char *ja_status_string(int status) {
    switch (status) {
    case JA_OK: return "ok";
    case JA_ERR_NULL: return "a required pointer is NULL";
    case JA_ERR_SHAPE: return "a size or range argument is out of range";
    case JA_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, activation, bias kind or pass, or a tensor of 4 GiB or more";
    case JA_ERR_WORKSPACE: return "workspace NULL, not 256-byte aligned, or too small";
    case JA_ERR_BAD_OFFSETS: return "offsets break the layout rules (found by the JA_CHECK_OFFSETS=1 validation)";
    case JA_ERR_HIP: return "a HIP launch failed";
    default: return "unknown status";
    }
}

int ja_last_hip_error(void) { return g_last_hip_error; }

int ja_version(void) { return 200; }

}  // extern "C"
