// Work-list planner: jagged offsets -> per-unit cost -> counting sort (most
// expensive first) -> list of (sample, tile) pairs + unit counter + cursor.
//
// Tile lists (query tiles, key tiles) are ordered sample by sample: samples
// by total cost, most expensive first, and each sample's tiles together, most
// expensive first.  The kernels number their units head-major over the list,
// so consecutive units are consecutive tiles of one (sample, head): the
// workgroups that pick them up at about the same time stream the same keys
// and values (or queries) and share them through the caches instead of each
// fetching them from HBM.  Whole-sample lists are ordered unit by unit.
//
// The pages report that naive jagged kernels leave compute units idle when
// short sequences finish early and that software tile scheduling turned a 6x
// imbalance into a near-balanced one ("GEM Training: How Meta Doubled the
// Efficiency...", section "What happened"; "Meta redesigns AI training
// infrastructure...", section "Custom Kernels and 5D Parallelism for
// Trillion-Parameter Scale").  Here the balancing is longest-first greedy
// dispatch: the persistent attention kernels pull units in this order from an
// atomic cursor, so every workgroup takes the most expensive unit left.
//
// One workgroup of 1024 threads; all state in LDS.  The list only orders the
// work: every output tile is owned by exactly one unit, so the attention
// results do not depend on the order or on which workgroup runs a unit.  The
// tile lists are nevertheless a pure function of the offsets (ties in cost keep
// sample order), since the bias-table gradient's summation order follows them.
#include "ja_device.h"
#include "ja_kernels.h"

namespace ja {

constexpr int PLAN_THREADS = 1024;
constexpr int PLAN_BUCKETS = 2048;

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

struct PlanSample {
    int lq, lk, ntiles;
};

__device__ __forceinline__ bool skipped_as_short(const PlanParams &p, int lk) {
    return p.only_short && lk <= FUSED_MAX_LK;
}

__device__ PlanSample plan_sample(const PlanParams &p, int b) {
    PlanSample s;
    s.lq = p.q_off ? p.q_off[b + 1] - p.q_off[b] : p.lq_fixed;
    s.lk = p.kv_off[b + 1] - p.kv_off[b];
    s.lq = s.lq < 0 ? 0 : s.lq;
    s.lk = s.lk < 0 ? 0 : s.lk;
    if (p.kind == PLAN_Q_TILES) {
        s.ntiles = skipped_as_short(p, s.lk) ? 0 : ceil_div(s.lq, p.tile_rows);
    } else if (p.kind == PLAN_KV_TILES) {
        s.ntiles = skipped_as_short(p, s.lk) ? 0 : ceil_div(s.lk, p.tile_rows);
    } else {
        s.ntiles = (s.lk <= FUSED_MAX_LK && (s.lq > 0 || s.lk > 0)) ? 1 : 0;
    }
    return s;
}

// Cost of tile t of a sample, in inner-loop steps (+1 for the unit's own
// loads and stores).
__device__ int tile_cost(const PlanParams &p, const PlanSample &s, int t) {
    if (p.kind == PLAN_Q_TILES) {
        int last = (t + 1) * p.tile_rows;
        last = (last < s.lq ? last : s.lq) - 1;
        const int kend = key_end(last, s.lq, s.lk, p.causal, p.window);
        const int kbeg = key_begin(t * p.tile_rows, s.lq, s.lk, p.window) / p.inner_rows * p.inner_rows;
        return ceil_div(kend > kbeg ? kend - kbeg : 0, p.inner_rows) + 1;
    }
    if (p.kind == PLAN_KV_TILES) {
        // query rows that see some key of the tile (aligned position ia = i + lk - lq)
        const int shift = s.lk - s.lq, j0 = t * p.tile_rows, w = p.window;
        int first_q = p.causal ? j0 - shift : (w ? j0 - w - shift + 1 : 0);
        first_q = first_q < 0 ? 0 : first_q;
        int end_q = w ? j0 + p.tile_rows - 1 + w - shift : s.lq;
        end_q = end_q > s.lq ? s.lq : end_q;
        const int nq = end_q - first_q;
        return ceil_div(nq > 0 ? nq : 0, p.inner_rows) + 1;
    }
    return ceil_div(s.lq, p.inner_rows) + 1;
}

__device__ __forceinline__ int bucket_of(int cost) {
    cost = cost < PLAN_BUCKETS - 1 ? cost : PLAN_BUCKETS - 1;
    return PLAN_BUCKETS - 1 - cost;  // ascending bucket = descending cost
}

// Bucket of a whole sample's cost on a logarithmic scale (32 steps per
// octave), so any total up to 2^31 fits the histogram; descending cost.
__device__ __forceinline__ int sample_bucket_of(int64_t cost) {
    if (cost < 1) cost = 1;
    if (cost > 0x7fffffff) cost = 0x7fffffff;
    const uint32_t c = (uint32_t)cost;
    const int l = 31 - __builtin_clz(c);
    const int frac = l >= 5 ? (int)((c >> (l - 5)) & 31u) : (int)((c << (5 - l)) & 31u);
    return PLAN_BUCKETS - 1 - (l * 32 + frac);
}

__device__ __forceinline__ bool grouped(const PlanParams &p) { return p.kind != PLAN_SAMPLES; }

// Cost of a whole sample for ordering the tile lists: its valid (query, key)
// pairs, in closed form (a sum over rows of the clamped causal key counts),
// so a sample with many tiles is not walked tile by tile.
__device__ int64_t sample_cost(const PlanParams &p, const PlanSample &s) {
    const int64_t lq = s.lq, lk = s.lk;
    if (p.window) {  // an estimate: rows times the keys a full window holds
        const int64_t span = p.causal ? p.window : 2 * (int64_t)p.window - 1;
        return lq * (span < lk ? span : lk);
    }
    if (!p.causal) return lq * lk;
    // row i sees clamp(i + lk - lq + 1, 0, lk) keys
    auto tri = [](int64_t n) { return n * (n + 1) / 2; };  // 1 + ... + n
    const int64_t i0 = lq - lk > 0 ? lq - lk : 0;              // first row that sees a key
    const int64_t n = lq - i0;                                  // rows that see keys: counts lk - n + 1 .. lk
    return n > 0 ? tri(lk) - tri(lk - n) : 0;
}

// Emit a sample's tiles in non-increasing cost order without evaluating the
// costs: causal query tiles get dearer with t, causal key tiles cheaper, and
// without causal masking every tile of a sample costs the same.
template <class F>
__device__ void for_each_tile_desc(const PlanParams &p, const PlanSample &s, F fn) {
    const bool descending = p.causal && p.kind == PLAN_Q_TILES;
    for (int k = 0; k < s.ntiles; ++k) fn(descending ? s.ntiles - 1 - k : k);
}

// Visit the tiles of a sample as runs of equal cost, in non-increasing cost
// order: fn(first_tile, count, step, cost).
template <class F>
__device__ void for_each_run(const PlanParams &p, const PlanSample &s, F fn) {
    if (s.ntiles == 0) return;
    // causal query tiles get dearer with t; causal key tiles get cheaper.
    const bool descending = p.causal && p.kind == PLAN_Q_TILES;
    const int step = descending ? -1 : 1;
    int t = descending ? s.ntiles - 1 : 0;
    int left = s.ntiles;
    while (left > 0) {
        const int cost = tile_cost(p, s, t);
        int n = 1;
        if (p.causal) {
            while (n < left && tile_cost(p, s, t + n * step) == cost) ++n;
        } else {
            n = left;  // every tile of a sample costs the same without causal masking
        }
        fn(t, n, step, cost);
        t += n * step;
        left -= n;
    }
}

__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(const PlanBatch batch) {
    const PlanParams &p = batch.list[blockIdx.x];
    __shared__ int hist[PLAN_BUCKETS];
    __shared__ int wave_tot[PLAN_THREADS / WAVE];
    __shared__ int s_total;
    const int tid = threadIdx.x;
    for (int i = tid; i < PLAN_BUCKETS; i += PLAN_THREADS) hist[i] = 0;
    __syncthreads();

    for (int b = tid; b < p.B; b += PLAN_THREADS) {
        const PlanSample s = plan_sample(p, b);
        if (grouped(p)) {
            if (s.ntiles > 0) atomicAdd(&hist[sample_bucket_of(sample_cost(p, s))], s.ntiles);
        } else {
            for_each_run(p, s, [&](int, int n, int, int cost) { atomicAdd(&hist[bucket_of(cost)], n); });
        }
    }
    __syncthreads();

    // Exclusive scan of the histogram: thread tid owns buckets 2 tid, 2 tid + 1.
    const int a = hist[2 * tid], c = hist[2 * tid + 1];
    int incl = a + c;
    const int lane = tid & (WAVE - 1), wv = tid / WAVE;
    for (int d = 1; d < WAVE; d <<= 1) {
        const int o = __shfl_up(incl, d, WAVE);
        if (lane >= d) incl += o;
    }
    if (lane == WAVE - 1) wave_tot[wv] = incl;
    __syncthreads();
    if (wv == 0) {
        int x = lane < PLAN_THREADS / WAVE ? wave_tot[lane] : 0;
        for (int d = 1; d < PLAN_THREADS / WAVE; d <<= 1) {
            const int o = __shfl_up(x, d, WAVE);
            if (lane >= d) x += o;
        }
        if (lane < PLAN_THREADS / WAVE) wave_tot[lane] = x;  // inclusive over waves
    }
    __syncthreads();
    const int excl = incl - (a + c) + (wv > 0 ? wave_tot[wv - 1] : 0);
    if (tid == PLAN_THREADS - 1) s_total = excl + a + c;
    __syncthreads();
    hist[2 * tid] = excl;
    hist[2 * tid + 1] = excl + a;
    __syncthreads();

    if (grouped(p)) {
        // Stable placement: within a cost bucket, samples keep their index order,
        // so the list is a function of the offsets alone.  Samples are taken in
        // chunks of PLAN_THREADS (one per thread) and the chunk's waves in turn;
        // inside a wave, lanes sharing a bucket get their positions from a prefix
        // sum of their tile counts, one distinct bucket at a time.
        for (int c0 = 0; c0 < p.B; c0 += PLAN_THREADS) {
            const int b = c0 + tid;
            const PlanSample s = b < p.B ? plan_sample(p, b) : PlanSample{0, 0, 0};
            const int bk = s.ntiles > 0 ? sample_bucket_of(sample_cost(p, s)) : -1;
            int pos = 0;
            for (int w = 0; w < PLAN_THREADS / WAVE; ++w) {
                if (wv == w) {
                    uint64_t todo = __builtin_amdgcn_ballot_w64(bk >= 0);
                    while (todo) {
                        const int leader = __builtin_ctzll(todo);
                        const int key = __shfl(bk, leader, WAVE);
                        const bool mine = bk == key;
                        int incl = mine ? s.ntiles : 0;
                        for (int d = 1; d < WAVE; d <<= 1) {
                            const int o = __shfl_up(incl, d, WAVE);
                            if (lane >= d) incl += o;
                        }
                        const int base = hist[key];  // read by every lane before the update below
                        if (mine) pos = base + incl - s.ntiles;
                        const int total = __shfl(incl, WAVE - 1, WAVE);
                        if (lane == leader) hist[key] = base + total;
                        todo &= ~__builtin_amdgcn_ballot_w64(mine);
                    }
                }
                __syncthreads();
            }
            if (bk >= 0)
                for_each_tile_desc(p, s, [&](int t) {
                    if (pos < p.max_tiles) p.tiles[pos] = make_int2(b, t);
                    ++pos;
                });
        }
    } else {
        for (int b = tid; b < p.B; b += PLAN_THREADS) {
            const PlanSample s = plan_sample(p, b);
            for_each_run(p, s, [&](int t0, int n, int step, int cost) {
                const int pos = atomicAdd(&hist[bucket_of(cost)], n);
                for (int k = 0; k < n; ++k)
                    if (pos + k < p.max_tiles) p.tiles[pos + k] = make_int2(b, t0 + k * step);
            });
        }
    }
    if (tid == 0) {
        const int n = s_total < p.max_tiles ? s_total : p.max_tiles;
        p.counters->units = n * p.H;
        p.counters->cursor = 0;
    }
    if (tid < XCDS) p.counters->xcursor[tid][0] = 0;
}

// Offsets validation (opt-in): q_offsets (when given) and kv_offsets must start
// at 0, never decrease and end at the row counts; with a key-count bound every
// sample's key count must respect it.  One workgroup; writes 1 to *flag when
// anything is wrong, else 0.
__global__ __launch_bounds__(PLAN_THREADS) void check_offsets_kernel(const OffsetsCheck c) {
    __shared__ int bad;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    int mine = 0;
    if (threadIdx.x == 0) {
        if (c.q_off && (c.q_off[0] != 0 || (int64_t)c.q_off[c.B] != c.total_q)) mine = 1;
        if (c.kv_off[0] != 0 || (int64_t)c.kv_off[c.B] != c.total_k) mine = 1;
    }
    for (int b = threadIdx.x; b < c.B; b += PLAN_THREADS) {
        const int lk = c.kv_off[b + 1] - c.kv_off[b];
        if (lk < 0 || (c.max_kv_len > 0 && lk > c.max_kv_len)) mine = 1;
        if (c.q_off && c.q_off[b + 1] < c.q_off[b]) mine = 1;
    }
    if (mine) bad = 1;  // any writer stores the same value
    __syncthreads();
    if (threadIdx.x == 0) *c.flag = bad;
}

hipError_t launch_check_offsets(const OffsetsCheck &c, hipStream_t stream) {
    const KernelTimer &t = kernel_timer();
    t.begin(K_CHECK_OFFSETS, stream);
    hipLaunchKernelGGL(check_offsets_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, c);
    t.end(K_CHECK_OFFSETS, stream);
    return hipGetLastError();
}

hipError_t launch_plan(const PlanParams *lists, int n, hipStream_t stream) {
    if (n < 1 || n > PLAN_MAX) return hipErrorInvalidValue;
    PlanBatch batch{};
    for (int i = 0; i < n; ++i) batch.list[i] = lists[i];
    const KernelTimer &t = kernel_timer();
    t.begin(K_PLAN, stream);
    hipLaunchKernelGGL(plan_kernel, dim3(n), dim3(PLAN_THREADS), 0, stream, batch);
    t.end(K_PLAN, stream);
    return hipGetLastError();
}

}  // namespace ja
