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
// One workgroup of 1024 threads per list; all state in LDS.  The list only
// orders the work: every output tile is owned by exactly one unit, so the
// attention results do not depend on the order or on which workgroup runs a
// unit, and samples of equal cost take their places by LDS atomics.  The list
// of the bias-table gradient is the exception (PlanParams::stable): its
// summation order follows the list, so there ties in cost keep sample order, by
// a stable radix sort of each chunk of samples, and the list is a function of
// the offsets alone.
#include "ja_device.h"
#include "ja_kernels.h"

namespace ja {

constexpr int PLAN_THREADS = 1024;
constexpr int PLAN_BUCKETS = 2048;

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

struct PlanSample {
    int lq, lk, ntiles;
};

__device__ __forceinline__ bool skipped_by_length(const PlanParams &p, int lk) {
    return p.only_short == 2 ? lk > FUSED_MAX_LK : (p.only_short && lk <= FUSED_MAX_LK);
}

__device__ PlanSample plan_sample(const PlanParams &p, int b) {
    PlanSample s;
    s.lq = p.q_off ? p.q_off[b + 1] - p.q_off[b] : p.lq_fixed;
    s.lk = p.kv_off[b + 1] - p.kv_off[b];
    s.lq = s.lq < 0 ? 0 : s.lq;
    s.lk = s.lk < 0 ? 0 : s.lk;
    if (p.kind == PLAN_Q_TILES) {
        s.ntiles = skipped_by_length(p, s.lk) ? 0 : ceil_div(s.lq, p.tile_rows);
    } else if (p.kind == PLAN_KV_TILES) {
        s.ntiles = skipped_by_length(p, s.lk) ? 0 : ceil_div(s.lk, p.tile_rows);
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

// Exclusive prefix sum of v over the workgroup's threads (in thread order);
// *total receives the sum.  Every thread must call it (it synchronises).
__device__ int block_scan_excl(int v, int *wave_tot, int *total) {
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    int incl = v;
    for (int d = 1; d < WAVE; d <<= 1) {
        const int o = __shfl_up(incl, d, WAVE);
        if (lane >= d) incl += o;
    }
    __syncthreads();  // wave_tot free for reuse
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
    *total = wave_tot[PLAN_THREADS / WAVE - 1];
    return incl - v + (wv > 0 ? wave_tot[wv - 1] : 0);
}

// Stable sort of one key per thread (keys below 4096) by a least-significant-
// digit radix sort in LDS, three passes of 4 bits: on return key[k], id[k] hold
// the k-th smallest key and the thread that contributed it, equal keys in
// thread order.  Each pass ranks a thread's digit within its wave by ballots
// and across waves and digits by one prefix sum over the (digit, wave) counts.
struct SortSpace {
    int key[2][PLAN_THREADS], id[2][PLAN_THREADS];
    int cnt[16 * (PLAN_THREADS / WAVE)];  // (digit, wave) counts, digit-major, then their offsets
};
__device__ void block_sort12(int my_key, SortSpace &sp, int *wave_tot) {
    constexpr int NW = PLAN_THREADS / WAVE;
    static_assert(16 * NW <= PLAN_THREADS, "one (digit, wave) count per thread");
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    const uint64_t lt = lane ? (~0ull >> (WAVE - lane)) : 0ull;  // lanes below this one
    int k = my_key, me = tid, buf = 0;
    for (int shift = 0; shift < 12; shift += 4) {
        const int dig = (k >> shift) & 15;
        int rank = 0;
        for (int d = 0; d < 16; ++d) {
            const uint64_t m = __builtin_amdgcn_ballot_w64(dig == d);
            if (dig == d) rank = __builtin_popcountll(m & lt);
            if (lane == d) sp.cnt[d * NW + wv] = __builtin_popcountll(m);
        }
        __syncthreads();
        int total;
        const int c = tid < 16 * NW ? sp.cnt[tid] : 0;
        const int off = block_scan_excl(c, wave_tot, &total);
        if (tid < 16 * NW) sp.cnt[tid] = off;
        __syncthreads();
        const int dst = sp.cnt[dig * NW + wv] + rank;
        sp.key[buf][dst] = k;
        sp.id[buf][dst] = me;
        __syncthreads();
        k = sp.key[buf][tid];
        me = sp.id[buf][tid];
        buf ^= 1;
        __syncthreads();  // counts and this buffer are reused by the next pass
    }
    sp.key[0][tid] = k;
    sp.id[0][tid] = me;
    __syncthreads();
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

    if (grouped(p) && !p.stable) {
        for (int b = tid; b < p.B; b += PLAN_THREADS) {
            const PlanSample s = plan_sample(p, b);
            if (s.ntiles == 0) continue;
            int pos = atomicAdd(&hist[sample_bucket_of(sample_cost(p, s))], s.ntiles);
            for_each_tile_desc(p, s, [&](int t) {
                if (pos < p.max_tiles) p.tiles[pos] = make_int2(b, t);
                ++pos;
            });
        }
    } else if (grouped(p)) {
        // Stable placement: within a cost bucket, samples keep their index order,
        // so the list is a function of the offsets alone.  Samples are taken in
        // chunks of PLAN_THREADS (one per thread): the chunk is sorted by bucket,
        // stably, and each sample's position is its bucket's running start plus the
        // tiles of the bucket's earlier samples (a prefix sum in sorted order).
        __shared__ SortSpace sp;
        __shared__ int s_nt[PLAN_THREADS];
        __shared__ int s_seg[PLAN_BUCKETS + 1];
        for (int c0 = 0; c0 < p.B; c0 += PLAN_THREADS) {
            const int b = c0 + tid;
            const PlanSample s = b < p.B ? plan_sample(p, b) : PlanSample{0, 0, 0};
            const int bk = s.ntiles > 0 ? sample_bucket_of(sample_cost(p, s)) : PLAN_BUCKETS;  // none: last
            s_nt[tid] = s.ntiles;
            block_sort12(bk, sp, wave_tot);
            const int key = sp.key[0][tid], src = sp.id[0][tid];
            const int nt = s_nt[src];
            int total;
            const int excl = block_scan_excl(nt, wave_tot, &total);
            const bool head = tid == 0 || sp.key[0][tid - 1] != key;
            const bool tail = tid == PLAN_THREADS - 1 || sp.key[0][tid + 1] != key;
            if (head) s_seg[key] = excl;
            __syncthreads();
            const int pos0 = key < PLAN_BUCKETS ? hist[key] + excl - s_seg[key] : 0;
            __syncthreads();  // every thread has read its bucket's start
            if (tail && key < PLAN_BUCKETS) hist[key] += excl + nt - s_seg[key];
            if (key < PLAN_BUCKETS) {
                const PlanSample t = plan_sample(p, c0 + src);
                int pos = pos0;
                for_each_tile_desc(p, t, [&](int tt) {
                    if (pos < p.max_tiles) p.tiles[pos] = make_int2(c0 + src, tt);
                    ++pos;
                });
            }
            __syncthreads();  // hist, s_nt and the sort space are reused by the next chunk
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
