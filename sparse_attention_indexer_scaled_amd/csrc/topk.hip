// Row-wise top-k over indexer logits (gfx950).
//
// The consumer of the indexer is a top-k over each logits row (index_topk of
// 2048 or 512 on the pages: aiter PR 5047 page, "Integration" and the
// end-to-end serving notes; the issue page about next_n tiling, "Setup").  The
// pages do not define the selection, so this kernel implements one total
// order: entries are ranked by value, larger first, equal values by smaller
// column first; -inf and NaN entries (positions outside a row's window) are
// never selected; -0.0 ranks equal to +0.0.  Row r's output is the first
// min(k, #selectable) columns of that order, then -1.
//
// One workgroup (16 waves) per row.  Values map to 32-bit keys whose unsigned
// order is the value order (key 0 = not selectable); an entry is the key in
// the high word and ~column in the low word, so entry order is the output
// order.  Every path ends with at most kSortCap entries in LDS that contain
// the row's top k, and a sort of them: a bucket sort over the key range
// (linear work) unless some bucket is crowded, else a bitonic sort.
//
//  1. Rows of at most kSortCap columns: gather every listable entry.
//  2. Longer rows: a threshold from a sample of kSample entries (256 runs of
//     16 adjacent columns), aimed at ~1.25 k survivors; one pass keeps every
//     entry at or above it.  If between k and kSortCap entries survive, they
//     hold the top k.
//  3. Otherwise an exact radix select over the key bits (12 + 12 + 8): each
//     pass histograms, in LDS, the keys that still share the threshold
//     prefix, until the bucket holding the k-th key has at most kCand
//     entries; then every key at or above that bucket is gathered.  A bucket
//     that is still larger after all 32 bits is one repeated key: its first
//     columns are taken in column order by a block-wide ordered compaction.
//
// Row reads are 16-byte loads, kUnroll per thread in flight: one workgroup
// streams a whole row, so the bytes in flight per CU set its read rate.
#include "device.h"
#include "launch.h"
#include "order_key.h"

#include <atomic>

namespace mqa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBins = 4096;              // 12-bit digits
constexpr int kSortCap = 8192;              // entries gathered into LDS and sorted
constexpr int kCand = kSortCap - kMaxTopK;  // largest bucket gathered (keys above it < k)
constexpr int kSample = 4096;               // entries sampled for the threshold
constexpr int kBucketMax = 32;              // largest bucket whose entries rank themselves
constexpr uint32_t kPosInfKey = 0xff800000u;  // order key of +inf
constexpr int kCrowdMax = 2 * kThreads;     // largest bucket ranked by the whole block
constexpr int kMaxCrowd = kSortCap / (kBucketMax + 1) + 1;  // crowded buckets at most
constexpr int kUnroll = 8;                  // 16-byte loads in flight per thread

static_assert(kSample == 4 * kThreads, "the sample is four entries per thread");
static_assert(kFusedSampleCols == kSample, "the fused sample fills one threshold sample");
static_assert(kSortCap <= 16 * kThreads, "the sort holds every gathered entry");

// Raise a kernel's dynamic LDS limit once per device.
hipError_t raise_lds_limit(const void *fn, int bytes, std::atomic<uint64_t> &raised)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const uint64_t bit = 1ull << (dev & 63);
    if (!(raised.load() & bit)) {
        e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        if (e != hipSuccess)
            return e;
        raised.fetch_or(bit);
    }
    return hipSuccess;
}

struct TopkShared {
    uint32_t hist[kMaxBins];
    uint64_t buf[kSortCap];
    uint64_t sorted[kSortCap];  // bucket sort output
    int count;                  // entries appended to buf (including any past its capacity)
    int wave_total[kWaves];
    int bcast[4];
    uint32_t kmin, kmax, maxb;
    int ncrowd;                     // buckets of kBucketMax < m <= kCrowdMax entries
    int crowd_start[kMaxCrowd];
    int crowd_m[kMaxCrowd];
};

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d, 64);
        if (lane >= d)
            v += o;
    }
    return v;
}

// The block finds the digit b such that  above + #(digits > b) < k <= above +
// #(digits >= b),  scanning nbins digits from the top: thread t first sums
// digits [nbins - (t+1) w, nbins - t w) with w = nbins / min(nbins, NT) (every
// thread of the block at once), a block scan finds the thread whose span holds
// b, and that thread's wave then scans the span one digit per lane.  Writes b,
// the new `above` and the bucket size to sh.bcast[0..2] (not written when
// above + total < k), and the total to bcast[3].  Every thread of the block
// calls it (it holds a barrier); the caller syncs before reading bcast.
template <int NT, class SH>
__device__ __forceinline__ void find_threshold(SH &sh, int nbins, int above, int k, int tid)
{
    constexpr int NW = NT / 64;
    const int lane = tid & 63, wave = tid >> 6;
    const int owners = min(nbins, NT);  // threads that own a span (powers of two)
    const int w = nbins / owners;
    const bool owner = tid < owners;
    const int hi = nbins - tid * w;  // exclusive upper digit of this thread's span
    int mine = 0;
    // lane l starts its span at offset l: neighbouring lanes read different banks
    if (owner)
        for (int j = 0; j < w; ++j)
            mine += (int)sh.hist[hi - w + ((j + lane) & (w - 1))];
    const int incl_w = wave_inclusive_scan(mine, lane);
    if (lane == 63)
        sh.wave_total[wave] = incl_w;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        const int c = sh.wave_total[v];
        before += v < wave ? c : 0;
        total += c;
    }
    const int incl = before + incl_w;
    const int excl = incl - mine;
    if (tid == 0)
        sh.bcast[3] = total;
    const uint64_t hit = __ballot(owner && above + excl < k && above + incl >= k);
    if (hit == 0ull)
        return;
    const int span = __ffsll((unsigned long long)hit) - 1;  // lane of this wave
    const int base = above + __shfl(excl, span, 64);
    const int d = nbins - (wave * 64 + span) * w - 1 - lane;  // lane j: the j-th digit from the top
    const int c = lane < w ? (int)sh.hist[d] : 0;
    const int run = base + wave_inclusive_scan(c, lane);  // keys with digit >= d
    const uint64_t reach = __ballot(lane < w && run >= k);
    if (lane == __ffsll((unsigned long long)reach) - 1) {
        sh.bcast[0] = d;
        sh.bcast[1] = run - c;
        sh.bcast[2] = c;
    }
}

template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int lane)
{
    if constexpr (M == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, false);
    } else if constexpr (M == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4e, 0xf, 0xf, false);
    } else if constexpr (M <= 16) {
        return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1f | (M << 10));
    } else {
        static_assert(M == 32, "lane exchange distance");
        // new a = (a_lo, b_lo), new b = (a_hi, b_hi) with a = b = v
        auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return lane < 32 ? r[1] : r[0];
    }
}

__device__ __forceinline__ uint64_t keep_side(uint64_t mine, uint64_t other, int e, int stride,
                                              int size)
{
    const bool want_max = ((e & stride) == 0) == ((e & size) == 0);
    return want_max ? (mine > other ? mine : other) : (mine < other ? mine : other);
}

constexpr int E = 16;  // entries each sorting thread holds

// Compare-exchange of a pair: after it, a >= b when desc, else a <= b.
// Selects, not a branch, so lanes never diverge.
__device__ __forceinline__ void cmpx(uint64_t &a, uint64_t &b, bool desc)
{
    const bool swap = (a < b) == desc;
    const uint64_t x = a, y = b;
    a = swap ? y : x;
    b = swap ? x : y;
}

// Compare-exchange at distance S < E: both entries are in this thread.
template <int S>
__device__ __forceinline__ void stage_thread(uint64_t (&v)[E], int tid, int size)
{
#pragma unroll
    for (int r = 0; r < E; ++r) {
        if (r & S)
            continue;
        cmpx(v[r], v[r + S], ((E * tid + r) & size) == 0);
    }
}

// Compare-exchange at distance M E: the partner is lane ^ M of this wave.
template <int M>
__device__ __forceinline__ void stage_lanes(uint64_t (&v)[E], int tid, int size, int lane)
{
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const uint32_t lo = xor_lane<M>((uint32_t)v[r], lane);
        const uint32_t hi = xor_lane<M>((uint32_t)(v[r] >> 32), lane);
        v[r] = keep_side(v[r], ((uint64_t)hi << 32) | lo, E * tid + r, M * E, size);
    }
}

// Bitonic sort of sh.buf[0, n2) into descending order (n2 a power of two, at
// most kSortCap; entries past n2 up to the next multiple of 64 E are sorted
// alongside and must hold padding).  The first max(n2 / E, 64) threads hold E
// consecutive entries each in registers: partners at distance < E are in the
// same thread, up to 32 E in the same wave (lane exchanges), and further ones
// go through LDS.
__device__ void sort_desc(TopkShared &sh, int n2, int tid, int lane)
{
    const bool act = tid < max(n2 / E, 64);  // whole waves
    uint64_t v[E];
    if (act) {
#pragma unroll
        for (int r = 0; r < E; ++r)
            v[r] = sh.buf[E * tid + r];
    }
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= 64 * E) {
                __syncthreads();
                if (act) {
#pragma unroll
                    for (int r = 0; r < E; ++r)
                        sh.buf[E * tid + r] = v[r];
                }
                __syncthreads();
                if (act) {
#pragma unroll
                    for (int r = 0; r < E; ++r) {
                        const int e = E * tid + r;
                        v[r] = keep_side(v[r], sh.buf[e ^ stride], e, stride, size);
                    }
                }
                continue;
            }
            if (!act)
                continue;
            switch (stride) {
            case 1: stage_thread<1>(v, tid, size); break;
            case 2: stage_thread<2>(v, tid, size); break;
            case 4: stage_thread<4>(v, tid, size); break;
            case 8: stage_thread<8>(v, tid, size); break;
            case E: stage_lanes<1>(v, tid, size, lane); break;
            case 2 * E: stage_lanes<2>(v, tid, size, lane); break;
            case 4 * E: stage_lanes<4>(v, tid, size, lane); break;
            case 8 * E: stage_lanes<8>(v, tid, size, lane); break;
            case 16 * E: stage_lanes<16>(v, tid, size, lane); break;
            default: stage_lanes<32>(v, tid, size, lane); break;
            }
        }
    }
    __syncthreads();
    if (act) {
#pragma unroll
        for (int r = 0; r < E; ++r)
            sh.buf[E * tid + r] = v[r];
    }
    __syncthreads();
}

// Bucket sort of sh.buf[0, n), descending; positions [0, min(n, k)) of the
// result are in sh.buf (sh.sorted is the scratch), and buckets that start at
// or past position k, whose entries are never output, are left unranked.  Keys are spread over kMaxBins buckets linearly in the
// value, bucket 0 holding the largest; a prefix sum places the buckets and
// the entries are scattered to them.  Then every entry of a bucket of up to
// kBucketMax entries finds its place by itself: the number of entries of its
// bucket above it (entries are distinct, as their columns are), so the work
// is spread over entries rather than buckets and no lane waits on another's
// large bucket.  Larger buckets (equal logits, such as the exact zeros of
// tokens whose head scores are all negative) are ranked by the whole block,
// one bucket at a time, the same way.  Linear work for spread-out keys, where
// a bitonic sort is n log^2 n.  Returns false, with sh.buf unchanged, when
// some bucket holds more than kCrowdMax entries; the caller then sorts
// sh.buf itself.
__device__ __forceinline__ bool bucket_sort(TopkShared &sh, int n, int k, int tid, int lane,
                                            int wave)
{
    if (tid == 0) {
        sh.kmin = 0xffffffffu;
        sh.kmax = 0u;
        sh.maxb = 0u;
        sh.ncrowd = 0;
    }
    for (int i = tid; i < kMaxBins; i += kThreads)
        sh.hist[i] = 0;
    __syncthreads();
    // key range over the finite values (+inf, key 0xff800000, goes to the
    // top bucket by itself)
    uint32_t lo = 0xffffffffu, hi = 0u;
    for (int i = tid; i < n; i += kThreads) {
        const uint32_t key = (uint32_t)(sh.buf[i] >> 32);
        lo = min(lo, key);
        if (key != kPosInfKey)
            hi = max(hi, key);
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, d, 64));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, d, 64));
    }
    if (lane == 0) {
        atomicMin(&sh.kmin, lo);
        atomicMax(&sh.kmax, hi);
    }
    __syncthreads();
    // Buckets are linear in the value, not in the key: keys are log-spaced,
    // so a key-linear map would crowd everything into few buckets whenever
    // the range also holds values near zero.  Double arithmetic: no overflow,
    // and the map stays monotone (correctly rounded subtraction and product).
    const double vmin = (double)key_value(max(sh.kmin, 0x00800000u));
    const double vmax = sh.kmax >= sh.kmin ? (double)key_value(max(sh.kmax, 0x00800000u)) : vmin;
    const double scale = vmax > vmin ? (double)(kMaxBins - 1) / (vmax - vmin) : 0.0;
    auto bucket_of = [&](uint64_t e) {
        const uint32_t key = (uint32_t)(e >> 32);
        if (key == kPosInfKey)
            return 0;
        const double t = ((double)key_value(key) - vmin) * scale;
        return kMaxBins - 1 - min((int)t, kMaxBins - 1);
    };
    for (int i = tid; i < n; i += kThreads)
        atomicAdd(&sh.hist[bucket_of(sh.buf[i])], 1u);
    __syncthreads();

    // exclusive prefix sum: thread t owns buckets 4t..4t+3
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        c[j] = sh.hist[4 * tid + j];
    const int mine = (int)(c[0] + c[1] + c[2] + c[3]);
    const int incl = wave_inclusive_scan(mine, lane);
    if (lane == 63)
        sh.wave_total[wave] = incl;
    uint32_t big = max(max(c[0], c[1]), max(c[2], c[3]));
#pragma unroll
    for (int d = 1; d < 64; d <<= 1)
        big = max(big, (uint32_t)__shfl_xor((int)big, d, 64));
    if (lane == 0)
        atomicMax(&sh.maxb, big);
    __syncthreads();
    int before = 0;
    for (int v = 0; v < wave; ++v)
        before += sh.wave_total[v];
    if (sh.maxb > (uint32_t)kCrowdMax)
        return false;  // uniform: every thread read the same maxb
    int run = before + incl - mine;
    int start[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        start[j] = run;
        sh.hist[4 * tid + j] = run;  // becomes the bucket's write cursor
        run += (int)c[j];
    }
    __syncthreads();
    for (int i = tid; i < n; i += kThreads) {
        const uint64_t e = sh.buf[i];
        sh.sorted[atomicAdd(&sh.hist[bucket_of(e)], 1u)] = e;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int m = (int)c[j];
        if (m > kBucketMax) {
            const int slot = atomicAdd(&sh.ncrowd, 1);
            sh.crowd_start[slot] = start[j];
            sh.crowd_m[slot] = m;
        }
    }
    // sh.hist[b] now holds the end of bucket b (its cursor after the scatter)
    for (int i = tid; i < n; i += kThreads) {
        const uint64_t e = sh.sorted[i];
        const int b = bucket_of(e);
        const int end = (int)sh.hist[b];
        const int st = b > 0 ? (int)sh.hist[b - 1] : 0;
        if (end - st > kBucketMax || st >= k)
            continue;  // ranked below by the whole block, or past the output
        // eight reads in flight per round (a dependent read per entry would
        // wait out the LDS latency each time)
        int r = 0;
        for (int j = st; j < end; j += 8) {
            uint64_t o[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                o[q] = sh.sorted[min(j + q, end - 1)];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                r += (j + q < end) && o[q] > e;
        }
        sh.buf[st + r] = e;
    }
    __syncthreads();
    const int ncrowd = sh.ncrowd;
    for (int cb = 0; cb < ncrowd; ++cb) {
        const int st = sh.crowd_start[cb], m = sh.crowd_m[cb];
        if (st >= k)
            continue;  // uniform: past the output
        const uint64_t e0 = tid < m ? sh.sorted[st + tid] : 0ull;
        const uint64_t e1 = tid + kThreads < m ? sh.sorted[st + tid + kThreads] : 0ull;
        int r0 = 0, r1 = 0;
        int j = 0;
        for (; j + 8 <= m; j += 8) {
            uint64_t o[8];  // same addresses in every lane: broadcasts, eight in flight
#pragma unroll
            for (int q = 0; q < 8; ++q)
                o[q] = sh.sorted[st + j + q];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                r0 += o[q] > e0;
                r1 += o[q] > e1;
            }
        }
        for (; j < m; ++j) {
            const uint64_t o = sh.sorted[st + j];
            r0 += o > e0;
            r1 += o > e1;
        }
        if (tid < m)
            sh.buf[st + r0] = e0;
        if (tid + kThreads < m)
            sh.buf[st + r1] = e1;
    }
    __syncthreads();
    return true;
}

// c ? a : b per component (a select of whole float4 objects can be lowered
// through scratch memory).
__device__ __forceinline__ float4 select4(bool c, float4 a, float4 b)
{
    return make_float4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

// Call f(v, c) for the row in groups of four columns: v holds columns
// c..c+3; past the row end v is padded with -inf, which no caller keeps.
// kUnroll 16-byte loads per thread are issued before any is used.
template <typename F>
__device__ __forceinline__ void for_each4(const float *x, int cols, int tid, F f)
{
    const float ninf = -__builtin_inff();
    int i0 = 0;
    if ((reinterpret_cast<uintptr_t>(x) & 15) == 0) {
        const int n4 = cols >> 2;
        const float4 *x4 = reinterpret_cast<const float4 *>(x);
        const float4 pad = make_float4(ninf, ninf, ninf, ninf);
        for (int b = tid; b < n4; b += kUnroll * kThreads) {
            float4 v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                // unconditional in-bounds load (index clamped), then select,
                // so the compiler keeps one 16-byte load per element
                const int i = b + u * kThreads;
                v[u] = select4(i < n4, x4[min(i, n4 - 1)], pad);
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int i = b + u * kThreads;
                if (i < n4)
                    f(v[u], 4 * i);
            }
        }
        i0 = 4 * n4;
    }
    for (int i = i0 + 4 * tid; i < cols; i += 4 * kThreads)
        f(make_float4(x[i], i + 1 < cols ? x[i + 1] : ninf, i + 2 < cols ? x[i + 2] : ninf,
                      i + 3 < cols ? x[i + 3] : ninf),
          i);
}

// Append the active lanes' kept entries to sh.buf with one LDS atomic per
// wave; every kept entry is counted in sh.count, entries past the capacity are
// dropped (the caller checks sh.count).
__device__ __forceinline__ void append(TopkShared &sh, bool keep, uint64_t e, int lane)
{
    const uint64_t active = __ballot(1);
    const uint64_t kept = __ballot(keep);
    if (kept == 0ull)
        return;
    const int leader = __ffsll((unsigned long long)active) - 1;
    int base = 0;
    if (lane == leader)
        base = atomicAdd(&sh.count, __popcll(kept));
    base = __shfl(base, leader, 64);
    const int pos = base + __popcll(kept & ((1ull << lane) - 1ull));
    if (keep && pos < kSortCap)
        sh.buf[pos] = e;
}

__device__ __forceinline__ void append4(TopkShared &sh, float4 v, int c, bool k0, bool k1, bool k2,
                                        bool k3, int lane)
{
    if (__ballot(k0 || k1 || k2 || k3) == 0ull)
        return;
    append(sh, k0, entry(order_key(v.x), c), lane);
    append(sh, k1, entry(order_key(v.y), c + 1), lane);
    append(sh, k2, entry(order_key(v.z), c + 2), lane);
    append(sh, k3, entry(order_key(v.w), c + 3), lane);
}

// One batch of the filter pass on a 16-byte aligned row: groups b + u kThreads
// (columns 4 i .. 4 i + 3), u < kUnroll.  Groups past the row end (i >= n4 =
// cols / 4 >= 1) read the last group again, and the caller drops them by
// index: nothing here consumes the loads, so the first batch, requested
// before the sampling, is only waited for by the filter pass.
__device__ __forceinline__ void load_batch(const float *x, int n4, int b, float4 (&v)[kUnroll])
{
    const float4 *x4 = reinterpret_cast<const float4 *>(x);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
        v[u] = x4[min(b + u * kThreads, n4 - 1)];
}

// Append every entry >= f0 (a finite value) to sh.buf, counting them all in
// sh.count.  Each wave loads kUnroll 16-byte groups per thread, then takes one
// LDS atomic for all of their survivors: lane offsets come from the ballots
// of the four components, so no lane exchange is needed.  On an aligned row
// `first` holds the thread's first batch (load_batch at b = tid).
template <bool ALIGNED>
__device__ void filter_pass(TopkShared &sh, const float *x, int cols, float f0, int tid, int lane,
                            const float4 (&first)[kUnroll])
{
    const uint64_t lt = (1ull << lane) - 1ull;
    auto emit = [&](const float4 (&v)[kUnroll], const int (&col)[kUnroll],
                    const bool (&ok)[kUnroll]) {
        int total = 0;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            total += __popcll(__ballot(ok[u] && v[u].x >= f0)) +
                     __popcll(__ballot(ok[u] && v[u].y >= f0)) +
                     __popcll(__ballot(ok[u] && v[u].z >= f0)) +
                     __popcll(__ballot(ok[u] && v[u].w >= f0));
        if (total == 0)
            return;
        const uint64_t active = __ballot(1);
        int base = 0;
        if (lane == __ffsll((unsigned long long)active) - 1)
            base = atomicAdd(&sh.count, total);
        base = __builtin_amdgcn_readfirstlane(base);
        auto put = [&](bool keep, float f, int c) {
            const uint64_t b = __ballot(keep);
            if (keep && base + __popcll(b & lt) < kSortCap)
                sh.buf[base + __popcll(b & lt)] = entry(order_key(f), c);
            base += __popcll(b);
        };
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            put(ok[u] && v[u].x >= f0, v[u].x, col[u]);
            put(ok[u] && v[u].y >= f0, v[u].y, col[u] + 1);
            put(ok[u] && v[u].z >= f0, v[u].z, col[u] + 2);
            put(ok[u] && v[u].w >= f0, v[u].w, col[u] + 3);
        }
    };
    float4 v[kUnroll];
    int col[kUnroll];
    bool ok[kUnroll];
    if constexpr (ALIGNED) {
        const int n4 = cols >> 2;
        for (int b = tid; b < n4; b += kUnroll * kThreads) {
            if (b == tid) {
#pragma unroll
                for (int u = 0; u < kUnroll; ++u)
                    v[u] = first[u];
            } else {
                load_batch(x, n4, b, v);
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                col[u] = 4 * (b + u * kThreads);
                ok[u] = b + u * kThreads < n4;
            }
            emit(v, col, ok);
        }
        if ((cols & 3) == 0)
            return;
    }
    const float ninf = -__builtin_inff();
    const int i0 = ALIGNED ? cols & ~3 : 0;
    for (int b = i0 + 4 * tid; b < cols; b += 4 * kUnroll * kThreads) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = b + 4 * u * kThreads;
            v[u] = make_float4(ninf, ninf, ninf, ninf);
            if (i < cols)
                v[u].x = x[i];
            if (i + 1 < cols)
                v[u].y = x[i + 1];
            if (i + 2 < cols)
                v[u].z = x[i + 2];
            if (i + 3 < cols)
                v[u].w = x[i + 3];
            col[u] = i;
            ok[u] = true;
        }
        emit(v, col, ok);
    }
}

// Zero the 4096 bins, as straight-line code (a loop here would make the
// compiler drain every outstanding load at its head).
template <int NT, class SH>
__device__ __forceinline__ void clear_hist(SH &sh, int tid)
{
    static_assert(kMaxBins % NT == 0, "whole rounds of the block");
#pragma unroll
    for (int r = 0; r < kMaxBins / NT; ++r)
        sh.hist[tid + r * NT] = 0;
}

// The 24-bit prefix of the ts-th largest of the keys the block holds
// (EPT per thread; 0 = not listable), located by two 12-bit histograms; 0
// when fewer than ts keys are listable.
template <int NT, int EPT, class SH>
__device__ __forceinline__ uint32_t keys_threshold(SH &sh, const uint32_t (&samp)[EPT], int ts,
                                                   int tid, int lane, int wave)
{
    clear_hist<NT>(sh, tid);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < EPT; ++s)
        if (samp[s] != 0u)
            atomicAdd(&sh.hist[samp[s] >> 20], 1u);
    __syncthreads();
    find_threshold<NT>(sh, kMaxBins, 0, ts, tid);
    __syncthreads();
    if (sh.bcast[3] < ts)
        return 0u;
    const uint32_t b0 = (uint32_t)sh.bcast[0];
    const int above0 = sh.bcast[1];
    __syncthreads();  // hist and bcast are reused below
    clear_hist<NT>(sh, tid);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < EPT; ++s)
        if (samp[s] != 0u && (samp[s] >> 20) == b0)
            atomicAdd(&sh.hist[(samp[s] >> 8) & 0xfffu], 1u);
    __syncthreads();
    find_threshold<NT>(sh, kMaxBins, above0, ts, tid);
    __syncthreads();
    const uint32_t t0 = (b0 << 20) | ((uint32_t)sh.bcast[0] << 8);
    __syncthreads();
    return t0 > 0u ? t0 : 1u;
}

// Survivor target of a sampled threshold: the ts-th largest of a sample
// that holds m expected members of the top k leaves about 1.25 k entries of
// the population at or above it, plus a few standard deviations.
__device__ __forceinline__ int sample_rank(float m)
{
    return (int)ceilf(1.25f * m + 3.0f * sqrtf(m) + 4.0f);
}

// The threshold sample: entries g = EPT tid .. EPT tid + EPT - 1 of kSample,
// entry g at run g / 16, offset g % 16 of 256 evenly spaced 16-column runs.
template <int NT>
struct RowSample {
    static constexpr int EPT = kSample / NT;
    static_assert(EPT % 4 == 0 && 16 % EPT == 0, "whole float4 groups inside one run");
    float4 f[EPT / 4];
};

template <int NT, bool ALIGNED>
__device__ __forceinline__ void sample_load(RowSample<NT> &rs, const float *x, int cols, int tid)
{
    constexpr int EPT = RowSample<NT>::EPT;
    const int g = EPT * tid;
    const int pos = (int)(((int64_t)(g / 16) * cols / 256) & ~(int64_t)15) + g % 16;
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j) {
        const int q = pos + 4 * j;
        if constexpr (ALIGNED)
            rs.f[j] = *reinterpret_cast<const float4 *>(x + q);
        else
            rs.f[j] = make_float4(x[q], x[q + 1], x[q + 2], x[q + 3]);
    }
}

// A key t0 such that, judging by the row's sample, about 1.25 k entries plus a
// few standard deviations are >= t0.  0 when the sample holds too few listable
// keys.  Needs cols > kSample.
template <int NT, class SH>
__device__ __forceinline__ uint32_t sample_threshold(SH &sh, const RowSample<NT> &rs, int cols,
                                                     int k, int tid, int lane, int wave)
{
    constexpr int EPT = RowSample<NT>::EPT;
    uint32_t samp[EPT];
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j) {
        samp[4 * j + 0] = order_key(rs.f[j].x);
        samp[4 * j + 1] = order_key(rs.f[j].y);
        samp[4 * j + 2] = order_key(rs.f[j].z);
        samp[4 * j + 3] = order_key(rs.f[j].w);
    }
    const int ts = sample_rank((float)kSample * (float)k / (float)cols);
    return keys_threshold<NT, EPT>(sh, samp, ts, tid, lane, wave);
}

// A long row: the sampled threshold and one filter pass.  Returns the number
// of survivors when they hold the row's top k (between k and kSortCap), else
// -1.  On a 16-byte aligned row the first batch of the pass is requested right
// behind the sample, so its latency overlaps the sampling.
template <bool ALIGNED>
__device__ __forceinline__ int filter_row(TopkShared &sh, const float *x, int cols, int k, int tid,
                                          int lane, int wave)
{
    RowSample<kThreads> rs;
    sample_load<kThreads, ALIGNED>(rs, x, cols, tid);
    float4 first[kUnroll];
    if constexpr (ALIGNED)
        load_batch(x, cols >> 2, tid, first);
    const uint32_t t0 = sample_threshold(sh, rs, cols, k, tid, lane, wave);
    if (t0 == 0u)
        return -1;
    // order_key(v) >= t0  <=>  v >= f0 (t0 raised to the smallest listable
    // key changes nothing and keeps f0 finite, so -inf and NaN never pass)
    const float f0 = key_value(max(t0, 0x00800000u));
    filter_pass<ALIGNED>(sh, x, cols, f0, tid, lane, first);
    __syncthreads();
    const int c = sh.count;
    __syncthreads();
    return c >= k && c <= kSortCap ? c : -1;
}

// Exact selection by radix passes (the path for any row the sampled
// threshold does not resolve).  Leaves the entries to sort in sh.buf and
// returns their number.
__device__ int radix_select(TopkShared &sh, const float *x, int cols, int k, int tid, int lane,
                            int wave)
{
    // The selected keys are: every key whose top `pbits` bits exceed `prefix`
    // (there are `above` of them, fewer than k), then the largest keys of the
    // bucket whose top bits equal `prefix`.
    uint32_t prefix = 0;
    int pbits = 0;
    int above = 0;
    int bucket = 0;
    bool take_all = false;
    for (int pass = 0; pass < 3; ++pass) {
        const int bits = pass < 2 ? 12 : 8;
        const int nbins = 1 << bits;
        for (int i = tid; i < nbins; i += kThreads)
            sh.hist[i] = 0;
        __syncthreads();
        const int shift = 32 - pbits - bits;
        auto count = [&](float v) {
            const uint32_t key = order_key(v);
            if (key != 0u && (pbits == 0 || (key >> (32 - pbits)) == prefix))
                atomicAdd(&sh.hist[(key >> shift) & (uint32_t)(nbins - 1)], 1u);
        };
        for_each4(x, cols, tid, [&](float4 v, int) {
            count(v.x);
            count(v.y);
            count(v.z);
            count(v.w);
        });
        __syncthreads();
        find_threshold<kThreads>(sh, nbins, above, k, tid);
        __syncthreads();
        if (pass == 0 && sh.bcast[3] <= k) {
            take_all = true;  // at most k listable entries in the row
            break;
        }
        prefix = (prefix << bits) | (uint32_t)sh.bcast[0];
        pbits += bits;
        above = sh.bcast[1];
        bucket = sh.bcast[2];
        __syncthreads();  // bcast is rewritten by the next pass
        if (bucket <= kCand)
            break;
    }

    if (tid == 0)
        sh.count = 0;
    __syncthreads();
    if (take_all || bucket <= kCand) {
        // Every listable key (take_all: at most k), or every key at or above
        // the bucket (above + bucket < k + kCand).
        auto keep = [&](float v) {
            const uint32_t key = order_key(v);
            return key != 0u && (take_all || (key >> (32 - pbits)) >= prefix);
        };
        for_each4(x, cols, tid, [&](float4 v, int c) {
            append4(sh, v, c, keep(v.x), keep(v.y), keep(v.z), keep(v.w), lane);
        });
        __syncthreads();
        return sh.count;
    }
    // pbits == 32: the bucket is one key T repeated more than kCand times.
    // Every key above T is taken (above < k of them), then the first k - above
    // occurrences of T in column order, by an ordered compaction over chunks.
    const uint32_t T = prefix;
    const int need = k - above;
    int taken = 0;
    for (int base = 0; base < cols; base += kThreads) {
        const int i = base + tid;
        const uint32_t key = i < cols ? order_key(x[i]) : 0u;
        append(sh, key > T, entry(key, i), lane);
        const bool tie = key == T;
        const uint64_t ballot = __ballot(tie);
        const int in_wave = __popcll(ballot & ((1ull << lane) - 1ull));
        if (lane == 0)
            sh.wave_total[wave] = __popcll(ballot);
        __syncthreads();
        int before = 0, chunk = 0;
        for (int v = 0; v < kWaves; ++v) {
            const int c = sh.wave_total[v];
            before += v < wave ? c : 0;
            chunk += c;
        }
        const int rank = taken + before + in_wave;
        if (tie && rank < need)
            sh.buf[above + rank] = entry(key, i);
        taken += chunk;
        __syncthreads();  // wave_total is rewritten by the next chunk
    }
    // keys above T are at [0, above) in any order, the ties at [above, k)
    return k;
}

// ---- segment gather (the selects of the fused and the split top-k) --------
// A row's survivors sit in `split` segments of its entry region, segment s
// starting at entry seg_start(s) with counts[s] entries, and the select wants
// them in segment order in sh.buf.  Thread t requests entries
// j = t % L + L e (e < kWinLoads, L = kThreads / split) of segment t / L as the
// workgroup starts, beside the counts: a window of W = L kWinLoads entries at
// the head of every segment, read before its count is known (what lies past
// the count is ignored; every read stays inside the row's region).  Once the
// counts' prefix is in sh.hist the windows' entries go straight to their
// places, and only segments longer than W take a second round of loads.
constexpr int kWinLoads = 8;

struct SegWindow {
    uint64_t v[kWinLoads];
    int seg, j0, L;
};

template <class SegStart>
__device__ __forceinline__ void window_request(SegWindow &g, const uint64_t *row, int64_t limit,
                                               int split, SegStart seg_start, int tid)
{
    g.L = max(kThreads / split, 1);
    g.seg = tid / g.L;
    g.j0 = tid - g.seg * g.L;
    const int64_t base = seg_start(min(g.seg, split - 1)) + g.j0;
#pragma unroll
    for (int e = 0; e < kWinLoads; ++e)
        g.v[e] = row[min(base + (int64_t)g.L * e, limit - 1)];
}

// Puts the n entries in segment order into sh.buf: window entries (W = the
// window length, 0 when the windows were read at other starts than
// seg_start's) from registers, the rest of every segment longer than W
// (`over`: some segment is, the same in every thread) by a binary search over
// the prefix in sh.hist and one round of loads.
template <class SegStart>
__device__ __forceinline__ void window_place(TopkShared &sh, const SegWindow &g, const uint64_t *row,
                                             int split, int n, SegStart seg_start, int W, bool over,
                                             int tid)
{
    if (W > 0 && g.seg < split) {
        const int st = (int)sh.hist[g.seg];
        const int cnt = (g.seg + 1 < split ? (int)sh.hist[g.seg + 1] : n) - st;
#pragma unroll
        for (int e = 0; e < kWinLoads; ++e) {
            const int j = g.j0 + g.L * e;
            if (j < cnt)
                sh.buf[st + j] = g.v[e];
        }
    }
    if (!over)
        return;
    // entry i (in segment order) belongs to the last segment whose prefix is
    // <= i (empty segments share their successor's prefix)
    constexpr int EPT = kSortCap / kThreads;
    int64_t src[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = tid + e * kThreads;
        src[e] = -1;
        if (i < n) {
            int lo = 0, hi = split - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if ((int)sh.hist[mid] <= i)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            const int j = i - (int)sh.hist[lo];
            if (j >= W)
                src[e] = seg_start(lo) + j;
        }
    }
    uint64_t v[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e)
        v[e] = src[e] >= 0 ? row[src[e]] : 0ull;
#pragma unroll
    for (int e = 0; e < EPT; ++e)
        if (src[e] >= 0)
            sh.buf[tid + e * kThreads] = v[e];
}

// Sort the n entries gathered in sh.buf (n <= kSortCap; they hold the row's
// top min(n, k)) and write the row's k output columns.
__device__ __forceinline__ void sort_and_write(TopkShared &sh, int n, int32_t *out, int k, int tid,
                                               int lane, int wave)
{
    if (!bucket_sort(sh, n, k, tid, lane, wave)) {
        // Many equal or clustered keys: bitonic sort of the smallest power of
        // two >= n, padded with 0 (ranks last).
        int n2 = 1;
        while (n2 < n)
            n2 <<= 1;
        const int span = max(n2, 64 * E);
        for (int i = n + tid; i < span; i += kThreads)
            sh.buf[i] = 0ull;
        __syncthreads();
        sort_desc(sh, n2, tid, lane);
    }
    const uint64_t *order = sh.buf;

    const int nsel = min(n, k);
    for (int j = tid; j < k; j += kThreads)
        out[j] = j < nsel ? (int32_t)(~(uint32_t)(order[j] & 0xffffffffull)) : -1;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float *__restrict__ logits,
                                                        int32_t *__restrict__ indices, int cols,
                                                        int k)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t topk_lds[];
    TopkShared &sh = *reinterpret_cast<TopkShared *>(topk_lds);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const float *x = logits + (int64_t)blockIdx.x * cols;
    int32_t *out = indices + (int64_t)blockIdx.x * k;

    if (tid == 0)
        sh.count = 0;
    __syncthreads();
    int n = -1;  // entries gathered in sh.buf, once the row is resolved
    if (cols <= kSortCap) {
        for_each4(x, cols, tid, [&](float4 v, int c) {
            append4(sh, v, c, order_key(v.x) != 0u, order_key(v.y) != 0u, order_key(v.z) != 0u,
                    order_key(v.w) != 0u, lane);
        });
        __syncthreads();
        n = sh.count;
    } else {
        n = (reinterpret_cast<uintptr_t>(x) & 15) == 0 ? filter_row<true>(sh, x, cols, k, tid, lane, wave)
                                                         : filter_row<false>(sh, x, cols, k, tid, lane, wave);
        if (n < 0)
            n = radix_select(sh, x, cols, k, tid, lane, wave);
    }
    __syncthreads();
    sort_and_write(sh, n, out, k, tid, lane, wave);
}

// ---- split row top-k (mqa_topk_indices_ws) ---------------------------------
// One workgroup per row streams the row at one CU's read rate, which its
// outstanding misses cap near 30-40 GB/s, so with fewer rows than CUs most of
// the GPU idles.  With a caller workspace the row is split: `split`
// workgroups of kSplitThreads threads per row each take the row's threshold
// from the same sample (so all of them find the same key), keep the entries of
// their slice at or above it in their own segment of the row's workspace region
// and count them; then one workgroup per row gathers the segments and sorts
// them as the one-row path does.  A row whose segments cannot hold its top k
// (the sample misjudged it, or it has too few listable entries) is selected
// from its logits in full by that workgroup, so the output is the one-row
// path's for every input.
constexpr int kSplitThreads = 256;
// 16-byte groups per thread and batch (16 KiB per workgroup; the first batch is
// requested before the sampling).  Measured on 96 rows of 131072 columns, one
// GPU: 31.3 us at 4 with 16 workgroups per row, 31.9 at 8 with 8, 35.2 with the
// whole slice in one batch of 16 (its loads then delay the sample's); 32 or 64
// workgroups per row repeat the sampling too often (36-49 us).
constexpr int kSplitUnroll = 4;

struct SplitShared {
    uint32_t hist[kMaxBins];
    int bcast[4];
    int wave_total[kSplitThreads / 64];
    int count;
};

// Workgroup (row r, slice c): groups [c slice4, (c + 1) slice4) of the row's
// cols / 4 16-byte groups (the row is 16-byte aligned and cols a multiple of
// 4).  Its segment starts at entry 4 c slice4 of the row's region, so it holds
// the slice's survivors whatever their number.  counts[r][c] is the number
// kept, or -1 when the sample gives no threshold.
__global__ __launch_bounds__(kSplitThreads) void topk_split_filter_kernel(
    const float *__restrict__ logits, int cols, int k, int split, int slice4,
    uint64_t *__restrict__ entries, int64_t ent_stride, int *__restrict__ counts)
{
    __shared__ SplitShared sh;
    constexpr int U = kSplitUnroll;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = blockIdx.x / split, c = blockIdx.x % split;
    const float *x = logits + (int64_t)r * cols;
    const float4 *x4 = reinterpret_cast<const float4 *>(x);
    const int n4 = cols >> 2;
    const int g0 = min(c * slice4, n4), g1 = min(g0 + slice4, n4);
    const int nb = (g1 - g0 + U * kSplitThreads - 1) / (U * kSplitThreads);
    RowSample<kSplitThreads> rs;
    sample_load<kSplitThreads, true>(rs, x, cols, tid);
    // the slice's first batch, requested behind the sample (groups past the
    // slice read its last group and are dropped by index)
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        v[u] = x4[max(min(g0 + u * kSplitThreads + tid, g1 - 1), 0)];
    if (tid == 0)
        sh.count = 0;
    const uint32_t t0 = sample_threshold(sh, rs, cols, k, tid, lane, wave);
    int *cnt = counts + (int64_t)r * split + c;
    if (t0 == 0u) {  // uniform
        if (tid == 0)
            *cnt = -1;
        return;
    }
    const float f0 = key_value(max(t0, 0x00800000u));
    uint64_t *seg = entries + (int64_t)r * ent_stride + 4 * (int64_t)g0;
    const uint64_t lt = (1ull << lane) - 1ull;
    // keep the batch's entries >= f0: one LDS atomic per wave for the slots
    auto emit = [&](int j) {
        int i[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            i[u] = g0 + j * U * kSplitThreads + u * kSplitThreads + tid;
            ok[u] = i[u] < g1;
        }
        int total = 0;
#pragma unroll
        for (int u = 0; u < U; ++u)
            total += __popcll(__ballot(ok[u] && v[u].x >= f0)) +
                     __popcll(__ballot(ok[u] && v[u].y >= f0)) +
                     __popcll(__ballot(ok[u] && v[u].z >= f0)) +
                     __popcll(__ballot(ok[u] && v[u].w >= f0));
        if (total == 0)
            return;
        int base = 0;
        if (lane == 0)
            base = atomicAdd(&sh.count, total);
        base = __builtin_amdgcn_readfirstlane(base);
        auto put = [&](bool keep, float f, int col) {
            const uint64_t b = __ballot(keep);
            if (keep)
                seg[base + __popcll(b & lt)] = entry(order_key(f), col);
            base += __popcll(b);
        };
#pragma unroll
        for (int u = 0; u < U; ++u) {
            put(ok[u] && v[u].x >= f0, v[u].x, 4 * i[u]);
            put(ok[u] && v[u].y >= f0, v[u].y, 4 * i[u] + 1);
            put(ok[u] && v[u].z >= f0, v[u].z, 4 * i[u] + 2);
            put(ok[u] && v[u].w >= f0, v[u].w, 4 * i[u] + 3);
        }
    };
    emit(0);
    for (int j = 1; j < nb; ++j) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = x4[min(g0 + j * U * kSplitThreads + u * kSplitThreads + tid, g1 - 1)];
        emit(j);
    }
    __syncthreads();
    if (tid == 0)
        *cnt = sh.count;
}

// Row r: gather its segments (their prefix over the slices) and sort, or, when
// some slice had no threshold or the segments cannot hold the top k, select
// from the logits row in full.
__global__ __launch_bounds__(kThreads) void topk_split_select_kernel(
    const float *__restrict__ logits, int cols, int k, int split, int slice4,
    const uint64_t *__restrict__ entries, int64_t ent_stride, const int *__restrict__ counts,
    int32_t *__restrict__ indices)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t topk_lds[];
    TopkShared &sh = *reinterpret_cast<TopkShared *>(topk_lds);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = blockIdx.x;
    const float *x = logits + (int64_t)r * cols;
    const uint64_t *row = entries + (int64_t)r * ent_stride;
    int32_t *out = indices + (int64_t)r * k;
    const int c_in = counts[(int64_t)r * split + min(tid, split - 1)];
    const auto seg_start = [&](int g) { return 4 * (int64_t)slice4 * g; };
    SegWindow win;
    window_request(win, row, ent_stride, split, seg_start, tid);
    const int c = tid < split ? c_in : 0;
    const bool none = __syncthreads_or(c < 0);
    const int cc = max(c, 0);
    const int incl = wave_inclusive_scan(cc, lane);
    if (lane == 63)
        sh.wave_total[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < kWaves; ++w) {
        before += w < wave ? sh.wave_total[w] : 0;
        total += sh.wave_total[w];
    }
    if (tid < split)
        sh.hist[tid] = (uint32_t)(before + incl - cc);
    const int W = win.L * kWinLoads;
    const bool over = __syncthreads_or(cc > W);
    int n;
    if (!none && total >= k && total <= kSortCap) {  // uniform
        window_place(sh, win, row, split, total, seg_start, W, over, tid);
        n = total;
    } else {
        if (tid == 0)
            sh.count = 0;
        __syncthreads();
        n = radix_select(sh, x, cols, k, tid, lane, wave);
    }
    __syncthreads();
    sort_and_write(sh, n, out, k, tid, lane, wave);
}

// ---- fused decode top-k -------------------------------------------------
// The decode kernel's sample mode leaves kFusedSampleCols logits per row (-inf
// outside the window); its filter mode then keeps, per row, every entry at or
// above the row's threshold in per-workgroup segments.  The threshold comes
// from the sample as in the one-row top-k.  The select step then has exactly
// what the one-row filter would have kept, and sorts it the same way.  A row
// it cannot resolve (the sample misjudged it) is recomputed in full by the
// same workgroup: its logits into its own workspace segment, then the exact
// radix select.  So the output equals the top-k of the logits call's output.

// Listable positions of row r (p <= ctx - next_n + j, p < min(ctx, mml)).
__device__ __forceinline__ int row_population(const int32_t *ctx_lens, int r, int next_n, int mml)
{
    const int b = r / next_n, j = r % next_n;
    const int ctx = ctx_lens[b];
    const int nvalid = max(min(ctx, mml), 0);
    return max(0, min(ctx - next_n + j + 1, nvalid));
}

// The row-recompute inputs of the fused select (a kernel argument).
struct FusedRowArgs {
    uint64_t *entries;
    int64_t ent_stride;
    const int32_t *ctx_lens;
    int next_n;
    int mml;
    const uint8_t *q;
    const uint8_t *cache;
    const float *weights;
    const int32_t *tables;
    int mbps;
    int tiled;
    int block_size;  // tokens per cache block: 1, 16, 64 or 128
};

constexpr int kThresholdThreads = 256;  // 4 waves: 16 sample keys each thread, fewer waves per barrier

struct ThresholdShared {
    uint32_t hist[kMaxBins];
    int bcast[4];
    int listable;
    int wave_total[kThresholdThreads / 64];
};


__global__ __launch_bounds__(kThresholdThreads) void fused_threshold_kernel(
    const float *__restrict__ sample, const int32_t *__restrict__ ctx_lens, int next_n, int mml,
    int k, uint32_t *__restrict__ threshold)
{
    __shared__ ThresholdShared sh;
    const int tid = threadIdx.x;
    const int r = blockIdx.x;
    // The sample (every row's is written) is requested together with the
    // context length, so the two loads share one round of memory latency.
    constexpr int EPT = kFusedSampleCols / kThresholdThreads;
    const float *x = sample + (int64_t)r * kFusedSampleCols + EPT * tid;
    float4 f[EPT / 4];
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j)
        f[j] = *reinterpret_cast<const float4 *>(x + 4 * j);
    const int pop = row_population(ctx_lens, r, next_n, mml);
    if (pop <= kSortCap) {
        // short row: keep every listable entry (key >= 1)
        if (tid == 0)
            threshold[r] = 1u;
        return;
    }
    uint32_t samp[EPT];
    int mine = 0;
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j) {
        samp[4 * j + 0] = order_key(f[j].x);
        samp[4 * j + 1] = order_key(f[j].y);
        samp[4 * j + 2] = order_key(f[j].z);
        samp[4 * j + 3] = order_key(f[j].w);
        mine += (samp[4 * j] != 0u) + (samp[4 * j + 1] != 0u) + (samp[4 * j + 2] != 0u) +
                (samp[4 * j + 3] != 0u);
    }
    if (tid == 0)
        sh.listable = 0;
    __syncthreads();
    atomicAdd(&sh.listable, mine);
    __syncthreads();
    const int listable = sh.listable;
    const int ts = sample_rank((float)listable * (float)k / (float)pop);
    uint32_t t0 = 0u;  // 0: no threshold (the row is recomputed in full)
    if (ts <= listable)
        t0 = keys_threshold<kThresholdThreads, EPT>(sh, samp, ts, tid, tid & 63, tid >> 6);
    if (tid == 0)
        threshold[r] = t0;
}

// Row r's logits (the decode call's values, -inf outside the window) into
// x[0, mml): the workgroup's waves take the row's 64-token steps in turn and
// compute them with the decode kernel's contraction and epilogue (one row of
// 32 HT heads per wave, K straight from the cache), so every value equals the
// decode call's.  Each lane finds its token's block through the table, for
// any block size; entries past the last one holding a window token are never
// read (a later token reuses it, and its value is never kept).  DIM is the
// head dim (128 or 64).
template <int HT, int DIM>
__device__ __forceinline__ void recompute_row(float *x, const FusedRowArgs &ra, int r, int tid,
                                              int lane, int wave)
{
    constexpr int H = kHeads * HT;
    const int b = r / ra.next_n, j = r % ra.next_n;
    const int ctx = ra.ctx_lens[b];
    const int nvalid = max(min(ctx, ra.mml), 0);
    const int nsteps = (nvalid + kStep - 1) / kStep;
    const int bound = ctx - ra.next_n + j;  // inclusive
    const int t = lane & 31, g = lane >> 5;
    const int bs = ra.block_size;
    const int64_t blk_bytes = (int64_t)bs * (DIM + 4);
    const int last = max(nvalid - 1, 0) / bs;
    // With 16 waves a workgroup has 128 VGPRs per lane, so at most one head
    // tile's Q and weights stay in registers: 32 heads keep theirs for the
    // whole row, more heads reload them per step, tile by tile, summed in the
    // decode kernel's order.
    const uint8_t *qrow = ra.q + (int64_t)r * (H * DIM) + t * DIM;
    const float *wrow = ra.weights + (int64_t)r * H;
    Operand<DIM> q0;
    Weights16 w0;
    if constexpr (HT == 1) {
        load_frag(q0, qrow, lane);
        load_weights(w0, wrow, lane);
    }
    const int32_t *table = ra.tables + (int64_t)b * ra.mbps;
    const float ninf = -__builtin_inff();
    for (int st = wave; st < nsteps; st += kWaves) {
        KStepOf<DIM> k;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int p = st * kStep + kTile * h + t;
            const int slot = p % bs;
            const uint8_t *blk = ra.cache + (int64_t)table[min(p / bs, last)] * blk_bytes;
#pragma unroll
            for (int c = 0; c < DIM / 32; ++c) {
                const int u = 2 * c + g;  // 16-byte granule of the row
                const int off = ra.tiled ? (slot >> 4) * (16 * DIM) + u * 256 + (slot & 15) * 16
                                         : slot * DIM + u * 16;
                if (bs == 1) {
                    // per-token records are 132 bytes: K rows only 4-byte aligned
                    const int *src = reinterpret_cast<const int *>(blk + off);
                    k.t[h].c[c] = i32x4{src[0], src[1], src[2], src[3]};
                } else {
                    k.t[h].c[c] = *reinterpret_cast<const i32x4 *>(blk + off);
                }
            }
            k.sc[h] = *reinterpret_cast<const float *>(blk + bs * DIM + 4 * slot);
        }
        float part[2];
        if constexpr (HT == 1) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
                part[h] = relu_weight_sum(row_scores(q0, k.t[h]), w0);
        } else {
#pragma unroll 1
            for (int ht = 0; ht < HT; ++ht) {
                Operand<DIM> q;
                Weights16 w;
                load_frag(q, qrow + ht * (kHeads * DIM), lane);
                load_weights(w, wrow + ht * kHeads, lane);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float v = relu_weight_sum(row_scores(q, k.t[h]), w);
                    part[h] = ht == 0 ? v : part[h] + v;
                }
            }
        }
        float tot[2];  // the cross-lane step runs with every lane active
#pragma unroll
        for (int h = 0; h < 2; ++h)
            tot[h] = pair_head_sum(part[h], part[h]) * k.sc[h];
        if (lane < 32) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int p = st * kStep + h * kTile + t;
                if (p < ra.mml)
                    x[p] = p <= bound ? tot[h] : ninf;
            }
        }
    }
    for (int p = nsteps * kStep + tid; p < ra.mml; p += kThreads)
        x[p] = ninf;
}

template <int HT, int DIM>
__global__ __launch_bounds__(kThreads) void fused_select_kernel(FusedRowArgs ra,
                                                                const int *__restrict__ counts,
                                                                int split, int k,
                                                                int32_t *__restrict__ indices,
                                                                int *__restrict__ recomputed)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t topk_lds[];
    TopkShared &sh = *reinterpret_cast<TopkShared *>(topk_lds);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = blockIdx.x;
    const int b = r / ra.next_n;
    const int *cnt = counts + (int64_t)r * split;
    uint64_t *row = ra.entries + (int64_t)r * ra.ent_stride;
    int32_t *out = indices + (int64_t)r * k;
    // The counts and the segment windows are requested before the context
    // length is known, the windows at the segment starts of a context that
    // fills max_model_len; other rows gather every entry after the prefix.
    const int c_in = cnt[min(tid, split - 1)];
    const int64_t full_steps = ((int64_t)ra.mml + 63) / 64;
    SegWindow win;
    window_request(win, row, ra.ent_stride, split,
                   [&](int s) { return full_steps * s / split * 64; }, tid);
    const int pop = row_population(ra.ctx_lens, r, ra.next_n, ra.mml);
    const int nvalid = max(min(ra.ctx_lens[b], ra.mml), 0);
    const int nsteps = (nvalid + 63) / 64;

    // exclusive prefix of the segment counts (split <= kThreads) in sh.hist
    const int c = tid < split ? c_in : 0;
    const int incl = wave_inclusive_scan(c, lane);
    if (lane == 63)
        sh.wave_total[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int v = 0; v < kWaves; ++v) {
        before += v < wave ? sh.wave_total[v] : 0;
        total += sh.wave_total[v];
    }
    if (tid < split)
        sh.hist[tid] = (uint32_t)(before + incl - c);
    // Every entry at or above the threshold survived; if at least k did (or
    // every listable one did), they hold the row's top k.
    const bool ok = (total >= k || total == pop) && total <= kSortCap;
    if (tid == 0)
        recomputed[r] = ok ? 0 : 1;
    // segment s starts at the first column of the filter workgroup s
    const int W = nsteps == full_steps ? win.L * kWinLoads : 0;
    const bool over = __syncthreads_or(c > W);
    int n;
    if (ok) {  // uniform
        window_place(sh, win, row, split, total,
                     [&](int s) { return (int64_t)nsteps * s / split * 64; }, W, over, tid);
        n = total;
    } else {
        // the row's own segment region (>= mml floats) now holds its logits
        float *x = reinterpret_cast<float *>(row);
        recompute_row<HT, DIM>(x, ra, r, tid, lane, wave);
        __threadfence_block();
        __syncthreads();
        n = radix_select(sh, x, ra.mml, k, tid, lane, wave);
    }
    __syncthreads();
    sort_and_write(sh, n, out, k, tid, lane, wave);
}

template <int HT, int DIM>
hipError_t launch_fused_select_ht(const FusedTopkLaunch &p, const FusedRowArgs &ra,
                                  hipStream_t stream)
{
    static std::atomic<uint64_t> raised{0};
    hipError_t e = raise_lds_limit(reinterpret_cast<const void *>(&fused_select_kernel<HT, DIM>),
                                   (int)sizeof(TopkShared), raised);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((fused_select_kernel<HT, DIM>), dim3(p.batch * p.next_n), dim3(kThreads),
                       sizeof(TopkShared), stream, ra, p.ws->counts, p.split, p.k, p.indices,
                       p.ws->recomputed);
    return hipGetLastError();
}

} // namespace

hipError_t launch_fused_threshold(const FusedTopkLaunch &p, hipStream_t stream)
{
    hipLaunchKernelGGL(fused_threshold_kernel, dim3(p.batch * p.next_n), dim3(kThresholdThreads), 0,
                       stream, p.ws->sample, p.context_lens, p.next_n, p.mml, p.k, p.ws->threshold);
    return hipGetLastError();
}

hipError_t launch_fused_select(const FusedTopkLaunch &p, hipStream_t stream)
{
    FusedRowArgs ra;
    ra.entries = p.ws->entries;
    ra.ent_stride = p.ws->ent_stride;
    ra.ctx_lens = p.context_lens;
    ra.next_n = p.next_n;
    ra.mml = p.mml;
    ra.q = p.q;
    ra.cache = p.cache;
    ra.weights = p.weights;
    ra.tables = p.block_tables;
    ra.mbps = p.max_blocks_per_seq;
    ra.tiled = p.tiled;
    ra.block_size = p.block_size;
    switch (p.head_tiles * 1000 + p.head_dim) {
    case 1128: return launch_fused_select_ht<1, 128>(p, ra, stream);
    case 2128: return launch_fused_select_ht<2, 128>(p, ra, stream);
    case 4128: return launch_fused_select_ht<4, 128>(p, ra, stream);
    case 1064: return launch_fused_select_ht<1, 64>(p, ra, stream);
    case 2064: return launch_fused_select_ht<2, 64>(p, ra, stream);
    case 4064: return launch_fused_select_ht<4, 64>(p, ra, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_topk_split(const TopkSplitLaunch &p, hipStream_t stream)
{
    static std::atomic<uint64_t> raised{0};
    hipError_t e = raise_lds_limit(reinterpret_cast<const void *>(&topk_split_select_kernel),
                                   (int)sizeof(TopkShared), raised);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(topk_split_filter_kernel, dim3(p.rows * p.split), dim3(kSplitThreads), 0,
                       stream, p.logits, p.cols, p.k, p.split, p.slice4, p.ws.entries,
                       p.ws.ent_stride, p.ws.counts);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(topk_split_select_kernel, dim3(p.rows), dim3(kThreads), sizeof(TopkShared),
                       stream, p.logits, p.cols, p.k, p.split, p.slice4, p.ws.entries,
                       p.ws.ent_stride, p.ws.counts, p.indices);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkLaunch &p, hipStream_t stream)
{
    // The LDS block (~146 KiB) is above the default dynamic limit.
    static std::atomic<uint64_t> raised{0};
    hipError_t e = raise_lds_limit(reinterpret_cast<const void *>(&topk_kernel),
                                   (int)sizeof(TopkShared), raised);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(topk_kernel, dim3(p.rows), dim3(kThreads), sizeof(TopkShared), stream,
                       p.logits, p.indices, p.cols, p.k);
    return hipGetLastError();
}

} // namespace mqa
