// C-ABI entry points: argument validation, the support gate, the host launch
// heuristic and the per-thread error string.  Declared in include/mqa_indexer.h.
#include "mqa_indexer.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok()
{
    g_last_error.clear();
    return MQA_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// gfx950 check for the current device, cached per device id (threads may race
// to fill an entry; they store the same value).
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices]; // 0 unknown, 1 gfx950, -1 other

int current_device_is_gfx950(int *dev_out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return -1;
    }
    if (dev_out)
        *dev_out = dev;
    if (dev < kMaxDevices) {
        const int known = g_arch_ok[dev].load(std::memory_order_relaxed);
        if (known != 0)
            return known > 0 ? 1 : 0;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return -1;
    }
    const int is950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    if (dev < kMaxDevices)
        g_arch_ok[dev].store(is950 ? 1 : -1, std::memory_order_relaxed);
    return is950;
}

int check_device()
{
    int dev = -1;
    const int r = current_device_is_gfx950(&dev);
    if (r < 0)
        return fail(MQA_ERR_DEVICE, "no usable HIP device");
    if (r == 0)
        return fail(MQA_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    return MQA_OK;
}

// 32, 64 or 128 index heads (the pages sweep all three); head dim 128 or 64
// (the prefill page's test sweep covers head dims 64 and 128, the decode
// page's only 128; the decode takes 64 too); cache blocks of 1, 16, 64 or 128
// tokens for decode (0 asks about prefill), at every head count and head dim.
bool shape_supported(int num_heads, int head_dim, int kv_block_size)
{
    if (num_heads != 32 && num_heads != 64 && num_heads != 128)
        return false;
    if (head_dim != 128 && head_dim != 64)
        return false;
    return kv_block_size == 0 || kv_block_size == 1 || kv_block_size == 16 ||
           kv_block_size == 64 || kv_block_size == 128;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Optional one-line trace of the chosen launch (MQA_TRACE=1).
bool trace_on()
{
    static const bool on = [] {
        const char *e = std::getenv("MQA_TRACE");
        return e && e[0] == '1';
    }();
    return on;
}

} // namespace

extern "C" int mqa_is_supported(int num_heads, int head_dim, int kv_block_size)
{
    if (!shape_supported(num_heads, head_dim, kv_block_size))
        return 0;
    return current_device_is_gfx950(nullptr) == 1 ? 1 : 0;
}

extern "C" const char *mqa_last_error(void) { return g_last_error.c_str(); }

extern "C" int mqa_logits_prefill(const uint8_t *q_fp8, const uint8_t *k_fp8, const float *kv_scale,
                                  const float *weights, const int32_t *cu_seqlen_ks,
                                  const int32_t *cu_seqlen_ke, float *logits, int M, int N,
                                  int num_heads, int head_dim, int clean_logits,
                                  const mqa_tunables *tun, hipStream_t stream)
{
    if (M < 0 || N < 0)
        return fail(MQA_ERR_INVALID_ARG, "M=%d, N=%d must be >= 0", M, N);
    if (!shape_supported(num_heads, head_dim, 0))
        return fail(MQA_ERR_UNSUPPORTED,
                    "prefill supports num_heads 32, 64 or 128 and head_dim 64 or 128 (got %d, %d)",
                    num_heads, head_dim);
    const int head_tiles = num_heads / 32;
    const int max_block_m = 8 / head_tiles;  // Q and weights of a wave's rows stay in VGPRs
    mqa_tunables t = {};
    if (tun)
        t = *tun;
    if (t.block_m != 0 && t.block_m != 1 && t.block_m != 2 && t.block_m != 4 && t.block_m != 8)
        return fail(MQA_ERR_INVALID_ARG, "block_m must be 0, 1, 2, 4 or 8 (got %d)", t.block_m);
    if (t.block_m > max_block_m)
        return fail(MQA_ERR_INVALID_ARG, "block_m is at most %d with %d heads (got %d)", max_block_m,
                    num_heads, t.block_m);
    if (t.split_n < 0 || t.num_warps < 0 || t.num_warps > 4)
        return fail(MQA_ERR_INVALID_ARG, "split_n >= 0 and num_warps in 0..4 required");
    if (t.reverse_rows < -1 || t.reverse_rows > 1)
        return fail(MQA_ERR_INVALID_ARG, "reverse_rows must be -1, 0 or 1");
    if (t.ring_depth < 0 || t.ring_depth > 7)
        return fail(MQA_ERR_INVALID_ARG, "prefill ring_depth must be 0, 1 (per-wave K) or 2..7 "
                    "(got %d)", t.ring_depth);
    // the shared-K ring: 4 waves of 4 rows at 32 heads (depth 2..7), of 2 rows
    // at 64 heads and of 1 row at 128 heads (depth 3 or 4), head dim 128
    const int ring_rows = num_heads == 32 ? 4 : num_heads == 64 ? 2 : 1;
    if (t.ring_depth >= 2 &&
        (head_dim != 128 || (num_heads != 32 && t.ring_depth > 4) ||
         (t.block_m != 0 && t.block_m != ring_rows) || (t.num_warps != 0 && t.num_warps != 4)))
        return fail(MQA_ERR_INVALID_ARG, "the shared-K prefill runs head_dim 128 with num_warps 4 "
                    "(or 0): 32 heads with ring_depth 2..7 and block_m 4, 64 heads with ring_depth "
                    "3 or 4 and block_m 2, 128 heads with ring_depth 3 or 4 and block_m 1");
    if (M == 0 || N == 0)
        return ok();
    if (!q_fp8 || !k_fp8 || !kv_scale || !weights || !cu_seqlen_ks || !cu_seqlen_ke || !logits)
        return fail(MQA_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(q_fp8, 16) || !aligned(k_fp8, 16) || !aligned(kv_scale, 16) ||
        !aligned(weights, 16) || !aligned(logits, 16) || !aligned(cu_seqlen_ks, 4) ||
        !aligned(cu_seqlen_ke, 4))
        return fail(MQA_ERR_INVALID_ARG, "data pointers must be 16-byte aligned, int32 arrays 4-byte");
    if (int rc = check_device())
        return rc;

    mqa::PrefillLaunch p;
    p.q = q_fp8;
    p.k = k_fp8;
    p.kv_scale = kv_scale;
    p.weights = weights;
    p.ks = cu_seqlen_ks;
    p.ke = cu_seqlen_ke;
    p.logits = logits;
    p.M = M;
    p.N = N;
    p.clean = clean_logits ? 1 : 0;
    // Heuristic (measured on MI355X; both pages, "Technical Details", make
    // the row block, split and wave count host-chosen).  The per-wave kernel
    // (head dim 64, small problems, explicit block_m / num_warps): 4 rows per
    // wave share each K step, with one wave per workgroup for long chunks and
    // 4 waves for short ones; and enough column splits for ~2048 workgroups
    // while each wave keeps >= 4 steps.  4 rows (228 VGPRs, 2 waves per SIMD) measured
    // faster than 8 rows (1 wave per SIMD) on the long chunk although K is
    // re-read from L2 twice as often: M 4096, N 32768 took 525 against 536 us
    // at head dim 128 and 356 against 384 us at head dim 64 (means of three
    // alternating runs on one MI355X).  High-m first for long causal chunks
    // (aiter PR 5046 page, "Technical Details": N > 2048).
    //   Small problems (at most 16384 row-steps, e.g. 64 rows x 512
    //   columns) are latency-bound: one row and one wave per workgroup and
    //   splits down to 2 steps per wave measured 2.3x faster than 4 rows x 4
    //   waves on M 64, N 512.
    p.head_tiles = head_tiles;
    p.head_dim = head_dim;
    const int64_t steps = ceil_div(N, 64);
    const bool small = M < 1024 && (int64_t)M * steps <= 16384;
    // The shared-K ring (4 waves of 4, 2 or 1 rows at 32, 64 or 128 heads; K
    // through LDS) at head dim 128 for all but the small problems, unless the
    // tunables ask otherwise: M 4096, N 32768 went from 508.3 to 447.6 us at 32
    // heads, from 1023.6 to 903.4 us at 64 and from 1793.8 to 1608.1 us at 128
    // (one MI355X, medians of three rounds).  At head dim 64 the per-wave
    // kernel stays (319.8 against 322.9 us with the ring at its best split).
    const bool ring_default = head_dim == 128 && !small && t.block_m == 0 && t.num_warps == 0;
    p.ring = t.ring_depth >= 2 ? t.ring_depth : (t.ring_depth == 0 && ring_default ? 4 : 0);
    p.block_m = p.ring ? ring_rows : t.block_m ? t.block_m : (small ? 1 : std::min(4, max_block_m));
    p.num_warps = p.ring ? 4 : t.num_warps ? t.num_warps : (M >= 1024 || small ? 1 : 4);
    const int64_t nrb = ceil_div(M, p.ring ? p.block_m * p.num_warps : p.block_m);
    if (t.split_n) {
        p.split_n = t.split_n;
    } else if (p.ring) {
        // ~1024 workgroups (two 4-wave workgroups per CU are resident) and at
        // least 2 column parts, each walking at least 8 steps: on M 4096,
        // N 32768 split 4 took 447.6 us against 450.1 with 2 and 451.4 with 8
        // at 32 heads, split 2 903.4 against 902.7 with 4 at 64 heads, and
        // 1608.1 against 1628.8 with 1 at 128 heads; ring depth 4 against 5
        // and 6 level, 3 slower (one MI355X, medians of three rounds)
        int64_t want = std::max<int64_t>(2, ceil_div(1024, nrb));
        int64_t cap = std::max<int64_t>(1, steps / 8);
        int64_t split = std::min(want, cap);
        // and the grid rounded down to whole rounds of 256 workgroups (as the
        // decode's), keeping two parts: causal chunks of N 32768 with M 1000
        // took 142.9 us at split 17 (1071 workgroups) against 129.0 at 16,
        // M 3000 368.2 against 351.9 us (6 -> 5), and M 2500, N 16384 162.5
        // against 151.3 us (7 -> 6), one MI355X
        if (nrb * split > 256) {
            const int64_t r = nrb * split / 256 * 256 / nrb;
            if (r >= 2)
                split = r;
        }
        p.split_n = (int)split;
    } else {
        // ~2048 workgroups; ~8192 at head dim 64 (split 8 on the long chunk: 355
        // against 366 us with split 2, three alternating runs on one MI355X)
        int64_t want = std::max<int64_t>(1, ceil_div(head_dim == 64 ? 8192 : 2048, nrb));
        int64_t cap = std::max<int64_t>(1, steps / ((small ? 2 : 4) * p.num_warps));
        p.split_n = (int)std::min(want, cap);
    }
    p.reverse = t.reverse_rows ? (t.reverse_rows > 0) : (N > 2048);
    if (nrb * p.split_n > INT32_MAX)
        return fail(MQA_ERR_INVALID_ARG, "grid too large (row blocks %lld x split %d)", (long long)nrb,
                    p.split_n);
    if (trace_on())
        std::fprintf(stderr, "[mqa] prefill M=%d N=%d block_m=%d split_n=%d warps=%d reverse=%d "
                     "ring=%d\n", M, N, p.block_m, p.split_n, p.num_warps, p.reverse, p.ring);
    hipError_t e = mqa::launch_prefill(p, stream);
    if (e != hipSuccess)
        return fail(MQA_ERR_LAUNCH, "prefill launch failed: %s", hipGetErrorString(e));
    return ok();
}

namespace {

constexpr int kNoop = 1;  // prepare_decode: valid arguments, nothing to do

// Validate the paged-decode arguments shared by the logits call and the
// fused top-k, and fill the launch (pointers and the launch heuristic).
// Returns MQA_OK, kNoop, or a (recorded) error code.  `logits` is only
// checked when need_logits.
int prepare_decode(const uint8_t *q_fp8, const uint8_t *kv_cache, const float *weights,
                   const int32_t *context_lens, const int32_t *block_tables, float *logits,
                   bool need_logits, int batch, int next_n, int num_heads, int head_dim,
                   int kv_block_size, int kv_layout, int num_blocks, int max_blocks_per_seq,
                   int max_model_len, int clean_logits, const mqa_tunables *tun,
                   mqa::DecodeLaunch &p)
{
    if (batch < 0 || num_blocks < 0 || max_blocks_per_seq < 0 || max_model_len < 0)
        return fail(MQA_ERR_INVALID_ARG, "negative size argument");
    if (next_n < 1 || next_n > 8)
        return fail(MQA_ERR_INVALID_ARG, "next_n must be in 1..8 (got %d)", next_n);
    if (kv_layout != MQA_KV_SLOT_MAJOR && kv_layout != MQA_KV_PRESHUFFLED)
        return fail(MQA_ERR_INVALID_ARG, "kv_layout must be MQA_KV_SLOT_MAJOR or MQA_KV_PRESHUFFLED "
                    "(got %d)", kv_layout);
    if (!shape_supported(num_heads, head_dim, kv_block_size) || kv_block_size == 0)
        return fail(MQA_ERR_UNSUPPORTED,
                    "decode supports num_heads 32, 64 or 128, head_dim 128 or 64 and "
                    "kv_block_size 1, 16, 64 or 128 (got %d, %d, %d)",
                    num_heads, head_dim, kv_block_size);
    if (kv_layout == MQA_KV_PRESHUFFLED && kv_block_size < 16)
        return fail(MQA_ERR_UNSUPPORTED, "the preshuffled layout needs kv_block_size 16, 64 or 128 "
                    "(got %d)", kv_block_size);
    mqa_tunables t = {};
    if (tun)
        t = *tun;
    const int head_tiles = num_heads / 32;
    const int max_rows = 4 / head_tiles;  // Q and weights of a wave's rows stay in VGPRs
    const bool any_depth = kv_block_size == 64 && head_tiles == 1 && head_dim == 128;
    // the one ring depth the other layouts instantiate (see the heuristic)
    const int fixed_depth = kv_block_size == 1 ? 4 : 3;
    if (t.rows_per_block < 0 || t.rows_per_block > max_rows || t.split_kv < 0 ||
        t.num_warps != 0 || t.ring_depth < 0 || t.ring_depth == 1 || t.ring_depth > 7 ||
        (!any_depth && t.ring_depth != 0 && t.ring_depth != fixed_depth))
        return fail(MQA_ERR_INVALID_ARG,
                    "decode tunables: rows_per_block in 0..%d, split_kv >= 0, ring_depth 0 or 2..7 "
                    "(0 or %d unless 32 heads, head_dim 128 and kv_block_size 64), num_warps 0",
                    max_rows, fixed_depth);
    if (batch == 0 || max_model_len == 0)
        return kNoop;
    if (!q_fp8 || !kv_cache || !weights || !context_lens || !block_tables ||
        (need_logits && !logits))
        return fail(MQA_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(q_fp8, 16) || !aligned(kv_cache, 16) || !aligned(weights, 16) ||
        (need_logits && !aligned(logits, 16)) || !aligned(context_lens, 4) ||
        !aligned(block_tables, 4))
        return fail(MQA_ERR_INVALID_ARG, "data pointers must be 16-byte aligned, int32 arrays 4-byte");
    if (int rc = check_device())
        return rc;

    p = mqa::DecodeLaunch{};
    p.q = q_fp8;
    p.cache = kv_cache;
    p.weights = weights;
    p.context_lens = context_lens;
    p.block_tables = block_tables;
    p.logits = logits;
    p.batch = batch;
    p.next_n = next_n;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.max_model_len = max_model_len;
    p.clean = clean_logits ? 1 : 0;
    // Heuristic (aiter PR 5047 page, "Technical Details": rows per K stream and
    // the KV split are chosen on the host from batch * max_model_len, since the
    // device-resident context lengths are not visible without a sync).
    // Measured on MI355X:
    //   rows: every wave of a workgroup reads the same LDS ring, so all next_n
    //         rows share one HBM stream whatever the row split.  From next_n 4
    //         on, 3 or 4 waves of at most 2 rows (at most ~160 VGPRs, 3 waves
    //         per SIMD) beat 2 waves of 3 or 4 rows: next_n 6 as 3 x 2 rows
    //         68.5 against 69.7 us, next_n 4 as 4 x 1 row 144.6 against
    //         146.7 us (ragged batch), each the mean of three alternating runs.
    //         Below that, ceil(next_n / 2) rows per wave.
    //   depth: 3 steps (25 KiB) per workgroup; deeper rings cost workgroups
    //          per CU and measured slower.  The other layouts instantiate one
    //          depth: 3 (16-token blocks 68.5 against 69-73 us at depth 4,
    //          128-token blocks 69.9 against 70-73 us, the rest level) and 4
    //          for per-token blocks (level).
    //   split: at least ~1024 workgroups, and at most 32 steps (2048 tokens)
    //          per workgroup at the longest context, but at least 2 steps;
    //          more workgroups per sequence than that measured slower (longer
    //          prologues relative to the work, more concurrent streams).  At
    //          128 heads a wave holds one row (~218 VGPRs, 2 waves per SIMD), so
    //          one next_n-wave workgroup fills a CU: there the target is ~256
    //          workgroups and at most 128 steps each (B 16, 131072 tokens,
    //          next_n 6, one GPU: split 16 210.8 us, 32 212.6 us; the 1024-
    //          workgroup rule's 64: 220-226 us).
    const int rows_default = next_n == 4 ? 1 : next_n > 4 ? 2 : (next_n + 1) / 2;
    int rows = t.rows_per_block ? t.rows_per_block : rows_default;
    rows = std::min(std::min(rows, next_n), max_rows);
    p.head_tiles = head_tiles;
    p.head_dim = head_dim;
    p.rows = rows;
    //   short contexts (at most 128 steps): one step per workgroup, with a
    //   2-step ring (B 16, 8192 tokens: 6.6 -> 6.2 us).
    const int64_t steps_max = ceil_div(max_model_len, 64);
    const bool short_ctx = steps_max <= 128;
    p.depth = t.ring_depth ? t.ring_depth : (any_depth ? (short_ctx ? 2 : 3) : fixed_depth);
    p.block_size = kv_block_size;
    p.tiled = kv_layout == MQA_KV_PRESHUFFLED;
    if (t.split_kv) {
        p.split_kv = t.split_kv;
    } else {
        const bool one_wg_per_cu = head_tiles == 4;
        const int64_t want =
            short_ctx ? steps_max
                      : one_wg_per_cu ? std::max(ceil_div(256, batch), ceil_div(steps_max, 128))
                                      : std::max(ceil_div(1024, batch), ceil_div(steps_max, 32));
        const int64_t cap = std::max<int64_t>(1, short_ctx ? steps_max : steps_max / 2);
        int64_t split = std::max<int64_t>(1, std::min(want, cap));
        // The grid is rounded down to whole rounds of workgroups over the 256
        // CUs: a few workgroups past a multiple of 256 give some CUs one more
        // than the others, and the call waits for those (with four resident
        // per CU, the extra one runs as a second round).  Next_n 6, 131072
        // tokens: B 6 split 171 (1026 workgroups) 39.09 us against 170 (1020)
        // 30.96 us, B 12 86 against 85 67.14 / 53.30 us, B 3 22.39 / 19.30 us;
        // where the step cap binds, B 1, next_n 2, 32768 tokens in per-token
        // blocks 333 -> 256 workgroups, 6.64 -> 5.70 us (one MI355X).
        if (!short_ctx && batch * split > 256)
            split = std::max<int64_t>(1, batch * split / 256 * 256 / batch);
        p.split_kv = (int)split;
    }
    if ((int64_t)batch * p.split_kv > INT32_MAX)
        return fail(MQA_ERR_INVALID_ARG, "grid too large");
    if (trace_on())
        std::fprintf(stderr, "[mqa] decode B=%d next_n=%d mml=%d rows=%d split_kv=%d depth=%d\n", batch,
                     next_n, max_model_len, p.rows, p.split_kv, p.depth);
    return MQA_OK;
}

} // namespace

extern "C" int paged_mqa_logits_decode(const uint8_t *q_fp8, const uint8_t *kv_cache,
                                       const float *weights, const int32_t *context_lens,
                                       const int32_t *block_tables, float *logits, int batch,
                                       int next_n, int num_heads, int head_dim, int kv_block_size,
                                       int kv_layout, int num_blocks, int max_blocks_per_seq,
                                       int max_model_len, int clean_logits,
                                       const mqa_tunables *tun, hipStream_t stream)
{
    mqa::DecodeLaunch p;
    const int rc = prepare_decode(q_fp8, kv_cache, weights, context_lens, block_tables, logits, true,
                                  batch, next_n, num_heads, head_dim, kv_block_size, kv_layout,
                                  num_blocks, max_blocks_per_seq, max_model_len, clean_logits, tun, p);
    if (rc == kNoop)
        return ok();
    if (rc != MQA_OK)
        return rc;
    hipError_t e = mqa::launch_decode(p, stream);
    if (e != hipSuccess)
        return fail(MQA_ERR_LAUNCH, "decode launch failed: %s", hipGetErrorString(e));
    return ok();
}

extern "C" size_t paged_mqa_topk_workspace_size(int batch, int next_n, int max_model_len)
{
    if (batch <= 0 || next_n < 1 || next_n > 8 || max_model_len <= 0 ||
        (int64_t)batch * next_n > INT32_MAX)
        return 0;
    return mqa::fused_workspace(nullptr, batch * next_n, max_model_len).bytes;
}

extern "C" int paged_mqa_topk_decode(const uint8_t *q_fp8, const uint8_t *kv_cache,
                                     const float *weights, const int32_t *context_lens,
                                     const int32_t *block_tables, int32_t *indices, int batch,
                                     int next_n, int num_heads, int head_dim, int kv_block_size,
                                     int kv_layout, int num_blocks, int max_blocks_per_seq,
                                     int max_model_len, int k, void *workspace,
                                     size_t workspace_bytes, const mqa_tunables *tun,
                                     hipStream_t stream)
{
    if (k < 1 || k > mqa::kMaxTopK)
        return fail(MQA_ERR_INVALID_ARG, "k must be in 1..%d (got %d)", mqa::kMaxTopK, k);
    if (!shape_supported(num_heads, head_dim, kv_block_size) || kv_block_size == 0)
        return fail(MQA_ERR_UNSUPPORTED,
                    "the fused top-k takes the decode's shapes: num_heads 32, 64 or 128, head_dim "
                    "128 or 64, kv_block_size 1, 16, 64 or 128 (got %d, %d, %d)", num_heads,
                    head_dim, kv_block_size);
    // the sample and filter modes are built for the logits call's default ring
    const int depth = kv_block_size == 1 ? 4 : 3;
    if (tun && tun->ring_depth != 0 && tun->ring_depth != depth)
        return fail(MQA_ERR_INVALID_ARG, "the fused top-k runs the default ring depth (0 or %d "
                    "for this shape)", depth);
    if (batch > 0 && max_model_len > 0 && next_n >= 1 && next_n <= 8) {
        if ((int64_t)batch * next_n > INT32_MAX)
            return fail(MQA_ERR_INVALID_ARG, "batch %d x next_n %d rows exceed INT32_MAX", batch,
                        next_n);
        if (!indices || !workspace)
            return fail(MQA_ERR_INVALID_ARG, "NULL pointer argument");
        if (!aligned(indices, 4) || !aligned(workspace, 256))
            return fail(MQA_ERR_INVALID_ARG, "indices must be 4-byte aligned, workspace 256-byte");
        const size_t need = paged_mqa_topk_workspace_size(batch, next_n, max_model_len);
        if (workspace_bytes < need)
            return fail(MQA_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu bytes "
                        "paged_mqa_topk_workspace_size asks for", workspace_bytes, need);
    }
    mqa::DecodeLaunch p;
    const int rc = prepare_decode(q_fp8, kv_cache, weights, context_lens, block_tables, nullptr,
                                  false, batch, next_n, num_heads, head_dim, kv_block_size,
                                  kv_layout, num_blocks, max_blocks_per_seq, max_model_len, 1, tun,
                                  p);
    if (rc == kNoop)
        return ok();
    if (rc != MQA_OK)
        return rc;
    if (p.split_kv > mqa::kFusedMaxSplit)
        return fail(MQA_ERR_INVALID_ARG, "the fused top-k takes split_kv <= %d (got %d)",
                    mqa::kFusedMaxSplit, p.split_kv);
    p.depth = depth;
    const int rows = batch * next_n;
    const mqa::FusedWorkspace w = mqa::fused_workspace(workspace, rows, max_model_len);
    mqa::FusedTopkLaunch f{&w,      context_lens, indices, batch,   next_n,
                           max_model_len, k,   p.split_kv, q_fp8, kv_cache,
                           weights, block_tables, max_blocks_per_seq, p.tiled,
                           kv_block_size, p.head_tiles, head_dim};
    hipError_t e;
    // 1. the sample: kFusedSampleChunks runs of steps per sequence
    mqa::DecodeLaunch ps = p;
    ps.mode = 1;
    ps.split_kv = mqa::kFusedSampleChunks;
    ps.sample = w.sample;
    e = mqa::launch_decode(ps, stream);
    // 2. per-row thresholds
    if (e == hipSuccess)
        e = mqa::launch_fused_threshold(f, stream);
    // 3. the filtering decode
    if (e == hipSuccess) {
        mqa::DecodeLaunch pf = p;
        pf.mode = 2;
        pf.threshold = w.threshold;
        pf.entries = w.entries;
        pf.counts = w.counts;
        pf.ent_stride = w.ent_stride;
        e = mqa::launch_decode(pf, stream);
    }
    // 4. select and sort; a row the sample misjudged is recomputed in full
    if (e == hipSuccess)
        e = mqa::launch_fused_select(f, stream);
    if (e != hipSuccess)
        return fail(MQA_ERR_LAUNCH, "fused top-k launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Device scratch of the allocation-free fused top-k (paged_mqa_topk_decode_noalloc):
// the workspace paged_mqa_topk_decode takes from its caller, held by the library
// instead.  Every device the library runs on holds one copy at its own address
// until the process ends.  128 MiB covers 96 rows of 131072 positions (about 8
// bytes per row and position).
constexpr size_t kNoAllocScratchBytes = MQA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // per device; guarded by g_scratch_mu

// The device address of `scratch` on the current device, looked up once per
// device (the host-side name `scratch` is only a stand-in for it).
int scratch_of_current_device(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(MQA_ERR_DEVICE, "no usable HIP device");
    }
    if (dev >= kMaxDevices)
        return fail(MQA_ERR_DEVICE, "device %d is past the %d devices the library tracks", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return fail(MQA_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MQA_OK;
}

} // namespace

extern "C" int paged_mqa_topk_decode_noalloc(const uint8_t *q_fp8, const uint8_t *kv_cache,
                                             const float *weights, const int32_t *context_lens,
                                             const int32_t *block_tables, int32_t *indices,
                                             int batch, int next_n, int num_heads, int head_dim,
                                             int kv_block_size, int kv_layout, int num_blocks,
                                             int max_blocks_per_seq, int max_model_len, int k,
                                             const mqa_tunables *tun, hipStream_t stream)
{
    const size_t need = paged_mqa_topk_workspace_size(batch, next_n, max_model_len);
    if (need > kNoAllocScratchBytes)
        return fail(MQA_ERR_INVALID_ARG, "batch %d x next_n %d rows of max_model_len %d need %zu "
                    "bytes of scratch; the library's static scratch holds %zu", batch, next_n,
                    max_model_len, need, kNoAllocScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        if (int rc = check_device())
            return rc;
        if (int rc = scratch_of_current_device(&ws))
            return rc;
    }
    // Nothing in the workspace has to start at zero: every word whose value a
    // kernel uses was written earlier in the same call (the select also reads
    // ahead into its segments and ignores what lies past their counts).
    return paged_mqa_topk_decode(q_fp8, kv_cache, weights, context_lens, block_tables, indices,
                                 batch, next_n, num_heads, head_dim, kv_block_size, kv_layout,
                                 num_blocks, max_blocks_per_seq, max_model_len, k, ws,
                                 kNoAllocScratchBytes, tun, stream);
}

namespace {

// The split top-k's workgroups per row: about six 4-wave workgroups per CU
// over all rows, each slice at least 4096 columns; 1 = the one-row path.
// 96 rows of 131072 columns (16 per row): 31.3 us against 32.4 at 8 per row
// and 36-37 at 32, one GPU.
constexpr int kTopkSplitTarget = 1536;
constexpr int kTopkMinSlice4 = 1024;  // 16-byte groups

int topk_split_of(int rows, int cols, const float *logits)
{
    if (cols <= 8192 || (cols & 3) != 0 || !aligned(logits, 16) || rows >= kTopkSplitTarget / 2)
        return 1;
    const int64_t want = ceil_div(kTopkSplitTarget, rows);
    const int64_t cap = std::min<int64_t>(mqa::kTopkMaxSplit, (cols / 4) / kTopkMinSlice4);
    return (int)std::max<int64_t>(1, std::min(want, cap));
}

} // namespace

extern "C" size_t mqa_topk_workspace_size(int rows, int cols)
{
    if (rows <= 0 || cols <= 0 || (double)rows * ((double)cols + 64) * 8 > 1152921504606846976.0)
        return 0;
    return mqa::topk_split_workspace(nullptr, rows, cols).bytes;
}

extern "C" int mqa_topk_indices_ws(const float *logits, int rows, int cols, int k,
                                   int32_t *indices, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream)
{
    if (!workspace)
        return mqa_topk_indices(logits, rows, cols, k, indices, stream);
    if (rows < 0 || cols < 0)
        return fail(MQA_ERR_INVALID_ARG, "rows=%d, cols=%d must be >= 0", rows, cols);
    if (k < 1 || k > mqa::kMaxTopK)
        return fail(MQA_ERR_INVALID_ARG, "k must be in 1..%d (got %d)", mqa::kMaxTopK, k);
    if (rows == 0)
        return ok();
    if (!aligned(workspace, 256))
        return fail(MQA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const size_t need = mqa_topk_workspace_size(rows, cols);
    if (cols > 0 && (need == 0 || workspace_bytes < need))
        return fail(MQA_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu bytes "
                    "mqa_topk_workspace_size asks for", workspace_bytes, need);
    const int split = topk_split_of(rows, cols, logits);
    if (split < 2)
        return mqa_topk_indices(logits, rows, cols, k, indices, stream);
    if (!indices || !logits)
        return fail(MQA_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(indices, 4))
        return fail(MQA_ERR_INVALID_ARG, "indices must be 4-byte aligned");
    if (int rc = check_device())
        return rc;
    mqa::TopkSplitLaunch p;
    p.logits = logits;
    p.indices = indices;
    p.rows = rows;
    p.cols = cols;
    p.k = k;
    p.split = split;
    p.slice4 = (int)ceil_div(cols / 4, split);
    p.ws = mqa::topk_split_workspace(workspace, rows, cols);
    if (trace_on())
        std::fprintf(stderr, "[mqa] topk rows=%d cols=%d k=%d split=%d\n", rows, cols, k, split);
    hipError_t e = mqa::launch_topk_split(p, stream);
    if (e != hipSuccess)
        return fail(MQA_ERR_LAUNCH, "topk launch failed: %s", hipGetErrorString(e));
    return ok();
}

extern "C" int mqa_topk_indices(const float *logits, int rows, int cols, int k, int32_t *indices,
                                hipStream_t stream)
{
    if (rows < 0 || cols < 0)
        return fail(MQA_ERR_INVALID_ARG, "rows=%d, cols=%d must be >= 0", rows, cols);
    if (k < 1 || k > mqa::kMaxTopK)
        return fail(MQA_ERR_INVALID_ARG, "k must be in 1..%d (got %d)", mqa::kMaxTopK, k);
    if (rows == 0)
        return ok();
    if (!indices || (cols > 0 && !logits))
        return fail(MQA_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(logits, 4) || !aligned(indices, 4))
        return fail(MQA_ERR_INVALID_ARG, "logits and indices must be 4-byte aligned");
    if (int rc = check_device())
        return rc;
    mqa::TopkLaunch p;
    p.logits = logits;
    p.indices = indices;
    p.rows = rows;
    p.cols = cols;
    p.k = k;
    if (trace_on())
        std::fprintf(stderr, "[mqa] topk rows=%d cols=%d k=%d\n", rows, cols, k);
    hipError_t e = mqa::launch_topk(p, stream);
    if (e != hipSuccess)
        return fail(MQA_ERR_LAUNCH, "topk launch failed: %s", hipGetErrorString(e));
    return ok();
}

extern "C" int mqa_kcache_quantize_insert(const void *k, int k_dtype, const int64_t *slot_mapping,
                                          uint8_t *kv_cache, int num_tokens, int head_dim,
                                          int kv_block_size, int kv_layout, int num_blocks,
                                          hipStream_t stream)
{
    if (num_tokens < 0 || num_blocks < 0)
        return fail(MQA_ERR_INVALID_ARG, "num_tokens=%d, num_blocks=%d must be >= 0", num_tokens,
                    num_blocks);
    if (k_dtype != MQA_DTYPE_FP32 && k_dtype != MQA_DTYPE_BF16)
        return fail(MQA_ERR_INVALID_ARG, "k_dtype must be MQA_DTYPE_FP32 or MQA_DTYPE_BF16 (got %d)",
                    k_dtype);
    if (!shape_supported(32, head_dim, kv_block_size) || kv_block_size == 0)
        return fail(MQA_ERR_UNSUPPORTED,
                    "K-cache insert supports head_dim 128 or 64 and kv_block_size 1, 16, 64 or "
                    "128 "
                    "(got %d, %d)",
                    head_dim, kv_block_size);
    if (kv_layout != MQA_KV_SLOT_MAJOR && kv_layout != MQA_KV_PRESHUFFLED)
        return fail(MQA_ERR_INVALID_ARG, "kv_layout must be MQA_KV_SLOT_MAJOR or MQA_KV_PRESHUFFLED "
                    "(got %d)", kv_layout);
    if (kv_layout == MQA_KV_PRESHUFFLED && kv_block_size < 16)
        return fail(MQA_ERR_UNSUPPORTED, "the preshuffled layout needs kv_block_size 16, 64 or 128 "
                    "(got %d)", kv_block_size);
    if (num_tokens == 0)
        return ok();
    if (!k || !slot_mapping || !kv_cache)
        return fail(MQA_ERR_INVALID_ARG, "NULL pointer argument");
    if (!aligned(k, 16) || !aligned(kv_cache, 16) || !aligned(slot_mapping, 8))
        return fail(MQA_ERR_INVALID_ARG, "k and kv_cache must be 16-byte aligned, slot_mapping 8-byte");
    if (int rc = check_device())
        return rc;
    mqa::KcacheLaunch p;
    p.k = k;
    p.head_dim = head_dim;
    p.slots = slot_mapping;
    p.cache = kv_cache;
    p.tokens = num_tokens;
    p.block_size = kv_block_size;
    p.num_slots = (int64_t)num_blocks * kv_block_size;
    p.bf16 = k_dtype == MQA_DTYPE_BF16;
    p.tiled = kv_layout == MQA_KV_PRESHUFFLED;
    if (trace_on())
        std::fprintf(stderr, "[mqa] kcache insert tokens=%d dtype=%d\n", num_tokens, k_dtype);
    hipError_t e = mqa::launch_kcache_insert(p, stream);
    if (e != hipSuccess)
        return fail(MQA_ERR_LAUNCH, "kcache insert launch failed: %s", hipGetErrorString(e));
    return ok();
}
