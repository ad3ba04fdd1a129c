// Internal interface between the C-ABI entry points (api.cpp) and the kernel
// translation units.  Everything here is already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mqa {

struct PrefillLaunch {
    const uint8_t *q;
    const uint8_t *k;
    const float *kv_scale;
    const float *weights;
    const int32_t *ks;
    const int32_t *ke;
    float *logits;
    int M;
    int N;
    int clean;
    int block_m;   // rows per wave: 1, 2, 4 or 8
    int split_n;   // workgroups per row block
    int num_warps; // waves per workgroup
    int reverse;   // 1: high-m row blocks first
    int head_tiles;  // num_heads / 32: 1, 2 or 4
    int head_dim;    // 64 or 128
    int ring;        // 0: every wave streams its own K; else the shared-K ring's depth
};

struct DecodeLaunch {
    const uint8_t *q;
    const uint8_t *cache;
    const float *weights;
    const int32_t *context_lens;
    const int32_t *block_tables;
    float *logits;
    int batch;
    int next_n;
    int max_blocks_per_seq;
    int64_t max_model_len;
    int clean;
    int rows;      // rows per wave (R), 1..4, <= next_n; ceil(next_n / R) waves per workgroup
    int split_kv;  // workgroups per sequence
    int depth;     // 64-token steps in each workgroup's LDS ring, 2..7 (at most 64 KiB);
                   // 4 for block sizes other than 64
    int block_size;  // tokens per cache block: 1, 16, 64 or 128
    int head_tiles;  // num_heads / 32: 1, 2 or 4
    int head_dim;    // 128 or 64
    int tiled;       // 1: K rows in the preshuffled (16,16) order (block size >= 16)
    // fused top-k only (zero / NULL for the logits call):
    int mode;              // 0 logits, 1 sample, 2 filter (modes 1, 2: the default depth,
                           // 3 for 64-token blocks at 32 heads, else 4)
    float *sample;         // [rows][kFusedSampleCols]
    const uint32_t *threshold;  // [rows]
    uint64_t *entries;     // [rows][ent_stride]
    int *counts;           // [rows][split_kv]
    int64_t ent_stride;
};

// Fused decode top-k: sample shape (chunks of steps per sequence), largest KV
// split it accepts, and its workspace layout.
constexpr int kFusedSampleChunks = 16;
constexpr int kFusedSampleSteps = 4;
constexpr int kFusedSampleCols = kFusedSampleChunks * kFusedSampleSteps * 64;
constexpr int kFusedMaxSplit = 1024;

struct FusedWorkspace {
    uint64_t *entries;    // [rows][ent_stride]; a recomputed row's fp32 logits go to its own
    int *counts;          // [rows][kFusedMaxSplit]
    uint32_t *threshold;  // [rows]
    int *recomputed;      // [rows]: 1 where the select recomputed the row in full
    float *sample;        // [rows][kFusedSampleCols]
    int64_t ent_stride;
    size_t bytes;
};

inline size_t fused_align(size_t v) { return (v + 255) & ~(size_t)255; }

// Layout of the fused top-k workspace at `base` (NULL: sizes only).
inline FusedWorkspace fused_workspace(void *base, int rows, int64_t mml)
{
    FusedWorkspace w;
    w.ent_stride = (mml + 63) / 64 * 64;
    size_t off = 0;
    char *b = static_cast<char *>(base);
    auto take = [&](size_t n) {
        char *q = b ? b + off : nullptr;
        off = fused_align(off + n);
        return q;
    };
    w.entries = reinterpret_cast<uint64_t *>(take((size_t)rows * w.ent_stride * 8));
    w.counts = reinterpret_cast<int *>(take((size_t)rows * kFusedMaxSplit * 4));
    w.threshold = reinterpret_cast<uint32_t *>(take((size_t)rows * 4));
    w.recomputed = reinterpret_cast<int *>(take((size_t)rows * 4));
    w.sample = reinterpret_cast<float *>(take((size_t)rows * kFusedSampleCols * 4));
    w.bytes = off;
    return w;
}

// Largest k of the row-wise top-k.
constexpr int kMaxTopK = 2048;

struct TopkLaunch {
    const float *logits;
    int32_t *indices;
    int rows;
    int cols;
    int k;  // 1..kMaxTopK
};

// Split row top-k (mqa_topk_indices_ws): the workspace holds each row's
// segments (an entry region of ent_stride >= cols entries per row) and the
// slices' counts.
constexpr int kTopkMaxSplit = 64;

struct TopkSplitWorkspace {
    uint64_t *entries;  // [rows][ent_stride]
    int *counts;        // [rows][split]
    int64_t ent_stride;
    size_t bytes;
};

inline TopkSplitWorkspace topk_split_workspace(void *base, int rows, int cols)
{
    TopkSplitWorkspace w;
    w.ent_stride = ((int64_t)cols + 63) / 64 * 64;
    const size_t ent = fused_align((size_t)rows * w.ent_stride * 8);
    char *b = static_cast<char *>(base);
    w.entries = reinterpret_cast<uint64_t *>(b);
    w.counts = reinterpret_cast<int *>(b ? b + ent : nullptr);
    w.bytes = ent + fused_align((size_t)rows * kTopkMaxSplit * 4);
    return w;
}

struct TopkSplitLaunch {
    const float *logits;  // [rows, cols], 16-byte aligned rows (cols % 4 == 0)
    int32_t *indices;
    int rows;
    int cols;
    int k;
    int split;   // workgroups per row, 2..kTopkMaxSplit
    int slice4;  // 16-byte groups per workgroup
    TopkSplitWorkspace ws;
};

// Fused top-k steps after the sampling decode and before the filtering one
// (thresholds from the sample), and after it (select, or flag the row).
struct FusedTopkLaunch {
    const FusedWorkspace *ws;
    const int32_t *context_lens;
    int32_t *indices;
    int batch;
    int next_n;
    int mml;
    int k;
    int split;  // the filtering decode's KV split
    // what a row needs to be recomputed in full
    const uint8_t *q;
    const uint8_t *cache;
    const float *weights;
    const int32_t *block_tables;
    int max_blocks_per_seq;
    int tiled;
    int block_size;  // 1, 16, 64 or 128
    int head_tiles;  // num_heads / 32: 1, 2 or 4
    int head_dim;    // 128 or 64
};

struct KcacheLaunch {
    const void *k;        // [tokens, head_dim] fp32 or bf16
    const int64_t *slots; // [tokens]
    uint8_t *cache;       // [num_slots / block_size] blocks of block_size * (head_dim + 4) bytes
    int head_dim;         // 128, or 64 (blocks of 16 or more tokens)
    int tokens;
    int block_size;
    int64_t num_slots;    // num_blocks * block_size
    int bf16;
    int tiled;            // 1: K rows in the preshuffled (16,16) order
};


hipError_t launch_prefill(const PrefillLaunch &p, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch &p, hipStream_t stream);
hipError_t launch_decode_heads(const DecodeLaunch &p, hipStream_t stream);  // 64, 128 heads
hipError_t launch_decode_d64(const DecodeLaunch &p, hipStream_t stream);    // head dim 64
hipError_t launch_decode_fused(const DecodeLaunch &p, hipStream_t stream);  // modes 1 and 2
hipError_t launch_decode_fused_d64(const DecodeLaunch &p, hipStream_t stream);  // at head dim 64
hipError_t launch_topk(const TopkLaunch &p, hipStream_t stream);
hipError_t launch_topk_split(const TopkSplitLaunch &p, hipStream_t stream);
hipError_t launch_fused_threshold(const FusedTopkLaunch &p, hipStream_t stream);
hipError_t launch_fused_select(const FusedTopkLaunch &p, hipStream_t stream);
hipError_t launch_kcache_insert(const KcacheLaunch &p, hipStream_t stream);

} // namespace mqa
