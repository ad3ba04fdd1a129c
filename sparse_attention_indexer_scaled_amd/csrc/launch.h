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
    int head_tiles;  // num_heads / 32: 1, 2 or 4 (2 and 4: block size 64, depth 4)
    int tiled;       // 1: K rows in the preshuffled (16,16) order (block size >= 16)
};

// Largest k of the row-wise top-k.
constexpr int kMaxTopK = 2048;

struct TopkLaunch {
    const float *logits;
    int32_t *indices;
    int rows;
    int cols;
    int k;  // 1..kMaxTopK
};

struct KcacheLaunch {
    const void *k;        // [tokens, 128] fp32 or bf16
    const int64_t *slots; // [tokens]
    uint8_t *cache;       // [num_slots / block_size] blocks of block_size * 132 bytes
    int tokens;
    int block_size;
    int64_t num_slots;    // num_blocks * block_size
    int bf16;
    int tiled;            // 1: K rows in the preshuffled (16,16) order
};

// Bytes of LDS a decode workgroup uses for a ring of `depth` blocks.
int decode_ring_bytes(int depth);

hipError_t launch_prefill(const PrefillLaunch &p, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch &p, hipStream_t stream);
hipError_t launch_topk(const TopkLaunch &p, hipStream_t stream);
hipError_t launch_kcache_insert(const KcacheLaunch &p, hipStream_t stream);

} // namespace mqa
