// Paged decode logits kernel (gfx950).
//
// What it computes (aiter PR 5047 page, "Motivation" and "Technical Details"):
// row j of sequence b gets  sum_h relu(<Q[b,j,h,:], K[p,:]>) * w[b,j,h] * scale[p]
// for every cached position p <= ctx_b - next_n + j, K and its per-token scale
// read from a paged cache through the block table; -inf elsewhere (fused fill).
//
// Work decomposition.  A workgroup owns one (sequence b, group of R
// consecutive next_n rows, KV split s).  The R rows share one K stream: every
// K byte a wave loads is used by all R rows (both pages, "Technical Details":
// rows that share one K stream; the next_n-tiling issue page asks for exactly
// this, next_n folded into the tile instead of the program count).  The
// group's KV range [0, nvalid) is cut into 64-token steps (one cache block),
// the steps into `split` contiguous parts, one per workgroup, and the waves of
// a workgroup take interleaved steps of that part.  Each wave:
//   - keeps its R rows' Q (16 VGPR each) and head weights (16 VGPR each) in
//     registers for its whole life;
//   - per step, reads one block-table entry (scalar load), the block's 64 K
//     rows straight from HBM into VGPRs (no LDS) and the 64 scales, with the
//     next step's loads in flight while this one computes;
//   - per 32-token tile and row, runs two fp8 MFMAs, the in-lane relu.weight
//     sum over 16 heads, and pairs rows for one permlane32 swap + add;
//   - scales by kv_scale once per column (the hoist: kv_scale >= 0 and relu is
//     positive-homogeneous) and stores 64 lanes = 2 rows x 32 tokens.
// Positions past the group's window up to max_model_len are written -inf by
// the same waves, split the same way.  A position is selected by an integer
// compare, never by arithmetic, so cache slots past the context (which may
// hold NaN bytes) cannot reach an output.
#include "device.h"
#include "launch.h"

namespace mqa {
namespace {

struct DecodeArgs {
    const uint8_t *q;
    const uint8_t *cache;
    const float *w;
    const int32_t *ctx;
    const int32_t *bt;
    float *out;
    int64_t mml;
    int next_n;
    int mbps;
    int clean;
    int groups;
    int split;
};

// One 64-token cache block: two K tiles and the 64 scales.
struct KStep {
    Frag t[2];
    float sc[2];
};

__device__ __forceinline__ void load_kstep(KStep &k, const uint8_t *blk, int lane)
{
    const int t = lane & 31;
    load_frag(k.t[0], blk + t * kDim, lane);
    load_frag(k.t[1], blk + (kTile + t) * kDim, lane);
    const float *sc = reinterpret_cast<const float *>(blk + kBlock * kDim);
    k.sc[0] = sc[t];
    k.sc[1] = sc[kTile + t];
}

template <int R>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a)
{
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    int id = blockIdx.x;
    const int s = id % a.split;
    id /= a.split;
    const int grp = id % a.groups;
    const int b = id / a.groups;

    const int ctx = a.ctx[b];
    const int row0 = grp * R;
    const int nrows = min(R, a.next_n - row0);
    // Inclusive bound of the group's first row; row row0 + i covers p <= first_bound + i.
    const int64_t first_bound = (int64_t)ctx - a.next_n + row0;
    int64_t nvalid = first_bound + nrows;
    nvalid = min(nvalid, (int64_t)ctx);
    nvalid = min(nvalid, a.mml);
    nvalid = max(nvalid, (int64_t)0);
    const int64_t nsteps = (nvalid + kStep - 1) / kStep;
    const int64_t st0 = nsteps * s / a.split;
    const int64_t st1 = nsteps * (s + 1) / a.split;
    const int64_t row_base = (int64_t)b * a.next_n + row0;
    float *out = a.out + row_base * a.mml;
    const int t = lane & 31;
    const float ninf = -__builtin_inff();

    int64_t st = st0 + wave;
    if (st < st1) {
        Frag q[R];
        Weights16 w[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r < nrows) {
                load_frag(q[r], a.q + (row_base + r) * (kHeads * kDim) + t * kDim, lane);
                load_weights(w[r], a.w + (row_base + r) * kHeads, lane);
            }
        }
        const int32_t *table = a.bt + (int64_t)b * a.mbps;
        KStep cur;
        load_kstep(cur, a.cache + (int64_t)table[st] * kBlockBytes, lane);
        for (; st < st1; st += nw) {
            // Prefetch the wave's next step (the last step re-reads itself,
            // which keeps every load in bounds without a branch).
            const int64_t sn = min(st + nw, st1 - 1);
            KStep nxt;
            load_kstep(nxt, a.cache + (int64_t)table[sn] * kBlockBytes, lane);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t p = st * kStep + h * kTile + t;
                float part[R];
#pragma unroll
                for (int r = 0; r < R; ++r)
                    if (r < nrows)
                        part[r] = relu_weight_sum(row_scores(q[r], cur.t[h]), w[r]);
#pragma unroll
                for (int r = 0; r < R; r += 2) {
                    if (r < nrows) {
                        const bool has_b = (r + 1 < nrows);
                        // has_b implies r + 1 < R; the clamp only keeps the
                        // index in range for the compiler.
                        const float pb = has_b ? part[(r + 1 < R) ? r + 1 : r] : part[r];
                        const float tot = pair_head_sum(part[r], pb) * cur.sc[h];
                        const int rr = (lane < 32) ? r : r + 1;
                        const bool valid = p <= first_bound + rr;
                        if ((lane < 32 || has_b) && p < a.mml && (valid || a.clean))
                            out[rr * a.mml + p] = valid ? tot : ninf;
                    }
                }
            }
            cur = nxt;
        }
    }
    if (a.clean) {
        const int64_t f0 = min(nsteps * kStep, a.mml);
        for (int r = 0; r < nrows; ++r)
            fill_neg_inf(out + r * a.mml, f0, a.mml, s * nw + wave, a.split * nw, lane);
    }
}

template <int R>
hipError_t launch_r(const DecodeArgs &a, int grid, int block, hipStream_t stream)
{
    hipLaunchKernelGGL(decode_kernel<R>, dim3(grid), dim3(block), 0, stream, a);
    return hipGetLastError();
}

} // namespace

hipError_t launch_decode(const DecodeLaunch &p, hipStream_t stream)
{
    DecodeArgs a;
    a.q = p.q;
    a.cache = p.cache;
    a.w = p.weights;
    a.ctx = p.context_lens;
    a.bt = p.block_tables;
    a.out = p.logits;
    a.mml = p.max_model_len;
    a.next_n = p.next_n;
    a.mbps = p.max_blocks_per_seq;
    a.clean = p.clean;
    a.groups = (p.next_n + p.rows - 1) / p.rows;
    a.split = p.split_kv;
    const int grid = p.batch * a.groups * a.split;
    const int block = 64 * p.num_warps;
    switch (p.rows) {
    case 1: return launch_r<1>(a, grid, block, stream);
    case 2: return launch_r<2>(a, grid, block, stream);
    case 3: return launch_r<3>(a, grid, block, stream);
    case 4: return launch_r<4>(a, grid, block, stream);
    case 5: return launch_r<5>(a, grid, block, stream);
    case 6: return launch_r<6>(a, grid, block, stream);
    case 7: return launch_r<7>(a, grid, block, stream);
    case 8: return launch_r<8>(a, grid, block, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mqa
