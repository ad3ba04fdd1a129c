// Paged decode logits kernel (gfx950).
//
// What it computes (aiter PR 5047 page, "Motivation" and "Technical Details"):
// row j of sequence b gets  sum_h relu(<Q[b,j,h,:], K[p,:]>) * w[b,j,h] * scale[p]
// for every cached position p <= ctx_b - next_n + j, K and its per-token scale
// read from a paged cache through the block table; -inf elsewhere (fused fill).
//
// Work decomposition.  A workgroup owns one (sequence b, KV split s).  Its
// waves are G row groups x W KV streams: a row group is R consecutive next_n
// rows that share one K stream (both pages, "Technical Details": rows that
// share one K stream; the next_n-tiling issue page asks for exactly this,
// next_n folded into the tile rather than the program count).  G = 1 when all
// next_n rows fit one wave's registers; otherwise the G waves of a stream walk
// the same cache blocks together and all but one hit the CU's L1.  The
// sequence's KV range [0, nvalid) is cut into 64-token steps (one cache
// block), the steps into `split` contiguous parts, one per workgroup, and the
// W streams take interleaved steps of that part.  Each wave:
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

// Sizes and launch shape; the pointers are separate __restrict__ kernel
// arguments so the compiler may read the block table with scalar loads.
struct DecodeArgs {
    int mml;
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

// Scores, relu.weight sums and kv-scaled head sums for one cache block (two
// 32-token tiles) and the wave's R rows.  tot[h][i] holds the result of row
// pair i for tile h: lanes 0..31 row 2i, lanes 32..63 row 2i + 1.  Kept free
// of branches so the compiler can overlap one row's epilogue (VALU) with the
// next row's MFMAs.
template <int R>
__device__ __forceinline__ void step_scores(const KStep &k, const Frag (&q)[R],
                                            const Weights16 (&w)[R], float (&tot)[2][(R + 1) / 2])
{
    // Row-tiles in the order (tile 0: rows 0..R-1, tile 1: rows 0..R-1), software
    // pipelined by one: the MFMAs of row-tile i+1 are issued before the
    // relu.weight epilogue of row-tile i, so the epilogue never waits for the
    // MFMA it consumes and the matrix core has work queued meanwhile.
    constexpr int NT = 2 * R;
    float part[2][R];
    f32x16 prev = row_scores(q[0], k.t[0]);
#pragma unroll
    for (int it = 1; it < NT; ++it) {
        const int h = it / R, r = it % R;
        const int ph = (it - 1) / R, pr = (it - 1) % R;
        f32x16 cur = row_scores(q[r], k.t[h]);
        part[ph][pr] = relu_weight_sum(prev, w[pr]);
        prev = cur;
    }
    part[1][R - 1] = relu_weight_sum(prev, w[R - 1]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < (R + 1) / 2; ++i) {
            // an odd last row is paired with itself; its upper half is never stored
            const float pb = (2 * i + 1 < R) ? part[h][(2 * i + 1 < R) ? 2 * i + 1 : 2 * i] : part[h][2 * i];
            tot[h][i] = pair_head_sum(part[h][2 * i], pb) * k.sc[h];
        }
    }
}

// Up to 8 waves per workgroup while a wave fits in 256 registers (2 waves per
// SIMD), 4 once it needs more.
template <int R>
constexpr int max_block() { return R <= 4 ? 512 : 256; }

template <int R>
__global__ __launch_bounds__(max_block<R>()) void decode_kernel(const uint8_t *__restrict__ qbuf,
                                                     const uint8_t *__restrict__ cache,
                                                     const float *__restrict__ wbuf,
                                                     const int32_t *__restrict__ ctx_lens,
                                                     const int32_t *__restrict__ tables,
                                                     float *__restrict__ logits, DecodeArgs a)
{
    constexpr int NP = (R + 1) / 2;
    const int lane = lane_id();
    // Wave layout: the workgroup's waves are `groups` row groups x nw KV
    // streams.  The row groups of one stream walk the same cache blocks side
    // by side, so all but the first read each block from the CU's L1.
    const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave_all % a.groups;
    const int wave = wave_all / a.groups;
    const int nw = (blockDim.x >> 6) / a.groups;
    const int s = blockIdx.x % a.split;
    const int b = blockIdx.x / a.split;

    const int ctx = ctx_lens[b];
    const int mml = a.mml;
    const int row0 = grp * R;
    const int nrows = min(R, a.next_n - row0);
    // Inclusive bound of the group's first row; row row0 + i covers p <= first_bound + i.
    const int first_bound = ctx - a.next_n + row0;
    const int nvalid = max(min(min(first_bound + nrows, ctx), mml), 0);
    const int nsteps = (nvalid + kStep - 1) / kStep;
    const int st0 = (int)((int64_t)nsteps * s / a.split);
    const int st1 = (int)((int64_t)nsteps * (s + 1) / a.split);
    const int64_t row_base = (int64_t)b * a.next_n + row0;
    float *out = logits + row_base * mml;
    const int t = lane & 31;
    const int half = lane >> 5;
    const float ninf = -__builtin_inff();

    int st = st0 + wave;
    if (st < st1) {
        Frag q[R];
        Weights16 w[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            // a short last group computes its missing rows as copies of its
            // last row and never stores them: the loop body stays branch-free
            const int64_t row = row_base + min(r, nrows - 1);
            load_frag(q[r], qbuf + row * (kHeads * kDim) + t * kDim, lane);
            load_weights(w[r], wbuf + row * kHeads, lane);
        }
        // This lane's output row within each pair and its window bound.
        float *orow[NP];
        int obound[NP];
        bool ostore[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int rr = 2 * i + half;
            orow[i] = out + (int64_t)min(rr, nrows - 1) * mml;
            obound[i] = first_bound + rr;
            ostore[i] = rr < nrows;
        }
        const bool clean = a.clean != 0;
        auto store_step = [&](int step, const float (&tot)[2][NP]) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int p = step * kStep + h * kTile + t;
#pragma unroll
                for (int i = 0; i < NP; ++i) {
                    const bool valid = p <= obound[i];
                    if (ostore[i] && p < mml && (valid || clean))
                        orow[i][p] = valid ? tot[h][i] : ninf;
                }
            }
        };

        // Two step buffers used alternately.  Each half issues the next
        // step's K loads, then the scalar load of the table entry one step
        // further on, then waits for and computes the current step; the
        // sched_barriers pin that order, so a step's loads are always in
        // flight while the previous one computes and no wait for a table
        // entry ever stalls behind freshly issued loads.
        const int32_t *table = tables + (int64_t)b * a.mbps;
        KStep A, B;
        load_kstep(A, cache + (int64_t)table[st] * kBlockBytes, lane);
        int ph_next = table[min(st + nw, st1 - 1)];
        while (true) {
            load_kstep(B, cache + (int64_t)ph_next * kBlockBytes, lane);
            __builtin_amdgcn_sched_barrier(0);
            ph_next = table[min(st + 2 * nw, st1 - 1)];
            __builtin_amdgcn_sched_barrier(0);
            float tot[2][NP];
            step_scores<R>(A, q, w, tot);
            store_step(st, tot);
            st += nw;
            if (st >= st1)
                break;
            load_kstep(A, cache + (int64_t)ph_next * kBlockBytes, lane);
            __builtin_amdgcn_sched_barrier(0);
            ph_next = table[min(st + 2 * nw, st1 - 1)];
            __builtin_amdgcn_sched_barrier(0);
            step_scores<R>(B, q, w, tot);
            store_step(st, tot);
            st += nw;
            if (st >= st1)
                break;
        }
    }
    if (a.clean) {
        const int64_t f0 = min((int64_t)nsteps * kStep, (int64_t)mml);
        for (int r = 0; r < nrows; ++r)
            fill_neg_inf(out + (int64_t)r * mml, f0, mml, s * nw + wave, a.split * nw, lane);
    }
}

template <int R>
hipError_t launch_r(const DecodeLaunch &p, const DecodeArgs &a, int grid, int block,
                    hipStream_t stream)
{
    hipLaunchKernelGGL(decode_kernel<R>, dim3(grid), dim3(block), 0, stream, p.q, p.cache,
                       p.weights, p.context_lens, p.block_tables, p.logits, a);
    return hipGetLastError();
}

} // namespace

hipError_t launch_decode(const DecodeLaunch &p, hipStream_t stream)
{
    DecodeArgs a;
    a.mml = (int)p.max_model_len;
    a.next_n = p.next_n;
    a.mbps = p.max_blocks_per_seq;
    a.clean = p.clean;
    a.groups = (p.next_n + p.rows - 1) / p.rows;
    a.split = p.split_kv;
    const int grid = p.batch * a.split;
    const int block = 64 * p.num_warps * a.groups;
    switch (p.rows) {
    case 1: return launch_r<1>(p, a, grid, block, stream);
    case 2: return launch_r<2>(p, a, grid, block, stream);
    case 3: return launch_r<3>(p, a, grid, block, stream);
    case 4: return launch_r<4>(p, a, grid, block, stream);
    case 5: return launch_r<5>(p, a, grid, block, stream);
    case 6: return launch_r<6>(p, a, grid, block, stream);
    case 7: return launch_r<7>(p, a, grid, block, stream);
    case 8: return launch_r<8>(p, a, grid, block, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mqa
