// Prefill logits kernel (gfx950).
//
// What it computes (aiter PR 5046 page, "Motivation"): for query row m and
// K token n of a contiguous, already-gathered K buffer,
//   logits[m, n] = sum_h relu(<Q[m,h,:], K[n,:]>) * kv_scale[n] * weights[m,h]
// for max(ks[m],0) <= n < min(ke[m],N), and -inf elsewhere when clean_logits.
//
// Work decomposition.  A workgroup owns one block of BM consecutive query rows
// and one of `split` contiguous parts of that block's column range (both pages,
// "Technical Details": a row block shares one K stream; a column split fills the
// device when the row grid is small).  The column range is the union of the
// rows' windows rounded out to 64-column steps; the waves of the workgroup take
// interleaved steps of the part (waves split the tile range, not the rows, so
// each wave keeps its own independent K stream in flight).  Each wave keeps
// its BM rows' Q and weights in VGPRs and, per step, loads 64 K rows + scales
// straight into VGPRs (no LDS; the whole K buffer is shared by every row block
// and stays L2/MALL resident), runs 2 fp8 MFMAs per (row, 32-token tile), the
// in-lane relu.weight sum, one permlane32 swap + add per row pair, the
// once-per-column kv_scale multiply, and a masked store.  With clean_logits the
// same waves write -inf left and right of the column range.
//
// Row blocks are dispatched high-m first when the host asks (causal chunks:
// the last rows have the longest windows, so starting them first keeps them
// out of the tail; aiter PR 5046 page, "Technical Details").
#include "device.h"
#include "launch.h"

namespace mqa {
namespace {

struct PrefillArgs {
    const uint8_t *q;
    const uint8_t *k;
    const float *sc;
    const float *w;
    const int32_t *ks;
    const int32_t *ke;
    float *out;
    int M;
    int N;
    int clean;
    int split;
    int nrb;
    int reverse;
};

struct KStep {
    Frag t[2];
    float sc[2];
};

// Step starting at column n0.  Rows past N are clamped to N - 1: the load stays
// in bounds and the column is never stored.
__device__ __forceinline__ void load_kstep(KStep &k, const uint8_t *kbuf, const float *scale,
                                           int64_t n0, int N, int lane)
{
    const int t = lane & 31;
    const int64_t n_a = min(n0 + t, (int64_t)N - 1);
    const int64_t n_b = min(n0 + kTile + t, (int64_t)N - 1);
    load_frag(k.t[0], kbuf + n_a * kDim, lane);
    load_frag(k.t[1], kbuf + n_b * kDim, lane);
    k.sc[0] = scale[n_a];
    k.sc[1] = scale[n_b];
}

template <int BM>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a)
{
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    int id = blockIdx.x;
    const int s = id % a.split;
    int rb = id / a.split;
    if (a.reverse)
        rb = a.nrb - 1 - rb;
    const int m0 = rb * BM;
    const int nrows = min(BM, a.M - m0);
    const int N = a.N;
    const float ninf = -__builtin_inff();

    int lo[BM], hi[BM];
    int ulo = N, uhi = 0;
#pragma unroll
    for (int r = 0; r < BM; ++r) {
        lo[r] = 0;
        hi[r] = 0;
        if (r < nrows) {
            lo[r] = max(a.ks[m0 + r], 0);
            hi[r] = min(a.ke[m0 + r], N);
            if (hi[r] > lo[r]) {
                ulo = min(ulo, lo[r]);
                uhi = max(uhi, hi[r]);
            }
        }
    }
    if (uhi <= ulo) {
        ulo = 0;
        uhi = 0;
    }
    const int64_t sb = ulo / kStep;
    const int64_t se = ((int64_t)uhi + kStep - 1) / kStep;
    const int64_t nsteps = se - sb;
    const int64_t st0 = sb + nsteps * s / a.split;
    const int64_t st1 = sb + nsteps * (s + 1) / a.split;
    float *out = a.out + (int64_t)m0 * N;
    const int t = lane & 31;

    int64_t st = st0 + wave;
    if (st < st1) {
        Frag q[BM];
        Weights16 w[BM];
#pragma unroll
        for (int r = 0; r < BM; ++r) {
            if (r < nrows) {
                load_frag(q[r], a.q + (int64_t)(m0 + r) * (kHeads * kDim) + t * kDim, lane);
                load_weights(w[r], a.w + (int64_t)(m0 + r) * kHeads, lane);
            }
        }
        KStep cur;
        load_kstep(cur, a.k, a.sc, st * kStep, N, lane);
        for (; st < st1; st += nw) {
            const int64_t sn = min(st + nw, st1 - 1);
            KStep nxt;
            load_kstep(nxt, a.k, a.sc, sn * kStep, N, lane);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t n = st * kStep + h * kTile + t;
                float part[BM];
#pragma unroll
                for (int r = 0; r < BM; ++r)
                    if (r < nrows)
                        part[r] = relu_weight_sum(row_scores(q[r], cur.t[h]), w[r]);
#pragma unroll
                for (int r = 0; r < BM; r += 2) {
                    if (r < nrows) {
                        const bool has_b = (r + 1 < nrows);
                        // has_b implies r + 1 < BM; the clamp only keeps the
                        // index in range for the compiler.
                        const float pb = has_b ? part[(r + 1 < BM) ? r + 1 : r] : part[r];
                        const float tot = pair_head_sum(part[r], pb) * cur.sc[h];
                        const int rr = (lane < 32) ? r : r + 1;
                        const int rlo = (lane < 32) ? lo[r] : lo[(r + 1 < BM) ? r + 1 : r];
                        const int rhi = (lane < 32) ? hi[r] : hi[(r + 1 < BM) ? r + 1 : r];
                        const bool valid = n >= rlo && n < rhi;
                        if ((lane < 32 || has_b) && n < N && (valid || a.clean))
                            out[(int64_t)rr * N + n] = valid ? tot : ninf;
                    }
                }
            }
            cur = nxt;
        }
    }
    if (a.clean) {
        const int part = s * nw + wave;
        const int nparts = a.split * nw;
        const int64_t left = min(sb * kStep, (int64_t)N);
        const int64_t right = min(se * kStep, (int64_t)N);
        for (int r = 0; r < nrows; ++r) {
            fill_neg_inf(out + (int64_t)r * N, 0, left, part, nparts, lane);
            fill_neg_inf(out + (int64_t)r * N, right, N, part, nparts, lane);
        }
    }
}

template <int BM>
hipError_t launch_bm(const PrefillArgs &a, int grid, int block, hipStream_t stream)
{
    hipLaunchKernelGGL(prefill_kernel<BM>, dim3(grid), dim3(block), 0, stream, a);
    return hipGetLastError();
}

} // namespace

hipError_t launch_prefill(const PrefillLaunch &p, hipStream_t stream)
{
    PrefillArgs a;
    a.q = p.q;
    a.k = p.k;
    a.sc = p.kv_scale;
    a.w = p.weights;
    a.ks = p.ks;
    a.ke = p.ke;
    a.out = p.logits;
    a.M = p.M;
    a.N = p.N;
    a.clean = p.clean;
    a.split = p.split_n;
    a.nrb = (p.M + p.block_m - 1) / p.block_m;
    a.reverse = p.reverse;
    const int grid = a.nrb * a.split;
    const int block = 64 * p.num_warps;
    switch (p.block_m) {
    case 1: return launch_bm<1>(a, grid, block, stream);
    case 2: return launch_bm<2>(a, grid, block, stream);
    case 4: return launch_bm<4>(a, grid, block, stream);
    case 8: return launch_bm<8>(a, grid, block, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mqa
