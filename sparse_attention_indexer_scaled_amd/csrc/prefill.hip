// Prefill logits kernel (gfx950).
//
// What it computes (aiter PR 5046 page, "Motivation"): for query row m and
// K token n of a contiguous, already-gathered K buffer,
//   logits[m, n] = sum_h relu(<Q[m,h,:], K[n,:]>) * kv_scale[n] * weights[m,h]
// for max(ks[m],0) <= n < min(ke[m],N), and -inf elsewhere when clean_logits.
//
// Two kernels, one arithmetic (the same step_scores and stores, so the same
// bits).  Both give a workgroup a block of consecutive query rows and one of
// `split` contiguous parts of the block's column range (both pages, "Technical
// Details": a row block shares one K stream; a column split fills the device
// when the row grid is small); the column range is the union of the rows'
// windows rounded out to 64-column steps.  Each wave keeps its rows' Q and
// weights in VGPRs and per step runs D/64 fp8 MFMAs per (row, 32-token tile),
// the in-lane relu.weight sum, one permlane32 swap + add per row pair, the
// once-per-column kv_scale multiply and a masked store; with clean_logits the
// same waves write -inf left and right of the column range.
//
//   prefill_kernel (per-wave K; head dim 64, small problems): a workgroup owns
//     BM rows and its waves take interleaved steps of the part, each loading
//     its steps' 64 K rows + scales straight into VGPRs one step ahead.
//   prefill_ring_kernel (shared K; the default at head dim 128): a workgroup
//     of 4 waves owns 4 BM rows, every wave walks every step for its own BM
//     rows, and the step arrives once for all four through an LDS ring (see
//     the shared-K section below).
//
// Row blocks are dispatched high-m first when the host asks (causal chunks:
// the last rows have the longest windows, so starting them first keeps them
// out of the tail; aiter PR 5046 page, "Technical Details").
#include "device.h"
#include "launch.h"
#include "ring.h"

namespace mqa {
namespace {

// Sizes and launch shape; the pointers are separate __restrict__ kernel
// arguments so the compiler knows the output never aliases an input.
struct PrefillArgs {
    int M;
    int N;
    int clean;
    int split;
    int nrb;
    int reverse;
};


// Step starting at column n0.  Rows past N are clamped to N - 1: the load stays
// in bounds and the column is never stored.  A step that ends at or before N
// (every step but possibly the last) needs no clamp; that path is only taken
// at 32 heads (FAST), where it does not cost the kernel a wave per SIMD.
template <int D, bool FAST>
__device__ __forceinline__ void load_kstep(KStepOf<D> &k, const uint8_t *kbuf, const float *scale,
                                           int64_t n0, int N, int lane)
{
    const int t = lane & 31;
    if (FAST && n0 + kStep <= N) {
        const uint8_t *p = kbuf + (n0 + t) * D;
        load_frag(k.t[0], p, lane);
        load_frag(k.t[1], p + kTile * D, lane);
        k.sc[0] = scale[n0 + t];
        k.sc[1] = scale[n0 + kTile + t];
        return;
    }
    const int64_t n_a = min(n0 + t, (int64_t)N - 1);
    const int64_t n_b = min(n0 + kTile + t, (int64_t)N - 1);
    load_frag(k.t[0], kbuf + n_a * D, lane);
    load_frag(k.t[1], kbuf + n_b * D, lane);
    k.sc[0] = scale[n_a];
    k.sc[1] = scale[n_b];
}

template <int BM, int HT, int D>
__global__ __launch_bounds__(256) void prefill_kernel(const uint8_t *__restrict__ qbuf,
                                                      const uint8_t *__restrict__ kbuf,
                                                      const float *__restrict__ scale,
                                                      const float *__restrict__ wbuf,
                                                      const int32_t *__restrict__ ks,
                                                      const int32_t *__restrict__ ke,
                                                      float *__restrict__ logits, PrefillArgs a)
{
    constexpr int NP = (BM + 1) / 2;
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
    // Columns inside every row's window: [ilo, ihi) (empty unless the block
    // has all BM rows and each of them a non-empty window)
    int ilo = 0, ihi = nrows == BM ? N : 0;
#pragma unroll
    for (int r = 0; r < BM; ++r) {
        lo[r] = 0;
        hi[r] = 0;
        if (r < nrows) {
            lo[r] = max(ks[m0 + r], 0);
            hi[r] = min(ke[m0 + r], N);
            if (hi[r] > lo[r]) {
                ulo = min(ulo, lo[r]);
                uhi = max(uhi, hi[r]);
            }
            ilo = max(ilo, lo[r]);
            ihi = min(ihi, hi[r]);
        }
    }
    if (uhi <= ulo) {
        ulo = 0;
        uhi = 0;
    }
    const int sb = ulo / kStep;
    const int se = (uhi + kStep - 1) / kStep;
    const int nsteps = se - sb;
    const int st0 = sb + (int)((int64_t)nsteps * s / a.split);
    const int st1 = sb + (int)((int64_t)nsteps * (s + 1) / a.split);
    float *out = logits + (int64_t)m0 * N;
    const int t = lane & 31;
    const int half = lane >> 5;
    // Window of this lane's row in each pair.
    int rlo[NP], rhi[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int ra = 2 * i, rb2 = (2 * i + 1 < BM) ? 2 * i + 1 : 2 * i;
        rlo[i] = half ? lo[rb2] : lo[ra];
        rhi[i] = half ? hi[rb2] : hi[ra];
        if (half && 2 * i + 1 >= BM)
            rhi[i] = 0; // no such row
    }

    int st = st0 + wave;
    if (st < st1) {
        constexpr int H = kHeads * HT;
        Operand<D> q[BM][HT];
        Weights16 w[BM][HT];
#pragma unroll
        for (int r = 0; r < BM; ++r) {
            const int64_t row = m0 + min(r, nrows - 1);
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                load_frag(q[r][ht], qbuf + row * (H * D) + (ht * kHeads + t) * D, lane);
                load_weights(w[r][ht], wbuf + row * H + ht * kHeads, lane);
            }
        }
        // this lane's output element relative to row 2i, column 0 of a pair.
        // Logits are stored non-temporally: they are written once and never
        // read here, and K, which every row block re-reads, keeps the L2 (the
        // long chunk 542.6 -> 536.5 us, head dim 64 337.2 -> 332.5 us, one GPU).
        const int laneoff = half * N + t;
        auto store_step = [&](int step, const float (&tot)[2][NP]) {
            const int n0 = step * kStep;
            if (HT == 1 && n0 >= ilo && n0 + kStep <= ihi) {
                // every column of the step is inside every row's window (and
                // the block has all BM rows; an odd BM's last pair is a single
                // row whose upper half stores nothing)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < NP; ++i)
                        if (2 * i + 1 < BM || !half)
                            __builtin_nontemporal_store(
                                tot[h][i], &(out + (int64_t)(2 * i) * N + n0 + h * kTile)[laneoff]);
                return;
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int n = step * kStep + h * kTile + t;
#pragma unroll
                for (int i = 0; i < NP; ++i) {
                    const int rr = 2 * i + half;
                    const bool valid = n >= rlo[i] && n < rhi[i];
                    if (rr < nrows && n < N && (valid || a.clean))
                        __builtin_nontemporal_store(valid ? tot[h][i] : ninf,
                                                    &out[(int64_t)rr * N + n]);
                }
            }
        };
        // Two step buffers used alternately; each half issues the next
        // step's loads before waiting for the current one (the
        // sched_barrier keeps the compiler from hoisting the wait above them).
        KStepOf<D> A, B;
        load_kstep<D, HT == 1>(A, kbuf, scale, (int64_t)st * kStep, N, lane);
        while (true) {
            load_kstep<D, HT == 1>(B, kbuf, scale, (int64_t)min(st + nw, st1 - 1) * kStep, N, lane);
            __builtin_amdgcn_sched_barrier(0);
            float tot[2][NP];
            step_scores<BM, HT, D>(A, q, w, tot);
            store_step(st, tot);
            st += nw;
            if (st >= st1)
                break;
            load_kstep<D, HT == 1>(A, kbuf, scale, (int64_t)min(st + nw, st1 - 1) * kStep, N, lane);
            __builtin_amdgcn_sched_barrier(0);
            step_scores<BM, HT, D>(B, q, w, tot);
            store_step(st, tot);
            st += nw;
            if (st >= st1)
                break;
        }
    }
    if (a.clean) {
        const int part = s * nw + wave;
        const int nparts = a.split * nw;
        const int64_t left = min((int64_t)sb * kStep, (int64_t)N);
        const int64_t right = min((int64_t)se * kStep, (int64_t)N);
        for (int r = 0; r < nrows; ++r) {
            fill_neg_inf(out + (int64_t)r * N, 0, left, part, nparts, lane);
            fill_neg_inf(out + (int64_t)r * N, right, N, part, nparts, lane);
        }
    }
}

// ---- shared-K variant -------------------------------------------------------
// The kernel above gives every wave its own K stream, one step ahead in VGPRs.
// Here a workgroup of G waves owns G BM consecutive rows (wave g: rows g BM ..
// g BM + BM - 1) and one part of the union of their windows, and its waves
// share each K step through an LDS ring of DR slots, the decode's slot layout
// (ring.h): the step's 1 KiB chunks and its 256 bytes of scales are split
// between the waves' global->LDS loads, step k + DR - 1 is requested while step
// k computes, one barrier per step publishes a slot, and every wave reads the
// step from LDS into the MFMA operand layout.  K is requested DR - 1 steps
// ahead without holding a register, and it leaves L2 once per workgroup and
// step instead of once per wave.  A step's rows past N are read as row N - 1
// (never stored).  The loads keep the default cache policy: every row block
// reads K again, so K should stay in L2.
template <int G, int DIM>
__device__ __forceinline__ void request_contig(lds_u8 *slot, const uint8_t *kbuf,
                                               const float *scale, int64_t n0, int N, int g,
                                               int lane)
{
    constexpr int KC = k_chunks<DIM>();
    constexpr int TPC = rows_per_chunk<DIM>();
    constexpr int J = (KC + G - 1) / G;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int c = g + G * j;
        if (G * J == KC || c < KC) {
            // granule q = TPC u + tau: 16-byte granule u of chunk row tau
            const int q = DIM == 128 ? lane ^ (8 * (c & 1)) : lane;
            const int64_t row = min(n0 + TPC * c + q % TPC, (int64_t)N - 1);
            __builtin_amdgcn_global_load_lds(kbuf + row * DIM + (q / TPC) * 16, slot + 1024 * c,
                                             16, 0, 0);
        }
    }
    if (G == 1 || g == G - 1)
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const uint8_t *>(scale + min(n0 + lane, (int64_t)N - 1)),
            slot + kStep * DIM, 4, 0, 0);
}

template <int BM, int HT, int G, int DR, int D>
__global__ __launch_bounds__(64 * G) void prefill_ring_kernel(const uint8_t *__restrict__ qbuf,
                                                              const uint8_t *__restrict__ kbuf,
                                                              const float *__restrict__ scale,
                                                              const float *__restrict__ wbuf,
                                                              const int32_t *__restrict__ ks,
                                                              const int32_t *__restrict__ ke,
                                                              float *__restrict__ logits,
                                                              PrefillArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t ring_mem[];
    constexpr int NP = (BM + 1) / 2;
    constexpr int RB = G * BM;
    constexpr int SB = slot_bytes<D>();
    const int lane = lane_id();
    const int g = G == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int s = blockIdx.x % a.split;
    int rb = blockIdx.x / a.split;
    if (a.reverse)
        rb = a.nrb - 1 - rb;
    const int M = a.M, N = a.N;
    const int wm0 = rb * RB;     // the workgroup's first row
    const int m0 = wm0 + g * BM;  // this wave's first row
    const int nrows = max(0, min(BM, M - m0));
    const float ninf = -__builtin_inff();

    // The union of every row's window in the workgroup: all waves walk the
    // same steps (one K stream).
    int ulo = N, uhi = 0;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        if (wm0 + r < M) {
            const int l = max(ks[wm0 + r], 0), h = min(ke[wm0 + r], N);
            if (h > l) {
                ulo = min(ulo, l);
                uhi = max(uhi, h);
            }
        }
    }
    if (uhi <= ulo) {
        ulo = 0;
        uhi = 0;
    }
    // This wave's rows: windows, and the columns inside all of them [ilo, ihi)
    int lo[BM], hi[BM];
    int ilo = 0, ihi = nrows == BM ? N : 0;
#pragma unroll
    for (int r = 0; r < BM; ++r) {
        lo[r] = 0;
        hi[r] = 0;
        if (r < nrows) {
            lo[r] = max(ks[m0 + r], 0);
            hi[r] = min(ke[m0 + r], N);
            ilo = max(ilo, lo[r]);
            ihi = min(ihi, hi[r]);
        }
    }
    const int sb = ulo / kStep;
    const int se = (uhi + kStep - 1) / kStep;
    const int nsteps = se - sb;
    const int st0 = sb + (int)((int64_t)nsteps * s / a.split);
    const int st1 = sb + (int)((int64_t)nsteps * (s + 1) / a.split);
    float *out = logits + (int64_t)min(m0, M - 1) * N;
    const int t = lane & 31;
    const int half = lane >> 5;
    int rlo[NP], rhi[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int ra = 2 * i, rb2 = (2 * i + 1 < BM) ? 2 * i + 1 : 2 * i;
        rlo[i] = half ? lo[rb2] : lo[ra];
        rhi[i] = half ? hi[rb2] : hi[ra];
        if (half && 2 * i + 1 >= BM)
            rhi[i] = 0;  // no such row
    }

    if (st0 < st1) {  // uniform over the workgroup
        constexpr int H = kHeads * HT;
        Operand<D> q[BM][HT];
        Weights16 w[BM][HT];
#pragma unroll
        for (int r = 0; r < BM; ++r) {
            const int64_t row = min(m0 + r, M - 1);  // rows past M: computed, never stored
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                load_frag(q[r][ht], qbuf + row * (H * D) + (ht * kHeads + t) * D, lane);
                load_weights(w[r][ht], wbuf + row * H + ht * kHeads, lane);
            }
        }
        const int laneoff = half * N + t;
        auto store_step = [&](int step, const float (&tot)[2][NP]) {
            const int n0 = step * kStep;
            if (n0 >= ilo && n0 + kStep <= ihi) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < NP; ++i)
                        if (2 * i + 1 < BM || !half)
                            __builtin_nontemporal_store(
                                tot[h][i], &(out + (int64_t)(2 * i) * N + n0 + h * kTile)[laneoff]);
                return;
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int n = n0 + h * kTile + t;
#pragma unroll
                for (int i = 0; i < NP; ++i) {
                    const int rr = 2 * i + half;
                    const bool valid = n >= rlo[i] && n < rhi[i];
                    if (rr < nrows && n < N && (valid || a.clean))
                        __builtin_nontemporal_store(valid ? tot[h][i] : ninf,
                                                    &out[(int64_t)rr * N + n]);
                }
            }
        };
        lds_u8 *ring = (lds_u8 *)ring_mem;
        const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
#pragma unroll
        for (int i = 0; i < DR - 1; ++i)
            if (st0 + i < st1)
                request_contig<G, D>(ring + i * SB, kbuf, scale, (int64_t)(st0 + i) * kStep, N, g,
                                     lane);
        // Between requesting step k and waiting for it a wave requests the
        // DR - 2 following steps, at least min_loads_per_step loads each (loads
        // complete in order; stores counted as well only make the wait stricter).
        constexpr int kWait = (DR - 2) * min_loads_per_step(G, 1, k_chunks<D>());
        int rd = 0, wr = DR - 1;
        float prev_tot[2][NP];
        for (int st = st0; st < st1; ++st) {
            if (st + DR - 2 < st1)
                wait_vm<kWait>();
            else
                wait_vm<0>();
            __builtin_amdgcn_s_barrier();
            if (st + DR - 1 < st1)
                request_contig<G, D>(ring + wr * SB, kbuf, scale, (int64_t)(st + DR - 1) * kStep,
                                     N, g, lane);
            KStepOf<D> kb;
            read_block<D>(kb, ring_addr + rd * SB, lane);
            if (st > st0)
                store_step(st - 1, prev_tot);
            rd = (rd + 1 == DR) ? 0 : rd + 1;
            wr = (wr + 1 == DR) ? 0 : wr + 1;
            read_wait<D>(kb);
            step_scores<BM, HT, D>(kb, q, w, prev_tot);
        }
        store_step(st1 - 1, prev_tot);
        // no global->LDS load may still be in flight when the workgroup ends
        wait_vm<0>();
    }
    if (a.clean) {
        const int64_t left = min((int64_t)sb * kStep, (int64_t)N);
        const int64_t right = min((int64_t)se * kStep, (int64_t)N);
        for (int r = 0; r < nrows; ++r) {
            fill_neg_inf(out + (int64_t)r * N, 0, left, s, a.split, lane);
            fill_neg_inf(out + (int64_t)r * N, right, N, s, a.split, lane);
        }
    }
}

template <int BM, int HT, int G, int DR, int D>
hipError_t launch_ring(const PrefillLaunch &p, const PrefillArgs &a, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL((prefill_ring_kernel<BM, HT, G, DR, D>), dim3(grid), dim3(64 * G),
                       DR * slot_bytes<D>(), stream, p.q, p.k, p.kv_scale, p.weights, p.ks, p.ke,
                       p.logits, a);
    return hipGetLastError();
}

template <int BM, int HT, int D>
hipError_t launch_bm(const PrefillLaunch &p, const PrefillArgs &a, int grid, int block,
                     hipStream_t stream)
{
    hipLaunchKernelGGL((prefill_kernel<BM, HT, D>), dim3(grid), dim3(block), 0, stream, p.q, p.k,
                       p.kv_scale, p.weights, p.ks, p.ke, p.logits, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dim(const PrefillLaunch &p, const PrefillArgs &a, int grid, int block,
                      hipStream_t stream)
{
    if (p.head_tiles == 2) {  // 64 heads: at most 4 rows per wave
        switch (p.block_m) {
        case 1: return launch_bm<1, 2, D>(p, a, grid, block, stream);
        case 2: return launch_bm<2, 2, D>(p, a, grid, block, stream);
        case 4: return launch_bm<4, 2, D>(p, a, grid, block, stream);
        default: return hipErrorInvalidValue;
        }
    }
    if (p.head_tiles == 4) {  // 128 heads: at most 2 rows per wave
        switch (p.block_m) {
        case 1: return launch_bm<1, 4, D>(p, a, grid, block, stream);
        case 2: return launch_bm<2, 4, D>(p, a, grid, block, stream);
        default: return hipErrorInvalidValue;
        }
    }
    switch (p.block_m) {
    case 1: return launch_bm<1, 1, D>(p, a, grid, block, stream);
    case 2: return launch_bm<2, 1, D>(p, a, grid, block, stream);
    case 4: return launch_bm<4, 1, D>(p, a, grid, block, stream);
    case 8: return launch_bm<8, 1, D>(p, a, grid, block, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

hipError_t launch_prefill(const PrefillLaunch &p, hipStream_t stream)
{
    PrefillArgs a;
    a.M = p.M;
    a.N = p.N;
    a.clean = p.clean;
    a.split = p.split_n;
    a.reverse = p.reverse;
    if (p.ring) {  // shared-K workgroups of num_warps waves x block_m rows
        const int rows = p.block_m * p.num_warps;
        a.nrb = (p.M + rows - 1) / rows;
        const int grid = a.nrb * a.split;
        if (p.head_dim != 128 || p.num_warps != 4)
            return hipErrorInvalidValue;
        if (p.head_tiles == 2 && p.block_m == 2) {  // 64 heads: 2 rows per wave
            switch (p.ring) {
            case 3: return launch_ring<2, 2, 4, 3, 128>(p, a, grid, stream);
            case 4: return launch_ring<2, 2, 4, 4, 128>(p, a, grid, stream);
            default: return hipErrorInvalidValue;
            }
        }
        if (p.head_tiles == 4 && p.block_m == 1) {  // 128 heads: 1 row per wave
            switch (p.ring) {
            case 3: return launch_ring<1, 4, 4, 3, 128>(p, a, grid, stream);
            case 4: return launch_ring<1, 4, 4, 4, 128>(p, a, grid, stream);
            default: return hipErrorInvalidValue;
            }
        }
        if (p.head_tiles != 1 || p.block_m != 4)
            return hipErrorInvalidValue;
        switch (p.ring) {
        case 2: return launch_ring<4, 1, 4, 2, 128>(p, a, grid, stream);
        case 3: return launch_ring<4, 1, 4, 3, 128>(p, a, grid, stream);
        case 4: return launch_ring<4, 1, 4, 4, 128>(p, a, grid, stream);
        case 5: return launch_ring<4, 1, 4, 5, 128>(p, a, grid, stream);
        case 6: return launch_ring<4, 1, 4, 6, 128>(p, a, grid, stream);
        case 7: return launch_ring<4, 1, 4, 7, 128>(p, a, grid, stream);
        default: return hipErrorInvalidValue;
        }
    }
    a.nrb = (p.M + p.block_m - 1) / p.block_m;
    const int grid = a.nrb * a.split;
    const int block = 64 * p.num_warps;
    switch (p.head_dim) {
    case 64: return launch_dim<64>(p, a, grid, block, stream);
    case 128: return launch_dim<128>(p, a, grid, block, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mqa
