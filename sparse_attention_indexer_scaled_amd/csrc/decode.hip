// Paged decode logits kernel (gfx950).
//
// What it computes (aiter PR 5047 page, "Motivation" and "Technical Details"):
// row j of sequence b gets  sum_h relu(<Q[b,j,h,:], K[p,:]>) * w[b,j,h] * scale[p]
// for every cached position p <= ctx_b - next_n + j, K and its per-token scale
// read from a paged cache through the block table; -inf elsewhere (fused fill).
//
// Work decomposition.  A workgroup owns one (sequence b, KV split s) and walks
// the split's 64-token steps (one cache block each) in order.  Its G waves are
// row groups: wave g holds rows [g R, g R + R) of the sequence's next_n rows
// (Q: 16 VGPR per row, head weights: 16 VGPR per row, for the wave's whole
// life).  All rows of the sequence share ONE K stream (both pages, "Technical
// Details": rows share one K stream; the next_n-tiling issue page asks for
// next_n folded into the tile rather than into the program count):
//
//   - K and scales travel HBM -> LDS by direct loads (global_load_lds, no
//     VGPRs) into a ring of D slots, each slot one cache block (8 KiB of K in a
//     bank-conflict-free order + 256 B of scales).  Step k+D-1 is requested
//     while step k computes, so D-1 blocks per workgroup are always in flight
//     and the ring, not the register file, holds the bytes in flight.
//   - The G waves split each block's nine load instructions between them,
//     then every wave reads the whole block from LDS (ds_read_b128) into the
//     MFMA operand layout.  One s_barrier per step publishes the block to all
//     waves and retires the slot the next request overwrites.
//   - Per 32-token tile and row: two fp8 MFMAs, the in-lane relu.weight sum
//     over 16 heads, one permlane32 swap + add per row pair, kv_scale once per
//     column (the hoist: kv_scale >= 0, relu positive-homogeneous).
//   - A step's results are stored one step later, so the stores retire while
//     the next step computes.
// Positions past the sequence's context up to max_model_len are written -inf
// by the same waves.  A position is selected by an integer compare, never by
// arithmetic, so cache slots past the context (which may hold NaN bytes)
// cannot reach an output.
#include "device.h"
#include "launch.h"

namespace mqa {
namespace {

constexpr int kSlotBytes = kBlockBytes;            // one cache block per ring slot
constexpr int kChunks = kDim * kBlock / 1024 + 1;  // 8 x 1 KiB of K + 1 x 256 B of scales

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

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Cache-policy bits of the global->LDS loads: nt (non-temporal).  Every cache
// byte is read once per call, so the loads are marked streaming; measured on
// MI355X this is worth about 10% on the long-context decode.
constexpr int kStreamHint = 2;

// Request one cache block into ring slot `slot`.  Chunk c < 8 moves tokens
// 8c..8c+7 (1 KiB of whole 128-byte rows, so the global read is fully
// coalesced); chunk 8 moves the 64 scales.  A global_load_lds instruction
// writes lane i's 16 bytes at slot + 1024 c + 16 i, so the lane -> granule
// assignment decides the LDS layout: position i of chunk c holds granule
// q = i ^ (8 (c & 1)) of the chunk, where q = 8 u + tau is 16-byte granule u
// of token 8c + tau.  Odd chunks swap the two 128-byte halves of each 256-byte
// row, so that one 16-lane pass of ds_read_b128, which reads two neighbouring
// chunks, covers all 64 LDS banks once.  Wave g of G issues K chunks g, g + G,
// ... and the last wave also the scales, so every wave issues at least
// kChunks / G loads per block.
template <int G>
__device__ __forceinline__ void request_block(lds_u8 *slot, const uint8_t *blk, int g, int lane)
{
    constexpr int KC = kChunks - 1;
    constexpr int J = (KC + G - 1) / G;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int c = g + G * j;
        if (G * J == KC || c < KC) {
            const int q = lane ^ (8 * (c & 1));
            __builtin_amdgcn_global_load_lds(blk + (8 * c + (q & 7)) * kDim + (q >> 3) * 16,
                                             slot + 1024 * c, 16, 0, kStreamHint);
        }
    }
    if (G == 1 || g == G - 1)
        __builtin_amdgcn_global_load_lds(blk + kBlock * kDim + lane * 4, slot + kBlock * kDim, 4, 0,
                                         kStreamHint);
}

// Wait until at most N vector memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One cache block in the MFMA operand layout: two K tiles and the 64 scales.
struct KStep {
    Frag t[2];
    float sc[2];
};

// Read a ring slot into registers.  Lane (t, g') needs token 32 h + t,
// granules u = 2j + g', j = 0..3: chunk c = 4h + t/8 (same parity for both
// tiles), logical granule q = 16 j + 8 g' + t % 8, stored at position
// q ^ 8 (c & 1) = 16 j + 8 (g' ^ (c & 1)) + t % 8, so read j sits 256 bytes
// after read 0.  The reads are inline asm because the compiler would
// otherwise make every LDS read wait for all outstanding global->LDS loads;
// read_wait() completes them.
__device__ __forceinline__ void read_block(KStep &k, uint32_t slot, int lane)
{
    const int t = lane & 31, gq = lane >> 5;
    const int c = t >> 3;  // chunk within the tile; tile 1 adds 4 (same parity)
    const int p0 = 8 * (gq ^ (c & 1)) + (t & 7);
    const uint32_t a0 = slot + (c * 1024 + p0 * 16);
    const uint32_t a1 = a0 + 4096;
    const uint32_t sa = slot + kBlock * kDim + t * 4;
    asm volatile("ds_read_b128 %0, %1 offset:0" : "=v"(k.t[0].c[0]) : "v"(a0));
    asm volatile("ds_read_b128 %0, %1 offset:256" : "=v"(k.t[0].c[1]) : "v"(a0));
    asm volatile("ds_read_b128 %0, %1 offset:512" : "=v"(k.t[0].c[2]) : "v"(a0));
    asm volatile("ds_read_b128 %0, %1 offset:768" : "=v"(k.t[0].c[3]) : "v"(a0));
    asm volatile("ds_read_b128 %0, %1 offset:0" : "=v"(k.t[1].c[0]) : "v"(a1));
    asm volatile("ds_read_b128 %0, %1 offset:256" : "=v"(k.t[1].c[1]) : "v"(a1));
    asm volatile("ds_read_b128 %0, %1 offset:512" : "=v"(k.t[1].c[2]) : "v"(a1));
    asm volatile("ds_read_b128 %0, %1 offset:768" : "=v"(k.t[1].c[3]) : "v"(a1));
    asm volatile("ds_read_b32 %0, %1 offset:0" : "=v"(k.sc[0]) : "v"(sa));
    asm volatile("ds_read_b32 %0, %1 offset:128" : "=v"(k.sc[1]) : "v"(sa));
}

// Wait for read_block's results; the registers pass through the asm, so no
// use of them can be scheduled before the wait.
__device__ __forceinline__ void read_wait(KStep &k)
{
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(k.t[0].c[0]), "+v"(k.t[0].c[1]), "+v"(k.t[0].c[2]), "+v"(k.t[0].c[3]),
                   "+v"(k.t[1].c[0]), "+v"(k.t[1].c[1]), "+v"(k.t[1].c[2]), "+v"(k.t[1].c[3]),
                   "+v"(k.sc[0]), "+v"(k.sc[1])
                 :
                 : "memory");
}

// Scores, relu.weight sums and kv-scaled head sums for one cache block (two
// 32-token tiles) and the wave's R rows.  tot[h][i] holds row pair i of tile
// h: lanes 0..31 row 2i, lanes 32..63 row 2i + 1.  Row-tiles are software
// pipelined by one: the MFMAs of row-tile i+1 are issued before the
// relu.weight epilogue of row-tile i, so the epilogue never waits on the MFMA
// it consumes.
template <int R>
__device__ __forceinline__ void step_scores(const KStep &k, const Frag (&q)[R],
                                            const Weights16 (&w)[R], float (&tot)[2][(R + 1) / 2])
{
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

template <int R, int G, int D>
__global__ __launch_bounds__(64 * G) void decode_kernel(const uint8_t *__restrict__ qbuf,
                                                        const uint8_t *__restrict__ cache,
                                                        const float *__restrict__ wbuf,
                                                        const int32_t *__restrict__ ctx_lens,
                                                        const int32_t *__restrict__ tables,
                                                        float *__restrict__ logits, DecodeArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t ring_mem[];
    constexpr int NP = (R + 1) / 2;
    const int lane = lane_id();
    const int g = G == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); // row group
    const int s = blockIdx.x % a.split;
    const int b = blockIdx.x / a.split;

    const int ctx = ctx_lens[b];
    const int mml = a.mml;
    const int row0 = g * R;
    const int nrows = min(R, a.next_n - row0);
    // Inclusive bound of this wave's first row; row row0 + i covers p <= first_bound + i.
    const int first_bound = ctx - a.next_n + row0;
    // Every wave of the workgroup walks the sequence's whole window (the last
    // row's bound is ctx - 1), so all of them execute the same barriers.
    const int nvalid = max(min(ctx, mml), 0);
    const int nsteps = (nvalid + kStep - 1) / kStep;
    const int st0 = (int)((int64_t)nsteps * s / a.split);
    const int st1 = (int)((int64_t)nsteps * (s + 1) / a.split);
    const int64_t row_base = (int64_t)b * a.next_n + row0;
    float *out = logits + row_base * mml;
    const int t = lane & 31;
    const int half = lane >> 5;
    const float ninf = -__builtin_inff();

    if (st0 < st1) {
        Frag q[R];
        Weights16 w[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            // a short last group computes its missing rows as copies of its
            // last row and never stores them, so the loop body stays branch-free
            const int64_t row = row_base + min(r, nrows - 1);
            load_frag(q[r], qbuf + row * (kHeads * kDim) + t * kDim, lane);
            load_weights(w[r], wbuf + row * kHeads, lane);
        }
        // This lane's output row (and column t) within each pair, its window
        // bound, and whether the row exists.
        float *orow[NP];
        int obound[NP];
        bool ostore[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int rr = 2 * i + half;
            orow[i] = out + (int64_t)min(rr, nrows - 1) * mml + t;
            obound[i] = first_bound + rr;
            ostore[i] = rr < nrows;
        }
        const bool clean = a.clean != 0;
        auto store_step = [&](int step, const float (&tot)[2][NP]) {
            const int p0 = step * kStep;
            if (p0 + kStep - 1 <= first_bound && p0 + kStep <= mml) {
                // every column of the step is inside every row's window
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < NP; ++i)
                        if (ostore[i])
                            orow[i][p0 + h * kTile] = tot[h][i];
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int p = p0 + h * kTile + t;
#pragma unroll
                    for (int i = 0; i < NP; ++i) {
                        const bool valid = p <= obound[i];
                        if (ostore[i] && p < mml && (valid || clean))
                            orow[i][p0 + h * kTile] = valid ? tot[h][i] : ninf;
                    }
                }
            }
        };

        const int32_t *table = tables + (int64_t)b * a.mbps;
        lds_u8 *ring = (lds_u8 *)ring_mem;
        const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
        // Fill D-1 slots (fewer when the split has fewer steps).
#pragma unroll
        for (int i = 0; i < D - 1; ++i)
            if (st0 + i < st1)
                request_block<G>(ring + i * kSlotBytes, cache + (int64_t)table[st0 + i] * kBlockBytes,
                                 g, lane);
        // Between requesting block k and waiting for it a wave requests the
        // D - 2 following blocks, at least kChunks / G loads each, so waiting
        // until at most that many loads are outstanding guarantees block k
        // (loads complete in order; stores counted as well only make the wait
        // stricter).  In the last D - 2 steps fewer blocks follow and the wave
        // waits for everything.
        constexpr int kWait = (D - 2) * (kChunks / G);
        int rd = 0;      // slot of step st
        int wr = D - 1;  // slot of step st + D - 1
        // Block-table entries are read one step ahead: a scalar load is only
        // waited for together with every outstanding LDS read, so its result
        // must not be needed between read_block and read_wait.
        int32_t next_blk = table[min(st0 + D - 1, st1 - 1)];
        float prev_tot[2][NP];
        for (int st = st0; st < st1; ++st) {
            // this wave's part of block st has landed ...
            if (st + D - 2 < st1)
                wait_vm<kWait>();
            else
                wait_vm<0>();
            // ... and every wave's part; nobody reads slot st-1 any more
            __builtin_amdgcn_s_barrier();
            if (st + D - 1 < st1)
                request_block<G>(ring + wr * kSlotBytes, cache + (int64_t)next_blk * kBlockBytes, g,
                                 lane);
            next_blk = table[min(st + D, st1 - 1)];
            KStep kb;
            read_block(kb, ring_addr + rd * kSlotBytes, lane);
            if (st > st0)
                store_step(st - 1, prev_tot);
            rd = (rd + 1 == D) ? 0 : rd + 1;
            wr = (wr + 1 == D) ? 0 : wr + 1;
            read_wait(kb);
            step_scores<R>(kb, q, w, prev_tot);
        }
        store_step(st1 - 1, prev_tot);
        // No global->LDS load may still be in flight once the workgroup ends
        // and its LDS goes to the next workgroup.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if (a.clean) {
        const int64_t f0 = min((int64_t)nsteps * kStep, (int64_t)mml);
        for (int r = 0; r < nrows; ++r)
            fill_neg_inf(out + (int64_t)r * mml, f0, mml, s, a.split, lane);
    }
}

template <int R, int G, int D>
hipError_t launch_rgd(const DecodeLaunch &p, const DecodeArgs &a, int grid, hipStream_t stream)
{
    const size_t lds = (size_t)D * kSlotBytes;
    hipLaunchKernelGGL((decode_kernel<R, G, D>), dim3(grid), dim3(64 * G), lds, stream, p.q,
                       p.cache, p.weights, p.context_lens, p.block_tables, p.logits, a);
    return hipGetLastError();
}

template <int R, int G>
hipError_t launch_rg(const DecodeLaunch &p, const DecodeArgs &a, int grid, hipStream_t stream)
{
    switch (p.depth) {
    case 2: return launch_rgd<R, G, 2>(p, a, grid, stream);
    case 3: return launch_rgd<R, G, 3>(p, a, grid, stream);
    case 4: return launch_rgd<R, G, 4>(p, a, grid, stream);
    case 5: return launch_rgd<R, G, 5>(p, a, grid, stream);
    case 6: return launch_rgd<R, G, 6>(p, a, grid, stream);
    case 7: return launch_rgd<R, G, 7>(p, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

int decode_ring_bytes(int depth) { return depth * kSlotBytes; }

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
    // (rows, row groups) pairs that next_n in 1..8 can produce
    switch (p.rows * 16 + a.groups) {
    case 1 * 16 + 1: return launch_rg<1, 1>(p, a, grid, stream);
    case 1 * 16 + 2: return launch_rg<1, 2>(p, a, grid, stream);
    case 1 * 16 + 3: return launch_rg<1, 3>(p, a, grid, stream);
    case 1 * 16 + 4: return launch_rg<1, 4>(p, a, grid, stream);
    case 1 * 16 + 5: return launch_rg<1, 5>(p, a, grid, stream);
    case 1 * 16 + 6: return launch_rg<1, 6>(p, a, grid, stream);
    case 1 * 16 + 7: return launch_rg<1, 7>(p, a, grid, stream);
    case 1 * 16 + 8: return launch_rg<1, 8>(p, a, grid, stream);
    case 2 * 16 + 1: return launch_rg<2, 1>(p, a, grid, stream);
    case 2 * 16 + 2: return launch_rg<2, 2>(p, a, grid, stream);
    case 2 * 16 + 3: return launch_rg<2, 3>(p, a, grid, stream);
    case 2 * 16 + 4: return launch_rg<2, 4>(p, a, grid, stream);
    case 3 * 16 + 1: return launch_rg<3, 1>(p, a, grid, stream);
    case 3 * 16 + 2: return launch_rg<3, 2>(p, a, grid, stream);
    case 3 * 16 + 3: return launch_rg<3, 3>(p, a, grid, stream);
    case 4 * 16 + 1: return launch_rg<4, 1>(p, a, grid, stream);
    case 4 * 16 + 2: return launch_rg<4, 2>(p, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mqa
