// Paged decode kernel template (gfx950), shared by the logits call (decode.hip,
// decode_heads.hip, decode_d64.hip) and the fused top-k's sample and filter
// modes (decode_fused.hip, decode_fused_d64.hip).
//
// What it computes (aiter PR 5047 page, "Motivation" and "Technical Details"):
// row j of sequence b gets  sum_h relu(<Q[b,j,h,:], K[p,:]>) * w[b,j,h] * scale[p]
// for every cached position p <= ctx_b - next_n + j, K and its per-token scale
// read from a paged cache through the block table; -inf elsewhere (fused fill).
//
// Work decomposition.  A workgroup owns one (sequence b, KV split s) and walks
// the split's 64-token steps (one cache block each) in order.  Its G waves are
// row groups: wave g holds rows [g R, g R + R) of the sequence's next_n rows
// (Q: DIM / 8 VGPR per row and head tile, head weights: 16 VGPR per row and
// head tile, for the wave's whole life).  All rows of the sequence share ONE
// K stream (both pages, "Technical Details": rows share one K stream; the
// next_n-tiling issue page asks for next_n folded into the tile rather than
// into the program count):
//
//   - K and scales travel HBM -> LDS by direct loads (global_load_lds, no
//     VGPRs) into a ring of D slots, each slot one 64-token step (64 DIM bytes
//     of K in a bank-conflict-free order + 256 B of scales).  Step k+D-1 is
//     requested while step k computes, so D-1 steps per workgroup are always
//     in flight and the ring, not the register file, holds the bytes in
//     flight.
//   - The G waves split each step's loads (DIM / 16 chunks of 1 KiB and the
//     scales) between them, then every wave reads the whole step from LDS
//     (ds_read_b128) into the MFMA operand layout.  One s_barrier per step
//     publishes the step to all waves and retires the slot the next request
//     overwrites.
//   - Per 32-token tile, row and 32-head tile: DIM / 64 fp8 MFMAs and the
//     in-lane relu.weight sum over 16 heads; per row pair one permlane32 swap
//     + add, then kv_scale once per column (the hoist: kv_scale >= 0, relu
//     positive-homogeneous).
//   - A step's results are stored one step later, after that step's request
//     and LDS reads, so the stores retire while the next step computes.
//     (Stored before the request, they lead the compiler to wait for every
//     outstanding load before each global->LDS load in some instantiations:
//     128 heads ran at half speed.)
// Positions past the sequence's context up to max_model_len are written -inf
// by the same waves.  A position is selected by an integer compare, never by
// arithmetic, so cache slots past the context (which may hold NaN bytes)
// cannot reach an output.
//
// The same kernel serves the fused decode top-k in two more modes (see
// DecodeMode): a sample of each sequence's steps, and a filter that keeps
// only the entries at or above each row's threshold instead of storing logits.
#pragma once

#include "device.h"
#include "launch.h"
#include "order_key.h"
#include "ring.h"

namespace mqa {
namespace {

constexpr int kSampleChunks = kFusedSampleChunks;
constexpr int kSampleSteps = kFusedSampleSteps;
constexpr int kSampleCols = kFusedSampleCols;

// LDS bytes of a workgroup's ring (and, for per-token blocks, its table
// ring).
template <int D, int BS, int DIM>
constexpr int ring_lds_bytes()
{
    return D * slot_bytes<DIM>() + (BS == 1 ? (2 * D - 2) * kStep * 4 : 0);
}

// Sizes and launch shape; the pointers are separate __restrict__ kernel
// arguments so the compiler may read the block table with scalar loads.
struct DecodeArgs {
    int mml;
    int next_n;
    int mbps;
    int clean;
    int groups;
    int split;
    int tiled;  // K rows of a block in the preshuffled (16,16) order
    // Fused top-k (see the kernel's modes; unused by the plain logits call):
    float *sample;                // sample mode: [rows][kSampleCols]
    const uint32_t *threshold;    // filter mode: [rows] order-key thresholds
    uint64_t *entries;            // filter mode: [rows][ent_stride]
    int *counts;                  // filter mode: [rows][split]
    int64_t ent_stride;
};

// Kernel modes.  kLogits: the op's output.  The fused top-k adds two:
// kSample computes kSampleChunks evenly spaced runs of kSampleSteps steps of
// each sequence (the sample its thresholds are drawn from) into a small
// buffer, -inf outside the windows; kFilter computes every step like kLogits
// but, instead of storing the logits, appends the (key, column) entries of
// each row at or above the row's threshold to the workgroup's own segment of
// the row (it starts at the workgroup's first column, so it can never
// overflow), and stores their count.
enum DecodeMode { kLogits = 0, kSample = 1, kFilter = 2 };

// Cache-policy bits of the global->LDS loads: nt (non-temporal).  Every cache
// byte is read once per call, so the loads are marked streaming; measured on
// MI355X this is worth about 10% on the long-context decode.
constexpr int kStreamHint = 2;

// Where the 64 tokens of one step come from in a cache of BS-token blocks,
// and how they are requested into a ring slot.  The slot layout is the same
// for every block size of 16 or more tokens (see read_block): 8 x 1 KiB
// chunks of K rows, then the 64 scales (per-token blocks fill their slots in
// row order instead: see request_tokens).  A global_load_lds instruction writes lane i's 16 bytes at
// slot + 1024 c + 16 i, so the lane -> granule assignment decides the LDS
// layout: position i of chunk c holds granule q = i ^ (8 (c & 1)) of the
// chunk, where q = 8 u + tau is 16-byte granule u of token 8c + tau.  Odd
// chunks swap the two 128-byte halves of each 256-byte row, so that one
// 16-lane pass of ds_read_b128, which reads two neighbouring chunks, covers
// all 64 LDS banks once.  Wave g of G issues K chunks g, g + G, ... and the
// last wave also the scales, so every wave issues at least kChunks / G loads
// per step.
//
// Blocks of 16 or more tokens hold whole 8-token chunks, so each chunk is one
// coalesced 1 KiB read; the step's table entries (64 / BS of them, or one
// entry covering several steps) are read with scalar loads.
//
// Such blocks may also hold their K rows in the preshuffled (16,16) order
// (the 64-token pairing on the aiter PR 5047 page, "Technical Details"): the
// slots in groups of 16, each group storing 16-byte granule u of its 16 rows
// (row by row) before granule u + 1, so granule u of block row r sits at
// (r / 16) 2048 + 256 u + 16 (r % 16).  Only the source addresses change: a
// chunk's 64 granules are then eight 128-byte runs, and the two chunks of a
// 16-row group read one contiguous 2 KiB; the ring slot is filled exactly as
// from a slot-major block.
// The block pointers of one step (one per table entry the step touches).
template <int N>
struct StepBlocks {
    const uint8_t *p[N];
};

constexpr int entries_per_step(int bs) { return bs >= kStep ? 1 : kStep / bs; }

template <int BS, int DIM = kDim>
struct Gather {
    static_assert(BS == 16 || BS == 64 || BS == 128, "block sizes with whole chunks");
    static constexpr int kEntries = entries_per_step(BS);       // table entries per step
    static constexpr int64_t kBytes = (int64_t)BS * (DIM + 4);  // bytes per block

    struct Src {
        StepBlocks<kEntries> blk;
        int off;  // first token of the step within its block (BS > 64)
    };

    // last: index of the sequence's last table entry that holds a token of
    // the window.  Entries past it are never read (they may be padding): a
    // step that ends beyond the context reuses the last entry, whose data
    // never reaches an output.
    __device__ static __forceinline__ Src fetch(const uint8_t *cache, const int32_t *table, int st,
                                                int last)
    {
        Src src;
        if (BS >= kStep) {
            const int tok = st * kStep;
            src.blk.p[0] = cache + (int64_t)table[tok / BS] * kBytes;
            src.off = tok % BS;
        } else {
#pragma unroll
            for (int e = 0; e < kEntries; ++e)
                src.blk.p[e] = cache + (int64_t)table[min(st * kEntries + e, last)] * kBytes;
            src.off = 0;
        }
        return src;
    }

};

// Request a step into ring slot `slot` (wave g of G; see Gather): blk_of and
// off are the fields of the step's Gather<BS>::Src (passed by value, so the
// pointers stay in registers).
template <int G, int BS, int DIM = kDim>
__device__ __forceinline__ void request_step(lds_u8 *slot, StepBlocks<entries_per_step(BS)> blk_of,
                                             int off, bool tiled, int g, int lane)
{
    constexpr int kEntries = entries_per_step(BS);
    constexpr int KC = k_chunks<DIM>();
    constexpr int TPC = rows_per_chunk<DIM>();
    constexpr int J = (KC + G - 1) / G;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int c = g + G * j;
        if (G * J == KC || c < KC) {
            // granule q = TPC u + tau: 16-byte granule u of chunk row tau
            const int q = DIM == 128 ? lane ^ (8 * (c & 1)) : lane;
            const int e = BS >= kStep ? 0 : (TPC * c) / BS;  // wave-uniform
            const uint8_t *blk = blk_of.p[0];
#pragma unroll
            for (int i = 1; i < kEntries; ++i)  // selects, not a dynamic index
                if (e == i)
                    blk = blk_of.p[i];
            const int row = (BS >= kStep ? off + TPC * c : (TPC * c) % BS) + q % TPC;
            const int u = q / TPC;
            const int src = tiled ? (row >> 4) * (16 * DIM) + u * 256 + (row & 15) * 16
                                  : row * DIM + u * 16;
            __builtin_amdgcn_global_load_lds(blk + src, slot + 1024 * c, 16, 0, kStreamHint);
        }
    }
    if (G == 1 || g == G - 1) {
        const uint8_t *blk = blk_of.p[0];
        int row = off + lane;
        if (BS < kStep) {
#pragma unroll
            for (int e = 1; e < kEntries; ++e)
                if (lane >= e * BS)
                    blk = blk_of.p[e];
            row = lane % BS;
        }
        __builtin_amdgcn_global_load_lds(blk + BS * DIM + row * 4, slot + kStep * DIM, 4, 0,
                                         kStreamHint);
    }
}

// Per-token blocks (BS = 1, the plain co-packed layout): token p's DIM K
// bytes and 4 scale bytes sit at (DIM + 4) * table[p], so records are only
// 4-byte aligned and every token has its own table entry.  A step's 64 entries
// are staged in LDS (one global->LDS dword load, by wave 0, well ahead: see the
// kernel), each wave reads the entries its loads need, and K moves with 4-byte
// global->LDS loads.  Their slot holds the step's K rows in row order (row r at
// DIM r), each row's 16-byte granules swizzled: granule u of row r sits at
// position u ^ f(r), f(r) = (r / 2) % 8 at head dim 128 and (r / 4) % 4 at 64,
// so that a 16-lane pass of ds_read_b128 over 16 rows touches each group of 4
// banks once (read_block_rows).  A dword load writes 256 contiguous LDS bytes,
// i.e. 2 whole rows (4 at head dim 64): lane i of load jj of chunk c fills byte
// 4 (i % 4) of position (i % L) / 4 of chunk row R jj + i / L (R = 2, L = 32;
// R = 4, L = 16 at head dim 64), so each load reads 2 (4) whole records where a
// granule-ordered slot would need 32-byte pieces of 8 (16), and four loads
// move a chunk.
constexpr int kTokLoadsPerChunk = 4;

template <int DIM>
__device__ __forceinline__ int row_swizzle(int row)
{
    return DIM == 128 ? (row >> 1) & 7 : (row >> 2) & 3;
}

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

// The table entries a wave's per-token loads need: entries R rows apart
// (R = rows per load) at each of J chunk addresses, two ds_read2_b32 per chunk,
// and the step's scale entry at sa.  The entries become global addresses, so
// the reads and their wait are one asm block: no register is read, reused or
// copied before its value has landed.  (Plain LDS reads would wait for every
// outstanding global->LDS load.)
#define MQA_RD2(j)                                                                   \
    "ds_read2_b32 %[a" #j "], %[c" #j "] offset0:0 offset1:%[r1]\n\t"               \
    "ds_read2_b32 %[b" #j "], %[c" #j "] offset0:%[r2] offset1:%[r3]\n\t"
#define MQA_OUT2(j) [a##j] "=&v"(e[j][0]), [b##j] "=&v"(e[j][1])
#define MQA_IN1(j) [c##j] "v"(ca[j])
#define MQA_TAIL "ds_read_b32 %[s], %[sa]\n\ts_waitcnt lgkmcnt(0)"
#define MQA_CONST [s] "=&v"(es) : [sa] "v"(sa), [r1] "n"(R), [r2] "n"(2 * R), [r3] "n"(3 * R)
template <int J, int R>
__device__ __forceinline__ void read_entries(const uint32_t (&ca)[J], uint32_t sa,
                                             i32x2 (&e)[J][2], int32_t &es)
{
    static_assert(J == 1 || J == 2 || J == 3 || J == 4 || J == 8, "chunks per wave");
    if constexpr (J == 1)
        asm volatile(MQA_RD2(0) MQA_TAIL : MQA_OUT2(0), MQA_CONST, MQA_IN1(0) : "memory");
    else if constexpr (J == 2)
        asm volatile(MQA_RD2(0) MQA_RD2(1) MQA_TAIL
                     : MQA_OUT2(0), MQA_OUT2(1), MQA_CONST, MQA_IN1(0), MQA_IN1(1)
                     : "memory");
    else if constexpr (J == 3)
        asm volatile(MQA_RD2(0) MQA_RD2(1) MQA_RD2(2) MQA_TAIL
                     : MQA_OUT2(0), MQA_OUT2(1), MQA_OUT2(2), MQA_CONST, MQA_IN1(0), MQA_IN1(1),
                       MQA_IN1(2)
                     : "memory");
    else if constexpr (J == 4)
        asm volatile(MQA_RD2(0) MQA_RD2(1) MQA_RD2(2) MQA_RD2(3) MQA_TAIL
                     : MQA_OUT2(0), MQA_OUT2(1), MQA_OUT2(2), MQA_OUT2(3), MQA_CONST, MQA_IN1(0),
                       MQA_IN1(1), MQA_IN1(2), MQA_IN1(3)
                     : "memory");
    else
        asm volatile(MQA_RD2(0) MQA_RD2(1) MQA_RD2(2) MQA_RD2(3) MQA_RD2(4) MQA_RD2(5)
                         MQA_RD2(6) MQA_RD2(7) MQA_TAIL
                     : MQA_OUT2(0), MQA_OUT2(1), MQA_OUT2(2), MQA_OUT2(3), MQA_OUT2(4),
                       MQA_OUT2(5), MQA_OUT2(6), MQA_OUT2(7), MQA_CONST, MQA_IN1(0), MQA_IN1(1),
                       MQA_IN1(2), MQA_IN1(3), MQA_IN1(4), MQA_IN1(5), MQA_IN1(6), MQA_IN1(7)
                     : "memory");
}
#undef MQA_RD2
#undef MQA_OUT2
#undef MQA_IN1
#undef MQA_TAIL
#undef MQA_CONST

template <int G, int DIM = kDim>
__device__ __forceinline__ void request_tokens(lds_u8 *slot, uint32_t entries, const uint8_t *cache,
                                               int g, int lane)
{
    constexpr int KC = k_chunks<DIM>();
    constexpr int J = (KC + G - 1) / G;
    constexpr int R = 1024 / DIM / kTokLoadsPerChunk;  // rows per load
    constexpr int L = 64 / R;  // lanes per row
    static_assert(R * kTokLoadsPerChunk * DIM == 1024, "four loads move a 1 KiB chunk");
    // The lane's offsets are the same every step; formed here each time (an
    // opaque copy of the lane id), they are not hoisted out of the kernel's
    // loop into registers the waves need.
    asm volatile("" : "+v"(lane));
    // chunk c's entries for load jj: rows TPC c + R jj + lane / L (a chunk
    // index past the step, when G does not divide KC, rereads the last chunk's
    // entries and issues no load)
    uint32_t ca[J];
#pragma unroll
    for (int j = 0; j < J; ++j)
        ca[j] = entries + 4 * (rows_per_chunk<DIM>() * min(g + G * j, KC - 1) + lane / L);
    i32x2 ent[J][2];
    int32_t ent_s;
    read_entries<J, R>(ca, entries + 4 * lane, ent, ent_s);
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int c = g + G * j;
        if (G * J == KC || c < KC) {
#pragma unroll
            for (int jj = 0; jj < kTokLoadsPerChunk; ++jj) {
                const int row = rows_per_chunk<DIM>() * c + R * jj + lane / L;
                const int u = ((lane % L) >> 2) ^ row_swizzle<DIM>(row);
                const uint8_t *src = cache + (int64_t)ent[j][jj >> 1][jj & 1] * (DIM + 4) +
                                     16 * u + 4 * (lane & 3);
                __builtin_amdgcn_global_load_lds(src, slot + 1024 * c + 256 * jj, 4, 0, kStreamHint);
            }
        }
    }
    if (G == 1 || g == G - 1)
        __builtin_amdgcn_global_load_lds(cache + (int64_t)ent_s * (DIM + 4) + DIM,
                                         slot + kStep * DIM, 4, 0, kStreamHint);
}

// Read a per-token slot (rows in row order, granules swizzled: see
// request_tokens) into the MFMA operand layout: lane (t, g') takes granules
// u = 2j + g' of token 32 h + t, as read_block does from the other slots.
// Completed by read_wait.
template <int DIM>
__device__ __forceinline__ void read_block_rows(KStepOf<DIM> &k, uint32_t slot, int lane)
{
    asm volatile("" : "+v"(lane));  // see request_tokens
    const int t = lane & 31, gq = lane >> 5;
    const uint32_t sa = slot + kStep * DIM + t * 4;
    const int f = row_swizzle<DIM>(t);  // the same for row t and row 32 + t
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t rb = slot + (32 * h + t) * DIM;
#pragma unroll
        for (int j = 0; j < DIM / 32; ++j) {
            const uint32_t a = rb + 16 * ((2 * j + gq) ^ f);
            asm volatile("ds_read_b128 %0, %1" : "=v"(k.t[h].c[j]) : "v"(a));
        }
    }
    asm volatile("ds_read_b32 %0, %1 offset:0" : "=v"(k.sc[0]) : "v"(sa));
    asm volatile("ds_read_b32 %0, %1 offset:128" : "=v"(k.sc[1]) : "v"(sa));
}

template <int R, int G, int D, int BS, int HT, int MODE = kLogits, int DIM = kDim>
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
    int st0, st1;
    if constexpr (MODE == kSample) {
        // chunk s of kSampleChunks (a.split): kSampleSteps steps, evenly spaced
        const int span = max(nsteps - kSampleSteps, 0);
        st0 = (int)((int64_t)span * s / (kSampleChunks - 1));
        st1 = min(st0 + kSampleSteps, nsteps);
    } else {
        st0 = (int)((int64_t)nsteps * s / a.split);
        st1 = (int)((int64_t)nsteps * (s + 1) / a.split);
    }
    const int64_t row_base = (int64_t)b * a.next_n + row0;
    float *out = logits + row_base * mml;
    const int t = lane & 31;
    const int half = lane >> 5;
    const float ninf = -__builtin_inff();

    if (st0 < st1) {
        constexpr int H = kHeads * HT;
        Operand<DIM> q[R][HT];
        Weights16 w[R][HT];
        // kFilter: this lane's row threshold (as a float: key >= t <=> value >= f),
        // where its row's entries go, and how many each row of the pair has kept
        // so far (each row belongs to one wave, and within it to one half of the
        // lanes, so the counts are wave-uniform and need no atomics)
        float fthr[NP];
        uint64_t *ebase[NP];
        int kept_lo[NP], kept_hi[NP];
        // all ones in the upper half of the lanes (hmask) or the lower (lmask),
        // opaque so that the compiler keeps the masking below as two ANDs
        // instead of turning it into selects
        uint32_t hmask = half ? ~0u : 0u, lmask = ~hmask;
        asm volatile("" : "+v"(hmask), "+v"(lmask));
        if constexpr (MODE == kFilter) {
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const int rr = min(2 * i + half, nrows - 1);
                const uint32_t tk = a.threshold[row_base + rr];
                fthr[i] = tk == 0u ? __builtin_inff() : key_float(tk);
                ebase[i] = a.entries + (row_base + rr) * a.ent_stride + st0 * kStep;
                kept_lo[i] = 0;
                kept_hi[i] = 0;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            // a short last group computes its missing rows as copies of its
            // last row and never stores them, so the loop body stays branch-free
            const int64_t row = row_base + min(r, nrows - 1);
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                load_frag(q[r][ht], qbuf + row * (H * DIM) + (ht * kHeads + t) * DIM, lane);
                load_weights(w[r][ht], wbuf + row * H + ht * kHeads, lane);
            }
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
        // kFilter: the last column a lane's row may keep
        int olast[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i)
            olast[i] = min(obound[i], mml - 1);
        auto store_step = [&](int step, const float (&tot)[2][NP]) {
            const int p0 = step * kStep;
            if constexpr (MODE == kSample) {
                // columns of chunk s: [s kSampleSteps 64, (s + 1) kSampleSteps 64)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int p = p0 + h * kTile + t;
                    const int c = s * kSampleSteps * kStep + (p - st0 * kStep);
#pragma unroll
                    for (int i = 0; i < NP; ++i) {
                        const bool valid = p <= obound[i] && p < mml;
                        if (ostore[i])
                            a.sample[(row_base + 2 * i + half) * kSampleCols + c] =
                                valid ? tot[h][i] : ninf;
                    }
                }
                return;
            }
            if constexpr (MODE == kFilter) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int p = p0 + h * kTile + t;
#pragma unroll
                    for (int i = 0; i < NP; ++i) {
                        const float v = tot[h][i];
                        // (bitwise: lane masks combined without branches)
                        const bool keep = ostore[i] & (p <= olast[i]) & (v >= fthr[i]);
                        // lanes 0..31 hold row 2i, lanes 32..63 row 2i + 1
                        const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
                        const uint32_t lo = (uint32_t)bal, hi = (uint32_t)(bal >> 32);
                        if (keep) {
                            // this half's count so far plus its kept lanes below
                            // this one (mbcnt_hi counts nothing in the lower half;
                            // the mask keeps the lower half's bits from the upper)
                            const uint32_t base =
                                (uint32_t)kept_lo[i] + ((uint32_t)(kept_hi[i] - kept_lo[i]) & hmask);
                            const uint32_t slot = __builtin_amdgcn_mbcnt_hi(
                                hi, __builtin_amdgcn_mbcnt_lo(lo & lmask, base));
                            // a kept value is finite (v >= fthr >= -FLT_MAX): its
                            // order key, with -0 made +0 by the addition
                            const uint32_t u = __float_as_uint(v + 0.0f);
                            const uint32_t key = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
                            ebase[i][slot] = entry(key, p);
                        }
                        kept_lo[i] += __builtin_popcount(lo);
                        kept_hi[i] += __builtin_popcount(hi);
                    }
                }
                return;
            }
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
        const bool tiled = a.tiled != 0;
        lds_u8 *ring = (lds_u8 *)ring_mem;
        const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
        using Gth = Gather<(BS == 1 ? kBlock : BS), DIM>;  // unused for BS = 1
        constexpr int SB = slot_bytes<DIM>();
        const int last_entry = (nvalid - 1) / BS;
        // BS = 1: table ring of 2D - 2 steps of 64 entries after the K ring.
        // Entries for step y are loaded (by wave 0) in the iteration that
        // requests K for step y - D + 1, before that request, and read in the
        // iteration that requests step y: by then the wait for step
        // y - D + 1 has covered them, and the barrier published them.
        constexpr int kTabSlots = 2 * D - 2;
        lds_u8 *tring = ring + D * SB;
        const uint32_t tring_addr = ring_addr + D * SB;
        auto request_table = [&](int y) {  // wave 0 only
            const int tok = min(y * kStep + lane, last_entry);
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t *>(table + tok),
                                             tring + ((y - st0) % kTabSlots) * (kStep * 4), 4, 0, 0);
        };
        // Fill D-1 slots (fewer when the split has fewer steps).
        if constexpr (BS == 1) {
            if (g == 0) {
#pragma unroll
                for (int i = 0; i < kTabSlots; ++i)
                    if (st0 + i < st1)
                        request_table(st0 + i);
            }
            wait_vm<0>();
            __builtin_amdgcn_s_barrier();
#pragma unroll
            for (int i = 0; i < D - 1; ++i)
                if (st0 + i < st1)
                    request_tokens<G, DIM>(ring + i * SB, tring_addr + i * (kStep * 4), cache, g,
                                      lane);
        } else {
#pragma unroll
            for (int i = 0; i < D - 1; ++i)
                if (st0 + i < st1) {
                    const typename Gth::Src src = Gth::fetch(cache, table, st0 + i, last_entry);
                    request_step<G, BS, DIM>(ring + i * SB, src.blk, src.off, tiled, g, lane);
                }
        }
        // Between requesting block k and waiting for it a wave requests the
        // D - 2 following blocks, at least min_loads_per_step loads each, so
        // waiting until at most that many loads are outstanding guarantees
        // block k (loads complete in order; stores and table loads counted as
        // well only make the wait stricter).  In the last D - 2 steps fewer
        // blocks follow and the wave waits for everything.
        // (vmcnt holds at most 63; a smaller count is a stricter wait)
        constexpr int kWaitRaw =
            (D - 2) * min_loads_per_step(G, BS == 1 ? kTokLoadsPerChunk : 1, k_chunks<DIM>());
        constexpr int kWait = kWaitRaw < 63 ? kWaitRaw : 63;
        int rd = 0;      // slot of step st
        int wr = D - 1;  // slot of step st + D - 1
        // Block-table entries are read one step ahead: a scalar load is only
        // waited for together with every outstanding LDS read, so its result
        // must not be needed between read_block and read_wait.
        typename Gth::Src next{};
        if constexpr (BS != 1)
            next = Gth::fetch(cache, table, min(st0 + D - 1, st1 - 1), last_entry);
        float prev_tot[2][NP];
        for (int st = st0; st < st1; ++st) {
            // this wave's part of block st has landed ...
            if (st + D - 2 < st1)
                wait_vm<kWait>();
            else
                wait_vm<0>();
            // ... and every wave's part; nobody reads slot st-1 any more
            __builtin_amdgcn_s_barrier();
            if constexpr (BS == 1) {
                if (g == 0 && st + kTabSlots < st1)
                    request_table(st + kTabSlots);
                if (st + D - 1 < st1)
                    request_tokens<G, DIM>(ring + wr * SB,
                                      tring_addr + ((st + D - 1 - st0) % kTabSlots) * (kStep * 4),
                                      cache, g, lane);
            } else {
                if (st + D - 1 < st1)
                    request_step<G, BS, DIM>(ring + wr * SB, next.blk, next.off, tiled, g,
                                        lane);
                next = Gth::fetch(cache, table, min(st + D, st1 - 1), last_entry);
            }
            KStepOf<DIM> kb;
            if constexpr (BS == 1)
                read_block_rows<DIM>(kb, ring_addr + rd * SB, lane);
            else
                read_block<DIM>(kb, ring_addr + rd * SB, lane);
            if (st > st0)
                store_step(st - 1, prev_tot);
            rd = (rd + 1 == D) ? 0 : rd + 1;
            wr = (wr + 1 == D) ? 0 : wr + 1;
            read_wait<DIM>(kb);
            step_scores<R, HT, DIM>(kb, q, w, prev_tot);
        }
        store_step(st1 - 1, prev_tot);
        if constexpr (MODE == kFilter) {
#pragma unroll
            for (int i = 0; i < NP; ++i)
                if (ostore[i] && t == 0)
                    a.counts[(row_base + 2 * i + half) * a.split + s] = half ? kept_hi[i] : kept_lo[i];
        }
        // No global->LDS load may still be in flight once the workgroup ends
        // and its LDS goes to the next workgroup.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if constexpr (MODE == kSample) {
        // the chunk's columns past its last step (short sequences) are -inf
        const int done = max(st1 - st0, 0) * kStep;
        for (int r = 0; r < nrows; ++r)
            for (int c = done + lane; c < kSampleSteps * kStep; c += 64)
                a.sample[(row_base + r) * kSampleCols + s * kSampleSteps * kStep + c] = ninf;
        return;
    }
    if constexpr (MODE == kFilter) {
        // a workgroup with no step (empty sequence) keeps nothing
        if (st0 >= st1 && lane == 0)
            for (int r = 0; r < nrows; ++r)
                a.counts[(row_base + r) * a.split + s] = 0;
        return;
    }
    if (a.clean) {
        const int64_t f0 = min((int64_t)nsteps * kStep, (int64_t)mml);
        for (int r = 0; r < nrows; ++r)
            fill_neg_inf(out + (int64_t)r * mml, f0, mml, s, a.split, lane);
    }
}

template <int R, int G, int D, int BS, int HT = 1, int MODE = kLogits, int DIM = kDim>
hipError_t launch_rgdb(const DecodeLaunch &p, const DecodeArgs &a, int grid, hipStream_t stream)
{
    const size_t lds = (size_t)ring_lds_bytes<D, BS, DIM>();
    hipLaunchKernelGGL((decode_kernel<R, G, D, BS, HT, MODE, DIM>), dim3(grid), dim3(64 * G), lds,
                       stream, p.q, p.cache, p.weights, p.context_lens, p.block_tables, p.logits,
                       a);
    return hipGetLastError();
}

// The kernels a (rows per wave R, waves G, head tiles HT, mode, head dim)
// launch can take, by block size and ring depth: 64-token blocks at 32 heads
// and head dim 128 take ring depths 2..7 for the logits call and 3 for the
// fused top-k's modes; per-token blocks take depth 4 and every other layout
// depth 3.  (Q and weights of a wave's rows stay in VGPRs, so R HT <= 4.)
template <int R, int G, int HT, int MODE, int DIM = kDim>
hipError_t launch_rg(const DecodeLaunch &p, const DecodeArgs &a, int grid, hipStream_t stream)
{
    if constexpr (R * HT > 4) {
        return hipErrorInvalidValue;
    } else {
        if constexpr (HT == 1 && DIM == kDim) {
            if (p.block_size == 64) {
                if constexpr (MODE == kLogits) {
                    switch (p.depth) {
                    case 2: return launch_rgdb<R, G, 2, 64, 1, MODE>(p, a, grid, stream);
                    case 3: return launch_rgdb<R, G, 3, 64, 1, MODE>(p, a, grid, stream);
                    case 4: return launch_rgdb<R, G, 4, 64, 1, MODE>(p, a, grid, stream);
                    case 5: return launch_rgdb<R, G, 5, 64, 1, MODE>(p, a, grid, stream);
                    case 6: return launch_rgdb<R, G, 6, 64, 1, MODE>(p, a, grid, stream);
                    case 7: return launch_rgdb<R, G, 7, 64, 1, MODE>(p, a, grid, stream);
                    default: return hipErrorInvalidValue;
                    }
                } else {
                    return p.depth == 3 ? launch_rgdb<R, G, 3, 64, 1, MODE>(p, a, grid, stream)
                                        : hipErrorInvalidValue;
                }
            }
        }
        if (p.depth != (p.block_size == 1 ? 4 : 3))
            return hipErrorInvalidValue;
        switch (p.block_size) {
        case 1: return launch_rgdb<R, G, 4, 1, HT, MODE, DIM>(p, a, grid, stream);
        case 16: return launch_rgdb<R, G, 3, 16, HT, MODE, DIM>(p, a, grid, stream);
        case 64:
            if constexpr (HT > 1 || DIM != kDim)
                return launch_rgdb<R, G, 3, 64, HT, MODE, DIM>(p, a, grid, stream);
            else
                return hipErrorInvalidValue;  // handled above
        case 128: return launch_rgdb<R, G, 3, 128, HT, MODE, DIM>(p, a, grid, stream);
        default: return hipErrorInvalidValue;
        }
    }
}

// (rows, row groups) pairs that next_n in 1..8 can produce
template <int HT, int MODE, int DIM = kDim>
hipError_t launch_ht(const DecodeLaunch &p, const DecodeArgs &a, int grid, hipStream_t stream)
{
    switch (p.rows * 16 + a.groups) {
    case 1 * 16 + 1: return launch_rg<1, 1, HT, MODE, DIM>(p, a, grid, stream);
    case 1 * 16 + 2: return launch_rg<1, 2, HT, MODE, DIM>(p, a, grid, stream);
    case 1 * 16 + 3: return launch_rg<1, 3, HT, MODE, DIM>(p, a, grid, stream);
    case 1 * 16 + 4: return launch_rg<1, 4, HT, MODE, DIM>(p, a, grid, stream);
    case 1 * 16 + 5: return launch_rg<1, 5, HT, MODE, DIM>(p, a, grid, stream);
    case 1 * 16 + 6: return launch_rg<1, 6, HT, MODE, DIM>(p, a, grid, stream);
    case 1 * 16 + 7: return launch_rg<1, 7, HT, MODE, DIM>(p, a, grid, stream);
    case 1 * 16 + 8: return launch_rg<1, 8, HT, MODE, DIM>(p, a, grid, stream);
    case 2 * 16 + 1: return launch_rg<2, 1, HT, MODE, DIM>(p, a, grid, stream);
    case 2 * 16 + 2: return launch_rg<2, 2, HT, MODE, DIM>(p, a, grid, stream);
    case 2 * 16 + 3: return launch_rg<2, 3, HT, MODE, DIM>(p, a, grid, stream);
    case 2 * 16 + 4: return launch_rg<2, 4, HT, MODE, DIM>(p, a, grid, stream);
    case 3 * 16 + 1: return launch_rg<3, 1, HT, MODE, DIM>(p, a, grid, stream);
    case 3 * 16 + 2: return launch_rg<3, 2, HT, MODE, DIM>(p, a, grid, stream);
    case 3 * 16 + 3: return launch_rg<3, 3, HT, MODE, DIM>(p, a, grid, stream);
    case 4 * 16 + 1: return launch_rg<4, 1, HT, MODE, DIM>(p, a, grid, stream);
    case 4 * 16 + 2: return launch_rg<4, 2, HT, MODE, DIM>(p, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

// Kernel arguments of a validated launch.
inline DecodeArgs decode_args(const DecodeLaunch &p)
{
    DecodeArgs a;
    a.mml = (int)p.max_model_len;
    a.next_n = p.next_n;
    a.mbps = p.max_blocks_per_seq;
    a.clean = p.clean;
    a.groups = (p.next_n + p.rows - 1) / p.rows;
    a.split = p.split_kv;
    a.tiled = p.tiled;
    a.sample = p.sample;
    a.threshold = p.threshold;
    a.entries = p.entries;
    a.counts = p.counts;
    a.ent_stride = p.ent_stride;
    return a;
}

} // namespace
} // namespace mqa
