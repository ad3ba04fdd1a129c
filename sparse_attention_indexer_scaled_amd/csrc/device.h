// Device building blocks shared by the prefill and decode kernels (gfx950).
//
// One wave (64 lanes) computes the scores of one query row against a 32-token
// K tile with fp8 MFMAs, v_mfma_f32_32x32x64_f8f6f4 (two at head dim 128, one
// at head dim 64): A = the row's Q (32 heads x D dims), B = K^T (D dims x 32
// tokens), D = S[head][token] in fp32.  The contraction is a dense 32-head x
// token matrix product, which is why it runs on the matrix cores (both pages,
// "Technical Details": 32 heads x 32 tokens per fp8 MFMA tile).
//
// Operand placement.  Lane l = 32 g + t (t = l & 31, g = l >> 5) holds, for row
// t of its operand (a head of Q, a token of K), the 16-byte chunks at bytes
// (2j + g) * 16, j = 0..D/32-1.  Chunks j = 0, 1 feed the first MFMA (dims
// 0..63), chunks 2, 3 the second (dims 64..127).  The MFMA pairs A's byte slot
// (lane group, byte) with B's identical slot, so any placement that Q and K
// share computes the full dot product; this one lets lanes t and t + 32 read
// 32 adjacent bytes of the same K row per load instruction.
//
// Result placement (32x32 fp32 accumulator): lane l holds token t = l & 31 and
// the 16 heads 8 (r / 4) + 4 g + (r % 4), r = 0..15.  The ReLU . weight
// epilogue therefore runs in-lane over 16 heads, and the head sum needs only
// one cross-lane step between lane t and lane t + 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mqa {

constexpr int kHeads = 32;
constexpr int kDim = 128;
constexpr int kTile = 32;  // tokens per MFMA column tile
constexpr int kStep = 64;  // tokens per wave step: two tiles
constexpr int kBlock = 64; // cache block size whose blocks are exactly one step

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// D/2 fp8 bytes per lane of one 32-row x D-dim operand (a K tile or a Q row).
template <int D>
struct Operand {
    static_assert(D == 64 || D == 128, "head dim 64 or 128");
    i32x4 c[D / 32];
};
using Frag = Operand<kDim>;

// The 16 head weights matching this lane's accumulator registers.
struct Weights16 {
    f32x4 c[4];
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Row `rowptr` is this lane's own row (head or token) of the operand.
template <int D>
__device__ __forceinline__ void load_frag(Operand<D> &f, const uint8_t *rowptr, int lane)
{
    const uint8_t *p = rowptr + (lane >> 5) * 16;
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
        f.c[j] = *reinterpret_cast<const i32x4 *>(p + 32 * j);
}

// wrow: the 32 fp32 weights of one query row.  Register r of the accumulator
// holds head 8 (r / 4) + 4 g + r % 4, so chunk q covers heads 8 q + 4 g + 0..3.
__device__ __forceinline__ void load_weights(Weights16 &w, const float *wrow, int lane)
{
    const float *p = wrow + (lane >> 5) * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        w.c[q] = *reinterpret_cast<const f32x4 *>(p + 8 * q);
}

__device__ __forceinline__ f32x16 mfma_fp8(i32x4 a0, i32x4 a1, i32x4 b0, i32x4 b1, f32x16 c)
{
    i32x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    i32x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    // format codes 0, 0: both operands fp8 e4m3 (OCP); zero scale operands
    // select the unscaled instruction.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// S[head][token] for one query row and one 32-token tile.
template <int D>
__device__ __forceinline__ f32x16 row_scores(const Operand<D> &q, const Operand<D> &k)
{
    f32x16 acc = {};
#pragma unroll
    for (int j = 0; j < D / 64; ++j)
        acc = mfma_fp8(q.c[2 * j], q.c[2 * j + 1], k.c[2 * j], k.c[2 * j + 1], acc);
    return acc;
}

// sum over this lane's 16 heads of relu(S) * w, in register order: one max
// and one FMA per head (the first a multiply), in a single chain, since the
// items of a step give the scheduler independent chains enough.  Built with
// -fno-honor-nans, so each relu is a single v_max_f32 (no IEEE canonicalize
// first).
__device__ __forceinline__ float relu_weight_sum(const f32x16 &s, const Weights16 &w)
{
    float a = fmaxf(s[0], 0.f) * w.c[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r)
        a = fmaf(fmaxf(s[r], 0.f), w.c[r / 4][r % 4], a);
    return a;
}

// Finish the head sum of two rows at once.  v_permlane32_swap exchanges the
// upper half of `a` with the lower half of `b`, so after one swap and one add
// lanes 0..31 hold row a's 32 token sums and lanes 32..63 row b's (both pages,
// "Technical Details": the paired-row permlane32 swap replaces a ds_bpermute
// round trip through LDS).
__device__ __forceinline__ float pair_head_sum(float a, float b)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One 64-token step of K in the MFMA operand layout: two 32-token tiles and
// the tokens' scales (lane t of tile h holds the scale of token 32 h + t).
template <int D>
struct KStepOf {
    Operand<D> t[2];
    float sc[2];
};
using KStep = KStepOf<kDim>;

// Scores, relu.weight sums and kv-scaled head sums for one 64-token step and
// R query rows of 32 HT heads each (q[r][ht], w[r][ht]: head tile ht of row r).
// tot[h][i] holds row pair i of tile h: lanes 0..31 row 2i, lanes 32..63 row
// 2i + 1.  The (tile, row, head tile) items are software pipelined by one: the
// MFMAs of item i+1 are issued before the relu.weight epilogue of item i, so
// the epilogue never waits on the MFMA it consumes.  A row's head tiles are
// summed in order; with one head tile the sum is the item itself.
template <int R, int HT, int D = kDim>
__device__ __forceinline__ void step_scores(const KStepOf<D> &k, const Operand<D> (&q)[R][HT],
                                            const Weights16 (&w)[R][HT],
                                            float (&tot)[2][(R + 1) / 2])
{
    constexpr int NT = 2 * R * HT;
    float part[2][R];
    f32x16 prev = row_scores(q[0][0], k.t[0]);
#pragma unroll
    for (int it = 1; it <= NT; ++it) {
        f32x16 cur = prev;
        if (it < NT) {
            const int h = it / (R * HT), r = (it / HT) % R, ht = it % HT;
            cur = row_scores(q[r][ht], k.t[h]);
        }
        const int pit = it - 1;
        const int ph = pit / (R * HT), pr = (pit / HT) % R, pht = pit % HT;
        const float v = relu_weight_sum(prev, w[pr][pht]);
        part[ph][pr] = pht == 0 ? v : part[ph][pr] + v;
        prev = cur;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < (R + 1) / 2; ++i) {
            // an odd last row is paired with itself; its upper half is never stored
            const float pb = part[h][(2 * i + 1 < R) ? 2 * i + 1 : 2 * i];
            tot[h][i] = pair_head_sum(part[h][2 * i], pb) * k.sc[h];
        }
    }
}

// Write -inf over row[c0, c1), split into `nparts` contiguous parts of which
// this wave writes part `part`.  16-byte stores where alignment allows.
__device__ __forceinline__ void fill_neg_inf(float *row, int64_t c0, int64_t c1, int part,
                                             int nparts, int lane)
{
    if (c1 <= c0)
        return;
    const int64_t len = c1 - c0;
    const int64_t a = c0 + len * part / nparts;
    const int64_t e = c0 + len * (part + 1) / nparts;
    if (e <= a)
        return;
    const float ninf = -__builtin_inff();
    float *p = row + a;
    int64_t n = e - a;
    int64_t head = (int64_t)(((16u - ((uintptr_t)p & 15u)) & 15u) >> 2);
    if (head > n)
        head = n;
    if (lane < head)
        p[lane] = ninf;
    p += head;
    n -= head;
    const int64_t n4 = n >> 2;
    const f32x4 v = {ninf, ninf, ninf, ninf};
    for (int64_t i = lane; i < n4; i += 64)
        reinterpret_cast<f32x4 *>(p)[i] = v;
    const int64_t tail = n & 3;
    if (lane < tail)
        p[n4 * 4 + lane] = ninf;
}

} // namespace mqa
