// K-cache quantise-and-insert (gfx950): the step before decode that stores
// new K rows as fp8 e4m3fn beside a per-token fp32 dequant scale in the paged
// cache (aiter PR 5047 page, "Motivation"; the scale is the row's absolute
// maximum over 448, the largest e4m3fn value).
//
// One wave per token, DIM / 64 elements per lane (head dim 128 or 64):
//   amax  = max |k[t, :]|                          (wave reduction)
//   scale = max(amax, 1e-12) / 448                 (correctly rounded fp32 division)
//   q     = e4m3fn_rne(clamp(k / scale, -448, 448))
// then the DIM code bytes go to the token's slot (one row per wave, 2- or
// 1-byte stores) and lane 0 writes the scale, in the block-split layout of
// the decode cache: K rows slot-major, or in the preshuffled (16,16) order
// (byte d of slot s at (s/16) 16 DIM + (d/16) 256 + (s%16) 16 + d%16; the
// 64-token pairing on the aiter PR 5047 page, "Technical Details").  Tokens
// whose slot is negative or past the cache are skipped.  K must be finite.
#include "device.h"
#include "launch.h"

namespace mqa {
namespace {

constexpr int kTokensPerBlock = 4;  // waves per workgroup

// fp32 in [-448, 448] -> e4m3fn code, round to nearest, ties to even, sign
// kept (a negative value that rounds to zero gives -0).  Codes m 2^-9 below
// 2^-6 (subnormals, m = 0..8), else exponent E in [-6, 8] with three mantissa
// bits: code = (E + 7) << 3 | (mantissa).  Scaling by powers of two is exact,
// so the only rounding is the v_rndne of the scaled value.
__device__ __forceinline__ uint32_t e4m3fn_rne(float q)
{
    const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
    const float a = fabsf(q);
    uint32_t code;
    if (a < 0.015625f) {
        code = (uint32_t)rintf(a * 512.0f);  // 8 is 2^-6, the smallest normal
    } else {
        int e;
        (void)frexpf(a, &e);                  // a = f 2^e, f in [0.5, 1)
        uint32_t m = (uint32_t)rintf(ldexpf(a, 4 - e));  // 8..16
        int E = e - 1;
        if (m == 16u) {
            m = 8u;
            ++E;
        }
        code = ((uint32_t)(E + 7) << 3) | (m - 8u);
    }
    return sign | code;
}

template <bool BF16, int DIM>
__global__ __launch_bounds__(64 * kTokensPerBlock) void kcache_insert_kernel(
    const void *__restrict__ k, const int64_t *__restrict__ slots, uint8_t *__restrict__ cache,
    int tokens, int block_size, int64_t num_slots, int tiled)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kTokensPerBlock + (int)(threadIdx.x >> 6);
    if (t >= tokens)
        return;
    const int64_t s = slots[t];
    if (s < 0 || s >= num_slots)
        return;
    static_assert(DIM == 128 || DIM == 64, "head dim 128 or 64");
    float x0, x1 = 0.f;  // elements 2 lane, 2 lane + 1 (DIM 128) or lane (DIM 64)
    if (DIM == 128) {
        if (BF16) {
            const uint32_t w = reinterpret_cast<const uint32_t *>(k)[(int64_t)t * 64 + lane];
            x0 = __uint_as_float(w << 16);
            x1 = __uint_as_float(w & 0xffff0000u);
        } else {
            const float2 v = reinterpret_cast<const float2 *>(k)[(int64_t)t * 64 + lane];
            x0 = v.x;
            x1 = v.y;
        }
    } else {
        if (BF16)
            x0 = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(k)[(int64_t)t * 64 + lane]
                                 << 16);
        else
            x0 = reinterpret_cast<const float *>(k)[(int64_t)t * 64 + lane];
    }
    float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int d = 1; d < 64; d <<= 1)
        amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    const float scale = fmaxf(amax, 1e-12f) / 448.0f;
    const float q0 = fminf(fmaxf(x0 / scale, -448.0f), 448.0f);
    const float q1 = fminf(fmaxf(x1 / scale, -448.0f), 448.0f);
    const int64_t blk = s / block_size;
    const int slot = (int)(s - blk * block_size);
    uint8_t *base = cache + blk * (int64_t)block_size * (DIM + 4);
    const int d = (DIM / 64) * lane;
    const int off = tiled ? (slot >> 4) * (16 * DIM) + (d >> 4) * 256 + (slot & 15) * 16 + (d & 15)
                          : slot * DIM + d;
    if (DIM == 128)
        *reinterpret_cast<uint16_t *>(base + off) =
            (uint16_t)(e4m3fn_rne(q0) | (e4m3fn_rne(q1) << 8));
    else
        base[off] = (uint8_t)e4m3fn_rne(q0);
    if (lane == 0)
        *reinterpret_cast<float *>(base + (int64_t)block_size * DIM + 4 * slot) = scale;
}

template <bool BF16, int DIM>
hipError_t launch_insert(const KcacheLaunch &p, hipStream_t stream)
{
    const int grid = (p.tokens + kTokensPerBlock - 1) / kTokensPerBlock;
    hipLaunchKernelGGL((kcache_insert_kernel<BF16, DIM>), dim3(grid), dim3(64 * kTokensPerBlock), 0,
                       stream, p.k, p.slots, p.cache, p.tokens, p.block_size, p.num_slots, p.tiled);
    return hipGetLastError();
}

} // namespace

hipError_t launch_kcache_insert(const KcacheLaunch &p, hipStream_t stream)
{
    if (p.head_dim == 64)
        return p.bf16 ? launch_insert<true, 64>(p, stream) : launch_insert<false, 64>(p, stream);
    return p.bf16 ? launch_insert<true, 128>(p, stream) : launch_insert<false, 128>(p, stream);
}

} // namespace mqa
