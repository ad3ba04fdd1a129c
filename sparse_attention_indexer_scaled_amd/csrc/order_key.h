// The top-k's order on logits (gfx950 device code shared by the top-k kernel
// and the decode kernel's filter mode).
//
// A value maps to a 32-bit key whose unsigned order is the value order: 0 for
// -inf and NaN (never selected), -0.0 like +0.0.  A sort entry is the key in
// the high word and ~column in the low word, so a larger entry ranks first
// (larger value, then smaller column) and 0 is padding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mqa {

__device__ __forceinline__ uint32_t order_key(float v)
{
    uint32_t u = __float_as_uint(v);
    if (!(v == v) || v == -__builtin_inff())
        return 0u;
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key on keys >= 0x00800000 (the key of -FLT_MAX): for such
// a key t and any float v, order_key(v) >= t exactly when v >= key_value(t).
__device__ __forceinline__ float key_value(uint32_t t)
{
    return __uint_as_float((t & 0x80000000u) ? (t & 0x7fffffffu) : ~t);
}

// The float f with order_key(v) >= t <=> v >= f for every finite v (t >= 1).
__device__ __forceinline__ float key_float(uint32_t t)
{
    return key_value(t > 0x00800000u ? t : 0x00800000u);
}

__device__ __forceinline__ uint64_t entry(uint32_t key, int col)
{
    return ((uint64_t)key << 32) | (uint32_t)(~(uint32_t)col);
}

__device__ __forceinline__ uint64_t fused_entry(float v, int col)
{
    return entry(order_key(v), col);
}

} // namespace mqa
