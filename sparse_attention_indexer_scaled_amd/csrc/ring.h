// LDS ring of 64-token K steps (gfx950), shared by the paged decode and the
// prefill: the slot layout, the wait for a wave's own global->LDS loads, and
// the LDS reads into the MFMA operand layout.  A slot is filled by
// global_load_lds (the requesting code is the kernels' own, since the decode
// gathers through a block table and the prefill reads a contiguous K).
#pragma once

#include "device.h"

namespace mqa {
namespace {

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// A ring slot holds one 64-token step: the K rows (DIM bytes each), then the
// 64 scales.  The K rows arrive as 1 KiB chunks of 1024 / DIM rows each.
template <int DIM>
constexpr int slot_bytes() { return kStep * DIM + kStep * 4; }
template <int DIM>
constexpr int k_chunks() { return kStep * DIM / 1024; }
template <int DIM>
constexpr int rows_per_chunk() { return 1024 / DIM; }

// The fewest global->LDS loads any wave of G issues per step, with
// loads_per_chunk loads per each of kchunks K chunks and the scale load on the
// last wave.
constexpr int min_loads_per_step(int G, int loads_per_chunk, int kchunks)
{
    int m = 1 << 30;
    for (int g = 0; g < G; ++g) {
        int n = g == G - 1 ? 1 : 0;
        for (int c = g; c < kchunks; c += G)
            n += loads_per_chunk;
        m = n < m ? n : m;
    }
    return m;
}

// Wait until at most N vector memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Read a ring slot into registers (head dim 128).  Lane (t, g') needs token
// 32 h + t, granules u = 2j + g', j = 0..3: chunk c = 4h + t/8 (same parity
// for both tiles), logical granule q = 16 j + 8 g' + t % 8, stored at position
// q ^ 8 (c & 1) = 16 j + 8 (g' ^ (c & 1)) + t % 8, so read j sits 256 bytes
// after read 0.  Head dim 64: chunk c = 2h + t/16 holds rows 16c..16c+15
// unswizzled (granule u of row tau at position 16 u + tau), lane (t, g') reads
// u = 2j + g', j = 0, 1, at position 32 j + 16 g' + t % 16; each 16-lane pass
// of ds_read_b128 then reads 256 contiguous bytes, all 64 banks once.  The
// reads are inline asm because the compiler would otherwise make every LDS
// read wait for all outstanding global->LDS loads; read_wait() completes them.
template <int DIM>
__device__ __forceinline__ void read_block(KStepOf<DIM> &k, uint32_t slot, int lane)
{
    const int t = lane & 31, gq = lane >> 5;
    const uint32_t sa = slot + kStep * DIM + t * 4;
    if constexpr (DIM == 128) {
        const int c = t >> 3;  // chunk within the tile; tile 1 adds 4 (same parity)
        const int p0 = 8 * (gq ^ (c & 1)) + (t & 7);
        const uint32_t a0 = slot + (c * 1024 + p0 * 16);
        const uint32_t a1 = a0 + 4096;
        asm volatile("ds_read_b128 %0, %1 offset:0" : "=v"(k.t[0].c[0]) : "v"(a0));
        asm volatile("ds_read_b128 %0, %1 offset:256" : "=v"(k.t[0].c[1]) : "v"(a0));
        asm volatile("ds_read_b128 %0, %1 offset:512" : "=v"(k.t[0].c[2]) : "v"(a0));
        asm volatile("ds_read_b128 %0, %1 offset:768" : "=v"(k.t[0].c[3]) : "v"(a0));
        asm volatile("ds_read_b128 %0, %1 offset:0" : "=v"(k.t[1].c[0]) : "v"(a1));
        asm volatile("ds_read_b128 %0, %1 offset:256" : "=v"(k.t[1].c[1]) : "v"(a1));
        asm volatile("ds_read_b128 %0, %1 offset:512" : "=v"(k.t[1].c[2]) : "v"(a1));
        asm volatile("ds_read_b128 %0, %1 offset:768" : "=v"(k.t[1].c[3]) : "v"(a1));
    } else {
        static_assert(DIM == 64, "head dim 64 or 128");
        const uint32_t a0 = slot + (t >> 4) * 1024 + (16 * gq + (t & 15)) * 16;
        const uint32_t a1 = a0 + 2048;
        asm volatile("ds_read_b128 %0, %1 offset:0" : "=v"(k.t[0].c[0]) : "v"(a0));
        asm volatile("ds_read_b128 %0, %1 offset:512" : "=v"(k.t[0].c[1]) : "v"(a0));
        asm volatile("ds_read_b128 %0, %1 offset:0" : "=v"(k.t[1].c[0]) : "v"(a1));
        asm volatile("ds_read_b128 %0, %1 offset:512" : "=v"(k.t[1].c[1]) : "v"(a1));
    }
    asm volatile("ds_read_b32 %0, %1 offset:0" : "=v"(k.sc[0]) : "v"(sa));
    asm volatile("ds_read_b32 %0, %1 offset:128" : "=v"(k.sc[1]) : "v"(sa));
}

// Wait for read_block's results; the registers pass through the asm, so no
// use of them can be scheduled before the wait.
template <int DIM>
__device__ __forceinline__ void read_wait(KStepOf<DIM> &k)
{
    if constexpr (DIM == 128) {
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(k.t[0].c[0]), "+v"(k.t[0].c[1]), "+v"(k.t[0].c[2]), "+v"(k.t[0].c[3]),
                       "+v"(k.t[1].c[0]), "+v"(k.t[1].c[1]), "+v"(k.t[1].c[2]), "+v"(k.t[1].c[3]),
                       "+v"(k.sc[0]), "+v"(k.sc[1])
                     :
                     : "memory");
    } else {
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(k.t[0].c[0]), "+v"(k.t[0].c[1]), "+v"(k.t[1].c[0]), "+v"(k.t[1].c[1]),
                       "+v"(k.sc[0]), "+v"(k.sc[1])
                     :
                     : "memory");
    }
}

}  // namespace
}  // namespace mqa
