// Paged decode logits at head dim 64 (gfx950): 64-byte K rows, so a 64-token
// step is four 1 KiB chunks of 16 rows, and one fp8 MFMA per (row, tile, head
// tile) instead of two.  32, 64 and 128 heads; blocks of 16, 64 or 128 tokens
// in either K order; ring depth 3, or 4 for per-token blocks (kernel
// template in decode_kernel.h).
#include "decode_kernel.h"

namespace mqa {

hipError_t launch_decode_d64(const DecodeLaunch &p, hipStream_t stream)
{
    const DecodeArgs a = decode_args(p);
    const int grid = p.batch * a.split;
    switch (p.head_tiles) {
    case 1: return launch_ht<1, kLogits, 64>(p, a, grid, stream);
    case 2: return launch_ht<2, kLogits, 64>(p, a, grid, stream);
    case 4: return launch_ht<4, kLogits, 64>(p, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mqa
