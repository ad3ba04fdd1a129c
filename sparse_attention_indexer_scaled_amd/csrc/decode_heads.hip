// Paged decode logits at 64 and 128 index heads (gfx950): 2 or 4 MFMA head
// tiles per row over the same K stream, every block size and K order, ring
// depth 3, or 4 for per-token blocks (kernel template in decode_kernel.h).
#include "decode_kernel.h"

namespace mqa {

hipError_t launch_decode_heads(const DecodeLaunch &p, hipStream_t stream)
{
    const DecodeArgs a = decode_args(p);
    const int grid = p.batch * a.split;
    switch (p.head_tiles) {
    case 2: return launch_ht<2, kLogits>(p, a, grid, stream);
    case 4: return launch_ht<4, kLogits>(p, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mqa
