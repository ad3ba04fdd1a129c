// The fused decode top-k's sample and filter modes at head dim 64 (gfx950):
// 32, 64 and 128 heads, blocks of 1, 16, 64 or 128 tokens, the logits call's ring depth
// (kernel template in decode_kernel.h).
#include "decode_kernel.h"

namespace mqa {
namespace {

template <int MODE>
hipError_t launch_fused_d64_mode(const DecodeLaunch &p, const DecodeArgs &a, int grid,
                                 hipStream_t stream)
{
    switch (p.head_tiles) {
    case 1: return launch_ht<1, MODE, 64>(p, a, grid, stream);
    case 2: return launch_ht<2, MODE, 64>(p, a, grid, stream);
    case 4: return launch_ht<4, MODE, 64>(p, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

hipError_t launch_decode_fused_d64(const DecodeLaunch &p, hipStream_t stream)
{
    const DecodeArgs a = decode_args(p);
    const int grid = p.batch * a.split;
    switch (p.mode) {
    case kSample: return launch_fused_d64_mode<kSample>(p, a, grid, stream);
    case kFilter: return launch_fused_d64_mode<kFilter>(p, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mqa
