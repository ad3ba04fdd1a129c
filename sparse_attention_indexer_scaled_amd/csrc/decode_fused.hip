// The fused decode top-k's two decode modes (gfx950): the sample and the
// filter (decode_kernel.h, DecodeMode), for every cache layout and head count
// the logits call takes.  The ring depth is the logits call's default: 3
// steps, 4 for per-token blocks.
#include "decode_kernel.h"

namespace mqa {
namespace {

template <int MODE>
hipError_t launch_fused_mode(const DecodeLaunch &p, const DecodeArgs &a, int grid,
                             hipStream_t stream)
{
    switch (p.head_tiles) {
    case 1: return launch_ht<1, MODE>(p, a, grid, stream);
    case 2: return launch_ht<2, MODE>(p, a, grid, stream);
    case 4: return launch_ht<4, MODE>(p, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

hipError_t launch_decode_fused(const DecodeLaunch &p, hipStream_t stream)
{
    const DecodeArgs a = decode_args(p);
    const int grid = p.batch * a.split;
    switch (p.mode) {
    case kSample: return launch_fused_mode<kSample>(p, a, grid, stream);
    case kFilter: return launch_fused_mode<kFilter>(p, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mqa
