// The fused decode top-k's two decode modes (gfx950): the sample and the
// filter (decode_kernel.h, DecodeMode), for every cache layout and head count
// the logits call takes.  The ring depth is the logits call's default: 3
// steps for 64-token blocks at 32 heads, 4 for the rest.
#include "decode_kernel.h"

namespace mqa {
namespace {

template <int R, int G, int HT, int MODE>
hipError_t launch_fused_rg(const DecodeLaunch &p, const DecodeArgs &a, int grid, hipStream_t stream)
{
    if constexpr (R * HT > 4) {
        // Q and weights of a wave's rows stay in VGPRs: at most 4 / HT rows
        return hipErrorInvalidValue;
    } else if constexpr (HT == 1) {
        switch (p.block_size) {
        case 64:
            return p.depth == 3 ? launch_rgdb<R, G, 3, 64, 1, MODE>(p, a, grid, stream)
                                : hipErrorInvalidValue;
        case 1:
            return p.depth == 4 ? launch_rgdb<R, G, 4, 1, 1, MODE>(p, a, grid, stream)
                                : hipErrorInvalidValue;
        case 16:
            return p.depth == 4 ? launch_rgdb<R, G, 4, 16, 1, MODE>(p, a, grid, stream)
                                : hipErrorInvalidValue;
        case 128:
            return p.depth == 4 ? launch_rgdb<R, G, 4, 128, 1, MODE>(p, a, grid, stream)
                                : hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
        }
    } else {
        // 64 and 128 heads: 64-token blocks
        if (p.block_size != 64 || p.depth != 4)
            return hipErrorInvalidValue;
        return launch_rgdb<R, G, 4, 64, HT, MODE>(p, a, grid, stream);
    }
}

// (rows, row groups) pairs that next_n in 1..8 can produce
template <int HT, int MODE>
hipError_t launch_fused_ht(const DecodeLaunch &p, const DecodeArgs &a, int grid,
                           hipStream_t stream)
{
    switch (p.rows * 16 + a.groups) {
    case 1 * 16 + 1: return launch_fused_rg<1, 1, HT, MODE>(p, a, grid, stream);
    case 1 * 16 + 2: return launch_fused_rg<1, 2, HT, MODE>(p, a, grid, stream);
    case 1 * 16 + 3: return launch_fused_rg<1, 3, HT, MODE>(p, a, grid, stream);
    case 1 * 16 + 4: return launch_fused_rg<1, 4, HT, MODE>(p, a, grid, stream);
    case 1 * 16 + 5: return launch_fused_rg<1, 5, HT, MODE>(p, a, grid, stream);
    case 1 * 16 + 6: return launch_fused_rg<1, 6, HT, MODE>(p, a, grid, stream);
    case 1 * 16 + 7: return launch_fused_rg<1, 7, HT, MODE>(p, a, grid, stream);
    case 1 * 16 + 8: return launch_fused_rg<1, 8, HT, MODE>(p, a, grid, stream);
    case 2 * 16 + 1: return launch_fused_rg<2, 1, HT, MODE>(p, a, grid, stream);
    case 2 * 16 + 2: return launch_fused_rg<2, 2, HT, MODE>(p, a, grid, stream);
    case 2 * 16 + 3: return launch_fused_rg<2, 3, HT, MODE>(p, a, grid, stream);
    case 2 * 16 + 4: return launch_fused_rg<2, 4, HT, MODE>(p, a, grid, stream);
    case 3 * 16 + 1: return launch_fused_rg<3, 1, HT, MODE>(p, a, grid, stream);
    case 3 * 16 + 2: return launch_fused_rg<3, 2, HT, MODE>(p, a, grid, stream);
    case 3 * 16 + 3: return launch_fused_rg<3, 3, HT, MODE>(p, a, grid, stream);
    case 4 * 16 + 1: return launch_fused_rg<4, 1, HT, MODE>(p, a, grid, stream);
    case 4 * 16 + 2: return launch_fused_rg<4, 2, HT, MODE>(p, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int MODE>
hipError_t launch_fused_mode(const DecodeLaunch &p, const DecodeArgs &a, int grid,
                             hipStream_t stream)
{
    switch (p.head_tiles) {
    case 1: return launch_fused_ht<1, MODE>(p, a, grid, stream);
    case 2: return launch_fused_ht<2, MODE>(p, a, grid, stream);
    case 4: return launch_fused_ht<4, MODE>(p, a, grid, stream);
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
