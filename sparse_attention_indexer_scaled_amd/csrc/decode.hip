// Paged decode logits (gfx950): the launches of the logits call.  The kernel
// template, its work decomposition and its gather are in decode_kernel.h; the
// fused top-k's sample and filter modes are launched from decode_fused.hip.
#include "decode_kernel.h"

namespace mqa {
namespace {

template <int R, int G>
hipError_t launch_rg(const DecodeLaunch &p, const DecodeArgs &a, int grid, hipStream_t stream)
{
    if (p.block_size == 64) {
        switch (p.depth) {
        case 2: return launch_rgdb<R, G, 2, 64>(p, a, grid, stream);
        case 3: return launch_rgdb<R, G, 3, 64>(p, a, grid, stream);
        case 4: return launch_rgdb<R, G, 4, 64>(p, a, grid, stream);
        case 5: return launch_rgdb<R, G, 5, 64>(p, a, grid, stream);
        case 6: return launch_rgdb<R, G, 6, 64>(p, a, grid, stream);
        case 7: return launch_rgdb<R, G, 7, 64>(p, a, grid, stream);
        default: return hipErrorInvalidValue;
        }
    }
    // other block sizes: the default ring depth only
    if (p.depth != 4)
        return hipErrorInvalidValue;
    switch (p.block_size) {
    case 1: return launch_rgdb<R, G, 4, 1>(p, a, grid, stream);
    case 16: return launch_rgdb<R, G, 4, 16>(p, a, grid, stream);
    case 128: return launch_rgdb<R, G, 4, 128>(p, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

int decode_ring_bytes(int depth) { return depth * kSlotBytes; }

hipError_t launch_decode(const DecodeLaunch &p, hipStream_t stream)
{
    if (p.mode != kLogits)
        return launch_decode_fused(p, stream);
    const DecodeArgs a = decode_args(p);
    const int grid = p.batch * a.split;
    if (p.head_tiles == 2) {
        // 64 heads: at most 2 rows per wave (Q and weights take 64 VGPRs a row)
        switch (p.rows * 16 + a.groups) {
        case 1 * 16 + 1: return launch_rgdb<1, 1, 4, 64, 2>(p, a, grid, stream);
        case 1 * 16 + 2: return launch_rgdb<1, 2, 4, 64, 2>(p, a, grid, stream);
        case 1 * 16 + 3: return launch_rgdb<1, 3, 4, 64, 2>(p, a, grid, stream);
        case 1 * 16 + 4: return launch_rgdb<1, 4, 4, 64, 2>(p, a, grid, stream);
        case 1 * 16 + 5: return launch_rgdb<1, 5, 4, 64, 2>(p, a, grid, stream);
        case 1 * 16 + 6: return launch_rgdb<1, 6, 4, 64, 2>(p, a, grid, stream);
        case 1 * 16 + 7: return launch_rgdb<1, 7, 4, 64, 2>(p, a, grid, stream);
        case 1 * 16 + 8: return launch_rgdb<1, 8, 4, 64, 2>(p, a, grid, stream);
        case 2 * 16 + 1: return launch_rgdb<2, 1, 4, 64, 2>(p, a, grid, stream);
        case 2 * 16 + 2: return launch_rgdb<2, 2, 4, 64, 2>(p, a, grid, stream);
        case 2 * 16 + 3: return launch_rgdb<2, 3, 4, 64, 2>(p, a, grid, stream);
        case 2 * 16 + 4: return launch_rgdb<2, 4, 4, 64, 2>(p, a, grid, stream);
        default: return hipErrorInvalidValue;
        }
    }
    if (p.head_tiles == 4) {
        // 128 heads: one row per wave
        switch (a.groups) {
        case 1: return launch_rgdb<1, 1, 4, 64, 4>(p, a, grid, stream);
        case 2: return launch_rgdb<1, 2, 4, 64, 4>(p, a, grid, stream);
        case 3: return launch_rgdb<1, 3, 4, 64, 4>(p, a, grid, stream);
        case 4: return launch_rgdb<1, 4, 4, 64, 4>(p, a, grid, stream);
        case 5: return launch_rgdb<1, 5, 4, 64, 4>(p, a, grid, stream);
        case 6: return launch_rgdb<1, 6, 4, 64, 4>(p, a, grid, stream);
        case 7: return launch_rgdb<1, 7, 4, 64, 4>(p, a, grid, stream);
        case 8: return launch_rgdb<1, 8, 4, 64, 4>(p, a, grid, stream);
        default: return hipErrorInvalidValue;
        }
    }
    // (rows, row groups) pairs that next_n in 1..8 can produce
    switch (p.rows * 16 + a.groups) {
    case 1 * 16 + 1: return launch_rg<1, 1>(p, a, grid, stream);
    case 1 * 16 + 2: return launch_rg<1, 2>(p, a, grid, stream);
    case 1 * 16 + 3: return launch_rg<1, 3>(p, a, grid, stream);
    case 1 * 16 + 4: return launch_rg<1, 4>(p, a, grid, stream);
    case 1 * 16 + 5: return launch_rg<1, 5>(p, a, grid, stream);
    case 1 * 16 + 6: return launch_rg<1, 6>(p, a, grid, stream);
    case 1 * 16 + 7: return launch_rg<1, 7>(p, a, grid, stream);
    case 1 * 16 + 8: return launch_rg<1, 8>(p, a, grid, stream);
    case 2 * 16 + 1: return launch_rg<2, 1>(p, a, grid, stream);
    case 2 * 16 + 2: return launch_rg<2, 2>(p, a, grid, stream);
    case 2 * 16 + 3: return launch_rg<2, 3>(p, a, grid, stream);
    case 2 * 16 + 4: return launch_rg<2, 4>(p, a, grid, stream);
    case 3 * 16 + 1: return launch_rg<3, 1>(p, a, grid, stream);
    case 3 * 16 + 2: return launch_rg<3, 2>(p, a, grid, stream);
    case 3 * 16 + 3: return launch_rg<3, 3>(p, a, grid, stream);
    case 4 * 16 + 1: return launch_rg<4, 1>(p, a, grid, stream);
    case 4 * 16 + 2: return launch_rg<4, 2>(p, a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mqa
