// Paged decode logits (gfx950): the launches of the logits call at 32 heads.
// The kernel template, its work decomposition and its gather are in
// decode_kernel.h; 64 and 128 heads are launched from decode_heads.hip, head
// dim 64 from decode_d64.hip, the fused top-k's sample and filter modes from
// decode_fused.hip and decode_fused_d64.hip (separate translation units, so
// the instantiations compile in parallel).
#include "decode_kernel.h"

namespace mqa {

hipError_t launch_decode(const DecodeLaunch &p, hipStream_t stream)
{
    if (p.mode != kLogits)
        return p.head_dim == 64 ? launch_decode_fused_d64(p, stream) : launch_decode_fused(p, stream);
    if (p.head_dim == 64)
        return launch_decode_d64(p, stream);
    if (p.head_tiles != 1)
        return launch_decode_heads(p, stream);
    const DecodeArgs a = decode_args(p);
    return launch_ht<1, kLogits>(p, a, p.batch * a.split, stream);
}

} // namespace mqa
