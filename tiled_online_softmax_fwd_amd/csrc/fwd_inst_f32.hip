// fwd_inst_f32.hip -- instance table of the fp32 forward kernels.
#include "fwd_kernel.h"
#include "fwd_m16.h"
#include "fwd_tiles.h"

namespace attnk {
LaunchFn lookup_f32(int D, int BR, int BC)
{
#define X(d, br, bc) if (D == d && BR == br && BC == bc) return &launch_f32<d, br, bc>;
    ATTN_FWD_TILES(X, 64)
    ATTN_FWD_TILES(X, 128)
#undef X
#define X(d, br, bc) if (D == d && BR == br && BC == bc) return &launch_m16<float, d, br, bc>;
    ATTN_FWD_TILES_16(X, 64)
    ATTN_FWD_TILES_16(X, 128)
#undef X
    return nullptr;
}
}  // namespace attnk
