// fwd_inst_f16.hip -- instance table of the f16 forward kernels.
#include "fwd_kernel.h"
#include "fwd_m16.h"
#include "fwd_tiles.h"

namespace attnk {
LaunchFn lookup_f16(int D, int BR, int BC)
{
#define X(d, br, bc) if (D == d && BR == br && BC == bc) return &launch_h16<_Float16, d, br, bc>;
    ATTN_FWD_TILES(X, 64)
    ATTN_FWD_TILES(X, 128)
    ATTN_FWD_TILES_WIDE_64(X)
    ATTN_FWD_TILES_WIDE_128(X)
#undef X
#define X(d, br, bc) if (D == d && BR == br && BC == bc) return &launch_m16<_Float16, d, br, bc>;
    ATTN_FWD_TILES_16(X, 64)
    ATTN_FWD_TILES_16(X, 128)
#undef X
    return nullptr;
}
}  // namespace attnk
