// fwd_inst_sparse.hip -- instance table of the block-sparse 16-bit forward
// kernels (fwd_m32_h16 with SPARSE = true).
#include "fwd_kernel.h"
#include "fwd_tiles.h"

namespace attnk {
LaunchFn lookup_sparse(int dtype_bits, int D, int BR, int BC)
{
#define X(d, br, bc) if (D == d && BR == br && BC == bc) return &launch_h16<__bf16, d, br, bc, true>;
    if (dtype_bits == 0) {
        ATTN_FWD_TILES_SPARSE(X, 64)
        ATTN_FWD_TILES_SPARSE(X, 128)
    }
#undef X
#define X(d, br, bc) if (D == d && BR == br && BC == bc) return &launch_h16<_Float16, d, br, bc, true>;
    if (dtype_bits == 1) {
        ATTN_FWD_TILES_SPARSE(X, 64)
        ATTN_FWD_TILES_SPARSE(X, 128)
    }
#undef X
    return nullptr;
}
}  // namespace attnk
