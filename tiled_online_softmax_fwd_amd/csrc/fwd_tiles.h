// fwd_tiles.h -- the (BR, BC) tile shapes compiled for every input type and
// head size.  X(D, BR, BC) is expanded by each instance table.
#pragma once
#define ATTN_FWD_TILES(X, D) \
    X(D, 32, 32)  X(D, 32, 64)  X(D, 32, 128) \
    X(D, 64, 32)  X(D, 64, 64)  X(D, 64, 128) \
    X(D, 128, 32) X(D, 128, 64) X(D, 128, 128)

// 256-row tiles (eight waves) for the 16-bit kernels only; every wave needs at
// least one 1 KiB LDS-copy instruction per key tile.
#define ATTN_FWD_TILES_WIDE_64(X) X(64, 256, 64)
#define ATTN_FWD_TILES_WIDE_128(X) X(128, 256, 32) X(128, 256, 64) X(128, 256, 128)

// Tiles with 16 query rows or 16 keys (fwd_m16.h, 16x16 matrix-core shapes),
// for every input type and head size.
#define ATTN_FWD_TILES_16(X, D) \
    X(D, 16, 16)  X(D, 16, 32)  X(D, 16, 64) X(D, 16, 128) \
    X(D, 32, 16)  X(D, 64, 16)  X(D, 128, 16)

// Tiles with a block-sparse instance (16-bit inputs): the defaults and their
// neighbours.
#define ATTN_FWD_TILES_SPARSE(X, D) X(D, 64, 64) X(D, 128, 64) X(D, 128, 128) X(D, 256, 64)
