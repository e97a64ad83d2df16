// fwd_tiles.h -- the (BR, BC) tile shapes compiled for every input type and
// head size.  X(D, BR, BC) is expanded by each instance table.
#pragma once
#define ATTN_FWD_TILES(X, D) \
    X(D, 32, 32)  X(D, 32, 64)  X(D, 32, 128) \
    X(D, 64, 32)  X(D, 64, 64)  X(D, 64, 128) \
    X(D, 128, 32) X(D, 128, 64) X(D, 128, 128)
