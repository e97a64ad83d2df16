// attn_host.h -- host-only part of the C ABI declared in include/attn.h:
// argument checks, tile and grid planning, and the ATTN_TRACE dispatch log.
// No HIP type or call appears here, so the same code builds into libattn.so
// (attn_api.cpp) and, with a plain C++ compiler under AddressSanitizer and
// UndefinedBehaviorSanitizer, into the host checks of the test suite.
//
// Every check runs before any HIP call; a rejected call returns its attn_status
// with a message in attn_last_error() and touches no memory it was given
// (pointers are compared as integers, never dereferenced).
#pragma once
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "attn.h"
#include "fwd_tiles.h"

namespace attnh {

inline thread_local char g_err[512] = "";

inline int fail(int status, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

inline int ok()
{
    g_err[0] = '\0';
    return ATTN_OK;
}

inline bool valid_dtype(int dtype) { return dtype >= ATTN_F32 && dtype <= ATTN_BF16_OUT_F32; }
inline size_t elem_bytes_in(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }
inline size_t elem_bytes_out(int dtype)
{
    return (dtype == ATTN_F32 || dtype == ATTN_F16_OUT_F32 || dtype == ATTN_BF16_OUT_F32) ? 4 : 2;
}
inline bool is_f16(int dtype) { return dtype == ATTN_F16 || dtype == ATTN_F16_OUT_F32; }

inline const char* dtype_name(int dtype)
{
    switch (dtype) {
    case ATTN_F32: return "f32";
    case ATTN_F16: return "f16";
    case ATTN_BF16: return "bf16";
    case ATTN_F16_OUT_F32: return "f16>f32";
    case ATTN_BF16_OUT_F32: return "bf16>f32";
    default: return "?";
    }
}

// Byte ranges [a, a + na) and [b, b + nb) intersect (empty ranges never do).
inline bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

inline bool valid_tile(int t) { return t == 16 || t == 32 || t == 64 || t == 128; }
inline bool valid_br(int t) { return valid_tile(t) || t == 256; }

// Defaults per input type and head size (measured on MI355X): 16-bit inputs
// at d = 128 use 256 query rows per workgroup (eight waves of 32 rows sharing
// each K/V tile) and 64 keys per tile; at d = 64 the state is half as large and
// 128 x 128 tiles run best (three workgroups per compute unit); fp32 uses
// 128 x 64 (its tiles are twice as large in LDS).
inline void defaults(int dtype, int d, int causal, int* br, int* bc)
{
    (void)causal;
    if (dtype == ATTN_F32) { *br = 128; *bc = 64; }
    else if (d == 64) { *br = 128; *bc = 128; }
    else { *br = 256; *bc = 64; }
}

// The dense forward instances compiled into the library (fwd_tiles.h lists
// them; the fwd_inst_*.hip tables expand the same lists).
inline bool fwd_built(int dtype, int d, int br, int bc)
{
    if (!valid_dtype(dtype)) return false;
#define X(D_, BR_, BC_) if (d == D_ && br == BR_ && bc == BC_) return true;
    ATTN_FWD_TILES(X, 64)
    ATTN_FWD_TILES(X, 128)
    ATTN_FWD_TILES_16(X, 64)
    ATTN_FWD_TILES_16(X, 128)
    if (dtype != ATTN_F32) {
        ATTN_FWD_TILES_WIDE_64(X)
        ATTN_FWD_TILES_WIDE_128(X)
    }
#undef X
    return false;
}

// The block-sparse instances (16-bit inputs only).
inline bool sparse_built(int d, int br, int bc)
{
#define X(D_, BR_, BC_) if (d == D_ && br == BR_ && bc == BC_) return true;
    ATTN_FWD_TILES_SPARSE(X, 64)
    ATTN_FWD_TILES_SPARSE(X, 128)
#undef X
    return false;
}

// Everything that does not involve a pointer.
inline int check_scalars(int B, int H, int N, int d, float scale, int dtype)
{
    if (!valid_dtype(dtype)) return fail(ATTN_ERR_DTYPE, "dtype %d is not an attn_dtype", dtype);
    if (B < 0 || H < 0 || N < 0) return fail(ATTN_ERR_SHAPE, "negative size B=%d H=%d N=%d", B, H, N);
    if ((int64_t)B * H * N >= ((int64_t)1 << 31))
        return fail(ATTN_ERR_SHAPE, "B*H*N = %lld rows exceeds 2^31 - 1", (long long)B * H * N);
    if (d != 64 && d != 128) return fail(ATTN_ERR_HEAD_DIM, "head size d=%d, supported: 64, 128", d);
    if (!std::isfinite(scale)) return fail(ATTN_ERR_SCALE, "scale %g must be finite", (double)scale);
    return ATTN_OK;
}

// Kernels that keep a running maximum of raw scores take a positive factor:
// scale < 0 runs as |scale| on negated Q, scale = 0 as 1 on Q = 0 (both exact;
// the kernels apply the Q mode as they load Q).  Returns the factor the
// kernels use and sets the Q mode (0 as given, 1 negated, 2 zero).
inline float kernel_scale(float scale, int* qmode)
{
    if (scale > 0.f) { *qmode = 0; return scale; }
    if (scale < 0.f) { *qmode = 1; return -scale; }
    *qmode = 2;
    return 1.f;
}

// scale * log2(e), rounded once to fp32: the factor of the base-2 exponent.
inline float log2e_factor(float s) { return (float)((double)s * 1.4426950408889634); }

inline int check_pointers(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          int B, int H, int N, int d, int dtype)
{
    if (!q || !k || !v || !o) return fail(ATTN_ERR_NULL, "q, k, v and o must be non-NULL");
    const void* p16[4] = {q, k, v, o};
    const char* names[4] = {"q", "k", "v", "o"};
    for (int i = 0; i < 4; ++i)
        if ((uintptr_t)p16[i] % 16) return fail(ATTN_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    if (lse && ((uintptr_t)lse % 4)) return fail(ATTN_ERR_ALIGN, "lse is not 4-byte aligned");
    const size_t rows = (size_t)B * H * N;
    const size_t nin = rows * d * elem_bytes_in(dtype), nout = rows * d * elem_bytes_out(dtype);
    const size_t nlse = lse ? rows * sizeof(float) : 0;
    if (overlaps(o, nout, q, nin) || overlaps(o, nout, k, nin) || overlaps(o, nout, v, nin) ||
        overlaps(o, nout, lse, nlse))
        return fail(ATTN_ERR_ALIAS, "o overlaps q, k, v or lse");
    if (overlaps(lse, nlse, q, nin) || overlaps(lse, nlse, k, nin) || overlaps(lse, nlse, v, nin))
        return fail(ATTN_ERR_ALIAS, "lse overlaps q, k or v");
    return ATTN_OK;
}

inline int resolve_opts(int dtype, int d, int causal, const attn_opts* opts, int* br, int* bc, int* order,
                        int* slack, int* generic)
{
    defaults(dtype, d, causal, br, bc);
    *order = 0;
    *slack = 0;
    *generic = 0;
    if (!opts) return ATTN_OK;
    *generic = opts->generic_loop != 0;
    for (int i = 0; i < 3; ++i)
        if (opts->reserved[i] != 0) return fail(ATTN_ERR_TILE, "attn_opts.reserved[%d] must be 0", i);
    if (opts->br != 0) {
        if (!valid_br(opts->br)) return fail(ATTN_ERR_TILE, "br=%d not in {16,32,64,128,256}", opts->br);
        *br = opts->br;
    }
    if (opts->bc != 0) {
        if (!valid_tile(opts->bc)) return fail(ATTN_ERR_TILE, "bc=%d not in {16,32,64,128}", opts->bc);
        *bc = opts->bc;
        // br left to the library: use 128 rows where the wide tile is not built
        if (opts->br == 0 && !fwd_built(dtype, d, *br, *bc)) *br = 128;
    }
    if (opts->kv_order != 0 && opts->kv_order != 1) return fail(ATTN_ERR_TILE, "kv_order=%d not 0 or 1", opts->kv_order);
    *order = opts->kv_order;
    if (opts->ref_slack < 0 || opts->ref_slack > 15) return fail(ATTN_ERR_TILE, "ref_slack=%d not in 0..15", opts->ref_slack);
    *slack = opts->ref_slack;
    return ATTN_OK;
}

// ------------------------------------------------------------------ forward
// What a forward call runs: tiles, key order, reference lag, loop form, grid.
struct FwdPlan {
    int dtype = 0, d = 0, B = 0, H = 0, N = 0, causal = 0;
    int mask = 0, sparse = 0, block = 0;
    int br = 0, bc = 0, order = 0, slack = 0, generic = 0;
    int n_qt = 0;       // query tiles per (b, h)
    float kscale = 0.f; // factor the kernels use (> 0), see kernel_scale
    float c = 0.f;      // kscale * log2(e)
    int qmode = 0;
    int persist = 0;    // > 0: persistent grid of that many workgroups
    int xcd_affine = 0; // persistent items of head bh on XCD bh % 8
};

// Name of the kernel a plan launches (the choice the launchers make).
inline const char* fwd_kernel_name(const FwdPlan& p)
{
    if (p.br == 16 || p.bc == 16) return "fwd_m16";
    if (p.dtype == ATTN_F32) return 4 * p.bc * p.d * 4 <= 128 * 1024 ? "fwd_m32_f32_db" : "fwd_m32_f32";
    if (p.sparse) return "fwd_m32_h16_sparse";
    return p.mask ? "fwd_m32_h16_masked" : "fwd_m32_h16";
}

inline int fwd_block_threads(const FwdPlan& p) { return (p.br == 16 || p.bc == 16) ? p.br * 4 : p.br * 2; }

inline int64_t fwd_grid(const FwdPlan& p)
{
    return p.persist > 0 ? (int64_t)p.persist : (int64_t)p.B * p.H * p.n_qt;
}

// The 16-bit d = 128 kernel with 256 x 64 tiles, no mask and ascending keys
// runs its full unmasked key tiles through the software pipeline, with the
// exact or the lagging reference (unless generic_loop asks for the
// compiler-scheduled loop).
inline bool fwd_pipelined(const FwdPlan& p)
{
#ifdef ATTN_LDS_POISON
    // the LDS-poisoning debug build checks the copies the C++ loops issue; the
    // pipeline issues its own (its waits are checked by bitwise equality with
    // the C++ loop)
    (void)p;
    return false;
#else
    return p.dtype != ATTN_F32 && !p.sparse && !p.mask && p.d == 128 && p.br == 256 && p.bc == 64 &&
           !p.generic && p.order == 0;
#endif
}

// Persistent grid (pipelined instance only): one workgroup per compute unit
// when the items (query tiles, or causal pairs of query tiles of equal cost)
// split evenly over the G compute units; the items of a head then stay on one
// XCD when both the head count and the grid are multiples of the 8 XCDs.
// Otherwise one workgroup per query tile (the hardware's dynamic dispatch
// balances uneven work better).
inline void plan_persistent(FwdPlan& p, int G)
{
    p.persist = 0;
    p.xcd_affine = 0;
    if (!fwd_pipelined(p)) return;
    const int64_t BH = (int64_t)p.B * p.H;
    const int64_t iph = p.causal ? (p.n_qt + 1) / 2 : p.n_qt;
    const int64_t items = BH * iph;
    if (G <= 0 || items < G || items % G != 0) return;
    p.persist = G;
    p.xcd_affine = (BH % 8 == 0 && G % 8 == 0) ? 1 : 0;
}

inline void fill_fwd(FwdPlan& p, int B, int H, int N, int d, float scale, int causal, int dtype)
{
    p.dtype = dtype; p.d = d; p.B = B; p.H = H; p.N = N; p.causal = causal ? 1 : 0;
    p.n_qt = p.br > 0 ? (N + p.br - 1) / p.br : 0;
    p.kscale = kernel_scale(scale, &p.qmode);
    p.c = log2e_factor(p.kscale);
}

// attn_fwd / attn_fwd_ex / attn_check_args.  ATTN_OK with *empty set when
// B*H*N = 0 (nothing to launch).
inline int plan_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    int B, int H, int N, int d, float scale, int causal, const uint8_t* mask, int dtype,
                    const attn_opts* opts, FwdPlan* p, bool* empty)
{
    *empty = false;
    int st = check_scalars(B, H, N, d, scale, dtype);
    if (st) return st;
    st = resolve_opts(dtype, d, causal, opts, &p->br, &p->bc, &p->order, &p->slack, &p->generic);
    if (st) return st;
    if (!fwd_built(dtype, d, p->br, p->bc))
        return fail(ATTN_ERR_TILE, "no kernel for dtype %d, d=%d, br=%d, bc=%d", dtype, d, p->br, p->bc);
    p->mask = mask ? 1 : 0;
    fill_fwd(*p, B, H, N, d, scale, causal, dtype);
    if ((int64_t)B * H * N == 0) { *empty = true; return ATTN_OK; }
    return check_pointers(q, k, v, o, lse, B, H, N, d, dtype);
}

// attn_fwd_sparse.
inline int plan_sparse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       int B, int H, int N, int d, float scale, int causal, const uint8_t* mask,
                       const uint8_t* block_mask, int block, int dtype, const attn_opts* opts,
                       FwdPlan* p, bool* empty)
{
    *empty = false;
    int st = check_scalars(B, H, N, d, scale, dtype);
    if (st) return st;
    if (dtype == ATTN_F32) return fail(ATTN_ERR_DTYPE, "block-sparse forward: 16-bit inputs only");
    if (block < 32 || block % 32 != 0) return fail(ATTN_ERR_SHAPE, "block=%d must be a positive multiple of 32", block);
    st = resolve_opts(dtype, d, causal, opts, &p->br, &p->bc, &p->order, &p->slack, &p->generic);
    if (st) return st;
    if (p->order != 0) return fail(ATTN_ERR_TILE, "block-sparse forward: kv_order must be 0");
    // default 128 x 64: with blocks of 64 rows, wider workgroups visit tiles
    // where only some of their row blocks attend (measured on MI355X at
    // B1 H32 N8192, d = 64 and 128, random and sliding-window flags)
    if (!opts || opts->br == 0) p->br = 128;
    if (!opts || opts->bc == 0) p->bc = 64;
    if (!sparse_built(d, p->br, p->bc))
        return fail(ATTN_ERR_TILE, "no block-sparse kernel for d=%d, br=%d, bc=%d", d, p->br, p->bc);
    p->mask = mask ? 1 : 0;
    p->sparse = 1;
    p->block = block;
    fill_fwd(*p, B, H, N, d, scale, causal, dtype);
    if ((int64_t)B * H * N == 0) { *empty = true; return ATTN_OK; }
    st = check_pointers(q, k, v, o, lse, B, H, N, d, dtype);
    if (st) return st;
    if (!block_mask) return fail(ATTN_ERR_NULL, "block_mask must be non-NULL");
    const int nb = (N + block - 1) / block;
    const size_t nbm = (size_t)B * H * (size_t)nb * (size_t)nb;
    const size_t nout = (size_t)B * H * N * d * elem_bytes_out(dtype);
    if (overlaps(o, nout, block_mask, nbm) || overlaps(lse, lse ? (size_t)B * H * N * 4 : 0, block_mask, nbm))
        return fail(ATTN_ERR_ALIAS, "o or lse overlaps block_mask");
    return ATTN_OK;
}

// ------------------------------------------------------------ naive baseline
inline size_t naive_ws_bytes(int B, int H, int N, int dtype)
{
    if (B <= 0 || H <= 0 || N <= 0 || !valid_dtype(dtype)) return 0;
    return (size_t)B * H * (size_t)N * (size_t)N * elem_bytes_in(dtype);
}

inline int check_naive(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       int B, int H, int N, int d, float scale, int dtype, const void* workspace,
                       size_t workspace_bytes, bool* empty)
{
    *empty = false;
    int st = check_scalars(B, H, N, d, scale, dtype);
    if (st) return st;
    if ((int64_t)B * H * N == 0) { *empty = true; return ATTN_OK; }
    st = check_pointers(q, k, v, o, lse, B, H, N, d, dtype);
    if (st) return st;
    const size_t need = naive_ws_bytes(B, H, N, dtype);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % 16))
        return fail(ATTN_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned", need);
    const size_t rows = (size_t)B * H * N;
    const size_t nin = rows * d * elem_bytes_in(dtype);
    if (overlaps(workspace, need, q, nin) || overlaps(workspace, need, k, nin) || overlaps(workspace, need, v, nin) ||
        overlaps(workspace, need, o, rows * d * elem_bytes_out(dtype)) ||
        overlaps(workspace, need, lse, lse ? rows * 4 : 0))
        return fail(ATTN_ERR_ALIAS, "workspace overlaps an input or output");
    return ATTN_OK;
}

// ---------------------------------------------------------------- decode
// Key chunks of the decode path (whole 32-key tiles).  With units = B*H*ceil(Nq/16)
// row blocks, the library aims at about 1024 one-wave workgroups but takes
// fewer, down to about 512, where that keeps chunks at 1024 keys or more, and
// never makes chunks shorter than 256 keys.  Measured with the non-temporal tile
// copies (TB/s of the best split counts in brackets):
//   B8 H32 Nk 8192, Nq 1 or 16, d 64 or 128: 4 chunks (1024 workgroups) [6.2-6.4];
//   B1 H32 Nk 65536: 32 chunks (1024) [6.1]; B2 H8 Nk 32768: 32 chunks of 1024
//   keys (512) [4.7, against 4.3 for 64 chunks]; B1 H8 Nk 16384: 64 chunks of 256
//   keys (512) [2.0, against 1.3 for 16 chunks of 1024].
inline void decode_splits(int B, int H, int Nq, int Nk, int num_splits, int* splits, int* kps)
{
    const int tiles = (Nk + 31) / 32;
    int s = num_splits;
    if (s <= 0) {
        const int64_t units = (int64_t)B * H * ((Nq + 15) / 16);
        const int64_t hi = units > 0 ? (1024 + units - 1) / units : 1;   // about 1024 workgroups
        const int64_t lo = units > 0 ? (512 + units - 1) / units : 1;    // about 512 workgroups
        const int64_t long_chunks = tiles / 32 > 1 ? tiles / 32 : 1;     // chunks of >= 1024 keys
        const int64_t shortest = tiles / 8 > 1 ? tiles / 8 : 1;          // chunks of >= 256 keys
        int64_t want = long_chunks > lo ? long_chunks : lo;
        if (want > hi) want = hi;
        if (want > shortest) want = shortest;
        s = (int)(want < 1024 ? want : 1024);
    }
    if (s > tiles) s = tiles;
    if (s < 1) s = 1;
    const int per = (tiles + s - 1) / s;
    *kps = (per > 0 ? per : 1) * 32;
    *splits = Nk > 0 ? (Nk + *kps - 1) / *kps : 1;
}

inline size_t decode_ws_bytes(int B, int H, int Nq, int d, int splits)
{
    const size_t parts = (size_t)B * H * (size_t)splits * (size_t)Nq;
    return parts * (size_t)d * 4 + parts * 4;
}

inline size_t decode_ws_query(int B, int H, int Nq, int Nk, int d, int num_splits)
{
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk < 0 || (d != 64 && d != 128) || num_splits < 0 || num_splits > 1024) return 0;
    int splits, kps;
    decode_splits(B, H, Nq, Nk, num_splits, &splits, &kps);
    return decode_ws_bytes(B, H, Nq, d, splits);
}

struct DecPlan {
    int dtype = 0, d = 0, B = 0, H = 0, Nq = 0, Nk = 0, causal = 0, mask = 0;
    int splits = 0, kps = 0;
    float kscale = 0.f, c = 0.f;
    int qmode = 0;
    size_t ws_bytes = 0;
};

// attn_decode_fwd.  Stops at ATTN_ERR_WORKSPACE only when every other argument
// is valid; ATTN_OK with *empty set when B*H*Nq = 0.
inline int plan_decode(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       int B, int H, int Nq, int Nk, int d, float scale, int causal, const uint8_t* mask,
                       int dtype, const void* workspace, size_t workspace_bytes, int num_splits,
                       DecPlan* p, bool* empty)
{
    *empty = false;
    if (!valid_dtype(dtype)) return fail(ATTN_ERR_DTYPE, "dtype %d is not an attn_dtype", dtype);
    if (dtype == ATTN_F32) return fail(ATTN_ERR_DTYPE, "the decode path takes 16-bit q, k, v");
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return fail(ATTN_ERR_SHAPE, "negative size B=%d H=%d Nq=%d Nk=%d", B, H, Nq, Nk);
    const int64_t nmax = Nq > Nk ? Nq : Nk;
    if ((int64_t)B * H * nmax >= ((int64_t)1 << 31)) return fail(ATTN_ERR_SHAPE, "B*H*max(Nq, Nk) exceeds 2^31 - 1");
    if (d != 64 && d != 128) return fail(ATTN_ERR_HEAD_DIM, "head size d=%d, supported: 64, 128", d);
    if (!std::isfinite(scale)) return fail(ATTN_ERR_SCALE, "scale %g must be finite", (double)scale);
    if (num_splits < 0 || num_splits > 1024) return fail(ATTN_ERR_TILE, "num_splits=%d not in 0..1024", num_splits);
    p->dtype = dtype; p->d = d; p->B = B; p->H = H; p->Nq = Nq; p->Nk = Nk;
    p->causal = causal ? 1 : 0; p->mask = mask ? 1 : 0;
    p->kscale = kernel_scale(scale, &p->qmode);
    p->c = log2e_factor(p->kscale);
    if ((int64_t)B * H * Nq == 0) { *empty = true; return ATTN_OK; }
    if (!q || !o) return fail(ATTN_ERR_NULL, "q and o must be non-NULL");
    if (Nk > 0 && (!k || !v)) return fail(ATTN_ERR_NULL, "k and v must be non-NULL when Nk > 0");
    const void* p16[4] = {q, k, v, o};
    const char* names[4] = {"q", "k", "v", "o"};
    for (int i = 0; i < 4; ++i)
        if ((uintptr_t)p16[i] % 16) return fail(ATTN_ERR_ALIGN, "%s is not 16-byte aligned", names[i]);
    if (lse && ((uintptr_t)lse % 4)) return fail(ATTN_ERR_ALIGN, "lse is not 4-byte aligned");
    const size_t nq = (size_t)B * H * Nq * d * elem_bytes_in(dtype), nkv = (size_t)B * H * Nk * d * elem_bytes_in(dtype);
    const size_t no = (size_t)B * H * Nq * d * elem_bytes_out(dtype), nl = lse ? (size_t)B * H * Nq * 4 : 0;
    if (overlaps(o, no, q, nq) || overlaps(o, no, k, nkv) || overlaps(o, no, v, nkv) || overlaps(o, no, lse, nl))
        return fail(ATTN_ERR_ALIAS, "o overlaps q, k, v or lse");
    if (overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) || overlaps(lse, nl, v, nkv))
        return fail(ATTN_ERR_ALIAS, "lse overlaps q, k or v");
    decode_splits(B, H, Nq, Nk, num_splits, &p->splits, &p->kps);
    if ((int64_t)B * H * p->splits >= ((int64_t)1 << 31) || (Nq + 15) / 16 > 65535)
        return fail(ATTN_ERR_SHAPE, "decode grid too large (B*H*splits = %lld, Nq = %d)", (long long)B * H * p->splits, Nq);
    const size_t need = decode_ws_bytes(B, H, Nq, d, p->splits);
    p->ws_bytes = need;
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % 16))
        return fail(ATTN_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned", need);
    if (overlaps(workspace, need, q, nq) || overlaps(workspace, need, k, nkv) || overlaps(workspace, need, v, nkv) ||
        overlaps(workspace, need, o, no) || overlaps(workspace, need, lse, nl))
        return fail(ATTN_ERR_ALIAS, "workspace overlaps an input or output");
    return ATTN_OK;
}

// ---------------------------------------------------------------- backward
// The dK/dV and dQ kernels of the 16-bit d = 128 gradient without a
// key-padding mask run their full tiles through their software pipelines.
// Those address a head's rows and its lse2 (from its D, in the same
// workspace) with 32-bit byte offsets, which the sizes must allow.
inline bool bwd_pipelined(int d, bool mask, int B, int H, int N)
{
#ifdef ATTN_LDS_POISON
    // the poisoned build checks the C++ loops' copies; the pipelines' waits
    // are checked by bitwise equality with those loops
    (void)d;
    (void)mask;
    (void)B;
    (void)H;
    (void)N;
    return false;
#else
    const uint64_t rows = (uint64_t)B * H * N;
    return d == 128 && !mask && (uint64_t)N * 256u <= 0xffffffffull && 4u * rows + 4u * (uint64_t)N <= 0xffffffffull;
#endif
}

inline size_t bwd_ws_bytes(int B, int H, int N)
{
    if (B <= 0 || H <= 0 || N <= 0) return 0;
    return (size_t)B * H * (size_t)N * 8;
}

inline int check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     const float* dq, const float* dk, const float* dv, int B, int H, int N, int d, float scale,
                     int dtype, const void* workspace, size_t workspace_bytes, bool* empty)
{
    *empty = false;
    if (!valid_dtype(dtype)) return fail(ATTN_ERR_DTYPE, "dtype %d is not an attn_dtype", dtype);
    if (dtype != ATTN_BF16 && dtype != ATTN_F16) return fail(ATTN_ERR_DTYPE, "the backward takes ATTN_BF16 or ATTN_F16");
    int st = check_scalars(B, H, N, d, scale, dtype);
    if (st) return st;
    if ((int64_t)B * H * N == 0) { *empty = true; return ATTN_OK; }
    const void* in[5] = {q, k, v, o, dout};
    const char* nin[5] = {"q", "k", "v", "o", "dout"};
    const void* out[3] = {dq, dk, dv};
    const char* nout[3] = {"dq", "dk", "dv"};
    for (int i = 0; i < 5; ++i) {
        if (!in[i]) return fail(ATTN_ERR_NULL, "%s must be non-NULL", nin[i]);
        if ((uintptr_t)in[i] % 16) return fail(ATTN_ERR_ALIGN, "%s is not 16-byte aligned", nin[i]);
    }
    for (int i = 0; i < 3; ++i) {
        if (!out[i]) return fail(ATTN_ERR_NULL, "%s must be non-NULL", nout[i]);
        if ((uintptr_t)out[i] % 16) return fail(ATTN_ERR_ALIGN, "%s is not 16-byte aligned", nout[i]);
    }
    if (!lse) return fail(ATTN_ERR_NULL, "lse must be non-NULL");
    if ((uintptr_t)lse % 4) return fail(ATTN_ERR_ALIGN, "lse is not 4-byte aligned");
    const size_t rows = (size_t)B * H * N;
    const size_t nt = rows * d * 2, nf = rows * d * 4, nl = rows * 4;
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 5; ++j)
            if (overlaps(out[i], nf, in[j], nt)) return fail(ATTN_ERR_ALIAS, "%s overlaps %s", nout[i], nin[j]);
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(out[i], nf, out[j], nf)) return fail(ATTN_ERR_ALIAS, "%s overlaps %s", nout[i], nout[j]);
        if (overlaps(out[i], nf, lse, nl)) return fail(ATTN_ERR_ALIAS, "%s overlaps lse", nout[i]);
    }
    const size_t need = bwd_ws_bytes(B, H, N);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % 16))
        return fail(ATTN_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned", need);
    for (int j = 0; j < 5; ++j)
        if (overlaps(workspace, need, in[j], nt)) return fail(ATTN_ERR_ALIAS, "workspace overlaps %s", nin[j]);
    for (int i = 0; i < 3; ++i)
        if (overlaps(workspace, need, out[i], nf)) return fail(ATTN_ERR_ALIAS, "workspace overlaps %s", nout[i]);
    if (overlaps(workspace, need, lse, nl)) return fail(ATTN_ERR_ALIAS, "workspace overlaps lse");
    return ATTN_OK;
}

// ---------------------------------------------------------------- ATTN_TRACE
// With ATTN_TRACE set to anything but "" or "0" when the library first checks
// it, every entry point writes one line to stderr: the plan it launched, or
// the status it returned without launching.  Lines start with "attn: ".
inline bool trace_on()
{
    static const bool on = [] {
        const char* e = std::getenv("ATTN_TRACE");
        return e && *e && std::strcmp(e, "0") != 0;
    }();
    return on;
}

inline const char* status_name(int st)
{
    switch (st) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE";
    case ATTN_ERR_HEAD_DIM: return "ATTN_ERR_HEAD_DIM";
    case ATTN_ERR_DTYPE: return "ATTN_ERR_DTYPE";
    case ATTN_ERR_ALIGN: return "ATTN_ERR_ALIGN";
    case ATTN_ERR_TILE: return "ATTN_ERR_TILE";
    case ATTN_ERR_SCALE: return "ATTN_ERR_SCALE";
    case ATTN_ERR_ALIAS: return "ATTN_ERR_ALIAS";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    default: return "?";
    }
}

inline int trace_fwd_line(char* buf, size_t n, const char* entry, const FwdPlan& p)
{
    return snprintf(buf, n,
                    "attn: %s kernel=%s<%s,d%d,%dx%d> B=%d H=%d N=%d causal=%d mask=%d sparse_block=%d "
                    "order=%d slack=%d loop=%s grid=%lld block=%d persistent=%d xcd_affine=%d qmode=%d "
                    "scale=%.9g\n",
                    entry, fwd_kernel_name(p), dtype_name(p.dtype), p.d, p.br, p.bc, p.B, p.H, p.N, p.causal,
                    p.mask, p.sparse ? p.block : 0, p.order, p.slack, fwd_pipelined(p) ? "pipelined" : "generic",
                    (long long)fwd_grid(p), fwd_block_threads(p), p.persist > 0 ? 1 : 0, p.xcd_affine, p.qmode,
                    (double)p.kscale);
}

inline int trace_decode_line(char* buf, size_t n, const char* entry, const DecPlan& p, bool scratch)
{
    return snprintf(buf, n,
                    "attn: %s kernel=dec_split+dec_merge<%s,d%d> B=%d H=%d Nq=%d Nk=%d causal=%d mask=%d "
                    "splits=%d keys_per_split=%d grid=%lldx%d workspace=%zu%s qmode=%d scale=%.9g\n",
                    entry, dtype_name(p.dtype), p.d, p.B, p.H, p.Nq, p.Nk, p.causal, p.mask, p.splits, p.kps,
                    (long long)p.B * p.H * p.splits, (p.Nq + 15) / 16, p.ws_bytes,
                    scratch ? " (library scratch)" : "", p.qmode, (double)p.kscale);
}

inline int trace_plain_line(char* buf, size_t n, const char* entry, const char* kernels, int dtype, int B, int H,
                            int N, int d, int causal, int mask, size_t ws, const char* tail = "")
{
    return snprintf(buf, n, "attn: %s kernel=%s<%s,d%d> B=%d H=%d N=%d causal=%d mask=%d workspace=%zu%s\n", entry,
                    kernels, dtype_name(dtype), d, B, H, N, causal ? 1 : 0, mask, ws, tail);
}

inline int trace_status_line(char* buf, size_t n, const char* entry, int st)
{
    if (st == ATTN_OK) return snprintf(buf, n, "attn: %s nothing to launch (empty)\n", entry);
    return snprintf(buf, n, "attn: %s returned %s: %s\n", entry, status_name(st), g_err);
}

inline void trace_emit(const char* line)
{
    std::fputs(line, stderr);
    std::fflush(stderr);
}

}  // namespace attnh
