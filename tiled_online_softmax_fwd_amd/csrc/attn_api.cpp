// attn_api.cpp -- host side of the C ABI declared in include/attn.h:
// argument checks (host only, before any HIP call), tile selection, dispatch
// to the kernel instance tables, and error reporting.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "attn.h"
#include "bwd.h"
#include "decode.h"
#include "fwd_kernel.h"
#include "naive_kernel.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int ok()
{
    g_err[0] = '\0';
    return ATTN_OK;
}

size_t elem_bytes_in(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }
size_t elem_bytes_out(int dtype) { return (dtype == ATTN_F32 || dtype == ATTN_F16_OUT_F32 || dtype == ATTN_BF16_OUT_F32) ? 4 : 2; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

bool valid_tile(int t) { return t == 16 || t == 32 || t == 64 || t == 128; }
bool valid_br(int t) { return valid_tile(t) || t == 256; }

// Defaults per input type and head size (measured on MI355X): 16-bit inputs
// at d = 128 use 256 query rows per workgroup (eight waves of 32 rows sharing
// each K/V tile) and 64 keys per tile; at d = 64 the state is half as large and
// 128 x 128 tiles run best (three workgroups per compute unit); fp32 uses
// 128 x 64 (its tiles are twice as large in LDS).
void defaults(int dtype, int d, int causal, int* br, int* bc)
{
    (void)causal;
    if (dtype == ATTN_F32) { *br = 128; *bc = 64; }
    else if (d == 64) { *br = 128; *bc = 128; }
    else { *br = 256; *bc = 64; }
}

// Compute units of the current device, queried once per device.
int cu_count()
{
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cache[dev] > 0) return cache[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
    return n;
}

// Persistent grid of the 16-bit d = 128 forward with 256 x 64 tiles (the one
// instance that has it): one workgroup per compute unit when the items (query
// tiles, or causal pairs of query tiles of equal cost) split evenly over the
// compute units; the items of a head then stay on one XCD when both the head
// count and the grid are multiples of the 8 XCDs.  Otherwise one workgroup per
// query tile (the hardware's dynamic dispatch balances uneven work better).
void persistent_grid(attnk::FwdParams& p, int dtype, int d, int br, int bc)
{
    p.persist = 0;
    p.xcd_affine = 0;
    if (dtype == ATTN_F32 || d != 128 || br != 256 || bc != 64 || p.mask || !p.pipe || p.kv_order || p.slack != 0.f)
        return;
    const int G = cu_count();
    const int64_t BH = (int64_t)p.B * p.H;
    const int64_t iph = p.causal ? (p.n_qt + 1) / 2 : p.n_qt;
    const int64_t items = BH * iph;
    if (G <= 0 || items < G || items % G != 0) return;
    p.persist = G;
    p.xcd_affine = (BH % 8 == 0 && G % 8 == 0) ? 1 : 0;
}

attnk::LaunchFn find(int dtype, int d, int br, int bc)
{
    switch (dtype) {
    case ATTN_F32: return attnk::lookup_f32(d, br, bc);
    case ATTN_F16: case ATTN_F16_OUT_F32: return attnk::lookup_f16(d, br, bc);
    case ATTN_BF16: case ATTN_BF16_OUT_F32: return attnk::lookup_bf16(d, br, bc);
    default: return nullptr;
    }
}

// Everything that does not involve a pointer.
int check_scalars(int B, int H, int N, int d, float scale, int dtype)
{
    if (dtype < ATTN_F32 || dtype > ATTN_BF16_OUT_F32) return fail(ATTN_ERR_DTYPE, "dtype %d is not an attn_dtype", dtype);
    if (B < 0 || H < 0 || N < 0) return fail(ATTN_ERR_SHAPE, "negative size B=%d H=%d N=%d", B, H, N);
    if ((int64_t)B * H * N >= ((int64_t)1 << 31))
        return fail(ATTN_ERR_SHAPE, "B*H*N = %lld rows exceeds 2^31 - 1", (long long)B * H * N);
    if (d != 64 && d != 128) return fail(ATTN_ERR_HEAD_DIM, "head size d=%d, supported: 64, 128", d);
    if (!std::isfinite(scale)) return fail(ATTN_ERR_SCALE, "scale %g must be finite", (double)scale);
    return ATTN_OK;
}

// Kernels that keep a running maximum of raw scores take a positive factor:
// scale < 0 runs as |scale| on negated Q, scale = 0 as 1 on Q = 0 (q_mode16 in
// fwd_kernel.h).  Returns the factor the kernels use and sets the Q mode.
float kernel_scale(float scale, int* qmode)
{
    if (scale > 0.f) { *qmode = 0; return scale; }
    if (scale < 0.f) { *qmode = 1; return -scale; }
    *qmode = 2;
    return 1.f;
}

int check_pointers(const void* q, const void* k, const void* v, void* o, float* lse,
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

int resolve_opts(int dtype, int d, int causal, const attn_opts* opts, int* br, int* bc, int* order, int* slack,
                 int* generic = nullptr)
{
    defaults(dtype, d, causal, br, bc);
    *order = 0;
    *slack = 0;
    if (generic) *generic = 0;
    if (!opts) return ATTN_OK;
    if (generic) *generic = opts->generic_loop != 0;
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
        if (opts->br == 0 && !find(dtype, d, *br, *bc)) *br = 128;
    }
    if (opts->kv_order != 0 && opts->kv_order != 1) return fail(ATTN_ERR_TILE, "kv_order=%d not 0 or 1", opts->kv_order);
    *order = opts->kv_order;
    if (opts->ref_slack < 0 || opts->ref_slack > 15) return fail(ATTN_ERR_TILE, "ref_slack=%d not in 0..15", opts->ref_slack);
    *slack = opts->ref_slack;
    return ATTN_OK;
}

int check_all(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int N, int d, float scale, int causal, int dtype,
              const attn_opts* opts, int* br, int* bc, int* order, int* slack, int* generic = nullptr)
{
    int st = check_scalars(B, H, N, d, scale, dtype);
    if (st) return st;
    st = resolve_opts(dtype, d, causal, opts, br, bc, order, slack, generic);
    if (st) return st;
    if (!find(dtype, d, *br, *bc))
        return fail(ATTN_ERR_TILE, "no kernel for dtype %d, d=%d, br=%d, bc=%d", dtype, d, *br, *bc);
    if ((int64_t)B * H * N == 0) return ATTN_OK;
    return check_pointers(q, k, v, o, lse, B, H, N, d, dtype);
}

// Key chunks of the decode path (whole 32-key tiles).  With units = B*H*ceil(Nq/16)
// row blocks, the library aims at about 1024 one-wave workgroups but takes
// fewer, down to about 512, where that keeps chunks at 1024 keys or more, and
// never makes chunks shorter than 256 keys.  Measured with the non-temporal tile
// copies (TB/s of the best split counts in brackets):
//   B8 H32 Nk 8192, Nq 1 or 16, d 64 or 128: 4 chunks (1024 workgroups) [6.2-6.4];
//   B1 H32 Nk 65536: 32 chunks (1024) [6.1]; B2 H8 Nk 32768: 32 chunks of 1024
//   keys (512) [4.7, against 4.3 for 64 chunks]; B1 H8 Nk 16384: 64 chunks of 256
//   keys (512) [2.0, against 1.3 for 16 chunks of 1024].
void decode_splits(int B, int H, int Nq, int Nk, int num_splits, int* splits, int* kps)
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

size_t decode_ws_bytes(int B, int H, int Nq, int d, int splits)
{
    const size_t parts = (size_t)B * H * (size_t)splits * (size_t)Nq;
    return parts * (size_t)d * 4 + parts * 4;
}

}  // namespace

extern "C" {

int attn_check_args(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal,
                    const uint8_t* key_padding_mask, int dtype, const attn_opts* opts)
{
    (void)key_padding_mask;
    int br, bc, order, slack;
    const int st = check_all(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, opts, &br, &bc, &order, &slack);
    return st ? st : ok();
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int N, int d, float scale, int causal,
                const uint8_t* key_padding_mask, int dtype, void* stream,
                const attn_opts* opts)
{
    int br, bc, order, slack, generic;
    const int st = check_all(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, opts, &br, &bc, &order, &slack,
                             &generic);
    if (st) return st;
    if ((int64_t)B * H * N == 0) return ok();

    attnk::FwdParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse; p.mask = key_padding_mask;
    p.B = B; p.H = H; p.N = N;
    p.n_qt = (N + br - 1) / br;
    p.scale = kernel_scale(scale, &p.qmode);
    p.c = (float)((double)p.scale * 1.4426950408889634);   // scale * log2(e), rounded once
    p.causal = causal ? 1 : 0;
    p.kv_order = order;
    p.slack = (float)slack;
    p.pipe = generic ? 0 : 1;
    p.out_f32 = (dtype == ATTN_F16_OUT_F32 || dtype == ATTN_BF16_OUT_F32) ? 1 : 0;
    p.bmask = nullptr;
    p.blk = 0;
    p.nb = 0;
    persistent_grid(p, dtype, d, br, bc);
    const hipError_t e = find(dtype, d, br, bc)(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

int attn_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal,
                    const uint8_t* key_padding_mask, const uint8_t* block_mask, int block,
                    int dtype, void* stream, const attn_opts* opts)
{
    int st = check_scalars(B, H, N, d, scale, dtype);
    if (st) return st;
    if (dtype == ATTN_F32) return fail(ATTN_ERR_DTYPE, "block-sparse forward: 16-bit inputs only");
    if (block < 32 || block % 32 != 0) return fail(ATTN_ERR_SHAPE, "block=%d must be a positive multiple of 32", block);
    int br, bc, order, slack;
    st = resolve_opts(dtype, d, causal, opts, &br, &bc, &order, &slack);
    if (st) return st;
    if (order != 0) return fail(ATTN_ERR_TILE, "block-sparse forward: kv_order must be 0");
    // default 128 x 64: with blocks of 64 rows, wider workgroups visit tiles
    // where only some of their row blocks attend (measured on MI355X at
    // B1 H32 N8192, d = 64 and 128, random and sliding-window flags)
    if (!opts || opts->br == 0) br = 128;
    if (!opts || opts->bc == 0) bc = 64;
    const int bits = (dtype == ATTN_F16 || dtype == ATTN_F16_OUT_F32) ? 1 : 0;
    const attnk::LaunchFn fn = attnk::lookup_sparse(bits, d, br, bc);
    if (!fn) return fail(ATTN_ERR_TILE, "no block-sparse kernel for d=%d, br=%d, bc=%d", d, br, bc);
    if ((int64_t)B * H * N == 0) return ok();
    st = check_pointers(q, k, v, o, lse, B, H, N, d, dtype);
    if (st) return st;
    if (!block_mask) return fail(ATTN_ERR_NULL, "block_mask must be non-NULL");
    const int nb = (N + block - 1) / block;
    const size_t nbm = (size_t)B * H * (size_t)nb * (size_t)nb;
    const size_t nout = (size_t)B * H * N * d * elem_bytes_out(dtype);
    if (overlaps(o, nout, block_mask, nbm) || overlaps(lse, lse ? (size_t)B * H * N * 4 : 0, block_mask, nbm))
        return fail(ATTN_ERR_ALIAS, "o or lse overlaps block_mask");

    attnk::FwdParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse; p.mask = key_padding_mask;
    p.B = B; p.H = H; p.N = N;
    p.n_qt = (N + br - 1) / br;
    p.scale = kernel_scale(scale, &p.qmode);
    p.c = (float)((double)p.scale * 1.4426950408889634);
    p.causal = causal ? 1 : 0;
    p.kv_order = 0;
    p.slack = (float)slack;
    p.pipe = 0;
    p.persist = 0;
    p.xcd_affine = 0;
    p.out_f32 = (dtype == ATTN_F16_OUT_F32 || dtype == ATTN_BF16_OUT_F32) ? 1 : 0;
    p.bmask = block_mask;
    p.blk = block;
    p.nb = nb;
    const hipError_t e = fn(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d, float scale, int causal,
             const uint8_t* key_padding_mask, int dtype, void* stream)
{
    return attn_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask, dtype, stream, nullptr);
}

int attn_default_tiles(int dtype, int d, int causal, int* br, int* bc)
{
    if (dtype < ATTN_F32 || dtype > ATTN_BF16_OUT_F32) return fail(ATTN_ERR_DTYPE, "dtype %d is not an attn_dtype", dtype);
    if (d != 64 && d != 128) return fail(ATTN_ERR_HEAD_DIM, "head size d=%d, supported: 64, 128", d);
    if (!br || !bc) return fail(ATTN_ERR_NULL, "br and bc must be non-NULL");
    defaults(dtype, d, causal, br, bc);
    return ok();
}

size_t attn_naive_workspace_bytes(int B, int H, int N, int dtype)
{
    if (B <= 0 || H <= 0 || N <= 0 || dtype < ATTN_F32 || dtype > ATTN_BF16_OUT_F32) return 0;
    return (size_t)B * H * (size_t)N * (size_t)N * elem_bytes_in(dtype);
}

int attn_naive_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* key_padding_mask, int dtype, void* stream,
                   void* workspace, size_t workspace_bytes)
{
    int st = check_scalars(B, H, N, d, scale, dtype);
    if (st) return st;
    if ((int64_t)B * H * N == 0) return ok();
    st = check_pointers(q, k, v, o, lse, B, H, N, d, dtype);
    if (st) return st;
    const size_t need = attn_naive_workspace_bytes(B, H, N, dtype);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % 16))
        return fail(ATTN_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned", need);
    const size_t nws = need;
    const size_t rows = (size_t)B * H * N;
    if (overlaps(workspace, nws, q, rows * d * elem_bytes_in(dtype)) || overlaps(workspace, nws, k, rows * d * elem_bytes_in(dtype)) ||
        overlaps(workspace, nws, v, rows * d * elem_bytes_in(dtype)) || overlaps(workspace, nws, o, rows * d * elem_bytes_out(dtype)) ||
        overlaps(workspace, nws, lse, lse ? rows * 4 : 0))
        return fail(ATTN_ERR_ALIAS, "workspace overlaps an input or output");
    attnk::NaiveParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse; p.mask = key_padding_mask; p.ws = workspace;
    p.B = B; p.H = H; p.N = N; p.d = d;
    p.scale = scale;
    p.causal = causal ? 1 : 0;
    p.in_kind = dtype == ATTN_F32 ? 0 : ((dtype == ATTN_F16 || dtype == ATTN_F16_OUT_F32) ? 1 : 2);
    p.out_f32 = elem_bytes_out(dtype) == 4 ? 1 : 0;
    const hipError_t e = attnk::naive_launch(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "naive launch: %s", hipGetErrorString(e));
    return ok();
}

size_t attn_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits)
{
    if (B <= 0 || H <= 0 || Nq <= 0 || Nk < 0 || (d != 64 && d != 128) || num_splits < 0 || num_splits > 1024) return 0;
    int splits, kps;
    decode_splits(B, H, Nq, Nk, num_splits, &splits, &kps);
    return decode_ws_bytes(B, H, Nq, d, splits);
}

int attn_decode_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Nq, int Nk, int d, float scale, int causal,
                    const uint8_t* key_padding_mask, int dtype, void* stream,
                    void* workspace, size_t workspace_bytes, int num_splits)
{
    if (dtype < ATTN_F32 || dtype > ATTN_BF16_OUT_F32) return fail(ATTN_ERR_DTYPE, "dtype %d is not an attn_dtype", dtype);
    if (dtype == ATTN_F32) return fail(ATTN_ERR_DTYPE, "the decode path takes 16-bit q, k, v");
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return fail(ATTN_ERR_SHAPE, "negative size B=%d H=%d Nq=%d Nk=%d", B, H, Nq, Nk);
    const int64_t nmax = Nq > Nk ? Nq : Nk;
    if ((int64_t)B * H * nmax >= ((int64_t)1 << 31)) return fail(ATTN_ERR_SHAPE, "B*H*max(Nq, Nk) exceeds 2^31 - 1");
    if (d != 64 && d != 128) return fail(ATTN_ERR_HEAD_DIM, "head size d=%d, supported: 64, 128", d);
    if (!std::isfinite(scale)) return fail(ATTN_ERR_SCALE, "scale %g must be finite", (double)scale);
    if (num_splits < 0 || num_splits > 1024) return fail(ATTN_ERR_TILE, "num_splits=%d not in 0..1024", num_splits);
    if ((int64_t)B * H * Nq == 0) return ok();
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
    int splits, kps;
    decode_splits(B, H, Nq, Nk, num_splits, &splits, &kps);
    if ((int64_t)B * H * splits >= ((int64_t)1 << 31) || (Nq + 15) / 16 > 65535)
        return fail(ATTN_ERR_SHAPE, "decode grid too large (B*H*splits = %lld, Nq = %d)", (long long)B * H * splits, Nq);
    const size_t need = decode_ws_bytes(B, H, Nq, d, splits);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % 16))
        return fail(ATTN_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned", need);
    if (overlaps(workspace, need, q, nq) || overlaps(workspace, need, k, nkv) || overlaps(workspace, need, v, nkv) ||
        overlaps(workspace, need, o, no) || overlaps(workspace, need, lse, nl))
        return fail(ATTN_ERR_ALIAS, "workspace overlaps an input or output");

    attnk::DecParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse; p.mask = key_padding_mask;
    p.part_o = (float*)workspace;
    p.part_lse = (float*)workspace + (size_t)B * H * splits * (size_t)Nq * d;
    p.B = B; p.H = H; p.Nq = Nq; p.Nk = Nk;
    p.splits = splits; p.keys_per_split = kps;
    p.scale = kernel_scale(scale, &p.qmode);
    p.c = (float)((double)p.scale * 1.4426950408889634);
    p.slack = 0.f;
    p.causal = causal ? 1 : 0;
    p.out_f32 = elem_bytes_out(dtype) == 4 ? 1 : 0;
    const int bits = (dtype == ATTN_BF16 || dtype == ATTN_BF16_OUT_F32) ? 0 : 1;
    const hipError_t e = attnk::lookup_decode(bits, d)(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return ok();
}

int attn_decode_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Nq, int Nk, int d, float scale, int causal,
                            const uint8_t* key_padding_mask, int dtype, void* stream, int num_splits)
{
    // Same checks and kernels as attn_decode_fwd; the partial results go to the
    // library's fixed device array instead of a caller workspace.  Every host
    // check runs first: without a workspace attn_decode_fwd stops at
    // ATTN_ERR_WORKSPACE only when every other argument is valid (and returns
    // ATTN_OK for empty sizes), before any HIP call.
    const int st = attn_decode_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, key_padding_mask, dtype,
                                   stream, nullptr, 0, num_splits);
    if (st != ATTN_ERR_WORKSPACE) return st;
    const size_t need = attn_decode_workspace_bytes(B, H, Nq, Nk, d, num_splits);
    if (need > attnk::DECODE_SCRATCH_BYTES)
        return fail(ATTN_ERR_WORKSPACE, "decode without allocation: %zu bytes of partial results exceed the "
                    "library's %zu-byte scratch (fewer rows or key splits needed)", need, attnk::DECODE_SCRATCH_BYTES);
    void* ws = nullptr;
    const hipError_t e = attnk::decode_scratch(&ws);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "decode scratch lookup: %s", hipGetErrorString(e));
    return attn_decode_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, key_padding_mask, dtype, stream,
                           ws, attnk::DECODE_SCRATCH_BYTES, num_splits);
}

size_t attn_bwd_workspace_bytes(int B, int H, int N)
{
    if (B <= 0 || H <= 0 || N <= 0) return 0;
    return (size_t)B * H * (size_t)N * 8;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             float* dq, float* dk, float* dv, int B, int H, int N, int d, float scale, int causal,
             const uint8_t* key_padding_mask, int dtype, void* stream, void* workspace, size_t workspace_bytes)
{
    if (dtype < ATTN_F32 || dtype > ATTN_BF16_OUT_F32) return fail(ATTN_ERR_DTYPE, "dtype %d is not an attn_dtype", dtype);
    if (dtype != ATTN_BF16 && dtype != ATTN_F16) return fail(ATTN_ERR_DTYPE, "the backward takes ATTN_BF16 or ATTN_F16");
    int st = check_scalars(B, H, N, d, scale, dtype);
    if (st) return st;
    if ((int64_t)B * H * N == 0) return ok();
    const void* in[5] = {q, k, v, o, dout};
    const char* nin[5] = {"q", "k", "v", "o", "dout"};
    void* out[3] = {dq, dk, dv};
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
    const size_t need = attn_bwd_workspace_bytes(B, H, N);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % 16))
        return fail(ATTN_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned", need);
    for (int j = 0; j < 5; ++j)
        if (overlaps(workspace, need, in[j], nt)) return fail(ATTN_ERR_ALIAS, "workspace overlaps %s", nin[j]);
    for (int i = 0; i < 3; ++i)
        if (overlaps(workspace, need, out[i], nf)) return fail(ATTN_ERR_ALIAS, "workspace overlaps %s", nout[i]);
    if (overlaps(workspace, need, lse, nl)) return fail(ATTN_ERR_ALIAS, "workspace overlaps lse");

    attnk::BwdParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
    p.dq = dq; p.dk = dk; p.dv = dv; p.mask = key_padding_mask;
    p.dsum = (float*)workspace;
    p.lse2 = (float*)workspace + rows;
    p.B = B; p.H = H; p.N = N;
    // the gradient forms P = exp(scale q.k - lse) and multiplies by scale at the
    // end: any finite scale as given
    p.scale = scale;
    p.c = (float)((double)scale * 1.4426950408889634);
    p.causal = causal ? 1 : 0;
    const hipError_t e = attnk::lookup_bwd(dtype == ATTN_BF16 ? 0 : 1, d)(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
    return ok();
}

const char* attn_status_string(int status)
{
    switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer";
    case ATTN_ERR_SHAPE: return "bad shape";
    case ATTN_ERR_HEAD_DIM: return "unsupported head size";
    case ATTN_ERR_DTYPE: return "unknown dtype";
    case ATTN_ERR_ALIGN: return "misaligned pointer";
    case ATTN_ERR_TILE: return "unsupported tile or order";
    case ATTN_ERR_SCALE: return "bad scale";
    case ATTN_ERR_ALIAS: return "output overlaps an input";
    case ATTN_ERR_HIP: return "HIP runtime error";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
    }
}

const char* attn_last_error(void) { return g_err; }

int attn_version(void) { return 100; }

}  // extern "C"
