// attn_api.cpp -- the C ABI declared in include/attn.h: host checks and
// planning (attn_host.h, before any HIP call), the compute-unit count, lookup
// in the kernel instance tables, launch, and error reporting.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "attn.h"
#include "attn_host.h"
#include "bwd.h"
#include "decode.h"
#include "fwd_kernel.h"
#include "naive_kernel.h"

namespace {

using attnh::fail;
using attnh::ok;

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

attnk::LaunchFn find(int dtype, int d, int br, int bc)
{
    switch (dtype) {
    case ATTN_F32: return attnk::lookup_f32(d, br, bc);
    case ATTN_F16: case ATTN_F16_OUT_F32: return attnk::lookup_f16(d, br, bc);
    case ATTN_BF16: case ATTN_BF16_OUT_F32: return attnk::lookup_bf16(d, br, bc);
    default: return nullptr;
    }
}

// Status of a call that launches nothing (rejected, or empty), traced.
int done(const char* entry, int st)
{
    if (attnh::trace_on()) {
        char line[768];
        attnh::trace_status_line(line, sizeof(line), entry, st);
        attnh::trace_emit(line);
    }
    return st == ATTN_OK ? ok() : st;
}

attnk::FwdParams fwd_params(const attnh::FwdPlan& pl, const void* q, const void* k, const void* v, void* o,
                            float* lse, const uint8_t* mask)
{
    attnk::FwdParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse; p.mask = mask;
    p.B = pl.B; p.H = pl.H; p.N = pl.N;
    p.n_qt = pl.n_qt;
    p.scale = pl.kscale;
    p.c = pl.c;
    p.qmode = pl.qmode;
    p.causal = pl.causal;
    p.kv_order = pl.order;
    p.slack = (float)pl.slack;
    p.pipe = attnh::fwd_pipelined(pl) ? 1 : 0;
    p.persist = pl.persist;
    p.xcd_affine = pl.xcd_affine;
    p.out_f32 = attnh::elem_bytes_out(pl.dtype) == 4 ? 1 : 0;
    p.bmask = nullptr;
    p.blk = 0;
    p.nb = 0;
    return p;
}

int launch_fwd(const char* entry, const attnh::FwdPlan& pl, attnk::LaunchFn fn, const attnk::FwdParams& p,
               void* stream)
{
    if (!fn) return fail(ATTN_ERR_TILE, "no kernel instance for dtype %d, d=%d, br=%d, bc=%d", pl.dtype, pl.d, pl.br, pl.bc);
    if (attnh::trace_on()) {
        char line[768];
        attnh::trace_fwd_line(line, sizeof(line), entry, pl);
        attnh::trace_emit(line);
    }
    const hipError_t e = fn(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int attn_check_args(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal,
                    const uint8_t* key_padding_mask, int dtype, const attn_opts* opts)
{
    attnh::FwdPlan pl;
    bool empty;
    const int st = attnh::plan_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask, dtype, opts,
                                   &pl, &empty);
    return st ? st : ok();
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int N, int d, float scale, int causal,
                const uint8_t* key_padding_mask, int dtype, void* stream,
                const attn_opts* opts)
{
    attnh::FwdPlan pl;
    bool empty;
    const int st = attnh::plan_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask, dtype, opts,
                                   &pl, &empty);
    if (st || empty) return done("attn_fwd", st);
    attnh::plan_persistent(pl, cu_count());
    return launch_fwd("attn_fwd", pl, find(dtype, d, pl.br, pl.bc), fwd_params(pl, q, k, v, o, lse, key_padding_mask),
                      stream);
}

int attn_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal,
                    const uint8_t* key_padding_mask, const uint8_t* block_mask, int block,
                    int dtype, void* stream, const attn_opts* opts)
{
    attnh::FwdPlan pl;
    bool empty;
    const int st = attnh::plan_sparse(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask, block_mask,
                                      block, dtype, opts, &pl, &empty);
    if (st || empty) return done("attn_fwd_sparse", st);
    attnk::FwdParams p = fwd_params(pl, q, k, v, o, lse, key_padding_mask);
    p.bmask = block_mask;
    p.blk = block;
    p.nb = (N + block - 1) / block;
    return launch_fwd("attn_fwd_sparse", pl, attnk::lookup_sparse(attnh::is_f16(dtype) ? 1 : 0, d, pl.br, pl.bc), p,
                      stream);
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d, float scale, int causal,
             const uint8_t* key_padding_mask, int dtype, void* stream)
{
    return attn_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask, dtype, stream, nullptr);
}

int attn_default_tiles(int dtype, int d, int causal, int* br, int* bc)
{
    if (!attnh::valid_dtype(dtype)) return fail(ATTN_ERR_DTYPE, "dtype %d is not an attn_dtype", dtype);
    if (d != 64 && d != 128) return fail(ATTN_ERR_HEAD_DIM, "head size d=%d, supported: 64, 128", d);
    if (!br || !bc) return fail(ATTN_ERR_NULL, "br and bc must be non-NULL");
    attnh::defaults(dtype, d, causal, br, bc);
    return ok();
}

size_t attn_naive_workspace_bytes(int B, int H, int N, int dtype)
{
    return attnh::naive_ws_bytes(B, H, N, dtype);
}

int attn_naive_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* key_padding_mask, int dtype, void* stream,
                   void* workspace, size_t workspace_bytes)
{
    bool empty;
    const int st = attnh::check_naive(q, k, v, o, lse, B, H, N, d, scale, dtype, workspace, workspace_bytes, &empty);
    if (st || empty) return done("attn_naive_fwd", st);
    attnk::NaiveParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse; p.mask = key_padding_mask; p.ws = workspace;
    p.B = B; p.H = H; p.N = N; p.d = d;
    p.scale = scale;
    p.causal = causal ? 1 : 0;
    p.in_kind = dtype == ATTN_F32 ? 0 : (attnh::is_f16(dtype) ? 1 : 2);
    p.out_f32 = attnh::elem_bytes_out(dtype) == 4 ? 1 : 0;
    if (attnh::trace_on()) {
        char line[768];
        attnh::trace_plain_line(line, sizeof(line), "attn_naive_fwd", "gemm_simt+row_softmax+gemm_simt", dtype, B, H,
                                N, d, causal, key_padding_mask ? 1 : 0, attnh::naive_ws_bytes(B, H, N, dtype));
        attnh::trace_emit(line);
    }
    const hipError_t e = attnk::naive_launch(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "naive launch: %s", hipGetErrorString(e));
    return ok();
}

size_t attn_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits)
{
    return attnh::decode_ws_query(B, H, Nq, Nk, d, num_splits);
}

namespace {

int decode_run(const char* entry, const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Nq, int Nk, int d, float scale, int causal, const uint8_t* key_padding_mask,
               int dtype, void* stream, void* workspace, size_t workspace_bytes, int num_splits, bool scratch)
{
    attnh::DecPlan pl;
    bool empty;
    const int st = attnh::plan_decode(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, key_padding_mask, dtype,
                                      workspace, workspace_bytes, num_splits, &pl, &empty);
    if (st || empty) return done(entry, st);
    attnk::DecParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse; p.mask = key_padding_mask;
    p.part_o = (float*)workspace;
    p.part_lse = (float*)workspace + (size_t)B * H * pl.splits * (size_t)Nq * d;
    p.B = B; p.H = H; p.Nq = Nq; p.Nk = Nk;
    p.splits = pl.splits; p.keys_per_split = pl.kps;
    p.scale = pl.kscale;
    p.c = pl.c;
    p.qmode = pl.qmode;
    p.slack = 0.f;
    p.causal = pl.causal;
    p.out_f32 = attnh::elem_bytes_out(dtype) == 4 ? 1 : 0;
    if (attnh::trace_on()) {
        char line[768];
        attnh::trace_decode_line(line, sizeof(line), entry, pl, scratch);
        attnh::trace_emit(line);
    }
    const hipError_t e = attnk::lookup_decode(attnh::is_f16(dtype) ? 1 : 0, d)(p, (hipStream_t)stream);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

int attn_decode_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Nq, int Nk, int d, float scale, int causal,
                    const uint8_t* key_padding_mask, int dtype, void* stream,
                    void* workspace, size_t workspace_bytes, int num_splits)
{
    return decode_run("attn_decode_fwd", q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, key_padding_mask, dtype,
                      stream, workspace, workspace_bytes, num_splits, false);
}

int attn_decode_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Nq, int Nk, int d, float scale, int causal,
                            const uint8_t* key_padding_mask, int dtype, void* stream, int num_splits)
{
    // Same checks and kernels as attn_decode_fwd; the partial results go to the
    // library's fixed device array instead of a caller workspace.  Every host
    // check runs first: without a workspace the plan stops at
    // ATTN_ERR_WORKSPACE only when every other argument is valid (and returns
    // ATTN_OK for empty sizes), before any HIP call.
    attnh::DecPlan pl;
    bool empty;
    const int st = attnh::plan_decode(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, key_padding_mask, dtype,
                                      nullptr, 0, num_splits, &pl, &empty);
    if (st != ATTN_ERR_WORKSPACE) return done("attn_decode_fwd_noalloc", st);
    if (pl.ws_bytes > attnk::DECODE_SCRATCH_BYTES)
        return done("attn_decode_fwd_noalloc",
                    fail(ATTN_ERR_WORKSPACE, "decode without allocation: %zu bytes of partial results exceed the "
                         "library's %zu-byte scratch (fewer rows or key splits needed)", pl.ws_bytes,
                         attnk::DECODE_SCRATCH_BYTES));
    void* ws = nullptr;
    const hipError_t e = attnk::decode_scratch(&ws);
    if (e != hipSuccess) return fail(ATTN_ERR_HIP, "decode scratch lookup: %s", hipGetErrorString(e));
    return decode_run("attn_decode_fwd_noalloc", q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, key_padding_mask,
                      dtype, stream, ws, attnk::DECODE_SCRATCH_BYTES, num_splits, true);
}

size_t attn_bwd_workspace_bytes(int B, int H, int N)
{
    return attnh::bwd_ws_bytes(B, H, N);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             float* dq, float* dk, float* dv, int B, int H, int N, int d, float scale, int causal,
             const uint8_t* key_padding_mask, int dtype, void* stream, void* workspace, size_t workspace_bytes)
{
    bool empty;
    const int st = attnh::check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, dtype, workspace,
                                    workspace_bytes, &empty);
    if (st || empty) return done("attn_bwd", st);
    attnk::BwdParams p;
    p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
    p.dq = dq; p.dk = dk; p.dv = dv; p.mask = key_padding_mask;
    p.dsum = (float*)workspace;
    p.lse2 = (float*)workspace + (size_t)B * H * N;
    p.B = B; p.H = H; p.N = N;
    // the gradient forms P = exp(scale q.k - lse) and multiplies by scale at the
    // end: any finite scale as given
    p.scale = scale;
    p.c = attnh::log2e_factor(scale);
    p.causal = causal ? 1 : 0;
    p.pipe = attnh::bwd_pipelined(d, key_padding_mask != nullptr, B, H, N) ? 1 : 0;
    if (attnh::trace_on()) {
        char line[768];
        attnh::trace_plain_line(line, sizeof(line), "attn_bwd", "bwd_pre+bwd_dkdv+bwd_dq", dtype, B, H, N, d, causal,
                                key_padding_mask ? 1 : 0, attnh::bwd_ws_bytes(B, H, N),
                                p.pipe ? " loops=pipelined" : " loops=generic");
        attnh::trace_emit(line);
    }
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

const char* attn_last_error(void) { return attnh::g_err; }

int attn_version(void) { return 100; }

}  // extern "C"
