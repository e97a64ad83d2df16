// host_san.cpp -- the library's host-side checks and planning (attn_host.h)
// built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and
// driven over valid and invalid argument sets.  Pointers are fake integers:
// the code under test only compares them, so any dereference is a sanitizer
// report (and a crash).  Exit status 0 when every expectation holds.
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>

#include "attn_host.h"

static int g_failures = 0;

#define EXPECT(cond)                                                                     \
    do {                                                                                 \
        if (!(cond)) {                                                                   \
            std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++g_failures;                                                                \
        }                                                                                \
    } while (0)

static const void* P(uintptr_t a) { return (const void*)a; }
static const float* PF(uintptr_t a) { return (const float*)a; }

// q, k, v, o, lse, workspace: 4 GiB apart (no test tensor reaches 4 GiB)
static const uintptr_t G4 = (uintptr_t)1 << 32;
static const uintptr_t Q = G4 * 16, K = G4 * 17, V = G4 * 18, O = G4 * 19, L = G4 * 20, W = G4 * 21;

static int fwd(int B, int H, int N, int d, float scale, int causal, int dtype, const attn_opts* opts,
               attnh::FwdPlan* pl, uintptr_t q = Q, uintptr_t o = O, uintptr_t lse = L, const uint8_t* mask = nullptr)
{
    bool empty;
    return attnh::plan_fwd(P(q), P(K), P(V), P(o), PF(lse), B, H, N, d, scale, causal, mask, dtype, opts, pl, &empty);
}

static void forward_plans()
{
    attnh::FwdPlan pl;
    // the benchmarked call: B1 H32 N8192 d128 bf16 causal
    EXPECT(fwd(1, 32, 8192, 128, 0.08838834764f, 1, ATTN_BF16, nullptr, &pl) == ATTN_OK);
    EXPECT(pl.br == 256 && pl.bc == 64 && pl.n_qt == 32 && pl.qmode == 0);
    EXPECT(attnh::fwd_pipelined(pl));
    EXPECT(std::strcmp(attnh::fwd_kernel_name(pl), "fwd_m32_h16") == 0);
    attnh::plan_persistent(pl, 256);   // 32 heads x 16 causal pairs = 512 items over 256 CUs
    EXPECT(pl.persist == 256 && pl.xcd_affine == 1 && attnh::fwd_grid(pl) == 256);
    char line[768];
    const int n = attnh::trace_fwd_line(line, sizeof(line), "attn_fwd", pl);
    EXPECT(n > 0 && n < (int)sizeof(line));
    EXPECT(std::strstr(line, "kernel=fwd_m32_h16<bf16,d128,256x64>") != nullptr);
    EXPECT(std::strstr(line, "loop=pipelined grid=256 block=512 persistent=1 xcd_affine=1") != nullptr);
    // a short buffer truncates without writing past its end
    char tiny[24];
    attnh::trace_fwd_line(tiny, sizeof(tiny), "attn_fwd", pl);
    EXPECT(std::strlen(tiny) == sizeof(tiny) - 1);

    // uneven work: no persistent grid; H not a multiple of 8: no XCD affinity
    attnh::FwdPlan p2;
    EXPECT(fwd(1, 3, 1000, 128, 0.1f, 0, ATTN_BF16, nullptr, &p2) == ATTN_OK);
    attnh::plan_persistent(p2, 256);
    EXPECT(p2.persist == 0 && attnh::fwd_grid(p2) == 3 * 4);
    attnh::FwdPlan p3;
    EXPECT(fwd(1, 4, 32768, 128, 0.1f, 1, ATTN_BF16, nullptr, &p3) == ATTN_OK);
    attnh::plan_persistent(p3, 256);   // 4 heads x 64 pairs = 256 items
    EXPECT(p3.persist == 256 && p3.xcd_affine == 0);

    // generic loop, masks, fp32 and the 16-row tiles: no pipeline, named kernels
    attn_opts g = {0, 0, 0, 0, 1, {0, 0, 0}};
    EXPECT(fwd(1, 32, 8192, 128, 0.1f, 1, ATTN_BF16, &g, &pl) == ATTN_OK);
    EXPECT(!attnh::fwd_pipelined(pl));
    attnh::plan_persistent(pl, 256);
    EXPECT(pl.persist == 0);
    const uint8_t fake_mask = 1;
    EXPECT(fwd(2, 2, 100, 128, 0.1f, 0, ATTN_BF16, nullptr, &pl, Q, O, L, &fake_mask) == ATTN_OK);
    EXPECT(std::strcmp(attnh::fwd_kernel_name(pl), "fwd_m32_h16_masked") == 0 && !attnh::fwd_pipelined(pl));
    EXPECT(fwd(1, 2, 100, 64, 0.1f, 0, ATTN_F32, nullptr, &pl) == ATTN_OK);
    EXPECT(pl.br == 128 && pl.bc == 64 && std::strcmp(attnh::fwd_kernel_name(pl), "fwd_m32_f32_db") == 0);
    attn_opts bc128 = {0, 128, 0, 0, 0, {0, 0, 0}};
    EXPECT(fwd(1, 2, 100, 128, 0.1f, 0, ATTN_F32, &bc128, &pl) == ATTN_OK);   // two 128-key fp32 tiles exceed 128 KiB
    EXPECT(std::strcmp(attnh::fwd_kernel_name(pl), "fwd_m32_f32") == 0);
    attn_opts t16 = {16, 64, 0, 0, 0, {0, 0, 0}};
    EXPECT(fwd(1, 2, 100, 64, 0.1f, 0, ATTN_F16, &t16, &pl) == ATTN_OK);
    EXPECT(std::strcmp(attnh::fwd_kernel_name(pl), "fwd_m16") == 0 && attnh::fwd_block_threads(pl) == 64);
    attn_opts bc32 = {0, 32, 0, 0, 0, {0, 0, 0}};
    EXPECT(fwd(1, 2, 100, 64, 0.1f, 0, ATTN_F32, &bc32, &pl) == ATTN_OK);
    EXPECT(pl.br == 128 && pl.bc == 32);   // f32 default rows; 256 rows are not built for f32
    EXPECT(fwd(1, 2, 100, 64, 0.1f, 0, ATTN_BF16, &bc32, &pl) == ATTN_OK);
    EXPECT(pl.br == 128 && pl.bc == 32);   // d64 default is 128 rows already

    // scales: negative runs as |scale| on negated Q, zero as 1 on Q = 0
    EXPECT(fwd(1, 1, 8, 64, -1.5f, 0, ATTN_BF16, nullptr, &pl) == ATTN_OK);
    EXPECT(pl.kscale == 1.5f && pl.qmode == 1);
    EXPECT(fwd(1, 1, 8, 64, 0.f, 0, ATTN_BF16, nullptr, &pl) == ATTN_OK);
    EXPECT(pl.kscale == 1.f && pl.qmode == 2);
    EXPECT(fwd(1, 1, 8, 64, -0.f, 0, ATTN_BF16, nullptr, &pl) == ATTN_OK);
    EXPECT(pl.qmode == 2);
    EXPECT(pl.c == (float)(1.0 * 1.4426950408889634));
}

static void forward_rejections()
{
    attnh::FwdPlan pl;
    const float inf = std::numeric_limits<float>::infinity(), nan = std::numeric_limits<float>::quiet_NaN();
    EXPECT(fwd(1, 2, 8, 96, 0.1f, 0, ATTN_BF16, nullptr, &pl) == ATTN_ERR_HEAD_DIM);
    EXPECT(std::strstr(attnh::g_err, "d=96") != nullptr);
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, 5, nullptr, &pl) == ATTN_ERR_DTYPE);
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, -1, nullptr, &pl) == ATTN_ERR_DTYPE);
    EXPECT(fwd(-1, 2, 8, 64, 0.1f, 0, ATTN_BF16, nullptr, &pl) == ATTN_ERR_SHAPE);
    EXPECT(fwd(1 << 16, 1 << 10, 1 << 5, 64, 0.1f, 0, ATTN_BF16, nullptr, &pl) == ATTN_ERR_SHAPE);   // 2^31 rows
    EXPECT(fwd(1, 2, 8, 64, nan, 0, ATTN_BF16, nullptr, &pl) == ATTN_ERR_SCALE);
    EXPECT(fwd(1, 2, 8, 64, -inf, 0, ATTN_BF16, nullptr, &pl) == ATTN_ERR_SCALE);
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_BF16, nullptr, &pl, 0) == ATTN_ERR_NULL);
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_BF16, nullptr, &pl, Q + 8) == ATTN_ERR_ALIGN);
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_BF16, nullptr, &pl, Q, O, L + 2) == ATTN_ERR_ALIGN);
    // o over q (2*8*64*2 = 2048 bytes of q), lse inside o, lse over v
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_BF16, nullptr, &pl, Q, Q + 2032) == ATTN_ERR_ALIAS);
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_BF16, nullptr, &pl, Q, Q + 2048) == ATTN_OK);   // adjacent is fine
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_BF16, nullptr, &pl, Q, O, O + 64) == ATTN_ERR_ALIAS);
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_BF16, nullptr, &pl, Q, O, V + 4) == ATTN_ERR_ALIAS);
    // fp32 output doubles o's extent
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_BF16_OUT_F32, nullptr, &pl, Q, Q - 4080) == ATTN_ERR_ALIAS);
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_BF16, nullptr, &pl, Q, Q - 4080) == ATTN_OK);
    // options
    attn_opts o1 = {48, 0, 0, 0, 0, {0, 0, 0}};
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_BF16, &o1, &pl) == ATTN_ERR_TILE);
    attn_opts o2 = {0, 256, 0, 0, 0, {0, 0, 0}};
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_BF16, &o2, &pl) == ATTN_ERR_TILE);
    attn_opts o3 = {256, 64, 0, 0, 0, {0, 0, 0}};
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_F32, &o3, &pl) == ATTN_ERR_TILE);   // no 256-row fp32 kernel
    attn_opts o4 = {256, 16, 0, 0, 0, {0, 0, 0}};
    EXPECT(fwd(1, 2, 8, 128, 0.1f, 0, ATTN_BF16, &o4, &pl) == ATTN_ERR_TILE);
    attn_opts o5 = {0, 0, 2, 0, 0, {0, 0, 0}};
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_BF16, &o5, &pl) == ATTN_ERR_TILE);
    attn_opts o6 = {0, 0, 0, 16, 0, {0, 0, 0}};
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_BF16, &o6, &pl) == ATTN_ERR_TILE);
    attn_opts o7 = {0, 0, 0, 0, 0, {0, 0, 1}};
    EXPECT(fwd(1, 2, 8, 64, 0.1f, 0, ATTN_BF16, &o7, &pl) == ATTN_ERR_TILE);
    // empty: every pointer may be NULL
    bool empty = false;
    EXPECT(attnh::plan_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 4, 8, 64, 0.1f, 0, nullptr, ATTN_BF16,
                           nullptr, &pl, &empty) == ATTN_OK && empty);
    // the message buffer holds any message without overflow
    attnh::fail(ATTN_ERR_SHAPE, "%s", std::string(2000, 'x').c_str());
    EXPECT(std::strlen(attnh::g_err) == sizeof(attnh::g_err) - 1);
    char line[768];
    attnh::trace_status_line(line, sizeof(line), "attn_fwd", ATTN_ERR_SHAPE);
    EXPECT(std::strncmp(line, "attn: attn_fwd returned ATTN_ERR_SHAPE: xxx", 43) == 0);
}

// Every (dtype, d, br, bc) the checks accept has an instance listed in
// fwd_tiles.h, and the list is what the library documents: all 16 shapes of
// {16, 32, 64, 128}^2 for every type and head size, plus 256-row tiles for
// 16-bit inputs (bc 64 at d = 64; bc 32, 64, 128 at d = 128).
static void instance_table()
{
    const int tiles[5] = {16, 32, 64, 128, 256};
    int count = 0;
    for (int dtype = ATTN_F32; dtype <= ATTN_BF16_OUT_F32; ++dtype)
        for (int d : {64, 128})
            for (int br : tiles)
                for (int bc : tiles) {
                    bool want = br <= 128 && bc <= 128;
                    if (br == 256 && dtype != ATTN_F32)
                        want = d == 64 ? bc == 64 : (bc == 32 || bc == 64 || bc == 128);
                    EXPECT(attnh::fwd_built(dtype, d, br, bc) == want);
                    count += want;
                }
    EXPECT(count == 5 * 2 * 16 + 4 * (1 + 3));
    EXPECT(!attnh::fwd_built(7, 64, 64, 64));
    int sparse = 0;
    for (int d : {64, 128})
        for (int br : tiles)
            for (int bc : tiles) sparse += attnh::sparse_built(d, br, bc);
    EXPECT(sparse == 8);
}

static void sparse_plans()
{
    attnh::FwdPlan pl;
    bool empty;
    const uint8_t* bm = (const uint8_t*)(G4 * 22);
    EXPECT(attnh::plan_sparse(P(Q), P(K), P(V), P(O), PF(L), 1, 2, 500, 64, 0.1f, 1, nullptr, bm, 64, ATTN_BF16,
                              nullptr, &pl, &empty) == ATTN_OK);
    EXPECT(pl.br == 128 && pl.bc == 64 && pl.sparse && !attnh::fwd_pipelined(pl));
    EXPECT(std::strcmp(attnh::fwd_kernel_name(pl), "fwd_m32_h16_sparse") == 0);
    EXPECT(attnh::plan_sparse(P(Q), P(K), P(V), P(O), PF(L), 1, 2, 500, 64, 0.1f, 1, nullptr, bm, 48, ATTN_BF16,
                              nullptr, &pl, &empty) == ATTN_ERR_SHAPE);
    EXPECT(attnh::plan_sparse(P(Q), P(K), P(V), P(O), PF(L), 1, 2, 500, 64, 0.1f, 1, nullptr, nullptr, 64, ATTN_BF16,
                              nullptr, &pl, &empty) == ATTN_ERR_NULL);
    EXPECT(attnh::plan_sparse(P(Q), P(K), P(V), P(O), PF(L), 1, 2, 500, 64, 0.1f, 1, nullptr, bm, 64, ATTN_F32,
                              nullptr, &pl, &empty) == ATTN_ERR_DTYPE);
    // block flags inside o
    EXPECT(attnh::plan_sparse(P(Q), P(K), P(V), P(O), PF(L), 1, 2, 500, 64, 0.1f, 1, nullptr, (const uint8_t*)O + 16,
                              64, ATTN_BF16, nullptr, &pl, &empty) == ATTN_ERR_ALIAS);
    attn_opts ord = {0, 0, 1, 0, 0, {0, 0, 0}};
    EXPECT(attnh::plan_sparse(P(Q), P(K), P(V), P(O), PF(L), 1, 2, 500, 64, 0.1f, 1, nullptr, bm, 64, ATTN_BF16,
                              &ord, &pl, &empty) == ATTN_ERR_TILE);
    attn_opts t32 = {32, 32, 0, 0, 0, {0, 0, 0}};
    EXPECT(attnh::plan_sparse(P(Q), P(K), P(V), P(O), PF(L), 1, 2, 500, 64, 0.1f, 1, nullptr, bm, 64, ATTN_BF16,
                              &t32, &pl, &empty) == ATTN_ERR_TILE);
}

static void naive_and_backward()
{
    bool empty;
    const size_t need = attnh::naive_ws_bytes(1, 2, 8, ATTN_BF16);
    EXPECT(need == 2 * 8 * 8 * 2);
    EXPECT(attnh::check_naive(P(Q), P(K), P(V), P(O), PF(L), 1, 2, 8, 64, 0.1f, ATTN_BF16, P(W), need, &empty) == ATTN_OK);
    EXPECT(attnh::check_naive(P(Q), P(K), P(V), P(O), PF(L), 1, 2, 8, 64, 0.1f, ATTN_BF16, P(W), need - 1, &empty) ==
           ATTN_ERR_WORKSPACE);
    EXPECT(attnh::check_naive(P(Q), P(K), P(V), P(O), PF(L), 1, 2, 8, 64, 0.1f, ATTN_BF16, P(O + 16), need, &empty) ==
           ATTN_ERR_ALIAS);
    EXPECT(attnh::naive_ws_bytes(0, 2, 8, ATTN_BF16) == 0 && attnh::naive_ws_bytes(1, 2, 8, 9) == 0);

    const float* dq = PF(G4 * 23);
    const float* dk = PF(G4 * 24);
    const float* dv = PF(G4 * 25);
    const size_t bw = attnh::bwd_ws_bytes(1, 2, 8);
    EXPECT(bw == 2 * 8 * 8);
    EXPECT(attnh::check_bwd(P(Q), P(K), P(V), P(O), P(G4 * 26), PF(L), dq, dk, dv, 1, 2, 8, 64, 0.1f, ATTN_BF16,
                            P(W), bw, &empty) == ATTN_OK);
    EXPECT(attnh::check_bwd(P(Q), P(K), P(V), P(O), P(G4 * 26), nullptr, dq, dk, dv, 1, 2, 8, 64, 0.1f,
                            ATTN_BF16, P(W), bw, &empty) == ATTN_ERR_NULL);
    EXPECT(attnh::check_bwd(P(Q), P(K), P(V), P(O), P(G4 * 26), PF(L), dq, dq, dv, 1, 2, 8, 64, 0.1f, ATTN_BF16,
                            P(W), bw, &empty) == ATTN_ERR_ALIAS);
    EXPECT(attnh::check_bwd(P(Q), P(K), P(V), P(O), P(G4 * 26), PF(L), dq, dk, dv, 1, 2, 8, 64, 0.1f,
                            ATTN_BF16_OUT_F32, P(W), bw, &empty) == ATTN_ERR_DTYPE);
    EXPECT(attnh::check_bwd(P(Q), P(K), P(V), P(O), P(G4 * 26), PF(L), dq, dk, dv, 1, 2, 8, 64, 0.1f, ATTN_BF16,
                            P(W), bw - 4, &empty) == ATTN_ERR_WORKSPACE);

    // the gradient pipelines: d = 128 without a mask, while a head's rows
    // (256 bytes each) and the distance from D to lse2 plus a head's lse2
    // (4 (B H N + N) bytes) stay within 32-bit offsets
    EXPECT(attnh::bwd_pipelined(128, false, 1, 32, 8192));
    EXPECT(!attnh::bwd_pipelined(64, false, 1, 32, 8192));
    EXPECT(!attnh::bwd_pipelined(128, true, 1, 32, 8192));
    EXPECT(attnh::bwd_pipelined(128, false, 1, 1, 1 << 24) == false);           // 2^24 rows of 256 bytes
    EXPECT(attnh::bwd_pipelined(128, false, 1, 1, (1 << 24) - 1));
    EXPECT(!attnh::bwd_pipelined(128, false, 4096, 64, 4096));                  // 4 B H N = 2^32
    EXPECT(attnh::bwd_pipelined(128, false, 2047, 64, 8192));                   // 4 (B H N + N) < 2^32
}

// Key chunks of the decode path: whole 32-key tiles, every key in exactly one
// chunk, no empty chunk, at most 1024 chunks.
static void decode_chunks()
{
    const int nks[] = {0, 1, 31, 32, 33, 100, 1000, 4096, 8191, 65536, 1 << 20};
    const int nqs[] = {1, 2, 16, 17, 300};
    for (int Nk : nks)
        for (int Nq : nqs)
            for (int s : {0, 1, 2, 3, 7, 64, 1024}) {
                int splits = -1, kps = -1;
                attnh::decode_splits(2, 8, Nq, Nk, s, &splits, &kps);
                EXPECT(kps > 0 && kps % 32 == 0);
                EXPECT(splits >= 1 && splits <= 1024);
                if (Nk > 0) {
                    EXPECT((int64_t)splits * kps >= Nk);
                    EXPECT((int64_t)(splits - 1) * kps < Nk);
                    if (s > 0) EXPECT(splits <= s);
                } else {
                    EXPECT(splits == 1);
                }
                const size_t ws = attnh::decode_ws_query(2, 8, Nq, Nk, 128, s);
                EXPECT(ws == attnh::decode_ws_bytes(2, 8, Nq, 128, splits));
            }
    attnh::DecPlan pl;
    bool empty;
    const size_t need = attnh::decode_ws_query(1, 4, 1, 4096, 128, 0);
    EXPECT(attnh::plan_decode(P(Q), P(K), P(V), P(O), PF(L), 1, 4, 1, 4096, 128, 0.1f, 1, nullptr, ATTN_BF16, P(W),
                              need, 0, &pl, &empty) == ATTN_OK);
    EXPECT(pl.ws_bytes == need);
    EXPECT(attnh::plan_decode(P(Q), P(K), P(V), P(O), PF(L), 1, 4, 1, 4096, 128, 0.1f, 1, nullptr, ATTN_BF16, nullptr,
                              0, 0, &pl, &empty) == ATTN_ERR_WORKSPACE);
    EXPECT(pl.ws_bytes == need);   // the size a caller without a workspace needs
    EXPECT(attnh::plan_decode(P(Q), P(K), P(V), P(O), PF(L), 1, 4, 1, 4096, 128, 0.1f, 1, nullptr, ATTN_F32, P(W),
                              need, 0, &pl, &empty) == ATTN_ERR_DTYPE);
    EXPECT(attnh::plan_decode(P(Q), P(K), P(V), P(O), PF(L), 1, 4, 1, 4096, 128, 0.1f, 1, nullptr, ATTN_BF16, P(W),
                              need, 1025, &pl, &empty) == ATTN_ERR_TILE);
    EXPECT(attnh::plan_decode(P(Q), nullptr, nullptr, P(O), PF(L), 1, 4, 1, 0, 128, 0.1f, 1, nullptr, ATTN_BF16, P(W),
                              attnh::decode_ws_query(1, 4, 1, 0, 128, 0), 0, &pl, &empty) == ATTN_OK);
    char line[768];
    attnh::trace_decode_line(line, sizeof(line), "attn_decode_fwd", pl, false);
    EXPECT(std::strstr(line, "kernel=dec_split+dec_merge<bf16,d128>") != nullptr);
}

int main()
{
    forward_plans();
    forward_rejections();
    instance_table();
    sparse_plans();
    naive_and_backward();
    decode_chunks();
    if (g_failures) {
        std::fprintf(stderr, "host_san: %d expectation(s) failed\n", g_failures);
        return 1;
    }
    std::printf("host_san: all host checks passed\n");
    return 0;
}
