/*
 * attn.h -- C ABI of the MI355X (gfx950) exact-attention forward library.
 *
 * What the library computes.  For every batch b, head h and query row i:
 *
 *     s_ij = scale * sum_c q[b,h,i,c] * k[b,h,j,c]     for the visible keys j
 *     o[b,h,i,:] = sum_j softmax_j(s_i.) * v[b,h,j,:]
 *     lse[b,h,i] = log sum_j exp(s_ij)                (natural log)
 *
 * This is the attention of Golden et al., "Is Flash Attention Stable?",
 * sec. II-A (softmax(Q K^T / sqrt(d_k)) V; the caller passes the factor as
 * `scale`), evaluated the FlashAttention way described in the same paper's
 * sec. II-B and in the yadro-code tutorial "How FlashAttention reduces GPU
 * memory traffic": key tiles are folded into a running row maximum, a running
 * sum of exponentials and an unnormalised output that is rescaled by
 * exp(m_old - m_new) whenever the maximum grows, and divided by the sum once at
 * the end.  The N x N score matrix is never stored.
 *
 * Visibility: key j is visible to query i unless `causal` is set and j > i
 * (the causal prefix of the tutorial's self-check), or key_padding_mask[b*N+j]
 * is non-zero.  Masked scores are a true -infinity, never a finite stand-in
 * (the first page warns about a hard-coded -50,000 in one library's kernels).
 * A row with no visible key has no softmax; this library defines its output as
 * +0.0 in every element and lse = -infinity.
 *
 * Entry points: the forward (attn_fwd, attn_fwd_ex, with host-only checks in
 * attn_check_args), its block-sparse variant (attn_fwd_sparse), the materialising baseline (attn_naive_fwd), a query
 * block against a key/value cache (attn_decode_fwd) and the gradient
 * (attn_bwd).  The last three take a caller-owned device workspace whose size
 * their *_workspace_bytes function gives.
 *
 * Conventions shared by every entry point below:
 *   - q, k, v, o: DEVICE pointers, contiguous [B][H][N][d] row-major, element
 *     type given by `dtype` (see attn_dtype), 16-byte aligned.  The caller owns
 *     them.  o must not overlap q, k, v or lse.
 *   - lse: DEVICE pointer to [B][H][N] float, 4-byte aligned, or NULL (then no
 *     lse is written).
 *   - key_padding_mask: DEVICE pointer to [B][N] bytes (non-zero = padded key,
 *     excluded from every query row of that batch), or NULL (no padding).
 *   - B, H, N >= 0 (any zero is a successful no-op), B*H*N < 2^31,
 *     d in {64, 128}; scale any finite float (1/sqrt(d) in the usual use; a
 *     negative scale is run as |scale| on negated q and scale 0 as a uniform
 *     softmax over the visible keys, both exact).
 *   - stream: a hipStream_t passed as void*; NULL is the null stream.  Every
 *     call is asynchronous on that stream; outputs are valid once the caller
 *     has synchronised it.  No entry point synchronises or allocates device
 *     memory.  State kept between calls: a thread-local error string, the
 *     compute-unit count of each device (queried once, for the grid), the
 *     ATTN_TRACE setting, and the device scratch of attn_decode_fwd_noalloc.
 *   - Errors: arguments are checked on the host before anything is launched; a
 *     failed check returns its status and writes nothing.  A launch failure
 *     returns ATTN_ERR_HIP.  attn_last_error() then holds a message.  No
 *     exception and no abort crosses this interface.
 *   - Dispatch log: with the environment variable ATTN_TRACE set to anything
 *     but "" or "0" when the library first reads it, every entry point except
 *     attn_check_args writes one line starting "attn: " to stderr: the
 *     kernel instance it launched (type, head size, tiles), the shape, the
 *     loop form, the grid and block, or the status it returned without a
 *     launch.
 *   - Determinism: identical inputs and options give bitwise-identical o and
 *     lse (no atomics, fixed reduction order).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o.  In the *_OUT_F32 flavours q, k, v are 16-bit
 * and o is written as float; the kernel and its arithmetic are the same, only
 * the final store differs. */
enum attn_dtype {
    ATTN_F32 = 0,          /* q, k, v, o float; fp32 matrix-core products, fp32 P      */
    ATTN_F16 = 1,          /* q, k, v, o IEEE half; P rounded to half for P.V           */
    ATTN_BF16 = 2,         /* q, k, v, o bfloat16; P rounded to bfloat16 for P.V        */
    ATTN_F16_OUT_F32 = 3,  /* q, k, v half; o float                                      */
    ATTN_BF16_OUT_F32 = 4  /* q, k, v bfloat16; o float                                  */
};

enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,      /* a required pointer is NULL                               */
    ATTN_ERR_SHAPE = 2,     /* negative size, or B*H*N too large                        */
    ATTN_ERR_HEAD_DIM = 3,  /* d not in {64, 128}                                       */
    ATTN_ERR_DTYPE = 4,     /* unknown dtype                                            */
    ATTN_ERR_ALIGN = 5,     /* q/k/v/o not 16-byte aligned, or lse not 4-byte aligned   */
    ATTN_ERR_TILE = 6,      /* tile shape, kv_order or ref_slack not supported          */
    ATTN_ERR_SCALE = 7,     /* scale not finite                                         */
    ATTN_ERR_ALIAS = 8,     /* o overlaps an input or lse                               */
    ATTN_ERR_HIP = 9,       /* the HIP runtime reported an error                        */
    ATTN_ERR_WORKSPACE = 10 /* workspace NULL, misaligned or too small                   */
};

/* Tile and fold-order options (attn_fwd_ex).
 *   br: query rows per workgroup tile, one of 16, 32, 64, 128, or 256 for the
 *       16-bit types with bc in {32, 64, 128} at d = 128 or bc = 64 at d = 64
 *       (0 = default: 256 for the 16-bit types at d = 128, 128 at d = 64
 *       and for fp32; 128 when only bc is given and no 256-row tile exists
 *       for it).
 *   bc: keys per key tile, one of 16, 32, 64, 128 (0 = default: 128 for the
 *       16-bit types at d = 64, 64 otherwise).  bc is also the
 *       rescaling granularity: the running maximum is updated once per tile.
 *   kv_order: 0 folds each row's key tiles first to last, 1 last to first.
 *   ref_slack: 0 (default) keeps the reference of the online merge at each
 *       row's exact running maximum, as the tutorial's merge does.  A value s
 *       in 1..15 lets the reference lag: it moves to a tile's maximum only
 *       when that maximum exceeds it by more than s in base-2 exponent units,
 *       so exponentials stay <= 2^s and most tiles skip the rescale of the
 *       accumulator.  The result is the same in exact arithmetic; in 16-bit
 *       modes the rounding of P no longer leaves the largest weight exact, which
 *       raises the deviation from the exact result (about 1.1x on N(0,1)
 *       inputs, 2x on strongly peaked rows) for a few percent of speed.
 *   generic_loop: 0 (default) lets the 16-bit d = 128 kernel with 256 x 64
 *       tiles run its key tiles that need no masking through the hand-
 *       scheduled software pipeline (score products of the next tile beside
 *       the softmax of the current one); non-zero forces the compiler-
 *       scheduled tile loop everywhere.  Both do the same operations in the
 *       same order per row, so their results are bitwise equal; the switch
 *       exists to check exactly that.
 * The tile sizes and block order are the knobs the stability paper's
 * sequence-length and perturbation sweeps vary (its Figs. 5 and 6). */
typedef struct attn_opts {
    int br;
    int bc;
    int kv_order;
    int ref_slack;
    int generic_loop;
    int reserved[3];   /* must be zero */
} attn_opts;

/* Exact attention forward with the default tiles and ascending fold order. */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d, float scale, int causal,
             const uint8_t* key_padding_mask, int dtype, void* stream);

/* Same as attn_fwd with explicit tiles and fold order; opts NULL = defaults. */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int N, int d, float scale, int causal,
                const uint8_t* key_padding_mask, int dtype, void* stream,
                const attn_opts* opts);

/* Block-sparse forward.  The yadro-code tutorial ("How FlashAttention reduces
 * GPU memory traffic", its overview of the NeurIPS 2022 paper) names a
 * block-sparse extension without describing it; this library's reading: the
 * rows and keys of each (b, h) are cut into blocks of `block` rows, and the
 * pair (i, j) is visible only if block_mask[((b*H + h)*nb + i/block)*nb +
 * j/block] is non-zero (nb = ceil(N / block)), in addition to the causal and
 * key-padding rules of attn_fwd.  Everything else (softmax over the visible
 * keys, empty rows -> 0 and -inf, lse) is attn_fwd's.  Key tiles without an
 * attended block are skipped: the work scales with the attended blocks.
 *   block_mask: DEVICE pointer to [B][H][nb][nb] bytes, caller-owned; must not
 *       overlap o or lse.
 *   block: a positive multiple of 32 (else ATTN_ERR_SHAPE).
 *   dtype: the 16-bit types and their *_OUT_F32 flavours (ATTN_F32 ->
 *       ATTN_ERR_DTYPE).
 *   opts: as attn_fwd_ex, with (br, bc) one of (64, 64), (128, 64),
 *       (128, 128), (256, 64) and kv_order 0; else ATTN_ERR_TILE.  Unset br
 *       or bc (0, or opts NULL) default to 128 and 64: wider workgroups
 *       visit tiles in which only some of their row blocks attend.
 * Errors and stream semantics as attn_fwd. */
int attn_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal,
                    const uint8_t* key_padding_mask, const uint8_t* block_mask, int block,
                    int dtype, void* stream, const attn_opts* opts);

/* Host-only argument check of attn_fwd_ex: returns the status attn_fwd_ex would
 * return before launching anything.  Touches no device and no pointer. */
int attn_check_args(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal,
                    const uint8_t* key_padding_mask, int dtype, const attn_opts* opts);

/* Default (br, bc) that attn_fwd uses for this dtype, head size and causality.
 * Returns ATTN_OK, or ATTN_ERR_DTYPE / ATTN_ERR_HEAD_DIM. */
int attn_default_tiles(int dtype, int d, int causal, int* br, int* bc);

/* Baseline attention that materialises the score matrix, for comparison only
 * (the stability paper's "baseline attention").  S = scale*q k^T is stored in
 * the workspace in the input type (float for ATTN_F32), the row softmax P is
 * computed in fp32 and stored back in the input type, then o = P v with fp32
 * accumulation.  Masking, fully masked rows and lse follow attn_fwd.
 * workspace: DEVICE pointer of at least attn_naive_workspace_bytes() bytes,
 * 16-byte aligned, owned by the caller. */
int attn_naive_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* key_padding_mask, int dtype, void* stream,
                   void* workspace, size_t workspace_bytes);

/* Workspace bytes attn_naive_fwd needs: B*H*N*N elements of the input type. */
size_t attn_naive_workspace_bytes(int B, int H, int N, int dtype);

/* Key/value-cache decoding: Nq query rows against Nk cached keys (the
 * tutorial distinguishes processing a long prompt from step-by-step generation
 * with a key/value cache; the shapes, reuse and bottleneck differ).
 *   q, o: DEVICE [B][H][Nq][d]; k, v: DEVICE [B][H][Nk][d]; lse [B][H][Nq] or
 *   NULL; key_padding_mask [B][Nk] bytes or NULL.  With Nk = 0 (empty cache)
 *   k and v may be NULL and every row gives O = 0, lse = -inf.  16-bit dtypes only
 *   (ATTN_F16, ATTN_BF16 and their *_OUT_F32 flavours); d in {64, 128}.
 *   causal: row i sits at position Nk - Nq + i of the sequence and sees keys
 *   j <= Nk - Nq + i (the end of the cache); rows that see no key give O = 0
 *   and lse = -inf, as in attn_fwd.
 * The keys of every (b, h) are split into chunks handled independently; each
 * chunk's partial result (acc / l, lse) goes to the workspace and a second
 * kernel merges them: lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s.
 *   num_splits: key chunks per (b, h), 0 = chosen by the library, at most 1024.
 *   workspace: DEVICE, 16-byte aligned, at least attn_decode_workspace_bytes()
 *   bytes, owned by the caller, not overlapping any other argument; its
 *   contents on return are unspecified.  Two calls may not share a workspace
 *   concurrently.
 * Errors and stream semantics as attn_fwd; a too small or missing workspace
 * returns ATTN_ERR_WORKSPACE, a bad num_splits ATTN_ERR_TILE. */
int attn_decode_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Nq, int Nk, int d, float scale, int causal,
                    const uint8_t* key_padding_mask, int dtype, void* stream,
                    void* workspace, size_t workspace_bytes, int num_splits);

/* Measurement helper, not part of any computation: launches `reps` rounds of
 * independent bf16 32x32x16 matrix-core products on every compute unit (eight
 * four-wave workgroups per unit, accumulators in AGPRs, pseudo-random finite
 * operands) and writes the launch's floating-point operation count to *flops.
 * Timing it on `stream` gives the matrix-core rate the part sustains at its
 * current clock: the ceiling the forward's rate is compared with, next to the
 * published peak.  Returns ATTN_ERR_SHAPE for reps <= 0 or flops NULL and
 * ATTN_ERR_HIP on a launch failure. */
int attn_probe_mfma(int reps, void* stream, double* flops);

/* Workspace bytes attn_decode_fwd needs for these sizes and num_splits
 * (0 for invalid sizes). */
size_t attn_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits);

/* attn_decode_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same checks, kernels and results, with the partial results held in a
 * fixed 16 MiB device array inside the library instead of a caller workspace.
 * Each GPU the library runs on keeps its own copy until the process ends; the
 * first call on a device looks its address up (hipGetSymbolAddress).  Nothing
 * is allocated, by this call or later.
 *   Limit: attn_decode_workspace_bytes(B, H, Nq, Nk, d, num_splits) must not
 *   exceed 16 MiB (16777216 bytes); larger calls return ATTN_ERR_WORKSPACE
 *   before anything is launched.
 *   Concurrency: every call on one GPU uses that GPU's array; calls that overlap
 *   in time on one GPU (other streams, other threads) race and must not be
 *   issued.  Every call writes each partial result it reads, so no state
 *   carries over between calls.
 * Other arguments, errors and stream semantics as attn_decode_fwd. */
int attn_decode_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Nq, int Nk, int d, float scale, int causal,
                            const uint8_t* key_padding_mask, int dtype, void* stream, int num_splits);

/* Gradient of attn_fwd w.r.t. q, k and v (the tutorial asks to check outputs
 * and gradients).  Recomputes P tile by tile from the forward's lse:
 * P_ij = exp(scale q_i.k_j - lse_i), D_i = sum_c dout_ic o_ic,
 * dv = P^T dout, ds = P (dout v^T - D), dq = scale ds k, dk = scale ds^T q.
 *   q, k, v, o, dout: DEVICE [B][H][N][d] in the input type, 16-byte aligned
 *   (o and lse as written by attn_fwd with the same arguments).
 *   lse: DEVICE [B][H][N] float.  dq, dk, dv: DEVICE [B][H][N][d] float,
 *   16-byte aligned, not overlapping anything else.
 *   dtype: ATTN_BF16 or ATTN_F16.  Masking as attn_fwd; rows with no visible
 *   key contribute nothing.
 *   workspace: DEVICE, 16-byte aligned, attn_bwd_workspace_bytes() bytes.
 * Deterministic (no atomics).  Errors and stream semantics as attn_fwd. */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             float* dq, float* dk, float* dv, int B, int H, int N, int d, float scale, int causal,
             const uint8_t* key_padding_mask, int dtype, void* stream, void* workspace, size_t workspace_bytes);

/* Workspace bytes attn_bwd needs (8 per row). */
size_t attn_bwd_workspace_bytes(int B, int H, int N);

/* Static description of a status code. */
const char* attn_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* attn_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
