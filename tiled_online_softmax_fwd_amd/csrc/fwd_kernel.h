// fwd_kernel.h -- gfx950 kernels of the tiled online-softmax attention forward.
//
// One workgroup owns BR query rows of one (batch, head) and walks that head's
// key tiles of BC rows.  Per key tile it (a) stages K and V in LDS, (b) forms
// the score tile on the matrix cores, (c) updates each query row's reference
// maximum m, running sum of exponentials l and unnormalised output acc -- the
// online merge of the yadro-code tutorial "How FlashAttention reduces GPU
// memory traffic" (a bigger reference rescales l and acc by exp(m_old - m_new);
// the reference lags the running maximum by a bounded amount, see ref_step)
// -- and (d) accumulates P.V on the matrix cores.  acc / l is formed once, at
// the end.  The score tile lives only in registers: the N x N matrix of Golden
// et al., "Is Flash Attention Stable?", sec. II-B, is never written anywhere.
//
// Orientation.  Each wave owns 32 query rows and computes the TRANSPOSED score
// tile S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16} (or 32x32x2_f32): in the
// 32x32 accumulator lane L holds query column L%32 and 16 key rows
// {8*(j/4) + 4*(L/32) + j%4}.  A query row's maximum and sum are therefore
// in-lane reductions plus one v_permlane32_swap, and m, l and the rescale
// factor are per-lane scalars.  The same registers, converted to the input
// type, are directly the B operand of O^T += V^T P^T (contraction over keys
// with a fixed permutation of the key index that V^T's operand reproduces).
// V^T's operand is read from row-major V in LDS with ds_read_b64_tr_b16.
//
// Scores are kept raw (q.k) in fp32; the softmax uses base 2 with the factor
// c = scale * log2(e) folded into one FMA: p = exp2(s*c - m*c).  Masked scores
// are -inf.  A row with no visible key yet uses 0 as its reference so that no
// exp2(-inf - -inf) is ever formed.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fwd_pipe_asm.h"

namespace attnk {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const uint8_t* mask;   // [B][N] or nullptr
    int B, H, N;
    int n_qt;              // query tiles per (b, h)
    float scale;           // natural-log domain factor of q.k
    float c;               // scale * log2(e)
    int causal;
    int kv_order;          // 0 ascending key tiles, 1 descending
    int out_f32;           // o is float instead of the input type
    float slack;           // lag allowed to the merge reference (base-2 units, 0 = exact maximum)
    int pipe;              // 16-bit d = 128, 256 x 64: software-pipelined steady tiles (0 = tile loop only)
    int qmode;             // 0: Q as stored; 1: Q negated (scale < 0); 2: Q taken as 0 (scale = 0)
    int persist;           // > 0: persistent grid of that many workgroups walking UnitSched's items
    int xcd_affine;        // persistent items of head bh run on XCD bh % 8 (B*H and the grid multiples of 8)
    const uint8_t* bmask;  // block-sparse kernels: [B][H][nb][nb] block flags, non-zero = attended
    int blk;               // block edge in rows (multiple of 32)
    int nb;                // ceil(N / blk)
};

typedef hipError_t (*LaunchFn)(const FwdParams&, hipStream_t);

// compile-time index (selects the LDS buffer of an unrolled loop body)
template <int V> struct Int { static constexpr int value = V; };

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xhalf_max(float x)
{
    // max over lanes L and L^32: permlane32_swap returns (lower, upper) halves
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                              __builtin_bit_cast(unsigned, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ float xhalf_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                              __builtin_bit_cast(unsigned, x), false, false);
    // both halves add (lower + upper) in the same order
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Non-positive scales.  The merge keeps the running maximum of raw scores q.k
// and applies the factor c > 0 in one fma, which presumes c > 0 (the pages'
// factor is 1/sqrt(d)).  A negative scale is run as |scale| on scores negated
// through Q (c (q.k) = |c| ((-q).k); a sign flip is exact and round-to-nearest
// is symmetric, so the products are exactly negated), and a zero scale as
// scale 1 on Q = 0 (every score 0: the softmax is uniform over the visible
// keys, lse = ln(count)).  The host picks the mode; Q is transformed once, in
// registers.
__device__ __forceinline__ u32x4 q_mode16(u32x4 w, int qmode)
{
    if (qmode == 1) return w ^ 0x80008000u;          // sign bits of both 16-bit halves
    if (qmode == 2) return (u32x4){0u, 0u, 0u, 0u};
    return w;
}
__device__ __forceinline__ float q_mode32(float x, int qmode) { return qmode == 1 ? -x : (qmode == 2 ? 0.f : x); }

// Key-padding flags of the four consecutive keys k..k+3 of one mask row, as
// the bytes of one word: one 32-bit load when the row is 4-byte aligned and
// the four keys lie inside it, else four byte loads at keys clamped to N - 1
// (keys past N are never visible, and key N - 1 lies in the same tile).
__device__ __forceinline__ uint32_t pad_word(const uint8_t* row, bool vec, int k, int N)
{
    if (vec && k + 3 < N) return *(const uint32_t*)(row + k);
    uint32_t w = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) w |= (uint32_t)row[min(k + r, N - 1)] << (8 * r);
    return w;
}
// Non-zero when some byte of w is zero (some of the four keys is not padded).
__device__ __forceinline__ uint32_t has_zero_byte(uint32_t w) { return (w - 0x01010101u) & ~w & 0x80808080u; }
// Byte j of w is zero: key j of the word is not padded.
__device__ __forceinline__ bool unpadded(uint32_t w, int j) { return ((w >> (8 * j)) & 0xffu) == 0; }

// Tile-level padding decision of one wave over the flag words of the keys its
// lanes hold (together every key of the tile): `any` when some key is padded
// (the tile takes the masked path), `none_visible` when every key is (the
// tile adds nothing: its maximum is -inf and every P is 0).
template <int NWORDS>
__device__ __forceinline__ void pad_tile(const uint32_t (&w)[NWORDS], bool& any, bool& none_visible)
{
    uint32_t a = 0, z = 0;
#pragma unroll
    for (int i = 0; i < NWORDS; ++i) {
        a |= w[i];
        z |= has_zero_byte(w[i]);
    }
    any = __builtin_amdgcn_ballot_w64(a != 0) != 0;
    none_visible = __builtin_amdgcn_ballot_w64(z != 0) == 0;
}

// Reference of the online merge.  The merge multiplies l and acc by
// exp(m_old - m_new) when the reference moves from m_old to m_new, and the
// result acc / l (and lse = m + ln l) is the same for any reference as long as
// no exponent overflows.  With slack 0 the reference is the exact running
// maximum (it moves whenever a tile's maximum exceeds it).  With slack s > 0 it
// moves only when a tile's maximum exceeds it by more than s in base-2 units,
// so P <= 2^s and most tiles skip the rescale of acc.  At the first visible key
// it always moves.  m = -inf means no visible key yet; exponents then use 0 as
// reference, so exp2(-inf - -inf) is never formed.
struct RefStep {
    float m;        // new reference (raw q.k units)
    float mc;       // reference used in the exponents, times c
    float alpha;    // rescale factor of l and acc (1 when the reference stays)
    bool moved;
};
__device__ __forceinline__ RefStep ref_step(float m, float mt, float c, float slack)
{
    RefStep r;
    r.moved = (mt - m) * c > slack;        // false for mt = -inf (NaN or -inf compare)
    r.m = r.moved ? mt : m;
    r.mc = (r.m == -INFINITY) ? 0.f : r.m * c;
    r.alpha = r.moved ? fast_exp2((m - r.m) * c) : 1.f;   // 0 when m = -inf
    return r;
}

// 16-bit element traits
template <typename T> struct H16;
template <> struct H16<__bf16> {
    using v8 = bf16x8;
    static __device__ __forceinline__ f32x16 mma32(v8 a, v8 b, f32x16 c)
    { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }
};
template <> struct H16<_Float16> {
    using v8 = f16x8;
    static __device__ __forceinline__ f32x16 mma32(v8 a, v8 b, f32x16 c)
    { return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0); }
};

// LDS swizzles, in 16-byte chunks.  CPR = chunks per row.
// K rows are read 16 bytes per lane with 32 consecutive rows at one column:
// XOR the chunk with the row so that 16 consecutive rows hit 16 distinct
// 16-byte bank groups.
template <int CPR> __device__ __forceinline__ int swz_k(int r, int c)
{
    if constexpr (CPR >= 16) return c ^ (r & 15);
    else return c ^ ((r >> 1) & 7);      // CPR == 8: two rows per 256 bytes
}
// 16-bit V rows are read by ds_read_b64_tr_b16: a half wave covers 4 rows x 64
// bytes; put the 4 rows in 4 distinct 64-byte bank groups.
template <int CPR> __device__ __forceinline__ int swz_v16(int r, int c)
{
    if constexpr (CPR >= 16) return c ^ ((r & 3) << 2);
    else return c ^ (((r >> 1) & 1) << 2);
}
// fp32 V rows are read 4 bytes per lane, 32 lanes on one row and 32 on row+4.
__device__ __forceinline__ int swz_v32(int r, int c) { return c ^ (((r >> 2) & 1) << 3); }
// 16-bit rows read both ways (the backward's Q, dO and K tiles): 16 bytes per
// lane down 16 consecutive rows, and transposed, a half wave over 4 rows x 64
// bytes.  The row term is a bijection over each 16-row group (the row reads
// hit distinct 16-byte groups) whose top two bits are r & 3 (the 4 rows of a
// transposed read land in 4 distinct 64-byte groups).  At 8 chunks per row
// (two rows per 256 bytes) the row term is a bijection of r >> 1 over rows of
// one parity, whose top bit is (r >> 1) & 1.
template <int CPR> __device__ __forceinline__ int swz_kt(int r, int c)
{
    if constexpr (CPR >= 16) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
    else return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Cooperative copy of ROWS x CPR 16-byte chunks from global rows (row stride
// CPR chunks) into LDS at chunk index r*CPR + SWZ(r, c).  Rows >= rows_valid are
// zero-filled, so padding keys of a ragged last tile carry V = 0 and never
// meet a stale or non-finite value.
template <int ROWS, int CPR, int NT, int KIND>
__device__ __forceinline__ void stage_tile(u32x4* __restrict__ lds, const u32x4* __restrict__ g,
                                           int rows_valid, int tid)
{
    constexpr int TOTAL = ROWS * CPR;
    constexpr int ITERS = (TOTAL + NT - 1) / NT;
    constexpr int BATCH = ITERS < 8 ? ITERS : 8;     // loads in flight per thread
#pragma unroll
    for (int it0 = 0; it0 < ITERS; it0 += BATCH) {
        u32x4 buf[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int idx = tid + (it0 + u) * NT;
            buf[u] = (u32x4){0u, 0u, 0u, 0u};
            if (it0 + u < ITERS && (TOTAL % NT == 0 || idx < TOTAL) && idx / CPR < rows_valid) buf[u] = g[idx];
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int idx = tid + (it0 + u) * NT;
            if (it0 + u < ITERS && (TOTAL % NT == 0 || idx < TOTAL)) {
                const int r = idx / CPR, c = idx % CPR;
                int sc;
                if constexpr (KIND == 0) sc = swz_k<CPR>(r, c);
                else if constexpr (KIND == 1) sc = swz_v16<CPR>(r, c);
                else if constexpr (KIND == 3) sc = swz_kt<CPR>(r, c);
                else sc = swz_v32(r, c);
                lds[r * CPR + sc] = buf[u];
            }
        }
    }
}

// Workgroup -> (b*H + h, query tile).  Causal: heaviest (last) query tiles of
// every head are issued first.  Consecutive workgroup ids go to consecutive
// heads, so with a multiple of 8 heads one head's tiles share one XCD's L2
// (workgroups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ void tile_of_block(const FwdParams& p, int& bh, int& qt)
{
    const int BH = p.B * p.H;
    const int lin = blockIdx.x;
    bh = lin % BH;
    qt = lin / BH;
    if (p.causal) qt = p.n_qt - 1 - qt;
}

// Persistent schedule.  The grid holds one workgroup per compute unit and each
// workgroup walks a list of items.  An item is one query tile, or under causal
// masking the pair of query tiles (n_qt-1-r, r) of one head: its two tiles
// cost the same number of key tiles for every r, so equal item counts give
// equal work.  With xcd_affine, the items of head bh go to the workgroups of
// XCD bh % 8 (workgroups are dealt to the 8 XCDs round-robin), so every head's
// K and V are read through one XCD's L2, and the workgroups of a head sweep its
// key tiles together (heaviest tile of each pair first: its phase reads the
// same key tile in every workgroup of the head at once; light tile first
// staggers them, and 32 distinct tiles per step overflow the XCD's L2 -- 1.68x
// the reads of heavy first at B1 H32 N8192 d128 causal on MI355X).
struct UnitSched {
    int item, stride, n_items, iph, n_qt, causal, xcd, part;

    __device__ __forceinline__ void init(const FwdParams& p)
    {
        n_qt = p.n_qt;
        causal = p.causal;
        iph = causal ? (n_qt + 1) / 2 : n_qt;
        const int BH = p.B * p.H;
        if (p.xcd_affine) {
            xcd = (int)blockIdx.x & 7;
            item = (int)blockIdx.x >> 3;
            stride = p.persist >> 3;
            n_items = (BH >> 3) * iph;
        } else {
            xcd = -1;
            item = (int)blockIdx.x;
            stride = p.persist;
            n_items = BH * iph;
        }
        part = 0;
    }
    // the unit at the current position; false when the list is done
    __device__ __forceinline__ bool get(int& bh, int& qt) const
    {
        if (item >= n_items) return false;
        const int h = item / iph, r = item % iph;
        bh = xcd >= 0 ? xcd + 8 * h : h;
        qt = !causal ? r : (part == 0 ? n_qt - 1 - r : r);
        return true;
    }
    __device__ __forceinline__ void advance()
    {
        const int r = item % iph;
        if (causal && part == 0 && n_qt - 1 - r != r) { part = 1; return; }
        part = 0;
        item += stride;
    }
};

// ============================================================ 16-bit, 32x32
// Wait until at most N vector-memory operations of this wave are outstanding
// (vmcnt only; LDS and scalar counters untouched).
template <int N> __device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// also wait for the in-flight tile prefetches).  The empty asm statements keep
// the compiler from moving memory operations across it; LDS reads before it
// have all been consumed, LDS DMA writes are waited for explicitly.
__device__ __forceinline__ void wg_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// One wave instruction of LDS DMA: lane L copies 16 bytes from global address
// gbase + voff(L) to LDS byte address lds_base + 16*L.  gbase and lds_base are
// wave-uniform (SGPRs; lds_base goes through M0, which is saved and restored).
// Written as inline asm so that the compiler does not treat the copy as an LDS
// store it must wait for before every later LDS read: completion is tracked
// explicitly with wait_vmcnt() and a barrier.
__device__ __forceinline__ uint64_t uniform_ptr(const void* p)
{
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// NT: the non-temporal cache policy, for data that is read exactly once (the
// key/value cache of the decode path); tiles that other workgroups read again
// from L2 (the forward) keep the default policy.
template <bool NT = false>
__device__ __forceinline__ void lds_dma16(uint64_t gbase, uint32_t voff, uint32_t lds_base)
{
    uint32_t saved;
    if constexpr (NT)
        asm volatile("s_mov_b32 %0, m0\n\t"
                     "s_mov_b32 m0, %3\n\t"
                     "global_load_lds_dwordx4 %1, %2 nt\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(saved)
                     : "v"(voff), "s"(gbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "memory");
    else
        asm volatile("s_mov_b32 %0, m0\n\t"
                     "s_mov_b32 m0, %3\n\t"
                     "global_load_lds_dwordx4 %1, %2\n\t"
                     "s_mov_b32 m0, %0"
                     : "=&s"(saved)
                     : "v"(voff), "s"(gbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_void*)p; }

// Copy plan of one BC-row tile (row stride CPR 16-byte chunks) into LDS with
// global_load_lds_dwordx4.  Each wave instruction i fills the 64 consecutive
// 16-byte LDS slots starting at p0 = (wave*NI + i)*64; slot p holds row p/CPR,
// logical chunk (p % CPR) ^ f(row), so the lane that owns slot p fetches that
// chunk.  The per-lane byte offsets within a tile are fixed and computed once;
// per tile only the uniform base pointer moves.  In the last tile rows past
// the end are clamped to row N-1, so every load stays in bounds and padding
// keys (masked to -inf) carry finite data.
template <int BC, int CPR, int NW, int KIND, bool NT = false>
struct TilePlan {
    static constexpr int CH = BC * CPR;
    static constexpr int NI = CH / (64 * NW);
    static_assert(NI >= 1 && CH % (64 * NW) == 0, "tile too small for the workgroup");
    uint32_t off[NI];   // byte offset of this lane's chunk, relative to the tile's row 0
    int row[NI];        // tile row this lane fetches

    __device__ __forceinline__ void init(int wave, int lane)
    {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int p = (wave * NI + i) * 64 + lane;
            const int r = p / CPR, pc = p % CPR;
            const int c = (KIND == 0) ? swz_k<CPR>(r, pc) : (KIND == 1) ? swz_v16<CPR>(r, pc)
                        : (KIND == 3) ? swz_kt<CPR>(r, pc) : swz_v32(r, pc);
            row[i] = r;
            off[i] = (uint32_t)(r * CPR + c) * 16u;
        }
    }

    template <typename T>
    __device__ __forceinline__ void issue(u32x4* lds_tile, const T* g, int k0, int N, int wave) const
    {
        const uint64_t gb = uniform_ptr(g + (size_t)k0 * (CPR * 8));
        const uint32_t lb = lds_addr(lds_tile);
#ifdef ATTN_LDS_POISON
        // Debug build: NaN into exactly the slots these copies fill, written
        // after the wait that freed them and before the copies are issued.  A
        // read that is not ordered after the copies' completion (a missing
        // wait or barrier) then sees NaN instead of the previous tile's data.
        {
            typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
            const uint32_t lane = (uint32_t)(threadIdx.x & 63);
#pragma unroll
            for (int i = 0; i < NI; ++i)
                *(lds_u32x4*)(uintptr_t)(lb + (uint32_t)(((wave * NI + i) * 64) * 16) + lane * 16u) =
                    (u32x4){0x7fc00000u, 0x7fc00000u, 0x7fc00000u, 0x7fc00000u};
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
#endif
        if (k0 + BC <= N) {
#pragma unroll
            for (int i = 0; i < NI; ++i) lds_dma16<NT>(gb, off[i], lb + (uint32_t)((wave * NI + i) * 64 * 16));
        } else {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int over = max(k0 + row[i] - (N - 1), 0);     // rows past N-1 -> N-1
                lds_dma16<NT>(gb, off[i] - (uint32_t)(over * CPR * 16), lb + (uint32_t)((wave * NI + i) * 64 * 16));
            }
        }
    }
};

template <typename T> struct Dot2;
template <> struct Dot2<__bf16> {
    typedef __attribute__((ext_vector_type(2))) __bf16 v2;
    static __device__ __forceinline__ float sum2(v2 a, float acc)
    { return __builtin_amdgcn_fdot2_f32_bf16(a, (v2){(__bf16)1.0f, (__bf16)1.0f}, acc, false); }
};
template <> struct Dot2<_Float16> {
    typedef __attribute__((ext_vector_type(2))) _Float16 v2;
    static __device__ __forceinline__ float sum2(v2 a, float acc)
    { return __builtin_amdgcn_fdot2(a, (v2){(_Float16)1.0f, (_Float16)1.0f}, acc, false); }
};

// Block-sparse walk (the tutorial names a block-sparse extension of
// FlashAttention without giving it; here the pair (i, j) is attended only if
// the flag of block (i / blk, j / blk) of its head is non-zero, on top of
// causality and key padding).  A workgroup visits, in ascending order, only
// the key tiles in which some row block of the workgroup attends some key
// block: tiles without an attended pair are neither copied nor computed.
// Flags are read 64 tiles at a time, one tile per lane, and reduced with a
// ballot: `act` bit j = tile base + j has an attended block for the
// workgroup; own[kb] bit j = this wave's row block attends the key block of
// 32-key sub-block kb of tile base + j.  The words come from ballots, so they
// are wave-uniform, and every wave of the workgroup derives the same `act`:
// all waves visit the same tiles and meet the same barriers.
template <int BR, int BC>
struct BlockScan {
    static constexpr int NKB = BC / 32;
    const uint8_t* flags;   // this head's [nb][nb] block flags
    int nb, blk, N, kt_end, qb_lo, qb_hi, qb_w;
    int base = -64;         // first tile of the loaded words
    uint64_t act = 0;
    uint64_t own[NKB];

    __device__ __forceinline__ void init(const FwdParams& p, int bh, int q0, int wave_q0, int kt_end_)
    {
        nb = p.nb;
        blk = p.blk;
        N = p.N;
        kt_end = kt_end_;
        flags = p.bmask + (size_t)bh * nb * nb;
        qb_lo = q0 / blk;
        qb_hi = (min(q0 + BR, N) - 1) / blk;
        qb_w = min(wave_q0, N - 1) / blk;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) own[kb] = 0;
    }

    __device__ __forceinline__ void load(int b0, int lane)
    {
        const int t = b0 + lane;
        bool any = false;
        bool w[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) w[kb] = false;
        if (t < kt_end) {
            const int k0 = t * BC;            // < N: t < kt_end
            const int kb_lo = k0 / blk, kb_hi = (min(k0 + BC, N) - 1) / blk;
            // every flag load issued at once (a short-circuit || would issue
            // them one after another, each waiting for the previous)
            for (int qb = qb_lo; qb <= qb_hi; ++qb)
                for (int kbl = kb_lo; kbl <= kb_hi; ++kbl) any |= flags[(size_t)qb * nb + kbl] != 0;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int key = k0 + 32 * kb;
                w[kb] = key < N && flags[(size_t)qb_w * nb + key / blk] != 0;
            }
        }
        act = __builtin_amdgcn_ballot_w64(any);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) own[kb] = __builtin_amdgcn_ballot_w64(w[kb]);
        base = b0;
    }

    // first tile >= from with an attended block, or kt_end
    __device__ __forceinline__ int next(int from, int lane)
    {
        while (from < kt_end) {
            const int b0 = from & ~63;
            if (b0 != base) load(b0, lane);
            const uint64_t w = act & (~0ull << (from - b0));
            if (w) return b0 + (int)__builtin_ctzll(w);
            from = b0 + 64;
        }
        return kt_end;
    }

    // sub-block flags (bit kb) of the wave for tile t, t in the loaded words
    __device__ __forceinline__ unsigned bits(int t) const
    {
        unsigned r = 0;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) r |= (unsigned)((own[kb] >> (t - base)) & 1u) << kb;
        return r;
    }
};

// Waves per SIMD the 16-bit kernel is register-budgeted for: two for the
// tiles whose state fits in 256 registers, one otherwise.
template <int D, int BC> struct H16Occ { static constexpr int value = (D * BC <= 128 * 64) ? 2 : 1; };

// MASKED: the instance for calls with a key-padding mask (dense walk only).
// Without one the padding test is compiled out; with one, the lane's padding
// flags of the next key tile are loaded one tile ahead (32-bit words of four
// flags), so that their latency hides behind a whole tile.
template <typename T, int D, int BR, int BC, bool SPARSE, bool MASKED = false>
__global__ void __launch_bounds__(BR * 2) __attribute__((amdgpu_waves_per_eu(H16Occ<D, BC>::value)))
fwd_m32_h16(FwdParams p)
{
    using TR = H16<T>;
    using v8 = typename TR::v8;
    using v2 = typename Dot2<T>::v2;
    constexpr int NW = BR / 32;
    constexpr int CPR = D * 2 / 16;            // 16-byte chunks per row
    constexpr int NKB = BC / 32, DK = D / 16, DB = D / 32, KS = BC / 16;
    using KPlan = TilePlan<BC, CPR, NW, 0>;
    using VPlan = TilePlan<BC, CPR, NW, 1>;
    static_assert(BR % 32 == 0 && BC % 32 == 0 && (D == 64 || D == 128), "tile");

    // two K/V tile buffers in LDS: the copy of tile it+1 is in flight while
    // tile it is computed
    __shared__ u32x4 sk[2][BC * CPR];
    __shared__ u32x4 sv[2][BC * CPR];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // wave-uniform
    const int hh = lane >> 5, col = lane & 31;
    // Units: one per workgroup, or the items of a persistent schedule (this
    // instance only).  A persistent workgroup copies the next unit's first K
    // and V tiles while it stores the current unit's output.
    constexpr bool PERSIST_OK = !SPARSE && !MASKED && D == 128 && BR == 256 && BC == 64;
    UnitSched sched;
    int bh, qt;
    if (PERSIST_OK && p.persist > 0) {
        sched.init(p);
        if (!sched.get(bh, qt)) return;
    } else {
        tile_of_block(p, bh, qt);
    }
    bool prefetched = false;
    for (;;) {
    const int N = p.N;
    const int b = bh / p.H;
    const int q0 = qt * BR;
    const size_t head = (size_t)bh * (size_t)N * D;
    const T* __restrict__ Q = (const T*)p.q + head;
    const T* __restrict__ K = (const T*)p.k + head;
    const T* __restrict__ V = (const T*)p.v + head;
    const int qi = q0 + wave * 32 + col;       // this lane's query row

    const int nkt = (N + BC - 1) / BC;
    int kt_end = nkt;
    if (p.causal) kt_end = min(nkt, (min(q0 + BR, N) - 1) / BC + 1);
    const int order = p.kv_order;
    auto tile_at = [&](int it) { return order ? (kt_end - 1 - it) : it; };

    // Q^T operand: lane holds Q[qi][16*ks + 8*hh + 0..7].  Block-sparse calls
    // load it before the flag scan (whose loads it then shares a round trip
    // with); dense calls after issuing the first K/V copies.
    u32x4 qw[DK];
    const int qrow = min(qi, N - 1);
    auto load_q = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < DK; ++ks)
            qw[ks] = q_mode16(*(const u32x4*)(Q + (size_t)qrow * D + ks * 16 + hh * 8), p.qmode);
    };

    // block-sparse: first tile with an attended block (kt_end if none)
    BlockScan<BR, BC> scan;
    int t0 = tile_at(0);
    if constexpr (SPARSE) {
        load_q();
        scan.init(p, bh, q0, q0 + wave * 32, kt_end);
        t0 = scan.next(0, lane);
    }

    // prologue: first K and V tiles in flight before Q is even loaded
    KPlan kplan;
    VPlan vplan;
    kplan.init(wave, lane);
    vplan.init(wave, lane);
    if ((!SPARSE || t0 < kt_end) && !prefetched) {
        kplan.issue(sk[0], K, t0 * BC, N, wave);
        vplan.issue(sv[0], V, t0 * BC, N, wave);
    }

    // The empty asm consumes Q here, so the compiler's wait for its loads sits
    // before the loop and not inside it (where it would also drain the tile
    // prefetches).
    if constexpr (!SPARSE) load_q();
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) asm volatile("" : "+v"(qw[ks]));
    v8 qf[DK];
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) qf[ks] = __builtin_bit_cast(v8, qw[ks]);

    float m = -INFINITY;       // reference of the merge (raw q.k units), see ref_step
    float l = 0.f;             // this lane's share of the running sum
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = (f32x16){};

    const int wave_q0 = q0 + wave * 32;
    const float c = p.c;

    // padding flags (MASKED): word (kb, g4) holds the flags of keys
    // k0 + 32*kb + 8*g4 + 4*hh + 0..3 in its four bytes; padw for the current
    // tile, padn for the next one.  A word is one 32-bit load when the mask row
    // is 4-byte aligned and the four keys lie inside the row, else four byte
    // loads at clamped keys (flags of keys past N are never used).
    static_assert(!(MASKED && SPARSE), "the block-sparse walk reads the mask in place");
    const uint8_t* const prow = MASKED ? p.mask + (size_t)b * N : nullptr;
    const bool pvec = MASKED && ((uintptr_t)prow & 3u) == 0;
    uint32_t padw[MASKED ? NKB : 1][4], padn[MASKED ? NKB : 1][4];
    auto load_pad = [&](int k1) __attribute__((always_inline)) {
        if constexpr (MASKED) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int kbase = k1 + kb * 32 + 8 * g4 + 4 * hh;
                    uint32_t w = 0;
                    if (pvec && kbase + 3 < N) {
                        w = *(const uint32_t*)(prow + kbase);
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) w |= (uint32_t)prow[min(kbase + r, N - 1)] << (8 * r);
                    }
                    padn[kb][g4] = w;
                }
        }
    };
    if constexpr (MASKED) load_pad(tile_at(0) * BC);
    const int g = (lane >> 4) & 1, rsrc = (lane & 15) >> 2, qsrc = lane & 3;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    // Per-lane LDS byte addresses of the operand reads in buffer 0: K rows
    // 32 kb + col at chunk 2 ks + hh, and the V^T pairs of rows 16 ks2 + 4 hh +
    // rsrc (+ 8) at head column block db.  Both swizzles depend only on a row's
    // position within its 16-row group, so the buffer, the key block kb and the
    // key step ks2 only add constants.
    constexpr uint32_t TILE_B = BC * CPR * 16;
    uint32_t kaddr[DK], vaddr[DB];
#pragma unroll
    for (int ks = 0; ks < DK; ++ks)
        kaddr[ks] = lds_addr(sk[0]) + (uint32_t)((col * CPR + swz_k<CPR>(col, ks * 2 + hh)) * 16);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int r = 4 * hh + rsrc;
        vaddr[db] = lds_addr(sv[0]) +
                    (uint32_t)((r * CPR + swz_v16<CPR>(r, db * 4 + 2 * g + (qsrc >> 1))) * 16 + (qsrc & 1) * 8);
    }

    // One key tile: the it-th of the fold order (dense), or the tile starting
    // at key sk0 followed by the one at sk0next (-1: none) with the wave's
    // sub-block flags `sub` (block-sparse).  BUF (the buffer the tile lives
    // in, alternating) is a compile-time constant: the loops below are
    // unrolled by two, so every LDS address is a fixed register plus an
    // immediate offset.
    auto body = [&](auto BUF, int it, int sk0, int sk0next, unsigned sub) {
        constexpr int buf = decltype(BUF)::value;
        const int k0 = SPARSE ? sk0 : tile_at(it) * BC;

        // this tile landed; every wave is done with the previous one, so the
        // other buffer can be refilled with the next tile
        wait_vmcnt<0>();
        wg_barrier();
        if constexpr (SPARSE) {
            if (sk0next >= 0) {
                kplan.issue(sk[buf ^ 1], K, sk0next, N, wave);
                vplan.issue(sv[buf ^ 1], V, sk0next, N, wave);
            }
            if (sub == 0) return;   // no attended pair for this wave's rows
        } else if (it + 1 < kt_end) {
            kplan.issue(sk[buf ^ 1], K, tile_at(it + 1) * BC, N, wave);
            vplan.issue(sv[buf ^ 1], V, tile_at(it + 1) * BC, N, wave);
        }
        bool pad_any = false;     // MASKED: some key of the tile is padded
        if constexpr (MASKED) {
            // this tile's flags arrived with the wait above; fetch the next
            // tile's
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) padw[kb][g4] = padn[kb][g4];
            if (it + 1 < kt_end) load_pad(tile_at(it + 1) * BC);
            // the two wave halves hold all the tile's keys: a tile without a
            // padded key takes the unmasked path, a tile with every key padded
            // has nothing for this wave (flags past N repeat key N-1's)
            uint32_t any = 0, zero = 0;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const uint32_t w = padw[kb][g4];
                    any |= w;
                    zero |= (w - 0x01010101u) & ~w & 0x80808080u;   // high bit of every zero byte
                }
            pad_any = __builtin_amdgcn_ballot_w64(any != 0) != 0;
            if (__builtin_amdgcn_ballot_w64(zero != 0) == 0) return;
        }
        // causal: every key of the tile comes after every row of the wave, so
        // the wave has nothing to add (it took part in the copy above)
        if (p.causal && k0 > wave_q0 + 31) return;

        // S^T = K Q^T : 32 keys x 32 queries per block
        f32x16 s[NKB];
        auto scores = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                s[kb] = (f32x16){};
#pragma unroll
                for (int ks = 0; ks < DK; ++ks) {
                    const u32x4 kv =
                        *(const lds_u32x4*)(uintptr_t)(kaddr[ks] + buf * TILE_B + kb * (32 * CPR * 16));
                    s[kb] = TR::mma32(__builtin_bit_cast(v8, kv), qf[ks], s[kb]);
                }
            }
        };

        // masking -> -inf.  Accumulator element (kb, j) of this lane is key
        // k0 + 32*kb + 8*(j/4) + 4*hh + j%4.  The score products are issued
        // inside each masking case, so that every case leaves its scores in
        // the registers the products wrote: issued once before the cases, the
        // compiler copied the whole tile to other registers where the cases
        // join (3-6% slower at d = 64; the results are bitwise the same).
        const bool diag = p.causal && k0 + BC - 1 > wave_q0;
        const bool tail = k0 + BC > N;
        // block-sparse: some 32-key sub-block of the tile not attended by the
        // wave's rows (never with tiles no wider than a block)
        const bool part = SPARSE && sub != (1u << NKB) - 1u;
        if (tail || (MASKED ? pad_any : p.mask != nullptr) || part) {
            scores();
            // ragged last tile, key padding or partly attended tile: full
            // visibility test (the MASKED instance has the padding flags in
            // padw; the others read them in place, which only the block-sparse
            // walk does: dense calls with a mask go to the MASKED instance)
            const uint8_t* mrow = (!MASKED && p.mask) ? p.mask + (size_t)b * N : nullptr;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const bool on = !SPARSE || ((sub >> kb) & 1u);
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = k0 + kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
                    bool vis = on && key < N && (!p.causal || key <= qi);
                    if constexpr (MASKED) vis = vis && ((padw[kb][j >> 2] >> (8 * (j & 3))) & 0xffu) == 0;
                    if (mrow) vis = vis && mrow[min(key, N - 1)] == 0;
                    if (!vis) s[kb][j] = -INFINITY;
                }
            }
        } else if (diag) {
            scores();
            // tile crossing the causal diagonal: key <= qi, one compare and
            // one select per element against a per-lane limit
            const int lim = qi - k0 - 4 * hh;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (kb * 32 + 8 * (j >> 2) + (j & 3) > lim) s[kb][j] = -INFINITY;
        } else {
            scores();
        }

        // tile maximum and reference step; the O rescale is skipped when no
        // row of the wave moved its reference (alpha == 1 exactly)
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) mt = fmaxf(mt, s[kb][j]);
        mt = xhalf_max(mt);
        const RefStep rs = ref_step(m, mt, c, p.slack);
        m = rs.m;
        l *= rs.alpha;
        if (__builtin_amdgcn_ballot_w64(rs.moved)) {
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] *= rs.alpha;
        }
        const float mc = rs.mc;

        // P = exp2(s*c - m*c) rounded to T; the rounded values feed both P.V
        // and the running sum (v_dot2 with (1, 1)), so the output is an exact
        // convex combination of value rows.
        v8 pb[KS];
#pragma unroll
        for (int ks2 = 0; ks2 < KS; ++ks2) {
            const int kb = ks2 >> 1, half = ks2 & 1;
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const float x0 = fast_exp2(fmaf(s[kb][8 * half + i], c, -mc));
                const float x1 = fast_exp2(fmaf(s[kb][8 * half + i + 1], c, -mc));
                const v2 pr = (v2){(T)x0, (T)x1};
                pb[ks2][i] = pr[0];
                pb[ks2][i + 1] = pr[1];
                l = Dot2<T>::sum2(pr, l);
            }
        }

        // O^T += V^T P^T; V^T operand: keys 16*ks2 + {4*hh + r, 8 + 4*hh + r}, d = 32*db + col
#pragma unroll
        for (int ks2 = 0; ks2 < KS; ++ks2) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const uint32_t a1 = vaddr[db] + buf * TILE_B + ks2 * (16 * CPR * 16);
                const uint32_t a2 = a1 + 8 * CPR * 16;
                const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a1);
                const i16x4 t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)a2);
                const u32x2 w1 = __builtin_bit_cast(u32x2, t1), w2 = __builtin_bit_cast(u32x2, t2);
                const u32x4 w = (u32x4){w1[0], w1[1], w2[0], w2[1]};
                o[db] = TR::mma32(__builtin_bit_cast(v8, w), pb[ks2], o[db]);
            }
        }
    };

    // Steady state (16-bit, d = 128, 256 x 64, ascending order, the exact or
    // the lagging reference): the key tiles that are full and need no mask
    // for any row of the workgroup run through the software pipeline of
    // fwd_pipe_asm.h (the score products of tile t+1 beside the softmax of
    // tile t, then P.V of tile t beside the maximum of tile t+1).  It does this body's operations
    // in this body's order per row.  It consumes the K/V copies issued above
    // and leaves the next tile's copies in flight in the buffers the loop
    // below expects (an even count of tiles), with m, l and o updated.
    int it_first = 0;
    if constexpr (!SPARSE && !MASKED && D == 128 && BR == 256 && BC == 64) {
        int n_st = p.causal ? (q0 + 1) / BC : N / BC;
        n_st = min(min(n_st, N / BC), kt_end) & ~1;
        if (p.pipe && order == 0 && n_st >= 2) {
            const uint32_t skb = lds_addr(sk[0]), svb = lds_addr(sv[0]);
            const uint32_t* ka = kaddr;
            const uint32_t* va = vaddr;
            constexpr uint32_t TB = BC * CPR * 16;       // bytes of one K or V tile
            uint32_t ko0 = kplan.off[0] + TB, ko1 = kplan.off[1] + TB;
            uint32_t vo0 = vplan.off[0] + TB, vo1 = vplan.off[1] + TB;
            const uint32_t kdst = __builtin_amdgcn_readfirstlane(skb + (uint32_t)(wave * 2 * 1024));
            const uint32_t vdst = __builtin_amdgcn_readfirstlane(svb + (uint32_t)(wave * 2 * 1024));
            const uint64_t kbase = uniform_ptr(K), vbase = uniform_ptr(V);
            uint32_t pairs = __builtin_amdgcn_readfirstlane((uint32_t)(n_st - 2) / 2);
            // the block copies the first tile after it (into buffer 0) only if
            // that tile is full: it does not clamp rows to the head's end
            const bool next_full = n_st < kt_end && (n_st + 1) * BC <= N;
            const uint32_t has_next = __builtin_amdgcn_readfirstlane(next_full ? 1u : 0u);
            uint64_t moved;
            uint32_t m0save;
            const float slack = p.slack;
            static_assert(KPlan::NI == 2 && VPlan::NI == 2, "pipeline copy plan");
            if constexpr (std::is_same<T, __bf16>::value)
                asm volatile(ATTN_PIPE_ASM_BF16 ATTN_PIPE_OPERANDS);
            else
                asm volatile(ATTN_PIPE_ASM_F16 ATTN_PIPE_OPERANDS);
            // rebuild the copy plans instead of keeping them live across the
            // block (the opaque wave copy stops the compiler from reusing the
            // values computed before it)
            int wv = wave;
            asm volatile("" : "+s"(wv));
            kplan.init(wv, lane);
            vplan.init(wv, lane);
            if (n_st < kt_end && !next_full) {
                // ragged tile next: copied here with rows clamped to N - 1; the
                // block's last barrier has released both buffers 0
                kplan.issue(sk[0], K, n_st * BC, N, wave);
                vplan.issue(sv[0], V, n_st * BC, N, wave);
            }
            it_first = n_st;
        }
    }

    if constexpr (SPARSE) {
        int t = t0;
        while (t < kt_end) {
            const unsigned st = scan.bits(t);
            const int t1 = scan.next(t + 1, lane);
            body(Int<0>{}, 0, t * BC, t1 < kt_end ? t1 * BC : -1, st);
            if (t1 >= kt_end) break;
            const unsigned st1 = scan.bits(t1);
            t = scan.next(t1 + 1, lane);
            body(Int<1>{}, 0, t1 * BC, t < kt_end ? t * BC : -1, st1);
        }
    } else {
        for (int it = it_first; it < kt_end; it += 2) {
            body(Int<0>{}, it, 0, 0, 0u);
            if (it + 1 < kt_end) body(Int<1>{}, it + 1, 0, 0, 0u);
        }
    }

    // persistent: the next unit's first K/V tiles are copied while this unit's
    // output is normalised and stored (every wave is done with the LDS buffers
    // after the barrier)
    int nbh = 0, nqt = 0;
    bool more = false;
    if constexpr (PERSIST_OK) {
        if (p.persist > 0) {
            sched.advance();
            more = sched.get(nbh, nqt);
            if (more) {
                const size_t nhead = (size_t)nbh * (size_t)N * D;
                wg_barrier();
                kplan.issue(sk[0], (const T*)p.k + nhead, 0, N, wave);
                vplan.issue(sv[0], (const T*)p.v + nhead, 0, N, wave);
            }
        }
    }

    // epilogue: O = acc / l, lse = m*scale + ln(l); empty rows -> (0, -inf)
    const float lt = xhalf_sum(l);
    if (qi < N) {
        const size_t orow = (size_t)bh * N + qi;
        const bool empty = !(lt > 0.f);
        const float inv = empty ? 0.f : 1.f / lt;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = db * 32 + 8 * g4 + 4 * hh;
                float x[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] = empty ? 0.f : o[db][4 * g4 + r] * inv;
                if (p.out_f32) {
                    *(f32x4*)((float*)p.o + orow * D + d0) = (f32x4){x[0], x[1], x[2], x[3]};
                } else {
                    typedef __attribute__((ext_vector_type(4))) T t4;
                    *(t4*)((T*)p.o + orow * D + d0) = (t4){(T)x[0], (T)x[1], (T)x[2], (T)x[3]};
                }
            }
        }
        if (p.lse && hh == 0)
            p.lse[orow] = empty ? -INFINITY : fmaf(m, p.scale, __builtin_amdgcn_logf(lt) * 0.69314718055994530942f);
    }
    if (!more) break;
    bh = nbh;
    qt = nqt;
    prefetched = true;
    }   // units
}

// ============================================================ fp32, 32x32x2
template <int D, int BR, int BC>
__global__ void __launch_bounds__(BR * 2)
fwd_m32_f32(FwdParams p)
{
    constexpr int NW = BR / 32, NT = NW * 64;
    constexpr int CPR = D * 4 / 16;
    constexpr int NKB = BC / 32, DB = D / 32, DH = D / 2, DC = D / 8;
    static_assert(BR % 32 == 0 && BC % 32 == 0 && (D == 64 || D == 128), "tile");

    __shared__ u32x4 sk[BC * CPR];
    __shared__ u32x4 sv[BC * CPR];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, col = lane & 31;
    int bh, qt;
    tile_of_block(p, bh, qt);
    const int N = p.N;
    const int b = bh / p.H;
    const int q0 = qt * BR;
    const size_t head = (size_t)bh * (size_t)N * D;
    const float* __restrict__ Q = (const float*)p.q + head;
    const float* __restrict__ K = (const float*)p.k + head;
    const float* __restrict__ V = (const float*)p.v + head;
    const int qi = q0 + wave * 32 + col;

    // Q^T operand of 32x32x2: step t uses d = t + (D/2)*hh
    float qf[DH];
#pragma unroll
    for (int t = 0; t < DC; ++t) {
        f32x4 w = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (qi < N) w = *(const f32x4*)(Q + (size_t)qi * D + 4 * t + DH * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[4 * t + e] = q_mode32(w[e], p.qmode);
    }

    float m = -INFINITY, l = 0.f;
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = (f32x16){};

    const int nkt = (N + BC - 1) / BC;
    int kt_end = nkt;
    if (p.causal) {
        const int last_q = min(q0 + BR, N) - 1;
        kt_end = min(nkt, last_q / BC + 1);
    }
    const int wave_q0 = q0 + wave * 32;
    const float c = p.c;
    const float* svf = (const float*)sv;
    // key-padding flags: word (kb, g4) holds keys k0 + 32 kb + 8 g4 + 4 hh + 0..3
    const uint8_t* const prow = p.mask ? p.mask + (size_t)b * N : nullptr;
    const bool pvec = prow && ((uintptr_t)prow & 3u) == 0;
    uint32_t padw[NKB * 4];

    for (int it = 0; it < kt_end; ++it) {
        const int kt = p.kv_order ? (kt_end - 1 - it) : it;
        const int k0 = kt * BC;
        const int rows_valid = min(BC, N - k0);
        // the flags load while the tile is staged
        if (prow) {
#pragma unroll
            for (int w = 0; w < NKB * 4; ++w) padw[w] = pad_word(prow, pvec, k0 + (w >> 2) * 32 + 8 * (w & 3) + 4 * hh, N);
        }
        __syncthreads();
        stage_tile<BC, CPR, NT, 0>(sk, (const u32x4*)(K + (size_t)k0 * D), rows_valid, tid);
        stage_tile<BC, CPR, NT, 2>(sv, (const u32x4*)(V + (size_t)k0 * D), rows_valid, tid);
        __syncthreads();
        // causal: every key of the tile comes after every row of the wave
        // (the wave took part in the staging and both barriers)
        if (p.causal && k0 > wave_q0 + 31) continue;
        // padding: only tiles with a padded key take the masked path, and a
        // tile whose keys are all padded adds nothing
        bool pad_any = false, pad_all = false;
        if (prow) {
            pad_tile(padw, pad_any, pad_all);
            if (pad_all) continue;
        }

        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = (f32x16){};
            const int r = kb * 32 + col;
#pragma unroll
            for (int t = 0; t < DC; ++t) {
                const f32x4 kv = __builtin_bit_cast(f32x4, sk[r * CPR + swz_k<CPR>(r, t + DC * hh)]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[e], qf[4 * t + e], s[kb], 0, 0, 0);
            }
        }

        const bool need_mask = (p.causal && k0 + BC - 1 > wave_q0) || (k0 + BC > N) || pad_any;
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = k0 + kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
                    bool vis = key < N;
                    if (p.causal) vis = vis && key <= qi;
                    if (pad_any) vis = vis && unpadded(padw[kb * 4 + (j >> 2)], j & 3);
                    if (!vis) s[kb][j] = -INFINITY;
                }
            }
        }

        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) mt = fmaxf(mt, s[kb][j]);
        mt = xhalf_max(mt);
        const RefStep rs = ref_step(m, mt, c, p.slack);
        m = rs.m;
        l *= rs.alpha;
        if (__builtin_amdgcn_ballot_w64(rs.moved)) {
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] *= rs.alpha;
        }
        const float mc = rs.mc;

#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                s[kb][j] = fast_exp2(fmaf(s[kb][j], c, -mc));
                l += s[kb][j];
            }
            // O^T += V^T P^T, two keys per step: lane hh supplies key 8g+4hh+r
#pragma unroll
            for (int g = 0; g < 4; ++g) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = kb * 32 + 8 * g + 4 * hh + r;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const int dcol = db * 32 + col;
                        const float a = svf[(row * CPR + swz_v32(row, dcol >> 2)) * 4 + (dcol & 3)];
                        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kb][4 * g + r], o[db], 0, 0, 0);
                    }
                }
            }
        }
    }

    const float lt = xhalf_sum(l);
    if (qi < N) {
        const size_t orow = (size_t)bh * N + qi;
        const bool empty = !(lt > 0.f);
        const float inv = empty ? 0.f : 1.f / lt;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = db * 32 + 8 * g4 + 4 * hh;
                f32x4 x;
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] = empty ? 0.f : o[db][4 * g4 + r] * inv;
                *(f32x4*)((float*)p.o + orow * D + d0) = x;
            }
        }
        if (p.lse && hh == 0)
            p.lse[orow] = empty ? -INFINITY : fmaf(m, p.scale, __builtin_amdgcn_logf(lt) * 0.69314718055994530942f);
    }
}

// fp32 forward with the 16-bit kernel's staging: K and V tiles copied HBM ->
// LDS by DMA into two buffers, the copy of tile t+1 in flight while tile t is
// computed, one workgroup barrier per tile.  Used where two buffers of both
// tiles fit in LDS; the arithmetic is that of fwd_m32_f32.
template <int D, int BR, int BC>
__global__ void __launch_bounds__(BR * 2)
fwd_m32_f32_db(FwdParams p)
{
    constexpr int NW = BR / 32;
    constexpr int CPR = D * 4 / 16;
    constexpr int NKB = BC / 32, DB = D / 32, DH = D / 2, DC = D / 8;
    using KPlan = TilePlan<BC, CPR, NW, 0>;
    using VPlan = TilePlan<BC, CPR, NW, 2>;
    static_assert(BR % 32 == 0 && BC % 32 == 0 && (D == 64 || D == 128), "tile");

    __shared__ u32x4 sk[2][BC * CPR];
    __shared__ u32x4 sv[2][BC * CPR];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int hh = lane >> 5, col = lane & 31;
    int bh, qt;
    tile_of_block(p, bh, qt);
    const int N = p.N;
    const int b = bh / p.H;
    const int q0 = qt * BR;
    const size_t head = (size_t)bh * (size_t)N * D;
    const float* __restrict__ Q = (const float*)p.q + head;
    // the copy plans count rows in 2-byte units: one row is CPR * 8 of them
    const uint16_t* __restrict__ K = (const uint16_t*)((const float*)p.k + head);
    const uint16_t* __restrict__ V = (const uint16_t*)((const float*)p.v + head);
    const int qi = q0 + wave * 32 + col;
    const int wave_q0 = q0 + wave * 32;

    const int nkt = (N + BC - 1) / BC;
    int kt_end = nkt;
    if (p.causal) kt_end = min(nkt, (min(q0 + BR, N) - 1) / BC + 1);
    const int order = p.kv_order;
    auto tile_at = [&](int it) { return order ? (kt_end - 1 - it) : it; };

    KPlan kplan;
    VPlan vplan;
    kplan.init(wave, lane);
    vplan.init(wave, lane);
    kplan.issue(sk[0], K, tile_at(0) * BC, N, wave);
    vplan.issue(sv[0], V, tile_at(0) * BC, N, wave);

    // Q^T operand of 32x32x2: step t uses d = t + (D/2)*hh
    float qf[DH];
#pragma unroll
    for (int t = 0; t < DC; ++t) {
        f32x4 w = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (qi < N) w = *(const f32x4*)(Q + (size_t)qi * D + 4 * t + DH * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[4 * t + e] = q_mode32(w[e], p.qmode);
    }

    float m = -INFINITY, l = 0.f;
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = (f32x16){};
    const float c = p.c;

    // key-padding flags: word (kb, g4) holds keys k0 + 32 kb + 8 g4 + 4 hh +
    // 0..3; padw for the current tile, padn for the next one
    const uint8_t* const prow = p.mask ? p.mask + (size_t)b * N : nullptr;
    const bool pvec = prow && ((uintptr_t)prow & 3u) == 0;
    uint32_t padw[NKB * 4], padn[NKB * 4];
    auto load_pad = [&](int k1) __attribute__((always_inline)) {
#pragma unroll
        for (int w = 0; w < NKB * 4; ++w) padn[w] = pad_word(prow, pvec, k1 + (w >> 2) * 32 + 8 * (w & 3) + 4 * hh, N);
    };
    if (prow) load_pad(tile_at(0) * BC);

    auto body = [&](auto BUF, int it) __attribute__((always_inline)) {
        constexpr int buf = decltype(BUF)::value;
        const int k0 = tile_at(it) * BC;
        // this tile landed; every wave is done with the previous one, so the
        // other buffer can be refilled with the next tile
        wait_vmcnt<0>();
        wg_barrier();
        if (it + 1 < kt_end) {
            kplan.issue(sk[buf ^ 1], K, tile_at(it + 1) * BC, N, wave);
            vplan.issue(sv[buf ^ 1], V, tile_at(it + 1) * BC, N, wave);
        }
        // this tile's flags arrived with the wait above; fetch the next tile's
        bool pad_any = false, pad_all = false;
        if (prow) {
#pragma unroll
            for (int w = 0; w < NKB * 4; ++w) padw[w] = padn[w];
            if (it + 1 < kt_end) load_pad(tile_at(it + 1) * BC);
            pad_tile(padw, pad_any, pad_all);
        }
        // causal: every key of the tile comes after every row of the wave;
        // padding: every key of the tile padded
        if ((p.causal && k0 > wave_q0 + 31) || pad_all) return;

        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = (f32x16){};
            const int r = kb * 32 + col;
#pragma unroll
            for (int t = 0; t < DC; ++t) {
                const f32x4 kv = __builtin_bit_cast(f32x4, sk[buf][r * CPR + swz_k<CPR>(r, t + DC * hh)]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[e], qf[4 * t + e], s[kb], 0, 0, 0);
            }
        }

        // invisible scores -> -inf; element (kb, j) is key k0 + 32*kb + 8*(j/4) + 4*hh + j%4.
        // Rows of the ragged last tile past N hold row N-1's data (finite).
        const bool need_mask = (p.causal && k0 + BC - 1 > wave_q0) || (k0 + BC > N) || pad_any;
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = k0 + kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
                    bool vis = key < N;
                    if (p.causal) vis = vis && key <= qi;
                    if (pad_any) vis = vis && unpadded(padw[kb * 4 + (j >> 2)], j & 3);
                    if (!vis) s[kb][j] = -INFINITY;
                }
            }
        }

        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) mt = fmaxf(mt, s[kb][j]);
        mt = xhalf_max(mt);
        const RefStep rs = ref_step(m, mt, c, p.slack);
        m = rs.m;
        l *= rs.alpha;
        if (__builtin_amdgcn_ballot_w64(rs.moved)) {
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] *= rs.alpha;
        }
        const float mc = rs.mc;

        const float* svf = (const float*)sv[buf];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                s[kb][j] = fast_exp2(fmaf(s[kb][j], c, -mc));
                l += s[kb][j];
            }
            // O^T += V^T P^T, two keys per step: lane hh supplies key 8g+4hh+r
#pragma unroll
            for (int g = 0; g < 4; ++g) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = kb * 32 + 8 * g + 4 * hh + r;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const int dcol = db * 32 + col;
                        const float a = svf[(row * CPR + swz_v32(row, dcol >> 2)) * 4 + (dcol & 3)];
                        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kb][4 * g + r], o[db], 0, 0, 0);
                    }
                }
            }
        }
    };
    for (int it = 0; it < kt_end; it += 2) {
        body(Int<0>{}, it);
        if (it + 1 < kt_end) body(Int<1>{}, it + 1);
    }

    const float lt = xhalf_sum(l);
    if (qi < N) {
        const size_t orow = (size_t)bh * N + qi;
        const bool empty = !(lt > 0.f);
        const float inv = empty ? 0.f : 1.f / lt;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = db * 32 + 8 * g4 + 4 * hh;
                f32x4 x;
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] = empty ? 0.f : o[db][4 * g4 + r] * inv;
                *(f32x4*)((float*)p.o + orow * D + d0) = x;
            }
        }
        if (p.lse && hh == 0)
            p.lse[orow] = empty ? -INFINITY : fmaf(m, p.scale, __builtin_amdgcn_logf(lt) * 0.69314718055994530942f);
    }
}

// ---------------------------------------------------------------- launchers
template <typename T, int D, int BR, int BC, bool SPARSE = false>
hipError_t launch_h16(const FwdParams& p, hipStream_t st)
{
    const unsigned grid = p.persist > 0 ? (unsigned)p.persist : (unsigned)(p.B * p.H * p.n_qt);
    if (!SPARSE && p.mask)
        hipLaunchKernelGGL((fwd_m32_h16<T, D, BR, BC, false, true>), dim3(grid), dim3(BR * 2), 0, st, p);
    else
        hipLaunchKernelGGL((fwd_m32_h16<T, D, BR, BC, SPARSE, false>), dim3(grid), dim3(BR * 2), 0, st, p);
    return hipGetLastError();
}

template <int D, int BR, int BC>
hipError_t launch_f32(const FwdParams& p, hipStream_t st)
{
    const unsigned grid = (unsigned)(p.B * p.H * p.n_qt);
    // two buffers of both tiles: 4 * BC rows of D fp32 values
    if constexpr (4 * BC * D * 4 <= 128 * 1024)
        hipLaunchKernelGGL((fwd_m32_f32_db<D, BR, BC>), dim3(grid), dim3(BR * 2), 0, st, p);
    else
        hipLaunchKernelGGL((fwd_m32_f32<D, BR, BC>), dim3(grid), dim3(BR * 2), 0, st, p);
    return hipGetLastError();
}

// Instance tables, one per input type (defined in the fwd_inst_*.hip files).
LaunchFn lookup_bf16(int D, int BR, int BC);
LaunchFn lookup_f16(int D, int BR, int BC);
LaunchFn lookup_f32(int D, int BR, int BC);
// Block-sparse 16-bit instances (bits: 0 bf16, 1 f16).
LaunchFn lookup_sparse(int dtype_bits, int D, int BR, int BC);

}  // namespace attnk
