// bwd.hip -- gradient of the attention forward w.r.t. q, k and v.
//
// The tutorial's checklist asks for numerical closeness of outputs and of
// gradients.  The gradient is recomputed tile by tile from the forward's
// log-sum-exp, the same way the forward never stores the N x N matrix: with
// P_ij = exp(scale q_i.k_j - lse_i) and D_i = sum_c dO_ic O_ic,
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,
//     dK = scale dS^T Q.
// Three kernels, no atomics (bitwise deterministic):
//   bwd_pre   D_i and lse_i * log2(e) per row (+inf for a row with no visible
//             key, so that its P is exactly 0);
//   bwd_dkdv  one workgroup per 32*NW keys (each wave owns 32 keys; K^T in
//             registers, V^T in LDS), looping over 64-query tiles of Q and dO
//             staged in LDS (one barrier per tile, computed as two 32-row
//             halves): S = Q K^T and dP = dO V^T put a key in each
//             lane's column, which is the A-operand layout of dV += P^T dO and
//             dK += dS^T Q (their dO and Q operands are transposing LDS reads);
//   bwd_dq    one workgroup per 32*NW queries (Q and dO in registers; under
//             causal masking the last, heaviest query tiles are issued first), looping
//             over 64-key tiles of K and V in LDS: S^T = K Q^T and
//             dP^T = V dO^T put a query in each lane's column, the B-operand
//             layout of dQ^T += K^T dS^T (K^T read transposed from LDS).
// Products run on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation; P and
// dS are rounded to the input type for the MFMA, as P is in the forward.
// Tiles read both row-wise and transposed (Q and dO here, K in bwd_dq) are
// stored with swz_kt, under which neither read has LDS bank conflicts.
// At d = 128 without a key-padding mask both gradient kernels first run their
// full tiles (every pair visible, nothing past N) through generated
// instruction-scheduled loops (bwd_dkdv_pipe_asm.h, bwd_dq_pipe_asm.h), which
// keep the per-element arithmetic and accumulation order of the loops here and
// copy their tiles in operand-ordered layouts; the loops here take the
// diagonal and ragged tiles.
#include <hip/hip_runtime.h>
#include "bwd.h"
#include "fwd_kernel.h"
#include "bwd_dq_pipe_asm.h"
#include "bwd_dkdv_pipe_asm.h"


namespace attnk {

// D_i and the base-2 lse of each row.  D/8 consecutive lanes share a row and
// read it with one 16-byte load each; the partial sums meet by xor-shuffles.
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_pre(BwdParams p)
{
    constexpr int LPR = D / 8;                        // lanes per row
    const size_t rows = (size_t)p.B * p.H * p.N;
    const size_t row = (size_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    typedef __attribute__((ext_vector_type(8))) T t8;
    float acc = 0.f;
    if (row < rows) {
        const t8 a = *((const t8*)((const T*)p.o + row * D) + part);
        const t8 b = *((const t8*)((const T*)p.dout + row * D) + part);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
    }
#pragma unroll
    for (int w = LPR / 2; w >= 1; w /= 2) acc += __shfl_xor(acc, w);
    if (row < rows && part == 0) {
        p.dsum[row] = -acc;     // minus D: the dP products of dK/dV accumulate onto it
        const float l = p.lse[row];
        p.lse2[row] = (l == -INFINITY) ? INFINITY : l * 1.4426950408889634f;
    }
}

// Transposing LDS reads of the 32x32x16 operand that holds, for lane
// (column c = lane % 32 of the 32-column block db, half hh = lane / 32),
// tile[rows 16*ks2 + 4*hh + 0..3 and + 8 .. + 11][32*db + c] of a row-major
// tile stored with the swz_kt chunk swizzle (every tile the backward reads
// transposed is also read row-wise; swz_kt serves both without conflicts).
// The swizzle's row term depends on the row within its 16-row group only, so
// the per-lane byte offsets of the two 8-byte reads are fixed for each db
// (TrOffsets, computed once) and 16*ks2 rows add an immediate.
template <int CPR, int DB>
struct TrOffsets {
    uint32_t off[2][DB];
    __device__ __forceinline__ void init(int lane)
    {
        const int hh = lane >> 5, g = (lane >> 4) & 1, rsrc = (lane & 15) >> 2, qsrc = lane & 3;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int row = 4 * hh + rsrc + 8 * t;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int chunk = db * 4 + 2 * g + (qsrc >> 1);
                off[t][db] = (uint32_t)((row * CPR + swz_kt<CPR>(row, chunk)) * 16 + (qsrc & 1) * 8);
            }
        }
    }
};

template <int CPR, int DB>
__device__ __forceinline__ u32x4 tr_operand(const void* tile, const TrOffsets<CPR, DB>& to, int ks2, int db)
{
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    typedef __attribute__((address_space(3))) char lds_char;
    i16x4 t1, t2;
    if constexpr (CPR >= 16) {
        // d = 128: addresses formed as integers (the pointer form below made
        // the compiler spill at 256 registers)
        const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)tile +
                              (uint32_t)(ks2 * 16 * CPR * 16);
        t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(base + to.off[0][db]));
        t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(base + to.off[1][db]));
    } else {
        // d = 64: the tile base and the 16*ks2-row step fold into the
        // instructions' offset fields (the integer form cost an add per read)
        lds_char* base = (lds_char*)tile + ks2 * 16 * CPR * 16;
        t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + to.off[0][db]));
        t2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + to.off[1][db]));
    }
    const u32x2 w1 = __builtin_bit_cast(u32x2, t1), w2 = __builtin_bit_cast(u32x2, t2);
    return (u32x4){w1[0], w1[1], w2[0], w2[1]};
}

// One 4-byte global load per lane straight into LDS (lane i writes bytes
// lds_base + 4i .. +3); completion counts in vmcnt like the 16-byte form.
__device__ __forceinline__ void lds_dma4(uint64_t gbase, uint32_t voff, uint32_t lds_base)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %3\n\t"
                 "global_load_lds_dword %1, %2\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(voff), "s"(gbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory");
}

// Operand-ordered layouts of a 32-row tile with 256-byte rows (d = 128,
// 16-bit), used by the pipelined blocks: each read instruction of a wave takes
// one contiguous run, so one address register and the instruction's offset
// field serve every read, without bank conflicts.  The copy instruction of
// wave w fills bytes 1024 w .. 1024 w + 1023 of the tile; these give the byte
// offset, within the tile's rows in memory, of the 16-byte chunk that lane
// `lane` brings.
// Row operands: lane (r, hh) of the run for ks holds row r's chunk 2 ks + hh,
// the operand of lane (r, hh) (run ks = the copy of wave ks).
__device__ __forceinline__ uint32_t row_layout_src(int wave, int lane)
{
    return (uint32_t)(lane & 31) * 256u + (uint32_t)(2 * wave + (lane >> 5)) * 16u;
}
// Transposing reads: 512-byte run b = (tt*4 + db)*2 + u holds, at 16-byte slot
// k, row 16 tt + 8 u + 4 (k/16) + (k/2)%4 and chunk 4 db + 2 ((k/8)%2) + k%2,
// whose two 8-byte halves lanes 2k and 2k+1 read (the rows 16 tt + 4 hh +
// {0..3} (u = 0) or {8..11} (u = 1) of column block db).
__device__ __forceinline__ uint32_t tr_layout_src(int wave, int lane)
{
    const int b = 2 * wave + (lane >> 5), k = lane & 31;
    const int row = 16 * (b >> 3) + 8 * (b & 1) + 4 * (k >> 4) + ((k >> 1) & 3);
    const int chunk = 4 * ((b >> 1) & 3) + 2 * ((k >> 3) & 1) + (k & 1);
    return (uint32_t)row * 256u + (uint32_t)chunk * 16u;
}

// Round the 8 accumulator values of chunk ks2 (elements 8*ks2 .. 8*ks2+7) to T.
template <typename T>
__device__ __forceinline__ typename H16<T>::v8 pack8(const f32x16& x, int ks2)
{
    typename H16<T>::v8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (T)x[8 * ks2 + i];
    return r;
}

// KB key blocks of 32 per wave (KW = 32*KB keys): the Q and dO operands a
// wave reads from LDS (row-major for S and dP, transposed for dK and dV) serve
// all KB blocks, so LDS bytes per matrix product fall as KB grows (at d = 128,
// KB = 2 needs four waves, one per SIMD, with 256 accumulator registers).
// With KB = 1 the registers are capped for two waves per SIMD: two per
// workgroup at d = 128, and at d = 64 (four-wave workgroups) two workgroups
// per compute unit, whose tiles then hide each other's latencies.
// MASKED (calls with a key-padding mask): a wave whose keys are all padded
// takes part in the copies and barriers only (its dK and dV stay zero).
template <typename T, int D, int NW, int KB, bool MASKED = false>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(KB == 1 ? 2 : 1, KB == 1 ? 2 : 1)))
bwd_dkdv(BwdParams p)
{
    using TR = H16<T>;
    using v8 = typename TR::v8;
    constexpr int CPR = D * 2 / 16, DK = D / 16, DB = D / 32, BQ = 64, NH = BQ / 32, KW = 32 * KB;
    using Plan = TilePlan<BQ, CPR, NW, 3>;
    // 16-bit d = 128 without a key-padding mask, 32 keys per wave: the query
    // tiles whose rows see every key of the workgroup run through the software
    // pipeline of bwd_dkdv_pipe_asm.h
    constexpr bool PIPE = !MASKED && D == 128 && NW == 8 && KB == 1;
    // Q buffers sqg[0..1], dO buffers sqg[2..3]: one array, which the pipeline
    // also uses (with its own layouts)
    __shared__ u32x4 sqg[4][BQ * CPR];
    u32x4 (*const sq)[BQ * CPR] = sqg;
    u32x4 (*const sg)[BQ * CPR] = sqg + 2;
    __shared__ u32x4 s_vw[NW][KB][DK][64];   // each wave's V^T operands (registers are short)
    __shared__ __attribute__((aligned(16))) float s_l2[2][BQ];
    __shared__ __attribute__((aligned(16))) float s_d[2][BQ];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int hh = lane >> 5, col = lane & 31;
    const int N = p.N;
    const int bh = blockIdx.x % (p.B * p.H);
    const int kt = blockIdx.x / (p.B * p.H);
    const int b = bh / p.H;
    const size_t head = (size_t)bh * N * D;
    const T* __restrict__ Q = (const T*)p.q + head;
    const T* __restrict__ K = (const T*)p.k + head;
    const T* __restrict__ V = (const T*)p.v + head;
    const T* __restrict__ G = (const T*)p.dout + head;
    const float* __restrict__ L2 = p.lse2 + (size_t)bh * N;
    const float* __restrict__ DS = p.dsum + (size_t)bh * N;
    const int k_wave = kt * KW * NW + wave * KW;      // first key of this wave
    // this lane's key in block kb: k_wave + 32 kb + col
    bool key_on[KB];
    bool any_on = false, all_on = true;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int key = k_wave + 32 * kb + col;
        const int krow = min(key, N - 1);
        key_on[kb] = key < N && !(p.mask && p.mask[(size_t)b * N + krow]);
        any_on = any_on || key_on[kb];
        all_on = all_on && key_on[kb];
    }
    const bool keys_all_on = __builtin_amdgcn_ballot_w64(all_on) == ~0ull;   // wave-uniform
    const bool keys_all_off = MASKED && __builtin_amdgcn_ballot_w64(any_on) == 0;

    // K^T and V^T operands of the lane's keys: head columns 16*ks + 8*hh + 0..7.
    // K^T stays in registers; V^T goes to the wave's own LDS slots (each lane
    // reads back only what it wrote), which keeps the loop free of spills.
    u32x4 kw[KB][DK];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int krow = min(k_wave + 32 * kb + col, N - 1);
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) {
            kw[kb][ks] = *(const u32x4*)(K + (size_t)krow * D + ks * 16 + hh * 8);
            s_vw[wave][kb][ks][lane] = *(const u32x4*)(V + (size_t)krow * D + ks * 16 + hh * 8);
        }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int ks = 0; ks < DK; ++ks) asm volatile("" : "+v"(kw[kb][ks]));

    f32x16 dk[KB][DB], dv[KB][DB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int db = 0; db < DB; ++db) { dk[kb][db] = (f32x16){}; dv[kb][db] = (f32x16){}; }

    // query tiles that can see any key of the workgroup
    const int k_wg = kt * KW * NW;
    const int qt0 = p.causal ? k_wg / BQ : 0;
    const int nqt = (N + BQ - 1) / BQ;
    const float c = p.c;

    // lse2 and D of a query tile: loaded into registers one tile ahead by the
    // first BQ threads, stored to LDS at the top of the tile's step
    float nl2 = 0.f, nd = 0.f;
    auto row_terms = [&](int qt) __attribute__((always_inline)) {
        const int qi = qt * BQ + (int)threadIdx.x;
        const int qr = min(qi, N - 1);
        nl2 = qi < N ? L2[qr] : INFINITY;
        nd = DS[qr];
    };
    // Query tiles in the order qa .. nqt-1, then qt0 .. qa-1: under causal
    // masking the tiles that cross the workgroup's keys come last (qa is the
    // first tile whose rows all follow every key of the workgroup), so that
    // the pipelined block below can take a leading run of full tiles and this
    // loop the rest, in one order for every path.
    const int qa = p.causal ? min(qt0 + KW * NW / BQ, nqt) : 0;
    int q_first = qa;
    if constexpr (PIPE) {
        // Tiles qa .. qb-1 through the block: all 64 rows lie before N and
        // every key of the workgroup lies before N.  The block takes them as
        // 32-row steps and leaves dk and dv updated.
        const int qb = N / BQ;
        if (p.pipe && k_wg + KW * NW <= N && qb > qa) {
            __shared__ __attribute__((aligned(16))) float s_ld[NW][2][64];   // lse2 and D per step, per wave
            static_assert(CPR * 16 == 256, "256-byte rows");
            constexpr uint32_t TILE = 32 * 256, ROWQ = 0, ROWG = 2 * TILE;
            const int qs = qa * BQ;
            int pl = lane;
            asm volatile("" : "+v"(pl));
            const int phh = pl >> 5;
            uint32_t offr = (uint32_t)qs * 256u + row_layout_src(wave, pl);
            uint32_t offt = (uint32_t)qs * 256u + tr_layout_src(wave, pl);
            // lse2 (lanes 0..31) and D (lanes 32..63) of the step's rows,
            // addressed from the head's D (the host checks the distance fits)
            const uint32_t dl = (uint32_t)((const char*)p.lse2 - (const char*)p.dsum);
            uint32_t offl = pl < 32 ? dl + (uint32_t)(qs + pl) * 4u : (uint32_t)(qs + pl - 32) * 4u;
            const uint64_t qbase = uniform_ptr(Q), gbase = uniform_ptr(G), dbase = uniform_ptr(DS);
            const uint32_t lb = lds_addr(sqg[0]), ldb = lds_addr(&s_ld[0][0][0]);
            lds_dma16(qbase, offr, lb + ROWQ + (uint32_t)wave * 1024u);
            lds_dma16(gbase, offr, lb + ROWG + (uint32_t)wave * 1024u);
            lds_dma4(dbase, offl, ldb + (uint32_t)wave * 512u);
            offr += TILE;
            offl += 128u;
            const uint32_t ka = lb + (uint32_t)pl * 16u, tra = lb + (uint32_t)pl * 8u;
            const uint32_t vwa = lds_addr(&s_vw[wave][0][0][pl]);
            const uint32_t lda = ldb + (uint32_t)wave * 512u + (uint32_t)phh * 16u;
            const uint32_t kdst = __builtin_amdgcn_readfirstlane(lb + (uint32_t)wave * 1024u);
            const uint32_t ldst = __builtin_amdgcn_readfirstlane(ldb + (uint32_t)wave * 512u);
            uint32_t pairs = __builtin_amdgcn_readfirstlane((uint32_t)(qb - qa - 1));   // (steps - 2) / 2
            uint32_t m0save;
            f32x16 (&dk0)[DB] = dk[0];
            f32x16 (&dv0)[DB] = dv[0];
            u32x4 (&kw0)[DK] = kw[0];
            if constexpr (std::is_same<T, __bf16>::value)
                asm volatile(ATTN_DKDV_PIPE_ASM_BF16 ATTN_DKDV_PIPE_OPERANDS);
            else
                asm volatile(ATTN_DKDV_PIPE_ASM_F16 ATTN_DKDV_PIPE_OPERANDS);
            __syncthreads();    // every wave is done with the block's buffers
            q_first = qb;
        }
    }
    // the loop's share: tiles q_first .. nqt-1, then qt0 .. qa-1
    const int n_tail = nqt - q_first, cnt = n_tail + (qa - qt0);
    auto tile_at = [&](int i) __attribute__((always_inline)) { return i < n_tail ? q_first + i : qt0 + (i - n_tail); };
    // the copy plans are built after the block (not kept live across it):
    // opaque copies of the wave and lane stop the compiler from reusing values
    // computed before it
    int wv = wave, ln = lane;
    if constexpr (PIPE) asm volatile("" : "+s"(wv), "+v"(ln));
    Plan plan;
    plan.init(wv, ln);
    TrOffsets<CPR, DB> tro;
    tro.init(ln);
    auto stage = [&](int buf, int qt) __attribute__((always_inline)) {
        plan.issue(sq[buf], Q, qt * BQ, N, wave);
        plan.issue(sg[buf], G, qt * BQ, N, wave);
    };
    if (cnt > 0) {
        stage(0, tile_at(0));
        if (threadIdx.x < BQ) row_terms(tile_at(0));
    }

    for (int i = 0; i < cnt; ++i) {
        const int qt = tile_at(i);
        const int buf = i & 1;
        const int q0 = qt * BQ;
        // tile qt landed; every wave is done with tile qt-1 (other buffer)
        if (threadIdx.x < BQ) {
            s_l2[buf][threadIdx.x] = nl2;
            s_d[buf][threadIdx.x] = nd;
        }
        wait_vmcnt<0>();
        __syncthreads();
        if (i + 1 < cnt) {
            stage(buf ^ 1, tile_at(i + 1));
            if (threadIdx.x < BQ) row_terms(tile_at(i + 1));
        }

        if (keys_all_off) continue;
        // the tile's two 32-row halves, one after the other
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const int qh = q0 + 32 * h;
            // causal: every query of the half precedes every key of the wave, so
            // the wave has nothing to add (it still took part in the copy
            // above).  At d = 64 (one wave per SIMD) the two halves without the
            // skip form one block the compiler schedules better than the skip
            // saves (measured at B4 H16 N1024: 0.108 -> 0.104 ms); the masks
            // zero those pairs.
            if (D == 128 && p.causal && qh + 31 < k_wave) continue;

            // S = Q K^T: lane holds key column `col` of block kb, query rows
            // 8*(j/4) + 4*hh + j%4; each Q operand serves every key block
            f32x16 s[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) s[kb] = (f32x16){};
#pragma unroll
            for (int ks = 0; ks < DK; ++ks) {
                const u32x4 qa = sq[buf][(32 * h + col) * CPR + swz_kt<CPR>(32 * h + col, ks * 2 + hh)];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    s[kb] = TR::mma32(__builtin_bit_cast(v8, qa), __builtin_bit_cast(v8, kw[kb][ks]), s[kb]);
            }
            // P = exp2(s*c - lse2), lse2 of the lane's 16 query rows read as four
            // 16-byte LDS vectors.  At d = 128 each is read where its four rows
            // are used (holding all 16 values, and D's below, spilled registers
            // there); at d = 64 (one wave per SIMD, registers to spare) all four
            // are read first, so their latency overlaps.  Every exponential is
            // formed (rows past the end carry lse2 = +inf and give 0); the empty
            // asm keeps each one out of a per-element branch.  Pairs that are not
            // visible are then set to 0, on tiles that are not wholly visible only.
            constexpr bool LATE = D == 128;
            f32x4 l2e[LATE ? 1 : 4];
            if constexpr (!LATE) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) l2e[g4] = *(const f32x4*)&s_l2[buf][32 * h + 8 * g4 + 4 * hh];
            }
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 l2v = LATE ? *(const f32x4*)&s_l2[buf][32 * h + 8 * g4 + 4 * hh] : l2e[LATE ? 0 : g4];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        s[kb][4 * g4 + i] = fast_exp2(fmaf(s[kb][4 * g4 + i], c, -l2v[i]));
                        asm volatile("" : "+v"(s[kb][4 * g4 + i]));
                    }
            }
            const bool all = keys_all_on && qh + 32 <= N && (!p.causal || qh >= k_wave + KW - 1);
            if (!all) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int qi = qh + 8 * (j >> 2) + 4 * hh + (j & 3);
                        bool vis = key_on[kb] && qi < N;
                        if (p.causal) vis = vis && k_wave + 32 * kb + col <= qi;
                        s[kb][j] = vis ? s[kb][j] : 0.f;
                    }
            }
            v8 pa[KB][2];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) { pa[kb][0] = pack8<T>(s[kb], 0); pa[kb][1] = pack8<T>(s[kb], 1); }
            // dV += P^T dO (contraction over the half's 32 queries)
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const v8 gt = __builtin_bit_cast(v8, tr_operand(sg[buf], tro, 2 * h + t, db));
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) dv[kb][db] = TR::mma32(pa[kb][t], gt, dv[kb][db]);
                }
            // dP - D = dO V^T - D: the products accumulate onto -D of the
            // lane's rows (the workspace holds -D), read as four 16-byte
            // vectors straight into the accumulator; then dS = P (dP - D)
            f32x16 dp[KB];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 nd4 = *(const f32x4*)&s_d[buf][32 * h + 8 * g4 + 4 * hh];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dp[kb][4 * g4 + i] = nd4[i];
            }
#pragma unroll
            for (int ks = 0; ks < DK; ++ks) {
                const u32x4 ga = sg[buf][(32 * h + col) * CPR + swz_kt<CPR>(32 * h + col, ks * 2 + hh)];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    dp[kb] = TR::mma32(__builtin_bit_cast(v8, ga), __builtin_bit_cast(v8, s_vw[wave][kb][ks][lane]), dp[kb]);
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j) dp[kb][j] = s[kb][j] * dp[kb][j];
            v8 da[KB][2];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                da[kb][0] = pack8<T>(dp[kb], 0);
                da[kb][1] = pack8<T>(dp[kb], 1);
            }
            // dK += dS^T Q
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const v8 qt_ = __builtin_bit_cast(v8, tr_operand(sq[buf], tro, 2 * h + t, db));
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) dk[kb][db] = TR::mma32(da[kb][t], qt_, dk[kb][db]);
                }
        }
    }

    // dV[key][d] and dK[key][d]: accumulator block (kb, db) holds head column
    // 32*db + col and keys 32*kb + 8*(j/4) + 4*hh + j%4 of the wave's keys
    const float sc = p.scale;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int kr = k_wave + 32 * kb + 8 * (j >> 2) + 4 * hh + (j & 3);
                if (kr < N) {
                    const size_t idx = head + (size_t)kr * D + 32 * db + col;
                    p.dv[idx] = dv[kb][db][j];
                    p.dk[idx] = dk[kb][db][j] * sc;
                }
            }
        }
}

// MASKED (calls with a key-padding mask): each lane's padding flags of the next
// key tile are loaded one tile ahead (a 32-bit word holds the flags of four
// consecutive keys); a tile without a padded key takes the unmasked path and
// a tile whose keys are all padded is skipped.  Registers are capped for two
// waves per SIMD (at d = 64, two four-wave workgroups per compute unit).
template <typename T, int D, int NW, bool MASKED = false>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq(BwdParams p)
{
    using TR = H16<T>;
    using v8 = typename TR::v8;
    constexpr int CPR = D * 2 / 16, DK = D / 16, DB = D / 32, BC = 64, NKB = BC / 32, KS = BC / 16;
    // K tiles are read row-wise and transposed, V tiles row-wise: both use
    // swz_kt, so one copy plan serves both
    using Plan = TilePlan<BC, CPR, NW, 3>;
    // 16-bit d = 128 without a key-padding mask: the key tiles every row of
    // the workgroup sees in full run through the software pipeline of
    // bwd_dq_pipe_asm.h first
    constexpr bool PIPE = !MASKED && D == 128 && NW == 8;
    // K buffers kv[0..1], V buffers kv[2..3]: one array, so that the pipeline
    // addresses all of them from one base
    __shared__ u32x4 kv[4][BC * CPR];
    u32x4 (*const sk)[BC * CPR] = kv;
    u32x4 (*const sv)[BC * CPR] = kv + 2;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int hh = lane >> 5, col = lane & 31;
    const int N = p.N;
    const int bh = blockIdx.x % (p.B * p.H);
    int qt = blockIdx.x / (p.B * p.H);
    if (p.causal) qt = (N + 32 * NW - 1) / (32 * NW) - 1 - qt;   // heaviest query tiles first
    const int b = bh / p.H;
    const size_t head = (size_t)bh * N * D;
    const T* __restrict__ Q = (const T*)p.q + head;
    const T* __restrict__ K = (const T*)p.k + head;
    const T* __restrict__ V = (const T*)p.v + head;
    const T* __restrict__ G = (const T*)p.dout + head;
    const int q0 = qt * 32 * NW;
    const int wave_q0 = q0 + wave * 32;
    const int qi = wave_q0 + col;                     // this lane's query
    const int qrow = min(qi, N - 1);
    const float l2 = qi < N ? p.lse2[(size_t)bh * N + qrow] : INFINITY;
    const float ndsum = p.dsum[(size_t)bh * N + qrow];   // minus D
    // MASKED: padw[kb][g4] holds the flags of keys k0 + 32*kb + 8*g4 + 4*hh +
    // 0..3 of the current tile, padn those of the next; one 32-bit load when
    // the mask row is 4-byte aligned and the keys lie inside the row, else four
    // byte loads at clamped keys (flags past N are never used)
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

    u32x4 qw[DK], gw[DK];
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
        qw[ks] = *(const u32x4*)(Q + (size_t)qrow * D + ks * 16 + hh * 8);
        gw[ks] = *(const u32x4*)(G + (size_t)qrow * D + ks * 16 + hh * 8);
    }
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) { asm volatile("" : "+v"(qw[ks])); asm volatile("" : "+v"(gw[ks])); }

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = (f32x16){};

    const int nkt = (N + BC - 1) / BC;
    const int kt_end = p.causal ? min(nkt, (min(q0 + 32 * NW, N) - 1) / BC + 1) : nkt;
    const float c = p.c;
    int kt_first = 0;
    if constexpr (PIPE) {
        // The pipeline takes 32-key tiles 0 .. n32-1 (n32 even, every key
        // visible to every query of the workgroup, no tile past N) and leaves
        // dq updated; the loop below resumes at 64-key tile n32/2.
        int n32 = p.causal ? q0 / 32 : N / 32;
        n32 = min(n32, N / 32) & ~1;
        if (p.pipe && n32 >= 2) {
            static_assert(CPR * 16 == 256, "256-byte rows");
            constexpr uint32_t TILE = 32 * 256, ROWS_V = 4 * TILE;
            // the block's addresses come from an opaque copy of the lane: the
            // loop below computes its own after the block instead of keeping
            // shared values live across it
            int pl = lane;
            asm volatile("" : "+v"(pl));
            uint32_t offa = row_layout_src(wave, pl), offb = tr_layout_src(wave, pl);
            const uint64_t kbase = uniform_ptr(K), vbase = uniform_ptr(V);
            const uint32_t lb = lds_addr(kv[0]);
            // rows of tile 0 (K and V); the block copies the rest
            lds_dma16(kbase, offa, lb + (uint32_t)wave * 1024u);
            lds_dma16(vbase, offa, lb + ROWS_V + (uint32_t)wave * 1024u);
            offa += TILE;
            const uint32_t ka = lb + (uint32_t)pl * 16u, tra = lb + (uint32_t)pl * 8u;
            const uint32_t kdst = __builtin_amdgcn_readfirstlane(lb + (uint32_t)(wave * 1024));
            uint32_t pairs = __builtin_amdgcn_readfirstlane((uint32_t)(n32 - 2) / 2);
            uint32_t m0save;
            if constexpr (std::is_same<T, __bf16>::value)
                asm volatile(ATTN_DQ_PIPE_ASM_BF16 ATTN_DQ_PIPE_OPERANDS);
            else
                asm volatile(ATTN_DQ_PIPE_ASM_F16 ATTN_DQ_PIPE_OPERANDS);
            kt_first = n32 / 2;
            __syncthreads();    // every wave is done with the buffers the loop refills
        }
    }
    // the plans are built after the block (not kept live across it)
    int wv = wave;
    asm volatile("" : "+s"(wv));
    Plan plan;
    plan.init(wv, lane);
    TrOffsets<CPR, DB> tro;
    tro.init(lane);
    if (kt_first < kt_end) {
        plan.issue(sk[kt_first & 1], K, kt_first * BC, N, wave);
        plan.issue(sv[kt_first & 1], V, kt_first * BC, N, wave);
        if constexpr (MASKED) load_pad(kt_first * BC);
    }
    for (int kt = kt_first; kt < kt_end; ++kt) {
        const int buf = kt & 1;
        const int k0 = kt * BC;
        wait_vmcnt<0>();
        __syncthreads();
        if (kt + 1 < kt_end) {
            plan.issue(sk[buf ^ 1], K, k0 + BC, N, wave);
            plan.issue(sv[buf ^ 1], V, k0 + BC, N, wave);
        }
        bool pad_any = false;
        if constexpr (MASKED) {
            // this tile's flags arrived with the wait above; fetch the next
            // tile's.  The two wave halves hold all the tile's keys.
            uint32_t any = 0, zero = 0;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    padw[kb][g4] = padn[kb][g4];
                    any |= padw[kb][g4];
                    zero |= (padw[kb][g4] - 0x01010101u) & ~padw[kb][g4] & 0x80808080u;   // high bit of every zero byte
                }
            if (kt + 1 < kt_end) load_pad(k0 + BC);
            pad_any = __builtin_amdgcn_ballot_w64(any != 0) != 0;
            if (__builtin_amdgcn_ballot_w64(zero != 0) == 0) continue;   // every key padded
        }
        // causal: every key of the tile follows every query of the wave
        if (p.causal && k0 > wave_q0 + 31) continue;

        // The tile as two 32-key blocks: S^T = K Q^T and dP^T = V dO^T of each
        // block (lane holds query column `col`, key rows 32*kb + 8*(j/4) +
        // 4*hh + j%4), then block 0's vector work (dS^T = P^T (dP^T - D),
        // P^T = exp2(s*c - lse2), 0 for masked pairs) beside block 1's
        // products, and block 1's vector work beside the first half of
        // dQ^T += K^T dS^T.  Per element the operations and their order are
        // unchanged.  Every exponential is formed (a row past the end has
        // lse2 = +inf); the empty asm keeps each one out of a per-element
        // branch, and the visibility test runs only on tiles that are not
        // wholly visible.
        const bool all = !pad_any && k0 + BC <= N && wave_q0 + 31 < N && (!p.causal || k0 + BC - 1 <= wave_q0);
        {
            f32x16 s[NKB], dp[NKB];
            auto products = [&](int kb) __attribute__((always_inline)) {
                s[kb] = (f32x16){};
                dp[kb] = (f32x16){};
                const int r = kb * 32 + col;
#pragma unroll
                for (int ks = 0; ks < DK; ++ks) {
                    const u32x4 ka = sk[buf][r * CPR + swz_kt<CPR>(r, ks * 2 + hh)];
                    const u32x4 va = sv[buf][r * CPR + swz_kt<CPR>(r, ks * 2 + hh)];
                    s[kb] = TR::mma32(__builtin_bit_cast(v8, ka), __builtin_bit_cast(v8, qw[ks]), s[kb]);
                    dp[kb] = TR::mma32(__builtin_bit_cast(v8, va), __builtin_bit_cast(v8, gw[ks]), dp[kb]);
                }
            };
            auto vector = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    s[kb][j] = fast_exp2(fmaf(s[kb][j], c, -l2));
                    asm volatile("" : "+v"(s[kb][j]));
                }
                if (!all) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int key = k0 + kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
                        bool vis = key < N && qi < N;
                        if (p.causal) vis = vis && key <= qi;
                        if constexpr (MASKED) vis = vis && ((padw[kb][j >> 2] >> (8 * (j & 3))) & 0xffu) == 0;
                        s[kb][j] = vis ? s[kb][j] : 0.f;
                    }
                }
#pragma unroll
                for (int j = 0; j < 16; ++j) s[kb][j] = s[kb][j] * (dp[kb][j] + ndsum);
            };
            // dQ^T += K^T dS^T over the 16 keys of chunk ks2
            auto dq_chunk = [&](int ks2) __attribute__((always_inline)) {
                const v8 da = pack8<T>(s[ks2 >> 1], ks2 & 1);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const u32x4 ka = tr_operand(sk[buf], tro, ks2, db);
                    dq[db] = TR::mma32(__builtin_bit_cast(v8, ka), da, dq[db]);
                }
            };
            static_assert(NKB == 2 && KS == 4, "two 32-key blocks per tile");
            products(0);
            products(1);
            vector(0);
            dq_chunk(0);
            dq_chunk(1);
            vector(1);
            dq_chunk(2);
            dq_chunk(3);
        }
    }

    // dQ[query][d]: block db holds head columns 32*db + 8*(j/4) + 4*hh + j%4
    if (qi < N) {
        const float sc = p.scale;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = db * 32 + 8 * g4 + 4 * hh;
                *(f32x4*)(p.dq + head + (size_t)qi * D + d0) =
                    (f32x4){dq[db][4 * g4] * sc, dq[db][4 * g4 + 1] * sc, dq[db][4 * g4 + 2] * sc, dq[db][4 * g4 + 3] * sc};
            }
        }
    }
}

template <typename T, int D>
hipError_t launch_bwd(const BwdParams& p, hipStream_t st)
{
    // eight waves (two per SIMD) at d = 128; at d = 64 a 32-row tile has too
    // few 16-byte chunks for eight waves' copy instructions, so four, and two
    // workgroups share a compute unit
    constexpr int NW = D == 128 ? 8 : 4;
    const size_t rows = (size_t)p.B * p.H * p.N;
    constexpr size_t RPB = 256 / (D / 8);            // rows per block of bwd_pre
    hipLaunchKernelGGL((bwd_pre<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dK, dV: waves of 32 keys.  Waves of 64 keys (KB = 2, four per
    // workgroup, one per SIMD) read 43% fewer LDS bytes but measured 8% slower
    // at B1 H32 N8192 d128 causal on MI355X: one wave per SIMD leaves the LDS
    // and exponential latencies of each 32-query step exposed.
    constexpr int KB = 1, NWK = NW;
    const unsigned ktiles = (unsigned)((p.N + 32 * KB * NWK - 1) / (32 * KB * NWK));
    const dim3 kgrid((unsigned)(p.B * p.H) * ktiles), kblock(NWK * 64);
    if (p.mask) hipLaunchKernelGGL((bwd_dkdv<T, D, NWK, KB, true>), kgrid, kblock, 0, st, p);
    else hipLaunchKernelGGL((bwd_dkdv<T, D, NWK, KB, false>), kgrid, kblock, 0, st, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned tiles = (unsigned)((p.N + 32 * NW - 1) / (32 * NW));
    const dim3 grid((unsigned)(p.B * p.H) * tiles), block(NW * 64);
    if (p.mask) hipLaunchKernelGGL((bwd_dq<T, D, NW, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((bwd_dq<T, D, NW, false>), grid, block, 0, st, p);
    return hipGetLastError();
}

BwdLaunchFn lookup_bwd(int dtype_bits, int D)
{
    if (dtype_bits == 0) return D == 128 ? &launch_bwd<__bf16, 128> : D == 64 ? &launch_bwd<__bf16, 64> : nullptr;
    if (dtype_bits == 1) return D == 128 ? &launch_bwd<_Float16, 128> : D == 64 ? &launch_bwd<_Float16, 64> : nullptr;
    return nullptr;
}

}  // namespace attnk
