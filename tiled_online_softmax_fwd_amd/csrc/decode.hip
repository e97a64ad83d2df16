// decode.hip -- a block of Nq query rows against a key/value cache of Nk rows,
// split over the keys and merged by log-sum-exp.
//
// The yadro-code tutorial "How FlashAttention reduces GPU memory traffic"
// separates processing a long prompt from step-by-step generation with a
// key/value cache: few query rows meet many cached keys, there is little
// reuse, and the work is bound by reading K and V once from memory.  One
// wave then has too little work per head, so the keys of every (batch, head)
// are split into chunks handled by independent one-wave workgroups; each
// folds its chunk with the online merge (running reference m, sum l,
// accumulator, rescale by exp(m_old - m_new)) and writes a partial result
// (acc / l, lse).  A second kernel merges the partials of a row with the
// same rule one level up: lse = log sum_s exp(lse_s) and
// O = sum_s exp(lse_s - lse) O_s.
//
// Split kernel layout (per wave, 16 query rows): S^T = K Q^T on
// v_mfma_f32_16x16x32_{bf16,f16}; lane L holds query L%16 and keys
// 16*kb + 4*(L/16) + i of each 16-key block, which after rounding to the input
// type are the B operand of the 16x16x16 P.V product; V^T comes from LDS with
// ds_read_b64_tr_b16.  K and V tiles of 32 keys are copied HBM -> LDS with
// global_load_lds_dwordx4, double-buffered; the wave alone reads its LDS, so
// waiting for its own copies is enough (no workgroup barrier).
#include <hip/hip_runtime.h>
#include "decode.h"
#include "fwd_kernel.h"
#include "fwd_m16.h"

namespace attnk {

// MASKED: the instance for calls with a key-padding mask.  Each lane's padding
// flags of the next key tile are loaded one tile ahead (a 32-bit word holds
// the flags of four consecutive keys); a tile without a padded key skips the
// padding test and a tile whose keys are all padded is skipped.
template <typename T, int D, bool MASKED = false>
__global__ void __launch_bounds__(64) dec_split(DecParams p)
{
    constexpr int BC = 32;
    constexpr int CPR = D * 2 / 16;
    constexpr int NKB = BC / 16, DB = D / 16, NQ = D / 32;
    using KPlan = TilePlan<BC, CPR, 1, 0, true>;   // K and V are read once: non-temporal
    using VPlan = TilePlan<BC, CPR, 1, 1, true>;
    using v8 = typename M16<T>::v8;
    using v2 = typename Dot2<T>::v2;
    static_assert(D == 64 || D == 128, "head size");

    __shared__ u32x4 sk[2][BC * CPR];
    __shared__ u32x4 sv[2][BC * CPR];

    const int lane = threadIdx.x;
    const int g = lane >> 4, col = lane & 15;
    const int split = blockIdx.x % p.splits;
    const int bh = blockIdx.x / p.splits;
    const int b = bh / p.H;
    const int Nq = p.Nq, Nk = p.Nk;
    const int qi = blockIdx.y * 16 + col;             // this lane's query row
    const int qrow = min(qi, Nq - 1);
    const T* __restrict__ Q = (const T*)p.q + (size_t)bh * Nq * D;
    const T* __restrict__ K = (const T*)p.k + (size_t)bh * Nk * D;
    const T* __restrict__ V = (const T*)p.v + (size_t)bh * Nk * D;

    // keys of this split that any row of the block can see
    const int k_lo = split * p.keys_per_split;
    int k_hi = min(Nk, k_lo + p.keys_per_split);
    if (p.causal) k_hi = min(k_hi, Nk - Nq + min(blockIdx.y * 16 + 15, Nq - 1) + 1);
    const int ntile = k_hi > k_lo ? (k_hi - k_lo + BC - 1) / BC : 0;
    const int last = p.causal ? Nk - Nq + qi : Nk - 1;   // last key this row sees
    // MASKED: padw[kb] holds the flags of keys k0 + 16*kb + 4*g + 0..3 of the
    // current tile, padn those of the next one; one 32-bit load when the mask
    // row is 4-byte aligned and the keys lie inside the row, else four byte
    // loads at clamped keys (flags past the cache end are never used)
    const uint8_t* const prow = MASKED ? p.mask + (size_t)b * Nk : nullptr;
    const bool pvec = MASKED && ((uintptr_t)prow & 3u) == 0;
    uint32_t padw[MASKED ? NKB : 1], padn[MASKED ? NKB : 1];
    auto load_pad = [&](int k1) __attribute__((always_inline)) {
        if constexpr (MASKED) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int kbase = k1 + kb * 16 + 4 * g;
                uint32_t w = 0;
                if (pvec && kbase + 3 < Nk) {
                    w = *(const uint32_t*)(prow + kbase);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) w |= (uint32_t)prow[min(kbase + r, Nk - 1)] << (8 * r);
                }
                padn[kb] = w;
            }
        }
    };
    if (MASKED && ntile > 0) load_pad(k_lo);

    KPlan kplan;
    VPlan vplan;
    kplan.init(0, lane);
    vplan.init(0, lane);
    if (ntile > 0) {
        kplan.issue(sk[0], K, k_lo, Nk, 0);
        vplan.issue(sv[0], V, k_lo, Nk, 0);
    }

    // Q^T operand: step ks contracts head columns 32*ks + 8*g + 0..7
    u32x4 qw[NQ];
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) qw[ks] = q_mode16(*(const u32x4*)(Q + (size_t)qrow * D + 32 * ks + 8 * g), p.qmode);
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) asm volatile("" : "+v"(qw[ks]));

    float m = -INFINITY, l = 0.f;
    f32x4 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const float c = p.c;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    typedef __attribute__((address_space(3))) char lds_char;

    for (int t = 0; t < ntile; ++t) {
        const int buf = t & 1;
        const int k0 = k_lo + t * BC;
        wait_vmcnt<0>();                          // tile t landed in buffer buf
        asm volatile("" ::: "memory");
        if (t + 1 < ntile) {                      // buffer buf^1 was last read in step t-1
            kplan.issue(sk[buf ^ 1], K, k0 + BC, Nk, 0);
            vplan.issue(sv[buf ^ 1], V, k0 + BC, Nk, 0);
        }
        bool pad_any = false;
        if constexpr (MASKED) {
            // this tile's flags arrived with the wait above; fetch the next
            // tile's.  The four lane groups hold all the tile's keys.
            uint32_t any = 0, zero = 0;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                padw[kb] = padn[kb];
                any |= padw[kb];
                zero |= (padw[kb] - 0x01010101u) & ~padw[kb] & 0x80808080u;   // high bit of every zero byte
            }
            if (t + 1 < ntile) load_pad(k0 + BC);
            pad_any = __builtin_amdgcn_ballot_w64(any != 0) != 0;
            if (__builtin_amdgcn_ballot_w64(zero != 0) == 0) continue;   // every key padded
        }

        f32x4 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = (f32x4){0.f, 0.f, 0.f, 0.f};
            const int r = kb * 16 + col;
#pragma unroll
            for (int ks = 0; ks < NQ; ++ks) {
                const u32x4 kv = sk[buf][r * CPR + swz_k<CPR>(r, 4 * ks + g)];
                s[kb] = M16<T>::mma_s(__builtin_bit_cast(v8, kv), __builtin_bit_cast(v8, qw[ks]), s[kb]);
            }
        }

        // visibility: element (kb, i) of this lane is key k0 + 16*kb + 4*g + i
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = k0 + kb * 16 + 4 * g + i;
                bool vis = key < k_hi && key <= last;
                if constexpr (MASKED) vis = vis && (!pad_any || ((padw[kb] >> (8 * i)) & 0xffu) == 0);
                if (!vis) s[kb][i] = -INFINITY;
            }
        }

        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[kb][i]);
        mt = quad_max(mt);
        const RefStep rs = ref_step(m, mt, c, p.slack);
        m = rs.m;
        l *= rs.alpha;
        if (__builtin_amdgcn_ballot_w64(rs.moved)) {
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] *= rs.alpha;
        }
        const float mc = rs.mc;

        lds_char* vbase = (lds_char*)sv[buf];
        const int rr = col >> 2, qq = col & 3;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const v2 p01 = (v2){(T)fast_exp2(fmaf(s[kb][0], c, -mc)), (T)fast_exp2(fmaf(s[kb][1], c, -mc))};
            const v2 p23 = (v2){(T)fast_exp2(fmaf(s[kb][2], c, -mc)), (T)fast_exp2(fmaf(s[kb][3], c, -mc))};
            l = Dot2<T>::sum2(p01, l);
            l = Dot2<T>::sum2(p23, l);
            // lane 4r+q of each 16-lane group addresses key row 16*kb + 4*g + r,
            // columns 16*db + 4q..4q+3; the transposing read hands lane j the
            // four keys 16*kb + 4*g + 0..3 at column 16*db + j
            const int row = kb * 16 + 4 * g + rr;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int chunk = 2 * db + (qq >> 1);
                const int off = (row * CPR + swz_v16<CPR>(row, chunk)) * 16 + (qq & 1) * 8;
                const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vbase + off));
                o[db] = M16<T>::mma_pv(a, p01[0], p01[1], p23[0], p23[1], o[db]);
            }
        }
    }

    // partial result of this split: acc / l and its lse (empty -> 0, -inf)
    const float lt = quad_sum(l);
    if (qi < Nq) {
        const size_t prow = ((size_t)bh * p.splits + split) * Nq + qi;
        const bool empty = !(lt > 0.f);
        const float inv = empty ? 0.f : 1.f / lt;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d0 = db * 16 + 4 * g;
            f32x4 x;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = empty ? 0.f : o[db][i] * inv;
            *(f32x4*)(p.part_o + prow * D + d0) = x;
        }
        if (g == 0)
            p.part_lse[prow] = empty ? -INFINITY : fmaf(m, p.scale, __builtin_amdgcn_logf(lt) * 0.69314718055994530942f);
    }
}

// One workgroup per query row, one thread per head column: the partial
// results of the row's splits are combined with weights exp(lse_s - lse).
template <typename T, int D>
__global__ void __launch_bounds__(D) dec_merge(DecParams p)
{
    const int row = blockIdx.x;                       // (b*H + h)*Nq + qi
    const int bh = row / p.Nq, qi = row % p.Nq;
    const int dcol = threadIdx.x;
    const size_t base = (size_t)bh * p.splits * p.Nq + qi;   // split s at base + s*Nq
    float M = -INFINITY;
    for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.part_lse[base + (size_t)s * p.Nq]);
    float acc = 0.f, W = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < p.splits; ++s) {
            const float ls = p.part_lse[base + (size_t)s * p.Nq];
            const float w = fast_exp2((ls - M) * 1.4426950408889634f);     // 0 for an empty split
            W += w;
            acc = fmaf(w, p.part_o[(base + (size_t)s * p.Nq) * D + dcol], acc);
        }
    }
    const bool empty = !(W > 0.f);
    const float out = empty ? 0.f : acc / W;
    const size_t orow = (size_t)row * D + dcol;
    if (p.out_f32) ((float*)p.o)[orow] = out;
    else ((T*)p.o)[orow] = (T)out;
    if (p.lse && dcol == 0)
        p.lse[row] = empty ? -INFINITY : M + __builtin_amdgcn_logf(W) * 0.69314718055994530942f;
}

template <typename T, int D>
hipError_t launch_decode(const DecParams& p, hipStream_t st)
{
    const unsigned qblocks = (unsigned)((p.Nq + 15) / 16);
    if (p.mask)
        hipLaunchKernelGGL((dec_split<T, D, true>), dim3((unsigned)(p.B * p.H * p.splits), qblocks), dim3(64), 0, st, p);
    else
        hipLaunchKernelGGL((dec_split<T, D, false>), dim3((unsigned)(p.B * p.H * p.splits), qblocks), dim3(64), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dec_merge<T, D>), dim3((unsigned)(p.B * p.H * p.Nq)), dim3(D), 0, st, p);
    return hipGetLastError();
}

// The scratch of attn_decode_fwd_noalloc.  Host code never uses this name as
// an address (on the host it is only a stand-in for the device symbol): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[DECODE_SCRATCH_BYTES];

hipError_t decode_scratch(void** ptr)
{
    constexpr int MAX_DEV = 64;
    static void* addr[MAX_DEV];          // per device; a racing first lookup stores the same value
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
    if (!addr[dev]) {
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!a) return hipErrorInvalidSymbol;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

DecLaunchFn lookup_decode(int dtype_bits, int D)
{
    // dtype_bits: 0 bf16, 1 f16
    if (dtype_bits == 0) return D == 128 ? &launch_decode<__bf16, 128> : D == 64 ? &launch_decode<__bf16, 64> : nullptr;
    if (dtype_bits == 1) return D == 128 ? &launch_decode<_Float16, 128> : D == 64 ? &launch_decode<_Float16, 64> : nullptr;
    return nullptr;
}

}  // namespace attnk
