// fwd_m16.h -- forward kernel for the tile shapes with 16 query rows per
// workgroup or 16 keys per key tile (the smallest tiles of the tile-size
// sweeps in the news write-up of "Is Flash Attention Stable?", Fig. 6).
//
// Same algorithm as fwd_m32_*: per key tile, the transposed score tile
// S^T = K Q^T on the matrix cores, a true -inf for invisible keys, the online
// merge of the yadro-code tutorial "How FlashAttention reduces GPU memory
// traffic" (reference m, running sum l, accumulator rescaled by
// exp(m_old - m_new); see ref_step), P.V on the matrix cores, and acc / l once
// at the end.
//
// Each wave owns 16 query rows.  In the 16x16 accumulator of S^T lane L holds
// query column L%16 and keys 4*(L/16) + i (i = 0..3) of a 16-key block; those
// four values, rounded to the input type, are exactly the B operand of a
// 16x16x16 MFMA over keys, so P goes from the exponentials straight into
// O^T += V^T P^T.  The V^T operand (4 consecutive keys at one column per
// lane) is one ds_read_b64_tr_b16 per 16-key block and 16 columns.  fp32 uses
// 16x16x4 with the same layouts, one key (or four head columns) per step.
//
// These shapes are for the numerical sweeps; K and V are staged through
// registers into one padded LDS buffer per tile with two barriers.
#pragma once
#include <type_traits>
#include "fwd_kernel.h"

namespace attnk {

typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;

template <typename T> struct M16;
template <> struct M16<__bf16> {
    using v8 = bf16x8;
    static __device__ __forceinline__ f32x4 mma_s(v8 a, v8 b, f32x4 c)
    { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
    static __device__ __forceinline__ f32x4 mma_pv(i16x4 a, __bf16 p0, __bf16 p1, __bf16 p2, __bf16 p3, f32x4 c)
    {
        const i16x4 b = (i16x4){__builtin_bit_cast(short, p0), __builtin_bit_cast(short, p1),
                                __builtin_bit_cast(short, p2), __builtin_bit_cast(short, p3)};
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};
template <> struct M16<_Float16> {
    using v8 = f16x8;
    static __device__ __forceinline__ f32x4 mma_s(v8 a, v8 b, f32x4 c)
    { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
    static __device__ __forceinline__ f32x4 mma_pv(i16x4 a, _Float16 p0, _Float16 p1, _Float16 p2, _Float16 p3, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), (f16x4){p0, p1, p2, p3}, c, 0, 0, 0);
    }
};

// max / sum over the four lanes {L, L^16, L^32, L^48} that hold one query
// row.  Both partners of each exchange add the same two values, so every lane
// of the row ends with the same bits.
__device__ __forceinline__ float quad_max(float x)
{
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float quad_sum(float x)
{
    x = x + __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

template <typename T, int D, int BR, int BC>
__global__ void __launch_bounds__(BR * 4)
fwd_m16(FwdParams p)
{
    constexpr bool F32 = __is_same(T, float);
    constexpr int NW = BR / 16, NT = NW * 64;
    constexpr int ES = (int)sizeof(T);
    constexpr int CPR = D * ES / 16;           // 16-byte chunks per row
    constexpr int RS = D * ES + 16;            // padded LDS row stride, bytes
    constexpr int NKB = BC / 16, DB = D / 16;
    constexpr int NQ = F32 ? D / 4 : D / 32;   // Q operand registers (floats or 8-element vectors)
    static_assert(BR % 16 == 0 && BC % 16 == 0 && BR <= 128 && (D == 64 || D == 128), "tile");

    __shared__ __attribute__((aligned(16))) char sk[BC * RS];
    __shared__ __attribute__((aligned(16))) char sv[BC * RS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, col = lane & 15;
    int bh, qt;
    tile_of_block(p, bh, qt);
    const int N = p.N;
    const int b = bh / p.H;
    const int q0 = qt * BR;
    const size_t head = (size_t)bh * (size_t)N * D;
    const T* __restrict__ Q = (const T*)p.q + head;
    const T* __restrict__ K = (const T*)p.k + head;
    const T* __restrict__ V = (const T*)p.v + head;
    const int qi = q0 + wave * 16 + col;       // this lane's query row
    const int qrow = min(qi, N - 1);

    // Q^T operand.  16-bit: step ks contracts head columns 32*ks + 8*g + 0..7.
    // fp32: step t contracts head column g*(D/4) + t.
    using QV = typename std::conditional<F32, float, typename M16<typename std::conditional<F32, __bf16, T>::type>::v8>::type;
    QV qf[NQ];
    if constexpr (F32) {
#pragma unroll
        for (int u = 0; u < D / 16; ++u) {
            const f32x4 w = *(const f32x4*)((const float*)Q + (size_t)qrow * D + g * (D / 4) + 4 * u);
#pragma unroll
            for (int e = 0; e < 4; ++e) qf[4 * u + e] = q_mode32(w[e], p.qmode);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks)
            qf[ks] = __builtin_bit_cast(QV, q_mode16(*(const u32x4*)(Q + (size_t)qrow * D + 32 * ks + 8 * g), p.qmode));
    }

    float m = -INFINITY, l = 0.f;
    f32x4 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = (f32x4){0.f, 0.f, 0.f, 0.f};

    const int nkt = (N + BC - 1) / BC;
    int kt_end = nkt;
    if (p.causal) kt_end = min(nkt, (min(q0 + BR, N) - 1) / BC + 1);
    const float c = p.c;
    // key-padding flags: word kb holds keys k0 + 16 kb + 4 g + 0..3
    const uint8_t* const prow = p.mask ? p.mask + (size_t)b * N : nullptr;
    const bool pvec = prow && ((uintptr_t)prow & 3u) == 0;
    uint32_t padw[NKB];
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

    for (int it = 0; it < kt_end; ++it) {
        const int k0 = (p.kv_order ? (kt_end - 1 - it) : it) * BC;
        // the flags load while the tile is staged
        if (prow) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) padw[kb] = pad_word(prow, pvec, k0 + kb * 16 + 4 * g, N);
        }

        // stage K and V rows k0..k0+BC-1 (rows past N-1 repeat row N-1; their
        // scores are masked below)
        __syncthreads();
        constexpr int TOTAL = BC * CPR;
#pragma unroll
        for (int c0 = 0; c0 < TOTAL; c0 += NT) {
            const int idx = c0 + tid;
            if (TOTAL % NT == 0 || idx < TOTAL) {
                const int r = idx / CPR, cc = idx % CPR;
                const size_t src = (size_t)min(k0 + r, N - 1) * D * ES + cc * 16;
                const u32x4 kw = *(const u32x4*)((const char*)K + src);
                const u32x4 vw = *(const u32x4*)((const char*)V + src);
                *(u32x4*)(sk + r * RS + cc * 16) = kw;
                *(u32x4*)(sv + r * RS + cc * 16) = vw;
            }
        }
        __syncthreads();
        // causal: every key of the tile comes after every row of the wave;
        // padding: only tiles with a padded key take the masked path, and a
        // tile whose keys are all padded adds nothing (the wave took part in
        // the staging and both barriers)
        if (p.causal && k0 > q0 + wave * 16 + 15) continue;
        bool pad_any = false, pad_all = false;
        if (prow) {
            pad_tile(padw, pad_any, pad_all);
            if (pad_all) continue;
        }

        // S^T = K Q^T, 16 keys x 16 queries per block
        f32x4 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = (f32x4){0.f, 0.f, 0.f, 0.f};
            const char* krow = sk + (kb * 16 + col) * RS;
            if constexpr (F32) {
#pragma unroll
                for (int u = 0; u < D / 16; ++u) {
                    const f32x4 kv = *(const f32x4*)(krow + (g * (D / 4) + 4 * u) * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[e], qf[4 * u + e], s[kb], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < NQ; ++ks) {
                    const QV kv = __builtin_bit_cast(QV, *(const u32x4*)(krow + (32 * ks + 8 * g) * ES));
                    s[kb] = M16<T>::mma_s(kv, qf[ks], s[kb]);
                }
            }
        }

        // visibility: accumulator element (kb, i) of this lane is key k0 + 16*kb + 4*g + i
        if (p.causal || pad_any || k0 + BC > N) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = k0 + kb * 16 + 4 * g + i;
                    bool vis = key < N && (!p.causal || key <= qi);
                    if (pad_any) vis = vis && unpadded(padw[kb], i);
                    if (!vis) s[kb][i] = -INFINITY;
                }
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

#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            if constexpr (F32) {
                float pf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pf[i] = fast_exp2(fmaf(s[kb][i], c, -mc));
                    l += pf[i];
                }
                // step i contracts key 16*kb + 4*g + i in lane group g
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const char* vrow = sv + (kb * 16 + 4 * g + i) * RS;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const float a = *(const float*)(vrow + (db * 16 + col) * 4);
                        o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, pf[i], o[db], 0, 0, 0);
                    }
                }
            } else {
                using v2 = typename Dot2<T>::v2;
                const v2 p01 = (v2){(T)fast_exp2(fmaf(s[kb][0], c, -mc)), (T)fast_exp2(fmaf(s[kb][1], c, -mc))};
                const v2 p23 = (v2){(T)fast_exp2(fmaf(s[kb][2], c, -mc)), (T)fast_exp2(fmaf(s[kb][3], c, -mc))};
                l = Dot2<T>::sum2(p01, l);
                l = Dot2<T>::sum2(p23, l);
                // V^T operand: lane 4r+q of each 16-lane group addresses row
                // 16*kb + 4*g + r, columns 16*db + 4q..4q+3; the transposing
                // read hands lane j keys 16*kb + 4*g + 0..3 at column 16*db + j.
                const int r = col >> 2, q = col & 3;
                const char* vrow = sv + (kb * 16 + 4 * g + r) * RS;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4*)(vrow + (db * 16 + 4 * q) * ES));
                    o[db] = M16<T>::mma_pv(a, p01[0], p01[1], p23[0], p23[1], o[db]);
                }
            }
        }
    }

    // epilogue: O = acc / l, lse = m*scale + ln(l); empty rows -> (+0, -inf)
    const float lt = quad_sum(l);
    if (qi < N) {
        const size_t orow = (size_t)bh * N + qi;
        const bool empty = !(lt > 0.f);
        const float inv = empty ? 0.f : 1.f / lt;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d0 = db * 16 + 4 * g;     // accumulator rows are head columns d0..d0+3
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = empty ? 0.f : o[db][i] * inv;
            if (F32 || p.out_f32) {
                *(f32x4*)((float*)p.o + orow * D + d0) = (f32x4){x[0], x[1], x[2], x[3]};
            } else {
                typedef __attribute__((ext_vector_type(4))) T t4;
                *(t4*)((T*)p.o + orow * D + d0) = (t4){(T)x[0], (T)x[1], (T)x[2], (T)x[3]};
            }
        }
        if (p.lse && g == 0)
            p.lse[orow] = empty ? -INFINITY : fmaf(m, p.scale, __builtin_amdgcn_logf(lt) * 0.69314718055994530942f);
    }
}

template <typename T, int D, int BR, int BC>
hipError_t launch_m16(const FwdParams& p, hipStream_t st)
{
    const unsigned grid = (unsigned)(p.B * p.H * p.n_qt);
    hipLaunchKernelGGL((fwd_m16<T, D, BR, BC>), dim3(grid), dim3(BR * 4), 0, st, p);
    return hipGetLastError();
}

}  // namespace attnk
