// naive.hip -- kernels of the materialising baseline (see naive_kernel.h).
#include "naive_kernel.h"

namespace attnk {
namespace {

template <typename T> __device__ __forceinline__ float ld(const T* p, size_t i) { return (float)p[i]; }
template <typename T> __device__ __forceinline__ void st(T* p, size_t i, float x) { p[i] = (T)x; }

constexpr int TM = 64, TN = 64, TK = 16;

// C[i][j] = alpha * sum_c A[i][c] * B(c, j) for one (b, h).
//   B_T = true : B(c, j) = Bm[j][c]   (scores: B is K, row-major [N][d])
//   B_T = false: B(c, j) = Bm[c][j]   (output: B is V, row-major [N][d])
// A is [M][KD] row-major; C is [M][NC] row-major.  256 threads, 4x4 outputs each.
template <typename TA, typename TB, typename TC, bool B_T>
__global__ void __launch_bounds__(256)
gemm_simt(const TA* __restrict__ A, const TB* __restrict__ Bm, TC* __restrict__ C,
          int M, int NC, int KD, size_t strideA, size_t strideB, size_t strideC, float alpha)
{
    __shared__ float As[TK][TM + 4];
    __shared__ float Bs[TK][TN + 4];
    const int bh = blockIdx.z;
    A += bh * strideA; Bm += bh * strideB; C += bh * strideC;
    const int i0 = blockIdx.y * TM, j0 = blockIdx.x * TN;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int c0 = 0; c0 < KD; c0 += TK) {
        for (int e = threadIdx.x; e < TK * TM; e += 256) {
            const int r = e / TK, c = e % TK;        // A tile: row r, column c
            const int gi = i0 + r, gc = c0 + c;
            As[c][r] = (gi < M && gc < KD) ? ld(A, (size_t)gi * KD + gc) : 0.f;
        }
        for (int e = threadIdx.x; e < TK * TN; e += 256) {
            if (B_T) {
                const int r = e / TK, c = e % TK;    // B^T row j0+r, column c0+c
                const int gj = j0 + r, gc = c0 + c;
                Bs[c][r] = (gj < NC && gc < KD) ? ld(Bm, (size_t)gj * KD + gc) : 0.f;
            } else {
                const int c = e / TN, r = e % TN;    // B row c0+c, column j0+r
                const int gj = j0 + r, gc = c0 + c;
                Bs[c][r] = (gj < NC && gc < KD) ? ld(Bm, (size_t)gc * NC + gj) : 0.f;
            }
        }
        __syncthreads();
        for (int c = 0; c < TK; ++c) {
            float a[4], bb[4];
            for (int u = 0; u < 4; ++u) { a[u] = As[c][ty * 4 + u]; bb[u] = Bs[c][tx * 4 + u]; }
            for (int u = 0; u < 4; ++u)
                for (int w = 0; w < 4; ++w) acc[u][w] = fmaf(a[u], bb[w], acc[u][w]);
        }
        __syncthreads();
    }
    for (int u = 0; u < 4; ++u)
        for (int w = 0; w < 4; ++w) {
            const int gi = i0 + ty * 4 + u, gj = j0 + tx * 4 + w;
            if (gi < M && gj < NC) st(C, (size_t)gi * NC + gj, alpha * acc[u][w]);
        }
}

// One workgroup per score row: masked entries are excluded, P = exp(s - max) /
// sum in fp32, stored back in place; fully masked rows get P = 0, lse = -inf.
template <typename T>
__global__ void __launch_bounds__(256)
row_softmax(T* __restrict__ S, float* __restrict__ lse, const uint8_t* __restrict__ mask,
            int H, int N, int causal)
{
    __shared__ float red[256];
    const size_t row = blockIdx.x;                 // (b*H + h)*N + i
    const int i = (int)(row % N);
    const int b = (int)(row / N / H);
    T* s = S + row * (size_t)N;
    auto vis = [&](int j) { return (!causal || j <= i) && (!mask || mask[(size_t)b * N + j] == 0); };
    float mx = -INFINITY;
    for (int j = threadIdx.x; j < N; j += 256)
        if (vis(j)) mx = fmaxf(mx, ld(s, j));
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
        __syncthreads();
    }
    mx = red[0];
    __syncthreads();
    float sum = 0.f;
    if (mx != -INFINITY)
        for (int j = threadIdx.x; j < N; j += 256)
            if (vis(j)) sum += expf(ld(s, j) - mx);
    red[threadIdx.x] = sum;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    sum = red[0];
    const bool empty = !(sum > 0.f);
    for (int j = threadIdx.x; j < N; j += 256)
        st(s, j, (empty || !vis(j)) ? 0.f : expf(ld(s, j) - mx) / sum);
    if (lse && threadIdx.x == 0) lse[row] = empty ? -INFINITY : mx + logf(sum);
}

template <typename T>
hipError_t run(const NaiveParams& p, hipStream_t stream)
{
    const int N = p.N, d = p.d, BH = p.B * p.H;
    const T* q = (const T*)p.q;
    const T* k = (const T*)p.k;
    const T* v = (const T*)p.v;
    T* S = (T*)p.ws;
    const size_t sN = (size_t)N * N, sd = (size_t)N * d;
    dim3 g1((N + TN - 1) / TN, (N + TM - 1) / TM, BH);
    hipLaunchKernelGGL((gemm_simt<T, T, T, true>), g1, dim3(256), 0, stream, q, k, S, N, N, d, sd, sd, sN, p.scale);
    hipLaunchKernelGGL((row_softmax<T>), dim3((unsigned)((size_t)BH * N)), dim3(256), 0, stream,
                       S, p.lse, p.mask, p.H, N, p.causal);
    dim3 g3((d + TN - 1) / TN, (N + TM - 1) / TM, BH);
    if (p.out_f32)
        hipLaunchKernelGGL((gemm_simt<T, T, float, false>), g3, dim3(256), 0, stream, (const T*)S, v, (float*)p.o, N, d, N, sN, sd, sd, 1.f);
    else
        hipLaunchKernelGGL((gemm_simt<T, T, T, false>), g3, dim3(256), 0, stream, (const T*)S, v, (T*)p.o, N, d, N, sN, sd, sd, 1.f);
    return hipGetLastError();
}

}  // namespace

hipError_t naive_launch(const NaiveParams& p, hipStream_t st)
{
    switch (p.in_kind) {
    case 0: return run<float>(p, st);
    case 1: return run<_Float16>(p, st);
    default: return run<__bf16>(p, st);
    }
}

}  // namespace attnk
