// bwd.h -- parameters of the attention backward kernels (bwd.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnk {

struct BwdParams {
    const void* q;          // [B][H][N][D], input type
    const void* k;
    const void* v;
    const void* o;          // forward output, input type
    const void* dout;       // gradient of the output, input type
    const float* lse;       // [B][H][N] natural-log lse of the forward
    float* dq;              // [B][H][N][D] fp32
    float* dk;
    float* dv;
    const uint8_t* mask;    // [B][N] or nullptr
    float* dsum;            // [B][H][N] workspace: sum_c dO O
    float* lse2;            // [B][H][N] workspace: lse * log2(e), +inf for empty rows; it follows
                            // dsum in the same workspace (the dK/dV pipeline addresses a head's
                            // lse2 from its dsum with 32-bit offsets, which the host gate sizes)
    int B, H, N;
    float scale;            // natural-log factor of q.k
    float c;                // scale * log2(e)
    int causal;
    int pipe;               // 1: bwd_dkdv and bwd_dq run their full tiles through their pipelines
};

typedef hipError_t (*BwdLaunchFn)(const BwdParams&, hipStream_t);

// dtype_bits: 0 bf16, 1 f16; D in {64, 128}; nullptr otherwise
BwdLaunchFn lookup_bwd(int dtype_bits, int D);

}  // namespace attnk
