// naive_kernel.h -- baseline attention that materialises the score matrix
// (the "baseline attention" the stability paper compares FlashAttention with):
// S = scale * Q K^T stored in the input type, row softmax in fp32 stored back in
// the input type, then O = P V with fp32 accumulation.  Comparison only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnk {

struct NaiveParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const uint8_t* mask;
    void* ws;              // B*H*N*N elements of the input type
    int B, H, N, d;
    float scale;
    int causal;
    int in_kind;           // 0 float, 1 half, 2 bfloat16
    int out_f32;
};

hipError_t naive_launch(const NaiveParams& p, hipStream_t st);

}  // namespace attnk
