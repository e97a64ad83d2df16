// decode.h -- parameters of the key-split decode kernels (decode.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnk {

struct DecParams {
    const void* q;          // [B][H][Nq][D]
    const void* k;          // [B][H][Nk][D]
    const void* v;          // [B][H][Nk][D]
    void* o;                // [B][H][Nq][D], input type or float
    float* lse;             // [B][H][Nq] or nullptr
    const uint8_t* mask;    // [B][Nk] or nullptr
    float* part_o;          // [B*H][splits][Nq][D] partial outputs (workspace)
    float* part_lse;        // [B*H][splits][Nq] partial lse (workspace)
    int B, H, Nq, Nk;
    int splits;             // key chunks per (b, h)
    int keys_per_split;     // multiple of the 32-key tile
    float scale;            // natural-log factor of q.k
    float c;                // scale * log2(e)
    float slack;            // lag allowed to the merge reference (0 = exact maximum)
    int qmode;              // non-positive scales, see q_mode16 in fwd_kernel.h
    int causal;             // query row i sees keys j <= Nk - Nq + i
    int out_f32;
};

typedef hipError_t (*DecLaunchFn)(const DecParams&, hipStream_t);

// dtype_bits: 0 bf16, 1 f16; D in {64, 128}; nullptr otherwise
DecLaunchFn lookup_decode(int dtype_bits, int D);

// Device scratch of attn_decode_fwd_noalloc: the same partial outputs and lse
// the caller's workspace holds for attn_decode_fwd, in a fixed array of this
// many bytes that each GPU keeps until the process ends.
constexpr size_t DECODE_SCRATCH_BYTES = (size_t)16 << 20;

// Device address of the scratch array on the current device (looked up with
// hipGetSymbolAddress on the first call on each device, then cached).
hipError_t decode_scratch(void** ptr);

}  // namespace attnk
