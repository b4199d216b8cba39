// Internal launch interface between the C ABI (fa_api.hip) and the kernels.
// Arguments reaching these functions have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv, Sq, Sk, d;
    int causal;
    float scale;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* delta;          // [B, Hq, Sq] fp32 scratch
    int B, Hq, Hkv, Sq, Sk, d;
    int causal;
    float scale;
};

struct DecodeArgs {
    const void* q;
    const void* kcache;
    const void* vcache;
    const int32_t* block_table;
    const int32_t* seqlens;
    void* o;
    float* lse;
    int nseq, Hq, Hkv, max_blocks, num_blocks;
    float scale;
};

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);
// Bytes of device scratch launch_decode uses (256-byte aligned sections).
size_t decode_workspace_bytes(int nseq, int Hq, int Hkv);
hipError_t launch_decode(const DecodeArgs& a, void* workspace, hipStream_t stream);

}  // namespace fa
