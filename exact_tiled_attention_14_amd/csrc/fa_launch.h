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

struct DecodePlan {
    int pages_per_split;   // pages of one sequence handled by one workgroup
    int n_split;           // ranges per sequence at the table's capacity
    int64_t ws_o_elems;    // fp32 partial outputs [nseq, Hq, n_split, 128]
    int64_t ws_lse_elems;  // fp32 partial lse     [nseq, Hq, n_split]
    float* ws_o;
    float* ws_lse;
};

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
DecodePlan plan_decode(int nseq, int Hq, int Hkv, int max_blocks);
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream);

}  // namespace fa
