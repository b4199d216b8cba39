// Internal launch interface between the C ABI (fa_api.hip) and the kernels.
// Arguments reaching these functions have already been validated.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Events that the next API call on this thread records at its kernel
// boundaries (set by fa_time_next_call; every entry point clears them when it
// returns).
struct CallTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
CallTiming& call_timing();

// Every kernel of the library is launched through here.  With timing events
// set, the first launch of a call records `start` when its kernel begins and
// the launch marked LAST records `stop` when its kernel ends, so the two
// events span exactly the call's kernels.  Launch errors are read with
// hipGetLastError, as after hipLaunchKernelGGL.
template <bool LAST = true, typename... Params, typename... Args>
inline void launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t stream,
                          Args... args) {
    CallTiming& t = call_timing();
    hipEvent_t start = t.start;
    t.start = nullptr;
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, start, LAST ? t.stop : nullptr, 0u, args...);
}

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, Hq, Hkv, Sq, Sk, d;
    int causal;
    float scale;
    int sync_spins;        // poll bound of the wave-group barriers (pair grid)
};

// Default poll bound of a wave-group barrier, and the bound the next fa_fwd
// (or fa_fwd_fp8 or fa_bwd) call on this thread uses (set by
// fa_limit_next_sync_wait).
constexpr int kDefaultSyncSpins = 1 << 22;
int& next_sync_spins();
// Reads and clears the device's count of wave-group barrier timeouts.
hipError_t read_sync_timeouts(unsigned int* count);
// The same for the backward's pair-grid dQ kernel and the FP8 forward.
hipError_t read_bwd_sync_timeouts(unsigned int* count);
hipError_t read_fp8_sync_timeouts(unsigned int* count);
// Reads a device-side unsigned counter (the address of a __device__ variable
// in host code, which names its symbol) of the current device once every queued kernel has finished,
// and clears it.
hipError_t read_device_counter(const void* symbol, unsigned int* count);

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
    int sync_spins;        // poll bound of the wave-group barriers (pair-grid dQ)
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

struct DecodeMqArgs {
    const void* q;         // [nseq, Sq, Hq, 128]
    const void* kcache;
    const void* vcache;
    const int32_t* block_table;
    const int32_t* seqlens;
    void* o;               // [nseq, Sq, Hq, 128]
    float* lse;            // [nseq, Sq, Hq] or nullptr
    int nseq, Sq, Hq, Hkv, max_blocks, num_blocks;
    float scale;
};

size_t decode_mq_workspace_bytes(int nseq, int Hkv, int max_blocks);
hipError_t launch_decode_mq(const DecodeMqArgs& a, void* workspace, hipStream_t stream);

// Latent-cache decode: H query heads of 128 over a paged cache of 512-wide
// latents, with per-head up-projections.
struct MlaArgs {
    const void* q;         // [nseq, H, 128]
    const void* w_uk;      // [H, 512, 128]
    const void* w_uv_t;    // [H, 128, 512]
    const void* ccache;    // [num_blocks, 16, 512]
    const int32_t* block_table;
    const int32_t* seqlens;
    void* o;               // [nseq, H, 128]
    float* lse;            // [nseq, H] or nullptr
    int nseq, H, max_blocks, num_blocks;
    float scale;
};

size_t mla_workspace_bytes(int nseq, int H, int max_blocks);
hipError_t launch_mla_decode(const MlaArgs& a, void* workspace, hipStream_t stream);

// FP8 block quantization of a [BH, S, 128] bf16 tensor.
struct QuantArgs {
    const void* x;
    const void* rot;       // [128, 128] bf16 or nullptr
    void* x8;
    uint8_t* scales;       // [BH, ceil(S / block_rows)] E8M0 bytes
    int64_t BH;
    int S, block_rows;
    int layout;            // 0 rows, 1 d-major 64-key V blocks
};

struct Fp8FwdArgs {
    const void* q8;        // E4M3 codes, or bf16 Q when q_bf16 is set
    const void* k8;
    const void* v8;        // d-major 64-key blocks
    const uint8_t* q_scale;
    const uint8_t* k_scale;
    const uint8_t* v_scale;
    void* o;
    float* lse;
    int B, Hq, Hkv, Sq, Sk;
    int causal;
    float scale;
    int sync_spins;        // poll bound of the wave-group barriers (pair grid)
    int q_bf16;            // q8 is bf16 Q, quantized by the kernel (q_scale unused)
    const void* rot;       // with q_bf16: bf16 [128, 128] rotation of Q, or NULL
};

hipError_t launch_quant_fp8(const QuantArgs& a, hipStream_t stream);
// Q (128-row blocks, rotated), K (64-row blocks, rotated) and V (64-key d-major
// blocks) in one launch; the rotation is q.rot (k.rot must be the same).
hipError_t launch_quant_fp8_qkv(const QuantArgs& q, const QuantArgs& k, const QuantArgs& v, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);
// Bytes of device scratch launch_decode uses (256-byte aligned sections).
size_t decode_workspace_bytes(int nseq, int Hq, int Hkv);
hipError_t launch_decode(const DecodeArgs& a, void* workspace, hipStream_t stream);
// The decode with its scratch in a fixed device array of this many bytes per
// GPU instead of a caller workspace (needs decode_workspace_bytes <= it).
constexpr size_t kDecodeNoallocScratchBytes = size_t(32) << 20;
hipError_t launch_decode_noalloc(const DecodeArgs& a, hipStream_t stream);

}  // namespace fa
