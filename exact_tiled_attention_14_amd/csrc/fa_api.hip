// The C ABI declared in include/fa.h: host-side validation and dispatch.
// Nothing here allocates, frees or synchronises; every launch goes to the
// caller's stream.
#include <cmath>
#include <cstdint>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Elements of a tensor must fit the 64-bit offsets the kernels use.
bool fits(int64_t a, int64_t b, int64_t c, int64_t d) {
    const int64_t lim = INT64_MAX / 4;
    int64_t x = a;
    for (int64_t y : {b, c, d}) {
        if (y != 0 && x > lim / y) return false;
        x *= y;
    }
    return true;
}

// Clears the timing events of fa_time_next_call when an entry point returns,
// whether or not it launched anything.
struct TimingScope {
    ~TimingScope() { fa::call_timing() = fa::CallTiming{}; }
};

// Restores the default barrier poll bound when fa_fwd, fa_fwd_fp8 or fa_bwd
// returns.
struct SpinScope {
    ~SpinScope() { fa::next_sync_spins() = fa::kDefaultSyncSpins; }
};

}  // namespace

namespace fa {
CallTiming& call_timing() {
    static thread_local CallTiming t;
    return t;
}
int& next_sync_spins() {
    static thread_local int n = kDefaultSyncSpins;
    return n;
}
hipError_t read_device_counter(const void* symbol, unsigned int* count) {
    // every kernel that may still add to the counter finishes first
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return e;
    unsigned int n = 0;
    e = hipMemcpyFromSymbol(&n, symbol, sizeof(n), 0, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return e;
    const unsigned int zero = 0;
    e = hipMemcpyToSymbol(symbol, &zero, sizeof(zero), 0, hipMemcpyHostToDevice);
    if (e != hipSuccess) return e;
    *count = n;
    return hipDeviceSynchronize();
}
}  // namespace fa

extern "C" {

int fa_time_next_call(void* start_event, void* stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr)) return FA_ERR_INVALID_ARG;
    fa::call_timing() = fa::CallTiming{static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
    return FA_OK;
}

int fa_limit_next_sync_wait(int spins) {
    if (spins < 0) return FA_ERR_INVALID_ARG;
    fa::next_sync_spins() = spins;
    return FA_OK;
}

int fa_sync_timeouts(unsigned int* count) {
    if (count == nullptr) return FA_ERR_INVALID_ARG;
    unsigned int nf = 0, nb = 0, n8 = 0;
    if (fa::read_sync_timeouts(&nf) != hipSuccess || fa::read_bwd_sync_timeouts(&nb) != hipSuccess ||
        fa::read_fp8_sync_timeouts(&n8) != hipSuccess)
        return FA_ERR_HIP;
    *count = nf + nb + n8;
    return FA_OK;
}

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
        case FA_ERR_HIP: return "FA_ERR_HIP";
        default: return "FA_UNKNOWN_STATUS";
    }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
           int Sq, int Sk, int d, int causal, float scale, int dtype, void* stream) {
    TimingScope timing_scope;
    SpinScope spin_scope;
    if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_INVALID_ARG;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return FA_ERR_INVALID_ARG;
    if (!fits(B, Hq, Sq, d) || !fits(B, Hkv, Sk, d)) return FA_ERR_INVALID_ARG;
    if (dtype == FA_BF16) {
        if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    } else if (dtype == FA_F32) {
        if (d != 32 && d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    } else {
        return FA_ERR_INVALID_ARG;
    }
    // The grid is one workgroup per (batch, query head, query block).
    const int64_t rows_per_wg = dtype == FA_BF16 ? 128 : 16;   // query rows per workgroup of each kernel
    if ((int64_t)B * Hq * ((Sq + rows_per_wg - 1) / rows_per_wg) > INT32_MAX) return FA_ERR_UNSUPPORTED;

    fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, causal, scale, fa::next_sync_spins()};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e = dtype == FA_BF16 ? fa::launch_fwd_bf16(a, s) : fa::launch_fwd_f32(a, s);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int B, int Hq, int Sq) {
    if (B < 1 || Hq < 1 || Sq < 1 || !fits(B, Hq, Sq, 4)) return 0;
    return ((size_t)B * Hq * Sq * sizeof(float) + 255) & ~(size_t)255;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale,
           void* workspace, size_t workspace_bytes, void* stream) {
    TimingScope timing_scope;
    SpinScope spin_scope;
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0 || (causal != 0 && causal != 1)) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    for (const void* p : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(lse) & 3u) return FA_ERR_INVALID_ARG;
    if (!fits(B, Hq, Sq, d) || !fits(B, Hkv, Sk, d)) return FA_ERR_INVALID_ARG;
    if (d != 128) return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * Hq * ((Sq + 127) / 128) > INT32_MAX || (int64_t)B * Hkv * ((Sk + 127) / 128) > INT32_MAX ||
        ((int64_t)B * Hq * Sq + 15) / 16 > INT32_MAX)
        return FA_ERR_UNSUPPORTED;
    const size_t need = fa_bwd_workspace_size(B, Hq, Sq);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return FA_ERR_WORKSPACE;

    fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, static_cast<float*>(workspace), B, Hq, Hkv, Sq, Sk, d,
                  causal, scale, fa::next_sync_spins()};
    const hipError_t e = fa::launch_bwd_bf16(a, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_quantize_fp8_bytes(int B, int H, int S, int d, int layout) {
    if (B < 1 || H < 1 || S < 1 || d != 128 || !fits(B, H, S, d)) return 0;
    if (layout == FA_FP8_ROWS) return (size_t)B * H * S * d;
    if (layout == FA_FP8_VBLOCKS) return (size_t)B * H * ((S + 63) / 64) * 64 * d;
    return 0;
}

int fa_quantize_fp8(const void* x, const void* rot, void* x8, uint8_t* scales, int B, int H, int S, int d,
                    int block_rows, int layout, void* stream) {
    TimingScope timing_scope;
    if (!x || !x8 || !scales) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || S < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (layout != FA_FP8_ROWS && layout != FA_FP8_VBLOCKS) return FA_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(x8) || (rot && !aligned16(rot))) return FA_ERR_INVALID_ARG;
    if (!fits(B, H, S, d)) return FA_ERR_INVALID_ARG;
    if (d != 128) return FA_ERR_UNSUPPORTED;
    if (layout == FA_FP8_ROWS && block_rows != 64 && block_rows != 128) return FA_ERR_UNSUPPORTED;
    if (layout == FA_FP8_VBLOCKS && (block_rows != 64 || rot != nullptr)) return FA_ERR_UNSUPPORTED;
    fa::QuantArgs a{x, rot, x8, scales, (int64_t)B * H, S, block_rows, layout};
    return fa::launch_quant_fp8(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_quantize_fp8_qkv(const void* q, const void* k, const void* v, const void* rot, void* q8,
                        uint8_t* q_scales, void* k8, uint8_t* k_scales, void* v8, uint8_t* v_scales, int B,
                        int Hq, int Hkv, int Sq, int Sk, int d, void* stream) {
    TimingScope timing_scope;
    if (!q || !k || !v || !q8 || !k8 || !v8 || !q_scales || !k_scales || !v_scales) return FA_ERR_INVALID_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q8) || !aligned16(k8) || !aligned16(v8) ||
        (rot && !aligned16(rot)))
        return FA_ERR_INVALID_ARG;
    if (!fits(B, Hq, Sq, d) || !fits(B, Hkv, Sk + 63, d)) return FA_ERR_INVALID_ARG;
    if (d != 128) return FA_ERR_UNSUPPORTED;
    const fa::QuantArgs aq{q, rot, q8, q_scales, (int64_t)B * Hq, Sq, 128, FA_FP8_ROWS};
    const fa::QuantArgs ak{k, rot, k8, k_scales, (int64_t)B * Hkv, Sk, 64, FA_FP8_ROWS};
    const fa::QuantArgs av{v, nullptr, v8, v_scales, (int64_t)B * Hkv, Sk, 64, FA_FP8_VBLOCKS};
    return fa::launch_quant_fp8_qkv(aq, ak, av, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK
                                                                                                     : FA_ERR_HIP;
}

int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const uint8_t* q_scale, const uint8_t* k_scale,
               const uint8_t* v_scale, void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal,
               float scale, void* stream) {
    TimingScope timing_scope;
    SpinScope spin_scope;
    if (!q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale || !o) return FA_ERR_INVALID_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0 || (causal != 0 && causal != 1)) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o)) return FA_ERR_INVALID_ARG;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return FA_ERR_INVALID_ARG;
    if (!fits(B, Hq, Sq, d) || !fits(B, Hkv, Sk + 63, d)) return FA_ERR_INVALID_ARG;
    if (d != 128) return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * Hq * ((Sq + 127) / 128) > INT32_MAX) return FA_ERR_UNSUPPORTED;
    fa::Fp8FwdArgs a{q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, Sq, Sk, causal, scale,
                     fa::next_sync_spins(), 0, nullptr};
    return fa::launch_fwd_fp8(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_fp8_qbf16(const void* q, const void* rot, const void* k8, const void* v8, const uint8_t* k_scale,
                     const uint8_t* v_scale, void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int d,
                     int causal, float scale, void* stream) {
    TimingScope timing_scope;
    SpinScope spin_scope;
    if (!q || !k8 || !v8 || !k_scale || !v_scale || !o) return FA_ERR_INVALID_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0 || (causal != 0 && causal != 1)) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k8) || !aligned16(v8) || !aligned16(o) || (rot && !aligned16(rot)))
        return FA_ERR_INVALID_ARG;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return FA_ERR_INVALID_ARG;
    if (!fits(B, Hq, Sq, d) || !fits(B, Hkv, Sk + 63, d)) return FA_ERR_INVALID_ARG;
    if (d != 128) return FA_ERR_UNSUPPORTED;
    if ((int64_t)B * Hq * ((Sq + 127) / 128) > INT32_MAX) return FA_ERR_UNSUPPORTED;
    fa::Fp8FwdArgs a{q, k8, v8, nullptr, k_scale, v_scale, o, lse, B, Hq, Hkv, Sq, Sk, causal, scale,
                     fa::next_sync_spins(), 1, rot};
    return fa::launch_fwd_fp8(a, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_decode_workspace_size(int nseq, int Hq, int Hkv, int d, int block_size, int max_blocks_per_seq) {
    if (nseq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_blocks_per_seq < 1) return 0;
    if (d != 128 || block_size != 16) return 0;
    return fa::decode_workspace_bytes(nseq, Hq, Hkv);
}

}  // extern "C"

namespace {

// Host-side checks shared by fa_decode and fa_decode_noalloc.
int check_decode(const void* q, const void* kcache, const void* vcache, const int32_t* block_table,
                 const int32_t* seqlens, const void* o, const float* lse, int nseq, int Hq, int Hkv, int d,
                 int block_size, int max_blocks_per_seq, int num_blocks, float scale) {
    if (!q || !kcache || !vcache || !block_table || !seqlens || !o) return FA_ERR_INVALID_ARG;
    if (nseq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_blocks_per_seq < 1 || num_blocks < 1)
        return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(o)) return FA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seqlens) & 3u))
        return FA_ERR_INVALID_ARG;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return FA_ERR_INVALID_ARG;
    if (d != 128 || block_size != 16) return FA_ERR_UNSUPPORTED;
    const int g = Hq / Hkv;
    if (g != 1 && g != 2 && g != 4 && g != 8) return FA_ERR_UNSUPPORTED;
    if (nseq > 65535 || Hkv > 65535) return FA_ERR_UNSUPPORTED;   // grid y limit of the combine step
    // pages of all (sequence, K/V head) pairs at the table's capacity: the
    // work split counts them in 32 bits per wave
    if ((int64_t)nseq * Hkv * max_blocks_per_seq > INT32_MAX) return FA_ERR_UNSUPPORTED;
    if (!fits(num_blocks, Hkv, block_size, d) || (int64_t)max_blocks_per_seq * block_size > INT32_MAX)
        return FA_ERR_INVALID_ARG;
    return FA_OK;
}

}  // namespace

static_assert(fa::kDecodeNoallocScratchBytes == FA_DECODE_NOALLOC_SCRATCH_BYTES,
              "the header states the scratch size of fa_decode_noalloc");

extern "C" {

int fa_decode(const void* q, const void* kcache, const void* vcache, const int32_t* block_table,
              const int32_t* seqlens, void* o, float* lse, int nseq, int Hq, int Hkv, int d, int block_size,
              int max_blocks_per_seq, int num_blocks, float scale, void* workspace, size_t workspace_bytes,
              void* stream) {
    TimingScope timing_scope;
    const int st = check_decode(q, kcache, vcache, block_table, seqlens, o, lse, nseq, Hq, Hkv, d, block_size,
                                max_blocks_per_seq, num_blocks, scale);
    if (st != FA_OK) return st;
    const size_t need = fa_decode_workspace_size(nseq, Hq, Hkv, d, block_size, max_blocks_per_seq);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return FA_ERR_WORKSPACE;

    fa::DecodeArgs a{q, kcache, vcache, block_table, seqlens, o, lse, nseq, Hq, Hkv, max_blocks_per_seq,
                     num_blocks, scale};
    const hipError_t e = fa::launch_decode(a, workspace, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_decode_noalloc(const void* q, const void* kcache, const void* vcache, const int32_t* block_table,
                      const int32_t* seqlens, void* o, float* lse, int nseq, int Hq, int Hkv, int d, int block_size,
                      int max_blocks_per_seq, int num_blocks, float scale, void* stream) {
    TimingScope timing_scope;
    const int st = check_decode(q, kcache, vcache, block_table, seqlens, o, lse, nseq, Hq, Hkv, d, block_size,
                                max_blocks_per_seq, num_blocks, scale);
    if (st != FA_OK) return st;
    if (fa_decode_workspace_size(nseq, Hq, Hkv, d, block_size, max_blocks_per_seq) > fa::kDecodeNoallocScratchBytes)
        return FA_ERR_WORKSPACE;
    fa::DecodeArgs a{q, kcache, vcache, block_table, seqlens, o, lse, nseq, Hq, Hkv, max_blocks_per_seq,
                     num_blocks, scale};
    const hipError_t e = fa::launch_decode_noalloc(a, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_decode_multi_workspace_size(int nseq, int Sq, int Hq, int Hkv, int d, int block_size,
                                      int max_blocks_per_seq) {
    if (nseq < 1 || Sq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_blocks_per_seq < 1) return 0;
    if (d != 128 || block_size != 16) return 0;
    return fa::decode_mq_workspace_bytes(nseq, Hkv, max_blocks_per_seq);
}

int fa_decode_multi(const void* q, const void* kcache, const void* vcache, const int32_t* block_table,
                    const int32_t* seqlens, void* o, float* lse, int nseq, int Sq, int Hq, int Hkv, int d,
                    int block_size, int max_blocks_per_seq, int num_blocks, float scale, void* workspace,
                    size_t workspace_bytes, void* stream) {
    TimingScope timing_scope;
    if (!q || !kcache || !vcache || !block_table || !seqlens || !o) return FA_ERR_INVALID_ARG;
    if (nseq < 1 || Sq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_blocks_per_seq < 1 || num_blocks < 1)
        return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(o)) return FA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seqlens) & 3u))
        return FA_ERR_INVALID_ARG;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return FA_ERR_INVALID_ARG;
    if (!fits(nseq, Sq, Hq, d) || !fits(num_blocks, Hkv, block_size, d) ||
        (int64_t)max_blocks_per_seq * block_size > INT32_MAX)
        return FA_ERR_INVALID_ARG;
    if (d != 128 || block_size != 16) return FA_ERR_UNSUPPORTED;
    const int g = Hq / Hkv;
    if ((g != 1 && g != 2 && g != 4 && g != 8) || g * Sq > 32) return FA_ERR_UNSUPPORTED;
    const int64_t nchunk = (max_blocks_per_seq + 127) / 128;
    if (nchunk * nseq * Hkv > INT32_MAX) return FA_ERR_UNSUPPORTED;
    const size_t need = fa_decode_multi_workspace_size(nseq, Sq, Hq, Hkv, d, block_size, max_blocks_per_seq);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return FA_ERR_WORKSPACE;
    fa::DecodeMqArgs a{q, kcache, vcache, block_table, seqlens, o, lse, nseq, Sq, Hq, Hkv, max_blocks_per_seq,
                       num_blocks, scale};
    return fa::launch_decode_mq(a, workspace, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK
                                                                                                  : FA_ERR_HIP;
}

size_t fa_mla_decode_workspace_size(int nseq, int H, int d_h, int d_c, int block_size, int max_blocks_per_seq) {
    if (nseq < 1 || H < 1 || max_blocks_per_seq < 1) return 0;
    if (d_h != 128 || d_c != 512 || block_size != 16 || H > 128) return 0;
    return fa::mla_workspace_bytes(nseq, H, max_blocks_per_seq);
}

int fa_mla_decode(const void* q, const void* w_uk, const void* w_uv_t, const void* ccache,
                  const int32_t* block_table, const int32_t* seqlens, void* o, float* lse, int nseq, int H,
                  int d_h, int d_c, int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                  void* workspace, size_t workspace_bytes, void* stream) {
    TimingScope timing_scope;
    if (!q || !w_uk || !w_uv_t || !ccache || !block_table || !seqlens || !o) return FA_ERR_INVALID_ARG;
    if (nseq < 1 || H < 1 || d_h < 1 || d_c < 1 || block_size < 1 || max_blocks_per_seq < 1 || num_blocks < 1)
        return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(w_uk) || !aligned16(w_uv_t) || !aligned16(ccache) || !aligned16(o))
        return FA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seqlens) & 3u))
        return FA_ERR_INVALID_ARG;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return FA_ERR_INVALID_ARG;
    if (!fits(nseq, H, d_h, 1) || !fits(H, d_c, d_h, 1) || !fits(num_blocks, block_size, d_c, 1) ||
        (int64_t)max_blocks_per_seq * block_size > INT32_MAX)
        return FA_ERR_INVALID_ARG;
    if (d_h != 128 || d_c != 512 || block_size != 16 || H > 128) return FA_ERR_UNSUPPORTED;
    // work items of the partial kernel (grid x) and sequence blocks of the
    // projections (grid z) stay within the launch limits
    if ((int64_t)nseq * max_blocks_per_seq > INT32_MAX / 2 || nseq > 65535 * 32) return FA_ERR_UNSUPPORTED;
    const size_t need = fa_mla_decode_workspace_size(nseq, H, d_h, d_c, block_size, max_blocks_per_seq);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return FA_ERR_WORKSPACE;
    fa::MlaArgs a{q, w_uk, w_uv_t, ccache, block_table, seqlens, o, lse, nseq, H, max_blocks_per_seq, num_blocks,
                  scale};
    return fa::launch_mla_decode(a, workspace, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK
                                                                                                 : FA_ERR_HIP;
}

}  // extern "C"
