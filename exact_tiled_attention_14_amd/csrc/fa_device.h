// Device-side helpers shared by the attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_inff();

// v_exp_f32: 2^x; 2^(-inf) = 0.
__device__ __forceinline__ float exp2f_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// v_log_f32: log2(x); log2(0) = -inf.
__device__ __forceinline__ float log2f_hw(float x) { return __builtin_amdgcn_logf(x); }

// bf16 bit pattern -> the equal fp32 value.
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values -> two bf16 (round to nearest even) packed low-first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// 32x32x16 bf16 matrix-core product with fp32 accumulation, D = A B + C.
// Operand a: lane l holds row (l % 32) of A, 8 contraction elements; operand b:
// lane l holds column (l % 32) of B, the same 8 contraction elements.  The
// accumulator holds D[i][j] in lane j + 32 * ((i / 4) % 2), register
// 4 * (i / 8) + i % 4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max / sum of a value over lanes l and l ^ 32 (the two halves of a wave),
// returned in every lane; one cross-lane VALU swap, no LDS round trip.
__device__ __forceinline__ float half_swap_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lane x moved by a DPP control within its 16-lane row (bound_ctrl: lanes
// the pattern does not feed read 0).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);   // row_half_mirror
    x += dpp<0x140>(x);   // row_mirror
    return x;
}

// Buffer load to LDS of 16 bytes per lane: lane l's bytes [voff, voff + 16)
// past `base` (plus the uniform `soff`) land at byte 16 l of the 1 KiB LDS
// slice `lds`.  `bytes` bounds the addressed range from `base`.  The buffer
// form matters for the waits: the compiler counts the global-to-LDS load as
// both a memory and an LDS access, and while one is outstanding it turns
// every wait for an LDS operand read into a wait for all of them.
__device__ __forceinline__ void buffer_load_lds16(const void* base, uint32_t bytes, uint8_t* lds, uint32_t voff,
                                                  uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)   // (the buffer builtins exist only for the device pass)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
#endif
}

// Barrier of the four waves of one wave group (two groups share a
// workgroup), through a counter in LDS: each wave adds 1 on arrival and
// leaves once all four have arrived for this round (the counter grows by 4
// per round; `target` is the wave's running round total).  The wait is
// bounded by `spins` polls, so no wave can spin forever; a wait that runs out
// is counted in `*timeouts` (a device-wide counter of the calling source) and
// returned as true, and the caller marks its rows as failed.
__device__ __forceinline__ bool group_barrier(uint8_t* ctr_p, int& target, int lane, int spins,
                                              unsigned int* timeouts) {
    int* const ctr = reinterpret_cast<int*>(ctr_p);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    target += 4;
    if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    bool timed_out = false;
    for (int spin = 0;; ++spin) {
        const int c = __builtin_amdgcn_readfirstlane(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (c >= target) break;
        if (spin >= spins) {
            timed_out = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    if (timed_out && lane == 0) __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return timed_out;
}

// ---- FP8 block encoding, one definition for the quantizer and the forward
// that quantizes Q itself, so both give the same codes ----

// E8M0 exponent of a block scale 2^e: the smallest e with amax <= 448 2^e.
// amax = M 2^E with M in [1, 2) and 448 = 1.75 2^8, so e = E - 8, plus one
// when M > 1.75; clamped to the E8M0 range; amax = 0 gives e = 0.
__device__ __forceinline__ int fp8_scale_exp(float amax) {
    if (!(amax > 0.f)) return 0;
    const uint32_t b = __float_as_uint(amax);
    const int E = (int)((b >> 23) & 255u) - 127;
    const int e = E - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return min(max(e, -127), 127);
}

// 2^-e as an fp32 value (e in [-127, 120] for any finite fp32 amax).
__device__ __forceinline__ float fp8_inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// Four fp32 values -> four E4M3 bytes (round to nearest even), low byte first.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

// Stage the 128 x 128 bf16 rotation R in LDS with NT threads, all loads in
// flight together; 16-byte chunk c of row n sits at chunk c ^ (n % 16), so
// operand reads of 32 rows and one chunk spread over all banks.  The caller
// issues the barrier.
template <int NT>
__device__ __forceinline__ void stage_rotation128(const uint16_t* __restrict__ rot, uint16_t* rt, int tid) {
    constexpr int D = 128;
    constexpr int NST = D * D / 8 / NT;
    static_assert(NST * NT * 8 == D * D, "staging split");
    u32x4 rv[NST];
#pragma unroll
    for (int i = 0; i < NST; ++i) {
        const int c = tid + NT * i;
        rv[i] = *reinterpret_cast<const u32x4*>(rot + (c / (D / 8)) * D + 8 * (c % (D / 8)));
    }
#pragma unroll
    for (int i = 0; i < NST; ++i) {
        const int c = tid + NT * i;
        const int n = c / (D / 8), ch = c % (D / 8);
        *reinterpret_cast<u32x4*>(rt + n * D + 8 * (ch ^ (n & 15))) = rv[i];
    }
}

// Row (lane % 32 is the column) index of accumulator register r in lane half h.
__device__ __forceinline__ constexpr int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

}  // namespace fa
