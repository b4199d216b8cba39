// FP8 block quantization for the FP8 attention forward, gfx950.
//
// "FlashAttention scaling, multi-GPU training and weight quantization",
// section 1 (FP8 support): Q, K and V are stored in an 8-bit float format,
// each small tile with its own scale (block quantization), and Q and K are
// multiplied by a random orthogonal matrix first (incoherent processing), so
// that Q K^T is unchanged while an outlier spreads over the head dimension.
//
// Encoding: OCP E4M3 with round-to-nearest-even (the hardware conversion
// v_cvt_pk_fp8_f32).  Block scale: 2^e with e the smallest integer such that
// amax <= 448 * 2^e, stored as its E8M0 byte e + 127, which is the format the
// matrix cores' scaled products take directly.
//
//   * quant_rows_kernel: rows of a [S, 128] slice, optionally rotated
//     (each row x -> R x on the matrix cores as D = R X^T, R's rows being the
//     A operand, staged in LDS once per workgroup; without R the identity is
//     staged, which is exact), written row-major.
//   * quant_v_kernel: 64-key blocks of V (no rotation), written d-major: per
//     block 128 rows (one per head-dim index) of 64 bytes, the keys of a row in
//     the order in which the attention kernel's lanes hold P (see include/fa.h),
//     so the PV product reads its operand without any transposition.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kQD = 128;
constexpr int kQThreads = 256;

// E8M0 exponent of the block scale: amax = M 2^E with M in [1, 2); since
// 448 = 1.75 * 2^8, e = E - 8, plus one when M > 1.75.  e is clamped to the
// E8M0 range; amax = 0 gives e = 0.
__device__ __forceinline__ int scale_exp(float amax) {
    if (!(amax > 0.f)) return 0;
    const uint32_t b = __float_as_uint(amax);
    const int E = (int)((b >> 23) & 255u) - 127;
    const int e = E - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return min(max(e, -127), 127);
}

// 2^-e as an fp32 value (e in [-127, 120] for any finite fp32 amax).
__device__ __forceinline__ float inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

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

// Largest |value| over the workgroup; every thread gets it.  `red` holds one
// float per wave; the caller separates consecutive uses with a barrier.
__device__ __forceinline__ float block_max(float x, float* red, int wave, int lane) {
    x = wave_max(x);
    if (lane == 0) red[wave] = x;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// R rows per block (64 or 128).  Wave w computes rows 32 (w % (R / 32)) ..
// +31 of the block against NB = R / 32 of the four 32-row blocks of the
// rotation: D = Rot X^T, so lane l holds entries n = 8 a + 4 h + e (h = l / 32)
// of the rotated block row l % 32, four consecutive columns per register
// group: exactly one 4-byte store per group.
template <int R>
__global__ __launch_bounds__(kQThreads) void quant_rows_kernel(const uint16_t* __restrict__ X,
                                                               const uint16_t* __restrict__ rot,
                                                               uint8_t* __restrict__ X8, uint8_t* __restrict__ scales,
                                                               int S, int nblk, int64_t total) {
    constexpr int NB = R / 32;                 // column blocks per wave
    __shared__ __attribute__((aligned(16))) uint16_t rt[kQD * kQD];   // R, swizzled (below)
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;

    const int rsub = wave % (R / 32);          // this wave's 32-row slice of the block
    const int nb0 = (wave / (R / 32)) * NB;    // its first column block
    // this lane's operands of block blk (its row of the slice), loaded one
    // block ahead so that the loads of the next block overlap this one
    bf16x8 xn[kQD / 16];
    auto load_x = [&](int64_t blk) {
        const int64_t bh = blk / nblk;
        const int row = (int)(blk % nblk) * R + rsub * 32 + l32;
        const uint16_t* xr = X + (bh * S + min(row, S - 1)) * kQD + 8 * hh;
#pragma unroll
        for (int s = 0; s < kQD / 16; ++s) xn[s] = *reinterpret_cast<const bf16x8*>(xr + 16 * s);
    };
    if (blockIdx.x < total) load_x(blockIdx.x);

    // stage R (or the identity) once, all loads in flight together; 16-byte
    // chunk c of row n sits at chunk c ^ (n % 16), so the operand reads (32
    // rows, one chunk) spread over all banks
    constexpr int NST = kQD * kQD / 8 / kQThreads;
    static_assert(NST * kQThreads * 8 == kQD * kQD, "staging split");
    u32x4 rv[NST];
    if (rot != nullptr) {
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            const int c = tid + kQThreads * i;
            rv[i] = *reinterpret_cast<const u32x4*>(rot + (c / (kQD / 8)) * kQD + 8 * (c % (kQD / 8)));
        }
    } else {
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            const int c = tid + kQThreads * i;
            const int n = c / (kQD / 8), ch = c % (kQD / 8);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int k0 = 8 * ch + 2 * k;
                rv[i][k] = (k0 == n ? 0x3F80u : 0u) | (k0 + 1 == n ? 0x3F800000u : 0u);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < NST; ++i) {
        const int c = tid + kQThreads * i;
        const int n = c / (kQD / 8), ch = c % (kQD / 8);
        *reinterpret_cast<u32x4*>(rt + n * kQD + 8 * (ch ^ (n & 15))) = rv[i];
    }
    __syncthreads();

    for (int64_t blk = blockIdx.x; blk < total; blk += gridDim.x) {
        const int64_t bh = blk / nblk;
        const int j = (int)(blk % nblk);
        const int row = j * R + rsub * 32 + l32;   // this lane's row of the slice
        bf16x8 xc[kQD / 16];
#pragma unroll
        for (int s = 0; s < kQD / 16; ++s) xc[s] = row < S ? xn[s] : bf16x8{};
        if (blk + gridDim.x < total) load_x(blk + gridDim.x);
        f32x16 acc[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) acc[i] = f32x16{};
#pragma unroll
        for (int s = 0; s < kQD / 16; ++s) {
            const bf16x8 xb = xc[s];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int n = 32 * (nb0 + i) + l32;
                const bf16x8 ra = *reinterpret_cast<const bf16x8*>(rt + n * kQD + 8 * ((2 * s + hh) ^ (n & 15)));
                acc[i] = mfma32(ra, xb, acc[i]);
            }
        }
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(acc[i][r]));
        const int e = scale_exp(block_max(m, red, wave, lane));
        const float inv = inv_scale(e);
        if (row < S) {
            uint8_t* out = X8 + (bh * S + row) * kQD;
#pragma unroll
            for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const uint32_t w = pack_fp8x4(acc[i][4 * a] * inv, acc[i][4 * a + 1] * inv,
                                                  acc[i][4 * a + 2] * inv, acc[i][4 * a + 3] * inv);
                    *reinterpret_cast<uint32_t*>(out + 32 * (nb0 + i) + 8 * a + 4 * hh) = w;
                }
        }
        if (tid == 0) scales[blk] = (uint8_t)(e + 127);
        __syncthreads();   // `red` is reused by the next block
    }
}

// Key of position p = 32 h + b of a d-major V row: the lanes of half h hold
// P for keys 8 (r / 4) + 4 h + r % 4 of each 32-key half-block in register r,
// and the P operand takes half-block 0's 16 registers, then half-block 1's.
__device__ __forceinline__ int v_key_of(int h, int b) { return 32 * (b >> 4) + 8 * ((b & 15) >> 2) + 4 * h + (b & 3); }

// One workgroup per 64-key block (persistent loop): stage the block in LDS,
// find its amax, then thread t writes half h = t % 2 of d-row t / 2.
__global__ __launch_bounds__(kQThreads) void quant_v_kernel(const uint16_t* __restrict__ V, uint8_t* __restrict__ V8,
                                                            uint8_t* __restrict__ scales, int S, int nblk,
                                                            int64_t total) {
    __shared__ __attribute__((aligned(16))) uint16_t vt[64 * kQD];
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int dr = tid >> 1, h = tid & 1;
    for (int64_t blk = blockIdx.x; blk < total; blk += gridDim.x) {
        const int64_t bh = blk / nblk;
        const int j = (int)(blk % nblk);
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + kQThreads * i;             // 16-byte chunk of the 64 x 128 block
            const int r = c >> 4, col = 8 * (c & 15);
            const int key = j * 64 + r;
            bf16x8 v = bf16x8{};
            if (key < S) v = *reinterpret_cast<const bf16x8*>(V + (bh * S + key) * kQD + col);
            *reinterpret_cast<bf16x8*>(vt + r * kQD + col) = v;
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)v[e]));
        }
        const int e = scale_exp(block_max(m, red, wave, lane));   // the barrier inside also publishes vt
        const float inv = inv_scale(e);
        uint32_t w[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            float f[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint16_t bits = vt[v_key_of(h, 4 * q + i) * kQD + dr];
                f[i] = __uint_as_float((uint32_t)bits << 16) * inv;
            }
            w[q] = pack_fp8x4(f[0], f[1], f[2], f[3]);
        }
        uint8_t* out = V8 + blk * (64 * kQD) + dr * 64 + 32 * h;
        *reinterpret_cast<u32x4*>(out) = u32x4{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4*>(out + 16) = u32x4{w[4], w[5], w[6], w[7]};
        if (tid == 0) scales[blk] = (uint8_t)(e + 127);
        __syncthreads();   // vt and `red` are rewritten by the next block
    }
}

int quant_grid(int64_t total) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    return (int)std::min<int64_t>(total, (int64_t)2 * n);
}

}  // namespace

hipError_t launch_quant_fp8(const QuantArgs& a, hipStream_t stream) {
    const int nblk = (a.S + a.block_rows - 1) / a.block_rows;
    const int64_t total = (int64_t)a.BH * nblk;
    const dim3 grid((unsigned)quant_grid(total));
    if (a.layout == 1) {
        launch_kernel(quant_v_kernel, grid, dim3(kQThreads), 0, stream, (const uint16_t*)a.x, (uint8_t*)a.x8,
                      a.scales, a.S, nblk, total);
    } else if (a.block_rows == 128) {
        launch_kernel((quant_rows_kernel<128>), grid, dim3(kQThreads), 0, stream, (const uint16_t*)a.x,
                      (const uint16_t*)a.rot, (uint8_t*)a.x8, a.scales, a.S, nblk, total);
    } else {
        launch_kernel((quant_rows_kernel<64>), grid, dim3(kQThreads), 0, stream, (const uint16_t*)a.x,
                      (const uint16_t*)a.rot, (uint8_t*)a.x8, a.scales, a.S, nblk, total);
    }
    return hipGetLastError();
}

}  // namespace fa
