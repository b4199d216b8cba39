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
//   * Row layout: each block of 64 or 128 rows of a [S, 128] slice is
//     optionally rotated (each row x -> R x on the matrix cores as
//     D = R X^T, R's rows being the A operand, staged in LDS once per
//     workgroup; without R the values are taken as they are, in the same
//     lane order), then written row-major.
//   * V layout: 64-key blocks of V (no rotation), written d-major: per block
//     128 rows (one per head-dim index) of 64 bytes, the keys of a row in the
//     order in which the attention kernel's lanes hold P (see include/fa.h),
//     so the PV product reads its operand without any transposition.
//   * One persistent kernel serves one tensor or Q, K and V together: each
//     workgroup walks the blocks of one part with a stride, stages the
//     rotation once, and keeps the loads of its next block in flight while
//     it processes one.
#include "fa_device.h"
#include "fa_launch.h"

#include <atomic>

namespace fa {
namespace {

constexpr int kQD = 128;
constexpr int kQThreads = 256;

// One block of R rows (64 or 128) of a row-major part.  Wave w computes rows
// 32 (w % (R / 32)) .. +31 of the block against NB = R / 32 of the four
// 32-row blocks of the rotation: D = Rot X^T, so lane l holds entries
// n = 8 a + 4 h + e (h = l / 32) of the rotated block row l % 32, four
// consecutive columns per register group: exactly one 4-byte store per group.
// Work unit: 128 rows (or keys) of one (b, h) slice, 32 KiB of bf16, whatever
// the scale block (128 or 64 rows).  The thread's loads of a unit are issued
// one unit ahead of its processing: 16-byte chunks c = tid + 256 i
// (i = 0..7) of the row-major unit, so one load instruction of a wave reads
// 4 whole rows (1 KiB of consecutive memory).  Rows past S repeat row S - 1
// and are zeroed where they are used.
constexpr int kUnit = 128;

__device__ __forceinline__ void unit_load(const uint16_t* __restrict__ X, int S, int nunit, int64_t u, int tid,
                                          u32x4 (&buf)[8]) {
    const int64_t bh = u / nunit;
    const int j = (int)(u % nunit);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = tid + kQThreads * i;
        const int r = c >> 4, col = 8 * (c & 15);
        const int row = min(j * kUnit + r, S - 1);
        buf[i] = *reinterpret_cast<const u32x4*>(X + (bh * S + row) * kQD + col);
    }
}

// Largest |value| of each scale block of the unit: m0 covers the thread's
// first four chunks' rows (0..63), m1 the last four (64..127).  Returns the
// maximum over the unit's first and second halves (`sb` 64) or over all of
// it (`sb` 128) for this thread's half `half`.  `red` holds 8 floats; the
// caller separates consecutive uses with a barrier.
__device__ __forceinline__ float unit_max(float m0, float m1, float* red, int wave, int lane, int sb, int half) {
    m0 = wave_max(m0);
    m1 = wave_max(m1);
    if (lane == 0) {
        red[2 * wave] = m0;
        red[2 * wave + 1] = m1;
    }
    __syncthreads();
    float a = red[0], b = red[1];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
        a = fmaxf(a, red[2 * w]);
        b = fmaxf(b, red[2 * w + 1]);
    }
    return sb == kUnit ? fmaxf(a, b) : (half ? b : a);
}

// One unit of a row-major part, scale blocks of SB rows (128 or 64).  The
// unit goes through LDS twice: its rows (16-byte chunk c of row r at chunk
// c ^ (r % 16), so the operand reads of 32 rows spread over all banks) and
// its codes (chunk c of row r at c ^ (r % 8)), so that both the loads and the
// stores of a wave cover whole rows.  Wave w computes rows 32 w .. +31
// against the four 32-row blocks of the rotation: D = Rot X^T, so lane l
// holds entries n = 8 a + 4 h + e (h = l / 32) of the rotated row l % 32.
template <int SB, bool DIRECT>
__device__ __forceinline__ void rows_unit(uint8_t* __restrict__ X8, uint8_t* __restrict__ scales, int S, int nunit,
                                          int64_t u, const uint16_t* rt, uint8_t* tile, float* red, int tid,
                                          const u32x4 (&buf)[8]) {
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int64_t bh = u / nunit;
    const int j = (int)(u % nunit);
    const int nrows = min(kUnit, S - j * kUnit);   // rows of this unit inside the sequence
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = tid + kQThreads * i;
        const int r = c >> 4, ch = c & 15;
        *reinterpret_cast<u32x4*>(tile + r * 256 + 16 * (ch ^ (r & 15))) = r < nrows ? buf[i] : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    const int rr = wave * 32 + l32;                // this lane's row of the unit
    f32x16 acc[4];
    if constexpr (DIRECT) {
        // no rotation: the same entries of the lane's row, read as they are
        // (a product with the identity would turn -0 into +0)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const u32x2 w = *reinterpret_cast<const u32x2*>(tile + rr * 256 + 16 * ((4 * i + a) ^ (rr & 15)) + 8 * hh);
                acc[i][4 * a + 0] = bf16lo_to_f32(w[0]);
                acc[i][4 * a + 1] = bf16hi_to_f32(w[0]);
                acc[i][4 * a + 2] = bf16lo_to_f32(w[1]);
                acc[i][4 * a + 3] = bf16hi_to_f32(w[1]);
            }
    } else {
        bf16x8 xc[kQD / 16];
#pragma unroll
        for (int s = 0; s < kQD / 16; ++s)
            xc[s] = *reinterpret_cast<const bf16x8*>(tile + rr * 256 + 16 * ((2 * s + hh) ^ (rr & 15)));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
#pragma unroll
        for (int s = 0; s < kQD / 16; ++s) {
            const bf16x8 xb = xc[s];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = 32 * i + l32;
                const bf16x8 ra = *reinterpret_cast<const bf16x8*>(rt + n * kQD + 8 * ((2 * s + hh) ^ (n & 15)));
                acc[i] = mfma32(ra, xb, acc[i]);
            }
        }
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(acc[i][r]));
    // waves 0, 1 hold rows 0..63, waves 2, 3 rows 64..127; the barrier inside
    // also ends every wave's reads of the rows
    const int half = wave >> 1;
    const int e = fp8_scale_exp(unit_max(half ? 0.f : m, half ? m : 0.f, red, wave, lane, SB, half));
    const float inv = fp8_inv_scale(e);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const uint32_t w = pack_fp8x4(acc[i][4 * a] * inv, acc[i][4 * a + 1] * inv, acc[i][4 * a + 2] * inv,
                                          acc[i][4 * a + 3] * inv);
            const int c16 = 2 * i + (a >> 1);
            *reinterpret_cast<uint32_t*>(tile + rr * 128 + 16 * (c16 ^ (rr & 7)) + 8 * (a & 1) + 4 * hh) = w;
        }
    __syncthreads();
    uint8_t* out = X8 + (bh * S + (int64_t)j * kUnit) * kQD;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = tid + kQThreads * k;         // 16-byte chunk of the unit's codes
        const int r = c >> 3, c16 = c & 7;
        if (r < nrows)
            *reinterpret_cast<u32x4*>(out + r * kQD + 16 * c16) =
                *reinterpret_cast<const u32x4*>(tile + r * 128 + 16 * (c16 ^ (r & 7)));
    }
    // one byte per scale block: thread 0 for the first, thread 128 (wave 2)
    // for the second block of 64
    const int nsb = (S + SB - 1) / SB;
    if (tid == 0) scales[bh * nsb + j * (kUnit / SB)] = (uint8_t)(e + 127);
    if (SB == 64 && tid == 128 && j * kUnit + 64 < S) scales[bh * nsb + 2 * j + 1] = (uint8_t)(e + 127);
    __syncthreads();   // the tile and `red` are reused by the next unit
}

// Key of position p = 32 h + b of a d-major V row: the lanes of half h hold
// P for keys 8 (r / 4) + 4 h + r % 4 of each 32-key half-block in register r,
// and the P operand takes half-block 0's 16 registers, then half-block 1's.
__device__ __forceinline__ int v_key_of(int h, int b) { return 32 * (b >> 4) + 8 * ((b & 15) >> 2) + 4 * h + (b & 3); }

// One unit of V: two 64-key blocks, each with its own scale.  Stage the rows
// in LDS, find each block's amax, then for each block thread t writes the
// 16-byte chunks t and t + 256 of the block's 8 KiB of codes (chunk c: d-row
// c / 4, positions 16 (c % 4) .. +15), so each store instruction of a wave
// covers 1 KiB of consecutive memory.
__device__ __forceinline__ void v_unit(uint8_t* __restrict__ V8, uint8_t* __restrict__ scales, int S, int nunit,
                                       int64_t u, uint16_t* vt, float* red, int tid, const u32x4 (&buf)[8]) {
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t bh = u / nunit;
    const int j = (int)(u % nunit);
    float m0 = 0.f, m1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = tid + kQThreads * i;         // rows 0..63 for i < 4, 64..127 after
        const int r = c >> 4, col = 8 * (c & 15);
        const bf16x8 v = j * kUnit + r < S ? __builtin_bit_cast(bf16x8, buf[i]) : bf16x8{};
        *reinterpret_cast<bf16x8*>(vt + r * kQD + col) = v;
        float mv = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) mv = fmaxf(mv, fabsf((float)v[e]));
        if (i < 4)
            m0 = fmaxf(m0, mv);
        else
            m1 = fmaxf(m1, mv);
    }
    // the barrier inside also publishes vt
    const float a0 = unit_max(m0, m1, red, wave, lane, 64, 0), a1 = unit_max(m0, m1, red, wave, lane, 64, 1);
    const int nblk = (S + 63) / 64;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        const int vb = 2 * j + hb;                 // the V block
        if (vb >= nblk) break;
        const int e = fp8_scale_exp(hb ? a1 : a0);
        const float inv = fp8_inv_scale(e);
        const uint16_t* vrows = vt + 64 * hb * kQD;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int c = tid + kQThreads * k;
            const int dr = c >> 2, h = (c >> 1) & 1, b0 = 16 * (c & 1);
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float f[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint16_t bits = vrows[v_key_of(h, b0 + 4 * q + i) * kQD + dr];
                    f[i] = __uint_as_float((uint32_t)bits << 16) * inv;
                }
                w[q] = pack_fp8x4(f[0], f[1], f[2], f[3]);
            }
            *reinterpret_cast<u32x4*>(V8 + (bh * nblk + vb) * (64 * kQD) + 16 * c) = u32x4{w[0], w[1], w[2], w[3]};
        }
        if (tid == 0) scales[bh * nblk + vb] = (uint8_t)(e + 127);
    }
    __syncthreads();   // vt and `red` are rewritten by the next unit
}

// Up to three tensors in one launch (Q, K and V of one attention call, or a
// single tensor).  The host splits the grid over the parts in proportion to
// their units and each workgroup walks the units of one part with a stride,
// so its loop is one straight sequence of one unit kind, with the loads of
// the next unit in flight while one is processed.
struct QuantPart {
    const uint16_t* x;
    uint8_t* x8;
    uint8_t* scales;
    int S, nunit;
    int kind;                    // 0: rows, scale blocks of 128; 1: rows, blocks of 64; 2: d-major V blocks
    int wg0, nwg;                // the part's workgroups
    int64_t units;
};
struct QuantParts {
    QuantPart p[3];
    int n;
};

template <int KIND, bool DIRECT>
__device__ __forceinline__ void run_part(const QuantPart& q, int64_t first, uint16_t* rt, uint8_t* tile, float* red,
                                         int tid) {
    // The thread index is made opaque in every call, so the many lane
    // addresses derived from it are formed where they are used instead of
    // being kept live across the loop (which spilled).
    auto process = [&](int64_t u, const u32x4 (&buf)[8]) __attribute__((always_inline)) {
        int t = tid;
        asm volatile("" : "+v"(t));
        if constexpr (KIND == 2)
            v_unit(q.x8, q.scales, q.S, q.nunit, u, reinterpret_cast<uint16_t*>(tile), red, t, buf);
        else
            rows_unit<KIND == 0 ? 128 : 64, DIRECT>(q.x8, q.scales, q.S, q.nunit, u, rt, tile, red, t, buf);
    };
    auto load = [&](int64_t u, u32x4 (&buf)[8]) __attribute__((always_inline)) {
        int t = tid;
        asm volatile("" : "+v"(t));
        unit_load(q.x, q.S, q.nunit, u, t, buf);
    };
    // two buffers: the next unit's loads are in flight while this one is
    // processed (unrolled by two so the buffers swap roles without copies)
    const int64_t g = q.nwg, total = q.units;
    u32x4 ba[8], bb[8];
    load(first, ba);
    for (int64_t u = first; u < total; u += 2 * g) {
        if (u + g < total) load(u + g, bb);
        process(u, ba);
        if (u + g >= total) break;
        if (u + 2 * g < total) load(u + 2 * g, ba);
        process(u + g, bb);
    }
}

__global__ __launch_bounds__(kQThreads, 2) void quant_kernel(QuantParts parts, const uint16_t* __restrict__ rot) {
    __shared__ __attribute__((aligned(16))) uint16_t rt[kQD * kQD];   // R, swizzled
    __shared__ __attribute__((aligned(16))) uint8_t tile[kUnit * 256]; // one unit (rows, codes or V)
    __shared__ float red[8];
    const int tid = threadIdx.x;
    const int w = blockIdx.x;
    QuantPart q = parts.p[0];
    if (parts.n > 1 && w >= parts.p[1].wg0) q = parts.p[1];
    if (parts.n > 2 && w >= parts.p[2].wg0) q = parts.p[2];
    const int64_t first = w - q.wg0;
    if (first >= q.units) return;                        // whole workgroup: no barrier reached
    if (q.kind == 2) {
        run_part<2, true>(q, first, rt, tile, red, tid);
    } else if (rot == nullptr) {
        if (q.kind == 0)
            run_part<0, true>(q, first, rt, tile, red, tid);
        else
            run_part<1, true>(q, first, rt, tile, red, tid);
    } else {
        stage_rotation128<kQThreads>(rot, rt, tid);
        __syncthreads();
        if (q.kind == 0)
            run_part<0, false>(q, first, rt, tile, red, tid);
        else
            run_part<1, false>(q, first, rt, tile, red, tid);
    }
}

// Resident workgroups of quant_kernel on the current device (queried once per
// device).
int quant_slots() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0, per_cu = 0;
    if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quant_kernel, kQThreads, 0) != hipSuccess || per_cu <= 0)
        per_cu = 2;
    if (dev >= 0 && dev < 64) cache[dev].store(per_cu * n, std::memory_order_relaxed);
    return per_cu * n;
}

QuantPart make_part(const QuantArgs& a) {
    const int nunit = (a.S + kUnit - 1) / kUnit;
    const int kind = a.layout == 1 ? 2 : (a.block_rows == 128 ? 0 : 1);
    return QuantPart{(const uint16_t*)a.x, (uint8_t*)a.x8, a.scales, a.S, nunit, kind, 0, 0, a.BH * nunit};
}

// Workgroups per part: the resident slots in proportion to each part's units
// (at least one, at most one per unit), laid out part after part.
hipError_t launch_parts(QuantParts& parts, const void* rot, hipStream_t stream) {
    const int slots = quant_slots();
    double all = 0;
    for (int i = 0; i < parts.n; ++i) all += (double)parts.p[i].units;
    int wg = 0;
    for (int i = 0; i < parts.n; ++i) {
        QuantPart& q = parts.p[i];
        const int64_t share = (int64_t)((double)slots * (double)q.units / all + 0.5);
        q.wg0 = wg;
        q.nwg = (int)std::max<int64_t>(1, std::min<int64_t>(share, q.units));
        wg += q.nwg;
    }
    if (wg <= 0) return hipSuccess;
    launch_kernel(quant_kernel, dim3((unsigned)wg), dim3(kQThreads), 0, stream, parts, (const uint16_t*)rot);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_fp8(const QuantArgs& a, hipStream_t stream) {
    QuantParts parts{};
    parts.p[0] = make_part(a);
    parts.n = 1;
    return launch_parts(parts, a.rot, stream);
}

hipError_t launch_quant_fp8_qkv(const QuantArgs& q, const QuantArgs& k, const QuantArgs& v, hipStream_t stream) {
    QuantParts parts{};
    parts.p[0] = make_part(q);
    parts.p[1] = make_part(k);
    parts.p[2] = make_part(v);
    parts.n = 3;
    return launch_parts(parts, q.rot, stream);
}

}  // namespace fa
