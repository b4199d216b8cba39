// Prefill attention forward on FP8 (E4M3) inputs with per-block scales,
// bf16 output, fp32 accumulation, gfx950, head dimension 128.
//
// The FP8 variant of "FlashAttention scaling, multi-GPU training and weight
// quantization", section 1: both products run on the FP8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4, twice the bf16 rate), and the block
// scales of Q, K and V are applied inside the product by the hardware (E8M0
// scale operands), so scores and the output accumulate in true units.  The
// algorithm is that of the bf16 kernel: one workgroup of 4 waves per 128
// query rows, 64-key blocks staged into LDS by buffer loads to LDS (K two
// blocks ahead, V one), S^T = K Q^T so a lane owns one query row, online
// softmax with a deferred rescale, O^T += V^T P^T, one division at the end.
//
// P is rounded to E4M3 for the second product (p <= 2^8, inside the E4M3
// range; the running sum adds the unrounded fp32 values).  Q, K and V arrive
// quantized by quant_fp8.hip: Q in 128-row blocks, K in 64-row blocks, V in
// d-major 64-key blocks whose key order is the order in which a lane holds P,
// so both operands of O^T += V^T P^T are plain 32-byte reads.
//
// With QB the kernel takes Q in bf16 and quantizes each job's 128-row block
// itself, exactly as the quantizer does (rotation D = R X^T on the bf16
// matrix cores with R staged in LDS, block maximum over the four waves, E8M0
// scale, E4M3 conversion), so the codes and the scale are those the quantizer
// would have written; the rotation leaves each lane half with alternate
// groups of four head-dim values, and one lane-half swap per group pair
// brings the 32 consecutive values the FP8 product's operand takes.
//
// LDS tiles: K rows are 128 bytes with 16-byte chunk c stored at
// c ^ ((row / 4) % 8); V^T rows are 64 bytes with chunk c at c ^ ((row / 8) % 4).
// Both operand read patterns (16 consecutive rows, one chunk) then hit
// distinct banks.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kD8 = 128;
constexpr int kWaves8 = 4;
constexpr int kThreads8 = 64 * kWaves8;
constexpr int kBM8 = 32 * kWaves8;     // query rows per workgroup (= Q scale block)
constexpr int kBN8 = 64;               // keys per step (= K and V scale block)
constexpr int kTile8 = kBN8 * kD8;     // bytes of one K or V tile
constexpr float kTau8 = 8.f;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// D = A B + C with E4M3 operands and E8M0 block scales sa (A) and sb (B).
// Operand a: lane l holds row l % 32, 32 contraction elements; b: lane l
// holds column l % 32, the same 32 contraction positions.
__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ int swz_k8(int row) { return (row >> 2) & 7; }
__device__ __forceinline__ int swz_v8(int row) { return (row >> 3) & 3; }

// K tile (64 rows x 128 bytes): load c of wave w fills 1 KiB slice
// c * 4 + w = 8 rows; lane l lands at byte 16 l and fetches the logical chunk
// the swizzle places there.  A lane's two loads are 32 rows apart (the swizzle
// period), so they share the lane offset.
__device__ __forceinline__ int k8_lane_offset(int wave, int lane) {
    const int row = wave * 8 + (lane >> 3);
    return row * kD8 + 16 * ((lane & 7) ^ swz_k8(row));
}

__device__ __forceinline__ void dma_k8(const uint8_t* __restrict__ src, uint8_t* stage, int lane_off, int kv0, int Sk,
                                       int wave) {
    const uint8_t* blk = src + (int64_t)kv0 * kD8;           // the block's first row
    if (kv0 + kBN8 <= Sk) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
            buffer_load_lds16(blk, kBN8 * kD8, stage + (c * kWaves8 + wave) * 1024, (uint32_t)lane_off,
                              32 * c * kD8);
    } else {
        // ragged last block: rows past Sk repeat row Sk - 1 (their scores are masked)
        const int row0 = lane_off / kD8;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int row = min(row0 + 32 * c, Sk - 1 - kv0);
            buffer_load_lds16(blk, kBN8 * kD8, stage + (c * kWaves8 + wave) * 1024,
                              (uint32_t)(row * kD8 + (lane_off - row0 * kD8)), 0);
        }
    }
}

// V^T tile (128 rows x 64 bytes, contiguous in memory): slice c * 4 + w =
// 16 rows; lane l -> row 16 slice + l / 4, physical chunk l % 4.
__device__ __forceinline__ int v8_lane_offset(int wave, int lane) {
    const int row = wave * 16 + (lane >> 2);
    return row * 64 + 16 * ((lane & 3) ^ swz_v8(row));
}

__device__ __forceinline__ void dma_v8(const uint8_t* __restrict__ blk, uint8_t* stage, int lane_off, int wave) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
        buffer_load_lds16(blk, 8192, stage + (c * kWaves8 + wave) * 1024, (uint32_t)lane_off, c * 4096);
}

__device__ __forceinline__ void wait_dma8() { __builtin_amdgcn_s_waitcnt(0x0F70); }

#define FA8_FENCE() __builtin_amdgcn_sched_barrier(0)

// 32 contiguous logical bytes (chunks c0, c0 + 1) of a swizzled tile row.
__device__ __forceinline__ i32x8 read32(const uint8_t* row_base, int c0, int sw) {
    const i32x4 a = *reinterpret_cast<const i32x4*>(row_base + 16 * (c0 ^ sw));
    const i32x4 b = *reinterpret_cast<const i32x4*>(row_base + 16 * ((c0 + 1) ^ sw));
    return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Keys past Sk and above this lane's causal diagonal: both bound the key
// kv0 + 32 blk + acc_row(r, hh) from above, so one per-lane limit per
// half-block, then one compare with the register's row offset and a select.
template <bool CAUSAL>
__device__ __forceinline__ void mask_block8(f32x16 (&sacc)[2], int kv0, int Sk, int my_q, int diag, int hh) {
    const int last = CAUSAL ? min(Sk - 1, my_q + diag) : Sk - 1;    // last visible key of this row
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        const int lim = last - kv0 - 32 * blk - 4 * hh;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[blk][r] = (8 * (r >> 2) + (r & 3)) <= lim ? sacc[blk][r] : kNegInf;
    }
}

// Wave-group barrier waits of this source that ran out, per device (read and
// cleared by read_fp8_sync_timeouts).
__device__ unsigned int g_fp8_sync_timeouts;
static_assert(kWaves8 == 4, "group_barrier counts four waves per group");

// One workgroup of 4 waves per (batch, query head, 128-row Q block), heaviest
// causal blocks first; or, as a pair grid (PAIR: causal, Sq = Sk, every pair
// resident at once), one 8-wave workgroup per pair (heavy block i = n-1-p,
// light block p) of a (batch, query head), as the bf16 kernel does: two
// 4-wave groups with their own K/V stages and barrier, group A walking key
// blocks [0, split) of block i, group B all of block p and then the rest of
// block i, and the two partial softmax states of block i merged through LDS.
template <bool CAUSAL, bool PAIR, bool QB>
__global__ __launch_bounds__(PAIR ? 2 * kThreads8 : kThreads8, PAIR ? 1 : 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const uint8_t* __restrict__ QS, const uint8_t* __restrict__ KS, const uint8_t* __restrict__ VS,
    const uint16_t* __restrict__ ROT, uint16_t* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv,
    int Sq, int Sk, float scale_log2, int n_qblk, int n_rank, int xcd_groups, int mirror, int split_bias,
    int sync_spins, int split_only) {
    constexpr int GROUP_LDS = 4 * kTile8;      // K stages 0, 1 and V stages 0, 1
    // pair mode: both groups' stages, their barrier counters, the merge's (m, l);
    // QB: then the rotation (32 KiB) and the Q block maxima of the groups' waves
    constexpr int BASE_LDS = PAIR ? 2 * GROUP_LDS + 64 + kWaves8 * 64 * 8 : GROUP_LDS;
    constexpr int ROT_LDS = (BASE_LDS + 1023) / 1024 * 1024;
    constexpr int AMAX_LDS = ROT_LDS + kD8 * kD8 * 2;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[QB ? AMAX_LDS + 2 * kWaves8 * 4 : BASE_LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = PAIR ? wave_id / kWaves8 : 0;       // wave group (pair mode: 0 = A, 1 = B)
    const int wave = PAIR ? wave_id % kWaves8 : wave_id;
    uint8_t* const kbuf = lds + grp * GROUP_LDS;         // K stages 0, 1
    uint8_t* const vbuf = kbuf + 2 * kTile8;             // V stages 0, 1
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int g = Hq / Hkv;
    int bar_target = 0;
    bool sync_fail = false;             // a wave-group barrier of this wave ran out (its rows become NaN)
    if constexpr (PAIR) {
        if (tid < 16) reinterpret_cast<int*>(lds + 2 * GROUP_LDS)[tid] = 0;
    }
    if constexpr (QB) {
        if (ROT != nullptr) stage_rotation128<PAIR ? 2 * kThreads8 : kThreads8>(ROT, reinterpret_cast<uint16_t*>(lds + ROT_LDS), tid);
    }
    if constexpr (PAIR || QB) __syncthreads();
    // barrier of the threads that share this workgroup's (or wave group's) K/V stages
    auto gsync = [&]() __attribute__((always_inline)) {
        if constexpr (PAIR) {
            sync_fail |=
                group_barrier(lds + 2 * GROUP_LDS + 16 * grp, bar_target, lane, sync_spins, &g_fp8_sync_timeouts);
        } else {
            __syncthreads();
        }
    };

    // ---- which (batch, head) and rank this workgroup owns (as the bf16 kernel) ----
    int b, hq, kvh, rank;
    {
        const int w = blockIdx.x;
        if (xcd_groups) {
            const int xcd = w & 7, j = w >> 3;
            const int per_rank = xcd_groups * g;
            rank = j / per_rank;
            const int rem = j % per_rank;
            const int u = (rem / g) * 8 + xcd;
            b = u / Hkv;
            kvh = u % Hkv;
            hq = kvh * g + rem % g;
        } else {
            const int bh = B * Hq;
            rank = w / bh;
            const int rem = w % bh;
            b = rem / Hq;
            hq = rem % Hq;
            kvh = hq / g;
        }
        if (mirror && rank >= (n_rank + 1) / 2) rank = n_rank - 1 - (rank - (n_rank + 1) / 2);
    }

    const int n_kblk = (Sk + kBN8 - 1) / kBN8;
    const int64_t bhq = (int64_t)b * Hq + hq;
    const int64_t bhk = (int64_t)b * Hkv + kvh;
    const uint8_t* KSh = KS + bhk * n_kblk;
    const uint8_t* VSh = VS + bhk * n_kblk;
    const int diag = Sk - Sq;
    f32x16 oacc[4];
    float m_run, l_run;

    // ---- epilogue of a query block: one division per row, bf16 output,
    // natural-log lse ----
    auto write_out = [&](const int qb) __attribute__((always_inline)) {
        const int my_q = qb * kBM8 + wave * 32 + l32;
        const float l_tot = half_swap_sum(l_run);
        const float inv = sync_fail ? __builtin_nanf("") : l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (my_q < Sq) {
            uint16_t* op = O + (bhq * Sq + my_q) * kD8;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int d0 = 32 * db + 8 * a + 4 * hh;
                    const u32x2 w = {pack_bf16x2(oacc[db][4 * a + 0] * inv, oacc[db][4 * a + 1] * inv),
                                     pack_bf16x2(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv)};
                    *reinterpret_cast<u32x2*>(op + d0) = w;
                }
            if (LSE != nullptr && hh == 0)
                LSE[bhq * Sq + my_q] = sync_fail    ? __builtin_nanf("")
                                       : l_tot > 0.f ? (m_run + log2f_hw(l_tot)) * kLn2
                                                     : kNegInf;
        }
    };

    // One job: query block qb against K/V blocks [kb0, kb1); with `final` the
    // output of the block is written, else the state stays in oacc/m_run/l_run.
    auto run_job = [&](const int qb, const int kb0, const int kb1, const bool final) __attribute__((always_inline)) {
    // (empty asm statements: the per-lane addresses are formed inside each job,
    // not kept live across the other job of a pair workgroup)
    int64_t k_off = bhk * Sk * kD8;
    int64_t v_off = bhk * n_kblk * kTile8;
    int k_lane_off = k8_lane_offset(wave, lane);
    int v_lane_off = v8_lane_offset(wave, lane);
    if constexpr (PAIR) {
        asm volatile("" : "+s"(k_off), "+s"(v_off));
        asm volatile("" : "+v"(k_lane_off), "+v"(v_lane_off));
    }
    const uint8_t* Kh = K + k_off;
    const uint8_t* Vh = V + v_off;
    const int q0 = qb * kBM8;
    const int qw = q0 + wave * 32;
    const int my_q = qw + l32;
    const int n_it = kb1 - kb0;

    // Q fragment (B operand of S^T = K Q^T): head-dim bytes 64 s + 32 h .. +31.
    // Lanes past the last query row read row Sq - 1; their scores are never
    // written out, and without a select on the values the loads' latency
    // overlaps that of the first K/V loads.
    i32x8 qf[2];
    int sq;
    // QB: this lane's bf16 row; with a rotation head-dim 16 s + 8 h .. +7 in xq[s]
    // (the rotation product's operand), without one the entries
    // 32 i + 8 a + 4 h .. +3 (a = 2 (s % 2) and a + 1, i = s / 2) that the
    // product would have left in this lane
    bf16x8 xq[kD8 / 16];
    if constexpr (QB) {
        // a row past Sq repeats row Sq - 1 (same block), so the block maximum is unchanged
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(Q) + (bhq * Sq + min(my_q, Sq - 1)) * kD8;
        if (ROT != nullptr) {
#pragma unroll
            for (int s = 0; s < kD8 / 16; ++s) xq[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s + 8 * hh);
        } else {
#pragma unroll
            for (int s = 0; s < kD8 / 16; ++s) {
                const u32x2 lo = *reinterpret_cast<const u32x2*>(qp + 32 * (s >> 1) + 16 * (s & 1) + 4 * hh);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(qp + 32 * (s >> 1) + 16 * (s & 1) + 8 + 4 * hh);
                xq[s] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
        }
    } else {
        sq = QS[bhq * n_qblk + qb];
        const uint8_t* qp = Q + (bhq * Sq + min(my_q, Sq - 1)) * kD8 + 32 * hh;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const i32x4 a = *reinterpret_cast<const i32x4*>(qp + 64 * s);
            const i32x4 c = *reinterpret_cast<const i32x4*>(qp + 64 * s + 16);
            qf[s] = i32x8{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
        }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};
    m_run = kNegInf;
    l_run = 0.f;

    auto needs_mask = [&](int kv0) { return (kv0 + kBN8 > Sk) || (CAUSAL && kv0 + kBN8 - 1 > qw + diag); };

    // scores of block j into sacc: two 32-key halves x two 64-byte head-dim steps;
    // `between(i)` after MFMA i (0..3)
    const int sw_k = swz_k8(l32);   // rows l32 and l32 + 32 share it (period 32)
    auto score = [&](f32x16 (&sacc)[2], const uint8_t* kt, int sk, auto&& between) __attribute__((always_inline)) {
        const uint8_t* r0 = kt + l32 * kD8;
        const uint8_t* r1 = r0 + 32 * kD8;
        i32x8 ka0 = read32(r0, 2 * hh, sw_k);
        i32x8 ka1 = read32(r1, 2 * hh, sw_k);
        const i32x8 kb0_ = read32(r0, 4 + 2 * hh, sw_k);
        const i32x8 kb1_ = read32(r1, 4 + 2 * hh, sw_k);
        FA8_FENCE();
        sacc[0] = mfma_f8(ka0, qf[0], sacc[0], sk, sq);
        FA8_FENCE();
        between(0);
        FA8_FENCE();
        sacc[1] = mfma_f8(ka1, qf[0], sacc[1], sk, sq);
        FA8_FENCE();
        between(1);
        FA8_FENCE();
        sacc[0] = mfma_f8(kb0_, qf[1], sacc[0], sk, sq);
        FA8_FENCE();
        between(2);
        FA8_FENCE();
        sacc[1] = mfma_f8(kb1_, qf[1], sacc[1], sk, sq);
        FA8_FENCE();
        between(3);
        FA8_FENCE();
    };

    // Block scales used by a step are loaded one step earlier (the first ones
    // here, ahead of the prologue's wait): a load issued in the step itself
    // would sit behind that step's K/V tile loads in the memory counter,
    // so waiting for it would wait for them too.
    const int sk0 = KSh[min(kb0, n_kblk - 1)];
    int sk_pref = KSh[min(kb0 + 1, n_kblk - 1)];   // K scale of block kb0 + it + 1
    int sv_pref = VSh[min(kb0, n_kblk - 1)];       // V scale of block kb0 + it
    if (n_it > 0) {
        dma_k8(Kh, kbuf, k_lane_off, kb0 * kBN8, Sk, wave);
        dma_v8(Vh + (int64_t)kb0 * kTile8, vbuf, v_lane_off, wave);
    }
    if (n_it > 1) dma_k8(Kh, kbuf + kTile8, k_lane_off, (kb0 + 1) * kBN8, Sk, wave);

    if constexpr (QB) {
        // ---- quantize the Q block while the first tiles load: D = R X^T for
        // this wave's 32 rows (lane: rotated entries 32 i + 8 a + 4 h + e of its
        // row), the block's largest |value| over the group's four waves, its
        // E8M0 scale, E4M3 codes ----
        const uint16_t* rt = reinterpret_cast<const uint16_t*>(lds + ROT_LDS);
        f32x16 acc[4];
        if (ROT != nullptr) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
#pragma unroll
            for (int s = 0; s < kD8 / 16; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = 32 * i + l32;
                    const bf16x8 ra = *reinterpret_cast<const bf16x8*>(rt + n * kD8 + 8 * ((2 * s + hh) ^ (n & 15)));
                    acc[i] = mfma32(ra, xq[s], acc[i]);
                }
        } else {
            // the values as they are (as the quantizer takes them without a rotation)
#pragma unroll
            for (int s = 0; s < kD8 / 16; ++s) {
                const u32x4 w = __builtin_bit_cast(u32x4, xq[s]);
                const int i = s >> 1, a = 2 * (s & 1);
                acc[i][4 * a + 0] = bf16lo_to_f32(w[0]);
                acc[i][4 * a + 1] = bf16hi_to_f32(w[0]);
                acc[i][4 * a + 2] = bf16lo_to_f32(w[1]);
                acc[i][4 * a + 3] = bf16hi_to_f32(w[1]);
                acc[i][4 * a + 4] = bf16lo_to_f32(w[2]);
                acc[i][4 * a + 5] = bf16hi_to_f32(w[2]);
                acc[i][4 * a + 6] = bf16lo_to_f32(w[3]);
                acc[i][4 * a + 7] = bf16hi_to_f32(w[3]);
            }
        }
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(acc[i][r]));
        m = wave_max(m);
        float* const amax = reinterpret_cast<float*>(lds + AMAX_LDS) + kWaves8 * grp;
        if (lane == 0) amax[wave] = m;
        gsync();
        m = fmaxf(fmaxf(amax[0], amax[1]), fmaxf(amax[2], amax[3]));
        const int e = fp8_scale_exp(m);
        sq = e + 127;
        const float inv = fp8_inv_scale(e);
        uint32_t c[4][4];                // codes of entries 32 i + 8 a + 4 h .. +3
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                c[i][a] = pack_fp8x4(acc[i][4 * a] * inv, acc[i][4 * a + 1] * inv, acc[i][4 * a + 2] * inv,
                                     acc[i][4 * a + 3] * inv);
        // operand s takes head-dim 64 s .. +31 in the lower lane half and
        // 64 s + 32 .. +31 in the upper: the lower half gets the upper half's
        // groups of block 2s, the upper half the lower half's of block 2s + 1
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            int w[8];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const auto r = __builtin_amdgcn_permlane32_swap(c[2 * s][a], c[2 * s + 1][a], false, false);
                w[2 * a] = (int)r[0];
                w[2 * a + 1] = (int)r[1];
            }
            qf[s] = i32x8{w[0], w[1], w[2], w[3], w[4], w[5], w[6], w[7]};
        }
    }
    wait_dma8();
    gsync();

    f32x16 s0[2] = {f32x16{}, f32x16{}};
    float mx_cur = kNegInf;
    if (n_it > 0) {
        score(s0, kbuf, sk0, [](int) {});
        if (needs_mask(kb0 * kBN8)) mask_block8<CAUSAL>(s0, kb0 * kBN8, Sk, my_q, diag, hh);
        float mx = kNegInf;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s0[blk][r]);
        mx_cur = half_swap_max(mx) * scale_log2;
    }
    // K stage 0 is rewritten (with block kb0 + 2) in the first step: every
    // wave must have finished reading it above.
    gsync();

    const int sw_v = swz_v8(l32);   // rows 32 db + l32 share it (period 32)
    // The LDS stages a step writes (loads to LDS of K_{it+2}, V_{it+1})
    // and reads (K_{it+1}, V_it) are disjoint; as restrict pointers the
    // compiler knows it, and does not wait for the loads just issued before
    // the first operand read of the step.
    auto step = [&](const int it, f32x16 (&scur)[2], f32x16 (&snxt)[2], uint8_t* __restrict__ k_dma,
                    uint8_t* __restrict__ v_dma, const uint8_t* __restrict__ k_rd,
                    const uint8_t* __restrict__ v_rd) __attribute__((always_inline)) {
        const bool has_next = it + 1 < n_it;
        const bool has_next2 = it + 2 < n_it;
        const int kb = kb0 + it;        // absolute K/V block of this step

        if (__builtin_amdgcn_ballot_w64(mx_cur > m_run + kTau8)) {
            const float m_new = fmaxf(m_run, mx_cur);
            const float alpha = exp2f_hw(m_run - (m_new == kNegInf ? 0.f : m_new));
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) oacc[i] *= alpha;
        }
        const float m_use = m_run == kNegInf ? 0.f : m_run;
        const int sv = sv_pref;
        const int sk_next = has_next ? sk_pref : 127;
        sk_pref = KSh[min(kb + 2, n_kblk - 1)];
        sv_pref = VSh[min(kb + 1, n_kblk - 1)];

        if (has_next2) dma_k8(Kh, k_dma, k_lane_off, (kb + 2) * kBN8, Sk, wave);
        if (has_next) dma_v8(Vh + (int64_t)(kb + 1) * kTile8, v_dma, v_lane_off, wave);

        // ---- phase X: scores of block it+1, exponentials of block it ----
        int pw[8];
        float rs = 0.f;
        auto exp_chunk = [&](int c) {    // scores of block c/4, registers 4(c%4) .. +3 -> P byte group c
            const int blk = c >> 2, r0 = 4 * (c & 3);
            const float p0 = exp2f_hw(fmaf(scur[blk][r0 + 0], scale_log2, -m_use));
            const float p1 = exp2f_hw(fmaf(scur[blk][r0 + 1], scale_log2, -m_use));
            const float p2 = exp2f_hw(fmaf(scur[blk][r0 + 2], scale_log2, -m_use));
            const float p3 = exp2f_hw(fmaf(scur[blk][r0 + 3], scale_log2, -m_use));
            rs += (p0 + p1) + (p2 + p3);
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
            pw[c] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
        };
        snxt[0] = f32x16{};
        snxt[1] = f32x16{};
        if (has_next) {
            score(snxt, k_rd, sk_next, [&](int i) {
                exp_chunk(2 * i);
                exp_chunk(2 * i + 1);
            });
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) exp_chunk(c);
        }
        l_run += rs;

        // ---- phase Y: O^T += V_it^T P_it^T, maximum of block it+1 ----
        if (has_next && needs_mask((kb + 1) * kBN8)) mask_block8<CAUSAL>(snxt, (kb + 1) * kBN8, Sk, my_q, diag, hh);
        float mxn = kNegInf;
        {
            const uint8_t* vt = v_rd + l32 * 64;
            const i32x8 pb = {pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
            i32x8 va[2];
            va[0] = read32(vt, 2 * hh, sw_v);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                if (db + 1 < 4) va[(db + 1) & 1] = read32(vt + (db + 1) * 32 * 64, 2 * hh, sw_v);
                FA8_FENCE();
                oacc[db] = mfma_f8(va[db & 1], pb, oacc[db], sv, 127);
                FA8_FENCE();
                if (has_next) {
                    const int blk = db >> 1, r0 = 8 * (db & 1);
#pragma unroll
                    for (int r = r0; r < r0 + 8; ++r) mxn = fmaxf(mxn, snxt[blk][r]);
                }
                FA8_FENCE();
            }
        }
        if (has_next) mx_cur = half_swap_max(mxn) * scale_log2;

        wait_dma8();
        gsync();
    };
    f32x16 s1[2];
    for (int it = 0; it < n_it; it += 2) {
        step(it, s0, s1, kbuf, vbuf + kTile8, kbuf + kTile8, vbuf);
        if (it + 1 < n_it) step(it + 1, s1, s0, kbuf + kTile8, vbuf, kbuf, vbuf + kTile8);
    }

    if (final) write_out(qb);
    };   // run_job

    if constexpr (PAIR) {
        // Pair workgroup p of (b, hq): heavy block i = n-1-p and light block p
        // (i == p for the middle block when n is odd, and for every block of
        // a split-only grid, whose workgroup r takes block n-1-r alone and
        // halves it between the groups).  Group A takes K/V
        // blocks [0, split) of block i; group B the whole of block p, then
        // [split, 2i + 2) of block i; `split_bias` blocks move from B to A,
        // since B also pays a second job start and the light block's output.
        const int i = n_qblk - 1 - rank, p = split_only ? i : rank;
        const int split = i != p ? min(n_qblk + 1 + split_bias, 2 * i + 2) : i + 1;
        if (grp == 0) {
            run_job(i, 0, split, false);
        } else {
            if (i != p) run_job(p, 0, 2 * p + 2, true);     // its output goes straight to memory
            if (split < 2 * i + 2) {
                run_job(i, split, 2 * i + 2, false);
            } else {                     // group A takes all of block i: B's share is empty
#pragma unroll
                for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
                m_run = kNegInf;
                l_run = 0.f;
            }
        }
        // ---- the halves of block i meet: M = max(m_A, m_B), acc = acc_A
        // 2^(m_A - M) + acc_B 2^(m_B - M), l likewise.  Group B's waves hold
        // the same rows and columns, lane for lane, as group A's. ----
        __syncthreads();                 // both groups done; every K/V stage is free
        float* const st = reinterpret_cast<float*>(lds) + wave * (64 * 64);
        float2* const sml = reinterpret_cast<float2*>(lds + 2 * GROUP_LDS + 64) + wave * 64;
        if (grp == 1) {
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    *reinterpret_cast<f32x4*>(st + ((db * 4 + a) * 64 + lane) * 4) =
                        f32x4{oacc[db][4 * a], oacc[db][4 * a + 1], oacc[db][4 * a + 2], oacc[db][4 * a + 3]};
            // (a failed barrier in group B reaches group A's write-out as a NaN sum)
            sml[lane] = make_float2(m_run, sync_fail ? __builtin_nanf("") : l_run);
        }
        __syncthreads();
        if (grp == 0) {
            const float2 ml = sml[lane];
            sync_fail |= __builtin_isnan(ml.y);
            const float M = fmaxf(m_run, ml.x);
            const float Mu = M == kNegInf ? 0.f : M;
            const float wa = exp2f_hw(m_run - Mu), wb = exp2f_hw(ml.x - Mu);
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const f32x4 o = *reinterpret_cast<const f32x4*>(st + ((db * 4 + a) * 64 + lane) * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) oacc[db][4 * a + e] = oacc[db][4 * a + e] * wa + o[e] * wb;
                }
            l_run = l_run * wa + ml.y * wb;
            m_run = M;
            write_out(i);
        }
    } else {
        const int qb = CAUSAL ? n_qblk - 1 - rank : rank;
        int kv_end = Sk;
        if (CAUSAL) kv_end = min(Sk, max(0, qb * kBM8 + kBM8 + diag));
        run_job(qb, 0, (kv_end + kBN8 - 1) / kBN8, true);
    }
}

int num_cus8() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 256;
    return n > 0 ? n : 256;
}

// K/V blocks of the heavy query block moved from group B to group A of a pair
// workgroup, for n query blocks: 4, 7 and 12 for n = 8, 16 and 32 (more than
// the bf16 kernel's, since group B quantizes two Q blocks when it takes them
// in bf16, and the plain form is flat over this range).
int fp8_split_bias(int n_qblk) { return 2 + 5 * n_qblk / 16; }

template <bool CAUSAL, bool QB>
hipError_t launch8(const Fp8FwdArgs& a, hipStream_t stream) {
    const int n_qblk = (a.Sq + kBM8 - 1) / kBM8;
    const int units = a.B * a.Hkv;
    const int xcd_groups = (units % 8 == 0) ? units / 8 : 0;
    const float scale_log2 = a.scale * kLog2e;
    const int cus = num_cus8();
    // Pair grid: a causal square problem whose query blocks, paired heavy with
    // light, fit one 8-wave workgroup per CU and take more than half the CUs.
    // With fewer pairs each block gets a workgroup of its own: from 6 query
    // blocks on halved between the two wave groups (split-only grid; with its
    // vector-bound steps this kernel repays the merge two blocks earlier than
    // the bf16 one), below that as one 4-wave workgroup.
    if constexpr (CAUSAL) {
        const int n_pairs = (n_qblk + 1) / 2;
        const int64_t n_pair_wg = (int64_t)a.B * a.Hq * n_pairs;
        const bool fills = 2 * n_pair_wg > cus;
        const int split_only = (!fills && n_qblk >= 6) ? 1 : 0;
        if (a.Sq == a.Sk && a.Sq % kBM8 == 0 && n_qblk >= 2 && n_pair_wg <= cus && (fills || split_only)) {
            const int64_t n_wg = split_only ? (int64_t)a.B * a.Hq * n_qblk : n_pair_wg;
            launch_kernel((fwd_fp8_kernel<CAUSAL, true, QB>), dim3((unsigned)n_wg), dim3(2 * kThreads8), 0, stream,
                          (const uint8_t*)a.q8, (const uint8_t*)a.k8, (const uint8_t*)a.v8, a.q_scale, a.k_scale,
                          a.v_scale, (const uint16_t*)a.rot, (uint16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.Sq, a.Sk,
                          scale_log2, n_qblk, split_only ? n_qblk : n_pairs, xcd_groups, 0, fp8_split_bias(n_qblk),
                          a.sync_spins, split_only);
            return hipGetLastError();
        }
    }
    const int64_t n_wg = (int64_t)a.B * a.Hq * n_qblk;
    // Two workgroups fit on a CU; if the whole grid is resident at once, pair
    // heavy and light causal Q blocks on the same CU.
    const int mirror = (CAUSAL && n_wg <= 2 * (int64_t)cus) ? 1 : 0;
    launch_kernel((fwd_fp8_kernel<CAUSAL, false, QB>), dim3((unsigned)n_wg), dim3(kThreads8), 0, stream,
                  (const uint8_t*)a.q8, (const uint8_t*)a.k8, (const uint8_t*)a.v8, a.q_scale, a.k_scale, a.v_scale,
                  (const uint16_t*)a.rot, (uint16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.Sq, a.Sk, scale_log2, n_qblk,
                  n_qblk, xcd_groups, mirror, 0, a.sync_spins, 0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream) {
    if (a.q_bf16) return a.causal ? launch8<true, true>(a, stream) : launch8<false, true>(a, stream);
    return a.causal ? launch8<true, false>(a, stream) : launch8<false, false>(a, stream);
}

hipError_t read_fp8_sync_timeouts(unsigned int* count) {
    return read_device_counter(&HIP_SYMBOL(g_fp8_sync_timeouts), count);
}

}  // namespace fa
