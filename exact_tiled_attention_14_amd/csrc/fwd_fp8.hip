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

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads8, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const uint8_t* __restrict__ QS, const uint8_t* __restrict__ KS, const uint8_t* __restrict__ VS,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int Sq, int Sk, float scale_log2,
    int n_qblk, int xcd_groups, int mirror) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * kTile8];
    uint8_t* const kbuf = lds;                 // K stages 0, 1
    uint8_t* const vbuf = lds + 2 * kTile8;    // V stages 0, 1

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int g = Hq / Hkv;

    // ---- which (batch, head, query block) this workgroup owns (as the bf16 kernel) ----
    int b, hq, kvh, qb;
    {
        const int w = blockIdx.x;
        int rank;
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
        if (mirror && rank >= (n_qblk + 1) / 2) rank = n_qblk - 1 - (rank - (n_qblk + 1) / 2);
        qb = CAUSAL ? n_qblk - 1 - rank : rank;
    }

    const int n_kblk = (Sk + kBN8 - 1) / kBN8;
    const int64_t bhq = (int64_t)b * Hq + hq;
    const int64_t bhk = (int64_t)b * Hkv + kvh;
    const uint8_t* Kh = K + bhk * Sk * kD8;
    const uint8_t* Vh = V + bhk * n_kblk * kTile8;
    const uint8_t* KSh = KS + bhk * n_kblk;
    const uint8_t* VSh = VS + bhk * n_kblk;
    const int q0 = qb * kBM8;
    const int qw = q0 + wave * 32;
    const int my_q = qw + l32;
    const int diag = Sk - Sq;
    const int sq = QS[bhq * n_qblk + qb];

    int kv_end = Sk;
    if (CAUSAL) kv_end = min(Sk, max(0, q0 + kBM8 + diag));
    const int n_it = (kv_end + kBN8 - 1) / kBN8;

    // Q fragment (B operand of S^T = K Q^T): head-dim bytes 64 s + 32 h .. +31.
    // Lanes past the last query row read row Sq - 1; their scores are never
    // written out, and without a select on the values the loads' latency
    // overlaps that of the first K/V loads.
    i32x8 qf[2];
    {
        const uint8_t* qp = Q + (bhq * Sq + min(my_q, Sq - 1)) * kD8 + 32 * hh;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const i32x4 a = *reinterpret_cast<const i32x4*>(qp + 64 * s);
            const i32x4 c = *reinterpret_cast<const i32x4*>(qp + 64 * s + 16);
            qf[s] = i32x8{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
        }
    }

    f32x16 oacc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};
    float m_run = kNegInf;
    float l_run = 0.f;

    auto needs_mask = [&](int kv0) { return (kv0 + kBN8 > Sk) || (CAUSAL && kv0 + kBN8 - 1 > qw + diag); };

    // scores of block j into sacc: two 32-key halves x two 64-byte head-dim steps;
    // `between(i)` after MFMA i (0..3)
    const int sw_k = swz_k8(l32);   // rows l32 and l32 + 32 share it (period 32)
    auto score = [&](f32x16 (&sacc)[2], const uint8_t* kt, int sk, auto&& between) __attribute__((always_inline)) {
        const uint8_t* r0 = kt + l32 * kD8;
        const uint8_t* r1 = r0 + 32 * kD8;
        i32x8 ka0 = read32(r0, 2 * hh, sw_k);
        i32x8 ka1 = read32(r1, 2 * hh, sw_k);
        const i32x8 kb0 = read32(r0, 4 + 2 * hh, sw_k);
        const i32x8 kb1 = read32(r1, 4 + 2 * hh, sw_k);
        FA8_FENCE();
        sacc[0] = mfma_f8(ka0, qf[0], sacc[0], sk, sq);
        FA8_FENCE();
        between(0);
        FA8_FENCE();
        sacc[1] = mfma_f8(ka1, qf[0], sacc[1], sk, sq);
        FA8_FENCE();
        between(1);
        FA8_FENCE();
        sacc[0] = mfma_f8(kb0, qf[1], sacc[0], sk, sq);
        FA8_FENCE();
        between(2);
        FA8_FENCE();
        sacc[1] = mfma_f8(kb1, qf[1], sacc[1], sk, sq);
        FA8_FENCE();
        between(3);
        FA8_FENCE();
    };

    const int k_lane_off = k8_lane_offset(wave, lane);
    const int v_lane_off = v8_lane_offset(wave, lane);
    // Block scales used by a step are loaded one step earlier (the first ones
    // here, ahead of the prologue's wait): a load issued in the step itself
    // would sit behind that step's K/V tile loads in the memory counter,
    // so waiting for it would wait for them too.
    const int sk0 = KSh[0];
    int sk_pref = KSh[min(1, n_kblk - 1)];   // K scale of block it + 1
    int sv_pref = VSh[0];                    // V scale of block it
    if (n_it > 0) {
        dma_k8(Kh, kbuf, k_lane_off, 0, Sk, wave);
        dma_v8(Vh, vbuf, v_lane_off, wave);
    }
    if (n_it > 1) dma_k8(Kh, kbuf + kTile8, k_lane_off, kBN8, Sk, wave);
    wait_dma8();
    __syncthreads();

    f32x16 s0[2] = {f32x16{}, f32x16{}};
    float mx_cur = kNegInf;
    if (n_it > 0) {
        score(s0, kbuf, sk0, [](int) {});
        if (needs_mask(0)) mask_block8<CAUSAL>(s0, 0, Sk, my_q, diag, hh);
        float mx = kNegInf;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s0[blk][r]);
        mx_cur = half_swap_max(mx) * scale_log2;
    }
    __syncthreads();

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
        sk_pref = KSh[min(it + 2, n_kblk - 1)];
        sv_pref = VSh[min(it + 1, n_kblk - 1)];

        if (has_next2) dma_k8(Kh, k_dma, k_lane_off, (it + 2) * kBN8, Sk, wave);
        if (has_next) dma_v8(Vh + (int64_t)(it + 1) * kTile8, v_dma, v_lane_off, wave);

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
        if (has_next && needs_mask((it + 1) * kBN8)) mask_block8<CAUSAL>(snxt, (it + 1) * kBN8, Sk, my_q, diag, hh);
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
        __syncthreads();
    };
    f32x16 s1[2];
    for (int it = 0; it < n_it; it += 2) {
        step(it, s0, s1, kbuf, vbuf + kTile8, kbuf + kTile8, vbuf);
        if (it + 1 < n_it) step(it + 1, s1, s0, kbuf + kTile8, vbuf, kbuf, vbuf + kTile8);
    }

    const float l_tot = half_swap_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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
            LSE[bhq * Sq + my_q] = l_tot > 0.f ? (m_run + log2f_hw(l_tot)) * kLn2 : kNegInf;
    }
}

int num_cus8() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 256;
    return n > 0 ? n : 256;
}

template <bool CAUSAL>
hipError_t launch8(const Fp8FwdArgs& a, hipStream_t stream) {
    const int n_qblk = (a.Sq + kBM8 - 1) / kBM8;
    const int64_t n_wg = (int64_t)a.B * a.Hq * n_qblk;
    const int units = a.B * a.Hkv;
    const int xcd_groups = (units % 8 == 0) ? units / 8 : 0;
    const int mirror = (CAUSAL && n_wg <= 2 * (int64_t)num_cus8()) ? 1 : 0;
    launch_kernel((fwd_fp8_kernel<CAUSAL>), dim3((unsigned)n_wg), dim3(kThreads8), 0, stream, (const uint8_t*)a.q8,
                  (const uint8_t*)a.k8, (const uint8_t*)a.v8, a.q_scale, a.k_scale, a.v_scale, (uint16_t*)a.o, a.lse,
                  a.B, a.Hq, a.Hkv, a.Sq, a.Sk, a.scale * kLog2e, n_qblk, xcd_groups, mirror);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t stream) {
    return a.causal ? launch8<true>(a, stream) : launch8<false>(a, stream);
}

}  // namespace fa
