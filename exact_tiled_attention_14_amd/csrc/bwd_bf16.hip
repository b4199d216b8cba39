// Attention backward, bf16 in / bf16 gradients, fp32 accumulation, gfx950.
//
// The backward pass keeps only O and the per-row log-sum-exp from the
// forward and recomputes the scores and probabilities block by block from
// Q, K, V ("Fast Inference and Training at Scale", section 6.21, Idea 2;
// "Week 13. GPUs and FlashAttention", Step 2).  With P = exp(scale S - lse)
// exact from the stored lse, the gradients of the definition are
//
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = sum_d dO_id O_id,
//   dQ = scale dS K,  dK = scale dS^T Q,
//
// (D_i equals sum_j P_ij dP_ij because O = P V).  Two kernels, no atomics:
//
//   * bwd_dq_kernel: one workgroup per (batch, query head, 128-row Q block),
//     walking the K/V blocks the rows can see, like the forward.  Each wave
//     owns 32 query rows; it forms D of its rows from the dO rows it holds
//     and the O rows (and stores D for the next kernel), computes S^T = K Q^T
//     and dP^T = V dO^T on the matrix cores (so every lane holds one query
//     row: its lse and D are one value), forms dS^T in registers, and
//     accumulates dQ^T += K^T dS^T with the K tile read transposed from LDS.
//   * bwd_dkdv_kernel: one workgroup per (batch, K/V head, 128-key block),
//     each wave owning 32 keys, walking the query heads of the GQA group and
//     their 32-row Q blocks that see the keys.  S = Q K^T and dP = dO V^T put
//     one key per lane; dV^T += dO^T P and dK^T += Q^T dS take P and dS
//     straight from registers and dO, Q read transposed from LDS.  Summing
//     over the query heads of the group is the GQA gradient.
//
// The LDS helpers take __restrict__ stage pointers: the compiler then does
// not make a read of one stage wait for the global-to-LDS prefetch into the
// other (the kernels' own wait and barrier before each step already order
// every read after the loads of its stage).
//
// LDS tiles are row-major 256-byte rows (d = 128) with 16-byte chunks
// XOR-swizzled by 4 (row mod 4) + (row / 4 mod 4): both the row reads (16
// rows, one chunk) and the transposing reads (4 rows, 4 chunks) of a tile
// then hit distinct banks.
#include <atomic>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kD = 128;
constexpr int kROWB = kD * 2;          // bytes per tile row
constexpr int kWavesB = 4;
constexpr int kThreadsB = 64 * kWavesB;
constexpr int kQRows = 32 * kWavesB;   // query rows per dQ workgroup
constexpr int kKRows = 32 * kWavesB;   // keys per dK/dV workgroup
constexpr int kKVBlk = 64;             // keys per dQ inner step
constexpr int kQBlk = 32;              // query rows per dK/dV inner step

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int swz(int row) { return 4 * (row & 3) + ((row >> 2) & 3); }

// Scheduling fence: LDS operand reads issued ahead of a group of products stay
// ahead of it, so their latency is covered by the products in between.
#define BWD_FENCE() __builtin_amdgcn_sched_barrier(0)

// Copy rows r0 .. r0+ROWS-1 of a [S, 128] bf16 matrix into an LDS tile with
// the buffer load to LDS; rows past S repeat row S-1.  Load sl fills the
// 1 KiB slice sl (4 rows); lane l lands at byte 16 l of it and fetches the
// logical chunk that the swizzle places there.
template <int ROWS>
__device__ __forceinline__ void dma_rows(const uint16_t* __restrict__ src, uint8_t* __restrict__ tile, int r0, int S,
                                         int wave, int lane) {
    static_assert(ROWS % (4 * kWavesB) == 0, "every wave issues the same number of loads");
    const int rr = lane >> 4, ch = lane & 15;
    const uint16_t* blk = src + (int64_t)r0 * kD;             // the tile's first row
#pragma unroll
    for (int i = 0; i < ROWS / 4 / kWavesB; ++i) {
        const int sl = wave + i * kWavesB;
        const int row = 4 * sl + rr;
        const uint32_t off = (uint32_t)((min(r0 + row, S - 1) - r0) * kD + 8 * (ch ^ swz(row))) * 2u;
        buffer_load_lds16(blk, ROWS * kD * 2, tile + sl * 1024, off, 0);
    }
}

__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// MFMA operand from tile row `row`: head-dim elements 16 s + 8 hh .. +7.
__device__ __forceinline__ bf16x8 row_operand(const uint8_t* __restrict__ tile, int row, int s, int hh) {
    return *reinterpret_cast<const bf16x8*>(tile + row * kROWB + 16 * ((2 * s + hh) ^ swz(row)));
}

__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t* __restrict__ p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const __attribute__((address_space(3))) uint8_t*)p);
}

// Transposed operand: lane l gets column 32 db + l % 32 of the tile for the
// tile rows 16 ks + 4 h + e and 16 ks + 8 + 4 h + e (h = l / 32, e = 0..3),
// the order in which a lane half holds a 16-row slice of an accumulator.
__device__ __forceinline__ bf16x8 tr_operand(const uint8_t* __restrict__ tile, int ks, int db, int lane) {
    const int s = lane & 15, g = lane >> 4, h = g >> 1;
    const int col = 32 * db + 16 * (g & 1) + 4 * (s & 3);
    const int row0 = 16 * ks + 4 * h + (s >> 2), row1 = row0 + 8;
    const int x = col >> 3, half = (col >> 2) & 1;
    const s16x4 a = lds_read_tr16(tile + row0 * kROWB + 16 * (x ^ swz(row0)) + 8 * half);
    const s16x4 b = lds_read_tr16(tile + row1 * kROWB + 16 * (x ^ swz(row1)) + 8 * half);
    const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Accumulator values -> bf16 B operands: k-step ks takes registers 8 ks .. +7
// of a 32x32 block (rows 16 ks + 4 h + e, 16 ks + 8 + 4 h + e in lane half h).
__device__ __forceinline__ void pack_operand(u32x4 (&out)[2], const float (&x)[16]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int w = 0; w < 4; ++w) out[ks][w] = pack_bf16x2(x[8 * ks + 2 * w], x[8 * ks + 2 * w + 1]);
}

// 8 head-dim elements of row `row` of a [S, 128] bf16 matrix for MFMA step s
// (elements 16 s + 8 hh .. +7), zero for rows past S.
__device__ __forceinline__ void load_row_operands(bf16x8 (&x)[kD / 16], const uint16_t* src, int row, int S, int hh) {
    const uint16_t* p = src + (int64_t)min(row, S - 1) * kD + 8 * hh;
#pragma unroll
    for (int s = 0; s < kD / 16; ++s) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(p + 16 * s);
        x[s] = row < S ? v : bf16x8{};
    }
}

// bf16 rows of an accumulator group written to a [S, 128] matrix: lane = row
// (`row`, skipped past S), register 4 a + e of block db = column 32 db + 8 a + 4 hh + e.
__device__ __forceinline__ void store_rows(uint16_t* dst, const f32x16 (&acc)[kD / 32], float mul, int row, int S,
                                           int hh) {
    if (row >= S) return;
    uint16_t* p = dst + (int64_t)row * kD;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int d0 = 32 * db + 8 * a + 4 * hh;
            const u32x2 w = {pack_bf16x2(acc[db][4 * a + 0] * mul, acc[db][4 * a + 1] * mul),
                             pack_bf16x2(acc[db][4 * a + 2] * mul, acc[db][4 * a + 3] * mul)};
            *reinterpret_cast<u32x2*>(p + d0) = w;
        }
}

// Wave-group barrier waits of the pair-grid dQ kernel that ran out, per
// device (read and cleared by read_bwd_sync_timeouts).
__device__ unsigned int g_bwd_sync_timeouts;
static_assert(kWavesB == 4, "group_barrier counts four waves per group");

// lse (natural log) -> the log2-domain offset of exp2; a row with no visible
// key (lse = -inf) gets +inf so that every p of it is exactly 0.
__device__ __forceinline__ float lse_offset(float lse) { return lse == kNegInf ? __builtin_inff() : lse * kLog2e; }

// dQ: one workgroup per (batch, query head, 128-row Q block), heaviest causal
// blocks first; or, as a pair grid (PAIR: causal, Sq = Sk, every pair resident
// at once), one 8-wave workgroup per pair (heavy block i = n-1-p, light block
// p) of a (batch, query head), its two 4-wave groups each with their own K/V
// stages and barrier: group A walks key blocks [0, split) of block i, group B
// all of block p and then [split, 2 i + 2) of block i, so both walk about
// n + 1 blocks and no CU keeps a heavy block running alone while its partner
// has finished.  The two halves of block i's dQ are added through LDS.
template <bool CAUSAL, bool PAIR>
__global__ __launch_bounds__(PAIR ? 2 * kThreadsB : kThreadsB, PAIR ? 1 : 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ delta, uint16_t* __restrict__ dQ, int B, int Hq, int Hkv, int Sq, int Sk, float scale_log2,
    float scale, int n_qblk, int split_bias, int sync_spins, int split_only) {
    // per wave group two stages of (K tile, V tile): the next block lands
    // while this one is used; pair mode adds the groups' barrier counters
    constexpr int GROUP_LDS = 2 * 2 * kKVBlk * kROWB;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[PAIR ? 2 * GROUP_LDS + 64 : GROUP_LDS];

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = PAIR ? wave_id / kWavesB : 0;                 // wave group (pair mode: 0 = A, 1 = B)
    const int wave = PAIR ? wave_id % kWavesB : wave_id;
    uint8_t* const kvs0 = lds + grp * GROUP_LDS;       // the group's stages 0 and 1
    uint8_t* const kvs1 = kvs0 + GROUP_LDS / 2;
    int bar_target = 0;
    bool sync_fail = false;             // a group barrier of this wave ran out (its rows become NaN)
    if constexpr (PAIR) {
        if (tid < 16) reinterpret_cast<int*>(lds + 2 * GROUP_LDS)[tid] = 0;
        __syncthreads();
    }
    // barrier of the waves that share this group's K/V stages
    auto gsync = [&]() __attribute__((always_inline)) {
        if constexpr (PAIR)
            sync_fail |= group_barrier(lds + 2 * GROUP_LDS + 16 * grp, bar_target, lane, sync_spins,
                                       &g_bwd_sync_timeouts);
        else
            __syncthreads();
    };

    const int bh_n = B * Hq;
    const int rank = blockIdx.x / bh_n, rem = blockIdx.x % bh_n;
    const int b = rem / Hq, hq = rem % Hq, kvh = hq / (Hq / Hkv);
    const int64_t bhq = (int64_t)b * Hq + hq;
    const uint16_t* Kh = K + ((int64_t)b * Hkv + kvh) * Sk * kD;
    const uint16_t* Vh = V + ((int64_t)b * Hkv + kvh) * Sk * kD;
    const int diag = Sk - Sq;
    // key blocks query block qb sees
    auto blocks_of = [&](int qb) {
        int kv_end = Sk;
        if (CAUSAL) kv_end = min(Sk, max(0, qb * kQRows + kQRows + diag));
        return (kv_end + kKVBlk - 1) / kKVBlk;
    };

    f32x16 dq[kD / 32];

    // One job: query block qb against key blocks [kb0, kb1); with `final` its
    // dQ is written, else it stays in dq.  The job that starts at key block 0
    // also writes D of its rows for the dK/dV kernel.
    auto run_job = [&](const int qb, const int kb0, const int kb1, const bool final) __attribute__((always_inline)) {
    const int qw = qb * kQRows + wave * 32;        // first query row of this wave
    const int my_q = qw + l32;
    bf16x8 qf[kD / 16], gf[kD / 16];
    load_row_operands(qf, Q + bhq * Sq * kD, my_q, Sq, hh);
    load_row_operands(gf, dO + bhq * Sq * kD, my_q, Sq, hh);
    const float lo = my_q < Sq ? lse_offset(LSE[bhq * Sq + my_q]) : __builtin_inff();
    // D = sum_d dO O of this lane's row: the lane's 64 head-dim elements, then
    // the other half of the row from lane l ^ 32 (rows past Sq: dO = 0, D = 0)
    float Dq;
    {
        bf16x8 of[kD / 16];
        load_row_operands(of, O + bhq * Sq * kD, my_q, Sq, hh);
        float part = 0.f;
#pragma unroll
        for (int s_ = 0; s_ < kD / 16; ++s_)
#pragma unroll
            for (int e = 0; e < 8; ++e) part = fmaf((float)gf[s_][e], (float)of[s_][e], part);
        Dq = half_swap_sum(part);
        if (kb0 == 0 && hh == 0 && my_q < Sq) delta[bhq * Sq + my_q] = Dq;
    }
#pragma unroll
    for (int i = 0; i < kD / 32; ++i) dq[i] = f32x16{};

    if (kb0 < kb1) {
        dma_rows<kKVBlk>(Kh, kvs0, kb0 * kKVBlk, Sk, wave, lane);
        dma_rows<kKVBlk>(Vh, kvs0 + kKVBlk * kROWB, kb0 * kKVBlk, Sk, wave, lane);
    }
    for (int it = 0; it < kb1 - kb0; ++it) {
        const int kv0 = (kb0 + it) * kKVBlk;
        // the lane index made opaque: the operand addresses derived from it
        // are formed in the step instead of being kept live across the loop
        int ln_ = tid & 63;
        asm volatile("" : "+v"(ln_));
        const int lane = ln_, l32 = ln_ & 31, hh = ln_ >> 5;
        // block it has landed for every wave of the group, and every wave is
        // done with block it-1, whose stage the next block goes to
        wait_vm();
        gsync();
        if (kb0 + it + 1 < kb1) {
            uint8_t* const nx = (it & 1) ? kvs0 : kvs1;
            dma_rows<kKVBlk>(Kh, nx, kv0 + kKVBlk, Sk, wave, lane);
            dma_rows<kKVBlk>(Vh, nx + kKVBlk * kROWB, kv0 + kKVBlk, Sk, wave, lane);
        }
        const uint8_t* kt = (it & 1) ? kvs1 : kvs0;
        const uint8_t* vt = kt + kKVBlk * kROWB;

        // S^T = K Q^T and dP^T = V dO^T for keys kv0 .. kv0+63 (two 32-key blocks)
        // (products in the order (s, block, S or dP); each one's LDS operand is
        // read one product ahead)
        f32x16 st[2] = {f32x16{}, f32x16{}}, pt[2] = {f32x16{}, f32x16{}};
        constexpr int NP = kD / 16 * 4;
        auto opnd = [&](int j) {
            const int s = j >> 2, blk = (j >> 1) & 1;
            return row_operand((j & 1) ? vt : kt, 32 * blk + l32, s, hh);
        };
        bf16x8 ring[2];
        ring[0] = opnd(0);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int s = j >> 2, blk = (j >> 1) & 1;
            if (j + 1 < NP) ring[(j + 1) & 1] = opnd(j + 1);
            BWD_FENCE();
            if (j & 1)
                pt[blk] = mfma32(ring[j & 1], gf[s], pt[blk]);
            else
                st[blk] = mfma32(ring[j & 1], qf[s], st[blk]);
            BWD_FENCE();
        }
        // dS^T = P^T o (dP^T - D): register r of block blk is key kv0 + 32 blk +
        // acc_row(r, hh).  Only a block that crosses the wave's diagonal or
        // runs past Sk is masked (a wave-uniform test); there key acc_row(r)
        // of half-block blk is kept iff 8 (r / 4) + r % 4 <= lim, one limit
        // per lane and half-block.
        const bool masked = (kv0 + kKVBlk > Sk) || (CAUSAL && kv0 + kKVBlk - 1 > qw + diag);
        const int last = CAUSAL ? min(Sk - 1, my_q + diag) : Sk - 1;     // last key this row may see
        u32x4 dsw[4];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            float ds[16];
            if (masked) {
                const int lim = last - kv0 - 32 * blk - 4 * hh;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = 8 * (r >> 2) + (r & 3) <= lim ? exp2f_hw(fmaf(st[blk][r], scale_log2, -lo)) : 0.f;
                    ds[r] = p * (pt[blk][r] - Dq);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) ds[r] = exp2f_hw(fmaf(st[blk][r], scale_log2, -lo)) * (pt[blk][r] - Dq);
            }
            u32x4 two[2];
            pack_operand(two, ds);
            dsw[2 * blk] = two[0];
            dsw[2 * blk + 1] = two[1];
        }
        // dQ^T += K^T dS^T over the 64 keys (4 steps of 16)
#pragma unroll
        for (int ks = 0; ks < kKVBlk / 16; ++ks) {
            const bf16x8 bop = __builtin_bit_cast(bf16x8, dsw[ks]);
#pragma unroll
            for (int db = 0; db < kD / 32; ++db) dq[db] = mfma32(tr_operand(kt, ks, db, lane), bop, dq[db]);
        }
    }
    if (final) store_rows(dQ + bhq * Sq * kD, dq, sync_fail ? __builtin_nanf("") : scale, my_q, Sq, hh);
    };   // run_job

    if constexpr (PAIR) {
        const int i = n_qblk - 1 - rank, p = split_only ? i : rank;
        const int ni = blocks_of(i);
        const int split = i != p ? min(n_qblk + 1 + split_bias, ni) : (ni + 1) / 2;
        if (grp == 0) {
            run_job(i, 0, split, false);
        } else {
            if (i != p) {
                run_job(p, 0, blocks_of(p), true);
                gsync();                 // every wave is done with the light block's stages
            }
            run_job(i, split, ni, false);   // (an empty range leaves dq = 0)
        }
        // the halves of block i's dQ meet: A's plus B's, through B's stages
        __syncthreads();                 // both groups done; every stage is free
        float* const st = reinterpret_cast<float*>(lds + GROUP_LDS) + wave * (64 * 16 * (kD / 32));
        if (grp == 1) {
            const float f = sync_fail ? __builtin_nanf("") : 1.f;   // a failed B barrier reaches A's rows
#pragma unroll
            for (int db = 0; db < kD / 32; ++db)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4)
                    *reinterpret_cast<f32x4*>(st + ((db * 4 + a4) * 64 + lane) * 4) =
                        f32x4{dq[db][4 * a4] * f, dq[db][4 * a4 + 1] * f, dq[db][4 * a4 + 2] * f, dq[db][4 * a4 + 3] * f};
        }
        __syncthreads();
        if (grp == 0) {
#pragma unroll
            for (int db = 0; db < kD / 32; ++db)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const f32x4 o = *reinterpret_cast<const f32x4*>(st + ((db * 4 + a4) * 64 + lane) * 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dq[db][4 * a4 + e] += o[e];
                }
            store_rows(dQ + bhq * Sq * kD, dq, sync_fail ? __builtin_nanf("") : scale, i * kQRows + wave * 32 + l32,
                       Sq, hh);
        }
    } else {
        const int qb = CAUSAL ? n_qblk - 1 - rank : rank;     // heaviest causal blocks first
        run_job(qb, 0, blocks_of(qb), true);
    }
}

// One stage of the dK/dV kernel: 32 query rows of Q and of dO (8 KiB each),
// then the rows' lse offsets and D (32 fp32 each), padded to 1 KiB.
constexpr int kQStage = 2 * kQBlk * kROWB + 1024;
constexpr int kQStages = 3;

// dK/dV: one workgroup per (batch, K/V head, 128-key block), each wave owning
// 32 keys whose K and V rows stay in registers for the whole kernel (the B
// operands of S = Q K^T and dP = dO V^T).  The workgroup walks the 32-row
// query blocks of every query head of the GQA group that see its keys; a
// step's Q and dO rows arrive in LDS by buffer loads one step ahead, with the
// rows' lse offsets and D, into three rotating stages.  Step t computes S and
// dP of its rows, then accumulates dV^T += dO^T P and dK^T += Q^T dS of step
// t-1 (its stage is still intact) while the vector unit turns step t's S and
// dP into P and dS, one of the 16 rows a lane holds after each product; the
// last step's dV and dK products follow the loop.
template <bool CAUSAL>
__global__ __launch_bounds__(kThreadsB, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int B, int Hq, int Hkv, int Sq, int Sk, float scale_log2,
    float scale) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kQStages][kQStage];

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh_n = B * Hkv;
    const int kb = blockIdx.x / bh_n, rem = blockIdx.x % bh_n;   // key block 0 (most causal work) first
    const int b = rem / Hkv, kvh = rem % Hkv;
    const int g = Hq / Hkv;
    const int64_t bhk = (int64_t)b * Hkv + kvh;
    const int diag = Sk - Sq;
    const int k0 = kb * kKRows;
    const int my_k = k0 + wave * 32 + l32;

    // this lane's key row of K and V: B operands of S and dP, head-dim step s
    bf16x8 kf[kD / 16], vf[kD / 16];
    {
        const int64_t at = (bhk * Sk + min(my_k, Sk - 1)) * kD + 8 * hh;
#pragma unroll
        for (int s = 0; s < kD / 16; ++s) {
            kf[s] = *reinterpret_cast<const bf16x8*>(K + at + 16 * s);
            vf[s] = *reinterpret_cast<const bf16x8*>(V + at + 16 * s);
        }
    }

    f32x16 dk[kD / 32], dv[kD / 32];
#pragma unroll
    for (int i = 0; i < kD / 32; ++i) dk[i] = dv[i] = f32x16{};

    // the first query row that sees key k0 (bottom-right causal)
    const int q_first = CAUSAL ? max(0, k0 - diag) : 0;
    const int qb0 = q_first / kQBlk, n_qb = (Sq + kQBlk - 1) / kQBlk;
    // the (query head, Q block) steps of this workgroup, flattened
    const int per_head = max(0, n_qb - qb0);
    const int n_steps = g * per_head;
    if (n_steps == 0) {
        store_rows(dK + bhk * Sk * kD, dk, scale, my_k, Sk, hh);
        store_rows(dV + bhk * Sk * kD, dv, 1.f, my_k, Sk, hh);
        return;
    }
    // A step is (query head h of the group, Q block qb0 + i); the loop carries
    // (h, i) and advances it with one compare instead of dividing the step
    // index by the blocks per head.
    struct StepIx {
        int h, i;
    };
    auto next_ix = [&](StepIx x) {
        return ++x.i == per_head ? StepIx{x.h + 1, 0} : x;
    };
    auto step_src = [&](StepIx x, int64_t& bhq, int& q0) {
        bhq = (int64_t)b * Hq + kvh * g + x.h;
        q0 = (qb0 + x.i) * kQBlk;
    };
    // Q and dO rows of step x into a stage (rows past Sq repeat row Sq-1);
    // lanes tid < kQBlk also load the raw lse and D of their row
    auto fetch = [&](StepIx x, uint8_t* __restrict__ st, float& l, float& d) {
        int64_t bhq;
        int q0;
        step_src(x, bhq, q0);
        dma_rows<kQBlk>(Q + bhq * Sq * kD, st, q0, Sq, wave, lane);
        dma_rows<kQBlk>(dO + bhq * Sq * kD, st + kQBlk * kROWB, q0, Sq, wave, lane);
        if (tid < kQBlk) {
            const int64_t at = bhq * Sq + min(q0 + tid, Sq - 1);
            l = LSE[at];
            d = delta[at];
        }
    };
    // once those loads have landed: the lse offset and D the products use (a
    // row past Sq or with no visible key gets offset +inf, so p = 0, and D = 0)
    auto put_rowvals = [&](StepIx x, uint8_t* __restrict__ st, float l, float d) {
        if (tid < kQBlk) {
            int64_t bhq_unused;
            int q0;
            step_src(x, bhq_unused, q0);
            const bool ok = q0 + tid < Sq;
            float* f = reinterpret_cast<float*>(st + 2 * kQBlk * kROWB);
            f[tid] = ok ? lse_offset(l) : __builtin_inff();
            f[kQBlk + tid] = ok ? d : 0.f;
        }
    };

    // Per-lane byte offsets of every LDS operand read within a stage, formed
    // once; a step adds its stage's uniform base.  (Empty asm statements make
    // them opaque, so the compiler neither re-derives them per stage nor
    // keeps one copy per stage.)
    uint32_t ro[kD / 16];               // Q / dO row operand of head-dim step s
    uint32_t to[kD / 32][2];            // transposed operand (ks = 0, db), two reads; ks = 1 is
                                        // 16 rows (4 KiB) further with the same swizzle
    uint32_t fo;                        // this lane half's lse offsets / D
#pragma unroll
    for (int s_ = 0; s_ < kD / 16; ++s_) {
        ro[s_] = (uint32_t)(l32 * kROWB + 16 * ((2 * s_ + hh) ^ swz(l32)));
        asm volatile("" : "+v"(ro[s_]));
    }
    {
        const int sl = lane & 15, gq = lane >> 4, h = gq >> 1;
#pragma unroll
        for (int db = 0; db < kD / 32; ++db) {
            const int col = 32 * db + 16 * (gq & 1) + 4 * (sl & 3);
            const int row0 = 4 * h + (sl >> 2), row1 = row0 + 8;
            const int x = col >> 3, half = (col >> 2) & 1;
            to[db][0] = (uint32_t)(row0 * kROWB + 16 * (x ^ swz(row0)) + 8 * half);
            to[db][1] = (uint32_t)(row1 * kROWB + 16 * (x ^ swz(row1)) + 8 * half);
            asm volatile("" : "+v"(to[db][0]), "+v"(to[db][1]));
        }
    }
    fo = (uint32_t)(2 * kQBlk * kROWB + 4 * 4 * hh);
    asm volatile("" : "+v"(fo));

    float lraw = 0.f, draw = 0.f;
    fetch(StepIx{0, 0}, lds[0], lraw, draw);
    wait_vm();
    put_rowvals(StepIx{0, 0}, lds[0], lraw, draw);
    __syncthreads();

    u32x4 pw_prev[2], dsw_prev[2];   // P and dS of the previous step, bf16 B operands

    // dV^T += dO^T P and dK^T += Q^T dS of the step whose stage is `st`; the
    // transposed operands read three products ahead; `between(j)` after product j
    auto dkdv = [&](const uint8_t* __restrict__ st, const u32x4 (&pw)[2], const u32x4 (&dsw)[2], auto&& between) {
        constexpr int NJ = 2 * 2 * (kD / 32);  // (ks, db, dV or dK)
        auto top = [&](int j) {
            const int ks = j / (2 * (kD / 32)), db = (j >> 1) % (kD / 32);
            const uint8_t* t0 = st + ((j & 1) ? 0 : kQBlk * kROWB);      // Q^T for dK, dO^T for dV
            const uint8_t* const tk = t0 + 16 * kROWB * ks;   // swz(row + 16) == swz(row)
            const s16x4 a = lds_read_tr16(tk + to[db][0]), c = lds_read_tr16(tk + to[db][1]);
            const s16x8 v = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
            return __builtin_bit_cast(bf16x8, v);
        };
        bf16x8 ring[4];
        ring[0] = top(0);
        ring[1] = top(1);
        ring[2] = top(2);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int ks = j / (2 * (kD / 32)), db = (j >> 1) % (kD / 32);
            if (j + 3 < NJ) ring[(j + 3) % 4] = top(j + 3);
            BWD_FENCE();
            if (j & 1)
                dk[db] = mfma32(ring[j % 4], __builtin_bit_cast(bf16x8, dsw[ks]), dk[db]);
            else
                dv[db] = mfma32(ring[j % 4], __builtin_bit_cast(bf16x8, pw[ks]), dv[db]);
            BWD_FENCE();
            between(j);
            BWD_FENCE();
        }
    };

    // Step t: its rows are in stage cur, step t-1's in prev (FIRST: none),
    // step t+1's rows go to nxt.  The stages come in as restrict pointers, so
    // the operand reads of two do not wait for the loads into the third.
    auto step = [&](auto first_c, const int t, const StepIx x, uint8_t* __restrict__ cur, uint8_t* __restrict__ prev,
                    uint8_t* __restrict__ nxt) __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first_c)::value;
        const bool has_next = t + 1 < n_steps;
        const StepIx xn = next_ix(x);
        float lnext = 0.f, dnext = 0.f;
        if (has_next) fetch(xn, nxt, lnext, dnext);

        // S = Q K^T and dP = dO V^T: register r is query row q0 + acc_row(r, hh),
        // lane = key; Q and dO operands read two products ahead
        f32x16 sc = f32x16{}, pc = f32x16{};
        {
            constexpr int NP = kD / 16 * 2;        // products: (s, S or dP)
            bf16x8 ring[3];
            auto opnd = [&](int j) {
                return *reinterpret_cast<const bf16x8*>(cur + ((j & 1) ? kQBlk * kROWB : 0) + ro[j >> 1]);
            };
            ring[0] = opnd(0);
            ring[1] = opnd(1);
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                if (j + 2 < NP) ring[(j + 2) % 3] = opnd(j + 2);
                BWD_FENCE();
                if (j & 1)
                    pc = mfma32(ring[j % 3], vf[j >> 1], pc);
                else
                    sc = mfma32(ring[j % 3], kf[j >> 1], sc);
                BWD_FENCE();
            }
        }
        // the rows' lse offsets and D come in four groups of four consecutive
        // rows; a group is read from the stage one group ahead of its use (two
        // groups in registers instead of all 32 values)
        const float* const rowf = reinterpret_cast<const float*>(cur + fo);
        f32x4 lo_g[2], dd_g[2];
        lo_g[0] = *reinterpret_cast<const f32x4*>(rowf);
        dd_g[0] = *reinterpret_cast<const f32x4*>(rowf + kQBlk);
        int64_t bhq_unused;
        int q0;
        step_src(x, bhq_unused, q0);
        // causal: key my_k is visible to row q iff q >= my_k - diag, i.e. the
        // register's constant row offset 8 (r / 4) + r % 4 >= thr
        const int thr = my_k - diag - q0 - 4 * hh;
        u32x4 pw[2], dsw[2];
        float pv[16], dsv[16];
        auto unit = [&](int r) {
            const int grp = r >> 2;
            if ((r & 3) == 0 && grp + 1 < 4) {
                lo_g[(grp + 1) & 1] = *reinterpret_cast<const f32x4*>(rowf + 8 * (grp + 1));
                dd_g[(grp + 1) & 1] = *reinterpret_cast<const f32x4*>(rowf + kQBlk + 8 * (grp + 1));
            }
            const float lo_r = lo_g[grp & 1][r & 3], dd_r = dd_g[grp & 1][r & 3];
            float x = fmaf(sc[r], scale_log2, -lo_r);
            asm volatile("" : "+v"(x));
            float e = exp2f_hw(x);
            if (CAUSAL) e = (8 * (r >> 2) + (r & 3)) >= thr ? e : 0.f;
            pv[r] = e;
            dsv[r] = e * (pc[r] - dd_r);
            if (r & 1) {
                uint32_t wp = pack_bf16x2(pv[r - 1], pv[r]), wd = pack_bf16x2(dsv[r - 1], dsv[r]);
                asm volatile("" : "+v"(wp), "+v"(wd));
                pw[r >> 3][(r & 7) >> 1] = wp;
                dsw[r >> 3][(r & 7) >> 1] = wd;
            }
        };
        if constexpr (FIRST) {
#pragma unroll
            for (int r = 0; r < 16; ++r) unit(r);
        } else {
            dkdv(prev, pw_prev, dsw_prev, [&](int j) { unit(j); });
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            pw_prev[i] = pw[i];
            dsw_prev[i] = dsw[i];
        }
        if (has_next) {
            wait_vm();
            put_rowvals(xn, nxt, lnext, dnext);
        }
        // step t+1's rows are in place; every wave is done with stage prev
        __syncthreads();
    };
    using First = std::integral_constant<bool, true>;
    using Later = std::integral_constant<bool, false>;
    // unrolled by three so that each step's stages are fixed addresses
    uint8_t* const st0 = lds[0];
    uint8_t* const st1 = lds[1];
    uint8_t* const st2 = lds[2];
    StepIx x{0, 0};
    step(First{}, 0, x, st0, st2, st1);
    for (int t = 1; t < n_steps; ++t) {
        x = next_ix(x);
        // the three stage bases as opaque scalars: one add per operand address
        uint32_t bc = (uint32_t)(t % kQStages) * kQStage, bp = (uint32_t)((t + 2) % kQStages) * kQStage,
                 bn = (uint32_t)((t + 1) % kQStages) * kQStage;
        asm volatile("" : "+s"(bc), "+s"(bp), "+s"(bn));
        step(Later{}, t, x, &lds[0][0] + bc, &lds[0][0] + bp, &lds[0][0] + bn);
    }
    // the last step's dV and dK products
    {
        uint8_t* const last = lds[(n_steps - 1) % kQStages];
        dkdv(last, pw_prev, dsw_prev, [](int) {});
    }
    store_rows(dK + bhk * Sk * kD, dk, scale, my_k, Sk, hh);
    store_rows(dV + bhk * Sk * kD, dv, 1.f, my_k, Sk, hh);
}

int bwd_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// K/V blocks of the heavy query block moved from group B to group A of a dQ
// pair (B also pays a second job start and the light block's output).
constexpr int kDqSplitBias = 0;

template <bool CAUSAL>
hipError_t launch(const BwdArgs& a, hipStream_t stream) {
    const float scale_log2 = a.scale * kLog2e;
    const int n_qblk = (a.Sq + kQRows - 1) / kQRows;
    const int n_pairs = (n_qblk + 1) / 2;
    // pair grid for dQ: a causal square problem whose heavy/light query-block
    // pairs all fit one 8-wave workgroup per CU; when they would fill half the
    // CUs or fewer and there are 8 or more query blocks, each block gets a
    // workgroup of its own, halved between the two wave groups (split-only)
    const int64_t n_pair_wg = (int64_t)a.B * a.Hq * n_pairs;
    const int split_only = (2 * n_pair_wg <= bwd_cus() && n_qblk >= 8) ? 1 : 0;
    if (CAUSAL && a.Sq == a.Sk && a.Sq % kQRows == 0 && n_qblk >= 2 && n_pair_wg <= bwd_cus()) {
        launch_kernel<false>((bwd_dq_kernel<CAUSAL, true>),
                             dim3((unsigned)(split_only ? (int64_t)a.B * a.Hq * n_qblk : n_pair_wg)),
                             dim3(2 * kThreadsB), 0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                             (const uint16_t*)a.v, (const uint16_t*)a.o, (const uint16_t*)a.dout, a.lse, a.delta,
                             (uint16_t*)a.dq, a.B, a.Hq, a.Hkv, a.Sq, a.Sk, scale_log2, a.scale, n_qblk, kDqSplitBias,
                             a.sync_spins, split_only);
    } else {
        launch_kernel<false>((bwd_dq_kernel<CAUSAL, false>), dim3((unsigned)((int64_t)a.B * a.Hq * n_qblk)),
                             dim3(kThreadsB), 0, stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                             (const uint16_t*)a.v, (const uint16_t*)a.o, (const uint16_t*)a.dout, a.lse, a.delta,
                             (uint16_t*)a.dq, a.B, a.Hq, a.Hkv, a.Sq, a.Sk, scale_log2, a.scale, n_qblk, 0,
                             a.sync_spins, 0);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_kblk = (a.Sk + kKRows - 1) / kKRows;
    launch_kernel((bwd_dkdv_kernel<CAUSAL>), dim3((unsigned)((int64_t)a.B * a.Hkv * n_kblk)), dim3(kThreadsB), 0,
                       stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, a.delta, (uint16_t*)a.dk, (uint16_t*)a.dv, a.B, a.Hq, a.Hkv,
                       a.Sq, a.Sk, scale_log2, a.scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
    return a.causal ? launch<true>(a, stream) : launch<false>(a, stream);
}

hipError_t read_bwd_sync_timeouts(unsigned int* count) {
    return read_device_counter(&HIP_SYMBOL(g_bwd_sync_timeouts), count);
}

}  // namespace fa
