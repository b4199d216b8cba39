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
// (D_i equals sum_j P_ij dP_ij because O = P V).  Three kernels, no atomics:
//
//   * bwd_delta_kernel: D for every query row (16 lanes per row, DPP sum).
//   * bwd_dq_kernel: one workgroup per (batch, query head, 128-row Q block),
//     walking the K/V blocks the rows can see, like the forward.  Each wave
//     owns 32 query rows and computes S^T = K Q^T and dP^T = V dO^T on the
//     matrix cores (so every lane holds one query row: its lse and D are one
//     value), forms dS^T in registers, and accumulates dQ^T += K^T dS^T with
//     the K tile read transposed from LDS.
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
// the global-to-LDS load; rows past S repeat row S-1.  Load sl fills the
// 1 KiB slice sl (4 rows); lane l lands at byte 16 l of it and fetches the
// logical chunk that the swizzle places there.
template <int ROWS>
__device__ __forceinline__ void dma_rows(const uint16_t* __restrict__ src, uint8_t* __restrict__ tile, int r0, int S,
                                         int wave, int lane) {
    static_assert(ROWS % (4 * kWavesB) == 0, "every wave issues the same number of loads");
    const int rr = lane >> 4, ch = lane & 15;
#pragma unroll
    for (int i = 0; i < ROWS / 4 / kWavesB; ++i) {
        const int sl = wave + i * kWavesB;
        const int row = 4 * sl + rr;
        const uint16_t* g = src + (int64_t)min(r0 + row, S - 1) * kD + 8 * (ch ^ swz(row));
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                         (__attribute__((address_space(3))) void*)(tile + sl * 1024), 16, 0, 0);
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

// D_i = sum_d dO_id O_id for every query row; one row per 16 lanes.
__global__ __launch_bounds__(kThreadsB) void bwd_delta_kernel(const uint16_t* __restrict__ O,
                                                              const uint16_t* __restrict__ dO,
                                                              float* __restrict__ delta, int64_t rows) {
    const int64_t row = (int64_t)blockIdx.x * (kThreadsB / 16) + (threadIdx.x >> 4);
    const int t = threadIdx.x & 15;
    float acc = 0.f;
    if (row < rows) {
        const u32x4 o = *reinterpret_cast<const u32x4*>(O + row * kD + 8 * t);
        const u32x4 g = *reinterpret_cast<const u32x4*>(dO + row * kD + 8 * t);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t ow = o[w], gw = g[w];
            acc = fmaf(bf16lo_to_f32(ow), bf16lo_to_f32(gw), acc);
            acc = fmaf(bf16hi_to_f32(ow), bf16hi_to_f32(gw), acc);
        }
    }
    acc = row_sum16(acc);
    if (row < rows && t == 0) delta[row] = acc;
}

// lse (natural log) -> the log2-domain offset of exp2; a row with no visible
// key (lse = -inf) gets +inf so that every p of it is exactly 0.
__device__ __forceinline__ float lse_offset(float lse) { return lse == kNegInf ? __builtin_inff() : lse * kLog2e; }

template <bool CAUSAL>
__global__ __launch_bounds__(kThreadsB, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
    uint16_t* __restrict__ dQ, int B, int Hq, int Hkv, int Sq, int Sk, float scale_log2, float scale, int n_qblk) {
    // two stages of (K tile, V tile): the next block lands while this one is used
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2 * kKVBlk * kROWB];

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh_n = B * Hq;
    const int rank = blockIdx.x / bh_n, rem = blockIdx.x % bh_n;
    const int qb = CAUSAL ? n_qblk - 1 - rank : rank;     // heaviest causal blocks first
    const int b = rem / Hq, hq = rem % Hq, kvh = hq / (Hq / Hkv);
    const int64_t bhq = (int64_t)b * Hq + hq;
    const uint16_t* Kh = K + ((int64_t)b * Hkv + kvh) * Sk * kD;
    const uint16_t* Vh = V + ((int64_t)b * Hkv + kvh) * Sk * kD;
    const int diag = Sk - Sq;
    const int my_q = qb * kQRows + wave * 32 + l32;

    bf16x8 qf[kD / 16], gf[kD / 16];
    load_row_operands(qf, Q + bhq * Sq * kD, my_q, Sq, hh);
    load_row_operands(gf, dO + bhq * Sq * kD, my_q, Sq, hh);
    const float lo = my_q < Sq ? lse_offset(LSE[bhq * Sq + my_q]) : __builtin_inff();
    const float Dq = my_q < Sq ? delta[bhq * Sq + my_q] : 0.f;

    int kv_end = Sk;
    if (CAUSAL) kv_end = min(Sk, max(0, qb * kQRows + kQRows + diag));
    const int n_it = (kv_end + kKVBlk - 1) / kKVBlk;

    f32x16 dq[kD / 32];
#pragma unroll
    for (int i = 0; i < kD / 32; ++i) dq[i] = f32x16{};

    if (n_it > 0) {
        dma_rows<kKVBlk>(Kh, lds[0], 0, Sk, wave, lane);
        dma_rows<kKVBlk>(Vh, lds[0] + kKVBlk * kROWB, 0, Sk, wave, lane);
    }
    for (int it = 0; it < n_it; ++it) {
        const int kv0 = it * kKVBlk;
        // block it has landed for every wave, and every wave is done with block it-1,
        // whose stage the next block goes to
        wait_vm();
        __syncthreads();
        if (it + 1 < n_it) {
            dma_rows<kKVBlk>(Kh, lds[(it + 1) & 1], kv0 + kKVBlk, Sk, wave, lane);
            dma_rows<kKVBlk>(Vh, lds[(it + 1) & 1] + kKVBlk * kROWB, kv0 + kKVBlk, Sk, wave, lane);
        }
        const uint8_t* kt = lds[it & 1];
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
        // dS^T = P^T o (dP^T - D): register r of block blk is key kv0 + 32 blk + acc_row(r, hh)
        u32x4 dsw[4];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            float ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 32 * blk + acc_row(r, hh);
                const bool ok = key < Sk && (!CAUSAL || key <= my_q + diag);
                const float p = ok ? exp2f_hw(fmaf(st[blk][r], scale_log2, -lo)) : 0.f;
                ds[r] = p * (pt[blk][r] - Dq);
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
    store_rows(dQ + bhq * Sq * kD, dq, scale, my_q, Sq, hh);
}

template <bool CAUSAL>
__global__ __launch_bounds__(kThreadsB, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int B, int Hq, int Hkv, int Sq, int Sk, float scale_log2,
    float scale) {
    // two stages of (Q tile, dO tile) and of the rows' lse offsets and D, and
    // the K and V rows of this workgroup's keys (operands of S and dP)
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2 * kQBlk * kROWB];
    __shared__ __attribute__((aligned(1024))) uint8_t kv_lds[2][kKRows * kROWB];
    __shared__ float s_lo[2][kQBlk], s_d[2][kQBlk];

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

    dma_rows<kKRows>(K + bhk * Sk * kD, kv_lds[0], k0, Sk, wave, lane);
    dma_rows<kKRows>(V + bhk * Sk * kD, kv_lds[1], k0, Sk, wave, lane);
    wait_vm();
    __syncthreads();
    const int krow = wave * 32 + l32;          // this lane's key row in kv_lds

    f32x16 dk[kD / 32], dv[kD / 32];
#pragma unroll
    for (int i = 0; i < kD / 32; ++i) dk[i] = dv[i] = f32x16{};

    // the first query row that sees key k0 (bottom-right causal)
    const int q_first = CAUSAL ? max(0, k0 - diag) : 0;
    const int qb0 = q_first / kQBlk, n_qb = (Sq + kQBlk - 1) / kQBlk;
    // the (query head, Q block) steps of this workgroup, flattened so that
    // the next step's tiles are loaded while the current one is computed
    const int per_head = max(0, n_qb - qb0);
    const int n_steps = g * per_head;
    auto step_src = [&](int t, int64_t& bhq, int& q0) {
        bhq = (int64_t)b * Hq + kvh * g + t / per_head;
        q0 = (qb0 + t % per_head) * kQBlk;
    };
    // The next step's Q and dO rows are loaded into registers while the
    // current step computes (each thread holds two 16-byte chunks of each
    // tile: chunk c = tid + 256 i is row c / 16, logical chunk c % 16) and
    // written to the other LDS stage, swizzled, at the start of the next
    // step; the raw lse and D of the rows (lanes < kQBlk, row clamped to
    // Sq-1) likewise.  Staging through registers instead of global-to-LDS
    // loads keeps the compiler from waiting for the prefetch before the
    // first LDS read of the step.
    constexpr int kChunks = kQBlk * kD / 8 / kThreadsB;    // 16-byte chunks per thread per tile
    u32x4 qn[kChunks], gn[kChunks];
    float lse_next = 0.f, d_next = 0.f;
    auto fetch = [&](int t) {
        int64_t bhq;
        int q0;
        step_src(t, bhq, q0);
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int c = tid + kThreadsB * i, row = c >> 4, ch = c & 15;
            const int64_t at = (bhq * Sq + min(q0 + row, Sq - 1)) * kD + 8 * ch;
            qn[i] = *reinterpret_cast<const u32x4*>(Q + at);
            gn[i] = *reinterpret_cast<const u32x4*>(dO + at);
        }
        if (tid < kQBlk) {
            const int64_t at = bhq * Sq + min(q0 + tid, Sq - 1);
            lse_next = LSE[at];
            d_next = delta[at];
        }
    };
    if (n_steps > 0) fetch(0);
    for (int t = 0; t < n_steps; ++t) {
        const int stage = t & 1;
        int64_t bhq_unused;
        int q0;
        step_src(t, bhq_unused, q0);
        uint8_t* const qt = lds[stage];
        uint8_t* const gt = qt + kQBlk * kROWB;
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int c = tid + kThreadsB * i, row = c >> 4, ch = c & 15;
            const int off = row * kROWB + 16 * (ch ^ swz(row));
            *reinterpret_cast<u32x4*>(qt + off) = qn[i];
            *reinterpret_cast<u32x4*>(gt + off) = gn[i];
        }
        if (tid < kQBlk) {
            const bool row_ok = q0 + tid < Sq;
            s_lo[stage][tid] = row_ok ? lse_offset(lse_next) : __builtin_inff();
            s_d[stage][tid] = row_ok ? d_next : 0.f;
        }
        // step t's tiles and row values are in place, and every wave is done
        // with step t-1 (the other stage, rewritten at the start of step t+1)
        __syncthreads();
        if (t + 1 < n_steps) fetch(t + 1);
        const float* lo_s = s_lo[stage];
        const float* d_s = s_d[stage];

        // S = Q K^T and dP = dO V^T: register r is query row q0 + acc_row(r, hh), lane = key
        // (one wave per SIMD: the operands of head-dim step s + 1 are read while
        // step s computes, and the rows' lse offsets and D before the products)
        float lo_r[16], dd_r[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            lo_r[r] = lo_s[acc_row(r, hh)];
            dd_r[r] = d_s[acc_row(r, hh)];
        }
        f32x16 st = f32x16{}, pt = f32x16{};
        bf16x8 qa[2], ka[2], ga[2], va[2];
        qa[0] = row_operand(qt, l32, 0, hh);
        ka[0] = row_operand(kv_lds[0], krow, 0, hh);
        ga[0] = row_operand(gt, l32, 0, hh);
        va[0] = row_operand(kv_lds[1], krow, 0, hh);
#pragma unroll
        for (int s = 0; s < kD / 16; ++s) {
            const int c = s & 1;
            if (s + 1 < kD / 16) {
                qa[c ^ 1] = row_operand(qt, l32, s + 1, hh);
                ka[c ^ 1] = row_operand(kv_lds[0], krow, s + 1, hh);
                ga[c ^ 1] = row_operand(gt, l32, s + 1, hh);
                va[c ^ 1] = row_operand(kv_lds[1], krow, s + 1, hh);
            }
            BWD_FENCE();
            st = mfma32(qa[c], ka[c], st);
            pt = mfma32(ga[c], va[c], pt);
            BWD_FENCE();
        }
        float p[16], ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int qi = acc_row(r, hh), q = q0 + qi;
            const bool ok = q < Sq && my_k < Sk && (!CAUSAL || my_k <= q + diag);
            const float e = exp2f_hw(fmaf(st[r], scale_log2, -lo_r[r]));
            p[r] = ok ? e : 0.f;
            ds[r] = p[r] * (pt[r] - dd_r[r]);
        }
        u32x4 pw[2], dsw[2];
        pack_operand(pw, p);
        pack_operand(dsw, ds);
        // dV^T += dO^T P and dK^T += Q^T dS over the 32 query rows (2 steps of 16)
#pragma unroll
        for (int ks = 0; ks < kQBlk / 16; ++ks) {
            const bf16x8 bp = __builtin_bit_cast(bf16x8, pw[ks]), bd = __builtin_bit_cast(bf16x8, dsw[ks]);
#pragma unroll
            for (int db = 0; db < kD / 32; ++db) {
                dv[db] = mfma32(tr_operand(gt, ks, db, lane), bp, dv[db]);
                dk[db] = mfma32(tr_operand(qt, ks, db, lane), bd, dk[db]);
            }
        }
    }
    store_rows(dK + bhk * Sk * kD, dk, scale, my_k, Sk, hh);
    store_rows(dV + bhk * Sk * kD, dv, 1.f, my_k, Sk, hh);
}

template <bool CAUSAL>
hipError_t launch(const BwdArgs& a, hipStream_t stream) {
    const float scale_log2 = a.scale * kLog2e;
    const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
    launch_kernel<false>(bwd_delta_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(kThreadsB), 0, stream,
                       (const uint16_t*)a.o, (const uint16_t*)a.dout, a.delta, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_qblk = (a.Sq + kQRows - 1) / kQRows;
    launch_kernel<false>((bwd_dq_kernel<CAUSAL>), dim3((unsigned)((int64_t)a.B * a.Hq * n_qblk)), dim3(kThreadsB), 0,
                       stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, a.delta, (uint16_t*)a.dq, a.B, a.Hq, a.Hkv, a.Sq, a.Sk,
                       scale_log2, a.scale, n_qblk);
    e = hipGetLastError();
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

}  // namespace fa
