// Prefill attention forward, bf16 in / bf16 out, fp32 accumulation, gfx950.
//
// One workgroup owns one block of 128 query rows of one (batch, query head)
// and walks the K/V blocks of its key/value head (the loop order of
// "FlashAttention scaling, multi-GPU training and weight quantization",
// section 1: outer loop over Q blocks spread across the grid, inner loop over
// K/V).  Per K/V block ("Fast Inference and Training at Scale", section 6.21,
// tiling):
//
//   1. K_j and V_j are copied from HBM/L2 straight into LDS with the
//      buffer load to LDS (no registers involved, 256-byte coalesced rows),
//      K one block ahead of V, each in its own double buffer; one barrier per
//      block.  Both tiles are row-major with XOR-swizzled 16-byte chunks, so
//      the operand reads below hit distinct banks.
//   2. Scores come from the matrix cores.  Each wave owns 32 query rows and
//      computes the transposed block S^T = K_j Q^T, so that every lane holds
//      scores of a single query row: the row maximum and row sum are in-lane
//      reductions plus one swap between lane halves.
//   3. Online softmax ("Hardware Co-Design"; "Week 13. GPUs and
//      FlashAttention", Step 2): p = 2^(s - m) with the scale and log2 e
//      folded into one multiply-add; the output and running sum are rescaled
//      by 2^(m_old - m_new) when the reference maximum moves.  A row with no
//      visible key so far keeps m = -inf and contributes exactly zero (the
//      -inf guard of the "Common mistakes" list).
//   4. O^T += V_j^T P^T on the matrix cores; P is rounded to bf16 once.  The
//      V^T operand is read from the row-major V tile with the transposing LDS
//      read (ds_read_b64_tr_b16), whose addresses also put the keys in the
//      order in which the lanes hold P.
//   5. After the last block the output is divided by the running sum once
//      (the division is postponed to the end, section 1 of the FlashAttention
//      page) and lse = (m + log2 l) ln 2 is written per row.
//
// The loop is software-pipelined inside each wave so the matrix core never
// waits for the softmax: while it computes the scores of block j+1 the wave
// exponentiates block j, and while it accumulates P_j V_j the wave takes the
// maximum of block j+1.  Scheduling fences fix that interleave.
//
// Causal: the loop stops at the last K/V block any row of the Q block can see
// and the elementwise mask is applied only to blocks that straddle the
// diagonal ("Week 13", Step 2: blocks fully above the diagonal are skipped).
// Workgroups are ordered heaviest-first and, when the number of K/V heads
// allows it, so that each of the 8 XCDs (each with its own L2) serves a
// disjoint set of K/V heads.  When the whole grid fits on the GPU at once, the
// second half of the grid runs the Q blocks in the opposite order, so that the
// two workgroups that share a CU carry complementary causal work.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per inner step
constexpr float kTau = 8.f;       // log2 of the growth allowed before a rescale

template <int D>
struct Tile {
    static constexpr int ROWB = D * 2;                   // bytes per K or V row (no padding)
    static constexpr int CHUNKS = D / 8;                 // 16-byte chunks per row
    static constexpr int K_BYTES = kBN * ROWB;           // one K stage
    static constexpr int V_BYTES = kBN * ROWB;           // one V stage
    static constexpr int ROWS_PER_LOAD = 1024 / ROWB;    // rows one wave-wide 16-byte load covers
    static constexpr int LOADS = kBN / ROWS_PER_LOAD / kWaves;   // loads per wave per tile
    static_assert(kBN % (ROWS_PER_LOAD * kWaves) == 0, "tile split");
};

// XOR swizzles of the 16-byte chunk index within a row.  K operand reads
// take one chunk from 16 consecutive rows; V^T operand reads take 8-byte
// pieces of 4 consecutive chunks from 4 consecutive rows.  Both patterns land
// on distinct banks with these maps.
template <int D>
__device__ __forceinline__ int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }

// Copy the 64-row block starting at row kv0 of a [S, D] tensor into an LDS
// stage with the buffer load to LDS.  Load c of wave w fills the 1 KiB slice
// c * kWaves + w of the stage, and its lane l lands at byte 16 l of that
// slice, so each lane fetches the logical chunk that the swizzle places
// there: row = slice * ROWS_PER_LOAD + l / CHUNKS, physical chunk l % CHUNKS.
// The swizzles repeat every 16 (K) or 4 (V) rows, a divisor of the rows
// between two loads of a lane, so a lane's loads share one chunk: a full
// block is addressed by a buffer resource at row kv0 (scalar registers), a
// per-load scalar offset and one loop-invariant lane offset `lane_off` (in
// elements).  In the ragged last block rows past Sk repeat row Sk - 1: their
// scores are masked and their p is exactly zero.
//
// The buffer form (rather than the global one) matters for the waits: the
// compiler counts a global-to-LDS load as both a memory and an LDS access,
// and while one is outstanding it turns every wait for an LDS operand read
// into a wait for all of them, which undoes the operand read-ahead.
template <int D, bool IS_K>
__device__ __forceinline__ int dma_lane_offset(int wave, int lane) {
    using T = Tile<D>;
    const int row = wave * T::ROWS_PER_LOAD + lane / T::CHUNKS;
    const int chunk = (lane % T::CHUNKS) ^ (IS_K ? swz_k<D>(row) : swz_v<D>(row));
    return row * D + chunk * 8;
}

template <int D>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ src, uint8_t* stage, int lane_off, int kv0,
                                         int Sk, int wave) {
    using T = Tile<D>;
    constexpr int ROW_STEP = kWaves * T::ROWS_PER_LOAD;   // rows between two loads of a lane
    static_assert(ROW_STEP % 16 == 0, "a lane's loads must share one swizzled chunk");
#if defined(__HIP_DEVICE_COMPILE__)   // (the buffer builtins exist only for the device pass)
    // every byte a lane of this block reads lies within the block's kBN rows
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src + (int64_t)kv0 * D), 0, kBN * T::ROWB, 0x00020000);
    if (kv0 + kBN <= Sk) {
        const uint32_t lane_bytes = (uint32_t)lane_off * 2u;
#pragma unroll
        for (int c = 0; c < T::LOADS; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(stage + (c * kWaves + wave) * 1024), 16, lane_bytes,
                c * ROW_STEP * T::ROWB, 0, 0);
    } else {
        const int row0 = lane_off / D;
#pragma unroll
        for (int c = 0; c < T::LOADS; ++c) {
            const int row = min(row0 + c * ROW_STEP, Sk - 1 - kv0);
            const uint32_t bytes = (uint32_t)(row * D + (lane_off - row0 * D)) * 2u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(stage + (c * kWaves + wave) * 1024), 16, bytes, 0, 0, 0);
        }
    }
#endif
}

// s_waitcnt vmcnt(0): every global(-to-LDS) load of this wave has landed.
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

typedef short s16x4 __attribute__((ext_vector_type(4)));

// 8 bytes at an LDS byte address, transposed across each 16-lane group:
// lane i of a group receives element i % 4 of the 8-byte pieces addressed by
// lanes 4k + i / 4 (k = 0..3).
__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const __attribute__((address_space(3))) uint8_t*)p);
}

#define FA_FENCE() __builtin_amdgcn_sched_barrier(0)

// Scores of one 64-key block for this wave's 32 rows: S^T = K Q^T, the two
// 32-key halves as interleaved MFMA chains, LDS operand reads one step ahead.
// After each product k (k = 0 .. 2 NS - 1) the callback `between(k)` is
// emitted, so independent vector work fills the matrix core's busy time
// instead of waiting behind a second product.
template <int D, typename F>
__device__ __forceinline__ void score_block(f32x16 (&sacc)[2], const uint8_t* kt, const bf16x8 (&qf)[D / 16],
                                            int l32, int hh, F&& between) {
    using T = Tile<D>;
    constexpr int NS = D / 16;
    // rows l32 and l32 + 32 share the swizzle (32 is a multiple of its period)
    const uint8_t* kr0 = kt + l32 * T::ROWB;
    const uint8_t* kr1 = kr0 + 32 * T::ROWB;
    const int sw = swz_k<D>(l32);
    auto rd = [&](const uint8_t* r, int s) {
        return *reinterpret_cast<const bf16x8*>(r + 16 * ((2 * s + hh) ^ sw));
    };
    // operands of step s in ring slot s % 3, read two steps ahead
    bf16x8 ka[3][2];
    ka[0][0] = rd(kr0, 0);
    ka[0][1] = rd(kr1, 0);
    if (NS > 1) {
        ka[1][0] = rd(kr0, 1);
        ka[1][1] = rd(kr1, 1);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (s + 2 < NS) {
            ka[(s + 2) % 3][0] = rd(kr0, s + 2);
            ka[(s + 2) % 3][1] = rd(kr1, s + 2);
        }
        FA_FENCE();
        sacc[0] = mfma32(ka[s % 3][0], qf[s], sacc[0]);
        FA_FENCE();
        between(2 * s);
        FA_FENCE();
        sacc[1] = mfma32(ka[s % 3][1], qf[s], sacc[1]);
        FA_FENCE();
        between(2 * s + 1);
        FA_FENCE();
    }
}

// V^T operand for output block db and key step ks (keys 16 ks .. +15): lane l
// (column c = l % 32 of the block, half h = l / 32) needs V[key][c] for the
// keys 4h + e (e = 0..3) and 8 + 4h + e, the order in which it holds P.  Two
// transposing reads: lane s of each 16-lane group g addresses row
// 16 ks + 4h + s / 4 (+ 8), columns 32 db + 16 (g % 2) + 4 (s % 4) .. +3.
template <int D>
__device__ __forceinline__ bf16x8 vt_operand(const uint8_t* vt, int ks, int db, int lane) {
    using T = Tile<D>;
    const int s = lane & 15, g = lane >> 4, h = g >> 1;
    const int col = 32 * db + 16 * (g & 1) + 4 * (s & 3);          // element column
    const int row0 = 16 * ks + 4 * h + (s >> 2);
    const int row1 = row0 + 8;
    const int x = col >> 3, half = (col >> 2) & 1;                  // 16-byte chunk, 8-byte half
    const uint8_t* p0 = vt + row0 * T::ROWB + 16 * (x ^ swz_v<D>(row0)) + 8 * half;
    const uint8_t* p1 = vt + row1 * T::ROWB + 16 * (x ^ swz_v<D>(row1)) + 8 * half;
    const s16x4 a = lds_read_tr16(p0), b = lds_read_tr16(p1);
    const s16x4 lo = a, hi = b;
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Mask the scores of block kv0 .. kv0+63: keys past Sk, and keys above the
// causal diagonal of this lane's row.  Accumulator register r of lane half
// hh holds key kv0 + 32 blk + acc_row(r, hh), and both conditions are an
// upper bound on that key, so each half-block needs one per-lane limit and
// then one compare with the register's constant row offset and one select
// per score.
template <bool CAUSAL>
__device__ __forceinline__ void mask_block(f32x16 (&sacc)[2], int kv0, int Sk, int my_q, int diag, int hh) {
    const int last = CAUSAL ? min(Sk - 1, my_q + diag) : Sk - 1;    // last visible key of this row
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        // visible iff 8 (r / 4) + r % 4 <= lim
        const int lim = last - kv0 - 32 * blk - 4 * hh;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[blk][r] = (8 * (r >> 2) + (r & 3)) <= lim ? sacc[blk][r] : kNegInf;
    }
}

// Wave-group barrier waits that ran out, per device (read and cleared by
// read_sync_timeouts).
__device__ unsigned int g_sync_timeouts;
static_assert(kWaves == 4, "group_barrier counts four waves per group");

template <int D, bool CAUSAL, bool PAIR>
__global__ __launch_bounds__(PAIR ? 2 * kThreads : kThreads, PAIR ? 1 : 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int Sq, int Sk,
    float scale_log2, int n_qblk, int n_rank, int xcd_groups, int mirror, int split_bias, int sync_spins,
    int split_only) {
    using T = Tile<D>;
    constexpr int NS = D / 16;          // MFMA steps of one score block
    constexpr int NDB = D / 32;         // 32-wide head-dim blocks of the output
    constexpr int GROUP_LDS = 2 * T::K_BYTES + 2 * T::V_BYTES;
    // pair mode: two wave groups, each with its own K/V stages, plus their barrier counters
    __shared__ __attribute__((aligned(1024))) uint8_t lds[PAIR ? 2 * GROUP_LDS + 64 : GROUP_LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int grp = PAIR ? wave_id / kWaves : 0;                  // wave group (pair mode: 0 = A, 1 = B)
    const int wave = PAIR ? wave_id % kWaves : wave_id;           // row slice and load slice in the group
    uint8_t* const kbuf = lds + grp * GROUP_LDS;                  // K stages 0, 1
    uint8_t* const vbuf = kbuf + 2 * T::K_BYTES;                  // V stages 0, 1
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int g = Hq / Hkv;
    int bar_target = 0;
    bool sync_fail = false;             // a wave-group barrier of this wave ran out (its rows become NaN)
    if constexpr (PAIR) {
        if (tid < 16) reinterpret_cast<int*>(lds + 2 * GROUP_LDS)[tid] = 0;
        __syncthreads();
    }
    // barrier of the threads that share this workgroup's (or wave group's) K/V stages
    auto gsync = [&]() __attribute__((always_inline)) {
        if constexpr (PAIR) {
            sync_fail |= group_barrier(lds + 2 * GROUP_LDS + 16 * grp, bar_target, lane, sync_spins, &g_sync_timeouts);
        } else {
            __syncthreads();
        }
    };

    // ---- which (batch, head) and rank this workgroup owns ----
    int b, hq, kvh, rank;
    {
        const int w = blockIdx.x;
        if (xcd_groups) {
            // 8 XCDs receive workgroups round-robin; keep each K/V head on one XCD.
            const int xcd = w & 7, j = w >> 3;
            const int per_rank = xcd_groups * g;        // workgroups per q-block rank per XCD
            rank = j / per_rank;
            const int rem = j % per_rank;
            const int u = (rem / g) * 8 + xcd;          // K/V head unit = b * Hkv + kvh
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
        // second half of a grid that is resident all at once: reverse order
        if (mirror && rank >= (n_rank + 1) / 2) rank = n_rank - 1 - (rank - (n_rank + 1) / 2);
    }

    const int64_t q_off = ((int64_t)b * Hq + hq) * Sq * D;
    const int diag = Sk - Sq;           // key j visible to row i iff j <= i + diag
    f32x16 oacc[NDB];
    float m_run, l_run;                 // reference maximum of scale*log2(e)*s; this lane's share of the row sum

    // ---- epilogue of a query block: one division per row, bf16 output,
    // natural-log lse ----
    // Each wave's 32 x D output tile passes through its own slice of LDS (free
    // after the loop's last barrier), so that every global store instruction
    // writes whole consecutive rows (1 KiB) instead of 16-byte pieces of 32
    // rows.  16-byte chunks are XOR-swizzled by row for conflict-free LDS
    // writes and reads.
    auto write_out = [&](const int qb) __attribute__((always_inline)) {
        const int qw = qb * kBM + wave * 32;
        int ln = lane;
        if constexpr (PAIR) asm volatile("" : "+v"(ln));   // staging addresses formed here (see run_job)
        const int l32 = ln & 31, hh = ln >> 5;
        const int my_q = qw + l32;
        const float l_tot = half_swap_sum(l_run);
        const float inv = sync_fail ? __builtin_nanf("") : l_tot > 0.f ? 1.f / l_tot : 0.f;
        constexpr int CH = D / 8;                 // 16-byte chunks per row
        constexpr int RPP = 64 / CH;              // rows per wave-wide 16-byte pass
        uint8_t* const ot = kbuf + wave * 32 * T::ROWB;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int c = 4 * db + a;         // chunk of head-dim columns 32 db + 8 a .. +7
                const u32x2 w = {pack_bf16x2(oacc[db][4 * a + 0] * inv, oacc[db][4 * a + 1] * inv),
                                 pack_bf16x2(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv)};
                *reinterpret_cast<u32x2*>(ot + l32 * T::ROWB + 16 * (c ^ (l32 & (CH - 1))) + 8 * hh) = w;
            }
        gsync();
        // Whole rows go out with the non-temporal hint: nothing in this
        // kernel reads O back.  (Only for these full-line stores: partial
        // 8-byte pieces stored this way were far slower.)
        const int rr = ln / CH, cc = ln % CH;
#pragma unroll
        for (int r8 = 0; r8 < 32 / RPP; ++r8) {
            const int r = r8 * RPP + rr;
            const u32x4 v = *reinterpret_cast<const u32x4*>(ot + r * T::ROWB + 16 * (cc ^ (r & (CH - 1))));
            if (qw + r < Sq)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(O + q_off + (int64_t)(qw + r) * D + 8 * cc));
        }
        if (LSE != nullptr && hh == 0 && my_q < Sq)
            LSE[((int64_t)b * Hq + hq) * Sq + my_q] = sync_fail    ? __builtin_nanf("")
                                                      : l_tot > 0.f ? (m_run + log2f_hw(l_tot)) * kLn2
                                                                    : kNegInf;
    };

    // One job: query block qb against K/V blocks [kb0, kb1); with `final` the
    // output of the block is written, else the state stays in oacc/m_run/l_run.
    auto run_job = [&](const int qb, const int kb0, const int kb1, const bool final) __attribute__((always_inline)) {
    // (empty asm statements: the per-lane addresses are formed inside each job,
    // not kept live, and spilled, across the other job of a pair workgroup)
    int64_t kv_off = ((int64_t)b * Hkv + kvh) * Sk * D;
    int k_lane_off = dma_lane_offset<D, true>(wave, lane);
    int v_lane_off = dma_lane_offset<D, false>(wave, lane);
    if constexpr (PAIR) {
        asm volatile("" : "+s"(kv_off));
        asm volatile("" : "+v"(k_lane_off), "+v"(v_lane_off));
    }
    const uint16_t* Kh = K + kv_off;
    const uint16_t* Vh = V + kv_off;
    const int q0 = qb * kBM;
    const int qw = q0 + wave * 32;      // first query row of this wave
    const int my_q = qw + l32;          // the query row this lane's scores belong to
    const int n_it = kb1 - kb0;         // K/V blocks of this job

    // Q fragment, the B operand of S^T = K Q^T: 8 contiguous head-dim elements
    // per step.  Lanes past the last query row read row Sq - 1 instead; their
    // scores are never written out.  The values are not touched before the
    // first product, so the loads' latency overlaps that of the K/V loads
    // issued next (a select on them here would wait for them first).
    bf16x8 qf[NS];
    {
        const uint16_t* qp = Q + q_off + (int64_t)min(my_q, Sq - 1) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < NS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
    }

#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
    m_run = kNegInf;
    l_run = 0.f;

    // a block needs the elementwise mask if it runs past Sk or crosses this wave's diagonal
    auto needs_mask = [&](int kv0) { return (kv0 + kBN > Sk) || (CAUSAL && kv0 + kBN - 1 > qw + diag); };

    // ---- prologue: K_kb0, V_kb0, K_kb0+1 into LDS; scores of block kb0 ----
    if (n_it > 0) {
        dma_tile<D>(Kh, kbuf, k_lane_off, kb0 * kBN, Sk, wave);
        dma_tile<D>(Vh, vbuf, v_lane_off, kb0 * kBN, Sk, wave);
    }
    if (n_it > 1) dma_tile<D>(Kh, kbuf + T::K_BYTES, k_lane_off, (kb0 + 1) * kBN, Sk, wave);
    wait_dma();
    gsync();

    f32x16 s0[2] = {f32x16{}, f32x16{}};
    float mx_cur = kNegInf;
    if (n_it > 0) {
        score_block<D>(s0, kbuf, qf, l32, hh, [](int) {});
        if (needs_mask(kb0 * kBN)) mask_block<CAUSAL>(s0, kb0 * kBN, Sk, my_q, diag, hh);
        float mx = kNegInf;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s0[blk][r]);
        mx_cur = half_swap_max(mx) * scale_log2;
    }
    // K stage 0 is rewritten (with K_2) at the end of the first iteration:
    // every wave must have finished reading it above.
    gsync();

    // One K/V block: `scur` holds this block's scores, `snxt` receives the next
    // block's.  The loop is unrolled by two so the buffers swap roles instead
    // of being copied, and its last step is peeled (HAS_NEXT false), so a
    // step has no data-dependent branch inside its product sequence.  The four
    // LDS stages a step touches (K and V written by this step's loads to
    // LDS, K and V read as operands) are disjoint; passing them as restrict
    // pointers tells the compiler so.  Without that it must assume the
    // transposing V reads may see the loads just issued, and waits for all of
    // them before the first P V product, which leaves only the score phase to
    // hide their latency instead of the whole step.
    //
    // Empty asm statements that take a value as an in/out operand fix where
    // it is computed: without them the compiler gathers the scale
    // multiply-adds at the top of the step and the running-sum additions and
    // the next block's maximum after the last product, and those runs of
    // vector work then leave the matrix core idle.
    auto step = [&](auto has_next_c, const int it, f32x16 (&scur)[2], f32x16 (&snxt)[2],
                    uint8_t* __restrict__ k_dma, uint8_t* __restrict__ v_dma, const uint8_t* __restrict__ k_rd,
                    const uint8_t* __restrict__ v_rd) __attribute__((always_inline)) {
        constexpr bool HAS_NEXT = decltype(has_next_c)::value;
        const bool has_next2 = it + 2 < n_it;
        const int kb = kb0 + it;        // absolute K/V block of this step

        // ---- move the reference maximum only when a row outgrows it by 2^kTau ----
        // Otherwise p <= 2^kTau and the stale reference cancels in the final
        // division, so the result is the same exact quantity.
        if (__builtin_amdgcn_ballot_w64(mx_cur > m_run + kTau)) {
            const float m_new = fmaxf(m_run, mx_cur);
            const float alpha = exp2f_hw(m_run - (m_new == kNegInf ? 0.f : m_new));
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;
        }
        const float m_use = m_run == kNegInf ? 0.f : m_run;

        // K_{it+2} into the K stage freed by block it, V_{it+1} into the V stage
        // freed by block it-1; both land while this block is computed.
        if (HAS_NEXT) {
            if (has_next2) dma_tile<D>(Kh, k_dma, k_lane_off, (kb + 2) * kBN, Sk, wave);
            dma_tile<D>(Vh, v_dma, v_lane_off, (kb + 1) * kBN, Sk, wave);
        }

        // ---- phase X: scores of block it+1 on the matrix core, exponentials of
        // the first 32 keys of block it; phase Y: O^T += V_it^T P_it^T on the
        // matrix core, exponentials of the other 32 keys (each one key step
        // ahead of the product that takes them), then the maximum of block
        // it+1.  One unit of vector work follows every product, so the matrix
        // core and the vector unit overlap.
        float pv[32];           // p of block it: value v is scur[v / 16][v % 16]
        u32x4 pfw[4];           // P operand of key step ks: pfw[ks]
        float rs = 0.f;
        auto exp_unit = [&](int v) {
            const int blk = v >> 4, r = v & 15;
            float t = fmaf(scur[blk][r], scale_log2, -m_use);
            asm volatile("" : "+v"(t));
            pv[v] = exp2f_hw(t);
            // the running sum adds the fp32 values: rounding p to bf16 would
            // move a short row's lse by up to 2^-9
            rs += pv[v];
            asm volatile("" : "+v"(rs));
            if (v & 1) {
                uint32_t w = pack_bf16x2(pv[v - 1], pv[v]);
                asm volatile("" : "+v"(w));
                pfw[2 * blk + (r >> 3)][(r & 7) >> 1] = w;
            }
        };
        constexpr int XS = 2 * NS;          // products of phase X
        if constexpr (HAS_NEXT) {
            snxt[0] = f32x16{};
            snxt[1] = f32x16{};
            score_block<D>(snxt, k_rd, qf, l32, hh, [&](int k) {
#pragma unroll
                for (int v = k * 16 / XS; v < (k + 1) * 16 / XS; ++v) exp_unit(v);
            });
            if (needs_mask((kb + 1) * kBN)) mask_block<CAUSAL>(snxt, (kb + 1) * kBN, Sk, my_q, diag, hh);
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) exp_unit(v);
        }

        float mxn = kNegInf;
        {
            const uint8_t* vt = v_rd;
            // V^T operands in product order j = ks NDB + db, read three products ahead
            constexpr int NJ = 4 * NDB;
            bf16x8 vr[4];
            vr[0] = vt_operand<D>(vt, 0, 0, lane);
            vr[1] = vt_operand<D>(vt, 1 / NDB, 1 % NDB, lane);
            vr[2] = vt_operand<D>(vt, 2 / NDB, 2 % NDB, lane);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 pb = __builtin_bit_cast(bf16x8, pfw[ks]);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int j = ks * NDB + db;
                    if (j + 3 < NJ) vr[(j + 3) % 4] = vt_operand<D>(vt, (j + 3) / NDB, (j + 3) % NDB, lane);
                    FA_FENCE();
                    oacc[db] = mfma32(vr[j % 4], pb, oacc[db]);
                    FA_FENCE();
                    if (ks < 2) {
                        // p of keys 32 + 16 ks .. +15 (P operand of key step ks + 2)
#pragma unroll
                        for (int v = 16 + 8 * ks + db * 8 / NDB; v < 16 + 8 * ks + (db + 1) * 8 / NDB; ++v) exp_unit(v);
                    } else if constexpr (HAS_NEXT) {
                        const int blk = ks - 2;
#pragma unroll
                        for (int r = db * 16 / NDB; r < (db + 1) * 16 / NDB; ++r) mxn = fmaxf(mxn, snxt[blk][r]);
                        asm volatile("" : "+v"(mxn));
                    }
                    FA_FENCE();
                }
            }
        }
        l_run += rs;
        if constexpr (HAS_NEXT) mx_cur = half_swap_max(mxn) * scale_log2;

        wait_dma();
        gsync();
    };
    using Next = std::integral_constant<bool, true>;
    using Last = std::integral_constant<bool, false>;
    f32x16 s1[2];
    // even steps: K_{it+2} -> K stage 0, V_{it+1} -> V stage 1; read K stage 1, V stage 0
    // odd steps:  K_{it+2} -> K stage 1, V_{it+1} -> V stage 0; read K stage 0, V stage 1
    int it = 0;
    for (; it + 2 < n_it; it += 2) {
        step(Next{}, it, s0, s1, kbuf, vbuf + T::V_BYTES, kbuf + T::K_BYTES, vbuf);
        step(Next{}, it + 1, s1, s0, kbuf + T::K_BYTES, vbuf, kbuf, vbuf + T::V_BYTES);
    }
    if (it + 1 < n_it) {
        step(Next{}, it, s0, s1, kbuf, vbuf + T::V_BYTES, kbuf + T::K_BYTES, vbuf);
        step(Last{}, it + 1, s1, s0, kbuf + T::K_BYTES, vbuf, kbuf, vbuf + T::V_BYTES);
    } else if (it < n_it) {
        step(Last{}, it, s0, s1, kbuf, vbuf + T::V_BYTES, kbuf + T::K_BYTES, vbuf);
    }

    if (final) write_out(qb);
    };   // run_job

    if constexpr (PAIR) {
        // Pair workgroup p of (b, hq): heavy block i = n-1-p and light block p
        // (n query blocks; i == p for the middle block when n is odd, and for
        // every block of a split-only grid, whose workgroup r takes block
        // n-1-r alone and halves it between the groups).  Group A
        // takes K/V blocks [0, split) of block i; group B the whole of block p,
        // then [split, 2i + 2) of block i, and the two groups run
        // unsynchronised on their own LDS stages.  An even split gives each
        // group n + 1 blocks, but group B also pays a second job start and the
        // light block's output; `split_bias` blocks move from B to A to even
        // out the finishing times.
        const int i = n_qblk - 1 - rank, p = split_only ? i : rank;
        const int split = i != p ? min(n_qblk + 1 + split_bias, 2 * i + 2) : i + 1;
        if (grp == 0) {
            run_job(i, 0, split, false);
        } else {
            if (i != p) {
                run_job(p, 0, 2 * p + 2, true);
                gsync();                 // its output staging is read before the next job's loads reuse the LDS
            }
            if (split < 2 * i + 2) {
                run_job(i, split, 2 * i + 2, false);
            } else {                     // group A takes all of block i: B's share is empty
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
                m_run = kNegInf;
                l_run = 0.f;
            }
        }
        // ---- the halves of block i meet: the online-softmax update of two
        // partial states, M = max(m_A, m_B), acc = acc_A 2^(m_A - M) + acc_B
        // 2^(m_B - M), l likewise.  Group B's waves hold the same rows and
        // columns, lane for lane, as group A's. ----
        __syncthreads();                 // both groups done; every K/V stage is free
        float* const st = reinterpret_cast<float*>(lds + GROUP_LDS) + wave * (64 * 16 * NDB);
        float2* const sml = reinterpret_cast<float2*>(lds + GROUP_LDS / 4 * 3) + wave * 64;
        if (grp == 1) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
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
            for (int db = 0; db < NDB; ++db)
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
        if (CAUSAL) kv_end = min(Sk, max(0, qb * kBM + kBM + diag));
        run_job(qb, 0, (kv_end + kBN - 1) / kBN, true);
    }
}

int num_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 256;
    return n > 0 ? n : 256;
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    const int n_qblk = (a.Sq + kBM - 1) / kBM;
    const int units = a.B * a.Hkv;
    const int xcd_groups = (units % 8 == 0) ? units / 8 : 0;
    const float scale_log2 = a.scale * kLog2e;
    const int cus = num_cus();
    // Pair grid: a causal square problem whose query blocks, paired heavy with
    // light, fit one 8-wave workgroup per CU; every workgroup then walks the
    // same number of K/V blocks.  With half the CUs or fewer taken by pairs,
    // a pair walks more K/V blocks than the heaviest block alone, so each
    // block gets a workgroup of its own (all on CUs of their own): from 8
    // query blocks on split between the two wave groups and merged like a
    // pair's heavy block (split-only grid), below that as one 4-wave
    // workgroup, where the halves are too short to repay the merge.
    if constexpr (D == 128 && CAUSAL) {
        const int n_pairs = (n_qblk + 1) / 2;
        const int64_t n_pair_wg = (int64_t)a.B * a.Hq * n_pairs;
        const bool fills = 2 * n_pair_wg > cus;
        const int split_only = (!fills && n_qblk >= 8) ? 1 : 0;
        if (a.Sq == a.Sk && a.Sq % kBM == 0 && n_qblk >= 2 && n_pair_wg <= cus && (fills || split_only)) {
            const int64_t n_wg = split_only ? (int64_t)a.B * a.Hq * n_qblk : n_pair_wg;
            // K/V blocks moved from group B to group A: B pays fixed extra costs
            // (a second job start, the light block's output) and its steps run
            // slower than A's, so the best bias grows with n: 3, 4 and 6 blocks
            // for n = 8, 16 and 32 query blocks (one block fewer than A and B's
            // fixed costs alone suggest, since A's steps speed up once B is done).
            const int split_bias = 2 + n_qblk / 8;
            launch_kernel((fwd_bf16_kernel<D, CAUSAL, true>), dim3((unsigned)n_wg), dim3(2 * kThreads), 0, stream,
                          (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                          a.B, a.Hq, a.Hkv, a.Sq, a.Sk, scale_log2, n_qblk, split_only ? n_qblk : n_pairs, xcd_groups, 0,
                          split_bias, a.sync_spins, split_only);
            return hipGetLastError();
        }
    }
    const int64_t n_wg = (int64_t)a.B * a.Hq * n_qblk;
    // Two workgroups fit on a CU; if the whole grid is resident at once, pair
    // heavy and light causal Q blocks on the same CU.
    const int mirror = (CAUSAL && n_wg <= 2 * (int64_t)cus) ? 1 : 0;
    launch_kernel((fwd_bf16_kernel<D, CAUSAL, false>), dim3((unsigned)n_wg), dim3(kThreads), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                       a.lse, a.B, a.Hq, a.Hkv, a.Sq, a.Sk, scale_log2, n_qblk, n_qblk, xcd_groups, mirror, 0,
                       a.sync_spins, 0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

hipError_t read_sync_timeouts(unsigned int* count) {
    return read_device_counter(&HIP_SYMBOL(g_sync_timeouts), count);
}

int64_t fwd_bf16_grid(const FwdArgs& a) {
    return (int64_t)a.B * a.Hq * ((a.Sq + kBM - 1) / kBM);
}

}  // namespace fa
