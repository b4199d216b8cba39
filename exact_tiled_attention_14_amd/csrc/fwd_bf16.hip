// Prefill attention forward, bf16 in / bf16 out, fp32 accumulation, gfx950.
//
// One workgroup owns one block of 128 query rows of one (batch, query head)
// and walks the K/V blocks of its key/value head (the loop order of
// "FlashAttention scaling, multi-GPU training and weight quantization",
// section 1: outer loop over Q blocks spread across the grid, inner loop over
// K/V).  Per K/V block ("Fast Inference and Training at Scale", section 6.21,
// tiling):
//
//   1. K_j and V_j are staged into LDS by the waves themselves: K one block
//      ahead of V, each in its own double buffer, global loads issued a block
//      before the LDS write, one barrier per block.
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
//   4. O^T += V_j^T P^T on the matrix cores; P is rounded to bf16 once.  V_j is
//      written to LDS transposed, in the key order that the lanes hold P in,
//      so each A operand is one 16-byte LDS read.
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
    static constexpr int KSTR = D + 8;            // K row stride in LDS (bf16), 16 B pad
    static constexpr int VSTR = kBN + 8;          // V^T row stride in LDS (bf16)
    static constexpr int K_ELEMS = kBN * KSTR;
    static constexpr int V_ELEMS = D * VSTR;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int KCHUNKS = kBN * D / 8 / kThreads;   // 16-byte K loads per thread
    static constexpr int VGROUPS = (kBN / 4) * (D / 8);       // 4-key x 8-column V groups
    static_assert(KCHUNKS >= 1 && (kBN * D / 8) % kThreads == 0, "K tile split");
    static_assert(VGROUPS <= kThreads, "one V group per thread at most");
};

// Slot of the first of 4 consecutive keys (4g .. 4g+3) inside the V^T tile.
// Within a 16-key chunk the key 8a + 4h + b sits at slot 8h + 4a + b, which is
// the order in which lane half h holds the probabilities of that chunk.
__device__ __forceinline__ int vt_slot(int g) {
    const int w = g & 3;
    return 16 * (g >> 2) + 4 * (((w & 1) << 1) | (w >> 1));
}

template <int D>
struct KStage {
    u32x4 k[Tile<D>::KCHUNKS];
};
struct VStage {
    u32x4 v[4];
};

template <int D>
__device__ __forceinline__ void load_k(KStage<D>& st, const uint16_t* __restrict__ Kh, int kv0, int Sk, int tid) {
#pragma unroll
    for (int c = 0; c < Tile<D>::KCHUNKS; ++c) {
        const int idx = c * kThreads + tid;
        const int row = idx / (D / 8), col = idx % (D / 8);
        // The address is clamped to a valid row; rows past Sk are zeroed when
        // stored, so nothing waits for the load before the LDS write.
        st.k[c] = *reinterpret_cast<const u32x4*>(Kh + (int64_t)min(kv0 + row, Sk - 1) * D + col * 8);
    }
}

template <int D>
__device__ __forceinline__ void store_k(const KStage<D>& st, uint16_t* kt, int kv0, int Sk, int tid) {
#pragma unroll
    for (int c = 0; c < Tile<D>::KCHUNKS; ++c) {
        const int idx = c * kThreads + tid;
        const int row = idx / (D / 8), col = idx % (D / 8);
        *reinterpret_cast<u32x4*>(kt + row * Tile<D>::KSTR + col * 8) =
            kv0 + row < Sk ? st.k[c] : u32x4{0, 0, 0, 0};
    }
}

// V staging: each thread owns 4 consecutive keys x 8 head-dim columns.  The
// key group is the fastest-varying lane index, so the transposed LDS write of
// one instruction fills whole V^T rows (no bank conflicts), at the price of
// 64-byte rather than 256-byte contiguous global segments.
template <int D>
__device__ __forceinline__ void load_v(VStage& st, const uint16_t* __restrict__ Vh, int kv0, int Sk, int tid) {
    if (tid < Tile<D>::VGROUPS) {
        const int kg = tid % (kBN / 4), cg = tid / (kBN / 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            st.v[i] = *reinterpret_cast<const u32x4*>(Vh + (int64_t)min(kv0 + 4 * kg + i, Sk - 1) * D + cg * 8);
        }
    }
}

template <int D>
__device__ __forceinline__ void store_v(const VStage& st, uint16_t* vt, int kv0, int Sk, int tid) {
    if (tid < Tile<D>::VGROUPS) {
        const int kg = tid % (kBN / 4), cg = tid / (kBN / 4);
        uint16_t* dst = vt + (cg * 8) * Tile<D>::VSTR + vt_slot(kg);
        const int key0 = kv0 + 4 * kg;
        u32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = key0 + i < Sk ? st.v[i] : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int w = c >> 1;
            const int sh = (c & 1) * 16;
            const uint32_t e0 = (v[0][w] >> sh) & 0xffffu;
            const uint32_t e1 = (v[1][w] >> sh) & 0xffffu;
            const uint32_t e2 = (v[2][w] >> sh) & 0xffffu;
            const uint32_t e3 = (v[3][w] >> sh) & 0xffffu;
            *reinterpret_cast<u32x2*>(dst + c * Tile<D>::VSTR) = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
        }
    }
}

#define FA_FENCE() __builtin_amdgcn_sched_barrier(0)

// Scores of one 64-key block for this wave's 32 rows: S^T = K Q^T, the two
// 32-key halves as interleaved MFMA chains, LDS operand reads two steps ahead.
// After MFMA step s the callback `between(s)` is emitted, so independent
// vector work can be interleaved with the matrix-core work.
template <int D, typename F>
__device__ __forceinline__ void score_block(f32x16 (&sacc)[2], const uint16_t* kt, const bf16x8 (&qf)[D / 16],
                                            int l32, int hh, F&& between) {
    constexpr int NS = D / 16;
    const uint16_t* kr0 = kt + l32 * Tile<D>::KSTR + 8 * hh;
    const uint16_t* kr1 = kr0 + 32 * Tile<D>::KSTR;
    bf16x8 ka[3][2];
    ka[0][0] = *reinterpret_cast<const bf16x8*>(kr0);
    ka[0][1] = *reinterpret_cast<const bf16x8*>(kr1);
    ka[1][0] = *reinterpret_cast<const bf16x8*>(kr0 + 16);
    ka[1][1] = *reinterpret_cast<const bf16x8*>(kr1 + 16);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (s + 2 < NS) {
            ka[(s + 2) % 3][0] = *reinterpret_cast<const bf16x8*>(kr0 + 16 * (s + 2));
            ka[(s + 2) % 3][1] = *reinterpret_cast<const bf16x8*>(kr1 + 16 * (s + 2));
        }
        FA_FENCE();
        sacc[0] = mfma32(ka[s % 3][0], qf[s], sacc[0]);
        sacc[1] = mfma32(ka[s % 3][1], qf[s], sacc[1]);
        FA_FENCE();
        between(s);
        FA_FENCE();
    }
}

// Mask the scores of block kv0 .. kv0+63: keys past Sk, and keys above the
// causal diagonal of this lane's row.
template <bool CAUSAL>
__device__ __forceinline__ void mask_block(f32x16 (&sacc)[2], int kv0, int Sk, int my_q, int diag, int hh) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * blk + acc_row(r, hh);
            const bool ok = key < Sk && (!CAUSAL || key <= my_q + diag);
            sacc[blk][r] = ok ? sacc[blk][r] : kNegInf;
        }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int Sq, int Sk,
    float scale_log2, int n_qblk, int xcd_groups, int mirror) {
    using T = Tile<D>;
    constexpr int NS = D / 16;          // MFMA steps of one score block
    constexpr int NDB = D / 32;         // 32-wide head-dim blocks of the output
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * T::K_ELEMS + 2 * T::V_ELEMS];
    uint16_t* const kbuf = lds;                     // K stages 0, 1
    uint16_t* const vbuf = lds + 2 * T::K_ELEMS;    // V^T stages 0, 1

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int g = Hq / Hkv;

    // ---- which (batch, head, query block) this workgroup owns ----
    int b, hq, kvh, qb;
    {
        const int w = blockIdx.x;
        int rank;
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
        if (mirror && rank >= (n_qblk + 1) / 2) rank = n_qblk - 1 - (rank - (n_qblk + 1) / 2);
        qb = CAUSAL ? n_qblk - 1 - rank : rank;
    }

    const int64_t q_off = ((int64_t)b * Hq + hq) * Sq * D;
    const int64_t kv_off = ((int64_t)b * Hkv + kvh) * Sk * D;
    const uint16_t* Kh = K + kv_off;
    const uint16_t* Vh = V + kv_off;
    const int q0 = qb * kBM;
    const int qw = q0 + wave * 32;      // first query row of this wave
    const int my_q = qw + l32;          // the query row this lane's scores belong to
    const int diag = Sk - Sq;           // key j visible to row i iff j <= i + diag

    int kv_end = Sk;
    if (CAUSAL) kv_end = min(Sk, max(0, q0 + kBM + diag));
    const int n_it = (kv_end + kBN - 1) / kBN;

    // Q fragment, the B operand of S^T = K Q^T: 8 contiguous head-dim elements per step.
    bf16x8 qf[NS];
    {
        const uint16_t* qp = Q + q_off + (int64_t)min(my_q, Sq - 1) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const bf16x8 val = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
            qf[s] = my_q < Sq ? val : bf16x8{};
        }
    }

    f32x16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
    float m_run = kNegInf;   // reference maximum of scale*log2(e)*s for this row
    float l_run = 0.f;       // running sum of this lane's share of the row

    // a block needs the elementwise mask if it runs past Sk or crosses this wave's diagonal
    auto needs_mask = [&](int kv0) { return (kv0 + kBN > Sk) || (CAUSAL && kv0 + kBN - 1 > qw + diag); };

    // ---- prologue: K_0, V_0, K_1 into LDS; scores of block 0 ----
    KStage<D> kst;
    VStage vst;
    if (n_it > 0) {
        load_k<D>(kst, Kh, 0, Sk, tid);
        load_v<D>(vst, Vh, 0, Sk, tid);
        store_k<D>(kst, kbuf, 0, Sk, tid);
        store_v<D>(vst, vbuf, 0, Sk, tid);
    }
    if (n_it > 1) {
        load_k<D>(kst, Kh, kBN, Sk, tid);
        store_k<D>(kst, kbuf + T::K_ELEMS, kBN, Sk, tid);
    }
    __syncthreads();

    f32x16 scur[2] = {f32x16{}, f32x16{}};
    float mx_cur = kNegInf;
    if (n_it > 0) {
        score_block<D>(scur, kbuf, qf, l32, hh, [](int) {});
        if (needs_mask(0)) mask_block<CAUSAL>(scur, 0, Sk, my_q, diag, hh);
        float mx = kNegInf;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, scur[blk][r]);
        mx_cur = half_swap_max(mx) * scale_log2;
    }
    // K stage 0 is rewritten (with K_2) at the end of the first iteration:
    // every wave must have finished reading it above.
    __syncthreads();

    for (int it = 0; it < n_it; ++it) {
        const bool has_next = it + 1 < n_it;
        const bool has_next2 = it + 2 < n_it;

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

        if (has_next2) load_k<D>(kst, Kh, (it + 2) * kBN, Sk, tid);
        if (has_next) load_v<D>(vst, Vh, (it + 1) * kBN, Sk, tid);

        // ---- phase X: scores of block it+1 on the matrix core, exponentials of block it ----
        u32x4 pfw[4];
        float rs = 0.f;
        auto exp_chunk = [&](int c) {    // 4 scores: block c/4, registers 4(c%4) .. +3
            const int blk = c >> 2, r0 = 4 * (c & 3);
            const float p0 = exp2f_hw(fmaf(scur[blk][r0 + 0], scale_log2, -m_use));
            const float p1 = exp2f_hw(fmaf(scur[blk][r0 + 1], scale_log2, -m_use));
            const float p2 = exp2f_hw(fmaf(scur[blk][r0 + 2], scale_log2, -m_use));
            const float p3 = exp2f_hw(fmaf(scur[blk][r0 + 3], scale_log2, -m_use));
            // the running sum adds the fp32 values: rounding p to bf16 would
            // move a short row's lse by up to 2^-9
            rs += (p0 + p1) + (p2 + p3);
            const uint32_t w01 = pack_bf16x2(p0, p1), w23 = pack_bf16x2(p2, p3);
            const int pk = 2 * blk + (r0 >> 3), pw = (r0 & 7) >> 1;
            pfw[pk][pw] = w01;
            pfw[pk][pw + 1] = w23;
        };
        f32x16 snxt[2] = {f32x16{}, f32x16{}};
        if (has_next) {
            score_block<D>(snxt, kbuf + ((it + 1) & 1) * T::K_ELEMS, qf, l32, hh, [&](int s) {
#pragma unroll
                for (int c = s * (8 / NS); c < (s + 1) * (8 / NS); ++c) exp_chunk(c);
            });
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) exp_chunk(c);
        }
        l_run += rs;

        // ---- phase Y: O^T += V_it^T P_it^T on the matrix core, maximum of block it+1 ----
        if (has_next && needs_mask((it + 1) * kBN)) mask_block<CAUSAL>(snxt, (it + 1) * kBN, Sk, my_q, diag, hh);
        float mxn = kNegInf;
        {
            const uint16_t* vr = vbuf + (it & 1) * T::V_ELEMS + l32 * T::VSTR + 8 * hh;
            bf16x8 va[2][NDB];
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                va[0][db] = *reinterpret_cast<const bf16x8*>(vr + 32 * db * T::VSTR);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (ks + 1 < 4) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        va[(ks + 1) & 1][db] = *reinterpret_cast<const bf16x8*>(vr + 32 * db * T::VSTR + 16 * (ks + 1));
                }
                FA_FENCE();
                const bf16x8 pb = __builtin_bit_cast(bf16x8, pfw[ks]);
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(va[ks & 1][db], pb, oacc[db]);
                FA_FENCE();
                if (has_next) {
                    const int blk = ks >> 1, r0 = 8 * (ks & 1);
#pragma unroll
                    for (int r = r0; r < r0 + 8; ++r) mxn = fmaxf(mxn, snxt[blk][r]);
                }
                FA_FENCE();
            }
        }
        if (has_next) mx_cur = half_swap_max(mxn) * scale_log2;

        if (has_next2) store_k<D>(kst, kbuf + (it & 1) * T::K_ELEMS, (it + 2) * kBN, Sk, tid);
        if (has_next) store_v<D>(vst, vbuf + ((it + 1) & 1) * T::V_ELEMS, (it + 1) * kBN, Sk, tid);
        __syncthreads();
        scur[0] = snxt[0];
        scur[1] = snxt[1];
    }

    // ---- epilogue: one division per row, bf16 output, natural-log lse ----
    const float l_tot = half_swap_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (my_q < Sq) {
        uint16_t* op = O + q_off + (int64_t)my_q * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int d0 = 32 * db + 8 * a + 4 * hh;
                const u32x2 w = {pack_bf16x2(oacc[db][4 * a + 0] * inv, oacc[db][4 * a + 1] * inv),
                                 pack_bf16x2(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv)};
                *reinterpret_cast<u32x2*>(op + d0) = w;
            }
        if (LSE != nullptr && hh == 0)
            LSE[((int64_t)b * Hq + hq) * Sq + my_q] = l_tot > 0.f ? (m_run + log2f_hw(l_tot)) * kLn2 : kNegInf;
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
    const int64_t n_wg = (int64_t)a.B * a.Hq * n_qblk;
    const int units = a.B * a.Hkv;
    const int xcd_groups = (units % 8 == 0) ? units / 8 : 0;
    const float scale_log2 = a.scale * kLog2e;
    // Two workgroups fit on a CU; if the whole grid is resident at once, pair
    // heavy and light causal Q blocks on the same CU.
    const int mirror = (CAUSAL && n_wg <= 2 * (int64_t)num_cus()) ? 1 : 0;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)n_wg), dim3(kThreads), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                       a.lse, a.B, a.Hq, a.Hkv, a.Sq, a.Sk, scale_log2, n_qblk, xcd_groups, mirror);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
    if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
}

int64_t fwd_bf16_grid(const FwdArgs& a) {
    return (int64_t)a.B * a.Hq * ((a.Sq + kBM - 1) / kBM);
}

}  // namespace fa
