// Prefill attention forward, bf16 in / bf16 out, fp32 accumulation, gfx950.
//
// One workgroup owns one block of BM query rows of one (batch, query head) and
// walks the K/V blocks of its key/value head (the loop order of "FlashAttention
// scaling, multi-GPU training and weight quantization", section 1: outer loop
// over Q blocks spread across the grid, inner loop over K/V).  Per K/V block
// ("Fast Inference and Training at Scale", section 6.21, tiling):
//
//   1. K_j and V_j are staged into LDS (double buffered: the next block's
//      global loads are issued before the current block's arithmetic and
//      written to the other buffer after it, one barrier per block).
//   2. The scores of the block are formed on the matrix cores.  Each wave owns
//      32 query rows and computes the transposed block S^T = K_j Q^T, so that
//      every lane holds scores of a single query row: the row maximum and row
//      sum are then in-lane reductions plus one exchange between lane halves.
//   3. Online softmax ("Hardware Co-Design"; "Week 13. GPUs and
//      FlashAttention", Step 2): m_new = max(m, rowmax), the unnormalised
//      output and running sum are multiplied by 2^(m - m_new), p = 2^(s - m_new).
//      Scores are kept in the log2 domain (scale * log2 e folded into one
//      multiply-add before the exponential).  A row with no visible key so far
//      keeps m = -inf and contributes exactly zero (the -inf guard).
//   4. O^T += V_j^T P^T on the matrix cores; P is rounded to bf16 once.  V_j is
//      written to LDS transposed, with the key order inside each 16-key chunk
//      permuted to match the lanes' accumulator layout, so each lane reads its
//      A operand with one 16-byte LDS load.
//   5. After the last block the output is divided by the running sum once
//      (division postponed to the end, section 1 of the FlashAttention-2/3
//      page) and lse = (m + log2 l) ln 2 is written per row.
//
// Causal: the loop stops at the last K/V block any row of the Q block can see
// and the elementwise mask is applied only to blocks that straddle the
// diagonal ("Week 13", Step 2: blocks fully above the diagonal are skipped).
// Workgroups are ordered heaviest-first and, when the number of K/V heads
// allows it, so that each of the 8 XCDs (each with its own L2) serves a
// disjoint set of K/V heads.
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
struct Staged {
    u32x4 k[Tile<D>::KCHUNKS];
    u32x4 v[4];
};

template <int D>
__device__ __forceinline__ void load_kv(Staged<D>& st, const uint16_t* __restrict__ Kh,
                                        const uint16_t* __restrict__ Vh, int kv0, int Sk, int tid) {
#pragma unroll
    for (int c = 0; c < Tile<D>::KCHUNKS; ++c) {
        const int idx = c * kThreads + tid;
        const int row = idx / (D / 8), col = idx % (D / 8);
        const int key = kv0 + row;
        // the address is clamped to a valid row; rows past Sk are replaced by zeros
        const u32x4 val = *reinterpret_cast<const u32x4*>(Kh + (int64_t)min(key, Sk - 1) * D + col * 8);
        st.k[c] = key < Sk ? val : u32x4{0, 0, 0, 0};
    }
    if (tid < Tile<D>::VGROUPS) {
        // Key group fastest across lanes: the transposed LDS write of one
        // instruction then fills whole V^T rows (no bank conflicts), at the
        // price of 64-byte rather than 256-byte contiguous global segments.
        const int kg = tid % (kBN / 4), cg = tid / (kBN / 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kv0 + 4 * kg + i;
            const u32x4 val = *reinterpret_cast<const u32x4*>(Vh + (int64_t)min(key, Sk - 1) * D + cg * 8);
            st.v[i] = key < Sk ? val : u32x4{0, 0, 0, 0};
        }
    }
}

template <int D>
__device__ __forceinline__ void store_kv(const Staged<D>& st, uint16_t* stage, int tid) {
    uint16_t* kt = stage;
    uint16_t* vt = stage + Tile<D>::K_ELEMS;
#pragma unroll
    for (int c = 0; c < Tile<D>::KCHUNKS; ++c) {
        const int idx = c * kThreads + tid;
        const int row = idx / (D / 8), col = idx % (D / 8);
        *reinterpret_cast<u32x4*>(kt + row * Tile<D>::KSTR + col * 8) = st.k[c];
    }
    if (tid < Tile<D>::VGROUPS) {
        const int kg = tid % (kBN / 4), cg = tid / (kBN / 4);
        uint16_t* dst = vt + (cg * 8) * Tile<D>::VSTR + vt_slot(kg);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int w = c >> 1;
            const int sh = (c & 1) * 16;
            const uint32_t e0 = (st.v[0][w] >> sh) & 0xffffu;
            const uint32_t e1 = (st.v[1][w] >> sh) & 0xffffu;
            const uint32_t e2 = (st.v[2][w] >> sh) & 0xffffu;
            const uint32_t e3 = (st.v[3][w] >> sh) & 0xffffu;
            *reinterpret_cast<u32x2*>(dst + c * Tile<D>::VSTR) = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
        }
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int Sq, int Sk,
    float scale_log2, int n_qblk, int xcd_groups) {
    using T = Tile<D>;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * T::STAGE];

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
        if (xcd_groups) {
            // 8 XCDs receive workgroups round-robin; keep each K/V head on one XCD.
            const int xcd = w & 7, j = w >> 3;
            const int per_rank = xcd_groups * g;        // workgroups per q-block rank per XCD
            const int rank = j / per_rank, rem = j % per_rank;
            const int u = (rem / g) * 8 + xcd;          // K/V head unit = b * Hkv + kvh
            b = u / Hkv;
            kvh = u % Hkv;
            hq = kvh * g + rem % g;
            qb = CAUSAL ? n_qblk - 1 - rank : rank;
        } else {
            const int bh = B * Hq;
            const int rank = w / bh, rem = w % bh;
            b = rem / Hq;
            hq = rem % Hq;
            kvh = hq / g;
            qb = CAUSAL ? n_qblk - 1 - rank : rank;
        }
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
    bf16x8 qf[D / 16];
    {
        const uint16_t* qp = Q + q_off + (int64_t)min(my_q, Sq - 1) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const bf16x8 val = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
            qf[s] = my_q < Sq ? val : bf16x8{};
        }
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    float m_run = kNegInf;   // running max of scale*log2(e)*s
    float l_run = 0.f;       // running sum of this lane's share of the row

    Staged<D> st;
    if (n_it > 0) {
        load_kv<D>(st, Kh, Vh, 0, Sk, tid);
        store_kv<D>(st, lds, tid);
    }
    __syncthreads();

    for (int it = 0; it < n_it; ++it) {
        const int kv0 = it * kBN;
        const uint16_t* kt = lds + (it & 1) * T::STAGE;
        const uint16_t* vt = kt + T::K_ELEMS;
        const bool more = it + 1 < n_it;
        if (more) load_kv<D>(st, Kh, Vh, kv0 + kBN, Sk, tid);

        // ---- S^T = K_j Q^T: two 32-key blocks, their chains interleaved ----
        // LDS operand reads run two steps ahead of the matrix-core ops that
        // use them; the scheduling fences keep the compiler from sinking
        // each read next to its use.
        f32x16 sacc[2] = {f32x16{}, f32x16{}};
        {
            const uint16_t* kr0 = kt + l32 * T::KSTR + 8 * hh;
            const uint16_t* kr1 = kr0 + 32 * T::KSTR;
            constexpr int NS = D / 16;
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
                __builtin_amdgcn_sched_barrier(0);
                sacc[0] = mfma32(ka[s % 3][0], qf[s], sacc[0]);
                sacc[1] = mfma32(ka[s % 3][1], qf[s], sacc[1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- mask: ragged tail and (causal) blocks that straddle the diagonal ----
        const bool need_mask = (kv0 + kBN > Sk) || (CAUSAL && kv0 + kBN - 1 > qw + diag);
        if (need_mask) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + 32 * blk + acc_row(r, hh);
                    const bool ok = key < Sk && (!CAUSAL || key <= my_q + diag);
                    sacc[blk][r] = ok ? sacc[blk][r] : kNegInf;
                }
        }

        // ---- online softmax on this lane's query row ----
        // The reference maximum m_run is raised (and the running sum and
        // output rescaled by 2^(m_run - m_new)) only when some row's block
        // maximum exceeds it by more than 2^kTau; otherwise p <= 2^kTau and
        // the stale reference cancels in the final division, so the result is
        // the same exact quantity with far fewer rescales.
        float mx = kNegInf;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[blk][r]);
        mx = half_swap_max(mx) * scale_log2;
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kTau)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = exp2f_hw(m_run - (m_new == kNegInf ? 0.f : m_new));
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
        }
        const float m_use = m_run == kNegInf ? 0.f : m_run;

        bf16x8 pf[4];
        float rs = 0.f;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = exp2f_hw(fmaf(sacc[blk][r], scale_log2, -m_use));
                rs += p;
                pf[2 * blk + (r >> 3)][r & 7] = (__bf16)p;
            }
        l_run += rs;

        // ---- O^T += V_j^T P^T: d-block chains interleaved, reads one step ahead ----
        {
            constexpr int NDB = D / 32;
            const uint16_t* vr = vt + l32 * T::VSTR + 8 * hh;
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
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(va[ks & 1][db], pf[ks], oacc[db]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        if (more) store_kv<D>(st, lds + ((it + 1) & 1) * T::STAGE, tid);
        __syncthreads();
    }

    // ---- epilogue: one division per row, bf16 output, natural-log lse ----
    const float l_tot = half_swap_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (my_q < Sq) {
        uint16_t* op = O + q_off + (int64_t)my_q * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
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

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    const int n_qblk = (a.Sq + kBM - 1) / kBM;
    const int64_t n_wg = (int64_t)a.B * a.Hq * n_qblk;
    const int units = a.B * a.Hkv;
    const int xcd_groups = (units % 8 == 0) ? units / 8 : 0;
    const float scale_log2 = a.scale * kLog2e;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)n_wg), dim3(kThreads), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                       a.lse, a.B, a.Hq, a.Hkv, a.Sq, a.Sk, scale_log2, n_qblk, xcd_groups);
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
