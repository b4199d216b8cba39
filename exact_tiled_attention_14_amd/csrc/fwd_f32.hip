// Prefill attention forward on fp32 inputs and outputs (gfx950 vector ALUs).
//
// The same tiled algorithm as the bf16 kernel, written for fp32 data: one
// workgroup (one wave) owns 64 query rows, one lane per row, holding its query
// and unnormalised output in registers.  K/V blocks of kBN keys are staged in
// LDS (every lane reads the same key row, an LDS broadcast), the block's
// scores are reduced to a block maximum, and the running state is updated with
// the online softmax of "Hardware Co-Design" / "Week 13. GPUs and
// FlashAttention", Step 2 (multiply the running sum and output by
// 2^(m_old - m_new); divide once at the end).  Causal blocks fully above the
// diagonal are skipped and a row with no visible key gets O = 0, lse = -inf.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kRows = 64;   // query rows per workgroup (one wave, one row per lane)

// Keys per inner step: the block's scores live in registers next to the
// query row and the output row, so larger head dims take smaller blocks.
template <int D>
constexpr int block_n() { return D >= 128 ? 16 : 32; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Sq, int Sk,
    float scale_log2, int n_qblk) {
    constexpr int kBN = block_n<D>();
    __shared__ float ks[kBN][D];
    __shared__ float vs[kBN][D];

    const int lane = threadIdx.x;
    const int qb = blockIdx.x % n_qblk;
    const int bh = blockIdx.x / n_qblk;
    const int b = bh / Hq, hq = bh % Hq;
    const int kvh = hq / (Hq / Hkv);
    const int64_t q_off = ((int64_t)b * Hq + hq) * Sq * D;
    const int64_t kv_off = ((int64_t)b * Hkv + kvh) * Sk * D;
    const int q0 = qb * kRows;
    const int my_q = q0 + lane;
    const int diag = Sk - Sq;

    float q[D], acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        const float val = Q[q_off + (int64_t)min(my_q, Sq - 1) * D + c];
        q[c] = my_q < Sq ? val : 0.f;
        acc[c] = 0.f;
    }
    float m_run = kNegInf, l_run = 0.f;

    int kv_end = Sk;
    if (CAUSAL) kv_end = min(Sk, max(0, q0 + kRows + diag));

    for (int kv0 = 0; kv0 < kv_end; kv0 += kBN) {
        __syncthreads();
        for (int i = lane; i < kBN * D; i += kRows) {
            const int r = i / D, c = i % D;
            const int key = kv0 + r;
            const int64_t at = kv_off + (int64_t)min(key, Sk - 1) * D + c;
            const float kval = K[at], vval = V[at];
            ks[r][c] = key < Sk ? kval : 0.f;
            vs[r][c] = key < Sk ? vval : 0.f;
        }
        __syncthreads();

        float s[kBN];
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < kBN; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) dot = fmaf(q[c], ks[j][c], dot);
            const int key = kv0 + j;
            const bool ok = key < Sk && (!CAUSAL || key <= my_q + diag);
            s[j] = ok ? dot * scale_log2 : kNegInf;
            mx = fmaxf(mx, s[j]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = exp2f_hw(m_run - m_use);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] *= alpha;
#pragma unroll
        for (int j = 0; j < kBN; ++j) {
            const float p = exp2f_hw(s[j] - m_use);
            l_run += p;
#pragma unroll
            for (int c = 0; c < D; ++c) acc[c] = fmaf(p, vs[j][c], acc[c]);
        }
    }

    if (my_q < Sq) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float* op = O + q_off + (int64_t)my_q * D;
#pragma unroll
        for (int c = 0; c < D; ++c) op[c] = acc[c] * inv;
        if (LSE != nullptr)
            LSE[((int64_t)b * Hq + hq) * Sq + my_q] = l_run > 0.f ? (m_run + log2f_hw(l_run)) * kLn2 : kNegInf;
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    const int n_qblk = (a.Sq + kRows - 1) / kRows;
    const int64_t n_wg = (int64_t)a.B * a.Hq * n_qblk;
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)n_wg), dim3(kRows), 0, stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                       a.Hq, a.Hkv, a.Sq, a.Sk, a.scale * kLog2e, n_qblk);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
    return a.causal ? launch<D, true>(a, stream) : launch<D, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
    switch (a.d) {
        case 32: return launch_d<32>(a, stream);
        case 64: return launch_d<64>(a, stream);
        default: return launch_d<128>(a, stream);
    }
}

}  // namespace fa
