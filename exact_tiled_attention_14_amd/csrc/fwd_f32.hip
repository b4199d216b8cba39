// Prefill attention forward on fp32 inputs and outputs (gfx950 vector ALUs).
//
// The exact-attention recurrence of the bf16 kernel, written for fp32 data
// and for latency: the fp32 path serves small problems, where the number of
// lanes at work matters more than arithmetic throughput.  Each query row is
// spread over the 16 lanes of a DPP row, lane t holding head-dim slice
// D/16 t .. D/16 (t + 1) of the query and of the unnormalised output, so a
// wave serves 4 rows and a workgroup of 4 waves 16 rows.  Keys are taken kKC
// at a time straight from global memory (the 16 lanes of a row read one key
// row together, coalesced); the score of a key is the lanes' partial dot
// products summed with a 4-step DPP reduction.  The block of kKC scores then
// updates the running state with the online softmax of "Hardware Co-Design" /
// "Week 13. GPUs and FlashAttention", Step 2 (multiply the running sum and
// output by 2^(m_old - m_new), divide once at the end).  A wave stops at the
// last key any of its rows can see (causal), keys past Sk and above the
// diagonal are masked, and a row with no visible key gets O = 0, lse = -inf.
// No LDS and no barriers: waves are independent.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kWavesF = 4;
constexpr int kRowsPerWave = 4;                    // one row per 16-lane DPP row
constexpr int kRowsF = kWavesF * kRowsPerWave;     // query rows per workgroup
constexpr int kKC = 8;                             // keys per step

// DP consecutive floats at p (16-byte aligned for DP >= 4).
template <int DP>
__device__ __forceinline__ void load_slice(float (&x)[DP], const float* p) {
    if constexpr (DP % 4 == 0) {
#pragma unroll
        for (int i = 0; i < DP; i += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(p + i);
            x[i] = v[0];
            x[i + 1] = v[1];
            x[i + 2] = v[2];
            x[i + 3] = v[3];
        }
    } else {
#pragma unroll
        for (int i = 0; i < DP; ++i) x[i] = p[i];
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kWavesF) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int Sq, int Sk,
    float scale_log2, int n_qblk) {
    constexpr int DP = D / 16;                     // head-dim elements per lane
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = lane & 15;                       // head-dim slice
    const int qb = blockIdx.x % n_qblk;
    const int bh = blockIdx.x / n_qblk;
    const int b = bh / Hq, hq = bh % Hq;
    const int kvh = hq / (Hq / Hkv);
    const int64_t q_off = ((int64_t)b * Hq + hq) * Sq * D;
    const int64_t kv_off = ((int64_t)b * Hkv + kvh) * Sk * D;
    const int q_wave = qb * kRowsF + wave * kRowsPerWave;
    const int my_q = q_wave + (lane >> 4);
    const int diag = Sk - Sq;

    float q[DP], acc[DP];
    load_slice<DP>(q, Q + q_off + (int64_t)min(my_q, Sq - 1) * D + t * DP);
#pragma unroll
    for (int i = 0; i < DP; ++i) acc[i] = 0.f;
    float m_run = kNegInf, l_run = 0.f;            // the same in the 16 lanes of a row

    int kv_end = Sk;
    if (CAUSAL) kv_end = min(Sk, max(0, q_wave + kRowsPerWave + diag));

    // K/V rows of keys kv0 .. kv0+kKC-1 (clamped to Sk-1; those past Sk are masked)
    auto load_chunk = [&](int kv0, float (&kr)[kKC][DP], float (&vr)[kKC][DP]) {
#pragma unroll
        for (int j = 0; j < kKC; ++j) {
            const int64_t row = kv_off + (int64_t)min(kv0 + j, Sk - 1) * D + t * DP;
            load_slice<DP>(kr[j], K + row);
            load_slice<DP>(vr[j], V + row);
        }
    };
    // Update the row state with keys kv0 .. kv0+kKC-1, whose rows are in kr/vr.
    auto chunk = [&](int kv0, const float (&kr)[kKC][DP], const float (&vr)[kKC][DP]) __attribute__((always_inline)) {
        float s[kKC];
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < kKC; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < DP; ++i) dot = fmaf(q[i], kr[j][i], dot);
            dot = row_sum16(dot);
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
        for (int i = 0; i < DP; ++i) acc[i] *= alpha;
#pragma unroll
        for (int j = 0; j < kKC; ++j) {
            const float p = exp2f_hw(s[j] - m_use);    // 0 for masked keys
            l_run += p;
            // a masked key may sit on a clamped row: p is exactly 0 and the
            // row holds finite data, so the product adds nothing
#pragma unroll
            for (int i = 0; i < DP; ++i) acc[i] = fmaf(p, vr[j][i], acc[i]);
        }
    };
    // two register buffers: the next chunk's loads are in flight while the
    // current one is computed
    float ka[kKC][DP], va[kKC][DP], kb[kKC][DP], vb[kKC][DP];
    if (kv_end > 0) load_chunk(0, ka, va);
    for (int kv0 = 0; kv0 < kv_end; kv0 += 2 * kKC) {
        if (kv0 + kKC < kv_end) load_chunk(kv0 + kKC, kb, vb);
        chunk(kv0, ka, va);
        if (kv0 + kKC < kv_end) {
            if (kv0 + 2 * kKC < kv_end) load_chunk(kv0 + 2 * kKC, ka, va);
            chunk(kv0 + kKC, kb, vb);
        }
    }

    if (my_q < Sq) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float* op = O + q_off + (int64_t)my_q * D + t * DP;
#pragma unroll
        for (int i = 0; i < DP; ++i) op[i] = acc[i] * inv;
        if (LSE != nullptr && t == 0)
            LSE[((int64_t)b * Hq + hq) * Sq + my_q] = l_run > 0.f ? (m_run + log2f_hw(l_run)) * kLn2 : kNegInf;
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    const int n_qblk = (a.Sq + kRowsF - 1) / kRowsF;
    const int64_t n_wg = (int64_t)a.B * a.Hq * n_qblk;
    launch_kernel((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)n_wg), dim3(64 * kWavesF), 0, stream,
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
