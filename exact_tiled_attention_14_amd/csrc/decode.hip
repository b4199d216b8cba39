// Paged KV-cache decode: one new query token per sequence (gfx950).
//
// Single-token decode reads every cached K and V once and does about
// Hq/Hkv FLOP per byte ("Week 13. GPUs and FlashAttention", Step 1), so it is
// bound by HBM bandwidth.  The design therefore aims at many bytes in flight
// and at reading each page exactly once:
//
//   * Grid = (range, K/V head, sequence).  Each sequence's cache is cut into
//     ranges of `pages_per_split` pages ("split-KV"); a workgroup attends the
//     G = Hq/Hkv query heads that share its K/V head ("Fast Inference and
//     Training at Scale", section 6.2) to one range, so a page is loaded once
//     for all G heads.
//   * Pages are found through the block table (section 6.3 PagedAttention).
//     A 16-token page of one head is 4 KiB of K and 4 KiB of V, contiguous;
//     a wave loads a whole page with 16-byte coalesced loads: lane l takes
//     head-dim slice 8 (l % 16) .. +8 of tokens l/16, l/16 + 4, +8, +12.
//   * Scores: packed bf16 dot products over the lane's slice, then a DPP sum
//     across the 16 lanes that share a token.
//   * Online softmax ("Hardware Co-Design") per lane row over the pages the
//     row visits; rows, then waves, are merged with the same update applied
//     to whole partial states, and the range's normalised partial output and
//     log-sum-exp go to the workspace.
//   * A second kernel merges the ranges of each (sequence, query head):
//     M = max lse_s, o = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M),
//     lse = M + ln sum_s e^(lse_s - M).
//
// Device values are made safe here: lengths are clamped to the table's
// capacity, block ids outside [0, num_blocks) contribute no key, and slots of
// a partly filled last page are masked with selects (never multiplied), so a
// NaN left in them cannot reach the output.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kD = 128;
constexpr int kPage = 16;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kTau = 8.f;   // log2 of the growth allowed before a rescale

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);   // row_half_mirror
    x += dpp<0x140>(x);   // row_mirror
    return x;
}

__device__ __forceinline__ float dot8_bf16(const u32x4& a, const u32x4& b) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        // Copy the element out first: a bit cast taken straight from a vector
        // element expression reads element 0 whatever the index.
        const uint32_t aw = a[w], bw = b[w];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aw), __builtin_bit_cast(bf16x2, bw), acc, false);
    }
    return acc;
}

template <int G>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(
    const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ KC, const uint16_t* __restrict__ VC,
    const int32_t* __restrict__ table, const int32_t* __restrict__ seqlens, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, int Hq, int Hkv, int max_blocks, int num_blocks, int pages_per_split,
    int n_split, float scale_log2) {
    __shared__ float sm_acc[kWaves][G][kD];
    __shared__ float sm_m[kWaves][G];
    __shared__ float sm_l[kWaves][G];

    const int split = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
    const int len = min(max(seqlens[seq], 0), max_blocks * kPage);
    const int n_pages = (len + kPage - 1) / kPage;
    const int page0 = split * pages_per_split;
    if (page0 >= n_pages) return;                 // whole workgroup: nothing in this range
    const int page1 = min(page0 + pages_per_split, n_pages);

    const int tid = threadIdx.x;
    // The wave index is made scalar so block-table reads are scalar loads:
    // waiting for one then does not also wait for the vector loads of the
    // page in flight.
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row = lane >> 4;                    // token slot: tokens row, row+4, row+8, row+12
    const int col = lane & 15;                    // head-dim slice 8*col .. 8*col+7
    const int hq0 = kvh * G;

    u32x4 qv[G];
#pragma unroll
    for (int h = 0; h < G; ++h)
        qv[h] = *reinterpret_cast<const u32x4*>(Qg + ((int64_t)seq * Hq + hq0 + h) * kD + 8 * col);

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kNegInf;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }

    const int32_t* trow = table + (int64_t)seq * max_blocks;
    // K and V of one page for this lane: tokens row + 4i (i = 0..3), head-dim
    // slice 8 col .. +7.  The next page of the wave is loaded while the
    // current one is computed.
    auto load_page = [&](int p, u32x4 (&kk)[4], u32x4 (&vv)[4]) {
        const int bid = trow[p];
        const bool blk_ok = bid >= 0 && bid < num_blocks;
        const int64_t base = ((int64_t)(blk_ok ? bid : 0) * Hkv + kvh) * (kPage * kD) + 8 * col;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t off = base + (int64_t)(row + 4 * i) * kD;
            // every page is read exactly once: stream it past the caches
            kk[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(KC + off));
            vv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(VC + off));
        }
        return blk_ok;
    };

    // Process page p from (kk, vv) while the wave's next page streams into
    // (kn, vn); the loop is unrolled by two so the buffers swap roles instead
    // of being copied (a copy would wait for the loads in flight).
    auto page = [&](const int p, u32x4 (&kk)[4], u32x4 (&vv)[4], const bool ok_cur, u32x4 (&kn)[4],
                    u32x4 (&vn)[4], bool& ok_nxt) __attribute__((always_inline)) {
        if (p + kWaves < page1) ok_nxt = load_page(p + kWaves, kn, vn);
        // tokens of this page in use; only a sequence's last page (or a page
        // behind an invalid block id) is partly masked
        const int valid = ok_cur ? min(kPage, len - p * kPage) : 0;
        const bool partial = valid < kPage;

        float s[G][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int h = 0; h < G; ++h) s[h][i] = row_sum16(dot8_bf16(kk[i], qv[h]));
        if (partial) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = row + 4 * i < valid;
#pragma unroll
                for (int h = 0; h < G; ++h) s[h][i] = ok ? s[h][i] : kNegInf;
                // masked slots may hold anything, NaN included: never multiply them
                if (!ok) vv[i] = u32x4{0, 0, 0, 0};
            }
        }

        // Online softmax per lane row.  The reference maximum moves only when
        // a row's page maximum outgrows it by 2^kTau (p <= 2^kTau otherwise;
        // the stale reference cancels in the final division).
        float mx[G];
        bool grow = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            mx[h] = fmaxf(fmaxf(s[h][0], s[h][1]), fmaxf(s[h][2], s[h][3])) * scale_log2;
            grow |= mx[h] > m[h] + kTau;
        }
        if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float m_new = fmaxf(m[h], mx[h]);
                const float alpha = exp2f_hw(m[h] - (m_new == kNegInf ? 0.f : m_new));
                m[h] = m_new;
                l[h] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
            }
        }

        // O += P V over the lane's tokens: P rounded to bf16 once, token pairs
        // (0,1) and (2,3) contracted with packed dot products.
        uint32_t v01lo[4], v01hi[4], v23lo[4], v23hi[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            v01lo[w] = __builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x05040100u);
            v01hi[w] = __builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x07060302u);
            v23lo[w] = __builtin_amdgcn_perm(vv[3][w], vv[2][w], 0x05040100u);
            v23hi[w] = __builtin_amdgcn_perm(vv[3][w], vv[2][w], 0x07060302u);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float m_use = m[h] == kNegInf ? 0.f : m[h];
            const float p0 = exp2f_hw(fmaf(s[h][0], scale_log2, -m_use));
            const float p1 = exp2f_hw(fmaf(s[h][1], scale_log2, -m_use));
            const float p2 = exp2f_hw(fmaf(s[h][2], scale_log2, -m_use));
            const float p3 = exp2f_hw(fmaf(s[h][3], scale_log2, -m_use));
            l[h] += (p0 + p1) + (p2 + p3);
            const uint32_t w01 = pack_bf16x2(p0, p1), w23 = pack_bf16x2(p2, p3);
            const bf16x2 b01 = __builtin_bit_cast(bf16x2, w01), b23 = __builtin_bit_cast(bf16x2, w23);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t a0 = v01lo[w], a1 = v23lo[w], c0 = v01hi[w], c1 = v23hi[w];
                float e0 = acc[h][2 * w], e1 = acc[h][2 * w + 1];
                e0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a0), b01, e0, false);
                e0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a1), b23, e0, false);
                e1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, c0), b01, e1, false);
                e1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, c1), b23, e1, false);
                acc[h][2 * w] = e0;
                acc[h][2 * w + 1] = e1;
            }
        }
    };

    u32x4 ka[4], va[4], kb[4], vb[4];
    bool oka = false, okb = false;
    const int p_first = page0 + wave;
    if (p_first < page1) oka = load_page(p_first, ka, va);
    for (int p = p_first; p < page1; p += 2 * kWaves) {
        page(p, ka, va, oka, kb, vb, okb);
        if (p + kWaves < page1) page(p + kWaves, kb, vb, okb, ka, va, oka);
    }

    // Merge the four token rows of the wave (lanes l, l^16, l^32, l^48 share a slice).
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = __shfl_xor(m[h], off);
            const float lo = __shfl_xor(l[h], off);
            const float M = fmaxf(m[h], mo);
            const float Mu = M == kNegInf ? 0.f : M;
            const float a = exp2f_hw(m[h] - Mu), bw = exp2f_hw(mo - Mu);
            l[h] = a * l[h] + bw * lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float ao = __shfl_xor(acc[h][e], off);
                acc[h][e] = a * acc[h][e] + bw * ao;
            }
            m[h] = M;
        }
    }
    if (row == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sm_acc[wave][h][8 * col + e] = acc[h][e];
            if (col == 0) {
                sm_m[wave][h] = m[h];
                sm_l[wave][h] = l[h];
            }
        }
    }
    __syncthreads();

    // Merge the waves and write the range's normalised output and lse.
    for (int idx = tid; idx < G * kD; idx += kThreads) {
        const int h = idx / kD, d = idx % kD;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
        const float Mu = M == kNegInf ? 0.f : M;
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float c = exp2f_hw(sm_m[w][h] - Mu);
            L = fmaf(c, sm_l[w][h], L);
            A = fmaf(c, sm_acc[w][h][d], A);
        }
        const int64_t slot = ((int64_t)seq * Hq + hq0 + h) * n_split + split;
        ws_o[slot * kD + d] = L > 0.f ? A / L : 0.f;
        if (d == 0) ws_lse[slot] = L > 0.f ? (M + log2f_hw(L)) * kLn2 : kNegInf;
    }
}

// One workgroup per (query head, sequence); one thread per head-dim element.
__global__ __launch_bounds__(kD) void decode_combine_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse, const int32_t* __restrict__ seqlens,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Hq, int max_blocks, int pages_per_split,
    int n_split) {
    const int hq = blockIdx.x, seq = blockIdx.y, d = threadIdx.x;
    const int len = min(max(seqlens[seq], 0), max_blocks * kPage);
    const int n_pages = (len + kPage - 1) / kPage;
    const int n = (n_pages + pages_per_split - 1) / pages_per_split;
    const int64_t slot0 = ((int64_t)seq * Hq + hq) * n_split;

    float M = kNegInf;
    for (int s = 0; s < n; ++s) M = fmaxf(M, ws_lse[slot0 + s]);
    const float Mu = M == kNegInf ? 0.f : M;
    float W = 0.f, A = 0.f;
    for (int s = 0; s < n; ++s) {
        const float w = exp2f_hw((ws_lse[slot0 + s] - Mu) * kLog2e);
        W += w;
        A = fmaf(w, ws_o[(slot0 + s) * kD + d], A);
    }
    const float o = W > 0.f ? A / W : 0.f;
    const int64_t oi = ((int64_t)seq * Hq + hq) * kD + d;
    const uint32_t packed = pack_bf16x2(o, 0.f);
    O[oi] = (uint16_t)(packed & 0xffffu);
    if (LSE != nullptr && d == 0) LSE[(int64_t)seq * Hq + hq] = W > 0.f ? Mu + log2f_hw(W) * kLn2 : kNegInf;
}

template <int G>
hipError_t launch_partial(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
    hipLaunchKernelGGL((decode_partial_kernel<G>), dim3(pl.n_split, a.Hkv, a.nseq), dim3(kThreads), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.kcache, (const uint16_t*)a.vcache, a.block_table,
                       a.seqlens, pl.ws_o, pl.ws_lse, a.Hq, a.Hkv, a.max_blocks, a.num_blocks, pl.pages_per_split,
                       pl.n_split, a.scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(int nseq, int Hq, int Hkv, int max_blocks) {
    DecodePlan pl{};
    // Enough ranges to give every CU several workgroups even when few
    // sequences are decoded; never more than the table can hold.
    const int64_t heads = (int64_t)nseq * Hkv;
    int pps = 32;
    while (pps > 4 && heads * ((max_blocks + pps - 1) / pps) < 2048) pps >>= 1;
    pl.pages_per_split = pps;
    pl.n_split = (max_blocks + pps - 1) / pps;
    pl.ws_o_elems = (int64_t)nseq * Hq * pl.n_split * kD;
    pl.ws_lse_elems = (int64_t)nseq * Hq * pl.n_split;
    return pl;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
    hipError_t e;
    switch (a.Hq / a.Hkv) {
        case 1: e = launch_partial<1>(a, pl, stream); break;
        case 2: e = launch_partial<2>(a, pl, stream); break;
        case 4: e = launch_partial<4>(a, pl, stream); break;
        default: e = launch_partial<8>(a, pl, stream); break;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(a.Hq, a.nseq), dim3(kD), 0, stream, pl.ws_o, pl.ws_lse,
                       a.seqlens, (uint16_t*)a.o, a.lse, a.Hq, a.max_blocks, pl.pages_per_split, pl.n_split);
    return hipGetLastError();
}

}  // namespace fa
