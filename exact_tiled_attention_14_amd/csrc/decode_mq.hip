// Multi-query paged attention: Sq new tokens per sequence (a speculative
// verify step or a chunk of prefill) against the paged KV cache, gfx950.
//
// "Fast Inference and Training at Scale", section 6.5 (the target model
// verifies the draft tokens in one pass, all their queries at once), with the
// cache of sections 6.1 and 6.3; new token t of a sequence of length n sits at
// position n - Sq + t and sees the keys up to its own position (bottom-right
// causal).  The step still reads every cached K and V once but now does
// Sq Hq/Hkv FLOP per byte ("Week 13. GPUs and FlashAttention", Step 1: a
// verify pass carries B (gamma + 1) tokens), which is too much for vector ALUs
// and far too little to be compute-bound: the products go to the matrix cores
// and the kernel is designed around HBM streaming.
//
//   * Rows: the G = Hq/Hkv query heads of a K/V head times the Sq tokens form
//     R = G Sq <= 32 rows, one 32-row matrix-core tile (row r = token r / G,
//     head r % G); a page is read once for all of them.
//   * Work: one workgroup per (chunk of 128 pages, sequence, K/V head),
//     chunk-major so the first chunks of all sequences go first; the chunk's
//     pages are split evenly over its 4 waves.  A step is 2 pages (32 keys):
//     its K and V arrive in registers by coalesced non-temporal loads (1 KiB
//     of contiguous memory per instruction), are written to the wave's own
//     LDS tile, and are read back as matrix-core operands: K rows for
//     S^T = K Q^T, V transposed (ds_read_b64_tr_b16) for O^T += V^T P^T.  The
//     next step's loads are issued right after this step's tile is written,
//     so they stream while this step computes.  Waves share no data and meet
//     only at the final merge.
//   * Online softmax per lane (one row) with the deferred rescale of the
//     prefill kernel; keys past the sequence or the wave's pages, above a
//     row's causal limit, or in pages whose block id is out of range are
//     masked with selects, so NaN left in unused page slots never propagates.
//   * The 4 wave states are merged through LDS; a sequence with one chunk is
//     written directly, otherwise each chunk writes a normalised partial
//     (o, lse) and mq_combine_kernel merges them.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kD = 128;
constexpr int kPage = 16;
constexpr int kWavesM = 4;
constexpr int kThreadsM = 64 * kWavesM;
constexpr int kPagesPerWave = 32;
constexpr int kChunkPages = kPagesPerWave * kWavesM;     // 128 pages per workgroup
static_assert(kPagesPerWave <= 64, "a wave's page ids fit one register across its lanes");
constexpr int kStepBytes = 2 * kPage * kD * 2;           // V of one 32-key step: 8 KiB
constexpr float kTauM = 8.f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ s16x4 lds_tr16(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const __attribute__((address_space(3))) uint8_t*)p);
}

// V^T operand of output block db, key step ks (keys 16 ks .. +15) from a
// row-major 32 x 128 V stage whose 16-byte chunk c of row r sits at
// c ^ 4 (r % 4): lane l (column 32 db + l % 32, half h = l / 32) receives the
// keys 4h + e and 8 + 4h + e, the order in which it holds P.
__device__ __forceinline__ bf16x8 vt_op(const uint8_t* st, int ks, int db, int lane) {
    const int s = lane & 15, g = lane >> 4, h = g >> 1;
    const int col = 32 * db + 16 * (g & 1) + 4 * (s & 3);
    const int row0 = 16 * ks + 4 * h + (s >> 2);
    const int row1 = row0 + 8;
    const int x = col >> 3, half = (col >> 2) & 1;
    const uint8_t* p0 = st + row0 * 256 + 16 * (x ^ (4 * (row0 & 3))) + 8 * half;
    const uint8_t* p1 = st + row1 * 256 + 16 * (x ^ (4 * (row1 & 3))) + 8 * half;
    const s16x4 a = lds_tr16(p0), b = lds_tr16(p1);
    const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, v);
}


// Slot (in the K/V cache, in elements) of row `row` of page `blk` for head kvh.
__device__ __forceinline__ int64_t page_row(int blk, int Hkv, int kvh, int row) {
    return (((int64_t)blk * Hkv + kvh) * kPage + row) * kD;
}

template <int G>
__global__ __launch_bounds__(kThreadsM, 2) void mq_partial_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ KC, const uint16_t* __restrict__ VC,
    const int32_t* __restrict__ table, const int32_t* __restrict__ seqlens, uint16_t* __restrict__ O,
    float* __restrict__ LSE, float* __restrict__ ws_o, float* __restrict__ ws_lse, int nseq, int Sq, int Hq, int Hkv,
    int max_blocks, int num_blocks, int nchunk, float scale_log2) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kWavesM * 2 * kStepBytes];   // 64 KiB
    __shared__ float s_m[kWavesM][32], s_l[kWavesM][32];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int R = G * Sq;

    // chunk-major order: (chunk, sequence, K/V head)
    const int per_chunk = nseq * Hkv;
    const int chunk = blockIdx.x / per_chunk;
    const int rem = blockIdx.x % per_chunk;
    const int s = rem / Hkv, kvh = rem % Hkv;
    const int len = min(max(seqlens[s], 0), max_blocks * kPage);
    const int npages = (len + kPage - 1) / kPage;
    const int nch = (npages + kChunkPages - 1) / kChunkPages;
    if (chunk >= max(nch, 1)) return;                     // whole workgroup: no barrier reached

    const int32_t* trow = table + (int64_t)s * max_blocks;
    // the chunk's pages, split evenly over the 4 waves (a last, partial chunk too)
    const int ch0 = chunk * kChunkPages, ch1 = min(ch0 + kChunkPages, npages);
    const int per = (ch1 - ch0 + kWavesM - 1) / kWavesM;
    const int p0 = min(ch0 + wave * per, ch1);
    const int p1 = min(p0 + per, ch1);
    const int n_steps = p1 > p0 ? (p1 - p0 + 1) / 2 : 0;

    // this lane's query row: token t, head kvh * G + j
    const int my_row = l32;
    const int t = my_row / G, j = my_row % G;
    const bool row_ok = my_row < R;
    const int lim = len - Sq + t;                         // last visible key position of the row
    bf16x8 qf[kD / 16];
    {
        const uint16_t* qp = Q + (((int64_t)s * Sq + min(t, Sq - 1)) * Hq + kvh * G + j) * kD + 8 * hh;
#pragma unroll
        for (int i = 0; i < kD / 16; ++i) {
            const bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 16 * i);
            qf[i] = row_ok ? v : bf16x8{};
        }
    }

    // This wave's LDS tile for one step: K rows 0..31 (8 KiB), then V rows
    // 0..31 (8 KiB), row-major 256-byte rows.  K chunks are XOR-swizzled by
    // row % 16 and V chunks by 4 (row % 4), so the K operand reads (32 rows,
    // one chunk) and the transposing V reads hit distinct banks.
    uint8_t* const ktile = lds + wave * 2 * kStepBytes;
    uint8_t* const vtile = ktile + kStepBytes;

    // The wave's page ids (at most 32), one per lane, loaded once; a step reads
    // its two ids from this register (uniform lane reads, no branch around
    // them) instead of waiting on table loads behind its own prefetch.
    const int tb_lane = (p0 + lane < p1) ? trow[p0 + lane] : -1;
    auto blk_of = [&](int p) -> int {                     // block id of page p, -1 if unusable
        const int b = __builtin_amdgcn_readlane(tb_lane, min(max(p - p0, 0), 63));
        return (p < p1 && b >= 0 && b < num_blocks) ? b : -1;
    };
    // One step's K and V straight into registers with coalesced 16-byte
    // non-temporal loads: load c (0..7) takes rows 4 (c % 4) .. +3 of page
    // c / 4, lane l row 4 (c % 4) + l / 16, 16-byte chunk l % 16 (1 KiB of
    // contiguous memory per instruction).  A lane-per-key layout would touch
    // 32 rows per instruction and streamed a third slower.
    u32x4 kr[8], vr[8];
    auto load_step = [&](int step) {
        const int pa = p0 + 2 * step;
        const int b0 = max(blk_of(pa), 0), b1 = max(blk_of(pa + 1), 0);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int64_t off = page_row(c < 4 ? b0 : b1, Hkv, kvh, 4 * (c & 3) + (lane >> 4)) + 8 * (lane & 15);
            kr[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(KC + off));
            vr[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(VC + off));
        }
    };

    f32x16 oacc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};
    float m_run = kNegInf, l_run = 0.f;

    if (n_steps > 0) load_step(0);
    const int sw_k = l32 & 15;                            // K swizzle of this lane's operand row
    auto step = [&](int it) __attribute__((always_inline)) {
        const int pa = p0 + 2 * it;
        const bool ok0 = blk_of(pa) >= 0, ok1 = blk_of(pa + 1) >= 0;
        const int end = min(len, p1 * kPage);            // first position this wave must not use
        // registers -> this wave's tile (the previous step's reads of it are
        // done: a wave's LDS operations complete in order); V rows of unusable
        // keys are written as zeros, as p = 0 alone does not cancel a NaN
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int r = 4 * c + (lane >> 4), ch = lane & 15;
            const bool bad = (r < 16 ? !ok0 : !ok1) || pa * kPage + r >= end;
            *reinterpret_cast<u32x4*>(ktile + r * 256 + 16 * (ch ^ (r & 15))) = kr[c];
            *reinterpret_cast<u32x4*>(vtile + r * 256 + 16 * (ch ^ (4 * (r & 3)))) = bad ? u32x4{0u, 0u, 0u, 0u} : vr[c];
        }
        if (it + 1 < n_steps) load_step(it + 1);          // in flight while this step computes
        f32x16 sacc = f32x16{};
        const uint8_t* krow = ktile + l32 * 256;
#pragma unroll
        for (int i = 0; i < kD / 16; ++i) {
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + 16 * ((2 * i + hh) ^ sw_k));
            sacc = mfma32(ka, qf[i], sacc);
        }
        // mask: keys of the step are pages pa, pa + 1 of this wave.  A step
        // whose 32 keys all lie in usable pages and at or before the first new
        // token's position (so every row sees them) needs none (a wave-uniform
        // test); padding rows past R then score against zero queries, and
        // their results are never written.
        float mx = kNegInf;
        if (ok0 && ok1 && pa * kPage + 31 <= len - Sq) {
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kk = acc_row(r, hh);            // key of the step, 0 .. 31
                const int pos = pa * kPage + kk;
                const bool ok = row_ok && (kk < 16 ? ok0 : ok1) && pos < len && pos <= lim;
                sacc[r] = ok ? sacc[r] : kNegInf;
                mx = fmaxf(mx, sacc[r]);
            }
        }
        mx = half_swap_max(mx) * scale_log2;
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kTauM)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = exp2f_hw(m_run - (m_new == kNegInf ? 0.f : m_new));
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) oacc[i] *= alpha;
        }
        const float m_use = m_run == kNegInf ? 0.f : m_run;
        u32x4 pw[2];
        float rs = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float a = exp2f_hw(fmaf(sacc[4 * q + 0], scale_log2, -m_use));
            const float b = exp2f_hw(fmaf(sacc[4 * q + 1], scale_log2, -m_use));
            const float c = exp2f_hw(fmaf(sacc[4 * q + 2], scale_log2, -m_use));
            const float d = exp2f_hw(fmaf(sacc[4 * q + 3], scale_log2, -m_use));
            rs += (a + b) + (c + d);
            pw[q >> 1][2 * (q & 1)] = pack_bf16x2(a, b);
            pw[q >> 1][2 * (q & 1) + 1] = pack_bf16x2(c, d);
        }
        l_run += rs;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pw[ks]);
#pragma unroll
            for (int db = 0; db < 4; ++db) oacc[db] = mfma32(vt_op(vtile, ks, db, lane), pb, oacc[db]);
        }
    };
    for (int it = 0; it < n_steps; ++it) step(it);

    // ---- merge the 4 waves: unnormalised o into this wave's own LDS stages ----
    const float l_tot = half_swap_sum(l_run);
    float* ow = reinterpret_cast<float*>(ktile);          // [32 rows][128] fp32 = the wave's 16 KiB tile
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int dcol = 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3);
            ow[my_row * kD + dcol] = oacc[db][r];
        }
    if (hh == 0) {
        s_m[wave][my_row] = m_run;
        s_l[wave][my_row] = l_tot;
    }
    __syncthreads();

    // thread: row tid / 8, head-dim elements 16 (tid % 8) .. +15
    const int row = tid >> 3, c0 = 16 * (tid & 7);
    if (row >= R) return;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWavesM; ++w) M = fmaxf(M, s_m[w][row]);
    float wt[kWavesM], L = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesM; ++w) {
        wt[w] = M == kNegInf ? 0.f : exp2f_hw(s_m[w][row] - M);
        L += wt[w] * s_l[w][row];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const float lse = L > 0.f ? (M + log2f_hw(L)) * kLn2 : kNegInf;
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesM; ++w) {
        const float* src = reinterpret_cast<const float*>(lds + w * 2 * kStepBytes) + row * kD + c0;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = fmaf(wt[w], src[e], acc[e]);
    }
    const int tt = row / G, jj = row % G;
    const int64_t orow = ((int64_t)s * Sq + tt) * Hq + kvh * G + jj;
    if (nch <= 1) {
        uint16_t* op = O + orow * kD + c0;
#pragma unroll
        for (int e = 0; e < 16; e += 2) *reinterpret_cast<uint32_t*>(op + e) = pack_bf16x2(acc[e] * inv, acc[e + 1] * inv);
        if (LSE != nullptr && (tid & 7) == 0) LSE[orow] = lse;
    } else {
        const int64_t slot = ((int64_t)s * Hkv + kvh) * nchunk + chunk;
        float* wo = ws_o + (slot * 32 + row) * kD + c0;
#pragma unroll
        for (int e = 0; e < 16; e += 4) *reinterpret_cast<f32x4*>(wo + e) = f32x4{acc[e] * inv, acc[e + 1] * inv,
                                                                                   acc[e + 2] * inv, acc[e + 3] * inv};
        if ((tid & 7) == 0) ws_lse[slot * 32 + row] = lse;
    }
}

// Merge the chunk partials of the (sequence, K/V head) pairs that have more
// than one chunk: M = max lse_c, o = sum_c e^(lse_c - M) o_c / sum_c e^(lse_c - M),
// lse = M + ln sum_c e^(lse_c - M).
template <int G>
__global__ __launch_bounds__(kThreadsM) void mq_combine_kernel(const float* __restrict__ ws_o,
                                                               const float* __restrict__ ws_lse,
                                                               const int32_t* __restrict__ seqlens,
                                                               uint16_t* __restrict__ O, float* __restrict__ LSE,
                                                               int Sq, int Hq, int Hkv, int max_blocks, int nchunk) {
    const int s = blockIdx.x / Hkv, kvh = blockIdx.x % Hkv;
    const int len = min(max(seqlens[s], 0), max_blocks * kPage);
    const int nch = ((len + kPage - 1) / kPage + kChunkPages - 1) / kChunkPages;
    if (nch <= 1) return;
    const int tid = threadIdx.x;
    const int row = tid >> 3, c0 = 16 * (tid & 7);
    if (row >= G * Sq) return;
    const int64_t slot0 = ((int64_t)s * Hkv + kvh) * nchunk;
    // (unrolled so that the reads of several chunks are in flight together)
    float M = kNegInf;
#pragma unroll 4
    for (int c = 0; c < nch; ++c) M = fmaxf(M, ws_lse[(slot0 + c) * 32 + row]);
    float acc[16], L = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll 4
    for (int c = 0; c < nch; ++c) {
        const float lc = ws_lse[(slot0 + c) * 32 + row];
        const float w = M == kNegInf ? 0.f : exp2f_hw((lc - M) * kLog2e);
        L += w;
        const float* src = ws_o + ((slot0 + c) * 32 + row) * kD + c0;
#pragma unroll
        for (int e = 0; e < 16; e += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(src + e);
            acc[e] = fmaf(w, v[0], acc[e]);
            acc[e + 1] = fmaf(w, v[1], acc[e + 1]);
            acc[e + 2] = fmaf(w, v[2], acc[e + 2]);
            acc[e + 3] = fmaf(w, v[3], acc[e + 3]);
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int tt = row / G, jj = row % G;
    const int64_t orow = ((int64_t)s * Sq + tt) * Hq + kvh * G + jj;
    uint16_t* op = O + orow * kD + c0;
#pragma unroll
    for (int e = 0; e < 16; e += 2) *reinterpret_cast<uint32_t*>(op + e) = pack_bf16x2(acc[e] * inv, acc[e + 1] * inv);
    if (LSE != nullptr && (tid & 7) == 0) LSE[orow] = L > 0.f ? M + log2f_hw(L) * kLn2 : kNegInf;
}

template <int G>
hipError_t launch_mq_g(const DecodeMqArgs& a, void* workspace, hipStream_t stream) {
    const int nchunk = (a.max_blocks + kChunkPages - 1) / kChunkPages;
    float* wo = static_cast<float*>(workspace);
    float* wl = wo + (size_t)a.nseq * a.Hkv * nchunk * 32 * kD;
    const int64_t n_wg = (int64_t)nchunk * a.nseq * a.Hkv;
    launch_kernel<false>((mq_partial_kernel<G>), dim3((unsigned)n_wg), dim3(kThreadsM), 0, stream,
                         (const uint16_t*)a.q, (const uint16_t*)a.kcache, (const uint16_t*)a.vcache, a.block_table,
                         a.seqlens, (uint16_t*)a.o, a.lse, wo, wl, a.nseq, a.Sq, a.Hq, a.Hkv, a.max_blocks,
                         a.num_blocks, nchunk, a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_kernel((mq_combine_kernel<G>), dim3((unsigned)(a.nseq * a.Hkv)), dim3(kThreadsM), 0, stream, wo, wl,
                  a.seqlens, (uint16_t*)a.o, a.lse, a.Sq, a.Hq, a.Hkv, a.max_blocks, nchunk);
    return hipGetLastError();
}

}  // namespace

size_t decode_mq_workspace_bytes(int nseq, int Hkv, int max_blocks) {
    const size_t nchunk = (size_t)(max_blocks + kChunkPages - 1) / kChunkPages;
    const size_t slots = (size_t)nseq * Hkv * nchunk * 32;
    return ((slots * kD + slots) * sizeof(float) + 255) & ~(size_t)255;
}

hipError_t launch_decode_mq(const DecodeMqArgs& a, void* workspace, hipStream_t stream) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_mq_g<1>(a, workspace, stream);
        case 2: return launch_mq_g<2>(a, workspace, stream);
        case 4: return launch_mq_g<4>(a, workspace, stream);
        default: return launch_mq_g<8>(a, workspace, stream);
    }
}

}  // namespace fa
