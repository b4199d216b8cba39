// Paged KV-cache decode: one new query token per sequence (gfx950).
//
// Single-token decode reads every cached K and V once and does about
// Hq/Hkv FLOP per byte ("Week 13. GPUs and FlashAttention", Step 1), so it is
// bound by HBM bandwidth.  The design aims at many bytes in flight, at reading
// each page exactly once, and at giving every wave the same number of pages
// however unequal the sequence lengths are:
//
//   * Work is the flat list of (sequence, K/V head, page) in that order; a
//     (sequence, K/V head) run of pages is a segment.  A one-workgroup
//     schedule kernel sums the page counts, then cuts the list into nw equal
//     contiguous ranges, one per wave of a grid sized to what the chip keeps
//     resident; each wave gets its start (sequence, head, page) and length.
//   * A wave attends the G = Hq/Hkv query heads that share its K/V head
//     ("Fast Inference and Training at Scale", section 6.2) to its range, so
//     a page is loaded once for all G heads.  Waves are independent: no LDS,
//     no barriers.  A wave that holds a whole segment writes the final output;
//     otherwise it writes a normalised partial output and log-sum-exp.
//   * Pages are found through the block table (section 6.3 PagedAttention).
//     A 16-token page of one head is 4 KiB of K and 4 KiB of V, contiguous;
//     a wave loads a whole page with 16-byte coalesced loads: lane l takes
//     head-dim slice 8 (l % 16) .. +8 of tokens l/16, l/16 + 4, +8, +12.  The
//     wave's next two pages are in flight while the current one is computed.
//   * Scores: packed bf16 dot products over the lane's slice, then a DPP sum
//     across the 16 lanes that share a token.
//   * Online softmax ("Hardware Co-Design") per lane row over the pages the
//     row visits; the four token rows of a wave are merged with the same
//     update applied to whole partial states.
//   * A combine kernel merges the partials of each split segment:
//     M = max lse_s, o = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M),
//     lse = M + ln sum_s e^(lse_s - M).
//
// Device values are made safe here: lengths are clamped to the table's
// capacity, block ids outside [0, num_blocks) contribute no key, and slots of
// a partly filled last page are masked with selects (never multiplied), so a
// NaN left in them cannot reach the output.
#include "fa_device.h"
#include "fa_launch.h"

#include <atomic>

namespace fa {
namespace {

constexpr int kD = 128;
constexpr int kPage = 16;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kTau = 8.f;            // log2 of the growth allowed before a rescale
constexpr int kMaxWaves = 4096;        // waves of the partial kernel, at most
constexpr int kMinPagesPerWave = 4;    // fewer waves than pages / 4 are never used
constexpr int kSchedThreads = 1024;

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

// Pages of sequence s: its length clamped to the table's capacity.
__device__ __forceinline__ int seq_pages(const int32_t* seqlens, int s, int max_blocks) {
    const int len = min(max(seqlens[s], 0), max_blocks * kPage);
    return (len + kPage - 1) / kPage;
}

// Exclusive scan over the workgroup under an associative op with identity
// `id`; *total gets the reduction of all x.
template <typename Op>
__device__ int64_t block_exclusive_scan(int64_t x, int64_t id, int64_t* sm, int64_t* total, Op op) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int64_t inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(inc, o);
        if (lane >= o) inc = op(inc, y);
    }
    const int64_t exc_in_wave = __shfl_up(inc, 1);
    if (lane == 63) sm[wv] = inc;
    __syncthreads();
    int64_t before = id, all = id;
    for (int w = 0; w < kSchedThreads / 64; ++w) {
        const int64_t t = sm[w];
        if (w < wv) before = op(before, t);
        all = op(all, t);
    }
    __syncthreads();
    *total = all;
    return lane == 0 ? before : op(before, exc_in_wave);
}

// floor(a / b) for 0 <= a < 2^53, 0 < b < 2^53: a double quotient (within one
// of the true one) corrected with integer products; integer 64-bit division
// is a long software sequence on this GPU.
__device__ __forceinline__ int64_t div_floor(int64_t a, int64_t b) {
    int64_t q = (int64_t)((double)a / (double)b);
    if (q * b > a) --q;
    else if ((q + 1) * b <= a) ++q;
    return q;
}

struct Add {
    __device__ int64_t operator()(int64_t a, int64_t b) const { return a + b; }
};
struct Max {
    __device__ int64_t operator()(int64_t a, int64_t b) const { return a > b ? a : b; }
};

// Header written by the schedule kernel: hdr[0] = T, the pages of all
// (sequence, K/V head) pairs; hdr[1] = nw, the waves that share them.  Wave g
// holds flat pages [lo(g), lo(g + 1)), lo(g) = g T / nw; the wave holding
// flat page x is ((x + 1) nw - 1) / T.  Sequence s owns flat pages
// [P(s) Hkv, P(s + 1) Hkv), P the exclusive prefix of the page counts, and
// the waves starting in it are those from ceil(P(s) Hkv nw / T) on, so the
// sequence of wave g is the largest non-empty s with that bound <= g.
constexpr int kPerThread = kMaxWaves / kSchedThreads;
static_assert(kPerThread * kSchedThreads == kMaxWaves, "the wave table is split evenly over the threads");

__global__ __launch_bounds__(kSchedThreads) void decode_schedule_kernel(
    const int32_t* __restrict__ seqlens, int nseq, int Hkv, int max_blocks, int max_waves,
    int64_t* __restrict__ hdr, int64_t* __restrict__ prefix, int4* __restrict__ wtab) {
    __shared__ int64_t sm[kSchedThreads / 64];
    __shared__ int owner[kMaxWaves];
    const int tid = threadIdx.x;

    int64_t pages_all = 0;
    for (int base = 0; base < nseq; base += kSchedThreads) {
        const int s = base + tid;
        int64_t chunk;
        block_exclusive_scan(s < nseq ? seq_pages(seqlens, s, max_blocks) : 0, 0, sm, &chunk, Add{});
        pages_all += chunk;
    }
    const int64_t T = pages_all * Hkv;
    const int64_t nw = T == 0 ? 0 : min((int64_t)max_waves, (T + kMinPagesPerWave - 1) / kMinPagesPerWave);   // constant divisor
    if (tid == 0) {
        hdr[0] = T;
        hdr[1] = nw;
        prefix[nseq] = pages_all;
    }
    for (int g = tid; g < kMaxWaves; g += kSchedThreads) owner[g] = -1;
    __syncthreads();

    // page prefix per sequence; mark the first wave that starts in each
    int64_t carry = 0;
    for (int base = 0; base < nseq; base += kSchedThreads) {
        const int s = base + tid;
        const int np = s < nseq ? seq_pages(seqlens, s, max_blocks) : 0;
        int64_t chunk;
        const int64_t P = carry + block_exclusive_scan(np, 0, sm, &chunk, Add{});
        if (s < nseq) prefix[s] = P;
        if (np > 0) {
            const int64_t g = div_floor(P * Hkv * nw + T - 1, T);
            if (g < nw) atomicMax(&owner[g], s);
        }
        carry += chunk;
    }
    __syncthreads();

    // the owner of every wave is the running maximum of the marks
    int own[kPerThread];
    int64_t run = -1;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        own[j] = owner[tid * kPerThread + j];
        run = max(run, (int64_t)own[j]);
    }
    int64_t unused;
    int64_t cur = block_exclusive_scan(run, -1, sm, &unused, Max{});
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        const int64_t g = tid * kPerThread + j;
        cur = max(cur, (int64_t)own[j]);
        if (g < nw) {
            const int s = (int)cur;
            const int np = seq_pages(seqlens, s, max_blocks);
            const int64_t lo = div_floor(g * T, nw), hi = div_floor((g + 1) * T, nw);
            const int off = (int)(lo - prefix[s] * Hkv);
            wtab[g] = make_int4(s, off / np, off % np, (int)(hi - lo));
        }
    }
}

// Wave-level form of the same split for batches of at most kInlineSeqs
// sequences: each wave reads every length once (kSeqsPerLane per lane), scans
// the page counts across the wave and finds the sequence holding its first
// flat page, so no separate schedule launch is needed.  Wave 0 publishes the
// header and the page prefix that the combine step reads.  Returns the job
// (sequence, K/V head, page, count); count is 0 for a wave without pages.
constexpr int kSeqsPerLane = 16;
constexpr int kInlineSeqs = 64 * kSeqsPerLane;

__device__ __forceinline__ int4 wave_job(const int32_t* __restrict__ seqlens, int nseq, int Hkv, int max_blocks,
                                         int max_waves, int gw, int lane, int64_t* __restrict__ hdr,
                                         int64_t* __restrict__ prefix) {
    const int s0 = lane * kSeqsPerLane;
    int np[kSeqsPerLane];
    int local = 0;
#pragma unroll
    for (int r = 0; r < kSeqsPerLane; ++r) {
        np[r] = s0 + r < nseq ? seq_pages(seqlens, s0 + r, max_blocks) : 0;
        local += np[r];
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    const int pages_all = __shfl(incl, 63);
    const int64_t T = (int64_t)pages_all * Hkv;
    const int64_t nw = T == 0 ? 0 : min((int64_t)max_waves, (T + kMinPagesPerWave - 1) / kMinPagesPerWave);
    int P = incl - local;   // pages before sequence s0
    if (gw == 0) {
        if (lane == 0) {
            hdr[0] = T;
            hdr[1] = nw;
            prefix[nseq] = pages_all;
        }
        int q = P;
#pragma unroll
        for (int r = 0; r < kSeqsPerLane; ++r) {
            if (s0 + r < nseq) prefix[s0 + r] = q;
            q += np[r];
        }
    }
    if (gw >= nw) return make_int4(0, 0, 0, 0);
    const int64_t lo = div_floor(gw * T, nw), hi = div_floor((gw + 1) * T, nw);
    int4 job = make_int4(0, 0, 0, 0);
    bool found = false;
#pragma unroll
    for (int r = 0; r < kSeqsPerLane; ++r) {
        const int64_t A = (int64_t)P * Hkv, B = (int64_t)(P + np[r]) * Hkv;
        if (np[r] > 0 && A <= lo && lo < B) {
            const int off = (int)(lo - A);
            job = make_int4(s0 + r, off / np[r], off % np[r], (int)(hi - lo));
            found = true;
        }
        P += np[r];
    }
    // exactly one lane holds the sequence of flat page lo
    const int src = __builtin_ctzll(__builtin_amdgcn_ballot_w64(found));
    return make_int4(__shfl(job.x, src), __shfl(job.y, src), __shfl(job.z, src), __shfl(job.w, src));
}

// Two resident waves per SIMD (two workgroups per CU) keep enough pages in
// flight once every wave has the same share of pages; a tighter register
// budget for three spills and measures slower.
template <int G>
__global__ __launch_bounds__(kThreads, G <= 4 ? 2 : 1) void decode_partial_kernel(
    const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ KC, const uint16_t* __restrict__ VC,
    const int32_t* __restrict__ table, const int32_t* __restrict__ seqlens, int64_t* hdr,
    const int4* __restrict__ wtab, uint16_t* __restrict__ O, float* __restrict__ LSE, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, int64_t* __restrict__ prefix, int inline_sched,
    int max_waves, int nseq, int Hq, int Hkv, int max_blocks, int num_blocks, float scale_log2) {
    const int tid = threadIdx.x;
    // The wave index is made scalar so the schedule and block-table reads are
    // scalar loads: waiting for one then does not also wait for the vector
    // loads of the page in flight.
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row = lane >> 4;                    // token slot: tokens row, row+4, row+8, row+12
    const int col = lane & 15;                    // head-dim slice 8*col .. 8*col+7
    const uint32_t lane_bytes = (uint32_t)(row * kD + 8 * col) * 2;
    const int gw = blockIdx.x * kWaves + wave;
    int4 job;
    if (inline_sched) {
        job = wave_job(seqlens, nseq, Hkv, max_blocks, max_waves, gw, lane, hdr, prefix);
    } else {
        if (gw >= hdr[1]) return;
        job = wtab[gw];
    }
    // the job is wave-uniform: keep it in scalar registers
    int seq = __builtin_amdgcn_readfirstlane(job.x), kvh = __builtin_amdgcn_readfirstlane(job.y);
    int p0 = __builtin_amdgcn_readfirstlane(job.z), remaining = __builtin_amdgcn_readfirstlane(job.w);

    while (remaining > 0 && seq < nseq) {
        const int len = min(max(seqlens[seq], 0), max_blocks * kPage);
        const int np = (len + kPage - 1) / kPage;
        const int n = min(remaining, np - p0);      // this wave's pages of the segment
        if (n <= 0) {                               // an empty sequence: no pages to take
            ++seq;
            kvh = 0;
            p0 = 0;
            continue;
        }
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
            // the page's base is wave-uniform (scalar registers); lanes add a
            // 32-bit offset
            const int64_t page_off = ((int64_t)(blk_ok ? bid : 0) * Hkv + kvh) * (kPage * kD * 2);
            const char* kp = reinterpret_cast<const char*>(KC) + page_off;
            const char* vp = reinterpret_cast<const char*>(VC) + page_off;
            // opaque to the optimiser, so the lane offset is not folded into
            // a loop-invariant 64-bit vector address
            uint32_t lb = lane_bytes;
            asm volatile("" : "+v"(lb));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // every page is read exactly once: stream it past the caches
                kk[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + lb + i * (4 * kD * 2)));
                vv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + lb + i * (4 * kD * 2)));
            }
            return blk_ok;
        };

        // Process page p from (kk, vv) and start loading page p + 2 into
        // (kn, vn); the loop is unrolled by three so the buffers rotate roles
        // instead of being copied (a copy would wait for the loads in flight).
        auto page = [&](const int p, u32x4 (&kk)[4], u32x4 (&vv)[4], const bool ok_cur, u32x4 (&kn)[4],
                        u32x4 (&vn)[4], bool& ok_nxt, const bool has_next) __attribute__((always_inline)) {
            if (has_next) ok_nxt = load_page(p + 2, kn, vn);
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


        // three page buffers: two pages in flight while one is computed
        u32x4 ka[4], va[4], kb[4], vb[4], kc[4], vc[4];
        bool oka = load_page(p0, ka, va), okb = false, okc = false;
        if (n > 1) okb = load_page(p0 + 1, kb, vb);
        for (int i = 0; i < n; i += 3) {
            page(p0 + i, ka, va, oka, kc, vc, okc, i + 2 < n);
            if (i + 1 < n) page(p0 + i + 1, kb, vb, okb, ka, va, oka, i + 3 < n);
            if (i + 2 < n) page(p0 + i + 2, kc, vc, okc, kb, vb, okb, i + 4 < n);
        }

        // Merge the four token rows of the wave (lanes l, l^16, l^32, l^48
        // share a slice); afterwards every row holds the merged state.
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
            const bool whole = p0 == 0 && n == np;   // no other wave saw this segment
            const int64_t slot = (int64_t)seq * Hkv + kvh + gw;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float inv = l[h] > 0.f ? 1.f / l[h] : 0.f;
                const float lse = l[h] > 0.f ? (m[h] + log2f_hw(l[h])) * kLn2 : kNegInf;
                if (whole) {
                    u32x4 packed;
#pragma unroll
                    for (int w = 0; w < 4; ++w) packed[w] = pack_bf16x2(acc[h][2 * w] * inv, acc[h][2 * w + 1] * inv);
                    *reinterpret_cast<u32x4*>(O + ((int64_t)seq * Hq + hq0 + h) * kD + 8 * col) = packed;
                    if (LSE != nullptr && col == 0) LSE[(int64_t)seq * Hq + hq0 + h] = lse;
                } else {
                    float* dst = ws_o + (slot * G + h) * kD + 8 * col;
                    *reinterpret_cast<f32x4*>(dst) = f32x4{acc[h][0] * inv, acc[h][1] * inv, acc[h][2] * inv, acc[h][3] * inv};
                    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[h][4] * inv, acc[h][5] * inv, acc[h][6] * inv, acc[h][7] * inv};
                    if (col == 0) ws_lse[slot * G + h] = lse;
                }
            }
        }

        remaining -= n;
        p0 = 0;
        if (++kvh == Hkv) {
            kvh = 0;
            ++seq;
        }
    }
}

// One workgroup per (K/V head, sequence), one thread per (query head of the
// group, head-dim element).  Segments one wave held whole were written by
// that wave and are skipped; the others merge their partials in one pass
// with the online-softmax update.
template <int G>
__global__ __launch_bounds__(G * kD) void decode_combine_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse, const int32_t* __restrict__ seqlens,
    const int64_t* __restrict__ hdr, const int64_t* __restrict__ prefix, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int Hq, int Hkv, int max_blocks) {
    const int kvh = blockIdx.x, seq = blockIdx.y;
    const int g = threadIdx.x / kD, d = threadIdx.x % kD;
    const int hq = kvh * G + g;
    const int np = seq_pages(seqlens, seq, max_blocks);
    const int64_t oi = ((int64_t)seq * Hq + hq) * kD + d;
    if (np == 0) {
        O[oi] = 0;
        if (LSE != nullptr && d == 0) LSE[(int64_t)seq * Hq + hq] = kNegInf;
        return;
    }
    const int64_t T = hdr[0], nw = hdr[1];
    const int64_t A = prefix[seq] * Hkv + (int64_t)kvh * np;   // the segment's first flat page
    const int64_t g0 = div_floor((A + 1) * nw - 1, T), g1 = div_floor((A + np) * nw - 1, T);
    if (g0 == g1) return;
    const int64_t slot0 = (int64_t)seq * Hkv + kvh;

    // partials are loaded kBatch at a time so their loads overlap
    constexpr int kBatch = 8;
    float M = kNegInf, W = 0.f, acc = 0.f;       // natural-log scale
    for (int64_t w0 = g0; w0 <= g1; w0 += kBatch) {
        float ls[kBatch], os[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t sl = (slot0 + min(w0 + j, g1)) * G + g;
            ls[j] = w0 + j <= g1 ? ws_lse[sl] : kNegInf;
            os[j] = ws_o[sl * kD + d];
        }
        float mb = kNegInf;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) mb = fmaxf(mb, ls[j]);
        if (mb == kNegInf) continue;            // no visible key in these ranges
        if (mb > M) {
            const float c = M == kNegInf ? 0.f : exp2f_hw((M - mb) * kLog2e);
            W *= c;
            acc *= c;
            M = mb;
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            // e^(-inf) = 0 drops ranges with no visible key (their o is 0)
            const float c = exp2f_hw((ls[j] - M) * kLog2e);
            W += c;
            acc = fmaf(c, os[j], acc);
        }
    }
    const float out = W > 0.f ? acc / W : 0.f;
    O[oi] = (uint16_t)(pack_bf16x2(out, 0.f) & 0xffffu);
    if (LSE != nullptr && d == 0) LSE[(int64_t)seq * Hq + hq] = W > 0.f ? M + log2f_hw(W) * kLn2 : kNegInf;
}

// Workspace: header, per-sequence page prefix, wave table, then the partial
// outputs and lse of (nseq Hkv + kMaxWaves) slots of G heads; a partial of
// segment (s, h) from wave g lives in slot s Hkv + h + g, unique because the
// waves of consecutive segments overlap in at most one wave.
struct Layout {
    size_t hdr, prefix, wtab, o, lse, total;
};

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

Layout layout(int nseq, int Hq, int Hkv) {
    const size_t G = (size_t)(Hq / Hkv), slots = (size_t)nseq * Hkv + kMaxWaves;
    Layout L{};
    L.hdr = 0;
    L.prefix = L.hdr + 256;
    L.wtab = L.prefix + round256(sizeof(int64_t) * ((size_t)nseq + 1));
    L.o = L.wtab + round256(sizeof(int4) * kMaxWaves);
    L.lse = L.o + round256(sizeof(float) * slots * G * kD);
    L.total = L.lse + round256(sizeof(float) * slots * G);
    return L;
}

int device_cus() {
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

template <int G>
int resident_per_cu() {
    static std::atomic<int> cache{0};
    int n = cache.load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_partial_kernel<G>, kThreads, 0) != hipSuccess || n <= 0)
        n = 1;
    cache.store(n, std::memory_order_relaxed);
    return n;
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, char* ws, const Layout& L, hipStream_t stream) {
    auto* hdr = reinterpret_cast<int64_t*>(ws + L.hdr);
    auto* prefix = reinterpret_cast<int64_t*>(ws + L.prefix);
    auto* wtab = reinterpret_cast<int4*>(ws + L.wtab);
    auto* wo = reinterpret_cast<float*>(ws + L.o);
    auto* wl = reinterpret_cast<float*>(ws + L.lse);

    // As many workgroups as stay resident, and no more than the pages at the
    // table's capacity can keep busy.
    const int64_t cap_pages = (int64_t)a.nseq * a.Hkv * a.max_blocks;
    int64_t wgs = (int64_t)resident_per_cu<G>() * device_cus();
    wgs = std::min<int64_t>(wgs, kMaxWaves / kWaves);
    wgs = std::min<int64_t>(wgs, (cap_pages + (int64_t)kMinPagesPerWave * kWaves - 1) / ((int64_t)kMinPagesPerWave * kWaves));
    wgs = std::max<int64_t>(wgs, 1);
    const int max_waves = (int)wgs * kWaves;

    // small batches: every wave finds its own range; larger ones: one
    // schedule workgroup writes the wave table first
    const int inline_sched = a.nseq <= kInlineSeqs ? 1 : 0;
    hipError_t e;
    if (!inline_sched) {
        launch_kernel<false>(decode_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, a.seqlens, a.nseq, a.Hkv,
                           a.max_blocks, max_waves, hdr, prefix, wtab);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    launch_kernel<false>((decode_partial_kernel<G>), dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.kcache, (const uint16_t*)a.vcache, a.block_table,
                       a.seqlens, hdr, wtab, (uint16_t*)a.o, a.lse, wo, wl, prefix, inline_sched, max_waves,
                       a.nseq, a.Hq, a.Hkv, a.max_blocks, a.num_blocks, a.scale * kLog2e);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_kernel((decode_combine_kernel<G>), dim3(a.Hkv, a.nseq), dim3(G * kD), 0, stream, wo, wl, a.seqlens,
                       hdr, prefix, (uint16_t*)a.o, a.lse, a.Hq, a.Hkv, a.max_blocks);
    return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int nseq, int Hq, int Hkv) { return layout(nseq, Hq, Hkv).total; }

hipError_t launch_decode(const DecodeArgs& a, void* workspace, hipStream_t stream) {
    const Layout L = layout(a.nseq, a.Hq, a.Hkv);
    char* ws = static_cast<char*>(workspace);
    switch (a.Hq / a.Hkv) {
        case 1: return launch_g<1>(a, ws, L, stream);
        case 2: return launch_g<2>(a, ws, L, stream);
        case 4: return launch_g<4>(a, ws, L, stream);
        default: return launch_g<8>(a, ws, L, stream);
    }
}

// Scratch of the allocation-free entry point: one array per GPU, held until
// the process ends.  In host code `scratch` only names the symbol; the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken
// once per device with that device current and kept below.  Every call on a
// GPU reuses its array; nothing in it has to start at zero (the decode
// writes every partial and table entry it reads within the same call), and
// calls that overlap on one GPU race on it.
static __device__ __align__(256) uint8_t scratch[kDecodeNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
}  // namespace

hipError_t launch_decode_noalloc(const DecodeArgs& a, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        // (two threads may both get here: they store the same address)
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        g_scratch_addr[dev].store(ptr, std::memory_order_release);
    }
    return launch_decode(a, ptr, stream);
}

}  // namespace fa
