// Latent-cache (MLA) decode: one new query token per sequence attending to a
// paged cache of compressed latents, gfx950.
//
// "Fast Inference and Training at Scale", section 6.4: the cache keeps only
// the latent c (d_c = 512 values per token) and the keys and values of head h
// are rebuilt from it, K_h = C W_K[h], V_h = C W_V[h].  Materialising them
// would cost H d_h (2 of them) values per cached token; the kernels use the
// same products in the other order (exact in real arithmetic):
//
//   score_hj = q_h . (c_j W_K[h]) = (W_K[h] q_h) . c_j
//   o_h      = sum_j p_hj c_j W_V[h] = (sum_j p_hj c_j) W_V[h]
//
// so the latent itself serves as the single shared key and value (one K/V
// head, as in section 6.2 with G = 1), and only the query and the output are
// projected:
//
//   1. mla_absorb_kernel: q~ = W_K[h] q_h (fp32, d_c per head) for all
//      sequences, on the matrix cores; one extra workgroup of the same launch
//      splits the work of step 2 (below).
//   2. mla_partial_kernel: attention of 16 absorbed queries (one head group)
//      over a range of at most 64 pages of one sequence.  Per
//      32-token step each wave loads 8 whole latent rows (1 KiB per load
//      instruction, two steps ahead, into registers) and writes them to a
//      workgroup tile in LDS kept as four 128-wide slices.  Wave w then
//      computes slice w's part of the scores, the four parts are summed
//      through LDS, so every wave holds the full scores of the 16 heads, and
//      wave w accumulates slice w of sum_j p_hj c_j.  Online softmax as in
//      the prefill kernel.  16 x 16 x 32 matrix-core products
//      (16 tokens x 16 heads), so 16 heads fill the tile with no padding.
//   3. mla_merge_upproj_kernel: merges the parts of each sequence
//      (log-sum-exp weights) into the normalised latent output (fp32) and
//      computes o_h = (sum_j p_hj c_j) W_V[h] from it on the matrix cores.
//
// Work split: sequence lengths differ widely and live on the device, so the
// scheduling workgroup sums the pages P of all sequences and cuts each
// sequence into ceil(pages / t) near-equal parts, t = ceil(P / slots) pages
// rounded up to even and capped at 64 (slots: workgroups of step 2 that stay
// resident, less one per sequence for the rounding).  Every part then takes
// about the same time and the whole grid runs in one wave; a sequence of one
// part writes its final latent output directly.
//
// q~ and the latent output are intermediate results, not inputs: rounding
// them to bf16 would add about 2^-9 relative error to every score and output
// on top of what the plain path has.  Each is kept in fp32 and enters the
// matrix cores as the sum of two bf16 terms (hi = bf16(x), lo = bf16(x - hi),
// two products into one fp32 accumulator), which keeps it to about 2^-17.
#include <algorithm>
#include <atomic>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kDC = 512;                // latent width
constexpr int kDH = 128;                // head dim
constexpr int kPageM = 16;
constexpr int kMaxPart = 64;            // pages per workgroup of the partial kernel, at most
constexpr int kHG = 16;                 // heads per workgroup of the partial kernel
constexpr int kMaxSlots = 1024;         // resident partial workgroups assumed when sizing the workspace
static_assert(kMaxPart <= 64, "a part's page ids fit one register across a wave's lanes");
constexpr int kThreadsL = 256;
constexpr float kTauL = 8.f;


typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// LDS tile rows are 256 bytes (128 bf16 of one token's latent slice); chunk c
// of row r sits at c ^ swz(r).  Conflict-free for the operand reads of the
// scores (16 consecutive rows, one chunk each), for the transposing reads of
// the weighted sum (8 consecutive rows, one aligned chunk pair each) and for
// the row writes (one row, 16 chunks).
__device__ __forceinline__ int swz(int r) { return (2 * (r & 7)) ^ ((r >> 3) & 1); }

__device__ __forceinline__ s16x4 lds_tr16(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(const __attribute__((address_space(3))) uint8_t*)p);
}

// 16x16x32 bf16 matrix-core product, fp32 accumulation: lane l holds row
// l % 16 of A and column l % 16 of B, contraction elements 8 (l / 16) .. +7;
// the accumulator holds D[4 (l / 16) + r][l % 16] in register r.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposed operand of the weighted sum for latent block blk (dims
// 16 blk .. +15 of the slice): lane l receives dim 16 blk + l % 16 of the
// tokens 4 g + e and 16 + 4 g + e (g = l / 16, e = 0..3), the order in which
// a lane holds p.  Each 16-lane group reads a 4-row x 16-column block per
// instruction and receives it transposed.
__device__ __forceinline__ bf16x8 tr_op(const uint8_t* tile, int blk, int lane) {
    const int s = lane & 15, g = lane >> 4;
    const int col = 16 * blk + 4 * (s & 3);
    const int r0 = 4 * g + (s >> 2), r1 = r0 + 16;
    const int x = col >> 3, half = (col >> 2) & 1;
    const s16x4 a = lds_tr16(tile + r0 * 256 + 16 * (x ^ swz(r0)) + 8 * half);
    const s16x4 b = lds_tr16(tile + r1 * 256 + 16 * (x ^ swz(r1)) + 8 * half);
    const s16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// Eight fp32 values as hi + lo bf16 operands.
__device__ __forceinline__ void split_bf16x8(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
    const u32x4 h = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                     pack_bf16x2(b[2], b[3])};
    const u32x4 l = {pack_bf16x2(a[0] - bf16lo_to_f32(h[0]), a[1] - bf16hi_to_f32(h[0])),
                     pack_bf16x2(a[2] - bf16lo_to_f32(h[1]), a[3] - bf16hi_to_f32(h[1])),
                     pack_bf16x2(b[0] - bf16lo_to_f32(h[2]), b[1] - bf16hi_to_f32(h[2])),
                     pack_bf16x2(b[2] - bf16lo_to_f32(h[3]), b[3] - bf16hi_to_f32(h[3]))};
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// ---- work split (one workgroup) ----
// work[i] = (sequence, first page, end page, 0) for i < W, sequence -1 after;
// part[s] = (first work index, number of parts) of sequence s.
__device__ void mla_schedule(const int32_t* __restrict__ seqlens, int nseq, int max_blocks, int target, int wcap,
                             int4* __restrict__ work, int2* __restrict__ part) {
    constexpr int kW = kThreadsL / 64;
    __shared__ int64_t wsum[kW];
    __shared__ int wscan[2][kW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    auto pages_of = [&](int s) { return (min(max(seqlens[s], 0), max_blocks * kPageM) + kPageM - 1) / kPageM; };
    int64_t local = 0;
    for (int s = tid; s < nseq; s += kThreadsL) local += pages_of(s);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) local += __shfl_xor(local, o);
    if (lane == 0) wsum[wave] = local;
    __syncthreads();
    int64_t P = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) P += wsum[w];
    int64_t t = (P + target - 1) / target;
    t = min<int64_t>(kMaxPart, max<int64_t>(2, (t + 1) & ~(int64_t)1));
    int base = 0;
    for (int c0 = 0, round = 0; c0 < nseq; c0 += kThreadsL, round ^= 1) {
        const int s = c0 + tid;
        const int pg = s < nseq ? pages_of(s) : 0;
        const int n = s < nseq ? max(1, (int)((pg + t - 1) / t)) : 0;
        int incl = n;                                     // inclusive scan within the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o);
            if (lane >= o) incl += v;
        }
        if (lane == 63) wscan[round][wave] = incl;        // alternate buffers: no barrier before the write
        __syncthreads();
        int before = base, total = 0;
#pragma unroll
        for (int w = 0; w < kW; ++w) {
            const int v = wscan[round][w];
            before += w < wave ? v : 0;
            total += v;
        }
        const int first = before + incl - n;
        if (s < nseq) {
            part[s] = int2{first, n};
            const int steps = (pg + 1) / 2;               // parts cut at even pages (whole 32-token steps)
            for (int k = 0; k < n; ++k) {
                const int a0 = (int)((int64_t)k * steps / n), a1 = (int)((int64_t)(k + 1) * steps / n);
                work[first + k] = int4{s, 2 * a0, min(2 * a1, pg), 0};
            }
        }
        base += total;
    }
    for (int i = base + tid; i < wcap; i += kThreadsL) work[i] = int4{-1, 0, 0, 0};
}

// ---- 1. absorbed queries: q~[s, h, :] = W_K[h] q[s, h] ----
// Workgroup (h, 128 latent rows, 32 sequences); wave w computes 32 of the
// rows: D[i][j] = sum_k W_K[h][i][k] q[s_j][h][k] (A = rows of W_K[h], B =
// query rows), all loads issued before the 8 products.
__global__ __launch_bounds__(kThreadsL) void mla_absorb_kernel(const uint16_t* __restrict__ Qin,
                                                               const uint16_t* __restrict__ WK,
                                                               float* __restrict__ Qa, int nseq, int H,
                                                               const int32_t* __restrict__ seqlens, int max_blocks,
                                                               int target, int wcap, int4* __restrict__ work,
                                                               int2* __restrict__ part) {
    if ((int)blockIdx.x == H) {                           // the scheduling workgroup
        if (blockIdx.y == 0 && blockIdx.z == 0) mla_schedule(seqlens, nseq, max_blocks, target, wcap, work, part);
        return;
    }
    const int h = blockIdx.x, s0 = blockIdx.z * 32;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int s = s0 + l32;
    const int i_base = 128 * blockIdx.y + 32 * wave;
    const uint16_t* qp = Qin + ((int64_t)min(s, nseq - 1) * H + h) * kDH + 8 * hh;
    const uint16_t* wp = WK + ((int64_t)h * kDC + i_base + l32) * kDH + 8 * hh;
    bf16x8 qb[kDH / 16], wa[kDH / 16];
#pragma unroll
    for (int k = 0; k < kDH / 16; ++k) {
        qb[k] = *reinterpret_cast<const bf16x8*>(qp + 16 * k);
        wa[k] = *reinterpret_cast<const bf16x8*>(wp + 16 * k);
    }
    f32x16 acc = f32x16{};
#pragma unroll
    for (int k = 0; k < kDH / 16; ++k) acc = mfma32(wa[k], qb[k], acc);
    if (s >= nseq) return;
    float* out = Qa + ((int64_t)s * H + h) * kDC + i_base;
#pragma unroll
    for (int a = 0; a < 4; ++a)
        *reinterpret_cast<f32x4*>(out + 8 * a + 4 * hh) = f32x4{acc[4 * a], acc[4 * a + 1], acc[4 * a + 2], acc[4 * a + 3]};
}

// ---- 2. attention over the latents, one chunk of a sequence, 16 heads ----
__global__ __launch_bounds__(kThreadsL, 2) void mla_partial_kernel(
    const float* __restrict__ Qa, const uint16_t* __restrict__ CC, const int32_t* __restrict__ table,
    const int32_t* __restrict__ seqlens, const int4* __restrict__ work, const int2* __restrict__ part,
    float* __restrict__ Olat, float* __restrict__ LSE, float* __restrict__ ws_o, float* __restrict__ ws_lse, int H,
    int Hp, int max_blocks, int num_blocks, float scale_log2) {
    // latent tile of a step, double buffered: [buffer][slice][32 tokens][256 B]
    __shared__ __attribute__((aligned(1024))) uint8_t tiles[2][4][32 * 256];
    __shared__ __attribute__((aligned(16))) float xs[4][2][64 * 4];      // per-wave partial scores

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;

    const int wi = blockIdx.x;
    const int4 item = work[wi];                           // (sequence, first page, end page)
    const int s = item.x;
    if (s < 0) return;                                    // whole workgroup: no barrier reached
    const int head = kHG * blockIdx.y + l16;              // this lane's head (>= H: padding)
    const int len = min(max(seqlens[s], 0), max_blocks * kPageM);
    const int p0 = item.y, p1 = item.z;                   // p1 - p0 <= 64, p0 even
    const int nparts = part[s].y;
    const int n_steps = (p1 - p0 + 1) / 2;                // 0 for an empty sequence
    const int32_t* trow = table + (int64_t)s * max_blocks;
    const int tb_lane = (p0 + lane < p1) ? trow[p0 + lane] : -1;   // the chunk's page ids, one per lane
    auto blk_of = [&](int p) -> int {
        const int b = __builtin_amdgcn_readlane(tb_lane, min(max(p - p0, 0), 63));
        return (p < p1 && b >= 0 && b < num_blocks) ? b : -1;
    };

    // this lane's 32 slice entries of its head's absorbed query (loaded here,
    // split into hi + lo bf16 once the first latent loads are issued): the
    // B operand of S^T = C Q~^T, contraction group g of 32 ks + ..
    const bool row_ok = head < H;
    f32x4 qraw[8];
    {
        const float* qp = Qa + ((int64_t)s * H + min(head, H - 1)) * kDC + 128 * wave + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            qraw[2 * ks] = *reinterpret_cast<const f32x4*>(qp + 32 * ks);
            qraw[2 * ks + 1] = *reinterpret_cast<const f32x4*>(qp + 32 * ks + 4);
        }
    }
    bf16x8 qh[4], ql[4];

    // coalesced loads of a step's latent rows: wave w takes tokens 8 w .. +7
    // (page pa + w / 2), one whole 1 KiB row per instruction, lane l bytes
    // 16 l .. +15.  Steps past the chunk read page 0 (never used).
    const int my_page = wave >> 1, my_row0 = 8 * (wave & 1);
    auto load_step = [&](int step, u32x4 (&cr)[8]) {
        const int b = max(blk_of(p0 + 2 * step + my_page), 0);
        const uint16_t* src = CC + ((int64_t)b * kPageM + my_row0) * kDC + 8 * lane;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            cr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + j * kDC));
    };

    f32x4 oacc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) oacc[i] = f32x4{};
    float m_run = kNegInf, l_run = 0.f;

    auto step = [&](int it, u32x4 (&cr)[8]) __attribute__((always_inline)) {
        const int pa = p0 + 2 * it;
        const bool ok0 = blk_of(pa) >= 0, ok1 = blk_of(pa + 1) >= 0;
        // registers -> tile (this lane's 16 bytes belong to slice l / 16);
        // rows of unusable tokens are zero (the tile also serves as the value
        // operand, where p = 0 would not cancel a NaN).  The other buffer may
        // still be read by waves finishing the previous step.
        uint8_t* const tbuf = tiles[it & 1][0];
        const bool okw = my_page == 0 ? ok0 : ok1;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 8 * wave + j, ch = lane & 15;
            const bool bad = !okw || pa * kPageM + r >= len;
            *reinterpret_cast<u32x4*>(tbuf + (lane >> 4) * (32 * 256) + r * 256 + 16 * (ch ^ swz(r))) =
                bad ? u32x4{0u, 0u, 0u, 0u} : cr[j];
        }
        load_step(it + 2, cr);                            // in flight for two steps
        __syncthreads();                                  // the step's tile is complete
        const uint8_t* const tile = tiles[it & 1][wave];
        // this wave's slice of the scores: S^T (16 tokens x 16 heads) per token block
        f32x4 sp[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            sp[tb] = f32x4{};
            const int r = 16 * tb + l16;
            const uint8_t* crow = tile + r * 256;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 ca = *reinterpret_cast<const bf16x8*>(crow + 16 * ((4 * ks + g) ^ swz(r)));
                sp[tb] = mfma16(ca, qh[ks], sp[tb]);
                sp[tb] = mfma16(ca, ql[ks], sp[tb]);
            }
        }
        // sum the four slices through LDS (every wave has finished reading
        // the previous step's sums: it passed the barrier above)
        float* xw = xs[wave][0] + lane * 4;
        *reinterpret_cast<f32x4*>(xw) = sp[0];
        *reinterpret_cast<f32x4*>(xw + 64 * 4) = sp[1];
        __syncthreads();
        f32x4 sa[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) sa[tb] += *reinterpret_cast<const f32x4*>(xs[w][tb] + lane * 4);
        // mask; token of (tb, e) is 16 tb + 4 g + e.  A step whose 32 tokens
        // all lie in usable pages before the length needs none (a
        // wave-uniform test); padding heads then score against zero
        // queries, and their results are never written.
        float mx = kNegInf;
        if (ok0 && ok1 && pa * kPageM + 32 <= len) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sa[tb][e]);
        } else {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int kk = 16 * tb + 4 * g + e;
                    const bool ok = row_ok && (tb == 0 ? ok0 : ok1) && pa * kPageM + kk < len;
                    sa[tb][e] = ok ? sa[tb][e] : kNegInf;
                    mx = fmaxf(mx, sa[tb][e]);
                }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kTauL)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = exp2f_hw(m_run - (m_new == kNegInf ? 0.f : m_new));
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < 8; ++i) oacc[i] *= alpha;
        }
        const float m_use = m_run == kNegInf ? 0.f : m_run;
        u32x4 pw;
        float rs = 0.f;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const float a = exp2f_hw(fmaf(sa[tb][0], scale_log2, -m_use));
            const float b = exp2f_hw(fmaf(sa[tb][1], scale_log2, -m_use));
            const float c = exp2f_hw(fmaf(sa[tb][2], scale_log2, -m_use));
            const float d = exp2f_hw(fmaf(sa[tb][3], scale_log2, -m_use));
            rs += (a + b) + (c + d);
            pw[2 * tb] = pack_bf16x2(a, b);
            pw[2 * tb + 1] = pack_bf16x2(c, d);
        }
        l_run += rs;
        // this wave's slice of sum_j p_hj c_j: O^T (latent x heads) += C^T P^T
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) oacc[blk] = mfma16(tr_op(tile, blk, lane), pb, oacc[blk]);
    };

    u32x4 crA[8], crB[8];
    load_step(0, crA);
    // keep the issue order (step 0 first): the loop waits only for the older
    // of the two steps in flight, which the wait counts can express only if
    // both paths into the loop issue the loads in the same order
    __builtin_amdgcn_sched_barrier(0);
    load_step(1, crB);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        split_bf16x8(row_ok ? qraw[2 * ks] : f32x4{}, row_ok ? qraw[2 * ks + 1] : f32x4{}, qh[ks], ql[ks]);
    for (int it = 0; it < n_steps; it += 2) {
        step(it, crA);
        if (it + 1 >= n_steps) break;                      // uniform: no barrier is skipped by some waves only
        step(it + 1, crB);
    }

    // every wave holds the same (m, l) per head; output this wave's slice
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse = l_tot > 0.f ? (m_run + log2f_hw(l_tot)) * kLn2 : kNegInf;
    if (!row_ok) return;
    float* op;
    if (nparts <= 1) {
        op = Olat + ((int64_t)s * H + head) * kDC + 128 * wave;
        if (LSE != nullptr && wave == 0 && g == 0) LSE[(int64_t)s * H + head] = lse;
    } else {
        op = ws_o + ((int64_t)wi * Hp + head) * kDC + 128 * wave;
        if (wave == 0 && g == 0) ws_lse[(int64_t)wi * Hp + head] = lse;
    }
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) *reinterpret_cast<f32x4*>(op + 16 * blk + 4 * g) = oacc[blk] * inv;
}

// ---- 3. merge the parts of each sequence, then up-project:
// o[s, h, j] = sum_i W_V^T[h][j][i] olat[s, h, i] ----
// Workgroup (h, 4 sequences).  Merge: wave w takes sequence 4 b + w, each
// lane 8 latent entries of every part's 2 KiB row (one coalesced row per
// part), folding the parts in with the online log-sum-exp update (running
// maximum, rescaled sum), so the loads of 8 parts are in flight at once; a
// sequence of one part reads the latent output the partial kernel wrote.  The
// merged rows (fp32) go to LDS.  Up-projection: wave w computes output dims
// 32 w .. 32 w + 31 of the 4 sequences with 16x16x32 products over the 512
// latent entries (W_V rows as A, loaded before the merge; the merged rows as
// hi + lo B operands; columns 4..15 repeat the 4 sequences and are dropped).
constexpr int kSeqU = 4;                  // sequences per workgroup (one per wave)
constexpr int kRowU = kDC + 4;            // LDS row stride in floats
__global__ __launch_bounds__(kThreadsL) void mla_merge_upproj_kernel(
    const float* __restrict__ Olat, const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
    const int2* __restrict__ part, const uint16_t* __restrict__ WVT, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int nseq, int H, int Hp) {
    __shared__ __attribute__((aligned(16))) float cl[kSeqU * kRowU];
    const int h = blockIdx.x, s0 = blockIdx.y * kSeqU;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, g = lane >> 4;

    // A operands: W_V^T[h][32 w + 16 jb + l16][32 ks + 8 g .. +7]
    bf16x8 wa[2][kDC / 32];
    {
        const uint16_t* wp = WVT + ((int64_t)h * kDH + 32 * wave + l16) * kDC + 8 * g;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int ks = 0; ks < kDC / 32; ++ks)
                wa[jb][ks] = *reinterpret_cast<const bf16x8*>(wp + (int64_t)16 * jb * kDC + 32 * ks);
    }

    // ---- merge ----
    {
        const int s = s0 + wave;                          // wave-uniform
        f32x4 va = f32x4{}, vb = f32x4{};
        if (s < nseq) {
            const int2 pt = part[s];
            if (pt.y <= 1) {
                const float* lp = Olat + ((int64_t)s * H + h) * kDC + 8 * lane;
                va = *reinterpret_cast<const f32x4*>(lp);
                vb = *reinterpret_cast<const f32x4*>(lp + 4);
            } else {
                const int64_t slot0 = pt.x;
                const int n = pt.y;
                float m = kNegInf, L = 0.f;
                // parts in batches of 8: all loads of a batch are issued
                // before the first of them is used (one memory round trip)
                constexpr int kB = 8;
                for (int c0 = 0; c0 < n; c0 += kB) {
                    float lcv[kB];
                    f32x4 xa[kB], xb[kB];
#pragma unroll
                    for (int j = 0; j < kB; ++j) {
                        const int64_t row = (slot0 + min(c0 + j, n - 1)) * Hp + h;
                        lcv[j] = ws_lse[row];
                        const float* vp = ws_o + row * kDC + 8 * lane;
                        xa[j] = *reinterpret_cast<const f32x4*>(vp);
                        xb[j] = *reinterpret_cast<const f32x4*>(vp + 4);
                    }
#pragma unroll
                    for (int j = 0; j < kB; ++j) {
                        // (a part past the last counts with weight 0 and
                        // leaves the state as it is)
                        const float lc = c0 + j < n ? lcv[j] : kNegInf;
                        const float mn = fmaxf(m, lc);
                        const float mu = mn == kNegInf ? 0.f : mn;
                        const float r = exp2f_hw((m - mu) * kLog2e), w = exp2f_hw((lc - mu) * kLog2e);
                        m = mn;
                        L = fmaf(L, r, w);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            va[e] = fmaf(va[e], r, w * xa[j][e]);
                            vb[e] = fmaf(vb[e], r, w * xb[j][e]);
                        }
                    }
                }
                const float inv = L > 0.f ? 1.f / L : 0.f;
                va *= inv;
                vb *= inv;
                if (LSE != nullptr && lane == 0) LSE[(int64_t)s * H + h] = L > 0.f ? m + log2f_hw(L) * kLn2 : kNegInf;
            }
        }
        float* dst = cl + wave * kRowU + 8 * lane;
        *reinterpret_cast<f32x4*>(dst) = va;
        *reinterpret_cast<f32x4*>(dst + 4) = vb;
    }
    __syncthreads();

    // ---- up-projection: D[j][s] over i ----
    f32x4 acc[2] = {f32x4{}, f32x4{}};
    const float* brow = cl + (l16 % kSeqU) * kRowU + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kDC / 32; ++ks) {
        const f32x4 xa = *reinterpret_cast<const f32x4*>(brow + 32 * ks);
        const f32x4 xb = *reinterpret_cast<const f32x4*>(brow + 32 * ks + 4);
        bf16x8 hi, lo;
        split_bf16x8(xa, xb, hi, lo);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            acc[jb] = mfma16(wa[jb][ks], hi, acc[jb]);
            acc[jb] = mfma16(wa[jb][ks], lo, acc[jb]);
        }
    }
    const int s = s0 + l16;
    if (l16 >= kSeqU || s >= nseq) return;
    uint16_t* out = O + ((int64_t)s * H + h) * kDH + 32 * wave + 4 * g;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
        *reinterpret_cast<u32x2*>(out + 16 * jb) =
            u32x2{pack_bf16x2(acc[jb][0], acc[jb][1]), pack_bf16x2(acc[jb][2], acc[jb][3])};
}

struct MlaLayout {
    size_t qa, olat, work, part, wo, wl, total;
    int64_t wcap;
};

int head_groups(int H) { return (H + kHG - 1) / kHG; }

// Work items the partial kernel may be given: at most target + nseq (parts
// of t >= P / target pages, one rounding per sequence) or, when t is capped,
// P / 64 + nseq with P <= nseq * max_blocks.
int64_t work_capacity(int nseq, int max_blocks, int64_t target) {
    return std::max<int64_t>(target, ((int64_t)nseq * max_blocks + kMaxPart - 1) / kMaxPart) + nseq;
}

MlaLayout mla_layout(int nseq, int H, int max_blocks) {
    const size_t Hp = (size_t)kHG * head_groups(H);
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    MlaLayout L{};
    L.wcap = work_capacity(nseq, max_blocks, kMaxSlots);
    L.qa = 0;
    L.olat = up(L.qa + (size_t)nseq * H * kDC * 4);
    L.work = up(L.olat + (size_t)nseq * H * kDC * 4);
    L.part = up(L.work + (size_t)L.wcap * sizeof(int4));
    L.wo = up(L.part + (size_t)nseq * sizeof(int2));
    L.wl = up(L.wo + (size_t)L.wcap * Hp * kDC * 4);
    L.total = up(L.wl + (size_t)L.wcap * Hp * 4);
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

}  // namespace

size_t mla_workspace_bytes(int nseq, int H, int max_blocks) { return mla_layout(nseq, H, max_blocks).total; }

hipError_t launch_mla_decode(const MlaArgs& a, void* workspace, hipStream_t stream) {
    const MlaLayout L = mla_layout(a.nseq, a.H, a.max_blocks);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* qa = reinterpret_cast<float*>(ws + L.qa);
    float* olat = reinterpret_cast<float*>(ws + L.olat);
    int4* work = reinterpret_cast<int4*>(ws + L.work);
    int2* part = reinterpret_cast<int2*>(ws + L.part);
    float* wo = reinterpret_cast<float*>(ws + L.wo);
    float* wl = reinterpret_cast<float*>(ws + L.wl);
    const int hg = head_groups(a.H);
    // two partial workgroups stay resident per CU; one part per slot, less
    // one per sequence for the rounding of the parts
    const int64_t slots = std::min<int64_t>(kMaxSlots, 2 * (int64_t)device_cus() / hg);
    const int64_t target = std::max<int64_t>(1, slots - a.nseq);
    const int64_t wcap = work_capacity(a.nseq, a.max_blocks, target);   // <= L.wcap: target <= kMaxSlots
    const unsigned sblocks = (unsigned)((a.nseq + 31) / 32);
    launch_kernel<false>(mla_absorb_kernel, dim3((unsigned)a.H + 1, kDC / 128, sblocks), dim3(kThreadsL), 0, stream,
                         (const uint16_t*)a.q, (const uint16_t*)a.w_uk, qa, a.nseq, a.H, a.seqlens, a.max_blocks,
                         (int)target, (int)wcap, work, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_kernel<false>(mla_partial_kernel, dim3((unsigned)wcap, (unsigned)hg), dim3(kThreadsL), 0, stream,
                         (const float*)qa, (const uint16_t*)a.ccache, a.block_table, a.seqlens, (const int4*)work,
                         (const int2*)part, olat, a.lse, wo, wl, a.H, kHG * hg, a.max_blocks, a.num_blocks,
                         a.scale * kLog2e);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_kernel(mla_merge_upproj_kernel, dim3((unsigned)a.H, (unsigned)((a.nseq + kSeqU - 1) / kSeqU)),
                  dim3(kThreadsL), 0, stream,
                  (const float*)olat, (const float*)wo, (const float*)wl, (const int2*)part, (const uint16_t*)a.w_uv_t,
                  (uint16_t*)a.o, a.lse, a.nseq, a.H, kHG * hg);
    return hipGetLastError();
}

}  // namespace fa
